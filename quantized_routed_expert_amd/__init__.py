"""MI355X-native routed mixture-of-experts layer over block-quantized experts.

The compute path is a HIP library for gfx950 behind a C ABI (include/moe.h);
``quantized_routed_expert_amd.moe`` is its thin Python binding.  Importing
this package loads nothing; the binding loads the library on first use and
raises if it is missing.
"""
