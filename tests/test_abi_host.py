"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/moe.h declares, and rejects bad arguments before touching a
device.  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from quantized_routed_expert_amd import moe
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_gfx950.so is not built (run quantized_routed_expert_amd.build)")
    return moe.lib()


def test_exports_match_header(L):
    names = header_functions()
    from quantized_routed_expert_amd import moe
    assert sorted(moe.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status(L):
    from quantized_routed_expert_amd import moe
    assert L.moe_version() == 100
    for s in (0, -1, -2, -3, -4, -5, -99):
        assert len(moe.status_string(s)) > 0
    assert moe.status_string(-3).startswith("workspace")


def test_expert_bytes(L):
    from quantized_routed_expert_amd import moe
    # bytes per expert = 3*H*F/32*B, B = 18 (4-bit) or 14 (3-bit)
    assert moe.expert_bytes(4, 256, 512) == 221184
    assert moe.expert_bytes(4, 2048, 768) == 2654208
    assert moe.expert_bytes(3, 2048, 768) == 2064384
    assert moe.expert_bytes(3, 2048, 512) == 1376256
    assert moe.expert_bytes(5, 2048, 512) == -1
    assert moe.expert_bytes(4, 2047, 512) == -1
    # per-projection widths: H*F/32 * (2*B_gate/up + B_down)
    assert moe.expert_bytes(3, 2048, 512, down_bits=4) == 2048 * 16 * (2 * 14 + 18)
    assert moe.expert_bytes(4, 2048, 768, down_bits=3) == 2048 * 24 * (2 * 18 + 14)
    assert moe.expert_bytes(3, 2048, 512, down_bits=3) == moe.expert_bytes(3, 2048, 512)
    assert moe.expert_bytes(3, 2048, 512, down_bits=5) == -1
    # the non-linear 4-bit block (code 20) has the 4-bit block's 18 bytes
    assert moe.expert_bytes(moe.BITS_NL4, 2048, 768) == 2654208
    assert moe.expert_bytes(3, 2048, 512, down_bits=moe.BITS_NL4) == 2048 * 16 * (2 * 14 + 18)
    assert moe.expert_bytes(21, 2048, 512) == -1


def test_workspace_bytes(L):
    from quantized_routed_expert_amd import moe
    for path in (0, 1, 2):
        n = moe.workspace_bytes(16, 128, 8, 2048, 768, 768, path)
        assert n > 16 * 8 * 2048 * 4
    assert L.moe_workspace_bytes(4, 8, 9, 256, 512, 512, 0) == moe.MOE_ERR_UNSUPPORTED  # k > E
    assert L.moe_workspace_bytes(-1, 8, 2, 256, 512, 512, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_bytes(4, 8, 2, 250, 512, 512, 0) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_bytes(4, 8, 2, 256, 512, 100, 0) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_bytes(4, 8, 2, 256, 512, 0, 7) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_bytes(4, 5000, 2, 256, 512, 0, 0) == moe.MOE_ERR_UNSUPPORTED


def test_rejects_before_launch(L):
    """Every error path returns its code on the host (no device is touched)."""
    from quantized_routed_expert_amd import moe
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert L.moe_route(None, 4, 8, 2, fake, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(fake, 4, 8, 9, fake, fake, 0) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_route(fake, 4, 8, 0, fake, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(fake, -4, 8, 2, fake, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(fake, 4, 8, 33, fake, fake, 0) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_group(fake, 4, 8, 2, fake, None, fake, fake, 1 << 20, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_group(fake, 4, 8, 2, fake, fake, fake, fake, 0, 0) == moe.MOE_ERR_WORKSPACE

    P = moe.LAYOUT_PREPARED
    w = moe.QWeights(fake, 4, 8, 256, 512, P)
    bad_bits = moe.QWeights(fake, 5, 8, 256, 512, P)
    bad_h = moe.QWeights(fake, 4, 8, 200, 512, P)
    bad_sh = moe.QWeights(fake, 4, 2, 256, 512, P)   # shared must hold one expert
    nodata = moe.QWeights(None, 4, 8, 256, 512, P)
    rows = moe.QWeights(fake, 4, 8, 256, 512, moe.LAYOUT_ROWS)  # not converted
    sh = moe.QWeights(fake, 4, 1, 256, 512, P)
    big = 1 << 30

    def lf(x=fake, dt=0, lg=fake, T=4, k=2, r=w, s=sh, y=fake, path=0, ws=fake, wsb=big):
        return L.moe_layer_forward(x, dt, lg, T, k, ctypes.byref(r), ctypes.byref(s) if s else None, y, None,
                                   None, None, path, ws, wsb, 0)

    assert lf(x=None) == moe.MOE_ERR_INVALID_ARG
    assert lf(lg=None) == moe.MOE_ERR_INVALID_ARG
    assert lf(y=None) == moe.MOE_ERR_INVALID_ARG
    assert lf(ws=None) == moe.MOE_ERR_INVALID_ARG
    assert lf(dt=3) == moe.MOE_ERR_INVALID_ARG
    assert lf(path=5) == moe.MOE_ERR_INVALID_ARG
    assert lf(r=bad_bits) == moe.MOE_ERR_UNSUPPORTED
    assert lf(r=bad_h) == moe.MOE_ERR_INVALID_ARG        # hidden differs from the shared expert's
    assert lf(r=bad_h, s=None) == moe.MOE_ERR_UNSUPPORTED  # hidden not a multiple of 256
    assert lf(r=nodata) == moe.MOE_ERR_INVALID_ARG
    assert lf(r=rows) == moe.MOE_ERR_UNSUPPORTED
    assert lf(s=moe.QWeights(fake, 4, 1, 256, 512, moe.LAYOUT_ROWS)) == moe.MOE_ERR_UNSUPPORTED
    assert lf(s=bad_sh) == moe.MOE_ERR_INVALID_ARG
    assert lf(k=9) == moe.MOE_ERR_UNSUPPORTED
    assert lf(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert lf(wsb=16) == moe.MOE_ERR_WORKSPACE
    assert lf(T=17, path=moe.PATH_DECODE) == moe.MOE_ERR_UNSUPPORTED
    # a shared expert whose bit width differs from the routed experts' is
    # refused on every path (each launch reads it in the routed format)
    for path in (moe.PATH_AUTO, moe.PATH_DECODE, moe.PATH_PREFILL):
        assert lf(s=moe.QWeights(fake, 3, 1, 256, 512, P), path=path) == moe.MOE_ERR_UNSUPPORTED
        # ... and so is one whose down width differs
        assert lf(s=moe.QWeights(fake, 4, 1, 256, 512, P, 3), path=path) == moe.MOE_ERR_UNSUPPORTED
        assert lf(r=moe.QWeights(fake, 4, 8, 256, 512, P, 3), path=path) == moe.MOE_ERR_UNSUPPORTED
        assert lf(r=moe.QWeights(fake, 4, 8, 256, 512, P, 5), path=path) == moe.MOE_ERR_UNSUPPORTED
        assert lf(r=moe.QWeights(fake, 3, 8, 256, 512, P), path=path) == moe.MOE_ERR_UNSUPPORTED
        assert lf(T=40, s=moe.QWeights(fake, 3, 1, 256, 512, P), path=path) == moe.MOE_ERR_UNSUPPORTED
    # non-linear 4-bit: the shared expert must carry the routed experts' table
    NL = moe.BITS_NL4
    r_nl = moe.qweights_at(fake, NL, 8, 256, 512, P, 0, tuple(range(-8, 8)))
    s_other = moe.qweights_at(fake, NL, 1, 256, 512, P, 0, tuple(range(8, -8, -1)))
    for path in (moe.PATH_AUTO, moe.PATH_DECODE, moe.PATH_PREFILL):
        assert lf(r=r_nl, s=s_other, path=path) == moe.MOE_ERR_UNSUPPORTED
    # a pair the decode launch does not build is refused on an explicit decode request
    r_mix = moe.qweights_at(fake, NL, 8, 256, 512, P, 3, tuple(range(-8, 8)))
    assert lf(r=r_mix, s=None, path=moe.PATH_DECODE) == moe.MOE_ERR_UNSUPPORTED
    assert lf(r=moe.QWeights(fake, 21, 8, 256, 512, P), s=None) == moe.MOE_ERR_UNSUPPORTED
    # T == 0 is a valid empty call: nothing is launched
    assert lf(T=0) == moe.MOE_OK

    def ef(x=fake, T=4, ww=w, off=fake, path=0, wsb=big, out=fake):
        return L.moe_expert_ffn(x, 1, T, ctypes.byref(ww), off, fake, fake, None, 2, out, path, fake, wsb, 0)

    assert ef(x=None) == moe.MOE_ERR_INVALID_ARG
    assert ef(off=None) == moe.MOE_ERR_INVALID_ARG
    assert ef(out=None) == moe.MOE_ERR_INVALID_ARG
    assert ef(ww=bad_bits) == moe.MOE_ERR_UNSUPPORTED
    assert ef(ww=rows) == moe.MOE_ERR_UNSUPPORTED
    assert ef(T=17, path=moe.PATH_DECODE) == moe.MOE_ERR_UNSUPPORTED
    assert ef(wsb=0) == moe.MOE_ERR_WORKSPACE
    assert ef(T=0) == moe.MOE_OK


def test_router_logits_rejects(L):
    """The router projection validates on the host before touching a device."""
    from quantized_routed_expert_amd import moe
    fake = ctypes.c_void_p(0x1000)
    rl = L.moe_router_logits
    assert rl(fake, 1, 4, 250, fake, 8, fake, 0) == moe.MOE_ERR_UNSUPPORTED   # hidden not a multiple of 256
    assert rl(fake, 1, 4, 8192, fake, 8, fake, 0) == moe.MOE_ERR_UNSUPPORTED  # hidden beyond 4096
    assert rl(fake, 1, 4, 256, fake, 5000, fake, 0) == moe.MOE_ERR_UNSUPPORTED
    assert rl(fake, 2, 4, 256, fake, 8, fake, 0) == moe.MOE_ERR_INVALID_ARG   # dtype
    assert rl(None, 1, 4, 256, fake, 8, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert rl(fake, 1, 4, 256, None, 8, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert rl(fake, 1, -1, 256, fake, 8, fake, 0) == moe.MOE_ERR_INVALID_ARG
    assert rl(fake, 1, 0, 256, fake, 8, None, 0) == moe.MOE_OK  # empty: nothing launched


def test_workspace_error_rejects(L):
    """The error query checks its arguments before touching the device."""
    from quantized_routed_expert_amd import moe
    fake = ctypes.c_void_p(0x1000)
    v = ctypes.c_uint32(7)
    assert L.moe_workspace_error(None, 1 << 20, ctypes.byref(v), 1, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_error(fake, 1 << 20, None, 1, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_error(fake, 64, ctypes.byref(v), 1, 0) == moe.MOE_ERR_WORKSPACE
    assert v.value == 7  # untouched on error


def test_prepare_rejects_before_launch(L):
    """moe_prepare_qweights validates on the host: null pointers, a source not
    in the row-by-row order, overlapping buffers, unsupported formats."""
    from quantized_routed_expert_amd import moe
    fake = ctypes.c_void_p(0x1000)
    eb = moe.expert_bytes(4, 256, 512)
    src = moe.QWeights(fake, 4, 8, 256, 512, moe.LAYOUT_ROWS)
    pf = L.moe_prepare_qweights
    assert pf(None, ctypes.c_void_p(0x10000000), 0) == moe.MOE_ERR_INVALID_ARG
    assert pf(ctypes.byref(src), None, 0) == moe.MOE_ERR_INVALID_ARG
    assert pf(ctypes.byref(moe.QWeights(None, 4, 8, 256, 512, 0)), ctypes.c_void_p(0x10000000), 0) == \
        moe.MOE_ERR_INVALID_ARG
    assert pf(ctypes.byref(moe.QWeights(fake, 4, 8, 256, 512, moe.LAYOUT_PREPARED)),
              ctypes.c_void_p(0x10000000), 0) == moe.MOE_ERR_INVALID_ARG
    # dst starting inside src, and src starting inside dst
    assert pf(ctypes.byref(src), ctypes.c_void_p(0x1000 + eb), 0) == moe.MOE_ERR_INVALID_ARG
    assert pf(ctypes.byref(moe.QWeights(ctypes.c_void_p(0x1000 + 64), 4, 8, 256, 512, 0)), fake, 0) == \
        moe.MOE_ERR_INVALID_ARG
    assert pf(ctypes.byref(moe.QWeights(fake, 5, 8, 256, 512, 0)), ctypes.c_void_p(0x10000000), 0) == \
        moe.MOE_ERR_UNSUPPORTED
    assert pf(ctypes.byref(moe.QWeights(fake, 4, 8, 200, 512, 0)), ctypes.c_void_p(0x10000000), 0) == \
        moe.MOE_ERR_UNSUPPORTED
    assert pf(ctypes.byref(moe.QWeights(fake, 4, 8, 256, 512, 0, 2)), ctypes.c_void_p(0x10000000), 0) == \
        moe.MOE_ERR_UNSUPPORTED
    # overlap is judged on the mixed-format size (gate/up 4-bit, down 3-bit)
    eb_mixed = moe.expert_bytes(4, 256, 512, down_bits=3)
    assert pf(ctypes.byref(moe.QWeights(fake, 4, 8, 256, 512, 0, 3)), ctypes.c_void_p(0x1000 + 8 * eb_mixed - 2),
              0) == moe.MOE_ERR_INVALID_ARG
