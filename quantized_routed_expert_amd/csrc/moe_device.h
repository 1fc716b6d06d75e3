// moe_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Quantized blocks (block of 32 weights with an fp16 scale; the 4-bit block
// is the one the forum thread "把 Strata 搬上 SGLang 引擎 的嘗試" names in §四):
//   4-bit, 18 bytes: d, then byte 2+i = code i (low nibble) | code i+16 (high nibble)
//   3-bit, 14 bytes: d, 8 bytes of 2-bit low parts (code i at bit 2*(i/8) of byte
//                    2+(i%8)), 32-bit word at bytes 10..13 holding bit 2 of code i at bit i
//   non-linear 4-bit (format code 20), 18 bytes: the 4-bit layout; weight =
//                    d * table[code], a 16-entry table of signed 8-bit values
//                    (the same section names this block; the table comes with
//                    the weights)
//
// MFMA mapping (v_mfma_f32_16x16x32_{f16,bf16}, K = 32 = one block): lane l holds
// row l%16 of A, column l%16 of B and the k-group l/16 of both; the result D
// has rows 4*(l/16)+r, column l%16.  The eight k values a lane feeds in a
// k-group are any eight of the block's 32 as long as A and B use the same
// ones in the same order, so each format picks the order that makes its
// codes cheapest to unpack, and activations are stored in that order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "moe_internal.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Formats with the 4-bit block's layout (linear and non-linear codes).
__host__ __device__ constexpr bool nib_layout(int bits) { return bits == 4 || bits == MOE_FMT_NL4; }
__host__ __device__ constexpr int blk_bytes(int bits) { return nib_layout(bits) ? 18 : 14; }

// ---------------------------------------------------------------------------
// Element order inside one k-group (8 values) for each format.
// pos_in_block(bits, g, e): which of the block's 32 weights is the e-th value
// a lane of k-group g feeds.  Used to lay activations out to match.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int pos_in_block(int bits, int g, int e) {
    if (nib_layout(bits)) {
        // e: 0:(4g) 1:(4g+2) 2:(16+4g) 3:(16+4g+2) 4:(4g+1) 5:(4g+3) 6:(16+4g+1) 7:(16+4g+3)
        int r = ((e >> 2) & 1) + ((e & 1) << 1);
        return 4 * g + r + ((e >> 1) & 1) * 16;
    } else {
        // natural order: weights 8g .. 8g+7 (the 2-bit field g of all eight low-part bytes)
        return 8 * g + e;
    }
}

// Inverse: weight i of a block -> (k-group g, slot e).
__host__ __device__ __forceinline__ void group_slot_of(int bits, int i, int &g, int &e) {
    if (nib_layout(bits)) {
        int r = i & 3, hi = (i >> 4) & 1;
        g = (i & 15) >> 2;
        e = ((r & 1) << 2) | (hi << 1) | (r >> 1);
    } else {
        g = i >> 3;
        e = i & 7;
    }
}

__device__ __forceinline__ uint32_t pk_fma_h2(uint32_t v, uint32_t scale, uint32_t add) {
    half2v a = __builtin_bit_cast(half2v, v);
    half2v s = __builtin_bit_cast(half2v, scale);
    half2v c = __builtin_bit_cast(half2v, add);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(a, s, c));
}

// fp16 constants as packed bit patterns (lo half first)
#define H2(lo, hi) ((uint32_t)(lo) | ((uint32_t)(hi) << 16))
// 1024 + m is exact in fp16 for 0 <= m < 1024: OR-ing a code into the low
// mantissa bits of 0x6400 builds it without a conversion instruction.
#define FP16_MAGIC 0x64006400u

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | c; }

// 4-bit: q = bytes qs[4g..4g+3] of one block -> 8 exact fp16 values (code - 8)
// in the order of pos_in_block(4, g, .).
__device__ __forceinline__ half8 unpack4(uint32_t q) {
    const uint32_t one = H2(0x3C00, 0x3C00);        // 1.0
    const uint32_t s16 = H2(0x2C00, 0x2C00);        // 1/16
    const uint32_t o_lo = H2(0xE408, 0xE408);       // -1032
    const uint32_t o_hi = H2(0xD480, 0xD480);       // -72
    uint32_t q8 = q >> 8;
    uint32_t v0 = and_or(q, 0x000F000Fu, FP16_MAGIC);   // 1024 + c
    uint32_t v1 = and_or(q, 0x00F000F0u, FP16_MAGIC);   // 1024 + 16 c
    uint32_t v2 = and_or(q8, 0x000F000Fu, FP16_MAGIC);
    uint32_t v3 = and_or(q8, 0x00F000F0u, FP16_MAGIC);
    u32x4 r;
    r.x = pk_fma_h2(v0, one, o_lo);
    r.y = pk_fma_h2(v1, s16, o_hi);
    r.z = pk_fma_h2(v2, one, o_lo);
    r.w = pk_fma_h2(v3, s16, o_hi);
    return __builtin_bit_cast(half8, r);
}

// 3-bit: weights 8g .. 8g+7 of one block -> 8 exact fp16 values (code - 4), in
// that order.  qs0 / qs1: low-part bytes 0..3 / 4..7 of the block, qh: its
// third-bit word.  The codes are assembled one per byte, then looked up in a
// byte table: fp16(c - 4) has a zero low byte for c = 0..7.
__device__ __forceinline__ half8 unpack3(uint32_t qs0, uint32_t qs1, uint32_t qh, uint32_t g) {
    const uint32_t l0 = (qs0 >> (2u * g)) & 0x03030303u;  // low parts, one per byte
    const uint32_t l1 = (qs1 >> (2u * g)) & 0x03030303u;
    const uint32_t t0 = (qh >> (8u * g)) & 15u;            // third bits of weights 8g .. 8g+3
    const uint32_t t1 = (qh >> (8u * g + 4u)) & 15u;
    // bit j of t -> bit 2 of byte j: t * (4 + 2^9 + 2^16 + 2^23); the other
    // partial products land on bits the mask drops (all distinct: no carries)
    const uint32_t c0 = and_or(__umul24(t0, 0x810204u), 0x04040404u, l0);
    const uint32_t c1 = and_or(__umul24(t1, 0x810204u), 0x04040404u, l1);
    // high bytes of fp16(c - 4), c = 0..7: C4 C2 C0 BC 00 3C 40 42
    const uint32_t tab_lo = 0xBCC0C2C4u, tab_hi = 0x42403C00u;
    const uint32_t h0 = __builtin_amdgcn_perm(tab_hi, tab_lo, c0);
    const uint32_t h1 = __builtin_amdgcn_perm(tab_hi, tab_lo, c1);
    // (zero, high byte) pairs: selector byte 0x0C is the constant zero
    u32x4 r;
    r.x = __builtin_amdgcn_perm(h0, h0, 0x050C040Cu);  // weights 0, 1
    r.y = __builtin_amdgcn_perm(h0, h0, 0x070C060Cu);  // weights 2, 3
    r.z = __builtin_amdgcn_perm(h1, h1, 0x050C040Cu);
    r.w = __builtin_amdgcn_perm(h1, h1, 0x070C060Cu);
    return __builtin_bit_cast(half8, r);
}

// Non-linear 4-bit codes -> 16-bit floats of their table values (fp16 or
// bf16: both hold 8-bit integers exactly), from the two byte tables of an
// NlTab (low bytes of entries 0..15 in t[0..3], high bytes in t[4..7]).
// c: four codes 0..15, one per byte.  v_perm_b32 picks among 8 bytes, so
// entries 0..7 and 8..15 are looked up apart and bit 3 of each code chooses
// (m: 0xFF in the bytes whose code is 8..15; (t << 5) - (t >> 3) turns each
// set bit 3 into a full byte, with no carry between bytes).
__device__ __forceinline__ void nl_lookup(uint32_t c, const NlTab &tb, uint32_t &lo, uint32_t &hi) {
    const uint32_t s = c & 0x07070707u;
    const uint32_t t = c & 0x08080808u;
    const uint32_t m = (t << 5) - (t >> 3);
    const uint32_t l0 = __builtin_amdgcn_perm(tb.t[1], tb.t[0], s), l1 = __builtin_amdgcn_perm(tb.t[3], tb.t[2], s);
    const uint32_t h0 = __builtin_amdgcn_perm(tb.t[5], tb.t[4], s), h1 = __builtin_amdgcn_perm(tb.t[7], tb.t[6], s);
    lo = (l1 & m) | (l0 & ~m);
    hi = (h1 & m) | (h0 & ~m);
}

// Non-linear 4-bit: q = bytes qs[4g..4g+3] of one block -> 8 fp16 table
// values in the order of pos_in_block(4, g, .) (tb: fp16 byte tables).
__device__ __forceinline__ half8 unpack_nl4(uint32_t q, const NlTab &tb) {
    uint32_t l0, h0, l1, h1;
    nl_lookup(q & 0x0F0F0F0Fu, tb, l0, h0);         // weights 4g .. 4g+3 (low nibbles)
    nl_lookup((q >> 4) & 0x0F0F0F0Fu, tb, l1, h1);  // weights 16+4g .. 16+4g+3 (high nibbles)
    u32x4 r;  // (low byte, high byte) of two values per dword
    r.x = __builtin_amdgcn_perm(h0, l0, 0x06020400u);  // weights 4g, 4g+2
    r.y = __builtin_amdgcn_perm(h1, l1, 0x06020400u);  // 16+4g, 16+4g+2
    r.z = __builtin_amdgcn_perm(h0, l0, 0x07030501u);  // 4g+1, 4g+3
    r.w = __builtin_amdgcn_perm(h1, l1, 0x07030501u);  // 16+4g+1, 16+4g+3
    return __builtin_bit_cast(half8, r);
}

__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4v mfma16bf(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h16 & 0xFFFFu));
}

// Round-to-nearest-even fp32 -> fp16 bits.
__device__ __forceinline__ uint16_t f2h_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// fp32 -> bf16 bit pattern, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Orderable key of an fp32 value (larger float -> larger key), -0 == +0.
__device__ __forceinline__ uint32_t float_key(float v) {
    uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-workgroup handoff without cache-wide maintenance.  On gfx950 each
// XCD has its own L2, so an agent-scope release/acquire fence turns into an
// L2 write-back / invalidate of the whole XCD cache.  Instead the data that
// crosses workgroups is written and read with device-coherent (agent-scope)
// relaxed atomic accesses, a wave waits for its own stores to complete
// (s_waitcnt) before it raises a counter, and counters are polled with relaxed
// agent-scope loads.
// tagged words: fp32 value in the low half, a tag in the high half, read and
// written as one 64-bit access
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)tag << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The error word of a workspace (see DecodeParams::err): bit 0 = a bounded
// wait ran out, bit 1 = a given grouping was malformed; the bits stay set
// until the host clears them.  The word after it holds the tag of the last
// call whose wait ran out: that call's other waits end at once, while later
// calls (other tags) wait normally.
__device__ __forceinline__ void note_timeout(uint32_t *err, uint32_t tag) {
    atomicOr(err, 1u);
    store_dev_u32(err + 1, tag);
}
__device__ __forceinline__ bool call_timed_out(const uint32_t *err, uint32_t tag) {
    return ld_dev_u32(err + 1) == tag;
}
// LDS written by some lanes of a wave, then read by other lanes of it
__device__ __forceinline__ void wave_lds_handoff() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for LDS data only: the wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for the wave's
// outstanding direct-to-LDS loads (a workgroup-scope release fence counts
// them as LDS writes and waits for all of them), so loads issued ahead stay
// in flight across it.  Global memory written before it is not ordered by it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // (no earlier access moves below it)
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// LDS as an address-space-3 pointer: the form the direct-to-LDS loads
// (global_load_lds) take their destination in (from a generic pointer the
// compiler does not derive M0 correctly)
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// vmcnt-only wait: until at most N vector memory operations of this wave are
// outstanding (expcnt and lgkmcnt at their maxima: not waited on)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// the same for a wave-uniform count n (0 <= n; counts above 15 wait for 15)
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<1>(); break;
        case 2: wait_vm<2>(); break;
        case 3: wait_vm<3>(); break;
        case 4: wait_vm<4>(); break;
        case 5: wait_vm<5>(); break;
        case 6: wait_vm<6>(); break;
        case 7: wait_vm<7>(); break;
        case 8: wait_vm<8>(); break;
        case 9: wait_vm<9>(); break;
        case 10: wait_vm<10>(); break;
        case 11: wait_vm<11>(); break;
        case 12: wait_vm<12>(); break;
        case 13: wait_vm<13>(); break;
        case 14: wait_vm<14>(); break;
        default: wait_vm<15>(); break;
    }
}

// The call's tag source without a grid-wide counter: EPOCH_SLOTS words, all
// equal to the number of calls made on the workspace.  Workgroup b reads
// word b at its start and, at its end, writes the next value into every word
// i with i % G == b: each word is written by exactly one workgroup of a call
// (so no workgroup overwrites a word another one has yet to read), and after
// the call every word holds the next value whatever the grid size G (<=
// EPOCH_SLOTS), so launches of any grid sharing the workspace stay in step.
__device__ __forceinline__ uint32_t epoch_read(const uint32_t *epoch) { return ld_dev_u32(epoch + blockIdx.x); }
__device__ __forceinline__ void epoch_advance(uint32_t *epoch, uint32_t e) {
    for (int i = blockIdx.x; i < EPOCH_SLOTS; i += gridDim.x) store_dev_u32(epoch + i, e + 1u);
}

// ---------------------------------------------------------------------------
// Wave reductions on DPP (gfx9 row broadcasts); result valid in every lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Inclusive prefix sum over the 64 lanes (row shifts within rows of 16, then
// row broadcasts across rows).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Router for one row by one wave (E <= 64 * EPL): k rounds of a wave-wide
// argmax, an equal logit going to the lower expert id; softmax over the k.
// The logits load (route_keys) is separate from the selection (route_pick),
// so a wave can issue other loads in between.
// route_load + route_keys_of: the raw logits loads and their keys apart, so a
// wave can issue several rows' loads before it waits for the first.
template <int EPL>
__device__ __forceinline__ void route_load(const float *row, int E, int lane, float (&v)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = row[e < E ? e : 0];  // every lane loads (in bounds), so the loads issue as one sequence
    }
}
template <int EPL>
__device__ __forceinline__ void route_keys_of(const float (&v)[EPL], int E, int lane, uint32_t (&key)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i < E ? float_key(v[i]) : 0u;  // finite values: keys > 0
}
template <int EPL>
__device__ __forceinline__ void route_keys(const float *row, int E, int lane, uint32_t (&key)[EPL]) {
    float v[EPL];
    route_load<EPL>(row, E, lane, v);
    route_keys_of<EPL>(v, E, lane, key);
}

// key back to its fp32 value
__device__ __forceinline__ float key_value(uint32_t m) {
    return __builtin_bit_cast(float, (m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// Best key of a lane and its index i (the lowest i among equal keys): a
// tree of depth log2(EPL).
template <int EPL>
__device__ __forceinline__ void lane_best(const uint32_t (&key)[EPL], uint32_t &bk, int &bi) {
    uint32_t k1[EPL];
    int i1[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        k1[i] = key[i];
        i1[i] = i;
    }
#pragma unroll
    for (int w = 1; w < EPL; w *= 2)
#pragma unroll
        for (int i = 0; i + w < EPL; i += 2 * w) {
            const bool hi = k1[i + w] > k1[i];  // strict: the lower index keeps a tie
            k1[i] = hi ? k1[i + w] : k1[i];
            i1[i] = hi ? i1[i + w] : i1[i];
        }
    bk = k1[0];
    bi = i1[0];
}

// One selection round with branches (more than 4 keys per lane): the lane's
// best key, the wave's largest (DPP), its holder by ballot; the rare tie
// across lanes resolved by a second wave reduction over the holders' ids.
template <int EPL>
__device__ __forceinline__ int route_round(uint32_t (&key)[EPL], uint32_t &m, int lane) {
    uint32_t bk = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (key[i] > bk) {  // strict: the lowest i wins among equal keys
            bk = key[i];
            bi = i;
        }
    m = wave_max_u32(bk);
    const uint64_t tied = __ballot(bk == m);
    int e;
    if (__popcll(tied) == 1) {
        const int wl = __ffsll((unsigned long long)tied) - 1;
        e = wl + 64 * __builtin_amdgcn_readlane(bi, wl);
    } else {
        e = (int)wave_min_u32(bk == m ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu);
    }
    if ((e & 63) == lane) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == (e >> 6)) key[i] = 0u;
    }
    return e;
}

// k rounds of a wave-wide argmax.  Up to 4 keys per lane without branches:
// each lane's best key
// (tree), the wave's largest (DPP), and among the lanes holding it the
// lowest expert id (one ballot per key index: the lowest index with a
// holder, then the lowest lane); the winner's key is cleared.  The softmax
// numerators exp(l_j - l_0) and their sum (slot order 0, 1, ..., k-1) are
// formed as the rounds go (the same values and order in both forms);
// out_idx / out_w (LDS, k entries) receive slot j's expert and weight.
template <int EPL>
__device__ __forceinline__ void route_pick(uint32_t (&key)[EPL], int k, int *out_idx, float *out_w, int lane) {
    float mine = 0.0f, l0 = 0.0f, s = 0.0f;
    int mine_id = 0;
    if constexpr (EPL > 4) {
        // (the numerators after the rounds: lane j holds slot j's logit)
        for (int j = 0; j < k; ++j) {
            uint32_t m;
            const int e = route_round<EPL>(key, m, lane);
            if (lane == j) {
                mine = key_value(m);
                mine_id = e;
            }
        }
        l0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mine)));
        const float ex = lane < k ? expf(mine - l0) : 0.0f;
        for (int j = 0; j < k; ++j)
            s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
        if (lane < k) {
            out_idx[lane] = mine_id;
            out_w[lane] = ex / s;
        }
        return;
    }
    for (int j = 0; j < k; ++j) {
        uint32_t bk;
        int bi;
        lane_best<EPL>(key, bk, bi);
        const uint32_t m = wave_max_u32(bk);
        const uint64_t held = __ballot(bk == m);
        uint64_t win = 0;
        int wi = 0;
#pragma unroll
        for (int i = EPL - 1; i >= 0; --i) {
            const uint64_t t = held & __ballot(bi == i);
            win = t ? t : win;
            wi = t ? i : wi;
        }
        const int wl = (int)__builtin_ctzll(win);
        const bool me = lane == wl;
#pragma unroll
        for (int i = 0; i < EPL; ++i) key[i] = (me && i == wi) ? 0u : key[i];
        const float v = key_value(m);
        if (j == 0) l0 = v;
        const float ex = expf(v - l0);
        s += ex;
        mine = lane == j ? ex : mine;
        mine_id = lane == j ? wl + 64 * wi : mine_id;
    }
    if (lane < k) {
        out_idx[lane] = mine_id;
        out_w[lane] = mine / s;
    }
}


}  // namespace moe
