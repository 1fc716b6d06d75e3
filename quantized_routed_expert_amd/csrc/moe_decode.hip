// moe_decode.hip -- the routed-expert layer for decode windows (T <= 16 rows)
// in ONE kernel launch per layer on gfx950.
//
// Why one launch: the forum thread "把 Strata 搬上 SGLang 引擎 的嘗試" (§三,
// decode timing) measures that a single-expert call is dominated by launches
// and that grouping all of a layer's experts into one call is what makes
// decode fast; on MI355X a graph node costs about 1.5 us, comparable to the
// whole 24 MB weight stream of a decode layer, so route, group, the expert
// FFNs and the combine share one launch here.
//
// Structure (persistent grid, every workgroup resident):
//  A. every workgroup loads the rows' activations (all threads, one quant
//     block each) while the waves owning a row compute its routing (top-k of
//     the fp32 logits, ties to the lower id, softmax over the k selected;
//     wave reductions on DPP).  Grouping is a counting sort in LDS.  The
//     activations are stored in LDS as fp16 in each format's k order with a
//     per-token power-of-two scale (exact), so any bf16/fp32 range fits fp16.
//  B. gate/up tasks.  A unit is (expert, 16 feature rows, gate or up, one K
//     chunk of up to 32 quant blocks), one wave's work; a task is the units
//     that complete whole 16-feature groups, one workgroup's.  A wave streams
//     its unit's quantized rows from HBM with 16-byte loads (the next unit's
//     chunk in flight while the current one computes), passes them through a
//     wave-private LDS buffer into the MFMA lane layout, unpacks exact fp16
//     codes and runs v_mfma_f32_16x16x32_f16 with the expert's (<= 16) rows
//     as the M dimension: every weight byte is read once per window for all
//     rows that share the expert (the read-once-per-window rule of Strata
//     "Several requests at once", opening section).  The fp16 block scale
//     multiplies each block's fp32 partial.  The workgroup sums its units'
//     partials in LDS in a fixed order, applies SwiGLU in fp32, writes h as
//     tagged words and counts the task done for its expert.
//  C. down tiles (expert, 128 output rows), then combine items, continuing the
//     same round robin.  A tile's first weight chunk streams in during the
//     previous work item; the tile waits for its expert's tasks, stages h in
//     LDS as fp16 hi + lo (about 22 bits) with a per-token power-of-two
//     scale, streams the down rows and writes w * o per (token, slot) pair.
//     A combine item is 16 rows of one 128-row slice of y for every token:
//     it waits for the slice's count of finished experts and sums each
//     output in the fixed slot order (deterministic; no floating-point
//     atomics).

// Data crossing workgroups (partials, pair rows) uses device-coherent accesses
// and per-wave store completion instead of agent-scope fences, which on this
// chip would write back or invalidate a whole XCD's L2.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

#ifdef MOE_PHASE_TRACE
// Phase timestamps (100 MHz device clock) per workgroup, for analysis builds
// only.  The buffer pointer is read once at kernel start (TRACE_INIT), so a
// trace point adds no global load (and no wait on outstanding loads).
__device__ uint64_t *g_trace = nullptr;
#define TRACE_INIT volatile uint64_t *const trace_buf = g_trace
#define TRACE(slot)                                                                                        \
    do {                                                                                                   \
        if (trace_buf && threadIdx.x == 0) trace_buf[blockIdx.x * 128 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
// per wave (no wait of its own)
#define TRACEW(slot)                                                                                        \
    do {                                                                                                    \
        if (trace_buf && (threadIdx.x & 63) == 0)                                                           \
            trace_buf[blockIdx.x * 128 + 32 + (threadIdx.x >> 6) * 12 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define TRACE_INIT \
    do {           \
    } while (0)
#define TRACE(slot) \
    do {            \
    } while (0)
#define TRACEW(slot) \
    do {             \
    } while (0)
#endif

// ---------------------------------------------------------------------------
// Chunk streaming: 16 consecutive rows x cb blocks of one matrix, read with
// 16-byte loads (consecutive lanes on consecutive bytes of a row) and staged
// in a wave-private LDS buffer whose rows are rs bytes apart.
// ---------------------------------------------------------------------------
struct Chunk {
    u32x4 r[DEC_MAX_LD];
};

// Per-lane byte offsets of a chunk's pieces: in global memory (from the first
// row's segment start) and in the LDS buffer (-1: no piece for this lane; its
// load re-reads the lane's first piece, so every lane issues the same fixed
// sequence of loads and the waits on them can be counted).
struct ChunkMap {
    int g[DEC_MAX_LD];
    int l[DEC_MAX_LD];
};

// A chunk is nrows runs of per_row 16-byte pieces (7..36), row_bytes apart in
// global memory and rs apart in LDS; inv = 65536 / per_row + 1 (j / per_row
// exactly for the j < 576 used here).
__device__ __forceinline__ void chunk_map(ChunkMap &m, int nrows, int per_row, uint32_t inv, int rs, int row_bytes,
                                          int lane) {
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) {
        const int j = lane + 64 * u;
        const int r = (int)(((uint32_t)j * inv) >> 16);
        const int col = j - r * per_row;
        const bool ok = j < nrows * per_row;
        m.g[u] = ok ? r * row_bytes + col * 16 : m.g[0];
        m.l[u] = ok ? r * rs + col * 16 : -1;
    }
}

__device__ __forceinline__ void chunk_load(Chunk &c, const uint8_t *base, const ChunkMap &m) {
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) c.r[u] = *(const u32x4 *)(base + m.g[u]);
}

__device__ __forceinline__ void chunk_store(const Chunk &c, uint8_t *buf, const ChunkMap &m) {
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u)
        if (m.l[u] >= 0) *(u32x4 *)(buf + m.l[u]) = c.r[u];
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t *p) { return *(const uint32_t *)p; }

// ---------------------------------------------------------------------------
// MFMA operands from a staged chunk, two blocks (36 or 28 bytes, 4-byte
// aligned) at a time.  Lane layout: weight row n = lane % 16 of the chunk,
// k-group g = lane / 16.  All reads are aligned dwords; with the odd-granule
// row stride the 16 rows x 4 k-groups of one read fall in distinct banks.
// ---------------------------------------------------------------------------
template <int BITS>
struct BVal {
    half8 b;  // exact fp16 codes minus the bias
    float d;  // block scale
};

// A operands of blocks b, b+1.  Rows past the window's tokens read a valid
// row too: an MFMA output row depends on its own A row only, and those rows
// are never used.
template <int NP>
__device__ __forceinline__ void load_a(half8 (&a)[2][NP], const uint8_t *ab, int b, int a_stride, int part_off) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int xp = 0; xp < NP; ++xp) a[i][xp] = *(const half8 *)(ab + (b + i) * a_stride + xp * part_off);
}

template <int BITS, int NP>
struct Pair;

// 4-bit pair: block b = bytes 0..17 (scale 0-1, codes 2..17), block b+1 = 18..35.
template <int NP>
struct Pair<4, NP> {
    uint32_t d0, d4, w0, w1, w5;
    half8 a[2][NP];
    __device__ __forceinline__ void load(const uint8_t *buf, int ro, int p, int g, const uint8_t *ab, int a_stride,
                                         int part_off) {
        const int o = ro + 36 * p;
        d0 = lds_u32(buf + o);
        d4 = lds_u32(buf + o + 16);
        w0 = lds_u32(buf + o + 4 * g);
        w1 = lds_u32(buf + o + 4 * g + 4);
        w5 = lds_u32(buf + o + 20 + 4 * g);
        load_a<NP>(a, ab, 2 * p, a_stride, part_off);
    }
    __device__ __forceinline__ BVal<4> get(int i, int g, const NlTab &) const {
        BVal<4> v;
        if (i == 0) {
            v.b = unpack4(__builtin_amdgcn_alignbyte(w1, w0, 2u));  // code bytes 2+4g .. 5+4g
            v.d = half_bits_to_float(d0);
        } else {
            v.b = unpack4(w5);  // code bytes 20+4g .. 23+4g
            v.d = half_bits_to_float(d4 >> 16);
        }
        return v;
    }
};

// Non-linear 4-bit pair: the 4-bit pair's bytes, codes looked up in the table.
template <int NP>
struct Pair<MOE_FMT_NL4, NP> : Pair<4, NP> {
    __device__ __forceinline__ BVal<MOE_FMT_NL4> get(int i, int g, const NlTab &tb) const {
        BVal<MOE_FMT_NL4> v;
        if (i == 0) {
            v.b = unpack_nl4(__builtin_amdgcn_alignbyte(this->w1, this->w0, 2u), tb);
            v.d = half_bits_to_float(this->d0);
        } else {
            v.b = unpack_nl4(this->w5, tb);
            v.d = half_bits_to_float(this->d4 >> 16);
        }
        return v;
    }
};

// 3-bit pair: block b = bytes 0..13 (scale 0-1, low parts 2..9, third bits
// 10..13), block b+1 = 14..27 (scale, low parts 16..23, third bits 24..27).
template <int NP>
struct Pair<3, NP> {
    uint32_t w[7];
    half8 a[2][NP];
    __device__ __forceinline__ void load(const uint8_t *buf, int ro, int p, int g, const uint8_t *ab, int a_stride,
                                         int part_off) {
        const int o = ro + 28 * p;
#pragma unroll
        for (int i = 0; i < 7; ++i) w[i] = lds_u32(buf + o + 4 * i);
        load_a<NP>(a, ab, 2 * p, a_stride, part_off);
    }
    __device__ __forceinline__ BVal<3> get(int i, int g, const NlTab &) const {
        BVal<3> v;
        if (i == 0) {
            v.b = unpack3(__builtin_amdgcn_alignbyte(w[1], w[0], 2u), __builtin_amdgcn_alignbyte(w[2], w[1], 2u),
                          __builtin_amdgcn_alignbyte(w[3], w[2], 2u), (uint32_t)g);
            v.d = half_bits_to_float(w[0]);
        } else {
            v.b = unpack3(w[4], w[5], w[6], (uint32_t)g);
            v.d = half_bits_to_float(w[3] >> 16);
        }
        return v;
    }
};

// d * (A . B) of one block, before scaling; A given as NP fp16 parts.
template <int BITS, int NP>
__device__ __forceinline__ float4v block_dot(const BVal<BITS> &v, const half8 *a) {
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    float4v dd = mfma16(a[0], v.b, z);
    if constexpr (NP == 2) dd = mfma16(a[1], v.b, dd);
    return dd;
}

// The products of one pair of blocks, before their scales are applied.
struct PairDot {
    float4v d0, d1;
    float s0, s1;
};
template <int BITS, int NP>
__device__ __forceinline__ PairDot pair_dot(const Pair<BITS, NP> &pr, int g, const NlTab &tb) {
    const BVal<BITS> v0 = pr.get(0, g, tb), v1 = pr.get(1, g, tb);
    return PairDot{block_dot<BITS, NP>(v0, pr.a[0]), block_dot<BITS, NP>(v1, pr.a[1]), v0.d, v1.d};
}
// acc += s0 * d0 then s1 * d1 (the block order of the sum)
__device__ __forceinline__ void pair_apply(float4v &acc, const PairDot &q) {
    acc.x = fmaf(q.s0, q.d0.x, acc.x);
    acc.y = fmaf(q.s0, q.d0.y, acc.y);
    acc.z = fmaf(q.s0, q.d0.z, acc.z);
    acc.w = fmaf(q.s0, q.d0.w, acc.w);
    acc.x = fmaf(q.s1, q.d1.x, acc.x);
    acc.y = fmaf(q.s1, q.d1.y, acc.y);
    acc.z = fmaf(q.s1, q.d1.z, acc.z);
    acc.w = fmaf(q.s1, q.d1.w, acc.w);
}

// Multiply-accumulate a staged chunk of cb blocks (cb a multiple of 4) into
// acc: two operand sets, the reads of one pair in flight while the other
// pair computes, and each pair's scaled products added one pair later, after
// the next pair's MFMAs have issued (the blocks are still summed in order).
// A operands: ab points at this lane's first block, a_stride bytes between
// blocks, part_off bytes between the NP parts.
template <int BITS, int NP>
__device__ __forceinline__ void chunk_mma(float4v &acc, const uint8_t *buf, int rs, int cb, int n, int g,
                                          const uint8_t *ab, int a_stride, int part_off, const NlTab &tb) {
    const int ro = n * rs;
    const int np = cb >> 1;
    Pair<BITS, NP> pa, pb;
    pa.load(buf, ro, 0, g, ab, a_stride, part_off);
    pb.load(buf, ro, 1, g, ab, a_stride, part_off);
    PairDot qa = pair_dot<BITS, NP>(pa, g, tb);                        // pair 0
    pa.load(buf, ro, 2 < np ? 2 : 0, g, ab, a_stride, part_off);  // (np = 2: unused re-read)
    PairDot qb = pair_dot<BITS, NP>(pb, g, tb);                        // pair 1
    pair_apply(acc, qa);
    pb.load(buf, ro, 3 < np ? 3 : 0, g, ab, a_stride, part_off);
    for (int p = 2; p < np; p += 2) {
        qa = pair_dot<BITS, NP>(pa, g, tb);  // pair p
        pair_apply(acc, qb);             // pair p - 1
        pa.load(buf, ro, p + 2 < np ? p + 2 : 0, g, ab, a_stride, part_off);  // (last round: unused re-read)
        qb = pair_dot<BITS, NP>(pb, g, tb);  // pair p + 1
        pair_apply(acc, qa);             // pair p
        pb.load(buf, ro, p + 3 < np ? p + 3 : 0, g, ab, a_stride, part_off);
    }
    pair_apply(acc, qb);  // pair np - 1
}

// ---------------------------------------------------------------------------
// Down chunks (column-block-major weights): block j of row n sits at
// j*rs + n*bb, 4-byte aligned for even n and 2 bytes past that for odd n, so
// each read takes the dword below and shifts by the byte offset (0 or 2),
// which makes the instruction stream the same for both parities.
// ---------------------------------------------------------------------------
template <int BITS>
struct DnBlk;

template <>
struct DnBlk<4> {
    uint32_t dw, lo, hi;
    half8 a[2];
    __device__ __forceinline__ void load(const uint8_t *buf, int a0, int qa, const uint8_t *ab) {
        dw = lds_u32(buf + (a0 & ~3));  // scale
        lo = lds_u32(buf + qa);         // code bytes 4g.. of the block, from the dword at or below
        hi = lds_u32(buf + qa + 4);
        a[0] = *(const half8 *)ab;
        a[1] = *(const half8 *)(ab + 16);
    }
    __device__ __forceinline__ BVal<4> get(uint32_t sh_d, uint32_t sh_c) const {
        BVal<4> v;
        v.b = unpack4(__builtin_amdgcn_alignbyte(hi, lo, sh_c));
        v.d = half_bits_to_float(dw >> sh_d);
        return v;
    }
};

template <>
struct DnBlk<MOE_FMT_NL4> : DnBlk<4> {
    __device__ __forceinline__ BVal<MOE_FMT_NL4> get(uint32_t sh_d, uint32_t sh_c, const NlTab &tb) const {
        BVal<MOE_FMT_NL4> v;
        v.b = unpack_nl4(__builtin_amdgcn_alignbyte(hi, lo, sh_c), tb);
        v.d = half_bits_to_float(dw >> sh_d);
        return v;
    }
};

template <>
struct DnBlk<3> {
    uint32_t dw, r0, r1, r2, r3;
    half8 a[2];
    // qa: the dword at or below the block's first low-part byte
    __device__ __forceinline__ void load(const uint8_t *buf, int a0, int qa, const uint8_t *ab) {
        dw = lds_u32(buf + (a0 & ~3));       // scale
        r0 = lds_u32(buf + qa);              // low parts and third bits from the dwords at qa ..
        r1 = lds_u32(buf + qa + 4);
        r2 = lds_u32(buf + qa + 8);
        r3 = lds_u32(buf + (a0 & ~3) + 12);  // (odd rows: the last dword is r2 and r3 goes unused)
        a[0] = *(const half8 *)ab;
        a[1] = *(const half8 *)(ab + 16);
    }
    // sh_d: scale shift (bits); sh_c: byte offset of the low parts in r0
    __device__ __forceinline__ BVal<3> get(uint32_t sh_d, uint32_t sh_c, int g) const {
        BVal<3> v;
        v.d = half_bits_to_float(dw >> sh_d);
        v.b = unpack3(__builtin_amdgcn_alignbyte(r1, r0, sh_c), __builtin_amdgcn_alignbyte(r2, r1, sh_c),
                      __builtin_amdgcn_alignbyte(r3, r2, sh_c), (uint32_t)g);
        return v;
    }
};

// acc += sum over the chunk's cb blocks (cb even) of d_j * (h . codes_j) for
// weight row n; A operands (staged h, two fp16 parts 16 bytes apart) at
// ab + j*128.  Two operand sets: block j+1's reads in flight while j computes.
template <int BITS>
__device__ __forceinline__ void dn_chunk_mma(float4v &acc, const uint8_t *buf, int rs, int cb, int n, int g,
                                             const uint8_t *ab, const NlTab &tb) {
    constexpr int bb = blk_bytes(BITS);
    const int a0 = n * bb;                                   // block 0 of row n
    const uint32_t par = (uint32_t)(n & 1);                  // a0 mod 4 = 2 * par
    const uint32_t sh_d = 16u * par;
    const int q = a0 + 2 + (nib_layout(BITS) ? 4 * g : 0);   // first code / low-part byte of this lane
    const int qa = q & ~3;
    const uint32_t sh_c = (uint32_t)(q & 3);
    auto step = [&](const DnBlk<BITS> &b) {
        BVal<BITS> v;
        if constexpr (BITS == MOE_FMT_NL4) v = b.get(sh_d, sh_c, tb);
        else if constexpr (BITS == 4) v = b.get(sh_d, sh_c);
        else v = b.get(sh_d, sh_c, g);
        const float4v d = block_dot<BITS, 2>(v, b.a);
        acc.x = fmaf(v.d, d.x, acc.x);
        acc.y = fmaf(v.d, d.y, acc.y);
        acc.z = fmaf(v.d, d.z, acc.z);
        acc.w = fmaf(v.d, d.w, acc.w);
    };
    DnBlk<BITS> ba, bq;
    ba.load(buf, a0, qa, ab);
    for (int j = 0; j < cb; j += 2) {
        bq.load(buf + (j + 1) * rs, a0, qa, ab + (j + 1) * 128);
        step(ba);
        const int jn = j + 2 < cb ? j + 2 : 0;  // (last round: unused re-read)
        ba.load(buf + jn * rs, a0, qa, ab + jn * 128);
        step(bq);
    }
}

// ---------------------------------------------------------------------------
// Activation k-groups: the 8 values of (token t, block b, k-group g) that one
// MFMA lane of k-group g feeds, i.e. the block's weights at pos_in_block(g, e)
// e = 0..7.  4-bit: elements 4g+0..3 and 16+4g+0..3 (two loads); 3-bit:
// elements 8g+0..7 (one load).  The value of slot e is loaded value xslot(e)
// of the group.
// ---------------------------------------------------------------------------
template <int BITS>
__host__ __device__ constexpr int xslot(int e) {
    // pos_in_block(BITS, 0, e) -> its index among the loaded elements
    return nib_layout(BITS) ? (pos_in_block(4, 0, e) < 16 ? pos_in_block(4, 0, e) : pos_in_block(4, 0, e) - 12)
                     : pos_in_block(3, 0, e);
}

template <int BITS, int XPARTS>
struct XGroup {
    uint32_t w[4 * XPARTS];  // bf16: 8 values in 4 dwords; fp32: 8 dwords
    // row: the token's activations; base: element index 4g (4-bit) or 8g (3-bit) of block b
    __device__ __forceinline__ void load(const void *row, int base) {
        if constexpr (nib_layout(BITS)) {
            if constexpr (XPARTS == 1) {
                const uint2 a = *(const uint2 *)((const uint16_t *)row + base);
                const uint2 b = *(const uint2 *)((const uint16_t *)row + base + 16);
                w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
            } else {
                const u32x4 a = *(const u32x4 *)((const float *)row + base);
                const u32x4 b = *(const u32x4 *)((const float *)row + base + 16);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
            }
        } else {
            if constexpr (XPARTS == 1) {
                const u32x4 a = *(const u32x4 *)((const uint16_t *)row + base);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            } else {
                const u32x4 a = *(const u32x4 *)((const float *)row + base);
                const u32x4 b = *(const u32x4 *)((const float *)row + base + 4);
                w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
            }
        }
    }
    // loaded value s (0..7) as fp32
    __device__ __forceinline__ float val(int s) const {
        if constexpr (XPARTS == 1) return __builtin_bit_cast(float, (w[s >> 1] >> (16 * (s & 1))) << 16);
        else return __builtin_bit_cast(float, w[s]);
    }
    __device__ __forceinline__ float absmax() const {
        float m = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) m = fmaxf(m, fabsf(val(s)));
        return m;
    }
    // fp16 hi [and lo] of value * 2^sc in slot order e = 0..7 (ldexp: exact
    // for any sc, also where 2^sc itself is not a normal float)
    __device__ __forceinline__ void convert(int sc, u32x4 &hi, u32x4 &lo) const {
        uint32_t h[4], l[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float v0 = ldexpf(val(xslot<BITS>(2 * e2)), sc), v1 = ldexpf(val(xslot<BITS>(2 * e2 + 1)), sc);
            const _Float16 a0 = (_Float16)v0, a1 = (_Float16)v1;
            h[e2] = __builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
            l[e2] = f2h_bits(v0 - (float)a0) | ((uint32_t)f2h_bits(v1 - (float)a1) << 16);
        }
        hi = u32x4{h[0], h[1], h[2], h[3]};
        lo = u32x4{l[0], l[1], l[2], l[3]};
    }
};


// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// BG: bit width of the gate and up projections, BD: of the down projection
// (per-projection formats, as the thread's §三 decode table pairs them).
template <int BG, int BD, int XPARTS>
__global__ __launch_bounds__(DEC_THREADS, 1) void k_decode_layer(DecodeParams P) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = P.T, k = P.k, E = P.E, H = P.H;
    const int TK = T * k;
    const bool has_shared = (P.mode & DEC_MODE_SHARED) != 0;
    const int hs = has_shared ? 1 : 0;
    const int G = gridDim.x;

    int *s_idx = (int *)(smem + P.lds_idx);
    float *s_w = (float *)(smem + P.lds_w);
    int *s_sorted = (int *)(smem + P.lds_sorted);
    int *s_hist = (int *)(smem + P.lds_hist);
    int *s_slot_start = (int *)(smem + P.lds_slot_start);
    int *s_slot_exp = (int *)(smem + P.lds_slot_exp);
    int *s_slot_cnt = (int *)(smem + P.lds_slot_cnt);
    int *s_tsc = (int *)(smem + P.lds_tsc);  // per token: the power of two sc of its staged activations
    int *s_hsc = (int *)(smem + P.lds_hsc);  // per row of a down tile: that of its staged h
    uint32_t *s_xmax = (uint32_t *)(smem + P.lds_xmax);
    int *s_misc = (int *)(smem + P.lds_misc);
    uint8_t *s_xa = smem + P.lds_xa;
    uint8_t *s_chunk = smem + P.lds_chunk + wave * P.chunk_stride;

    // ---- gate/up geometry (host-computed): a unit is 16 feature rows x one K
    // chunk of one matrix (one wave); a task is the 8 (or 16) units that
    // complete whole 16-feature groups (one workgroup)
    constexpr int bbD = blk_bytes(BD);  // bytes of a down block
    const int cbH = P.cbH, segH = P.segH, rowH = P.rowH, rsH = P.rsH;
    const int lg_nchH = P.lg_nchH, lg_upt = P.lg_upt, lg_nfgT = P.lg_nfgT, rounds = P.rounds;
    const int nchH = 1 << lg_nchH, upt = 1 << lg_upt, nfgT = 1 << lg_nfgT;
    const int F = P.F, Fs = has_shared ? P.Fs : 0;
    const size_t eb = P.eb;  // routed expert blob bytes
    const int tasks_sh = has_shared ? P.tasks_sh : 0, tasks_rt = P.tasks_rt;
    const int n_lane = lane & 15, g_lane = lane >> 4;

    // token of pair p (p / k; the reciprocal does not cover k = 1)
    auto div_k = [&](int p) { return k == 1 ? p : (int)__umulhi((uint32_t)p, P.m_k); };
    ChunkMap mapH;
    chunk_map(mapH, 16, P.perH, P.invH, rsH, rowH, lane);
    // task -> (slot, index of the task within its slot)
    auto task_slot = [&](int task, int &tl) {
        if (task < tasks_sh) {
            tl = task;
            return 0;
        }
        const int v = task - tasks_sh, si = (int)__umulhi((uint32_t)v, P.m_tasks_rt);
        tl = v - si * tasks_rt;
        return hs + si;
    };
    // this wave's chunk of unit (task, round)
    auto unit_rows = [&](int task, int rho) -> const uint8_t * {
        int tl;
        const int s = task_slot(task, tl);
        const bool sh = task < tasks_sh;
        const int Fx = sh ? Fs : F;
        const uint8_t *blob = sh ? P.w_shared : P.w_routed + (size_t)s_slot_exp[s] * eb;
        const int ui = rho * 8 + wave;
        const int fl = ui >> lg_upt, rem = ui & (upt - 1);
        const int mat = rem >> lg_nchH, kc = rem & (nchH - 1);
        return blob + (size_t)mat * Fx * rowH + (size_t)((tl << lg_nfgT) + fl) * 16 * rowH + (size_t)kc * segH;
    };

    TRACE_INIT;
    TRACE(0);
    // ======================= Phase A: routing, activations, grouping =======================
    // Waits on loads are in issue order, so each wave issues first what it
    // needs first: the call's tag (see DecodeParams), then (routing waves) the
    // logits, then the activation groups, then the first weight chunk.
    const uint32_t tag_v = epoch_read(P.epoch);
    const bool route_mode = (P.mode & DEC_MODE_ROUTE) != 0;
    const int route_w = DEC_WAVES - 1 - wave;  // routing: row t by wave DEC_WAVES-1 - t % DEC_WAVES
    const bool routes = route_mode && route_w < T;

    // activation k-groups of this thread: group ((tid - 64) mod 512) + 512 q,
    // so a one-row window leaves waves 0 and 7 (grouping, routing) without any
    constexpr int XG = XPARTS == 1 ? DEC_XG_BF16 : DEC_XG_F32;
    const int ngrp_x = T * P.xgrp;
    const int nq = (ngrp_x + DEC_THREADS - 1) / DEC_THREADS;
    XGroup<BG, XPARTS> xg[XG];
    int xg_t[XG], xg_pos[XG];  // token, (4b + g) of each group (-1: none)
    auto issue_x = [&]() {
#pragma unroll
        for (int q = 0; q < XG; ++q) {
            if (q < nq) {
                const int grp = ((tid + DEC_THREADS - 64) & (DEC_THREADS - 1)) + DEC_THREADS * q;
                const bool ok = grp < ngrp_x;
                const int gc = ok ? grp : 0;  // (an in-bounds load for lanes without a group)
                const int t = (int)__umulhi((uint32_t)gc, P.m_xgrp);
                const int rem = gc - t * P.xgrp;  // 4 b + g
                const int base = (rem >> 2) * 32 + (nib_layout(BG) ? 4 : 8) * (rem & 3);
                xg[q].load((const uint8_t *)P.x + (size_t)t * H * (XPARTS == 1 ? 2 : 4), base);
                xg_t[q] = ok ? t : -1;
                xg_pos[q] = rem;
            }
        }
    };

    Chunk c;
    bool pref = false;
    const bool shared_first = (int)blockIdx.x < tasks_sh;  // its first unit depends on no routing
    // routing by ranks (small T*E): every thread takes part; the keys and the
    // selected logits sit in the chunk buffers, unused until the gate/up phase
    const bool rank_mode = route_mode && P.route_rank;
    const int nkeys = T * E;
    uint32_t *s_keys = (uint32_t *)(smem + P.lds_chunk);
    float *s_lg = (float *)(smem + P.lds_chunk + (size_t)nkeys * 4);
    TRACEW(6);
    if (rank_mode) {
        constexpr int NL = DEC_RANK_MAX_KEYS / DEC_THREADS;
        const int nl = (nkeys + DEC_THREADS - 1) / DEC_THREADS;
        float lv[NL];
#pragma unroll
        for (int r = 0; r < NL; ++r)
            if (r < nl) lv[r] = P.logits[tid + DEC_THREADS * r < nkeys ? tid + DEC_THREADS * r : 0];
        issue_x();
#pragma unroll
        for (int r = 0; r < NL; ++r)
            if (r < nl && tid + DEC_THREADS * r < nkeys) s_keys[tid + DEC_THREADS * r] = float_key(lv[r]);
    } else if (routes) {
        const int epl = (E + 63) >> 6;
        auto route_wave = [&](auto epl_c) {
            constexpr int EPL = decltype(epl_c)::value;
            // both rows' logits (windows of up to 16 rows) in flight together
            const int t2 = route_w + DEC_WAVES;
            float v1[EPL], v2[EPL];
            uint32_t key[EPL];
            route_load<EPL>(P.logits + (size_t)route_w * E, E, lane, v1);
            if (t2 < T) route_load<EPL>(P.logits + (size_t)t2 * E, E, lane, v2);
            issue_x();
            route_keys_of<EPL>(v1, E, lane, key);
            route_pick<EPL>(key, k, s_idx + route_w * k, s_w + route_w * k, lane);
            if (t2 < T) {
                route_keys_of<EPL>(v2, E, lane, key);
                route_pick<EPL>(key, k, s_idx + t2 * k, s_w + t2 * k, lane);
            }
            for (int t = t2 + DEC_WAVES; t < T; t += DEC_WAVES) {
                route_keys<EPL>(P.logits + (size_t)t * E, E, lane, key);
                route_pick<EPL>(key, k, s_idx + t * k, s_w + t * k, lane);
            }
        };
        if (epl <= 2) route_wave(std::integral_constant<int, 2>{});
        else if (epl <= 4) route_wave(std::integral_constant<int, 4>{});
        else if (epl <= 8) route_wave(std::integral_constant<int, 8>{});
        else route_wave(std::integral_constant<int, 16>{});
        TRACEW(7);
    } else {
        issue_x();
    }
    if (shared_first) {
        chunk_load(c, unit_rows(blockIdx.x, 0), mapH);
        pref = true;
    }
    // (cleared only now: the loads above go out first)
    for (int i = tid; i < T; i += DEC_THREADS) s_xmax[i] = 0u;
    if (route_mode)
        for (int e = tid; e <= E; e += DEC_THREADS) s_hist[e] = 0;  // token masks
    __syncthreads();
    // per-token max |x| (the wait covers the tag, logits and activation
    // loads); reduced over the wave first when all its lanes hold one token
    const bool wave_tok = (P.xgrp & 63) == 0;
#pragma unroll
    for (int q = 0; q < XG; ++q) {
        if (q < nq) {
            const uint32_t mb = xg_t[q] >= 0 ? __builtin_bit_cast(uint32_t, xg[q].absmax()) : 0u;
            if (wave_tok) {
                const uint32_t wm = wave_max_u32(mb);
                if (lane == 0 && xg_t[q] >= 0) atomicMax(&s_xmax[xg_t[q]], wm);
            } else if (xg_t[q] >= 0) {
                atomicMax(&s_xmax[xg_t[q]], mb);
            }
        }
    }
    TRACEW(8);
    __syncthreads();  // routing and the token maxima complete
    const uint32_t tag = decode_tag(__builtin_amdgcn_readfirstlane(tag_v));  // this call's tag (see DecodeParams)
    TRACE(9);
    if (rank_mode) {
        // rank of logit (t, e) in its row: keys above it, plus equal keys of a
        // lower id (so an equal logit goes to the lower id); 2^lg_tpi threads
        // per logit, each over a contiguous part of the row, summed by DPP
        const int lg_tpi = P.lg_tpi, tpi = 1 << lg_tpi;
        const int per = E >> lg_tpi, sub = tid & (tpi - 1), j0 = sub * per;
        for (int item = tid >> lg_tpi; item < nkeys; item += DEC_THREADS >> lg_tpi) {
            const int t = (int)__umulhi((uint32_t)item, P.m_E), e = item - t * E;
            const uint32_t key = s_keys[item];
            const uint32_t *row = s_keys + t * E + j0;
            int cnt = 0;
            for (int j = 0; j < per; j += 4) {
                const u32x4 kv = *(const u32x4 *)(row + j);
                const int jj = j0 + j;
                cnt += (kv.x > key) + (kv.y > key) + (kv.z > key) + (kv.w > key);
                cnt += (kv.x == key && jj < e) + (kv.y == key && jj + 1 < e) + (kv.z == key && jj + 2 < e) +
                       (kv.w == key && jj + 3 < e);
            }
            if (tpi >= 2) cnt += __builtin_amdgcn_update_dpp(0, cnt, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
            if (tpi >= 4) cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
            if (tpi >= 8) cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x141, 0xF, 0xF, false);  // row_half_mirror
            if (tpi >= 16) cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x140, 0xF, 0xF, false); // row_mirror
            if (sub == 0 && cnt < k) {
                s_idx[t * k + cnt] = e;
                s_lg[t * k + cnt] = __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
            }
        }
        __syncthreads();
        // softmax over the k selected logits of the row (sum in slot order)
        for (int p = tid; p < TK; p += DEC_THREADS) {
            const int t = div_k(p);
            const float *lr = s_lg + t * k;
            const float l0 = lr[0];
            float sum = 0.0f;
            for (int j = 0; j < k; ++j) sum += expf(lr[j] - l0);
            s_w[p] = expf(s_lg[p] - l0) / sum;
        }
    }

    // Activations to fp16 (hi [+ lo]) of x * 2^sc_t in the format's k order:
    // part p, token t, block b, k-group g at p*T*x_rs + t*x_rs + (4b+g)*16.
    auto stage_x = [&]() {
#pragma unroll
        for (int q = 0; q < XG; ++q) {
            if (q < nq && xg_t[q] >= 0) {
                const int t = xg_t[q];
                const float mx = __builtin_bit_cast(float, s_xmax[t]);
                int ex = 0;
                if (mx > 0.0f) frexpf(mx, &ex);
                const int sc = mx > 0.0f ? 14 - ex : 0;  // max * 2^sc in [2^13, 2^14)
                if (xg_pos[q] == 0) s_tsc[t] = sc;
                u32x4 hi, lo;
                xg[q].convert(sc, hi, lo);
                uint8_t *dst = s_xa + (size_t)t * P.x_rs + (size_t)xg_pos[q] * 16;
                *(u32x4 *)dst = hi;
                if (XPARTS == 2) *(u32x4 *)(dst + (size_t)T * P.x_rs) = lo;
            }
        }
    };

    // grouping of the pairs by expert: slots in ascending expert id, pairs of
    // a slot in (token, slot) order.  A token's k experts are distinct, so an
    // expert's pairs are identified by a mask of its tokens: the pair of
    // token t sits at the expert's start + the number of earlier tokens.
    if (route_mode) {
        uint32_t *s_tmask = (uint32_t *)s_hist;  // [E] tokens that chose expert e
        int *s_start = s_sorted + TK;            // [E] first position of expert e
        for (int p = tid; p < TK; p += DEC_THREADS)
            atomicOr(&s_tmask[s_idx[p]], 1u << div_k(p));
        __syncthreads();
        if (wave == 0) {
            // exclusive scan of (count | active flag << 16) over the experts
            const int per = (E + 63) / 64;
            const int base = lane * per;
            int sum = 0;
            for (int i = 0; i < per; ++i) {
                const int e = base + i;
                if (e < E) {
                    const int cnt = __popc(s_tmask[e]);
                    sum += cnt | ((cnt > 0) << 16);
                }
            }
            const int incl = wave_incl_scan(sum);
            int run = incl - sum;
            for (int i = 0; i < per; ++i) {
                const int e = base + i;
                if (e < E) {
                    const int cnt = __popc(s_tmask[e]);
                    const int off = run & 0xFFFF, act = run >> 16;
                    if (cnt > 0) {
                        s_slot_exp[hs + act] = e;
                        s_slot_start[hs + act] = off;
                        s_slot_cnt[hs + act] = cnt;
                    }
                    s_start[e] = off;
                    run += cnt | ((cnt > 0) << 16);
                }
            }
            if (lane == 63) s_misc[0] = hs + (incl >> 16);  // number of slots
        }
        stage_x();  // (wave 0 after its scan; it holds groups only for windows of 2+ rows)
        __syncthreads();
        for (int p = tid; p < TK; p += DEC_THREADS) {
            const int e = s_idx[p], t = div_k(p);
            s_sorted[s_start[e] + __popc(s_tmask[e] & ((1u << t) - 1u))] = p;
        }
        if (blockIdx.x == 0) {
            for (int p = tid; p < TK; p += DEC_THREADS) {
                if (P.topk_idx_out) P.topk_idx_out[p] = s_idx[p];
                if (P.topk_w_out) P.topk_w_out[p] = s_w[p];
                if (P.heat) atomicAdd(&P.heat[s_idx[p]], 1);  // routing heat (integer adds: any order)
            }
        }
    } else {
        // a grouping given by the caller: sanitized so that bad entries give a
        // wrong answer (and err bit 1) but never an access out of bounds
        if (tid == 0) {
            int na = P.g_active[0];
            const int lim = min(E, TK);
            if (na < 0 || na > lim) {
                atomicOr(P.err, 2u);
                na = na < 0 ? 0 : lim;
            }
            s_misc[0] = hs + na;
        }
        stage_x();
        __syncthreads();
        const int na = s_misc[0] - hs;
        for (int a = tid; a < na; a += DEC_THREADS) {
            int e = P.g_active[1 + a];
            int st = 0, cnt = 0;
            if (e >= 0 && e < E) {
                st = P.g_offsets[e];
                cnt = P.g_offsets[e + 1] - st;
            }
            if (e < 0 || e >= E || st < 0 || cnt < 0 || cnt > MOE_DECODE_ROWS_DEV || st + cnt > TK) {
                atomicOr(P.err, 2u);
                e = (e >= 0 && e < E) ? e : 0;
                st = 0;
                cnt = 0;
            }
            s_slot_exp[hs + a] = e;
            s_slot_start[hs + a] = st;
            s_slot_cnt[hs + a] = cnt;
        }
        for (int q = tid; q < TK; q += DEC_THREADS) {
            int p = P.g_pairs[q];
            if (p < 0 || p >= TK) {
                atomicOr(P.err, 2u);
                p = 0;
            }
            s_sorted[q] = p;
        }
        for (int p = tid; p < TK; p += DEC_THREADS) s_w[p] = P.g_pair_w ? P.g_pair_w[p] : 1.0f;
    }
    if (tid == 0 && has_shared) {
        s_slot_exp[0] = -1;
        s_slot_start[0] = 0;
        s_slot_cnt[0] = T;
    }
    __syncthreads();  // slot tables and staged activations complete
    TRACE(13);
    const int n_slots = s_misc[0];
    const int n_tasks = tasks_sh + (n_slots - hs) * tasks_rt;

    // Down tiles (slot, 128 output rows) continue the round robin of the
    // gate/up tasks over the workgroups: tile i is work item n_tasks + i.
    // The round robin decides how many tiles a workgroup takes; which ones is
    // a contiguous run of the (slot-major) tile list, so that its tiles share
    // a slot and its staged h: workgroup r of the round robin, taking c_r =
    // n_tiles / G tiles (one more for r < n_tiles % G), takes the run that
    // starts after those of the workgroups before it.
    const int tiles_per_slot = P.tps;
    const int n_tiles = n_slots * tiles_per_slot;
    const int first_tile = (int)(((long long)blockIdx.x - n_tasks % G + G) % G);
    const int tl_m1 = n_tiles / G, tl_e = n_tiles - tl_m1 * G;
    const int tl_start = first_tile * tl_m1 + min(first_tile, tl_e);
    auto run_tile = [&](int ti) { return tl_start + (ti - first_tile) / G; };  // (ti < n_tiles, ti = first_tile mod G)
    struct Tile {
        const uint8_t *rows;  // this wave's 16 down rows
        int s, rg, Fx, cbF, nchF, segF, rowF, rsF, perF;
        uint32_t invF, m_ngrp;
        bool shared;
    };
    auto tile_of = [&](int ti) {
        Tile t;
        t.s = (int)__umulhi((uint32_t)ti, P.m_tps);
        t.rg = ti - t.s * tiles_per_slot;
        t.shared = s_slot_exp[t.s] < 0;
        const int i = t.shared ? 1 : 0;
        t.Fx = i ? P.fx[1] : P.fx[0];
        t.cbF = i ? P.cbF[1] : P.cbF[0];
        t.nchF = i ? P.nchF[1] : P.nchF[0];
        t.segF = i ? P.segF[1] : P.segF[0];
        t.rowF = i ? P.rowF[1] : P.rowF[0];
        t.rsF = i ? P.rsF[1] : P.rsF[0];
        t.perF = i ? P.perF[1] : P.perF[0];
        t.invF = i ? P.invF[1] : P.invF[0];
        t.m_ngrp = i ? P.m_ngrp[1] : P.m_ngrp[0];
        const uint8_t *blob = t.shared ? P.w_shared : P.w_routed + (size_t)s_slot_exp[t.s] * eb;
        // column-block-major down: this wave's 16 rows of column block 0
        t.rows = blob + (size_t)2 * t.Fx * rowH + (size_t)(t.rg * DEC_DN_ROWS + wave * 16) * bbD;
        return t;
    };
    // The first down chunk streams in as soon as the registers are free: here
    // for a workgroup without gate/up work, else during its last gate/up unit.
    ChunkMap mapF;
    int map_fx = -1;
    bool c_holds_tile = false;
    auto prefetch_first_tile = [&]() {
        if (first_tile < n_tiles) {
            const Tile t = tile_of(run_tile(first_tile));
            chunk_map(mapF, t.cbF, t.perF, t.invF, t.rsF, t.rowF, lane);
            map_fx = t.Fx;
            chunk_load(c, t.rows, mapF);
            c_holds_tile = true;
        }
    };
    if (!pref) {
        TRACEW(0);
        if ((int)blockIdx.x < n_tasks) chunk_load(c, unit_rows(blockIdx.x, 0), mapH);
        else prefetch_first_tile();
    }
    TRACEW(9);
    TRACE(2);

    // ======================= Phase B: gate/up tasks =======================
    bool first_task = true;
    for (int task = blockIdx.x; task < n_tasks; task += G) {
        int tl;
        const int s = task_slot(task, tl);
        const int n_tok = s_slot_cnt[s];
        const bool shared_slot = s_slot_exp[s] < 0;
        const int mrow = n_lane < n_tok ? n_lane : 0;  // A row of this lane (rows past n_tok: any valid row)
        const int tok = shared_slot ? mrow : div_k(s_sorted[s_slot_start[s] + mrow]);
        float4v accr[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        for (int rho = 0; rho < rounds; ++rho) {
            const int kc = (rho * 8 + wave) & (nchH - 1);
            __builtin_amdgcn_wave_barrier();
            chunk_store(c, s_chunk, mapH);
            if (first_task && rho == 0) TRACEW(1);
            wave_lds_handoff();
            // the registers are free again: the next unit's chunk streams in while this one computes
            int nt = task, nr = rho + 1;
            if (nr == rounds) {
                nt += G;
                nr = 0;
            }
            if (nt < n_tasks) chunk_load(c, unit_rows(nt, nr), mapH);
            else prefetch_first_tile();
            const uint8_t *ab = s_xa + (size_t)tok * P.x_rs + (size_t)(kc * cbH) * 64 + g_lane * 16;
            if (first_task && rho == 0) TRACEW(10);
            // (a register array indexed by rho would be read and written through
            // select chains over all its elements)
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            chunk_mma<BG, XPARTS>(acc, s_chunk, rsH, cbH, n_lane, g_lane, ab, 64, T * P.x_rs, P.nl);
            if (rho == 0) accr[0] = acc;
            else accr[1] = acc;
            if (first_task && rho == 0) TRACEW(11);
        }
        if (first_task) TRACEW(2);
        // unit partials (token m, feature n) into this wave's LDS buffer: round rho at [rho][m][n]
        float *sp = (float *)s_chunk;
#pragma unroll
        for (int rho = 0; rho < 2; ++rho) {
            if (rho < rounds) {
                sp[rho * 256 + (4 * g_lane + 0) * 16 + n_lane] = accr[rho].x;
                sp[rho * 256 + (4 * g_lane + 1) * 16 + n_lane] = accr[rho].y;
                sp[rho * 256 + (4 * g_lane + 2) * 16 + n_lane] = accr[rho].z;
                sp[rho * 256 + (4 * g_lane + 3) * 16 + n_lane] = accr[rho].w;
            }
        }
        __syncthreads();
        if (first_task) TRACEW(3);
        // h = silu(g) * u per (feature group, token, feature): K chunks summed
        // in order 0, 1, ...; back in the units of x; stored as tagged words in
        // the down projection's k order.  The count goes up without waiting for
        // the stores: a reader checks each word's tag.
        for (int i = tid; i < nfgT * 256; i += DEC_THREADS) {
            const int fl = i >> 8, m = (i >> 4) & 15, n = i & 15;
            if (m >= n_tok) continue;
            float gs = 0.0f, us = 0.0f;
            for (int kc = 0; kc < nchH; ++kc) {
                const int ug = fl * upt + kc, uu = ug + nchH;
                gs += *(const float *)(smem + P.lds_chunk + (ug & 7) * P.chunk_stride + ((ug >> 3) * 256 + m * 16 + n) * 4);
                us += *(const float *)(smem + P.lds_chunk + (uu & 7) * P.chunk_stride + ((uu >> 3) * 256 + m * 16 + n) * 4);
            }
            const int tk = shared_slot ? m : div_k(s_sorted[s_slot_start[s] + m]);
            const int tsc = s_tsc[tk];
            const float gv = ldexpf(gs, -tsc), uv = ldexpf(us, -tsc);
            const float h = gv / (1.0f + expf(-gv)) * uv;
            const int f = ((tl << lg_nfgT) + fl) * 16 + n;
            int pg, pe;
            group_slot_of(BD, f & 31, pg, pe);
            const int fo = (f >> 5) * 32 + pg * 8 + pe;
            const int row = shared_slot ? TK + m : s_slot_start[s] + m;
            st_tagged(P.hll + (size_t)row * P.h_stride + fo, h, tag);
        }
        __syncthreads();  // the unit partials have been read: the buffers are free again
        if (tid == 0) add_dev(&P.gu_count[s * DEC_CSTRIDE], 1u);
        if (first_task) TRACEW(4);
        first_task = false;
    }
    TRACE(3);

    // ======================= Phase C: down + weighted write + combine =======================
    // Combine items follow the down tiles in the same round robin (so they go
    // to the workgroups with one tile fewer): item ci = part ci % DEC_COMB_PARTS
    // of 128-row slice ci / DEC_COMB_PARTS, i.e. DEC_DN_ROWS / DEC_COMB_PARTS
    // rows of y for every token: ((w0 o0 + w1 o1) + ...) + shared.  It waits
    // for the slice's count of finished slots, loads every (term, output) word
    // of its rows (DEC_COMB_LOADS per thread in flight together), checks each
    // for this call's tag and parks it in LDS (the staged h and the chunk
    // buffers are free: these items come after the workgroup's tiles), then
    // sums each output in the fixed order.  The last part of a slice returns
    // the slice's counters to zero.
    constexpr int CROWS = DEC_DN_ROWS / DEC_COMB_PARTS;
    const int n_comb = (P.mode & DEC_MODE_COMBINE) ? tiles_per_slot * DEC_COMB_PARTS : 0;
    auto combine_part = [&](int ci) {
        const int crg = ci / DEC_COMB_PARTS, row0 = crg * DEC_DN_ROWS + (ci - crg * DEC_COMB_PARTS) * CROWS;
        uint32_t *cnt = &P.slice_count[crg * DEC_CSTRIDE];
        if (tid == 0) {
            uint32_t spins = 0;
            while (ld_dev_u32(cnt) < (uint32_t)n_slots) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > DEC_SPIN_LIMIT || call_timed_out(P.err, tag)) {
                    note_timeout(P.err, tag);
                    break;
                }
            }
        }
        __syncthreads();
        const int nterm = k + hs;
        const int nout = T * CROWS;
        float *s_terms = (float *)(smem + P.lds_xa);
        const int ob = min(nout, ((P.lds_total - P.lds_xa) >> 2) / nterm);
        for (int o0 = 0; o0 < nout; o0 += ob) {
            const int nb = min(ob, nout - o0);
            const int nw = nterm * nb;
            auto src_of = [&](int i) {
                const int j = i / nb, o = o0 + (i - j * nb);
                const int t = o / CROWS;
                return P.oll + (size_t)(j < k ? t * k + j : TK + t) * H + row0 + (o - t * CROWS);
            };
            for (int i0 = 0; i0 < nw; i0 += DEC_COMB_LOADS * DEC_THREADS) {
                uint64_t wd[DEC_COMB_LOADS];
#pragma unroll
                for (int q = 0; q < DEC_COMB_LOADS; ++q) {
                    const int i = i0 + q * DEC_THREADS + tid;
                    wd[q] = i < nw ? ld_dev_u64(src_of(i)) : 0;
                }
#pragma unroll
                for (int q = 0; q < DEC_COMB_LOADS; ++q) {
                    const int i = i0 + q * DEC_THREADS + tid;
                    if (i < nw) {
                        for (uint32_t spins = 0; (uint32_t)(wd[q] >> 32) != tag; ++spins) {
                            if (spins > DEC_SPIN_LIMIT) {
                                note_timeout(P.err, tag);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                            wd[q] = ld_dev_u64(src_of(i));
                        }
                        s_terms[i] = __builtin_bit_cast(float, (uint32_t)wd[q]);
                    }
                }
            }
            __syncthreads();
            for (int ol = tid; ol < nb; ol += DEC_THREADS) {
                const int o = o0 + ol;
                const int t = o / CROWS;
                float acc2 = s_terms[ol];
                for (int j = 1; j < nterm; ++j) acc2 += s_terms[j * nb + ol];  // ((w0 o0 + w1 o1) + ...) + shared
                P.y[(size_t)t * H + row0 + (o - t * CROWS)] = acc2;
            }
            __syncthreads();  // the terms are read before the next batch or item reuses the LDS
        }
        if (tid == 0 && add_dev(cnt + 1, 1u) == (uint32_t)(DEC_COMB_PARTS - 1)) {
            store_dev_u32(cnt, 0u);
            store_dev_u32(cnt + 1, 0u);
        }
    };
    // Thread 0 counts each finished tile and acts on the returned count of its
    // slot one tile later, so that the round trip overlaps the next tile.
    uint32_t p_dn = 0;
    int p_s = -1;
    auto settle = [&]() {
        if (p_s >= 0 && p_dn == (uint32_t)(tiles_per_slot - 1)) {
            // every tile of this slot has passed its wait: the counters can return to zero
            store_dev_u32(&P.gu_count[p_s * DEC_CSTRIDE], 0u);
            store_dev_u32(&P.dn_count[p_s * DEC_CSTRIDE], 0u);
        }
        p_s = -1;
    };
    int cur_slot = -1;
    bool c_next = c_holds_tile;  // c holds this tile's first chunk (loaded during the previous work item)
    for (int ti = first_tile; ti < n_tiles + n_comb; ti += G) {
        if (ti >= n_tiles) {
            combine_part(ti - n_tiles);
            continue;
        }
        const Tile tl = tile_of(run_tile(ti));
        const int s = tl.s, rg = tl.rg, Fx = tl.Fx;
        const bool shared_slot = tl.shared;
        const int cbF = tl.cbF, nchF = tl.nchF, segF = tl.segF, rsF = tl.rsF;
        const uint8_t *rows_d = tl.rows;
        if (Fx != map_fx) {
            chunk_map(mapF, cbF, tl.perF, tl.invF, rsF, tl.rowF, lane);
            map_fx = Fx;
        }
        const int n_tok = s_slot_cnt[s];
        if (!c_next) chunk_load(c, rows_d, mapF);  // before the wait
        c_next = false;

        if (s != cur_slot) {
            if (tid < T) s_xmax[tid] = 0u;
            __syncthreads();  // previous tile's readers of the staged h are done
            if (ti == first_tile) TRACE(4);
            if (tid == 0) {
                const uint32_t need = (uint32_t)(Fx >> (4 + lg_nfgT));
                uint32_t spins = 0;
                while (ld_dev_u32(&P.gu_count[s * DEC_CSTRIDE]) < need) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > DEC_SPIN_LIMIT || call_timed_out(P.err, tag)) {
                        note_timeout(P.err, tag);
                        break;
                    }
                }
            }
            __syncthreads();
            if (ti == first_tile) TRACE(5);
            // stage h * 2^sc_m (per-row power of two) as fp16 hi + lo: row m at
            // m*h_rs, k-group gi (8 values) at gi*32 (hi 16 B, lo 16 B)
            const int row0 = shared_slot ? TK : s_slot_start[s];
            const int ngrp = Fx >> 3;
            const int nit = n_tok * ngrp;
            // every item's words are loaded before any is checked (one round trip)
            float hv[4][8];
            uint64_t wd[4][8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int it = tid + DEC_THREADS * q;
                if (it < nit) {
                    const int m = (int)__umulhi((uint32_t)it, tl.m_ngrp), gi = it - m * ngrp;
                    const uint64_t *src = P.hll + (size_t)(row0 + m) * P.h_stride + gi * 8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) wd[q][e] = ld_dev_u64(src + e);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int it = tid + DEC_THREADS * q;
                if (it < nit) {
                    const int m = (int)__umulhi((uint32_t)it, tl.m_ngrp), gi = it - m * ngrp;
                    const uint64_t *src = P.hll + (size_t)(row0 + m) * P.h_stride + gi * 8;
                    for (uint32_t spins = 0;; ++spins) {  // until every word carries this call's tag
                        bool ok = true;
#pragma unroll
                        for (int e = 0; e < 8; ++e) ok = ok && (uint32_t)(wd[q][e] >> 32) == tag;
                        if (ok) break;
                        if (spins > DEC_SPIN_LIMIT) {
                            note_timeout(P.err, tag);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
#pragma unroll
                        for (int e = 0; e < 8; ++e) wd[q][e] = ld_dev_u64(src + e);
                    }
                    float mx = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        hv[q][e] = __builtin_bit_cast(float, (uint32_t)wd[q][e]);
                        mx = fmaxf(mx, fabsf(hv[q][e]));
                    }
                    atomicMax(&s_xmax[m], __builtin_bit_cast(uint32_t, mx));
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int it = tid + DEC_THREADS * q;
                if (it < nit) {
                    const int m = (int)__umulhi((uint32_t)it, tl.m_ngrp), gi = it - m * ngrp;
                    const float mx = __builtin_bit_cast(float, s_xmax[m]);
                    int ex = 0;
                    if (mx > 0.0f) frexpf(mx, &ex);
                    const int sc = mx > 0.0f ? 14 - ex : 0;
                    if (gi == 0) s_hsc[m] = sc;
                    uint32_t h4[4], l4[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const float v0 = ldexpf(hv[q][2 * e2], sc), v1 = ldexpf(hv[q][2 * e2 + 1], sc);
                        const _Float16 a0 = (_Float16)v0, a1 = (_Float16)v1;
                        h4[e2] = __builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                        l4[e2] = f2h_bits(v0 - (float)a0) | ((uint32_t)f2h_bits(v1 - (float)a1) << 16);
                    }
                    uint8_t *dst = s_xa + (size_t)m * P.h_rs + (size_t)gi * 32;
                    *(u32x4 *)dst = u32x4{h4[0], h4[1], h4[2], h4[3]};
                    *(u32x4 *)(dst + 16) = u32x4{l4[0], l4[1], l4[2], l4[3]};
                }
            }
            __syncthreads();
            if (ti == first_tile) TRACE(6);
            cur_slot = s;
        }

        float4v acc = {0.f, 0.f, 0.f, 0.f};
        const uint8_t *ab = s_xa + (size_t)(n_lane < n_tok ? n_lane : 0) * P.h_rs + g_lane * 32;
        for (int ci = 0; ci < nchF; ++ci) {
            __builtin_amdgcn_wave_barrier();
            chunk_store(c, s_chunk, mapF);
            if (ti == first_tile && ci == 0) TRACEW(5);
            wave_lds_handoff();
            if (ci + 1 < nchF) {
                chunk_load(c, rows_d + (size_t)(ci + 1) * segF, mapF);
            } else if (ti + G < n_tiles) {
                // the next tile's first chunk streams in while this one computes
                // (same chunk geometry only: the map is per FFN width)
                const Tile tn = tile_of(run_tile(ti + G));
                if (tn.Fx == map_fx) {
                    chunk_load(c, tn.rows, mapF);
                    c_next = true;
                }
            }
            dn_chunk_mma<BD>(acc, s_chunk, rsF, cbF, n_lane, g_lane, ab + (size_t)ci * cbF * 128, P.nl);
            wave_lds_handoff();
        }
        // o = acc * 2^-sc_m; weighted write per pair
        {
            const int hrow = rg * DEC_DN_ROWS + wave * 16 + n_lane;
            const float ov[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g_lane + r;
                if (m < n_tok) {
                    const float o = ldexpf(ov[r], -s_hsc[m]);
                    if (shared_slot) {
                        st_tagged(P.oll + (size_t)(TK + m) * H + hrow, o, tag);
                    } else {
                        const int p = s_sorted[s_slot_start[s] + m];
                        if (P.mode & DEC_MODE_COMBINE) st_tagged(P.oll + (size_t)p * H + hrow, s_w[p] * o, tag);
                        else P.out_pairs[(size_t)p * H + hrow] = s_w[p] * o;  // read after the launch only
                    }
                }
            }
        }
        if (ti == first_tile) TRACE(7);
        __syncthreads();  // every wave's output stores are issued before the workgroup counts this tile
        if (tid == 0) {
            settle();  // the previous tile's count has long arrived
            if (P.mode & DEC_MODE_COMBINE) add_dev(&P.slice_count[rg * DEC_CSTRIDE], 1u);
            p_dn = add_dev(&P.dn_count[s * DEC_CSTRIDE], 1u);
            p_s = s;
        }
    }
    if (tid == 0) settle();  // the last tile's count
    TRACE(8);
    // the workspace moves on to the next call's tag
    if (tid == 0) epoch_advance(P.epoch, __builtin_amdgcn_readfirstlane(tag_v));
}

// ---------------------------------------------------------------------------
// Host-side launcher (called from the C ABI layer)
// ---------------------------------------------------------------------------
template <int BG, int BD, int XPARTS>
static hipError_t launch_t(const DecodeParams &P, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_decode_layer<BG, BD, XPARTS>), dim3(grid), dim3(DEC_THREADS), P.lds_total, st, P);
    return hipGetLastError();
}

template <int BG, int BD, int XPARTS>
static hipError_t occupancy_t(int lds, int *nb) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(nb, k_decode_layer<BG, BD, XPARTS>, DEC_THREADS, lds);
}

template <int BG, int BD, int XPARTS>
static hipError_t set_lds_t(int lds) {
    return hipFuncSetAttribute((const void *)k_decode_layer<BG, BD, XPARTS>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

// compile-time formats (gate/up bits, down bits) and activation parts (1: bf16, 2: fp32);
// the pairs built here are the ones decode_format_ok accepts
#define DECODE_DISPATCH_F(FN, BG, BD, ...) \
    return xf ? FN<BG, BD, 2>(__VA_ARGS__) : FN<BG, BD, 1>(__VA_ARGS__)
#define DECODE_DISPATCH(FN, ...)                                                                    \
    do {                                                                                            \
        if (bg == 4 && bd == 4) DECODE_DISPATCH_F(FN, 4, 4, __VA_ARGS__);                           \
        if (bg == 3 && bd == 4) DECODE_DISPATCH_F(FN, 3, 4, __VA_ARGS__);                           \
        if (bg == 4 && bd == 3) DECODE_DISPATCH_F(FN, 4, 3, __VA_ARGS__);                           \
        if (bg == 3 && bd == 3) DECODE_DISPATCH_F(FN, 3, 3, __VA_ARGS__);                           \
        if (bg == MOE_FMT_NL4 && bd == MOE_FMT_NL4) DECODE_DISPATCH_F(FN, MOE_FMT_NL4, MOE_FMT_NL4, __VA_ARGS__); \
        if (bg == 3 && bd == MOE_FMT_NL4) DECODE_DISPATCH_F(FN, 3, MOE_FMT_NL4, __VA_ARGS__);       \
        return hipErrorInvalidValue;                                                                \
    } while (0)

bool decode_format_ok(int bg, int bd) {
    return ((bg == 3 || bg == 4) && (bd == 3 || bd == 4)) || (bg == MOE_FMT_NL4 && bd == MOE_FMT_NL4) ||
           (bg == 3 && bd == MOE_FMT_NL4);
}

hipError_t decode_launch(const DecodeParams &P, int grid, hipStream_t st) {
    const int bg = P.bits, bd = P.dbits, xf = P.x_f32;
    DECODE_DISPATCH(launch_t, P, grid, st);
}

int decode_occupancy(int bg, int bd, int xf, int lds) {
    int nb = 0;
    if ([&]() -> hipError_t { DECODE_DISPATCH(occupancy_t, lds, &nb); }() != hipSuccess) return 0;
    return nb;
}

hipError_t decode_set_lds(int bg, int bd, int xf, int lds) { DECODE_DISPATCH(set_lds_t, lds); }

#ifdef MOE_PHASE_TRACE
extern "C" int moe_trace_set(void *buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

}  // namespace moe
