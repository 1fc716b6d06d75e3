// moe_prefill.hip -- the routed-expert layer for prefill chunks (any number of
// rows): a grouped GEMM over per-expert row tiles.
//
// The forum thread "把 Strata 搬上 SGLang 引擎 的嘗試" (§二) shows that a
// prefill chunk must compute only the rows routed to each expert rather than
// the whole batch with a mask (the expert-scoped layout), and (§三, the MMQ
// prefill measurement) that a batch of tokens should share one read of the
// expert's weights.  Strata's batching document lists an option that sorts
// full expert groups by row count; here the tile schedule takes the largest
// groups first for the same reason (the long tiles start early).
//
// Kernels:
//   k_prefill_plan   one workgroup: active experts (+ the shared expert as a
//                    group of every row) ordered by decreasing size class
//                    (floor(log2(rows)); ties in expert order), and the prefix
//                    sums of their tile counts.
//   k_prefill_gemm   persistent grouped GEMM, tiles of 16, 32 or 64 rows (by
//                    the group's size) x 128 features (gate/up) or 256
//                    outputs (down).  Each wave dequantizes the weight
//                    fragments of its own MFMAs in registers, as bf16 holding
//                    the exact integer codes minus the bias; the activations
//                    (bf16, exact) are gathered into LDS by the group's row
//                    list; v_mfma_f32_16x16x32_bf16 covers one 32-wide quant
//                    block, and the fp16 block scale multiplies that block's
//                    fp32 partial.  Gate/up tiles compute both projections for
//                    the same 128 features and apply SwiGLU in fp32, storing h
//                    as bf16 hi + lo (h = hi + lo to 16 bits); down tiles run
//                    both parts through the MFMA and write w * o per (token,
//                    slot) pair.
//   k_prefill_combine  y_t = (((w_t0 o_t0 + w_t1 o_t1) + ...) + s_t) in slot
//                    order, four consecutive outputs per thread.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

#ifdef MOE_PHASE_TRACE
// Per-tile timestamps (100 MHz device clock), analysis builds only: word
// [mode][tile][4] = start, end, m-tiles, workgroup.
__device__ uint64_t *g_trace_pf = nullptr;
extern "C" int moe_trace_prefill_set(void *buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_trace_pf), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#define PTRACE(i, v)                                          \
    do {                                                      \
        if (g_trace_pf && threadIdx.x == 0) g_trace_pf[i] = (v); \
    } while (0)
#else
#define PTRACE(i, v) \
    do {             \
    } while (0)
#endif

constexpr int PF_KSB = 2;        // quant blocks per K step
constexpr int PF_THREADS = 512;  // eight waves
constexpr int PF_NF_GU = 128;    // features per gate/up tile (8 waves x 16)
constexpr int PF_NF_DN = 256;    // outputs per down tile (8 waves x 2 x 16)

// 16-row m-tiles per tile for a group of cnt rows: tiles of 16, 32 or 64 rows,
// so a small group does not pay for MFMAs over empty rows.
__device__ __forceinline__ int pf_mtl(int cnt) { return cnt <= 16 ? 1 : (cnt <= 32 ? 2 : 4); }

__global__ __launch_bounds__(1024) void k_prefill_plan(PlanParams P) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_sg[1024], s_sd[1024];
    const int tid = threadIdx.x;
    const int na = P.active[0];
    const int ns = na + (P.has_shared ? 1 : 0);
    uint64_t *keys = (uint64_t *)smem;                  // [ns]
    int *tg = (int *)(smem + 8 * (size_t)(P.E + 1));   // [ns] gate/up tiles per sorted slot
    int *td = tg + (P.E + 1);                          // [ns]
    auto slot_of = [&](int i, int &e, int &cnt) {
        if (P.has_shared && i == na) {
            e = -1;
            cnt = P.T;
        } else {
            e = P.active[1 + i];
            cnt = P.offsets[e + 1] - P.offsets[e];
        }
    };
    auto place = [&](int rank, int e, int cnt) {
        P.slot_exp[rank] = e;
        P.slot_cnt[rank] = cnt;
        P.slot_row0[rank] = e < 0 ? 0 : P.offsets[e];
        P.slot_hrow0[rank] = e < 0 ? P.T * P.k : P.offsets[e];
        const int mt = (cnt + 16 * pf_mtl(cnt) - 1) / (16 * pf_mtl(cnt));
        tg[rank] = mt * ((e < 0 ? P.Fs : P.F) / PF_NF_GU);
        td[rank] = mt * (P.H / PF_NF_DN);
    };
    if (ns <= 1024) {
        // order: size class floor(log2(rows)) descending, then the active list's
        // order (expert id; the shared expert, a group of every row, after the
        // routed ones of its class).  Rank = slots of larger classes + earlier
        // slots of the same class (ballots per class within a wave, then the
        // earlier waves' counts).
        __shared__ int s_wcnt[16][32];
        const int lane = tid & 63, wv = tid >> 6;
        int e = 0, cnt = 0, cls = -1;
        if (tid < ns) {
            slot_of(tid, e, cnt);
            cls = 31 - __builtin_clz((unsigned)cnt);
        }
        int within = 0;
        for (int v = 0; v < 32; ++v) {
            const uint64_t m = __ballot(cls == v);
            if (cls == v) within = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == 0) s_wcnt[wv][v] = __popcll(m);
        }
        __syncthreads();
        // per class: the earlier waves' counts (in place), then the slots of the
        // larger classes (one wave, a suffix sum over the 32 classes)
        __shared__ int s_above[32];
        if (tid < 32) {
            int run = 0;
            for (int w = 0; w < 16; ++w) {
                const int c = s_wcnt[w][tid];
                s_wcnt[w][tid] = run;
                run += c;
            }
            int above = 0;
            for (int v = 0; v < 32; ++v) {  // every lane takes part in every shuffle
                const int r = __shfl(run, v, 64);
                above += v > tid ? r : 0;
            }
            s_above[tid] = above;
        }
        __syncthreads();
        if (tid < ns) place(s_above[cls] + s_wcnt[wv][cls] + within, e, cnt);
    } else {
        // key: row count (desc), then expert id (asc; the shared expert is id -1 -> first)
        for (int i = tid; i < ns; i += 1024) {
            int e, cnt;
            slot_of(i, e, cnt);
            keys[i] = ((uint64_t)(uint32_t)cnt << 32) | (uint32_t)(0x7FFFFFFF - (e + 1));
        }
        __syncthreads();
        for (int i = tid; i < ns; i += 1024) {
            const uint64_t ki = keys[i];
            int rank = 0;
            for (int j = 0; j < ns; ++j) rank += keys[j] > ki;
            place(rank, 0x7FFFFFFF - (int)(uint32_t)ki - 1, (int)(ki >> 32));
        }
    }
    __syncthreads();
    // tile prefix sums: thread i owns a run of consecutive slots
    const int per = (ns + 1023) / 1024;
    const int i0 = min(ns, tid * per), i1 = min(ns, i0 + per);
    int sg = 0, sd = 0;
    for (int i = i0; i < i1; ++i) {
        sg += tg[i];
        sd += td[i];
    }
    s_sg[tid] = sg;
    s_sd[tid] = sd;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a = tid >= off ? s_sg[tid - off] : 0;
        const int b = tid >= off ? s_sd[tid - off] : 0;
        __syncthreads();
        s_sg[tid] += a;
        s_sd[tid] += b;
        __syncthreads();
    }
    int a = s_sg[tid] - sg, b = s_sd[tid] - sd;
    for (int i = i0; i < i1; ++i) {
        P.prefix_gu[i] = a;
        P.prefix_dn[i] = b;
        a += tg[i];
        b += td[i];
    }
    if (tid == 1023) {
        P.prefix_gu[ns] = s_sg[1023];
        P.prefix_dn[ns] = s_sd[1023];
        P.prefix_gu[P.E + 2] = ns;  // number of slots, for the GEMM kernels
        P.prefix_dn[P.E + 2] = ns;
    }
}


typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // 4-byte aligned 16-byte load

// ---------------------------------------------------------------------------
// In-register dequantization of one k-group (8 consecutive weights 8g..8g+7 of
// a 32-weight block) into 8 bf16 values that hold the integer codes minus the
// format's bias exactly (scale applied later to the fp32 MFMA result).
// ---------------------------------------------------------------------------

// 3-bit: weight i of a block = low part (field i/8 of low-part byte i%8) plus
// 4 * third bit i, minus 4.  The 3-bit codes of four weights are assembled
// one per byte, then each byte indexes two 8-entry byte tables (the high and
// the low byte of bf16(code - 4)) with v_perm_b32, and two more byte
// permutes interleave them into bf16 pairs.
__device__ __forceinline__ u32x4 deq3_group(uint32_t qs0, uint32_t qs1, uint32_t qh, uint32_t g) {
    const uint32_t sh = 2u * g;
    const uint32_t l0 = (qs0 >> sh) & 0x03030303u;
    const uint32_t l1 = (qs1 >> sh) & 0x03030303u;
    const uint32_t t0 = (qh >> (8u * g)) & 15u;
    const uint32_t t1 = (qh >> (8u * g + 4u)) & 15u;
    // bit j of t -> bit 2 of byte j: t * (4 + 2^9 + 2^16 + 2^23), the other
    // partial products land on bits the mask drops (no carries: all distinct)
    const uint32_t c0 = and_or(__umul24(t0, 0x810204u), 0x04040404u, l0);
    const uint32_t c1 = and_or(__umul24(t1, 0x810204u), 0x04040404u, l1);
    // bf16(c - 4), c = 0..7: C080 C040 C000 BF80 0000 3F80 4000 4040
    const uint32_t hi_lo = 0xBFC0C0C0u, hi_hi = 0x40403F00u;  // high bytes, codes 0-3 / 4-7
    const uint32_t lo_lo = 0x80004080u, lo_hi = 0x40008000u;  // low bytes
    const uint32_t h0 = __builtin_amdgcn_perm(hi_hi, hi_lo, c0), b0 = __builtin_amdgcn_perm(lo_hi, lo_lo, c0);
    const uint32_t h1 = __builtin_amdgcn_perm(hi_hi, hi_lo, c1), b1 = __builtin_amdgcn_perm(lo_hi, lo_lo, c1);
    u32x4 r;
    r.x = __builtin_amdgcn_perm(h0, b0, 0x05010400u);  // (low, high) byte of weights 0, 1
    r.y = __builtin_amdgcn_perm(h0, b0, 0x07030602u);  // weights 2, 3
    r.z = __builtin_amdgcn_perm(h1, b1, 0x05010400u);
    r.w = __builtin_amdgcn_perm(h1, b1, 0x07030602u);
    return r;
}

// 4-bit: weight i < 16 = low nibble of code byte i, weight i+16 = its high
// nibble, minus 8.  qa/qb: code dwords of the group's eight bytes, ns: nibble
// shift.  xor 0x8 turns c into the 4-bit two's complement of c - 8.
__device__ __forceinline__ u32x4 deq4_group(uint32_t qa, uint32_t qb, uint32_t ns) {
    qa ^= 0x88888888u;
    qb ^= 0x88888888u;
    uint32_t f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[j] = __builtin_bit_cast(uint32_t, (float)(int)__builtin_amdgcn_sbfe((int)qa, 8u * j + ns, 4u));
        f[4 + j] = __builtin_bit_cast(uint32_t, (float)(int)__builtin_amdgcn_sbfe((int)qb, 8u * j + ns, 4u));
    }
    u32x4 r;  // small integers: bf16 = the fp32 high half, exactly
    r.x = __builtin_amdgcn_perm(f[1], f[0], 0x07060302u);
    r.y = __builtin_amdgcn_perm(f[3], f[2], 0x07060302u);
    r.z = __builtin_amdgcn_perm(f[5], f[4], 0x07060302u);
    r.w = __builtin_amdgcn_perm(f[7], f[6], 0x07060302u);
    return r;
}

// Raw dwords of weight blocks as loaded from HBM, and the block fields.
//   MODE 0 (gate/up): NW = one pair of consecutive blocks of one weight row
//     (3-bit: 28 bytes = 7 dwords; 4-bit: 36 bytes = 9 dwords).
//   MODE 1 (down, column-block-major): one block of an even or odd row, the
//     row pair's dwords from the block's first one (3-bit: 4, 4-bit: 5).
template <int BITS>
struct BFields {
    uint32_t d;      // fp16 scale bits (low half)
    uint32_t q[BITS == 4 ? 4 : 3];  // 4-bit: code dwords; 3-bit: low parts (2), third bits
};

// Fields of one block from a run of dwords: `odd` = the block starts 2 bytes
// into dword o (scale in its high half, then aligned code dwords); otherwise
// it starts at dword 0 and every field is two bytes into a dword.
template <int BITS>
__device__ __forceinline__ BFields<BITS> block_fields(const uint32_t *w, bool odd, int o) {
    BFields<BITS> f;
    constexpr int NQ = BITS == 4 ? 4 : 3;
    if (!odd) {
        f.d = w[0];
#pragma unroll
        for (int i = 0; i < NQ; ++i) f.q[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], 16u);
    } else {
        f.d = w[o] >> 16;
#pragma unroll
        for (int i = 0; i < NQ; ++i) f.q[i] = w[o + 1 + i];
    }
    return f;
}

template <int BITS>
__device__ __forceinline__ u32x4 deq_group(const BFields<BITS> &f, uint32_t g) {
    if constexpr (BITS == 3) {
        return deq3_group(f.q[0], f.q[1], f.q[2], g);
    } else {
        const bool odd = g & 1u;
        return deq4_group(odd ? f.q[2] : f.q[0], odd ? f.q[3] : f.q[1], 4u * (g >> 1));
    }
}

template <int MODE, int BITS, int XP>
struct GemmSmem {
    uint16_t a[2][XP][4][PF_KSB][4][16][8];  // A, double-buffered: [buf][part][m-tile][block][k-group][row][8]
    int pair[64];                            // pair id of each tile row (down tiles)
};

struct TileInfo {
    int slot, cnt, nt, r0, nrows, Fx, hrow0, mtl;
    bool shared_slot;
    const uint8_t *blob;
    int a_pair;  // this thread's A row: its pair id (gate/up gather), -1 when none
    int pr64;    // thread tid < 64: pair id of tile row tid, -1 when none
};

template <int MODE, int BITS, int XP, int MTL>
__device__ __forceinline__ void gemm_tile(const GemmParams &P, GemmSmem<MODE, BITS, XP> &sm, const TileInfo &ti) {
    constexpr int NPASS = MODE == 0 ? 2 : 1;       // gate + up / down
    constexpr int NTW = MODE == 0 ? 1 : 2;         // 16-column n-tiles per wave
    constexpr int NFT = MODE == 0 ? PF_NF_GU : PF_NF_DN;
    constexpr int NB = NPASS * NTW;                // weight fragments per lane per block
    constexpr int bb = BITS == 4 ? 18 : 14;
    // dwords of one block pair: gate/up, two consecutive blocks of a row;
    // down, one block of the rows 2i (n-tile 0) and 2i+1 (n-tile 1)
    constexpr int NW = BITS == 4 ? 9 : 7;
    constexpr int NRAW = MODE == 0 ? NPASS : PF_KSB;  // pairs per lane per K step
    constexpr bool XF32 = MODE == 0 && XP == 2;              // fp32 activations, split into bf16 hi + lo
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_lane = lane & 15;
    const uint32_t g_lane = (uint32_t)(lane >> 4);
    const size_t rowH = (size_t)P.rowG;  // bytes of a gate/up row (the gate/up format's blocks)
    const int hs = P.h_stride;  // h row: hi plane [0, hs), lo plane [hs, 2 hs) (u16)
    // A staging: one chunk per thread = (m-tile, block, k-group, row) of 8 K-elements
    const int a_n = tid & 15, a_g = (tid >> 4) & 3, a_blk = (tid >> 6) & 1, a_m = tid >> 7;
    const int K = MODE == 0 ? P.H : ti.Fx;
    const int nks = K / (32 * PF_KSB);

    const int a_r = 16 * a_m + a_n;
    const bool a_st = a_m < MTL;
    const bool a_ld = a_st && a_r < ti.nrows;
    size_t a_off = 0;
    if (a_ld) {
        if (MODE == 0) {
            const int t = ti.shared_slot ? ti.r0 + a_r : ti.a_pair / P.k;
            a_off = (size_t)t * P.H + 32 * a_blk + 8 * a_g;
        } else {
            a_off = (size_t)(ti.hrow0 + ti.r0 + a_r) * (2 * hs) + 32 * a_blk + 8 * a_g;
        }
    }
    constexpr int PD = (MODE == 1 && BITS == 4) ? 2 : 3;  // K steps in flight: step s loads at the end of step s - PD
    auto load_a = [&](int ks, u32x4 (&ra)[2]) {
        ra[0] = u32x4{0u, 0u, 0u, 0u};
        ra[1] = u32x4{0u, 0u, 0u, 0u};
        if (a_ld) {
            const size_t o = a_off + (size_t)ks * (32 * PF_KSB);
            if (MODE == 0 && !XF32) {
                ra[0] = *(const u32x4 *)((const uint16_t *)P.x + o);
            } else if (XF32) {
                const u32x4 *src = (const u32x4 *)((const float *)P.x + o);
                ra[0] = src[0];
                ra[1] = src[1];
            } else {
                const uint16_t *hb16 = (const uint16_t *)P.hbuf;
                ra[0] = *(const u32x4 *)(hb16 + o);
                ra[1] = *(const u32x4 *)(hb16 + o + hs);
            }
        }
    };
    auto store_a = [&](int buf, const u32x4 (&ra)[2]) {
        if (!a_st) return;
        if (XF32) {
            uint32_t hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v0 = __builtin_bit_cast(float, i < 2 ? ra[0][2 * i] : ra[1][2 * i - 4]);
                const float v1 = __builtin_bit_cast(float, i < 2 ? ra[0][2 * i + 1] : ra[1][2 * i - 3]);
                const uint16_t h0 = f2bf_bits(v0), h1 = f2bf_bits(v1);
                const uint16_t l0 = f2bf_bits(v0 - bf16_bits_to_float(h0));
                const uint16_t l1 = f2bf_bits(v1 - bf16_bits_to_float(h1));
                hv[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lv[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            *(u32x4 *)&sm.a[buf][0][a_m][a_blk][a_g][a_n][0] = u32x4{hv[0], hv[1], hv[2], hv[3]};
            *(u32x4 *)&sm.a[buf][XP - 1][a_m][a_blk][a_g][a_n][0] = u32x4{lv[0], lv[1], lv[2], lv[3]};
        } else {
            *(u32x4 *)&sm.a[buf][0][a_m][a_blk][a_g][a_n][0] = ra[0];
            if (XP == 2) *(u32x4 *)&sm.a[buf][XP - 1][a_m][a_blk][a_g][a_n][0] = ra[1];
        }
    };

    // ---- weight sources of this lane: byte offsets from the tile's blob ----
    uint32_t woff[NRAW];
    size_t wstep;  // bytes per K step
    if (MODE == 0) {
        const uint32_t g_row = (uint32_t)((ti.nt * NFT + wave * 16 + n_lane) * rowH);
        woff[0] = g_row;
        if (NPASS == 2) woff[NPASS - 1] = g_row + (uint32_t)(ti.Fx * rowH);  // up row
        wstep = (size_t)PF_KSB * bb;
    } else {
        // wave w, n-tile t: rows nt*256 + 32 w + 2 n + t (t = row parity); the
        // pair (2i, 2i+1) of block c sits at (c*H + 2i)*bb
        const int hp = ti.nt * NFT + 32 * wave + 2 * n_lane;
        const uint32_t dn = (uint32_t)(2 * ti.Fx * rowH + (size_t)hp * bb);
#pragma unroll
        for (int b = 0; b < PF_KSB; ++b) woff[b] = dn + (uint32_t)(b * P.H * bb);
        wstep = (size_t)PF_KSB * P.H * bb;
    }
    auto load_w = [&](int ks, uint32_t (&dst)[NRAW][NW]) {
        const uint8_t *base = ti.blob + (size_t)ks * wstep;
#pragma unroll
        for (int b = 0; b < NRAW; ++b) {
            const uint32_t *s = (const uint32_t *)(base + woff[b]);
            const u32x4 v = *(const u32x4a4 *)s;
            dst[b][0] = v.x;
            dst[b][1] = v.y;
            dst[b][2] = v.z;
            dst[b][3] = v.w;
            if constexpr (NW == 7) {
                dst[b][4] = s[4];
                dst[b][5] = s[5];
                dst[b][6] = s[6];
            } else if constexpr (NW == 9) {
                const u32x4 u = *(const u32x4a4 *)(s + 4);
                dst[b][4] = u.x;
                dst[b][5] = u.y;
                dst[b][6] = u.z;
                dst[b][7] = u.w;
                dst[b][8] = s[8];
            }
        }
    };

    float4v acc[NB][MTL];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int m = 0; m < MTL; ++m) acc[a][m] = float4v{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int cur, const uint32_t (&rw)[NRAW][NW]) {
#pragma unroll
        for (int blk = 0; blk < PF_KSB; ++blk) {
            bf16x8 av[MTL][XP];
#pragma unroll
            for (int m = 0; m < MTL; ++m)
#pragma unroll
                for (int x = 0; x < XP; ++x) av[m][x] = *(const bf16x8 *)&sm.a[cur][x][m][blk][g_lane][n_lane][0];
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                // fragment f: gate/up pass f, or down n-tile f (row parity f)
                BFields<BITS> fl;
                if (MODE == 0) fl = block_fields<BITS>(rw[f], blk == 1, BITS == 4 ? 4 : 3);
                else fl = block_fields<BITS>(rw[blk], f == 1, BITS == 4 ? 4 : 3);
                const bf16x8 bq = __builtin_bit_cast(bf16x8, deq_group<BITS>(fl, g_lane));
                const float d = half_bits_to_float(fl.d);
                // the m-tiles' MFMAs issue back to back, then their scaling
                float4v dd[MTL];
#pragma unroll
                for (int m = 0; m < MTL; ++m) {
                    const float4v z = {0.f, 0.f, 0.f, 0.f};
                    dd[m] = mfma16bf(av[m][0], bq, z);
                    if (XP == 2) dd[m] = mfma16bf(av[m][XP - 1], bq, dd[m]);
                }
#pragma unroll
                for (int m = 0; m < MTL; ++m) {
                    acc[f][m].x = fmaf(d, dd[m].x, acc[f][m].x);
                    acc[f][m].y = fmaf(d, dd[m].y, acc[f][m].y);
                    acc[f][m].z = fmaf(d, dd[m].z, acc[f][m].z);
                    acc[f][m].w = fmaf(d, dd[m].w, acc[f][m].w);
                }
            }
        }
    };

    // ring of PD steps in registers (static slots: the step loop is unrolled by PD)
    uint32_t rw[PD][NRAW][NW];
    u32x4 ra[PD][2];
#pragma unroll
    for (int u = 0; u < PD; ++u) {
        if (u < nks) {
            load_a(u, ra[u]);
            load_w(u, rw[u]);
        }
    }
    store_a(0, ra[0]);
    __syncthreads();
    for (int k0 = 0; k0 < nks; k0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int ks = k0 + u;
            if (ks < nks) {
                compute(ks & 1, rw[u]);
                if (ks + 1 < nks) store_a((ks + 1) & 1, ra[(u + 1) % PD]);
                if (ks + PD < nks) {
                    load_a(ks + PD, ra[u]);
                    load_w(ks + PD, rw[u]);
                }
                __syncthreads();
            }
        }
    }
    // ---- epilogue ----
#pragma unroll
    for (int m = 0; m < MTL; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = m * 16 + 4 * (int)g_lane + r;
            if (rr >= ti.nrows) continue;
            if (MODE == 0) {
                const int col = ti.nt * NFT + wave * 16 + n_lane;  // feature
                const float g = acc[0][m][r], u = acc[NPASS - 1][m][r];
                const float h = g * u * __frcp_rn(1.0f + __expf(-g));
                const uint16_t hh = f2bf_bits(h);
                const uint16_t hl = f2bf_bits(h - bf16_bits_to_float(hh));
                uint16_t *dst = (uint16_t *)P.hout + (size_t)(ti.hrow0 + ti.r0 + rr) * (2 * hs) + col;
                dst[0] = hh;
                dst[hs] = hl;
            } else {
                const int pr = sm.pair[rr];
                const float wgt = (ti.shared_slot || !P.pair_w) ? 1.0f : P.pair_w[pr];
                float *orow = ti.shared_slot ? P.out_shared + (size_t)(ti.r0 + rr) * P.H
                                             : P.out_pairs + (size_t)pr * P.H;
#pragma unroll
                for (int t = 0; t < NTW; ++t)
                    orow[ti.nt * NFT + 32 * wave + 2 * n_lane + t] = wgt * acc[t][m][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM: persistent workgroups walk the tile list (slots by decreasing
// row count; within a slot, m-tiles of one 64-output n-tile are consecutive).
// Tile: 16*mtl rows (mtl = 1, 2, 4 by the group's size) x 128 features
// (gate/up) or 256 outputs (down), K in steps of two quant blocks.  Eight
// waves; wave w owns 16 features (gate/up: the gate and the up row of each)
// or 32 output rows (down) and dequantizes exactly the B fragments of its
// own MFMAs in registers: lane (n, g) holds k-group g of
// weight row n, as v_mfma_f32_16x16x32_bf16 expects.  A (activations, or h
// as bf16 hi + lo) goes through LDS, double-buffered: one barrier per K step,
// and the next step's A and weight loads are in flight during this step's
// math.
// ---------------------------------------------------------------------------
template <int MODE, int BITS, int XP>
__global__ __launch_bounds__(PF_THREADS) void k_prefill_gemm(GemmParams P) {
    __shared__ __align__(16) GemmSmem<MODE, BITS, XP> sm;
    // the slot plan, read once: prefix[ns + 1], then per slot exp, cnt, row0, hrow0
    extern __shared__ __align__(16) int s_plan[];
    const int tid = threadIdx.x;
    const int ns = P.prefix[P.E + 2];
    const int total = P.prefix[ns];
    int *s_prefix = s_plan, *s_exp = s_plan + ns + 1, *s_cnt = s_exp + ns, *s_row0 = s_cnt + ns,
        *s_hrow0 = s_row0 + ns;
    for (int i = tid; i <= ns; i += PF_THREADS) s_prefix[i] = P.prefix[i];
    for (int i = tid; i < ns; i += PF_THREADS) {
        s_exp[i] = P.slot_exp[i];
        s_cnt[i] = P.slot_cnt[i];
        s_row0[i] = P.slot_row0[i];
        s_hrow0[i] = P.slot_hrow0[i];
    }
    __syncthreads();

    // tile -> slot and rows, from LDS; the rows' pair ids are global loads,
    // issued one tile ahead
    auto tile_info = [&](int tile, TileInfo &ti) {
        int lo = 0, hi = ns - 1;  // slot: largest i with prefix[i] <= tile
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= tile) lo = mid;
            else hi = mid - 1;
        }
        ti.slot = lo;
        const int e = s_exp[lo];
        ti.cnt = s_cnt[lo];
        ti.shared_slot = e < 0;
        ti.Fx = ti.shared_slot ? P.Fs : P.F;
        ti.hrow0 = s_hrow0[lo];
        ti.mtl = pf_mtl(ti.cnt);
        const int MT = 16 * ti.mtl;
        const int mtiles = (ti.cnt + MT - 1) / MT;
        const int local = tile - s_prefix[lo];
        const int mt = local % mtiles;
        ti.nt = local / mtiles;
        ti.r0 = mt * MT;
        ti.nrows = min(MT, ti.cnt - ti.r0);
        ti.blob = ti.shared_slot ? P.w_shared : P.w_routed + (size_t)e * P.eb;
        const int row0 = s_row0[lo] + ti.r0;
        const int a_r = 16 * (tid >> 7) + (tid & 15);  // this thread's A row (see gemm_tile)
        ti.a_pair = (MODE == 0 && !ti.shared_slot && (tid >> 7) < ti.mtl && a_r < ti.nrows) ? P.pairs[row0 + a_r] : -1;
        ti.pr64 = (tid < 64 && tid < ti.nrows && !ti.shared_slot) ? P.pairs[row0 + tid] : -1;
    };

    int tile = blockIdx.x;
    TileInfo cur;
    if (tile < total) tile_info(tile, cur);
    for (; tile < total; tile += gridDim.x) {
        TileInfo nxt;
        const bool more = tile + (int)gridDim.x < total;
        if (more) tile_info(tile + gridDim.x, nxt);
        __syncthreads();  // the previous tile's epilogue is done with sm.pair
        if (tid < 64) sm.pair[tid] = cur.pr64;
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile, __builtin_amdgcn_s_memrealtime());
        if (cur.mtl == 4) gemm_tile<MODE, BITS, XP, 4>(P, sm, cur);
        else if (cur.mtl == 2) gemm_tile<MODE, BITS, XP, 2>(P, sm, cur);
        else gemm_tile<MODE, BITS, XP, 1>(P, sm, cur);
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 1, __builtin_amdgcn_s_memrealtime());
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 2, (uint64_t)cur.mtl);
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 3, (uint64_t)blockIdx.x);
        if (more) cur = nxt;
    }
}

// Four consecutive outputs per thread (H is a multiple of 256).
__global__ __launch_bounds__(256) void k_prefill_combine(CombineParams P) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)P.T * P.H) return;
    const size_t t = i / P.H, h = i - t * P.H;
    const float *src = P.out_pairs + t * P.k * P.H + h;
    float4v acc = *(const float4v *)src;
    for (int j = 1; j < P.k; ++j) {
        const float4v v = *(const float4v *)(src + (size_t)j * P.H);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (P.out_shared) {
        const float4v s = *(const float4v *)(P.out_shared + i);
        acc.x += s.x;
        acc.y += s.y;
        acc.z += s.z;
        acc.w += s.w;
    }
    *(float4v *)(P.y + i) = acc;
}

// ---------------------------------------------------------------------------
hipError_t prefill_plan_launch(const PlanParams &P, hipStream_t st) {
    const size_t lds = (size_t)(P.E + 1) * 16;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)k_prefill_plan, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)((MOE_MAX_EXPERTS_DEV + 1) * 16));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_prefill_plan, dim3(1), dim3(1024), lds, st, P);
    return hipGetLastError();
}

// Persistent grid: every workgroup resident (cus x workgroups per CU).
template <int MODE, int BITS, int XP>
static hipError_t gemm_t(const GemmParams &P, int cus, hipStream_t st) {
    // dynamic LDS: the slot plan (prefix[ns + 1] + 4 arrays of ns), ns <= E + 1
    const size_t plan_bytes = (size_t)(5 * (P.E + 1) + 1) * 4;
    static int occ = 0;
    if (occ == 0) {
        hipError_t e = hipFuncSetAttribute((const void *)k_prefill_gemm<MODE, BITS, XP>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (5 * (MOE_MAX_EXPERTS_DEV + 1) + 1) * 4);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)k_prefill_gemm<MODE, BITS, XP>, PF_THREADS,
                                                         (5 * (MOE_MAX_EXPERTS_DEV + 1) + 1) * 4);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
    }
    hipLaunchKernelGGL((k_prefill_gemm<MODE, BITS, XP>), dim3(cus * occ), dim3(PF_THREADS), plan_bytes, st, P);
    return hipGetLastError();
}

hipError_t prefill_gemm_launch(int mode, int bits, const GemmParams &P, int cus, hipStream_t st) {
    const int xp = (mode == 1 || P.x_f32) ? 2 : 1;
    if (mode == 0) {
        if (bits == 4) return xp == 2 ? gemm_t<0, 4, 2>(P, cus, st) : gemm_t<0, 4, 1>(P, cus, st);
        return xp == 2 ? gemm_t<0, 3, 2>(P, cus, st) : gemm_t<0, 3, 1>(P, cus, st);
    }
    if (bits == 4) return gemm_t<1, 4, 2>(P, cus, st);
    return gemm_t<1, 3, 2>(P, cus, st);
}

hipError_t prefill_combine_launch(const CombineParams &P, hipStream_t st) {
    const size_t n = (size_t)P.T * P.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_prefill_combine, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, P);
    return hipGetLastError();
}

}  // namespace moe
