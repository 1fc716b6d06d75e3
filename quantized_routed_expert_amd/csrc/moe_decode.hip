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
//  B. gate/up units: (expert, 16 output rows, gate or up, one K chunk of up
//     to 32 quant blocks), a few KB each, spread over every wave of the grid.
//     A wave streams its unit's quantized rows from HBM with 16-byte loads
//     (the next unit's chunk in flight while the current one computes),
//     passes them through a wave-private LDS buffer into the MFMA lane
//     layout, unpacks exact fp16 codes and runs v_mfma_f32_16x16x32_f16 with
//     the expert's (<= 16) rows as the M dimension: every weight byte is read
//     once per window for all rows that share the expert (the read-once-per-
//     window rule of Strata "Several requests at once", opening section).  The
//     fp16 block scale multiplies each block's fp32 partial.  A unit publishes
//     its fp32 partial sums and counts itself done for its expert.
//  C. down tiles: (expert, 128 output rows) per workgroup.  The tile prefetches
//     its weights, waits for its expert's units, sums the partials in a fixed
//     order, applies SwiGLU in fp32 and stages h in LDS as fp16 hi + lo (about
//     22 bits) with a per-token power-of-two scale, streams the down rows and
//     writes w * o per (token, slot) pair.  The workgroup that completes the
//     last expert of a 128-row slice sums that slice in the fixed slot order
//     into y (deterministic; no floating-point atomics).
//
// Data crossing workgroups (partials, pair rows) uses device-coherent accesses
// and per-wave store completion instead of agent-scope fences, which on this
// chip would write back or invalidate a whole XCD's L2.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

#ifdef MOE_PHASE_TRACE
// Phase timestamps (100 MHz device clock) per workgroup, for analysis builds only.
__device__ uint64_t *g_trace = nullptr;
#define TRACE(slot)                                                                                        \
    do {                                                                                                   \
        if (g_trace && threadIdx.x == 0) g_trace[blockIdx.x * 16 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define TRACE(slot) \
    do {            \
    } while (0)
#endif

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

// Router for one row by one wave (E <= 64 * EPL): k rounds of a wave-wide
// argmax, an equal logit going to the lower expert id; softmax over the k.
template <int EPL>
__device__ void route_row(const float *row, int E, int k, int *out_idx, float *out_w, int lane) {
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? float_key(row[e]) : 0u;  // finite values have keys > 0
    }
    float mine = 0.0f;
    int mine_id = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (key[i] > bk) {  // strict: the lowest i wins among equal keys
                bk = key[i];
                bi = i;
            }
        const uint32_t m = wave_max_u32(bk);
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
        const uint32_t u = (m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m;
        if (lane == j) {
            mine = __builtin_bit_cast(float, u);
            mine_id = e;
        }
    }
    const float l0 = __shfl(mine, 0, 64);
    const float ex = lane < k ? expf(mine - l0) : 0.0f;
    const float s = wave_sum_f(ex);
    if (lane < k) {
        out_idx[lane] = mine_id;
        out_w[lane] = ex / s;
    }
}

// ---------------------------------------------------------------------------
// Chunk streaming: 16 consecutive rows x CB blocks of one matrix.
// ---------------------------------------------------------------------------
struct Chunk {
    u32x4 r[DEC_MAX_LD];
};

__device__ __forceinline__ void chunk_load(Chunk &c, const uint8_t *rows, int row_bytes, int seg_off, int seg,
                                           int lane) {
    const int per_row = seg >> 4;  // 16-byte pieces per row segment
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) {
        const int j = lane + 64 * u;
        if (j < 16 * per_row) {
            const int r = j / per_row, col = j - r * per_row;
            c.r[u] = *(const u32x4 *)(rows + (size_t)r * row_bytes + seg_off + col * 16);
        }
    }
}

__device__ __forceinline__ void chunk_store_lds(const Chunk &c, uint8_t *buf, int seg, int lane) {
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) {
        const int j = lane + 64 * u;
        if (j < seg) *(u32x4 *)(buf + j * 16) = c.r[u];  // 16 rows * seg bytes = seg pieces
    }
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t *p) { return *(const uint32_t *)p; }
__device__ __forceinline__ uint32_t lds_u16(const uint8_t *p) { return *(const uint16_t *)p; }

// One block of the chunk in LDS as this lane's MFMA B operand(s) and scale.
// Lane layout: weight row n = lane % 16 of the chunk, k-group g = lane / 16.
// buf is 4-byte aligned; offsets stay integers so the accesses stay LDS reads.
template <int BITS>
struct BOp;

template <>
struct BOp<4> {
    half8 b;
    float d;
    __device__ __forceinline__ void load(const uint8_t *buf, int seg, int blk, int n, int g) {
        const int o = n * seg + blk * 18;
        d = half_bits_to_float(lds_u16(buf + o));
        const int qa = o + 2 + 4 * g, al = qa & ~3;
        const uint32_t w0 = lds_u32(buf + al), w1 = lds_u32(buf + al + 4);
        b = unpack4(__builtin_amdgcn_alignbyte(w1, w0, (uint32_t)(qa & 3)));
    }
};

template <>
struct BOp<3> {
    half8 lo, hb;
    float d;
    __device__ __forceinline__ void load(const uint8_t *buf, int seg, int blk, int n, int g) {
        const int o = n * seg + blk * 14;
        d = half_bits_to_float(lds_u16(buf + o));
        // low-part bytes ql[2g], ql[2g+1], each replicated into bytes 0 and 2
        const int qa = o + 2 + 2 * g;
        const uint32_t qw = lds_u32(buf + (qa & ~3));
        const uint32_t sh = (uint32_t)(qa & 3);
        const uint32_t sel0 = 0x0C000C00u | (sh << 16) | sh;
        const uint32_t p0 = __builtin_amdgcn_perm(qw, qw, sel0);
        const uint32_t p1 = __builtin_amdgcn_perm(qw, qw, sel0 + 0x00010001u);
        // third-bit word at bytes 10..13
        const int ha = o + 10, hal = ha & ~3;
        const uint32_t qh = __builtin_amdgcn_alignbyte(lds_u32(buf + hal + 4), lds_u32(buf + hal), (uint32_t)(ha & 3));
        unpack3(p0, p1, qh >> (2 * g), lo, hb);
    }
};

// acc += d * (A . B) for one block; A given as NP fp16 parts.
template <int BITS, int NP>
__device__ __forceinline__ void block_mma(float4v &acc, const BOp<BITS> &op, const half8 *a) {
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    float4v dd;
    if constexpr (BITS == 4) {
        dd = mfma16(a[0], op.b, z);
        if constexpr (NP == 2) dd = mfma16(a[1], op.b, dd);
    } else {
        dd = mfma16(a[0], op.lo, z);
        dd = mfma16(a[0], op.hb, dd);
        if constexpr (NP == 2) {
            dd = mfma16(a[1], op.lo, dd);
            dd = mfma16(a[1], op.hb, dd);
        }
    }
    acc.x = fmaf(op.d, dd.x, acc.x);
    acc.y = fmaf(op.d, dd.y, acc.y);
    acc.z = fmaf(op.d, dd.z, acc.z);
    acc.w = fmaf(op.d, dd.w, acc.w);
}

__host__ __device__ __forceinline__ int chunk_blocks(int nkb) {
    // largest of 32, 24, 16, 8 dividing nkb (nkb is a multiple of 8)
    return (nkb % 32 == 0) ? 32 : (nkb % 24 == 0) ? 24 : (nkb % 16 == 0) ? 16 : 8;
}

// Multiply-accumulate a whole chunk in LDS (cb blocks, a multiple of 4) into
// acc.  A operands: a_base points at this lane's first block, a_stride bytes
// between blocks, part_off bytes between the NP parts.
template <int BITS, int NP>
__device__ __forceinline__ void chunk_mma(float4v &acc, const uint8_t *buf, int seg, int cb, int n, int g,
                                          const uint8_t *a_base, int a_stride, int part_off, bool a_valid) {
    for (int b0 = 0; b0 < cb; b0 += 4) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            const int b = b0 + bi;
            half8 a[NP];
#pragma unroll
            for (int xp = 0; xp < NP; ++xp)
                a[xp] = a_valid ? *(const half8 *)(a_base + (size_t)b * a_stride + xp * part_off)
                                : half8{0, 0, 0, 0, 0, 0, 0, 0};
            BOp<BITS> op;
            op.load(buf, seg, b, n, g);
            block_mma<BITS, NP>(acc, op, a);
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int BITS, int XPARTS>
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
    float *s_tinv = (float *)(smem + P.lds_tinv);
    float *s_hinv = (float *)(smem + P.lds_hinv);
    uint32_t *s_xmax = (uint32_t *)(smem + P.lds_xmax);
    int *s_misc = (int *)(smem + P.lds_misc);
    uint8_t *s_xa = smem + P.lds_xa;
    uint8_t *s_chunk = smem + P.lds_chunk + wave * P.chunk_stride;

    TRACE(0);
    // ======================= Phase A: activations, routing, grouping =======================
    const int nkbH = H >> 5;
    for (int i = tid; i < T; i += DEC_THREADS) s_xmax[i] = 0u;
    if (P.mode & DEC_MODE_ROUTE)
        for (int e = tid; e <= E; e += DEC_THREADS) s_hist[e] = 0;
    __syncthreads();

    // activation blocks: thread owns blocks tid + 512 q (token t, block b)
    constexpr int QX = XPARTS == 1 ? DEC_X_BLOCKS_PER_THREAD : DEC_X_BLOCKS_PER_THREAD / 2;
    constexpr int NV = XPARTS == 1 ? 4 : 8;  // 16-byte pieces per block (bf16: 64 B, fp32: 128 B)
    u32x4 xr[QX][NV];
    const int nxb = T * nkbH;
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int j = tid + DEC_THREADS * q;
        if (j < nxb) {
            const u32x4 *src = (const u32x4 *)((const uint8_t *)P.x + (size_t)j * 32 * (XPARTS == 1 ? 2 : 4));
#pragma unroll
            for (int v = 0; v < NV; ++v) xr[q][v] = src[v];
        }
    }
    // routing of the rows owned by this wave (overlaps the activation loads)
    if (P.mode & DEC_MODE_ROUTE) {
        const int epl = (E + 63) >> 6;
        for (int t = wave; t < T; t += DEC_WAVES) {
            const float *row = P.logits + (size_t)t * E;
            if (epl <= 2) route_row<2>(row, E, k, s_idx + t * k, s_w + t * k, lane);
            else if (epl <= 4) route_row<4>(row, E, k, s_idx + t * k, s_w + t * k, lane);
            else if (epl <= 8) route_row<8>(row, E, k, s_idx + t * k, s_w + t * k, lane);
            else route_row<16>(row, E, k, s_idx + t * k, s_w + t * k, lane);
        }
    }
    // per-token max |x|
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int j = tid + DEC_THREADS * q;
        if (j < nxb) {
            float mx = 0.0f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t w4[4] = {xr[q][v].x, xr[q][v].y, xr[q][v].z, xr[q][v].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (XPARTS == 1) {
                        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w4[c] << 16)));
                        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w4[c] & 0xFFFF0000u)));
                    } else {
                        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w4[c])));
                    }
                }
            }
            atomicMax(&s_xmax[j / nkbH], __builtin_bit_cast(uint32_t, mx));
        }
    }
    TRACE(1);
    __syncthreads();

    // grouping: histogram, scan (wave 0), stable placement
    if (P.mode & DEC_MODE_ROUTE) {
        for (int p = tid; p < TK; p += DEC_THREADS) atomicAdd(&s_hist[s_idx[p]], 1);
        __syncthreads();
        if (wave == 0) {
            // exclusive scan of (count | active flag << 16) over E <= 1024 experts
            const int per = (E + 63) / 64;
            const int base = lane * per;
            int sum = 0;
            for (int i = 0; i < per; ++i) {
                const int e = base + i;
                if (e < E) {
                    const int c = s_hist[e];
                    sum += c | ((c > 0) << 16);
                }
            }
            int incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off, 64);
                if (lane >= off) incl += o;
            }
            int run = incl - sum;
            for (int i = 0; i < per; ++i) {
                const int e = base + i;
                if (e < E) {
                    const int c = s_hist[e];
                    const int off = run & 0xFFFF, act = run >> 16;
                    if (c > 0) {
                        s_slot_exp[hs + act] = e;
                        s_slot_start[hs + act] = off;
                        s_slot_cnt[hs + act] = c;
                    }
                    s_hist[e] = off;  // becomes the expert's first position
                    run += c | ((c > 0) << 16);
                }
            }
            if (lane == 63) s_misc[0] = hs + (incl >> 16);  // number of slots
        }
        __syncthreads();
        for (int p = tid; p < TK; p += DEC_THREADS) {
            const int e = s_idx[p];
            int rank = 0;
            for (int q = 0; q < p; ++q) rank += (s_idx[q] == e);
            s_sorted[s_hist[e] + rank] = p;
        }
        if (blockIdx.x == 0) {
            for (int p = tid; p < TK; p += DEC_THREADS) {
                if (P.topk_idx_out) P.topk_idx_out[p] = s_idx[p];
                if (P.topk_w_out) P.topk_w_out[p] = s_w[p];
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
        __syncthreads();
        const int na = s_misc[0] - hs;
        for (int a = tid; a < na; a += DEC_THREADS) {
            int e = P.g_active[1 + a];
            int st = 0, c = 0;
            if (e >= 0 && e < E) {
                st = P.g_offsets[e];
                c = P.g_offsets[e + 1] - st;
            }
            if (e < 0 || e >= E || st < 0 || c < 0 || c > MOE_DECODE_ROWS_DEV || st + c > TK) {
                atomicOr(P.err, 2u);
                e = (e >= 0 && e < E) ? e : 0;
                st = 0;
                c = 0;
            }
            s_slot_exp[hs + a] = e;
            s_slot_start[hs + a] = st;
            s_slot_cnt[hs + a] = c;
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
    // activations to fp16 (hi [+ lo]) of x * 2^sc_t in the format's k order
#pragma unroll
    for (int q = 0; q < QX; ++q) {
        const int j = tid + DEC_THREADS * q;
        if (j < nxb) {
            const int t = j / nkbH, b = j - t * nkbH;
            const float mx = __builtin_bit_cast(float, s_xmax[t]);
            int ex = 0;
            if (mx > 0.0f) frexpf(mx, &ex);
            const int sc = mx > 0.0f ? 14 - ex : 0;  // max * 2^sc in [2^13, 2^14)
            const float scale = __builtin_bit_cast(float, (uint32_t)(127 + sc) << 23);  // 2^sc, exact
            if (b == 0) s_tinv[t] = __builtin_bit_cast(float, (uint32_t)(127 - sc) << 23);
            uint32_t w[NV * 4];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                w[4 * v] = xr[q][v].x;
                w[4 * v + 1] = xr[q][v].y;
                w[4 * v + 2] = xr[q][v].z;
                w[4 * v + 3] = xr[q][v].w;
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t hv[4], lv[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    uint16_t hb2[2], lb2[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int pos = pos_in_block(BITS, g, 2 * e2 + h2);
                        float xv;
                        if (XPARTS == 1) xv = __builtin_bit_cast(float, (w[pos >> 1] >> (16 * (pos & 1))) << 16);
                        else xv = __builtin_bit_cast(float, w[pos]);
                        xv *= scale;
                        const _Float16 hh = (_Float16)xv;
                        hb2[h2] = __builtin_bit_cast(uint16_t, hh);
                        lb2[h2] = f2h_bits(xv - (float)hh);
                    }
                    hv[e2] = hb2[0] | ((uint32_t)hb2[1] << 16);
                    lv[e2] = lb2[0] | ((uint32_t)lb2[1] << 16);
                }
                *(u32x4 *)(s_xa + (((size_t)t * nkbH + b) * 4 + g) * 16) = u32x4{hv[0], hv[1], hv[2], hv[3]};
                if (XPARTS == 2)
                    *(u32x4 *)(s_xa + (((size_t)(T + t) * nkbH + b) * 4 + g) * 16) = u32x4{lv[0], lv[1], lv[2], lv[3]};
            }
        }
    }
    __syncthreads();
    TRACE(2);

    const int n_slots = s_misc[0];
    const int bb = block_bytes(BITS);
    const int F = P.F, Fs = has_shared ? P.Fs : 0;
    const int cbH = chunk_blocks(nkbH), nchH = nkbH / cbH, segH = cbH * bb;
    const size_t rowH = (size_t)nkbH * bb;
    const size_t eb = (size_t)3 * F * rowH;  // routed expert blob bytes
    const int units_sh = (Fs >> 4) * 2 * nchH, units_rt = (F >> 4) * 2 * nchH;
    const int n_units = units_sh + (n_slots - hs) * units_rt;
    const int n_lane = lane & 15, g_lane = lane >> 4;
    const int fstride = P.part_stride / (2 * nchH);  // Fmax

    // ======================= Phase B: gate/up units =======================
    {
        struct Unit {
            const uint8_t *rows;
            int s, fg, mat, kc;
        };
        auto unit_of = [&](int u) {
            Unit U;
            int Fx, r;
            const uint8_t *blob;
            if (u < units_sh) {
                U.s = 0;
                r = u;
                Fx = Fs;
                blob = P.w_shared;
            } else {
                const int v = u - units_sh;
                U.s = hs + v / units_rt;
                r = v - (U.s - hs) * units_rt;
                Fx = F;
                blob = P.w_routed + (size_t)s_slot_exp[U.s] * eb;
            }
            U.fg = r / (2 * nchH);
            const int rem = r - U.fg * 2 * nchH;
            U.mat = rem / nchH;
            U.kc = rem - U.mat * nchH;
            U.rows = blob + (size_t)U.mat * Fx * rowH + (size_t)U.fg * 16 * rowH;
            return U;
        };
        // unit order: wave 0 of every workgroup first, then wave 1, ...
        int u = wave * G + blockIdx.x;
        const int ustep = G * DEC_WAVES;
        Chunk c;
        if (u < n_units) {
            const Unit U = unit_of(u);
            chunk_load(c, U.rows, (int)rowH, U.kc * segH, segH, lane);
        }
        for (; u < n_units; u += ustep) {
            const Unit U = unit_of(u);
            __builtin_amdgcn_wave_barrier();
            chunk_store_lds(c, s_chunk, segH, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // the registers are free again: the next unit's chunk streams in
            // while this one computes
            const int un = u + ustep;
            if (un < n_units) {
                const Unit N = unit_of(un);
                chunk_load(c, N.rows, (int)rowH, N.kc * segH, segH, lane);
            }

            const int n_tok = s_slot_cnt[U.s];
            const bool shared_slot = s_slot_exp[U.s] < 0;
            const bool a_valid = n_lane < n_tok;
            int tok = 0;
            if (a_valid) tok = shared_slot ? n_lane : s_sorted[s_slot_start[U.s] + n_lane] / k;
            const uint8_t *a_base = s_xa + (((size_t)tok * nkbH + U.kc * cbH) * 4 + g_lane) * 16;
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            chunk_mma<BITS, XPARTS>(acc, s_chunk, segH, cbH, n_lane, g_lane, a_base, 64, T * nkbH * 64, a_valid);

            // publish the partial sums (back in the units of x), laid out in the
            // down projection's k order so the consumer reads whole groups
            const float av[4] = {acc.x, acc.y, acc.z, acc.w};
            const int f = U.fg * 16 + n_lane;
            int pg, pe;
            group_slot_of(BITS, f & 31, pg, pe);
            const int fo = (f >> 5) * 32 + pg * 8 + pe;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g_lane + r;
                if (m < n_tok) {
                    const int tk = shared_slot ? m : s_sorted[s_slot_start[U.s] + m] / k;
                    const int row = shared_slot ? TK + m : s_slot_start[U.s] + m;
                    st_dev(P.gu_part + (size_t)row * P.part_stride + (size_t)(U.mat * nchH + U.kc) * fstride + fo,
                           av[r] * s_tinv[tk]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            wait_all_mem();  // this wave's partial stores are complete before the count goes up
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) add_dev(&P.gu_count[U.s], 1u);
        }
    }
    TRACE(3);

    // ======================= Phase C: down + weighted write + combine =======================
    const int tiles_per_slot = H / DEC_DN_ROWS;
    const int n_tiles = n_slots * tiles_per_slot;
    const int t0 = (int)(((long long)blockIdx.x * n_tiles) / G);
    const int t1 = (int)(((long long)(blockIdx.x + 1) * n_tiles) / G);
    int cur_slot = -1;
    for (int ti = t0; ti < t1; ++ti) {
        const int s = ti / tiles_per_slot, rg = ti - s * tiles_per_slot;
        const bool shared_slot = (s_slot_exp[s] < 0);
        const int Fx = shared_slot ? Fs : F;
        const uint8_t *blob = shared_slot ? P.w_shared : P.w_routed + (size_t)s_slot_exp[s] * eb;
        const int nkbF = Fx >> 5;
        const int cbF = chunk_blocks(nkbF), nchF = nkbF / cbF, segF = cbF * bb;
        const size_t rowF = (size_t)nkbF * bb;
        const uint8_t *rows_d = blob + (size_t)2 * Fx * rowH + (size_t)(rg * DEC_DN_ROWS + wave * 16) * rowF;
        const int n_tok = s_slot_cnt[s];

        Chunk c;
        chunk_load(c, rows_d, (int)rowF, 0, segF, lane);  // prefetch before the wait

        if (s != cur_slot) {
            __syncthreads();  // previous tile's readers of s_xa are done
            if (ti == t0) TRACE(4);
            if (tid == 0) {
                const uint32_t need = (uint32_t)((Fx >> 4) * 2 * nchH);
                uint32_t spins = 0;
                while (ld_dev_u32(&P.gu_count[s]) < need) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > DEC_SPIN_LIMIT || (ld_dev_u32(P.err) & 1u)) {
                        atomicOr(P.err, 1u);
                        break;
                    }
                }
            }
            if (ti == t0) TRACE(5);
            __syncthreads();
            // h = silu(g) * u from the fixed-order sum of the partials; staged in
            // LDS as fp16 hi + lo of h * 2^sc_t (per-token power of two)
            const int row0 = shared_slot ? TK : s_slot_start[s];
            const int ngrp = Fx >> 3;  // groups of 8 values (one k-group of one block)
            for (int r = wave; r < n_tok; r += DEC_WAVES) {
                const float *pr = P.gu_part + (size_t)(row0 + r) * P.part_stride;
                float hv[2][8];
                float mx = 0.0f;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int gi = lane + 64 * q;
                    if (gi < ngrp) {
                        float gs[8], us[8];
                        const float *pg0 = pr + gi * 8;
                        const float *pu0 = pr + (size_t)nchH * fstride + gi * 8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            gs[e] = ld_dev(pg0 + e);
                            us[e] = ld_dev(pu0 + e);
                        }
                        for (int kc = 1; kc < nchH; ++kc) {  // fixed order: chunk 0, 1, ...
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                gs[e] += ld_dev(pg0 + (size_t)kc * fstride + e);
                                us[e] += ld_dev(pu0 + (size_t)kc * fstride + e);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float h = gs[e] / (1.0f + expf(-gs[e])) * us[e];
                            hv[q][e] = h;
                            mx = fmaxf(mx, fabsf(h));
                        }
                    }
                }
                mx = __builtin_bit_cast(float, wave_max_u32(__builtin_bit_cast(uint32_t, mx)));
                int ex = 0;
                if (mx > 0.0f) frexpf(mx, &ex);
                const int sc = mx > 0.0f ? 14 - ex : 0;
                const float scale = __builtin_bit_cast(float, (uint32_t)(127 + sc) << 23);
                if (lane == 0) s_hinv[r] = __builtin_bit_cast(float, (uint32_t)(127 - sc) << 23);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int gi = lane + 64 * q;
                    if (gi < ngrp) {
                        uint32_t h4[4], l4[4];
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            const float v0 = hv[q][2 * e2] * scale, v1 = hv[q][2 * e2 + 1] * scale;
                            const _Float16 a0 = (_Float16)v0, a1 = (_Float16)v1;
                            h4[e2] = __builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                            l4[e2] = f2h_bits(v0 - (float)a0) | ((uint32_t)f2h_bits(v1 - (float)a1) << 16);
                        }
                        uint8_t *dst = s_xa + (size_t)r * (Fx * 4) + (size_t)gi * 32;
                        *(u32x4 *)dst = u32x4{h4[0], h4[1], h4[2], h4[3]};
                        *(u32x4 *)(dst + 16) = u32x4{l4[0], l4[1], l4[2], l4[3]};
                    }
                }
            }
            __syncthreads();
            if (ti == t0) TRACE(6);
            cur_slot = s;
        }

        float4v acc = {0.f, 0.f, 0.f, 0.f};
        const bool a_valid = n_lane < n_tok;
        const uint8_t *a_base = s_xa + (size_t)n_lane * (Fx * 4) + g_lane * 32;
        for (int ci = 0; ci < nchF; ++ci) {
            __builtin_amdgcn_wave_barrier();
            chunk_store_lds(c, s_chunk, segF, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (ci + 1 < nchF) chunk_load(c, rows_d, (int)rowF, (ci + 1) * segF, segF, lane);
            chunk_mma<BITS, 2>(acc, s_chunk, segF, cbF, n_lane, g_lane, a_base + (size_t)ci * cbF * 128, 128, 16,
                               a_valid);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        // o = acc * 2^-sc_t; weighted write per pair
        {
            const int hrow = rg * DEC_DN_ROWS + wave * 16 + n_lane;
            const float ov[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g_lane + r;
                if (m < n_tok) {
                    const float o = ov[r] * s_hinv[m];
                    if (shared_slot) {
                        st_dev(&P.out_shared[(size_t)m * H + hrow], o);
                    } else {
                        const int p = s_sorted[s_slot_start[s] + m];
                        st_dev(&P.out_pairs[(size_t)p * H + hrow], s_w[p] * o);
                    }
                }
            }
        }
        if (ti == t0) TRACE(7);
        wait_all_mem();   // every wave's output stores are complete ...
        __syncthreads();  // ... before the workgroup counts this tile
        if (tid == 0) {
            int do_combine = 0;
            if (P.mode & DEC_MODE_COMBINE) {
                const uint32_t old = add_dev(&P.slice_count[rg], 1u);
                do_combine = (old == (uint32_t)(n_slots - 1));
            }
            const uint32_t dn = add_dev(&P.dn_count[s], 1u);
            if (dn == (uint32_t)(tiles_per_slot - 1)) {
                store_dev_u32(&P.gu_count[s], 0u);
                store_dev_u32(&P.dn_count[s], 0u);
            }
            s_misc[1] = do_combine;
        }
        __syncthreads();
        if (s_misc[1]) {
            for (int i = tid; i < T * DEC_DN_ROWS; i += DEC_THREADS) {
                const int t = i / DEC_DN_ROWS, hrow = rg * DEC_DN_ROWS + (i - t * DEC_DN_ROWS);
                float acc2 = ld_dev(&P.out_pairs[((size_t)t * k) * H + hrow]);
                for (int j = 1; j < k; ++j) acc2 += ld_dev(&P.out_pairs[((size_t)t * k + j) * H + hrow]);
                if (has_shared) acc2 += ld_dev(&P.out_shared[(size_t)t * H + hrow]);
                P.y[(size_t)t * H + hrow] = acc2;
            }
            __syncthreads();
            if (tid == 0) store_dev_u32(&P.slice_count[rg], 0u);
        }
    }
    TRACE(8);
}

// ---------------------------------------------------------------------------
// Host-side launcher (called from the C ABI layer)
// ---------------------------------------------------------------------------
template <int BITS, int XPARTS>
static hipError_t launch_t(const DecodeParams &P, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_decode_layer<BITS, XPARTS>), dim3(grid), dim3(DEC_THREADS), P.lds_total, st, P);
    return hipGetLastError();
}

template <int BITS, int XPARTS>
static int occupancy_t(int lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_layer<BITS, XPARTS>, DEC_THREADS, lds) != hipSuccess)
        return 0;
    return nb;
}

template <int BITS, int XPARTS>
static hipError_t set_lds_t(int lds) {
    return hipFuncSetAttribute((const void *)k_decode_layer<BITS, XPARTS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               lds);
}

hipError_t decode_launch(const DecodeParams &P, int grid, hipStream_t st) {
    if (P.bits == 4) return P.x_f32 ? launch_t<4, 2>(P, grid, st) : launch_t<4, 1>(P, grid, st);
    return P.x_f32 ? launch_t<3, 2>(P, grid, st) : launch_t<3, 1>(P, grid, st);
}

int decode_occupancy(int bits, int x_f32, int lds) {
    if (bits == 4) return x_f32 ? occupancy_t<4, 2>(lds) : occupancy_t<4, 1>(lds);
    return x_f32 ? occupancy_t<3, 2>(lds) : occupancy_t<3, 1>(lds);
}

hipError_t decode_set_lds(int bits, int x_f32, int lds) {
    if (bits == 4) return x_f32 ? set_lds_t<4, 2>(lds) : set_lds_t<4, 1>(lds);
    return x_f32 ? set_lds_t<3, 2>(lds) : set_lds_t<3, 1>(lds);
}

int decode_chunk_blocks(int nkb) { return chunk_blocks(nkb); }

#ifdef MOE_PHASE_TRACE
extern "C" int moe_trace_set(void *buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

}  // namespace moe
