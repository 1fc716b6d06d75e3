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
//  A. every workgroup computes the routing of the <= 16 rows itself (top-k of
//     fp32 logits, ties to the lower id, softmax over the k selected) and the
//     stable grouping by (expert, token, slot); the rows' activations are
//     staged in LDS as fp16 in each format's k order, with a per-token
//     power-of-two scale (exact) so any bf16/fp32 range fits fp16.
//  B. gate/up: wave-level items (one expert, 16 output features, gate AND up,
//     all of K).  Each wave streams its expert rows from HBM in 16-row chunks
//     with 16-byte loads (two chunks in flight in registers), passes them
//     through a wave-private LDS buffer to reach the MFMA lane layout,
//     unpacks exact fp16 codes, and runs v_mfma_f32_16x16x32_f16 with the
//     (<= 16) rows of the expert as the M dimension: every weight byte is read
//     once per window for all rows sharing the expert (the read-once-per-window
//     rule of Strata "Several requests at once", opening section).  The fp16
//     block scale is applied to each block's fp32 partial.  SwiGLU in fp32;
//     h is published in fp32.
//  C. down: workgroup tiles (one expert, 128 output rows).  The tile waits on
//     its expert's gate/up counter, stages that expert's h in LDS as fp16
//     hi + lo (about 22 bits) with a per-token power-of-two scale, streams the
//     down rows, and writes w * o per (token, slot) pair.  The workgroup that
//     completes the last expert of a 128-row slice sums that slice in the
//     fixed slot order into y (deterministic; no floating-point atomics).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Phase A helpers
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Chunk streaming: 16 consecutive rows x CB blocks of one matrix.
// ---------------------------------------------------------------------------
struct Chunk {
    u32x4 r[DEC_MAX_LD];
};

__device__ __forceinline__ void chunk_load(Chunk &c, const uint8_t *rows, int row_bytes, int seg_off,
                                           int seg, int lane) {
    const int per_row = seg >> 4;  // 16-byte pieces per row segment
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) {
        int j = lane + 64 * u;
        if (j < 16 * per_row) {
            int r = j / per_row, col = j - r * per_row;
            c.r[u] = *(const u32x4 *)(rows + (size_t)r * row_bytes + seg_off + col * 16);
        }
    }
}

__device__ __forceinline__ void chunk_store_lds(const Chunk &c, uint8_t *buf, int seg, int lane) {
    const int n16 = seg;  // 16 rows * seg bytes / 16
#pragma unroll
    for (int u = 0; u < DEC_MAX_LD; ++u) {
        int j = lane + 64 * u;
        if (j < n16) *(u32x4 *)(buf + j * 16) = c.r[u];
    }
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t *p) { return *(const uint32_t *)p; }
__device__ __forceinline__ uint32_t lds_u16(const uint8_t *p) { return *(const uint16_t *)p; }

// One block of the chunk in LDS, as this lane's MFMA B operand(s) and scale.
// Lane layout: weight row n = lane % 16 of the chunk, k-group g = lane / 16.
template <int BITS>
struct BOp;

template <>
struct BOp<4> {
    half8 b;
    float d;
    // buf: 4-byte aligned LDS chunk; offsets are kept as integers so the
    // accesses stay LDS reads.
    __device__ __forceinline__ void load(const uint8_t *buf, int seg, int blk, int n, int g) {
        const int o = n * seg + blk * 18;
        d = half_bits_to_float(lds_u16(buf + o));
        const int qa = o + 2 + 4 * g, al = qa & ~3;
        uint32_t w0 = lds_u32(buf + al), w1 = lds_u32(buf + al + 4);
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
        // ql[2g], ql[2g+1] replicated into bytes 0 and 2
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

// acc += d * (A . B) for one block; A given as XPARTS fp16 parts.
template <int BITS, int XPARTS>
__device__ __forceinline__ void block_mma(float4v &acc, const BOp<BITS> &op, const half8 *a) {
    float4v z = {0.f, 0.f, 0.f, 0.f};
    float4v dd;
    if constexpr (BITS == 4) {
        dd = mfma16(a[0], op.b, z);
        if constexpr (XPARTS == 2) dd = mfma16(a[1], op.b, dd);
    } else {
        dd = mfma16(a[0], op.lo, z);
        dd = mfma16(a[0], op.hb, dd);
        if constexpr (XPARTS == 2) {
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

    int *s_idx = (int *)(smem + P.lds_idx);
    float *s_w = (float *)(smem + P.lds_w);
    int *s_sorted = (int *)(smem + P.lds_sorted);
    int *s_hist = (int *)(smem + P.lds_hist);
    int *s_slot_start = (int *)(smem + P.lds_slot_start);
    int *s_slot_exp = (int *)(smem + P.lds_slot_exp);
    int *s_slot_cnt = (int *)(smem + P.lds_slot_cnt);
    float *s_tinv = (float *)(smem + P.lds_tinv);
    float *s_hinv = (float *)(smem + P.lds_hinv);
    int *s_misc = (int *)(smem + P.lds_misc);
    uint8_t *s_xa = smem + P.lds_xa;
    uint8_t *s_chunk = smem + P.lds_chunk + wave * P.chunk_stride;

    // ======================= Phase A: routing and grouping =======================
    if (P.mode & DEC_MODE_ROUTE) {
        for (int t = wave; t < T; t += DEC_WAVES)
            wave_topk_row<16>(P.logits + (size_t)t * E, E, k, s_idx + t * k, s_w + t * k, lane);
        for (int e = tid; e <= E; e += DEC_THREADS) s_hist[e] = 0;
        __syncthreads();
        for (int p = tid; p < TK; p += DEC_THREADS) atomicAdd(&s_hist[s_idx[p]], 1);
        __syncthreads();
        if (wave == 0) {
            // exclusive scan of (count | active flag << 16) over E <= 1024 experts
            const int per = (E + 63) / 64;
            int base = lane * per;
            int sum = 0;
            for (int i = 0; i < per; ++i) {
                int e = base + i;
                if (e < E) {
                    int c = s_hist[e];
                    sum += c | ((c > 0) << 16);
                }
            }
            int incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int o = __shfl_up(incl, off, 64);
                if (lane >= off) incl += o;
            }
            int run = incl - sum;
            for (int i = 0; i < per; ++i) {
                int e = base + i;
                if (e < E) {
                    int c = s_hist[e];
                    int off = run & 0xFFFF, act = run >> 16;
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
        // stable placement: rank of pair p among earlier pairs of the same expert
        for (int p = tid; p < TK; p += DEC_THREADS) {
            int e = s_idx[p], rank = 0;
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

    // activations: per-token power-of-two scale, fp16 in the format's k order
    {
        const int nkb = H >> 5;
        for (int t = wave; t < T; t += DEC_WAVES) {
            float mx = 0.0f;
            if (P.x_f32) {
                const float *xr = (const float *)P.x + (size_t)t * H;
                for (int i = lane; i < H; i += 64) mx = fmaxf(mx, fabsf(xr[i]));
            } else {
                const uint16_t *xr = (const uint16_t *)P.x + (size_t)t * H;
                for (int i = lane; i < H; i += 64) mx = fmaxf(mx, fabsf(bf16_bits_to_float(xr[i])));
            }
            mx = wave_max_f(mx);
            int ex = 0;
            if (mx > 0.0f) frexpf(mx, &ex);
            int sc = (mx > 0.0f) ? 14 - ex : 0;  // max * 2^sc in [2^13, 2^14)
            if (lane == 0) s_tinv[t] = ldexpf(1.0f, -sc);
            for (int grp = lane; grp < nkb * 4; grp += 64) {
                int b = grp >> 2, g = grp & 3;
                u32x4 hi4, lo4;
                uint16_t hv[8], lv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int pos = b * 32 + pos_in_block(BITS, g, e);
                    float xv = P.x_f32 ? ((const float *)P.x)[(size_t)t * H + pos]
                                       : bf16_bits_to_float(((const uint16_t *)P.x)[(size_t)t * H + pos]);
                    xv = ldexpf(xv, sc);
                    _Float16 h = (_Float16)xv;
                    hv[e] = __builtin_bit_cast(uint16_t, h);
                    lv[e] = f2h_bits(xv - (float)h);
                }
                hi4.x = hv[0] | ((uint32_t)hv[1] << 16);
                hi4.y = hv[2] | ((uint32_t)hv[3] << 16);
                hi4.z = hv[4] | ((uint32_t)hv[5] << 16);
                hi4.w = hv[6] | ((uint32_t)hv[7] << 16);
                *(u32x4 *)(s_xa + (((size_t)t * nkb + b) * 4 + g) * 16) = hi4;
                if (XPARTS == 2) {
                    lo4.x = lv[0] | ((uint32_t)lv[1] << 16);
                    lo4.y = lv[2] | ((uint32_t)lv[3] << 16);
                    lo4.z = lv[4] | ((uint32_t)lv[5] << 16);
                    lo4.w = lv[6] | ((uint32_t)lv[7] << 16);
                    *(u32x4 *)(s_xa + (((size_t)(T + t) * nkb + b) * 4 + g) * 16) = lo4;
                }
            }
        }
    }
    __syncthreads();

    const int n_slots = s_misc[0];
    const int bb = block_bytes(BITS);
    const int F = P.F, Fs = has_shared ? P.Fs : 0;
    const int nkbH = H >> 5;
    const int cbH = chunk_blocks(nkbH), nchH = nkbH / cbH, segH = cbH * bb;
    const size_t rowH = (size_t)nkbH * bb;
    const size_t eb = (size_t)3 * F * rowH;  // routed expert blob bytes
    const int items_sh = Fs >> 4, items_rt = F >> 4;
    const int n_items = items_sh + (n_slots - hs) * items_rt;
    const int n_lane = lane & 15, g_lane = lane >> 4;

    // ======================= Phase B: gate/up + SwiGLU =======================
    for (int it = blockIdx.x * DEC_WAVES + wave; it < n_items; it += gridDim.x * DEC_WAVES) {
        int s, fg, Fx;
        const uint8_t *blob;
        if (it < items_sh) {
            s = 0;
            fg = it;
            Fx = Fs;
            blob = P.w_shared;
        } else {
            int r = it - items_sh;
            s = hs + r / items_rt;
            fg = r - (s - hs) * items_rt;
            Fx = F;
            blob = P.w_routed + (size_t)s_slot_exp[s] * eb;
        }
        const size_t mat = (size_t)Fx * rowH;
        const uint8_t *rows_g = blob + (size_t)fg * 16 * rowH;
        const uint8_t *rows_u = rows_g + mat;
        const int n_tok = s_slot_cnt[s];
        const bool shared_slot = (s_slot_exp[s] < 0);
        const int m_tok = n_lane;  // A row (slot-local token) of this lane
        int tok = 0;
        if (m_tok < n_tok) tok = shared_slot ? m_tok : s_sorted[s_slot_start[s] + m_tok] / k;
        const bool a_valid = m_tok < n_tok;

        float4v accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
        const int nch = 2 * nchH;  // gate chunks then up chunks
        Chunk c0, c1;
        chunk_load(c0, rows_g, (int)rowH, 0, segH, lane);
        for (int ci = 0; ci < nch; ++ci) {
            // next chunk into the other register set
            if (ci + 1 < nch) {
                int cn = ci + 1;
                const uint8_t *rb = cn < nchH ? rows_g : rows_u;
                int kc = cn < nchH ? cn : cn - nchH;
                if (ci & 1) chunk_load(c0, rb, (int)rowH, kc * segH, segH, lane);
                else chunk_load(c1, rb, (int)rowH, kc * segH, segH, lane);
            }
            __builtin_amdgcn_wave_barrier();
            if (ci & 1) chunk_store_lds(c1, s_chunk, segH, lane);
            else chunk_store_lds(c0, s_chunk, segH, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int kc = ci < nchH ? ci : ci - nchH;
            float4v &acc = ci < nchH ? accg : accu;
            for (int b = 0; b < cbH; ++b) {
                const int gb = kc * cbH + b;  // block index along K
                half8 a[XPARTS];
#pragma unroll
                for (int xp = 0; xp < XPARTS; ++xp) {
                    if (a_valid)
                        a[xp] = *(const half8 *)(s_xa + (((size_t)(xp * T + tok) * nkbH + gb) * 4 + g_lane) * 16);
                    else
                        a[xp] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                }
                BOp<BITS> op;
                op.load(s_chunk, segH, b, n_lane, g_lane);
                block_mma<BITS, XPARTS>(acc, op, a);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        // SwiGLU in fp32; h published as fp32 in the down projection's k order
        const int f = fg * 16 + n_lane;
        int pb = f >> 5, pg, pe;
        group_slot_of(BITS, f & 31, pg, pe);
        float gv[4] = {accg.x, accg.y, accg.z, accg.w};
        float uv[4] = {accu.x, accu.y, accu.z, accu.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int m = 4 * g_lane + r;
            if (m < n_tok) {
                int tk = shared_slot ? m : s_sorted[s_slot_start[s] + m] / k;
                float ti = s_tinv[tk];
                float g1 = gv[r] * ti, u1 = uv[r] * ti;
                float h = g1 / (1.0f + expf(-g1)) * u1;
                int row = shared_slot ? TK + m : s_slot_start[s] + m;
                *(float *)(P.h_arr + (size_t)row * P.h_row_bytes + (size_t)pb * 128 + pg * 32 + pe * 4) = h;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) atomic_add_release(&P.gu_count[s], 1u);
    }

    // ======================= Phase C: down + weighted write + combine =======================
    const int tiles_per_slot = H / DEC_DN_ROWS;
    const int n_tiles = n_slots * tiles_per_slot;
    const int t0 = (int)(((long long)blockIdx.x * n_tiles) / gridDim.x);
    const int t1 = (int)(((long long)(blockIdx.x + 1) * n_tiles) / gridDim.x);
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

        Chunk c0, c1;
        chunk_load(c0, rows_d, (int)rowF, 0, segF, lane);  // prefetch before the wait

        if (s != cur_slot) {
            __syncthreads();  // previous tile's readers of s_xa are done
            if (tid == 0) {
                const uint32_t need = (uint32_t)(Fx >> 4);
                uint32_t spins = 0;
                while (atomic_load_acquire(&P.gu_count[s]) < need) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > DEC_SPIN_LIMIT || (atomic_load_acquire(P.err) & 1u)) {
                        atomicOr(P.err, 1u);
                        break;
                    }
                }
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            // stage this expert's h rows into LDS as fp16 hi + lo of h * 2^sc_t,
            // sc_t a per-token power of two putting max|h_t| in [2^13, 2^14)
            const int row0 = shared_slot ? TK : s_slot_start[s];
            const int ngrp = Fx >> 3;  // groups of 8 values (one k-group of one block)
            for (int r = wave; r < n_tok; r += DEC_WAVES) {
                const float *hr = (const float *)(P.h_arr + (size_t)(row0 + r) * P.h_row_bytes);
                float mx = 0.0f;
                for (int gi = lane; gi < ngrp; gi += 64) {
                    u32x4 a = *(const u32x4 *)(hr + gi * 8), b = *(const u32x4 *)(hr + gi * 8 + 4);
                    float v[8] = {__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, a.y),
                                  __builtin_bit_cast(float, a.z), __builtin_bit_cast(float, a.w),
                                  __builtin_bit_cast(float, b.x), __builtin_bit_cast(float, b.y),
                                  __builtin_bit_cast(float, b.z), __builtin_bit_cast(float, b.w)};
#pragma unroll
                    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
                }
                mx = wave_max_f(mx);
                int ex = 0;
                if (mx > 0.0f) frexpf(mx, &ex);
                const int sc = mx > 0.0f ? 14 - ex : 0;
                if (lane == 0) s_hinv[r] = ldexpf(1.0f, -sc);
                for (int gi = lane; gi < ngrp; gi += 64) {
                    u32x4 a = *(const u32x4 *)(hr + gi * 8), b = *(const u32x4 *)(hr + gi * 8 + 4);
                    uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                    uint16_t hv[8], lv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float v = ldexpf(__builtin_bit_cast(float, w8[e]), sc);
                        _Float16 hh = (_Float16)v;
                        hv[e] = __builtin_bit_cast(uint16_t, hh);
                        lv[e] = f2h_bits(v - (float)hh);
                    }
                    u32x4 h4, l4;
                    h4.x = hv[0] | ((uint32_t)hv[1] << 16);
                    h4.y = hv[2] | ((uint32_t)hv[3] << 16);
                    h4.z = hv[4] | ((uint32_t)hv[5] << 16);
                    h4.w = hv[6] | ((uint32_t)hv[7] << 16);
                    l4.x = lv[0] | ((uint32_t)lv[1] << 16);
                    l4.y = lv[2] | ((uint32_t)lv[3] << 16);
                    l4.z = lv[4] | ((uint32_t)lv[5] << 16);
                    l4.w = lv[6] | ((uint32_t)lv[7] << 16);
                    uint8_t *dst = s_xa + (size_t)r * (Fx * 4) + (size_t)gi * 32;
                    *(u32x4 *)dst = h4;
                    *(u32x4 *)(dst + 16) = l4;
                }
            }
            __syncthreads();
            cur_slot = s;
        }

        float4v acc = {0.f, 0.f, 0.f, 0.f};
        const bool a_valid = n_lane < n_tok;
        for (int ci = 0; ci < nchF; ++ci) {
            if (ci + 1 < nchF) {
                if (ci & 1) chunk_load(c0, rows_d, (int)rowF, (ci + 1) * segF, segF, lane);
                else chunk_load(c1, rows_d, (int)rowF, (ci + 1) * segF, segF, lane);
            }
            __builtin_amdgcn_wave_barrier();
            if (ci & 1) chunk_store_lds(c1, s_chunk, segF, lane);
            else chunk_store_lds(c0, s_chunk, segF, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int b = 0; b < cbF; ++b) {
                const int gb = ci * cbF + b;
                half8 a[2];
                if (a_valid) {
                    const uint8_t *ap = s_xa + (size_t)n_lane * (Fx * 4) + (size_t)gb * 128 + g_lane * 32;
                    a[0] = *(const half8 *)ap;
                    a[1] = *(const half8 *)(ap + 16);
                } else {
                    a[0] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                    a[1] = a[0];
                }
                BOp<BITS> op;
                op.load(s_chunk, segF, b, n_lane, g_lane);
                block_mma<BITS, 2>(acc, op, a);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        // o = acc * 2^8; weighted write per pair
        {
            const int hrow = rg * DEC_DN_ROWS + wave * 16 + n_lane;
            float ov[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int m = 4 * g_lane + r;
                if (m < n_tok) {
                    float o = ov[r] * s_hinv[m];
                    if (shared_slot) {
                        P.out_shared[(size_t)m * H + hrow] = o;
                    } else {
                        int p = s_sorted[s_slot_start[s] + m];
                        P.out_pairs[(size_t)p * H + hrow] = s_w[p] * o;
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) {
            int do_combine = 0;
            if (P.mode & DEC_MODE_COMBINE) {
                uint32_t old = atomic_add_release(&P.slice_count[rg], 1u);
                do_combine = (old == (uint32_t)(n_slots - 1));
            }
            uint32_t dn = atomic_add_release(&P.dn_count[s], 1u);
            if (dn == (uint32_t)(tiles_per_slot - 1)) {
                atomic_store_relaxed(&P.gu_count[s], 0u);
                atomic_store_relaxed(&P.dn_count[s], 0u);
            }
            s_misc[1] = do_combine;
        }
        __syncthreads();
        if (s_misc[1]) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            for (int i = tid; i < T * DEC_DN_ROWS; i += DEC_THREADS) {
                const int t = i / DEC_DN_ROWS, hrow = rg * DEC_DN_ROWS + (i - t * DEC_DN_ROWS);
                float acc2 = P.out_pairs[((size_t)t * k) * H + hrow];
                for (int j = 1; j < k; ++j) acc2 += P.out_pairs[((size_t)t * k + j) * H + hrow];
                if (has_shared) acc2 += P.out_shared[(size_t)t * H + hrow];
                P.y[(size_t)t * H + hrow] = acc2;
            }
            __syncthreads();
            if (tid == 0) atomic_store_relaxed(&P.slice_count[rg], 0u);
        }
    }
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
    return hipFuncSetAttribute((const void *)k_decode_layer<BITS, XPARTS>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

hipError_t decode_launch(const DecodeParams &P, int grid, hipStream_t st) {
    const int xp = P.x_f32 ? 2 : 1;
    if (P.bits == 4) return xp == 2 ? launch_t<4, 2>(P, grid, st) : launch_t<4, 1>(P, grid, st);
    return xp == 2 ? launch_t<3, 2>(P, grid, st) : launch_t<3, 1>(P, grid, st);
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

}  // namespace moe
