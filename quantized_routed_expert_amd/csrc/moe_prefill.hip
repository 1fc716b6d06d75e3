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
//                    group of every row) ordered by decreasing row count, and
//                    the prefix sums of their tile counts.
//   k_prefill_gemm   persistent grouped GEMM, 64 rows x 64 outputs per tile.
//                    The quantized weight tile is dequantized into LDS as bf16
//                    holding the exact integer codes; the activations (bf16,
//                    exact) are gathered into LDS by the group's row list;
//                    v_mfma_f32_16x16x32_bf16 covers one 32-wide quant block,
//                    and the fp16 block scale multiplies that block's fp32
//                    partial.  Gate/up tiles compute both projections for the
//                    same 64 features and apply SwiGLU in fp32 (h stored as
//                    fp32); down tiles split h into bf16 hi + lo (two MFMAs)
//                    and write w * o per (token, slot) pair.
//   k_prefill_combine  y_t = (((w_t0 o_t0 + w_t1 o_t1) + ...) + s_t) in slot
//                    order, one thread per output element.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int PF_MT = 64;      // rows per tile
constexpr int PF_NF = 64;      // output features per tile
constexpr int PF_KSB = 2;      // quant blocks per K step
constexpr int PF_THREADS = 256;

__global__ __launch_bounds__(1024) void k_prefill_plan(PlanParams P) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int na = P.active[0];
    const int ns = na + (P.has_shared ? 1 : 0);
    uint64_t *keys = (uint64_t *)smem;            // [ns]
    int *tg = (int *)(smem + 8 * (size_t)(P.E + 1));   // [ns] gate/up tiles per sorted slot
    int *td = tg + (P.E + 1);                          // [ns]
    // key: row count (desc), then expert id (asc; the shared expert is id -1 -> first)
    for (int i = tid; i < ns; i += 1024) {
        int e, cnt;
        if (P.has_shared && i == na) {
            e = -1;
            cnt = P.T;
        } else {
            e = P.active[1 + i];
            cnt = P.offsets[e + 1] - P.offsets[e];
        }
        keys[i] = ((uint64_t)(uint32_t)cnt << 32) | (uint32_t)(0x7FFFFFFF - (e + 1));
    }
    __syncthreads();
    for (int i = tid; i < ns; i += 1024) {
        uint64_t ki = keys[i];
        int rank = 0;
        for (int j = 0; j < ns; ++j) rank += keys[j] > ki;
        int e = 0x7FFFFFFF - (int)(uint32_t)ki - 1;
        int cnt = (int)(ki >> 32);
        P.slot_exp[rank] = e;
        P.slot_cnt[rank] = cnt;
        P.slot_row0[rank] = e < 0 ? 0 : P.offsets[e];
        P.slot_hrow0[rank] = e < 0 ? P.T * P.k : P.offsets[e];
        int mt = (cnt + PF_MT - 1) / PF_MT;
        tg[rank] = mt * ((e < 0 ? P.Fs : P.F) / PF_NF);
        td[rank] = mt * (P.H / PF_NF);
    }
    __syncthreads();
    if (tid == 0) {
        int a = 0, b = 0;
        for (int i = 0; i < ns; ++i) {
            P.prefix_gu[i] = a;
            P.prefix_dn[i] = b;
            a += tg[i];
            b += td[i];
        }
        P.prefix_gu[ns] = a;
        P.prefix_dn[ns] = b;
        P.prefix_gu[P.E + 2] = ns;  // number of slots, for the GEMM kernels
        P.prefix_dn[P.E + 2] = ns;
    }
}

__device__ __forceinline__ uint16_t f2bf_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Dequantize one quant block (32 weights) to exact bf16 codes (code - bias),
// natural order; returns the scale.  Reads exactly the block's bytes.
template <int BITS>
__device__ __forceinline__ float dequant_block_bf16(const uint8_t *blk, uint16_t *out32) {
    const uint16_t *h = (const uint16_t *)blk;  // blocks are 2-byte aligned
    float d = half_bits_to_float(h[0]);
    if constexpr (BITS == 4) {
        uint16_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = h[1 + i];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t byte = (w[i >> 1] >> (8 * (i & 1))) & 0xFFu;
            out32[i] = f2bf_bits((float)((int)(byte & 15u) - 8));
            out32[i + 16] = f2bf_bits((float)((int)(byte >> 4) - 8));
        }
    } else {
        uint16_t w[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) w[i] = h[1 + i];
        uint32_t qh = (uint32_t)w[4] | ((uint32_t)w[5] << 16);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            uint32_t byte = (w[(i & 7) >> 1] >> (8 * (i & 1))) & 0xFFu;
            int lo = (int)((byte >> (2 * (i >> 3))) & 3u);
            int hb = (int)((qh >> i) & 1u);
            out32[i] = f2bf_bits((float)((lo | (hb << 2)) - 4));
        }
    }
    return d;
}

// MODE 0: gate/up + SwiGLU -> hout.  MODE 1: down -> weighted pair rows.
template <int MODE, int BITS, int XP>
__global__ __launch_bounds__(PF_THREADS) void k_prefill_gemm(GemmParams P) {
    constexpr int NB = MODE == 0 ? 2 * PF_NF : PF_NF;  // weight rows staged
    constexpr int NT_B = NB / 16;
    __shared__ __align__(16) uint16_t sA[XP][4][PF_KSB][4][16][8];
    __shared__ __align__(16) uint16_t sB[NT_B][PF_KSB][4][16][8];
    __shared__ float sS[PF_KSB][NB];
    __shared__ int s_tok[PF_MT];
    __shared__ int s_pair[PF_MT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_lane = lane & 15, g_lane = lane >> 4;
    const int ns = P.prefix[P.E + 2];
    const int total = P.prefix[ns];
    const int bb = BITS == 4 ? 18 : 14;
    const size_t rowH = (size_t)(P.H >> 5) * bb;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        // slot: largest i with prefix[i] <= tile
        int lo = 0, hi = ns - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (P.prefix[mid] <= tile) lo = mid;
            else hi = mid - 1;
        }
        const int slot = lo;
        const int e = P.slot_exp[slot];
        const int cnt = P.slot_cnt[slot];
        const bool shared_slot = e < 0;
        const int Fx = shared_slot ? P.Fs : P.F;
        const int mtiles = (cnt + PF_MT - 1) / PF_MT;
        const int local = tile - P.prefix[slot];
        const int mt = local % mtiles, nt = local / mtiles;
        const int r0 = mt * PF_MT;
        const int nrows = min(PF_MT, cnt - r0);
        const uint8_t *blob = shared_slot ? P.w_shared : P.w_routed + (size_t)e * 3 * Fx * rowH;
        const uint8_t *wrows;
        size_t wrow_bytes;
        int K;
        if (MODE == 0) {
            wrows = blob + (size_t)nt * PF_NF * rowH;  // gate rows; up rows at + Fx*rowH
            wrow_bytes = rowH;
            K = P.H;
        } else {
            // down, column-block-major: block (h, c) at (c * H + h) * bb
            wrows = blob + (size_t)2 * Fx * rowH + (size_t)nt * PF_NF * bb;
            wrow_bytes = bb;
            K = Fx;
        }
        __syncthreads();
        if (tid < PF_MT) {
            int r = r0 + tid;
            int tok = 0, pr = -1;
            if (tid < nrows) {
                if (shared_slot) tok = r;
                else {
                    pr = P.pairs[P.slot_row0[slot] + r];
                    tok = pr / P.k;
                }
            }
            s_tok[tid] = tok;
            s_pair[tid] = pr;
        }
        __syncthreads();

        float4v acc[2][4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[a][m] = float4v{0.f, 0.f, 0.f, 0.f};

        const int nks = (K >> 5) / PF_KSB;
        for (int ks = 0; ks < nks; ++ks) {
            // ---- stage A: 64 rows x 64 K ----
            {
                const int r = tid >> 2, q = tid & 3;  // q: 16 K-elements
                const int blk = q >> 1, g0 = (q & 1) * 2;
                const int k0 = ks * 64 + q * 16;
                uint16_t hv[16], lv[16];
                if (r < nrows) {
                    if (MODE == 0) {
                        const int t = s_tok[r];
                        if (P.x_f32) {
                            const float *xr = (const float *)P.x + (size_t)t * P.H + k0;
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                float v = xr[i];
                                hv[i] = f2bf_bits(v);
                                lv[i] = f2bf_bits(v - bf16_bits_to_float(hv[i]));
                            }
                        } else {
                            const u32x4 *xr = (const u32x4 *)((const uint16_t *)P.x + (size_t)t * P.H + k0);
                            u32x4 v0 = xr[0], v1 = xr[1];
                            uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                hv[2 * i] = (uint16_t)(wv[i] & 0xFFFFu);
                                hv[2 * i + 1] = (uint16_t)(wv[i] >> 16);
                                lv[2 * i] = 0;
                                lv[2 * i + 1] = 0;
                            }
                        }
                    } else {
                        const float *hr = P.hbuf + (size_t)(P.slot_hrow0[slot] + r0 + r) * P.h_stride + k0;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            float v = hr[i];
                            hv[i] = f2bf_bits(v);
                            lv[i] = f2bf_bits(v - bf16_bits_to_float(hv[i]));
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) hv[i] = lv[i] = 0;
                }
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    u32x4 h4, l4;
                    h4.x = hv[8 * gg] | ((uint32_t)hv[8 * gg + 1] << 16);
                    h4.y = hv[8 * gg + 2] | ((uint32_t)hv[8 * gg + 3] << 16);
                    h4.z = hv[8 * gg + 4] | ((uint32_t)hv[8 * gg + 5] << 16);
                    h4.w = hv[8 * gg + 6] | ((uint32_t)hv[8 * gg + 7] << 16);
                    *(u32x4 *)&sA[0][r >> 4][blk][g0 + gg][r & 15][0] = h4;
                    if (XP == 2) {
                        l4.x = lv[8 * gg] | ((uint32_t)lv[8 * gg + 1] << 16);
                        l4.y = lv[8 * gg + 2] | ((uint32_t)lv[8 * gg + 3] << 16);
                        l4.z = lv[8 * gg + 4] | ((uint32_t)lv[8 * gg + 5] << 16);
                        l4.w = lv[8 * gg + 6] | ((uint32_t)lv[8 * gg + 7] << 16);
                        *(u32x4 *)&sA[XP - 1][r >> 4][blk][g0 + gg][r & 15][0] = l4;
                    }
                }
            }
            // ---- stage B: NB weight rows x 2 blocks, exact bf16 codes ----
            if (tid < NB * PF_KSB) {
                const int row = tid >> 1, blk = tid & 1;
                const uint8_t *src;
                if (MODE == 0) {
                    const int half = row / PF_NF;  // 0 gate, 1 up
                    src = wrows + (size_t)half * Fx * rowH + (size_t)(row - half * PF_NF) * wrow_bytes;
                    src += (size_t)(ks * PF_KSB + blk) * bb;
                } else {
                    src = wrows + (size_t)row * wrow_bytes + (size_t)(ks * PF_KSB + blk) * P.H * bb;
                }
                uint16_t codes[32];
                float d = dequant_block_bf16<BITS>(src, codes);
                sS[blk][row] = d;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x4 c4;
                    c4.x = codes[8 * g] | ((uint32_t)codes[8 * g + 1] << 16);
                    c4.y = codes[8 * g + 2] | ((uint32_t)codes[8 * g + 3] << 16);
                    c4.z = codes[8 * g + 4] | ((uint32_t)codes[8 * g + 5] << 16);
                    c4.w = codes[8 * g + 6] | ((uint32_t)codes[8 * g + 7] << 16);
                    *(u32x4 *)&sB[row >> 4][blk][g][row & 15][0] = c4;
                }
            }
            __syncthreads();
            // ---- MFMA ----
#pragma unroll
            for (int blk = 0; blk < PF_KSB; ++blk) {
                constexpr int NPASS = MODE == 0 ? 2 : 1;
#pragma unroll
                for (int pss = 0; pss < NPASS; ++pss) {
                    const int ntb = MODE == 0 ? (pss * 4 + wave) : wave;  // B n-tile
                    const bf16x8 b = *(const bf16x8 *)&sB[ntb][blk][g_lane][n_lane][0];
                    const float d = sS[blk][ntb * 16 + n_lane];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        float4v z = {0.f, 0.f, 0.f, 0.f};
                        float4v dd = mfma16bf(*(const bf16x8 *)&sA[0][m][blk][g_lane][n_lane][0], b, z);
                        if (XP == 2) dd = mfma16bf(*(const bf16x8 *)&sA[XP - 1][m][blk][g_lane][n_lane][0], b, dd);
                        acc[pss][m].x = fmaf(d, dd.x, acc[pss][m].x);
                        acc[pss][m].y = fmaf(d, dd.y, acc[pss][m].y);
                        acc[pss][m].z = fmaf(d, dd.z, acc[pss][m].z);
                        acc[pss][m].w = fmaf(d, dd.w, acc[pss][m].w);
                    }
                }
            }
            __syncthreads();
        }
        // ---- epilogue ----
        const int col = nt * PF_NF + wave * 16 + n_lane;  // feature (MODE 0) / output row (MODE 1)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float gv[4] = {acc[0][m].x, acc[0][m].y, acc[0][m].z, acc[0][m].w};
            float uv[4] = {acc[1][m].x, acc[1][m].y, acc[1][m].z, acc[1][m].w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = m * 16 + 4 * g_lane + r;
                if (rr < nrows) {
                    if (MODE == 0) {
                        float g = gv[r], u = uv[r];
                        float h = g / (1.0f + expf(-g)) * u;
                        P.hout[(size_t)(P.slot_hrow0[slot] + r0 + rr) * P.h_stride + col] = h;
                    } else {
                        if (shared_slot) {
                            P.out_shared[(size_t)(r0 + rr) * P.H + col] = gv[r];
                        } else {
                            const int pr = s_pair[rr];
                            const float wgt = P.pair_w ? P.pair_w[pr] : 1.0f;
                            P.out_pairs[(size_t)pr * P.H + col] = wgt * gv[r];
                        }
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_prefill_combine(CombineParams P) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)P.T * P.H) return;
    const size_t t = i / P.H, h = i - t * P.H;
    const float *src = P.out_pairs + t * P.k * P.H + h;
    float acc = src[0];
    for (int j = 1; j < P.k; ++j) acc += src[(size_t)j * P.H];
    if (P.out_shared) acc += P.out_shared[i];
    P.y[i] = acc;
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

template <int MODE, int BITS, int XP>
static void gemm_t(const GemmParams &P, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_prefill_gemm<MODE, BITS, XP>), dim3(grid), dim3(PF_THREADS), 0, st, P);
}

hipError_t prefill_gemm_launch(int mode, int bits, const GemmParams &P, int grid, hipStream_t st) {
    const int xp = (mode == 1 || P.x_f32) ? 2 : 1;
    if (mode == 0) {
        if (bits == 4) xp == 2 ? gemm_t<0, 4, 2>(P, grid, st) : gemm_t<0, 4, 1>(P, grid, st);
        else xp == 2 ? gemm_t<0, 3, 2>(P, grid, st) : gemm_t<0, 3, 1>(P, grid, st);
    } else {
        if (bits == 4) gemm_t<1, 4, 2>(P, grid, st);
        else gemm_t<1, 3, 2>(P, grid, st);
    }
    return hipGetLastError();
}

hipError_t prefill_combine_launch(const CombineParams &P, hipStream_t st) {
    const size_t n = (size_t)P.T * P.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_prefill_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, P);
    return hipGetLastError();
}

}  // namespace moe
