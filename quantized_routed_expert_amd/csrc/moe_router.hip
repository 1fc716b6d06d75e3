// moe_router.hip -- the router projection that produces the logits the
// layer ranks: logits[t][e] = sum_h x[t][h] * W[e][h], W the bf16 router
// matrix [E][H] (row e is expert e's router vector).  It is the step before
// the routed path: the extended-strata-moe "Reference", section "Tools"
// (route_dump / route_predict read a layer's router from its hidden state),
// and in the forum thread's post "prefill 36.8 -> 334" the decode wall is
// met with one captured graph per window over all 48 layers, which this
// launch joins next to the layer's own.
//
// One workgroup per tile of 16 rows x 16 experts, 8 waves, each wave one
// eighth of the K range on v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products
// are exact in fp32; fp32 x is split into bf16 hi + lo, two MFMAs).  The
// eight partial tiles are summed in LDS in wave order, so the result does
// not depend on timing, and a row's logits depend on that row only (an MFMA
// output row reads its own A row), whatever T is.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int RT_WAVES = 8;
constexpr int RT_THREADS = RT_WAVES * 64;

__device__ __forceinline__ float4v mfma16_bf16(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 hi + lo of 8 fp32 values (hi = round to nearest even; lo = the rest,
// rounded): together 16 significant bits
__device__ __forceinline__ void split_bf16(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t h0 = f2bf_bits(v[2 * i]), h1 = f2bf_bits(v[2 * i + 1]);
        const uint16_t l0 = f2bf_bits(v[2 * i] - bf16_bits_to_float(h0));
        const uint16_t l1 = f2bf_bits(v[2 * i + 1] - bf16_bits_to_float(h1));
        h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// Lane layout of the MFMA: lane l feeds row / column l % 16 and the eight
// consecutive k of k-group l / 16; it receives rows 4 (l / 16) + r,
// column l % 16 of the result.
template <int XF32, int NK>
__global__ __launch_bounds__(RT_THREADS) void k_router_logits(RouterParams P) {
    __shared__ float s_part[RT_WAVES][16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
    const int H = P.H, E = P.E, T = P.T;
    // rows and experts past the end read a valid row and are never stored
    const int e = min(e0 + n, E - 1);
    const int t = min(m0 + n, T - 1);
    const int kw = H / RT_WAVES;  // this wave's K range: [wave * kw, (wave + 1) * kw), NK steps of 32
    const size_t k0 = (size_t)wave * kw + 8 * g;
    const uint16_t *wr = P.w + (size_t)e * H + k0;
    // every load of the wave's range in flight at once
    u32x4 bw[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s) bw[s] = *(const u32x4 *)(wr + 32 * s);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (XF32) {
        const float *xr = (const float *)P.x + (size_t)t * H + k0;
        u32x4 xa[NK][2];
#pragma unroll
        for (int s = 0; s < NK; ++s) {
            xa[s][0] = *(const u32x4 *)(xr + 32 * s);
            xa[s][1] = *(const u32x4 *)(xr + 32 * s + 4);
        }
#pragma unroll
        for (int s = 0; s < NK; ++s) {
            // (components copied out first: a bit cast applied to a vector
            // component expression reads the vector's first component)
            const uint32_t q[8] = {xa[s][0].x, xa[s][0].y, xa[s][0].z, xa[s][0].w,
                                   xa[s][1].x, xa[s][1].y, xa[s][1].z, xa[s][1].w};
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, q[i]);
            bf16x8 hi, lo;
            split_bf16(v, hi, lo);
            const bf16x8 b = __builtin_bit_cast(bf16x8, bw[s]);
            acc = mfma16_bf16(hi, b, acc);
            acc = mfma16_bf16(lo, b, acc);
        }
    } else {
        const uint16_t *xr = (const uint16_t *)P.x + (size_t)t * H + k0;
        u32x4 xa[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s) xa[s] = *(const u32x4 *)(xr + 32 * s);
#pragma unroll
        for (int s = 0; s < NK; ++s)
            acc = mfma16_bf16(__builtin_bit_cast(bf16x8, xa[s]), __builtin_bit_cast(bf16x8, bw[s]), acc);
    }
    s_part[wave][4 * g + 0][n] = acc.x;
    s_part[wave][4 * g + 1][n] = acc.y;
    s_part[wave][4 * g + 2][n] = acc.z;
    s_part[wave][4 * g + 3][n] = acc.w;
    __syncthreads();
    if (tid < 256) {
        const int r = tid >> 4, c = tid & 15;
        float v = s_part[0][r][c];
#pragma unroll
        for (int w = 1; w < RT_WAVES; ++w) v += s_part[w][r][c];  // wave (K range) order
        if (m0 + r < T && e0 + c < E) P.logits[(size_t)(m0 + r) * E + e0 + c] = v;
    }
}

template <int XF32>
static hipError_t router_t(const RouterParams &P, hipStream_t st) {
    const dim3 grid((unsigned)((P.E + 15) / 16), (unsigned)((P.T + 15) / 16));
    const int nk = P.H / (32 * RT_WAVES);  // K steps per wave
    switch (nk) {
        case 1: hipLaunchKernelGGL((k_router_logits<XF32, 1>), grid, dim3(RT_THREADS), 0, st, P); break;
        case 2: hipLaunchKernelGGL((k_router_logits<XF32, 2>), grid, dim3(RT_THREADS), 0, st, P); break;
        case 4: hipLaunchKernelGGL((k_router_logits<XF32, 4>), grid, dim3(RT_THREADS), 0, st, P); break;
        case 8: hipLaunchKernelGGL((k_router_logits<XF32, 8>), grid, dim3(RT_THREADS), 0, st, P); break;
        case 16: hipLaunchKernelGGL((k_router_logits<XF32, 16>), grid, dim3(RT_THREADS), 0, st, P); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t router_logits_launch(const RouterParams &P, hipStream_t st) {
    return P.x_f32 ? router_t<1>(P, st) : router_t<0>(P, st);
}

}  // namespace moe
