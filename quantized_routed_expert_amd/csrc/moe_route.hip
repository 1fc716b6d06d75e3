// moe_route.hip -- router (top-k + softmax) and the stable counting-sort
// grouping of (token, expert) pairs, for any number of rows.
//
// Router: the k largest fp32 logits per token (an equal logit goes to the
// lower expert id) and a softmax over those k (forum thread "把 Strata 搬上
// SGLang 引擎 的嘗試", TL;DR and §三: top-10 of 512 experts; the
// extended-strata-moe "Reference", "Routing trace format": k ids and k
// weights per token).  One wave per row.
//
// Grouping: pairs p = t*k + j bucketed per expert so each expert computes only
// its own rows (thread §二, the expert-scoped layout), ordered by
// (expert, token, slot).  Three passes over chunks of 16 tokens: per-chunk
// histograms (LDS atomics: counts do not depend on order), one workgroup
// scanning (expert, chunk) counts into start positions, then each chunk
// placing its pairs in token order.  No global atomics, so the placement is
// the same on every run.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int EPL>
__global__ __launch_bounds__(256) void k_route(RouteParams P) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= P.T) return;
    __shared__ int s_idx[4][MOE_TOPK_MAX_LDS];
    __shared__ float s_w[4][MOE_TOPK_MAX_LDS];
    const int wv = threadIdx.x >> 6;
    uint32_t key[EPL];
    route_keys<EPL>(P.logits + (size_t)t * P.E, P.E, lane, key);
    route_pick<EPL>(key, P.k, s_idx[wv], s_w[wv], lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < P.k) {
        P.idx[(size_t)t * P.k + lane] = s_idx[wv][lane];
        P.w[(size_t)t * P.k + lane] = s_w[wv][lane];
    }
}

// Per-chunk expert histogram.
__global__ __launch_bounds__(256) void k_group_count(GroupParams P) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t *hist = (uint32_t *)smem;
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < P.E; e += 256) hist[e] = 0;
    __syncthreads();
    const size_t p0 = (size_t)c * GRP_CHUNK_TOKENS * P.k;
    const size_t p1 = min((size_t)(c + 1) * GRP_CHUNK_TOKENS * P.k, (size_t)P.T * P.k);
    for (size_t p = p0 + threadIdx.x; p < p1; p += 256) {
        const int e = P.idx[p];
        if ((unsigned)e < (unsigned)P.E) atomicAdd(&hist[e], 1u);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < P.E; e += 256) P.chunk_counts[(size_t)c * P.E + e] = hist[e];
}

// One workgroup: chunk_counts[c][e] -> first position of chunk c's pairs of
// expert e; offsets; active list.  Each thread reads its experts' counts in
// batches of GRP_SCAN_BATCH independent loads (one round trip per batch).
constexpr int GRP_SCAN_BATCH = 32;
__global__ __launch_bounds__(1024) void k_group_scan(GroupParams P) {
    __shared__ int s_part[1024];
    __shared__ int s_act[1024];
    const int tid = threadIdx.x;
    const int E = P.E, per = (E + 1023) / 1024;
    const int nc = P.nchunks;
    // per expert: total over chunks (independent loads)
    int tot[MOE_SCAN_PER_MAX];
    int my = 0, myact = 0;
    for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        int run = 0;
        if (e < E)
            for (int c0 = 0; c0 < nc; c0 += GRP_SCAN_BATCH) {  // independent loads per round trip
                uint32_t v[GRP_SCAN_BATCH];
#pragma unroll
                for (int j = 0; j < GRP_SCAN_BATCH; ++j)
                    v[j] = c0 + j < nc ? P.chunk_counts[(size_t)(c0 + j) * E + e] : 0u;
#pragma unroll
                for (int j = 0; j < GRP_SCAN_BATCH; ++j) run += (int)v[j];
            }
        tot[i] = run;
        my += run;
        myact += (run > 0);
    }
    s_part[tid] = my;
    s_act[tid] = myact;
    __syncthreads();
    // Hillis-Steele inclusive scans over the 1024 partial sums
    for (int off = 1; off < 1024; off <<= 1) {
        int a = tid >= off ? s_part[tid - off] : 0;
        int b = tid >= off ? s_act[tid - off] : 0;
        __syncthreads();
        s_part[tid] += a;
        s_act[tid] += b;
        __syncthreads();
    }
    int base = s_part[tid] - my, abase = s_act[tid] - myact;
    for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        if (e >= E) break;
        P.offsets[e] = base;
        // chunk c's first position: base + pairs of e in chunks before c
        // (a batch of counts read before any is overwritten)
        int run = base;
        for (int c0 = 0; c0 < nc; c0 += GRP_SCAN_BATCH) {
            uint32_t v[GRP_SCAN_BATCH];
#pragma unroll
            for (int j = 0; j < GRP_SCAN_BATCH; ++j)
                v[j] = c0 + j < nc ? P.chunk_counts[(size_t)(c0 + j) * E + e] : 0u;
#pragma unroll
            for (int j = 0; j < GRP_SCAN_BATCH; ++j) {
                if (c0 + j < nc) P.chunk_counts[(size_t)(c0 + j) * E + e] = (uint32_t)run;
                run += (int)v[j];
            }
        }
        if (tot[i] > 0) {
            P.active[1 + abase++] = e;
            // routing heat: this call's pairs of e (integer adds: any order)
            if (P.heat) atomicAdd(&P.heat[e], tot[i]);
        }
        base += tot[i];
    }
    if (tid == 1023) {
        P.offsets[E] = s_part[1023];
        P.active[0] = s_act[1023];
    }
}

// Each chunk places its pairs in (token, slot) order, 256 pairs per round,
// 64 per wave.  A pair's position is its expert's count before the round,
// plus the pairs of that expert in the earlier waves' batches of the round,
// plus the earlier ones in its own batch.  The chunk's expert ids are read
// into LDS first (one round of loads), padded with -1 to whole rounds.
constexpr int GRP_PLACE_THREADS = 256;

__global__ __launch_bounds__(GRP_PLACE_THREADS) void k_group_place(GroupParams P) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t *cnt = (uint32_t *)smem;               // [E]
    int *ids = (int *)(smem + ((4 * (size_t)P.E + 15) & ~(size_t)15));  // [chunk pairs rounded up to 256]
    const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t p0 = (int64_t)c * GRP_CHUNK_TOKENS * P.k;
    const int64_t p1 = min((int64_t)(c + 1) * GRP_CHUNK_TOKENS * P.k, (int64_t)P.T * P.k);
    const int n = (int)(p1 - p0);
    const int n_pad = (n + GRP_PLACE_THREADS - 1) / GRP_PLACE_THREADS * GRP_PLACE_THREADS;
    for (int e = tid; e < P.E; e += GRP_PLACE_THREADS) cnt[e] = P.chunk_counts[(size_t)c * P.E + e];
    for (int i = tid; i < n_pad; i += GRP_PLACE_THREADS) {
        const int e = i < n ? P.idx[p0 + i] : -1;
        ids[i] = (unsigned)e < (unsigned)P.E ? e : -1;  // ids outside [0, E) are not placed
    }
    __syncthreads();
    for (int b = 0; b < n; b += GRP_PLACE_THREADS) {
        const int i = b + 64 * wave + lane;
        const int e = ids[i];
        int dup = 0;
        bool later = false;
        for (int j = 0; j < 64; ++j) {
            const int ej = __builtin_amdgcn_readlane(e, j);
            dup += (j < lane) && (ej == e);
            later |= (j > lane) && (ej == e);
        }
        int prior = 0;
        for (int w2 = 0; w2 < wave; ++w2) {
            const u32x4 *row = (const u32x4 *)(ids + b + 64 * w2);
            for (int j = 0; j < 16; ++j) {
                const u32x4 v = row[j];
                prior += ((int)v.x == e) + ((int)v.y == e) + ((int)v.z == e) + ((int)v.w == e);
            }
        }
        const uint32_t base = e >= 0 ? cnt[e] : 0u;
        __syncthreads();
        if (e >= 0) {
            P.pairs[base + prior + dup] = (int32_t)(p0 + i);
            if (!later) atomicAdd(&cnt[e], (uint32_t)(dup + 1));  // this batch's pairs of e (a sum: any order)
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
hipError_t route_launch(const RouteParams &P, hipStream_t st) {
    const int grid = (P.T + 3) / 4;
    if (grid == 0) return hipSuccess;
    const int epl = (P.E + 63) / 64;
    if (epl <= 2) hipLaunchKernelGGL(k_route<2>, dim3(grid), dim3(256), 0, st, P);
    else if (epl <= 4) hipLaunchKernelGGL(k_route<4>, dim3(grid), dim3(256), 0, st, P);
    else if (epl <= 8) hipLaunchKernelGGL(k_route<8>, dim3(grid), dim3(256), 0, st, P);
    else if (epl <= 16) hipLaunchKernelGGL(k_route<16>, dim3(grid), dim3(256), 0, st, P);
    else if (epl <= 32) hipLaunchKernelGGL(k_route<32>, dim3(grid), dim3(256), 0, st, P);
    else hipLaunchKernelGGL(k_route<64>, dim3(grid), dim3(256), 0, st, P);
    return hipGetLastError();
}

hipError_t group_launch(const GroupParams &P, hipStream_t st) {
    const size_t lds = (size_t)P.E * 4;
    if (P.nchunks > 0) hipLaunchKernelGGL(k_group_count, dim3(P.nchunks), dim3(256), lds, st, P);
    hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, st, P);
    const size_t per_chunk = ((size_t)GRP_CHUNK_TOKENS * P.k + GRP_PLACE_THREADS - 1) / GRP_PLACE_THREADS *
                             GRP_PLACE_THREADS;
    const size_t lds_place = ((lds + 15) & ~(size_t)15) + per_chunk * 4;
    if (P.nchunks > 0)
        hipLaunchKernelGGL(k_group_place, dim3(P.nchunks), dim3(GRP_PLACE_THREADS), lds_place, st, P);
    return hipGetLastError();
}

}  // namespace moe
