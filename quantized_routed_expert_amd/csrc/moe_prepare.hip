// moe_prepare.hip -- one-time conversion of expert weights from the row-by-row
// block order (MOE_LAYOUT_ROWS) to the order the compute kernels read
// (MOE_LAYOUT_PREPARED): gate and up copied unchanged, the down projection's
// blocks reordered column-block-major.  Block format: a 32-weight block with
// an fp16 scale, 18 bytes (4-bit) or 14 bytes (3-bit), as in the thread
// "把 Strata 搬上 SGLang 引擎 的嘗試", §四.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

// Grid-stride over two kinds of work: 16-byte pieces of every expert's gate
// and up matrices (copied in place), then down blocks (moved from row-major
// index h*nc + c to index c*H + h).  Blocks are 2-byte aligned only, so they
// move as 16-bit halves.
__global__ void k_prepare(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, PrepareParams P) {
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t gu_pieces = P.gu_bytes / 16;  // per expert
    const size_t n_gu = gu_pieces * P.n_experts;
    for (size_t i = t0; i < n_gu; i += nthreads) {
        const size_t e = i / gu_pieces, q = i - e * gu_pieces;
        const size_t off = e * P.expert_bytes + q * 16;
        *(uint4 *)(dst + off) = *(const uint4 *)(src + off);
    }
    const size_t nblk = (size_t)P.H * P.nc;  // down blocks per expert
    const size_t n_dn = nblk * P.n_experts;
    const int halves = P.bb / 2;
    for (size_t i = t0; i < n_dn; i += nthreads) {
        const size_t e = i / nblk, j = i - e * nblk;  // j: destination index c*H + h
        const size_t c = j / P.H, h = j - c * P.H;
        const uint16_t *s = (const uint16_t *)(src + e * P.expert_bytes + P.gu_bytes + (h * P.nc + c) * P.bb);
        uint16_t *d = (uint16_t *)(dst + e * P.expert_bytes + P.gu_bytes + j * P.bb);
        for (int u = 0; u < halves; ++u) d[u] = s[u];
    }
}

hipError_t prepare_launch(const uint8_t *src, uint8_t *dst, const PrepareParams &P, hipStream_t st) {
    const size_t work = (size_t)P.n_experts * ((size_t)P.H * P.nc + P.gu_bytes / 16);
    size_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_prepare, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, P);
    return hipGetLastError();
}

}  // namespace moe
