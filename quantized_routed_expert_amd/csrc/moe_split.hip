// moe_split.hip -- the routed-expert layer for decode windows of one to four
// rows (at most 64 (row, expert) pairs), in one launch, split over 32-column
// slices of every expert's FFN.
//
// With so few rows the matrix cores would idle on most of their 16 rows,
// and the layer is a stream of quantized bytes: per row and weight it needs
// one multiply-add.  So this launch does integer dot products on the vector
// units instead (v_dot8_i32_i4: eight signed 4-bit products per instruction):
//  - activations x (and later h) are scaled per row by a power of two so the
//    largest |value| lies in [2^13, 2^14), rounded to integers (15 bits; the
//    relative rounding error is below 2^-14 of the row's largest value), and
//    cut into four signed radix-16 digits;
//  - 4-bit codes become signed nibbles (code - 8) with one xor; a 3-bit code
//    (0..7) is itself a nibble, with (code - 4) * a = code * a - 4a (the
//    block's sum of a is staged with the digits);
//  - a block's integer dot product is exact (it fits fp32's 24-bit
//    significand) and is scaled by the block's fp16 scale in fp32, the same
//    rounding point as the dequantized fp32 dot product of the pages;
//  - non-linear 4-bit codes become their table's signed bytes (byte-table
//    lookups), multiplied by two signed radix-256 digits of the activations
//    (v_dot4_i32_i8: four 8-bit products per instruction); the block's int32
//    sum is exact and rounds once (below 2^-24 relative) on its way to fp32.
//
// Work items: (expert, 32-column slice c of its FFN).  An item needs the 32
// gate rows and 32 up rows of the slice and column block c of down (the
// prepared down layout stores that column block contiguously): 3 * H * B
// bytes.  Each wave loads its own share of an item into registers, stages it
// in its own part of LDS and computes from it; the next item's loads are in
// flight during the current one.  The workgroup computes the slice's gate and
// up values, SwiGLU, and the slice's share of
// the down projection for all H output rows, and stores it as tagged words
// (value + call tag).  After all items, every workgroup sums a range of
// outputs over the slices (slice order fixed) and the k experts (top-k order)
// plus the shared expert: the same fixed order as the other launches, and no
// floating-point atomics.  Grouping (forum thread "把 Strata 搬上 SGLang 引擎
// 的嘗試", §二, the expert-scoped layout): only the experts some row routes
// to are read, each once per window.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int SPL_THREADS = 512;
constexpr int SPL_WAVES = SPL_THREADS / 64;

#ifdef MOE_PHASE_TRACE
// Phase timestamps (100 MHz device clock) per workgroup, analysis builds only.
__device__ uint64_t *g_trace_split = nullptr;
#define STRACE_INIT volatile uint64_t *const strace_buf = g_trace_split
#define STRACE(slot)                                                                                              \
    do {                                                                                                          \
        if (strace_buf && threadIdx.x == 0) strace_buf[blockIdx.x * 32 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
// per wave: slots base + wave (base 12 and 20, eight waves)
#define WTRACE(base)                                                                                              \
    do {                                                                                                          \
        if (strace_buf && (threadIdx.x & 63) == 0)                                                               \
            strace_buf[blockIdx.x * 32 + (base) + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime();        \
    } while (0)
extern "C" int moe_trace_split_set(void *buf) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_trace_split), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#else
#define STRACE_INIT \
    do {            \
    } while (0)
#define STRACE(slot) \
    do {             \
    } while (0)
#define WTRACE(base) \
    do {             \
    } while (0)
#endif

// ---------------------------------------------------------------------------
// Layouts for the integer dot products.  A "pair" is 64 consecutive k of a
// gate/up row (two blocks), or the same block of two consecutive down rows.
// Nibble-dwords: the 32-bit words whose eight nibbles multiply eight
// activation digits.  4-bit: the pair's 9 dwords (36 bytes) themselves;
// nibbles of scale bytes meet zero digits.  3-bit (28 bytes, 7 dwords): the
// whole codes, 8 per nibble-dword (8 nibble-dwords): per block, each of its
// two low-part dwords masked two ways (fields 0 and 2 of a byte, or 1 and 3)
// with the matching third bits spread in.
// ---------------------------------------------------------------------------
template <int BITS>
struct SFmt;
// non-linear 4-bit: the 4-bit pair's bytes; digit dwords [digit 2][parity 2][nibble-dword 9]
template <>
struct SFmt<MOE_FMT_NL4> {
    static constexpr int bb = 18, pb = 36, pw = 9, nnd = 9;
    static constexpr int xpd = 36;
    static constexpr int xps = 36;
};
template <>
struct SFmt<4> {
    static constexpr int bb = 18;   // bytes per block
    static constexpr int pb = 36;   // bytes per pair
    static constexpr int pw = 9;    // dwords per pair
    static constexpr int nnd = 9;   // nibble-dwords per pair
    static constexpr int xpd = 36;  // digit dwords per pair: [digit 4][nibble-dword 9]
    static constexpr int xps = 36;  // their stride in LDS
};
template <>
struct SFmt<3> {
    static constexpr int bb = 14;
    static constexpr int pb = 28;
    static constexpr int pw = 7;
    static constexpr int nnd = 8;
    static constexpr int xpd = 32;  // digit dwords per pair: [digit 4][nibble-dword 8]
    static constexpr int xps = 36;  // their stride in LDS (36 mod 64 banks spreads 8 pieces' reads)
};

// k (0..63 within the pair) that nibble i of nibble-dword nd multiplies, or -1.
template <int BITS>
__device__ __forceinline__ int nibble_k(int nd, int i) {
    const int h = i & 1;
    if constexpr (nib_layout(BITS)) {
        // byte 2+j of a block: code j (low nibble), code j+16 (high nibble)
        const int beta = 4 * nd + (i >> 1);
        if (beta >= 2 && beta <= 17) return beta - 2 + 16 * h;
        if (beta >= 20 && beta <= 35) return 32 + beta - 20 + 16 * h;
        return -1;  // a scale byte
    } else {
        // nibble-dword 4B + m of block B: byte j of the block's low-part dword
        // m >> 1 (bytes 4 (m >> 1) + j) holds the low bits of codes
        // 4 (m >> 1) + j + 8 f in its fields f = 0..3; mask m & 1 = 0 keeps
        // fields 0 and 2 (low and high nibble), 1 fields 1 and 3
        const int B = nd >> 2, m = nd & 3;
        return 32 * B + 8 * (m & 1) + 4 * (m >> 1) + (i >> 1) + 16 * (i & 1);
    }
}

// Digit dwords of nibble-dword nd from integer activations src[k & kmask]
// (kmask 63: a pair of blocks of one row; 31: one block read by two rows).
// Signed radix-16 digits n_j in [-8, 7] of v: with C = 8 * (1 + 16 + 16^2 +
// ...), v + C = sum (n_j + 8) 16^j, so nibble j of v + C is n_j + 8 and
// n_j as a 4-bit two's complement nibble is that nibble xor 8.  A missing
// value (v = 0) gives zero digits.
template <int BITS>
__device__ __forceinline__ void build_digits(const int16_t *src, int kmask, int nd, uint32_t *dst) {
    uint32_t D[4] = {0u, 0u, 0u, 0u};
    if constexpr (BITS == MOE_FMT_NL4) {
        // two signed radix-256 digits v = a0 + 256 a1 (a0 in [-128, 127],
        // |a1| <= 64); nibble i of the code dword is byte i/2 of the even
        // (i even) or the odd (i odd) code bytes: D[2 * digit + parity]
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = nibble_k<BITS>(nd, i);
            const int v = kk >= 0 ? (int)src[kk & kmask] : 0;
            const int a0 = (int)(int8_t)(v & 0xFF), a1 = (v - a0) >> 8;
            D[i & 1] |= (uint32_t)(a0 & 0xFF) << (8 * (i >> 1));
            D[2 + (i & 1)] |= (uint32_t)(a1 & 0xFF) << (8 * (i >> 1));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j * SFmt<BITS>::nnd + nd] = D[j];
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kk = nibble_k<BITS>(nd, i);
        int v = kk >= 0 ? (int)src[kk & kmask] : 0;
        const uint32_t u = (uint32_t)(v + 0x8888);  // |v| <= 2^14: four digits
#pragma unroll
        for (int j = 0; j < 4; ++j) D[j] |= ((u >> (4 * j)) & 15u) << (4 * i);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j * SFmt<BITS>::nnd + nd] = D[j] ^ 0x88888888u;
}

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// four codes (0..15, one per byte) -> their table's signed bytes (tb: the
// 16-byte table; entries 0..7 and 8..15 looked up apart, bit 3 choosing)
__device__ __forceinline__ uint32_t nl8_lookup(uint32_t c, const uint32_t *tb) {
    const uint32_t s = c & 0x07070707u;
    const uint32_t t = c & 0x08080808u;
    const uint32_t m = (t << 5) - (t >> 3);  // 0xFF in the bytes whose code is 8..15
    const uint32_t lo = __builtin_amdgcn_perm(tb[1], tb[0], s), hi = __builtin_amdgcn_perm(tb[3], tb[2], s);
    return (hi & m) | (lo & ~m);
}
// a0 + 16 a1 + 256 a2 + ...
template <int N>
__device__ __forceinline__ int radix16(const int (&a)[N]) {
    int v = a[N - 1];
#pragma unroll
    for (int j = N - 2; j >= 0; --j) v = (v << 4) + a[j];
    return v;
}

// Weights of one pair, unpacked once for all rows.
template <int BITS>
struct SPair;

template <>
struct SPair<MOE_FMT_NL4> {
    uint32_t be[9], bo[9];  // table bytes of the codes at even / odd nibbles of each code dword
    float d0, d1;
    __device__ __forceinline__ void set(const uint32_t (&w)[9], const uint32_t *tb) {
#pragma unroll
        for (int q = 0; q < 9; ++q) {  // (scale bytes give table bytes too: they meet zero digits)
            be[q] = nl8_lookup(w[q] & 0x0F0F0F0Fu, tb);
            bo[q] = nl8_lookup((w[q] >> 4) & 0x0F0F0F0Fu, tb);
        }
        d0 = half_bits_to_float(w[0] & 0xFFFFu);
        d1 = half_bits_to_float(w[4] >> 16);
    }
    __device__ __forceinline__ void blocks(const uint32_t *xd, int, int, int &A0, int &A1) const {
        int a0[2], a1[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int s0 = 0, s1 = 0;
#pragma unroll
            for (int q = 0; q < 5; ++q) {
                s0 = sdot4(be[q], xd[(2 * j) * 9 + q], s0);
                s0 = sdot4(bo[q], xd[(2 * j + 1) * 9 + q], s0);
            }
#pragma unroll
            for (int q = 5; q < 9; ++q) {
                s1 = sdot4(be[q], xd[(2 * j) * 9 + q], s1);
                s1 = sdot4(bo[q], xd[(2 * j + 1) * 9 + q], s1);
            }
            a0[j] = s0;
            a1[j] = s1;
        }
        A0 = a0[0] + (a0[1] << 8);
        A1 = a1[0] + (a1[1] << 8);
    }
};

template <>
struct SPair<4> {
    uint32_t wx[9];
    float d0, d1;
    __device__ __forceinline__ void set(const uint32_t (&w)[9]) {
#pragma unroll
        for (int q = 0; q < 9; ++q) wx[q] = w[q] ^ 0x88888888u;  // nibble c -> signed c - 8
        d0 = half_bits_to_float(w[0] & 0xFFFFu);
        d1 = half_bits_to_float(w[4] >> 16);
    }
    // exact integer dot products of block 0 and block 1 with a row's digits xd
    __device__ __forceinline__ void blocks(const uint32_t *xd, int, int, int &A0, int &A1) const {
        int a0[4], a1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int s0 = 0, s1 = 0;
#pragma unroll
            for (int q = 0; q < 5; ++q) s0 = sdot8(wx[q], xd[j * 9 + q], s0);
#pragma unroll
            for (int q = 5; q < 9; ++q) s1 = sdot8(wx[q], xd[j * 9 + q], s1);
            a0[j] = s0;
            a1[j] = s1;
        }
        A0 = radix16(a0);
        A1 = radix16(a1);
    }
};

template <>
struct SPair<3> {
    uint32_t C[8];  // the 64 codes, 8 per nibble-dword (order of nibble_k<3>)
    float d0, d1;
    __device__ __forceinline__ void set(const uint32_t (&w)[7]) {
        // block 0: bytes 0..13 (low parts 2..9, third bits 10..13); block 1: 14..27
        const uint32_t L[2][2] = {{__builtin_amdgcn_alignbyte(w[1], w[0], 2u), __builtin_amdgcn_alignbyte(w[2], w[1], 2u)},
                                  {w[4], w[5]}};
        const uint32_t Q[2] = {__builtin_amdgcn_alignbyte(w[3], w[2], 2u), w[6]};
        // bit q of t -> bit 2 of byte q: t * (4 + 2^9 + 2^16 + 2^23), the other
        // partial products land on bits the mask drops (all distinct: no carries)
        auto spread = [](uint32_t t) { return __umul24(t, 0x810204u) & 0x04040404u; };
#pragma unroll
        for (int B = 0; B < 2; ++B)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int c0 = 8 * (m & 1) + 4 * (m >> 1);  // code of byte 0's low nibble
                const uint32_t n = ((m & 1) ? L[B][m >> 1] >> 2 : L[B][m >> 1]) & 0x33333333u;
                const uint32_t tl = spread((Q[B] >> c0) & 15u), th = spread((Q[B] >> (c0 + 16)) & 15u);
                C[4 * B + m] = n | tl | (th << 4);
            }
        d0 = half_bits_to_float(w[0] & 0xFFFFu);
        d1 = half_bits_to_float(w[3] >> 16);
    }
    // S0, S1: the row's sums of the activations over block 0 / 1 (the -4a term)
    __device__ __forceinline__ void blocks(const uint32_t *xd, int S0, int S1, int &A0, int &A1) const {
        int a0[4], a1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int s0 = j == 0 ? -4 * S0 : 0, s1 = j == 0 ? -4 * S1 : 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) s0 = sdot8(C[q], xd[j * 8 + q], s0);
#pragma unroll
            for (int q = 4; q < 8; ++q) s1 = sdot8(C[q], xd[j * 8 + q], s1);
            a0[j] = s0;
            a1[j] = s1;
        }
        A0 = radix16(a0);
        A1 = radix16(a1);
    }
};

// 16-byte aligned
template <int N>
__device__ __forceinline__ void lds_read_b128(const uint8_t *p, uint32_t (&w)[N]) {
    static_assert(N % 4 == 0, "whole 16-byte reads");
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const u32x4 v = *(const u32x4 *)(p + 16 * i);
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// BG: bit width of the gate and up projections, BD: of the down projection
// (per-projection formats, as the thread's §三 decode table pairs them).
template <int BG, int BD, int TM, int XF32>
__global__ __launch_bounds__(SPL_THREADS, 1) void k_split_layer(SplitParams P) {
    using FG = SFmt<BG>;  // gate/up blocks and the activation digits
    using FD = SFmt<BD>;  // down blocks and the h digits
    constexpr int xps = FG::xps;
    static_assert(FG::xps == FD::xps, "one LDS stride for both digit layouts");
    extern __shared__ __align__(16) uint8_t smem[];
    SplitSmall &sm = *(SplitSmall *)(smem + P.lds_small);
    uint8_t *s_wt = smem + P.lds_wt;                    // item weights: gate rows | up rows | down column
    int16_t *s_a = (int16_t *)(smem + P.lds_a);         // [T][H] integer activations
    int *s_S = (int *)(smem + P.lds_S);                 // [T][H/32] block sums (3-bit)
    // [T][H/64 pair slots][xps] activation digits; pair 4m + j of a row sits in
    // slot j * (H/256) + m, so the pieces m = 0, 1, ... that the lanes of a
    // wave read together are xps dwords apart (distinct LDS banks)
    uint32_t *s_xd = (uint32_t *)(smem + P.lds_xd);
    float *s_gu = (float *)(smem + P.lds_gu);           // [T][64] gate then up values of the slice
    int16_t *s_ah = (int16_t *)(smem + P.lds_ah);       // [T][32] integer h of the slice
    uint32_t *s_hd = (uint32_t *)(smem + P.lds_hd);     // [T][xps] h digits

    // (the wave index read into a scalar: branches on it are uniform)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x;
    const int k = P.k, E = P.E, H = P.H;
    const int T = P.T;  // rows of the window, 1 <= T <= TM
    const int TK = T * k;
    const bool has_shared = (P.mode & DEC_MODE_SHARED) != 0;
    const int hs = has_shared ? 1 : 0;
    const bool route_mode = (P.mode & DEC_MODE_ROUTE) != 0;
    const int nc = P.nc, ncs = has_shared ? P.ncs : 0;
    const int RD = H * FD::bb;          // bytes of an item's down column block: H blocks
    const int npairs = H >> 6;          // pairs per gate/up row
    // gate/up tasks: qpr pieces of 4 consecutive pairs per row (H / 256)
    const int lg_qpr = P.lg_qpr, qpr = 1 << lg_qpr;
    const size_t eb = P.eb;             // bytes of a routed expert blob

    // ---- item -> (slot, column slice) and its three regions in global memory
    auto item_slot = [&](int it, int &c) {
        if (it < ncs) {
            c = it;
            return 0;
        }
        const int j = it - ncs;
        const int s = nc == 1 ? j : (int)__umulhi((uint32_t)j, P.m_nc);
        c = j - s * nc;
        return hs + s;
    };
    // Each wave owns a share of an item end to end: 8 of its 64 gate/up rows
    // (waves 0-3 gate rows 8w.., waves 4-7 up rows) and H/8 of its down rows.
    // Both go straight into the wave's own runs of LDS: NGU and ND
    // direct-to-LDS loads of 16 bytes per lane, 1 KB per load (lanes past
    // the rows load into the run's unused tail).  A wave computes its rows as
    // soon as their loads have landed: no other wave's data is waited for
    // until the gate/up values are complete.  The loads of a wave complete in
    // issue order, so the number of loads issued after a given one bounds the
    // wave's wait for it (stores in between only lengthen such a wait).  The
    // gate/up run is reloaded for the wave's next item as soon as the wave
    // has read it; the down run is loaded once the item's gate/up rows have
    // landed (so that all workgroups' gate/up bytes stream first).
    constexpr int NGU = nib_layout(BG) ? 9 : 7;  // ceil(8 rows * rowH / 16 / 64) at H = 2048
    constexpr int ND = nib_layout(BD) ? 5 : 4;   // ceil(H/8 rows * bb / 16 / 64) at H = 2048
    constexpr int GUB = 8 * NGU * 1024;     // bytes of the gate/up runs (the down runs follow)
    const int npw = (8 * P.rowH) >> 4;      // pieces of a wave's 8 gate/up rows
    const int npd = (H * FD::bb) >> 7;      // pieces of a wave's H/8 down rows
    lds_u8 *const s_gu_run = (lds_u8 *)s_wt + (size_t)wave * NGU * 1024;
    lds_u8 *const s_dn_run = (lds_u8 *)s_wt + GUB + (size_t)wave * ND * 1024;
    // parts: 1 this wave's gate/up rows, 2 its down rows; e: the routed expert, -1: the shared one
    auto issue_item_e = [&](int c, int e, int parts) {
        const bool sh = e < 0;
        const int Fx = sh ? P.Fs : P.F;
        const uint8_t *blob = sh ? P.w_shared : P.w_routed + (size_t)e * eb;
        if (parts & 1) {
            const int row0 = wave < 4 ? 32 * c + 8 * wave : Fx + 32 * c + 8 * (wave - 4);
            const uint8_t *g0 = blob + (size_t)row0 * P.rowH;
#pragma unroll
            for (int i = 0; i < NGU; ++i) {
                const int pc = lane + 64 * i, q = pc < npw ? pc : 0;
                __builtin_amdgcn_global_load_lds(g0 + (size_t)q * 16, s_gu_run + 1024 * i, 16, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // (keep the issue order)
        if (parts & 2) {
            const uint8_t *d0 = blob + (size_t)2 * Fx * P.rowH + (size_t)c * RD + (size_t)wave * (H >> 3) * FD::bb;
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                const int pc = lane + 64 * i, q = pc < npd ? pc : 0;
                __builtin_amdgcn_global_load_lds(d0 + (size_t)q * 16, s_dn_run + 1024 * i, 16, 0, 0);
            }
        }
    };
    auto issue_item = [&](int it, int parts) {
        int c;
        const int s = item_slot(it, c);
        issue_item_e(c, s < hs ? -1 : sm.slot_exp[s], parts);
    };

    // ======================= Phase A: routing, activations, slots =======================
    STRACE_INIT;
    STRACE(0);
    // the call's tag is read after the routing loads are issued (it is first
    // needed by the partial stores, so its load does not delay the logits)
    uint32_t tag_v = 0u;

    // activations: thread tid holds the groups of 8 elements g = tid + 512 r
    // of [T][H] (r < XR)
    constexpr int XR = TM > 2 ? 2 : 1;  // (T * H / 8 <= 512 * XR for H <= 2048)
    const int nx = T * H;
    bool has_x[XR];
    int xt[XR], xk[XR];
    float xv[XR][8];
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        const int e0 = 8 * (tid + SPL_THREADS * r);
        has_x[r] = e0 < nx;
        xt[r] = has_x[r] ? e0 / H : 0;
        xk[r] = has_x[r] ? e0 - xt[r] * H : 0;
    }
    auto load_x = [&]() {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int e0 = has_x[r] ? 8 * (tid + SPL_THREADS * r) : 0;
            if constexpr (XF32) {
                const u32x4 a = *(const u32x4 *)((const float *)P.x + e0);
                const u32x4 b = *(const u32x4 *)((const float *)P.x + e0 + 4);
                const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) xv[r][i] = __builtin_bit_cast(float, wv[i]);
            } else {
                const u32x4 a = *(const u32x4 *)((const uint16_t *)P.x + e0);
                const uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xv[r][2 * i] = __builtin_bit_cast(float, wv[i] << 16);
                    xv[r][2 * i + 1] = __builtin_bit_cast(float, wv[i] & 0xFFFF0000u);
                }
            }
        }
    };
    if (route_mode && wave < T) {
        // routing of row `wave` by this wave: logits first, then its
        // activations and the call's tag
        const int epl = (E + 63) >> 6;
        auto route_wave = [&](auto epl_c) {
            constexpr int EPL = decltype(epl_c)::value;
            float lv[EPL];
            route_load<EPL>(P.logits + (size_t)wave * E, E, lane, lv);
            load_x();
            tag_v = epoch_read(P.epoch);
            STRACE(10);
            uint32_t key[EPL];
            route_keys_of<EPL>(lv, E, lane, key);
            route_pick<EPL>(key, k, sm.idx + wave * k, sm.w + wave * k, lane);
            STRACE(11);
        };
        if (epl <= 2) route_wave(std::integral_constant<int, 2>{});
        else if (epl <= 4) route_wave(std::integral_constant<int, 4>{});
        else if (epl <= 8) route_wave(std::integral_constant<int, 8>{});
        else route_wave(std::integral_constant<int, 16>{});
    } else {
        load_x();
        tag_v = epoch_read(P.epoch);
    }
    {
        // per wave and row: the largest |x|
        uint32_t mb[XR];
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(xv[r][i]));
            mb[r] = has_x[r] ? __builtin_bit_cast(uint32_t, m) : 0u;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            uint32_t v = 0u;
#pragma unroll
            for (int r = 0; r < XR; ++r) v = max(v, xt[r] == t ? mb[r] : 0u);
            const uint32_t wm = wave_max_u32(v);
            if (lane == 0) sm.wmax[wave][t] = wm;
        }
    }
    // the shared expert's items need no routing: their weights stream in now
    if ((int)blockIdx.x < ncs) issue_item_e(blockIdx.x, -1, 1);
    lds_barrier();  // routing and the row maxima complete
    STRACE(1);
    const uint32_t tag = decode_tag(__builtin_amdgcn_readfirstlane(tag_v));
    // a one-row window: its first routed item is known from the routing alone
    // (slot hs + j is the row's j-th expert)
    int it = blockIdx.x;
    const bool early = T == 1 && route_mode;
    if (early) {
        const int n_items1 = ncs + k * nc;
        if (it < n_items1 && it >= ncs) {
            const int j = it - ncs, sl = nc == 1 ? j : (int)__umulhi((uint32_t)j, P.m_nc);
            issue_item_e(j - sl * nc, sm.idx[sl], 1);
        }
    }

    // integer activations a = rint(x * 2^sc), max |x| * 2^sc in [2^13, 2^14)
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        uint32_t mxb = 0u;
#pragma unroll
        for (int w = 0; w < SPL_WAVES; ++w) mxb = max(mxb, sm.wmax[w][xt[r]]);
        const float mx = __builtin_bit_cast(float, mxb);
        int ex = 0;
        if (mx > 0.0f) frexpf(mx, &ex);
        // (ldexp: exact for any sc, also where 2^sc is not a normal float)
        const int sc = mx > 0.0f ? 14 - ex : 0;
        int ai[8], bs = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ai[i] = (int)rintf(ldexpf(xv[r][i], sc));
            bs += ai[i];
        }
        if (has_x[r]) {
            const u32x4 pk = {(uint32_t)(ai[0] & 0xFFFF) | ((uint32_t)ai[1] << 16),
                              (uint32_t)(ai[2] & 0xFFFF) | ((uint32_t)ai[3] << 16),
                              (uint32_t)(ai[4] & 0xFFFF) | ((uint32_t)ai[5] << 16),
                              (uint32_t)(ai[6] & 0xFFFF) | ((uint32_t)ai[7] << 16)};
            *(u32x4 *)(s_a + xt[r] * H + xk[r]) = pk;
            if (xk[r] == 0) sm.tsc[xt[r]] = sc;
        }
        if (BG == 3) {
            // block sums: the four threads of a block are consecutive lanes
            bs += __builtin_amdgcn_update_dpp(0, bs, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
            bs += __builtin_amdgcn_update_dpp(0, bs, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
            if (has_x[r] && (tid & 3) == 0) s_S[xt[r] * (H >> 5) + (xk[r] >> 5)] = bs;
        }
    }

    // slots: the shared expert (slot 0 when present), then the routed experts
    // in order of first use (row 0's top-k order, then each later row's new
    // ones); pick p = t*k + j (T*k <= 64: one lane each)
    if (wave == 0) {
        if (route_mode) {
            const int p = lane;
            const bool valid = p < TK;
            const int e = valid ? sm.idx[p] : -1;
            int t = 0;
            while (t + 1 < T && (t + 1) * k <= p) ++t;
            // the first pick of this expert (a row's own picks are distinct)
            int first = p;
            if (valid)
                for (int q = t * k - 1; q >= 0; --q)
                    if (sm.idx[q] == e) first = q;
            const bool owner = valid && first == p;
            const uint64_t om = __ballot(owner);
            if (owner) {
                const int slot = hs + __popcll(om & ((1ull << lane) - 1ull));
                sm.slot_exp[slot] = e;
#pragma unroll
                for (int tt = 0; tt < TM; ++tt) sm.slot_pair[slot][tt] = tt == t ? p : -1;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (valid && !owner)  // a later row's pick of an expert an earlier row chose
                sm.slot_pair[hs + __popcll(om & ((1ull << first) - 1ull))][t] = p;
            if (lane == 0) sm.n_slots = hs + __popcll(om);
        } else {
            // a grouping given by the caller, sanitized so that bad entries
            // give a wrong answer (and err bit 1) but never an access out of bounds
            int na = P.g_active[0];
            const int lim = min(E, TK);
            if (na < 0 || na > lim) {
                if (lane == 0) atomicOr(P.err, 2u);
                na = na < 0 ? 0 : lim;
            }
            for (int a = lane; a < na; a += 64) {
                int e = P.g_active[1 + a];
                int st = 0, cnt = 0;
                if (e >= 0 && e < E) {
                    st = P.g_offsets[e];
                    cnt = P.g_offsets[e + 1] - st;
                }
                if (e < 0 || e >= E || st < 0 || cnt < 0 || cnt > T || st + cnt > TK) {
                    atomicOr(P.err, 2u);
                    e = (e >= 0 && e < E) ? e : 0;
                    cnt = 0;
                }
                sm.slot_exp[hs + a] = e;
                int pr[TM];
#pragma unroll
                for (int t = 0; t < TM; ++t) pr[t] = -1;
                for (int q = 0; q < cnt; ++q) {
                    int p = P.g_pairs[st + q];
                    if (p < 0 || p >= TK) {
                        atomicOr(P.err, 2u);
                        continue;
                    }
                    int t = 0;
                    while (t + 1 < T && (t + 1) * k <= p) ++t;
#pragma unroll
                    for (int tt = 0; tt < TM; ++tt)
                        if (tt == t) pr[tt] = p;
                }
#pragma unroll
                for (int t = 0; t < TM; ++t) sm.slot_pair[hs + a][t] = pr[t];
            }
            for (int p = lane; p < TK; p += 64) sm.w[p] = P.g_pair_w ? P.g_pair_w[p] : 1.0f;
            if (lane == 0) sm.n_slots = hs + na;
        }
        if (lane == 0 && has_shared) {
            sm.slot_exp[0] = -1;
#pragma unroll
            for (int t = 0; t < TM; ++t) sm.slot_pair[0][t] = t < T ? TK + t : -1;
        }
        if (!(P.mode & DEC_MODE_COMBINE)) {
            // the pairs present, for the per-pair outputs
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane == 0) {
                int n = 0;
                for (int s = 0; s < sm.n_slots; ++s)
                    for (int t = 0; t < TM; ++t)
                        if (sm.slot_pair[s][t] >= 0) sm.plist[n++] = sm.slot_pair[s][t];
                sm.n_pl = n;
            }
        }
    }
    if (blockIdx.x == 0 && route_mode && wave == 1) {
        for (int p = lane; p < TK; p += 64) {
            if (P.topk_idx_out) P.topk_idx_out[p] = sm.idx[p];
            if (P.topk_w_out) P.topk_w_out[p] = sm.w[p];
            if (P.heat) atomicAdd(&P.heat[sm.idx[p]], 1);  // routing heat (integer adds: any order)
        }
    }
    lds_barrier();  // slots, integer activations, block sums
    STRACE(2);
    const int n_slots = sm.n_slots;
    const int n_items = ncs + (n_slots - hs) * nc;
    if (!early && it < n_items && it >= ncs) issue_item(it, 1);

    // activation digits: (row, pair, nibble-dword) tasks
    {
        const int ntask = T * npairs * FG::nnd;
        for (int q = tid; q < ntask; q += SPL_THREADS) {
            const int t = q / (npairs * FG::nnd);
            const int r = q - t * npairs * FG::nnd;
            const int pr = r / FG::nnd, nd = r - pr * FG::nnd;
            const int slot = (pr & 3) * qpr + (pr >> 2);
            build_digits<BG>(s_a + t * H + pr * 64, 63, nd, s_xd + ((size_t)t * npairs + slot) * xps);
        }
    }

    lds_barrier();  // activation digits complete
    // ======================= Phase B: items =======================
    int my_items = 0;  // (for the trace points)
    for (; it < n_items; it += G) {
        int c;
        const int s = item_slot(it, c);
        const int nxt = it + G;  // (its loads go out while this item computes)
        bool row_in[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) row_in[t] = sm.slot_pair[s][t] >= 0;

        // gate/up: this wave's 8 rows once its gate/up loads have landed; only
        // then are the item's down rows issued, so the gate/up bytes of every
        // workgroup stream first and the down rows stream while the gate/up
        // values, SwiGLU and the h digits are computed.  Lane (row r, run m of
        // ppl consecutive pairs): lpr lanes per row (8, or 4 at H = 256), so
        // every lane of the 8 rows is busy at every H.
        {
            const lds_u8 *wr = s_gu_run;
            const int lpr = H >= 512 ? 8 : 4;  // lanes per row
            const int ppl = (H >> 6) / lpr;     // pairs per lane: 1, 2 or 4
            const int r = lane / lpr, m = lane - r * lpr;
            wait_vm_n(0);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the previous item's down rows are read
            issue_item(it, 2);
            if (my_items == 0) WTRACE(12);
            if (r < 8) {
                float acc[TM];
#pragma unroll
                for (int t = 0; t < TM; ++t) acc[t] = 0.0f;
                // the lane's run of pairs: 16-byte reads when it holds 4 pairs
                // (144 or 112 bytes at a 16-byte aligned offset), else dwords
                uint32_t wq[4 * FG::pw];
                const lds_u8 *run = wr + (size_t)r * P.rowH + (size_t)m * ppl * FG::pb;
                if (ppl == 4) {
#pragma unroll
                    for (int i = 0; i < FG::pw; ++i) {
                        const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(run + 16 * i);
                        wq[4 * i] = v.x;
                        wq[4 * i + 1] = v.y;
                        wq[4 * i + 2] = v.z;
                        wq[4 * i + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 2 * FG::pw; ++i)
                        wq[i] = i < ppl * FG::pw ? *(const __attribute__((address_space(3))) uint32_t *)(run + 4 * i) : 0u;
                }
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    if (pp >= ppl) break;
                    const int pr = m * ppl + pp, slot = (pr & 3) * qpr + (pr >> 2);
                    uint32_t w[FG::pw];
#pragma unroll
                    for (int i = 0; i < FG::pw; ++i) w[i] = wq[pp * FG::pw + i];
                    SPair<BG> sp;
                    if constexpr (BG == MOE_FMT_NL4) sp.set(w, P.nl8);
                    else sp.set(w);
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        if (!row_in[t]) continue;  // (uniform over the workgroup)
                        uint32_t xd[FG::xpd];
                        lds_read_b128<FG::xpd>((const uint8_t *)(s_xd + ((size_t)t * npairs + slot) * xps), xd);
                        const int S0 = BG == 3 ? s_S[t * (H >> 5) + 2 * pr] : 0;
                        const int S1 = BG == 3 ? s_S[t * (H >> 5) + 2 * pr + 1] : 0;
                        int A0, A1;
                        sp.blocks(xd, S0, S1, A0, A1);
                        acc[t] = fmaf(sp.d0, (float)A0, acc[t]);
                        acc[t] = fmaf(sp.d1, (float)A1, acc[t]);
                    }
                }
                // sum over the row's lpr lanes (consecutive lanes; a fixed tree)
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    float v = acc[t];
                    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
                    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
                    if (lpr >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
                    if (m == 0) s_gu[t * 64 + 8 * wave + r] = v;
                }
            }
            // the gate/up run is free again: the next item's gate/up rows
            if (nxt < n_items) {
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                issue_item(nxt, 1);
            }
        }
        if (my_items == 0) WTRACE(20);
        lds_barrier();  // gate/up values
        if (my_items == 0) STRACE(4);

        // SwiGLU and the h digits: wave t for row t
        if (wave < T) {
            const int t = wave;
            float h = 0.0f;
            if (lane < 32) {
                const int tsc = sm.tsc[t];
                const float g = ldexpf(s_gu[t * 64 + lane], -tsc), u = ldexpf(s_gu[t * 64 + 32 + lane], -tsc);
                h = g / (1.0f + expf(-g)) * u;
            }
            const float mx = __builtin_bit_cast(float, wave_max_u32(__builtin_bit_cast(uint32_t, fabsf(h))));
            int ex = 0;
            if (mx > 0.0f) frexpf(mx, &ex);
            const int sc = mx > 0.0f ? 14 - ex : 0;
            const int ah = (int)rintf(ldexpf(h, sc));
            if (lane < 32) s_ah[t * 32 + lane] = (int16_t)ah;
            if (BD == 3) {
                int sum = ah;
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
                if (lane == 0) sm.Sh[t] = sum;
            }
            if (lane == 0) sm.hsc[t] = sc;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < FD::nnd) build_digits<BD>(s_ah + t * 32, 31, lane, s_hd + t * xps);
        }
        lds_barrier();  // h digits
        if (my_items == 0) STRACE(5);

        // down: this wave's H/8 rows of column block c, as row pairs (2 rp, 2 rp + 1);
        // partial rows stored tagged
        {
            // this item's down rows have landed (the next item's gate/up loads,
            // issued after them, may still be in flight)
            wait_vm_n(nxt < n_items ? NGU : 0);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const lds_u8 *dcol = s_dn_run - (size_t)wave * (H >> 4) * FD::pb;  // (indexed by the global rp)
            int pid[TM];
            int hsc[TM];
            int Sh[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                pid[t] = sm.slot_pair[s][t];
                hsc[t] = sm.hsc[t];
                Sh[t] = BD == 3 ? sm.Sh[t] : 0;
            }
            // h digits in registers for one or two rows; re-read (LDS broadcast) for more
            constexpr int HR = TM <= 2 ? TM : 1;
            uint32_t hd[HR][FD::xpd];
            if constexpr (TM <= 2) {
#pragma unroll
                for (int t = 0; t < TM; ++t) lds_read_b128<FD::xpd>((const uint8_t *)(s_hd + t * xps), hd[t]);
            }
            for (int rp = wave * (H >> 4) + lane; rp < (wave + 1) * (H >> 4); rp += 64) {
                uint32_t w[FD::pw];
                const lds_u8 *pp8 = dcol + (size_t)rp * FD::pb;
#pragma unroll
                for (int i = 0; i < FD::pw; ++i) w[i] = *(const __attribute__((address_space(3))) uint32_t *)(pp8 + 4 * i);
                SPair<BD> sp;
                if constexpr (BD == MOE_FMT_NL4) sp.set(w, P.nl8);
                else sp.set(w);
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (pid[t] < 0) continue;
                    // the pair's two blocks are the rows 2rp and 2rp + 1
                    int A0, A1;
                    if constexpr (TM <= 2) {
                        sp.blocks(hd[t], Sh[t], Sh[t], A0, A1);
                    } else {
                        lds_read_b128<FD::xpd>((const uint8_t *)(s_hd + t * xps), hd[0]);
                        sp.blocks(hd[0], Sh[t], Sh[t], A0, A1);
                    }
                    // partial layout [pair][row / 8][slice][row % 8]: rows 2rp, 2rp+1 adjacent
                    uint64_t *dst = P.part + (((size_t)pid[t] * (H >> 3) + (rp >> 2)) * P.ncmax + c) * 8 + 2 * (rp & 3);
                    st_tagged(dst, ldexpf(sp.d0 * (float)A0, -hsc[t]), tag);
                    st_tagged(dst + 1, ldexpf(sp.d1 * (float)A1, -hsc[t]), tag);
                }
            }
        }
        if (my_items == 0) STRACE(6);
        ++my_items;
        // (no barrier: every wave reuses only its own staging area; the shared
        // gate/up values and h digits are next written after a barrier that
        // every wave reaches only once its down rows are done)
    }

    // ======================= Phase C: sums over the slices =======================
    // every wave is done with the item area (its LDS is reused below); the
    // partial stores need not have completed: the readers check the tags
    lds_barrier();
    STRACE(7);
    // outputs: COMBINE: (row t, output h) -> y; else (present pair, output h)
    const bool combine = (P.mode & DEC_MODE_COMBINE) != 0;
    const int n_out = combine ? T * H : sm.n_pl * H;
    const int u0 = blockIdx.x * P.units;
    const int nu = max(0, min(P.units, n_out - u0));
    const int nterm = combine ? k + hs : 1;
    const int ncm = P.ncmax;
    // units come in chunks of 8 outputs (8 consecutive rows of one pair or
    // row), which is how the partials are laid out: a term of a chunk is
    // ncx * 8 consecutive words
    const int nchk = nu >> 3;
    float *s_val = (float *)s_wt;                         // [chunk][term][slice][8]
    float *s_red = s_val + (size_t)nchk * nterm * ncm * 8;  // [unit][term]
    auto term = [&](int g, int j, int &p, float &wgt, int &rowc) {  // chunk g, term j
        const int u = u0 + 8 * g, t = u / H;
        rowc = (u - t * H) >> 3;
        if (combine) {
            p = j < k ? t * k + j : TK + t;
            wgt = j < k ? sm.w[p] : 1.0f;
        } else {
            p = sm.plist[t];
            wgt = p < TK ? sm.w[p] : 1.0f;
        }
    };
    // per (output, term): the sum over the slices in slice order, times the
    // router weight.  With many (output, term) pairs (windows of three or four
    // rows) each pair's thread reads its slices' words straight into
    // registers; with few, every thread of the workgroup polls a share of the
    // words and the sums read them from LDS (more threads polling).  (The
    // direct form is compiled only where it can be taken: its registers cost
    // the one- and two-row kernels time even unused.)
    bool direct = false;
    if constexpr (TM >= 3) direct = nu * nterm >= 256;
    if (direct) {
        const int per_term = ncm * 8;
        constexpr int RB = 24;  // words in flight per thread
        for (int q = tid; q < nu * nterm; q += SPL_THREADS) {
            const int ul = q / nterm, j = q - ul * nterm;
            const int g = ul >> 3, rr = ul & 7;
            int p, rowc;
            float wgt;
            term(g, j, p, wgt, rowc);
            const int ncx = p >= TK ? ncs : nc;
            const uint64_t *src = P.part + ((size_t)p * (H >> 3) + rowc) * per_term + rr;  // slice c: word 8 c
            float sum = 0.0f;
            for (int c0 = 0; c0 < ncx; c0 += RB) {
                uint64_t wd[RB];
#pragma unroll
                for (int i = 0; i < RB; ++i) wd[i] = c0 + i < ncx ? ld_dev_u64(src + 8 * (c0 + i)) : 0ull;
                for (uint32_t spins = 0;; ++spins) {
                    bool ok = true;
#pragma unroll
                    for (int i = 0; i < RB; ++i) ok = ok && (c0 + i >= ncx || (uint32_t)(wd[i] >> 32) == tag);
                    if (ok) break;
                    if (spins > DEC_SPIN_LIMIT) {
                        note_timeout(P.err, tag);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(4);
#pragma unroll
                    for (int i = 0; i < RB; ++i)
                        if (c0 + i < ncx && (uint32_t)(wd[i] >> 32) != tag) wd[i] = ld_dev_u64(src + 8 * (c0 + i));
                }
#pragma unroll
                for (int i = 0; i < RB; ++i)
                    if (c0 + i < ncx) sum += __builtin_bit_cast(float, (uint32_t)wd[i]);
            }
            s_red[q] = wgt * sum;
            if (!combine) {
                const int u = u0 + ul, t = u / H, row = u - t * H;
                if (p < TK) P.out_pairs[(size_t)p * H + row] = wgt * sum;
                else P.out_shared[(size_t)(p - TK) * H + row] = sum;
            }
        }
    } else {
        {
            // every word in flight at once (consecutive threads on consecutive
            // words), words not yet written by this call read again
            const int per_term = ncm * 8, nw = nchk * nterm * per_term;
            for (int q0 = tid; q0 < nw; q0 += 4 * SPL_THREADS) {
                uint64_t wd[4];
                const uint64_t *src[4];
                bool need[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = q0 + i * SPL_THREADS;
                    const int r = q % per_term, gj = q / per_term;
                    const int g = gj / nterm, j = gj - g * nterm;
                    int p = 0, rowc = 0;
                    float wgt;
                    if (q < nw) term(g, j, p, wgt, rowc);
                    need[i] = q < nw && (r >> 3) < (p >= TK ? ncs : nc);
                    src[i] = P.part + ((size_t)p * (H >> 3) + rowc) * per_term + (need[i] ? r : 0);
                    wd[i] = need[i] ? ld_dev_u64(src[i]) : 0ull;
                }
                for (uint32_t spins = 0;; ++spins) {
                    bool ok = true;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ok = ok && (!need[i] || (uint32_t)(wd[i] >> 32) == tag);
                    if (ok) break;
                    if (spins > DEC_SPIN_LIMIT) {
                        note_timeout(P.err, tag);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (need[i] && (uint32_t)(wd[i] >> 32) != tag) wd[i] = ld_dev_u64(src[i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (q0 + i * SPL_THREADS < nw) s_val[q0 + i * SPL_THREADS] = __builtin_bit_cast(float, (uint32_t)wd[i]);
            }
        }
        __syncthreads();
        // per (output, term): the sum over the slices in slice order, times the router weight
        for (int q = tid; q < nu * nterm; q += SPL_THREADS) {
            const int ul = q / nterm, j = q - ul * nterm;
            const int g = ul >> 3, rr = ul & 7;
            int p, rowc;
            float wgt;
            term(g, j, p, wgt, rowc);
            const int ncx = p >= TK ? ncs : nc;
            const float *v = s_val + ((size_t)g * nterm + j) * ncm * 8 + rr;
            float sum = 0.0f;
            for (int c0 = 0; c0 < ncx; c0 += 8) {  // eight reads in flight, added in order
                float vv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) vv[i] = c0 + i < ncx ? v[(c0 + i) * 8] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (c0 + i < ncx) sum += vv[i];
            }
            s_red[q] = wgt * sum;
            if (!combine) {
                const int u = u0 + ul, t = u / H, row = u - t * H;
                if (p < TK) P.out_pairs[(size_t)p * H + row] = wgt * sum;
                else P.out_shared[(size_t)(p - TK) * H + row] = sum;
            }
        }
    }
    STRACE(8);
    if (combine) {
        __syncthreads();
        for (int ul = tid; ul < nu; ul += SPL_THREADS) {
            const float *r = s_red + ul * nterm;
            float v = r[0];
            for (int j0 = 1; j0 < nterm; j0 += 8) {  // eight reads in flight, added in order
                float vv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) vv[i] = j0 + i < nterm ? r[j0 + i] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (j0 + i < nterm) v += vv[i];
            }
            P.y[u0 + ul] = v;
        }
    }

    // ---- end of call: the workspace moves on to the next call's tag
    STRACE(9);
    if (tid == 0) epoch_advance(P.epoch, __builtin_amdgcn_readfirstlane(tag_v));
}

template <int BG, int BD, int TM, int XF32>
static hipError_t split_launch_t(const SplitParams &P, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_split_layer<BG, BD, TM, XF32>), dim3(grid), dim3(SPL_THREADS), P.lds_total, st, P);
    return hipGetLastError();
}

template <int BG, int BD, int TM, int XF32>
static hipError_t split_attr_t(int lds) {
    return hipFuncSetAttribute((const void *)k_split_layer<BG, BD, TM, XF32>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

// compile-time formats (gate/up bits, down bits) and row maximum TM: 1, 2 or 4
#define SPLIT_DISPATCH_T(FN, BG, BD, ...)                                                        \
    do {                                                                                         \
        if (T == 1) return xf ? FN<BG, BD, 1, 1>(__VA_ARGS__) : FN<BG, BD, 1, 0>(__VA_ARGS__);   \
        if (T == 2) return xf ? FN<BG, BD, 2, 1>(__VA_ARGS__) : FN<BG, BD, 2, 0>(__VA_ARGS__);   \
        return xf ? FN<BG, BD, 4, 1>(__VA_ARGS__) : FN<BG, BD, 4, 0>(__VA_ARGS__);               \
    } while (0)
#define SPLIT_DISPATCH(FN, ...)                                           \
    do {                                                                  \
        if (bg == 4 && bd == 4) SPLIT_DISPATCH_T(FN, 4, 4, __VA_ARGS__);  \
        if (bg == 3 && bd == 4) SPLIT_DISPATCH_T(FN, 3, 4, __VA_ARGS__);  \
        if (bg == 4 && bd == 3) SPLIT_DISPATCH_T(FN, 4, 3, __VA_ARGS__);  \
        if (bg == 3 && bd == 3) SPLIT_DISPATCH_T(FN, 3, 3, __VA_ARGS__);  \
        if (bg == MOE_FMT_NL4 && bd == MOE_FMT_NL4)                       \
            SPLIT_DISPATCH_T(FN, MOE_FMT_NL4, MOE_FMT_NL4, __VA_ARGS__);  \
        if (bg == 3 && bd == MOE_FMT_NL4)                                 \
            SPLIT_DISPATCH_T(FN, 3, MOE_FMT_NL4, __VA_ARGS__);            \
        return hipErrorInvalidValue;                                      \
    } while (0)

hipError_t split_launch(const SplitParams &P, int grid, hipStream_t st) {
    const int bg = P.bits, bd = P.dbits, T = P.T, xf = P.x_f32;
    SPLIT_DISPATCH(split_launch_t, P, grid, st);
}

hipError_t split_set_lds(int bg, int bd, int T, int xf, int lds) { SPLIT_DISPATCH(split_attr_t, lds); }

}  // namespace moe
