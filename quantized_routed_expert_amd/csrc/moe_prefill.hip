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
//                    outputs (down).  Each K step's weight bytes and the
//                    activation rows of the group (gathered by its row list)
//                    stream into a ring of LDS slots with direct-to-LDS loads;
//                    each wave dequantizes the weight fragments of its own
//                    MFMAs from LDS into registers, as bf16 holding the exact
//                    integer codes minus the bias (bf16 activations are
//                    exact); v_mfma_f32_16x16x32_bf16 covers one 32-wide quant
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
        P.prefix_gu[P.E + 3] = 0;   // the GEMMs' tile counters
        P.prefix_dn[P.E + 3] = 0;
    }
}

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

// Non-linear 4-bit: the 4-bit block's codes (same bytes and nibbles as
// deq4_group), each looked up in the bf16 byte tables of the format's table
// (exact: bf16 holds 8-bit integers), natural order.
__device__ __forceinline__ u32x4 deqnl_group(uint32_t qa, uint32_t qb, uint32_t ns, const NlTab &tb) {
    uint32_t la, ha, lb, hb;
    nl_lookup((qa >> ns) & 0x0F0F0F0Fu, tb, la, ha);
    nl_lookup((qb >> ns) & 0x0F0F0F0Fu, tb, lb, hb);
    u32x4 r;  // (low byte, high byte) of two values per dword
    r.x = __builtin_amdgcn_perm(ha, la, 0x05010400u);  // weights 0, 1
    r.y = __builtin_amdgcn_perm(ha, la, 0x07030602u);  // weights 2, 3
    r.z = __builtin_amdgcn_perm(hb, lb, 0x05010400u);
    r.w = __builtin_amdgcn_perm(hb, lb, 0x07030602u);
    return r;
}

// Raw dwords of weight blocks as loaded from HBM, and the block fields.
//   MODE 0 (gate/up): NW = one pair of consecutive blocks of one weight row
//     (3-bit: 28 bytes = 7 dwords; 4-bit layouts: 36 bytes = 9 dwords).
//   MODE 1 (down, column-block-major): one block of an even or odd row, the
//     row pair's dwords from the block's first one (3-bit: 4, 4-bit: 5).
template <int BITS>
struct BFields {
    uint32_t d;      // fp16 scale bits (low half)
    uint32_t q[nib_layout(BITS) ? 4 : 3];  // 4-bit layouts: code dwords; 3-bit: low parts (2), third bits
};

// Fields of one block from a run of dwords: `odd` = the block starts 2 bytes
// into dword o (scale in its high half, then aligned code dwords); otherwise
// it starts at dword 0 and every field is two bytes into a dword.
template <int BITS>
__device__ __forceinline__ BFields<BITS> block_fields(const uint32_t *w, bool odd, int o) {
    BFields<BITS> f;
    constexpr int NQ = nib_layout(BITS) ? 4 : 3;
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
__device__ __forceinline__ u32x4 deq_group(const BFields<BITS> &f, uint32_t g, const NlTab &tb) {
    if constexpr (BITS == 3) {
        return deq3_group(f.q[0], f.q[1], f.q[2], g);
    } else if constexpr (BITS == MOE_FMT_NL4) {
        const bool odd = g & 1u;
        return deqnl_group(odd ? f.q[2] : f.q[0], odd ? f.q[3] : f.q[1], 4u * (g >> 1), tb);
    } else {
        const bool odd = g & 1u;
        return deq4_group(odd ? f.q[2] : f.q[0], odd ? f.q[3] : f.q[1], 4u * (g >> 1));
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM tiles with an LDS ring.
//
// A tile is 16, 32 or 64 rows (by the group's size; MT = its non-empty 16-row
// m-tiles, 1 to 4) x 128 features
// (gate/up: the gate and the up row of each, 256 weight rows) or 256 outputs
// (down).  Per K step the workgroup streams the step's weight bytes (256 rows
// x KS blocks) and its activation pieces into one slot of an NS-slot ring in
// LDS with direct-to-LDS loads (global_load_lds: no register holds data in
// flight, so NS - 1 steps of loads stay outstanding whatever their size).
// All loads are 16-byte pieces.  Down: a step is one contiguous, 16-byte
// aligned run (256 rows of one column block).  Gate/up: a step's 256 row
// runs (KS * bb = 28 or 36 bytes each) start at one common 4-byte phase
// within a 16-byte piece (rows are 16-byte multiples apart), so each row
// takes the 3 aligned pieces covering its run (48 bytes; the compute reads
// from the phase on).  Every thread of a wave issues the same loads per step
// (LW weight pieces, fewer for the waves past the step's pieces, slots past
// the real data taking a copy of a valid piece that nothing reads; and one
// activation piece), so `s_waitcnt vmcnt(loads per step * steps issued after
// s)` tells a wave that its share of step s has landed, and a plain
// s_barrier then tells every wave that all shares have (__syncthreads' fence
// would also wait for the later steps' loads).  One barrier per step.
//
// Reads: wave w, lane (n, g) takes k-group g of weight row n of its 16 (gate
// and up) or 2 x 16 (down, rows of both parities) rows: the dwords of the
// block pair, from LDS (the four k-group lanes of a row read the same
// addresses: a broadcast); it dequantizes its k-group into the bf16 B
// operand (exact codes minus the bias), runs v_mfma_f32_16x16x32_bf16 per
// m-tile and adds the block's fp16 scale times the product to its fp32
// accumulators, blocks in K order.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int MODE, int BITS, int XF32>
struct PfCfg {
    static constexpr int KS = MODE == 0 ? 2 : 1;   // quant blocks per K step
    // ring slots: steps in flight + the one computed (fp32 activations are
    // split on the way into LDS, which waits for every load: two slots); the
    // ring of a bf16 gate/up or a down launch leaves room for two workgroups
    static constexpr int NS = XF32 ? 2 : (MODE == 0 ? 3 : 4);
    static constexpr int bb = blk_bytes(BITS);
    // 16-byte weight pieces per step: gate/up 256 rows x PPR pieces covering
    // each row's KS*bb bytes at any 4-byte phase; down KS column blocks x 256
    // rows (one contiguous run each)
    static constexpr int PPR = 3;
    static constexpr int STEP_W = MODE == 0 ? 256 * PPR : 256 * KS * bb / 16;
    static constexpr int LW = (STEP_W + PF_THREADS - 1) / PF_THREADS;  // weight loads per thread per step (at most)
    static constexpr int W_BYTES = MODE == 0 ? STEP_W * 16 : LW * PF_THREADS * 16;
    static constexpr int XP = MODE == 0 ? (XF32 ? 2 : 1) : 2;  // A parts: bf16 x; fp32 x or h as hi + lo
    static constexpr int A_PIECES = 64 * 4 * KS * XP;          // 16-byte pieces (8 K of one row)
    static constexpr int A_BYTES = A_PIECES * 16;
    static constexpr int STAGE = W_BYTES + A_BYTES;
    static constexpr int RING = NS * STAGE;
    // dwords of one lane's block pair (7 or 9): gate/up, two blocks of a row;
    // down, one block of the rows 2i and 2i + 1
    static constexpr int NW = 2 * bb / 4;
    static_assert(MODE == 0 ? (STEP_W % 64 == 0 && PPR * 16 >= 12 + KS * bb) : STEP_W * 16 == 256 * KS * bb,
                  "gate/up: whole waves of pieces covering a run at any phase; down: whole pieces");
    static_assert(NW == (nib_layout(BITS) ? 9 : 7) && (MODE == 1 || KS == 2), "a pair is two blocks");
    static_assert(RING + ((5 * (MOE_MAX_EXPERTS_DEV + 1) + 1) * 4 + 15) / 16 * 16 <= 159 * 1024,
                  "the ring and the largest slot plan fit one workgroup's LDS");
    static_assert(A_PIECES == PF_THREADS * (MODE == 0 && XF32 ? 2 : 1), "one piece per thread (two for fp32 x)");
};

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0) only

struct TileInfo {
    int slot, cnt, nt, r0, nrows, Fx, hrow0, mtl;
    bool shared_slot;
    const uint8_t *blob;
    int a_pair;  // gate/up: the pair id of this thread's activation row, -1 when none
    int pr64;    // thread tid < 64: pair id of tile row tid, -1 when none
    float w64;   // thread tid < 64, down tiles: the router weight of tile row tid (1 for the shared expert)
};

// Piece tid of a step's activations, layout [part][m][blk][g][n] x 16 bytes:
// 8 consecutive K (k-group g of block blk) of row 16 m + n.  The pieces a
// wave's lanes read for one MFMA operand (16 rows n of one (part, m, blk, g))
// are consecutive: no bank conflicts.
template <int KS>
__device__ __forceinline__ void a_piece(int tid, int &part, int &m, int &blk, int &g, int &n) {
    n = tid & 15;
    g = (tid >> 4) & 3;
    const int r = tid >> 6;
    blk = KS == 2 ? (r & 1) : 0;
    m = KS == 2 ? (r >> 1) : (r & 3);
    part = KS == 2 ? 0 : (r >> 2);
}
template <int KS>
__device__ __forceinline__ int a_off(int part, int m, int blk, int g, int n) {
    return ((((part * 4 + m) * KS + blk) * 4 + g) * 16 + n) * 16;
}

template <int N>
__device__ __forceinline__ void lds_dwords(const lds_u8 *p, uint32_t (&w)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = *(const lds_u32_t *)(p + 4 * i);
}

template <int MODE, int BITS, int XF32, int MT>
__device__ __forceinline__ void gemm_tile(const GemmParams &P, lds_u8 *ring, const int *s_pair, const float *s_w,
                                          const TileInfo &ti) {
    using C = PfCfg<MODE, BITS, XF32>;
    constexpr int KS = C::KS, NS = C::NS, LW = C::LW, NW = C::NW, XP = C::XP;
    constexpr int NPASS = MODE == 0 ? 2 : 1;  // gate + up / down
    constexpr int NTW = MODE == 0 ? 1 : 2;    // 16-column n-tiles per wave
    constexpr int NB = NPASS * NTW;           // B fragments per lane per block
    constexpr int bb = C::bb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_lane = lane & 15;
    const int g_lane = lane >> 4;
    const size_t rowG = (size_t)P.rowG;  // bytes of a gate/up row
    const int hs = P.h_stride;           // h row: hi plane [0, hs), lo plane [hs, 2 hs) (u16)
    const int K = MODE == 0 ? P.H : ti.Fx;
    const int nks = K / (32 * KS);

    // ---- this thread's weight load slots: byte offsets from the blob at step 0 ----
    uint32_t woff[LW];
    int nw = 0;  // weight loads of this wave per step (wave-uniform)
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int q = i * PF_THREADS + tid;
        nw += (MODE == 1 || i * PF_THREADS + 64 * wave < C::STEP_W) ? 1 : 0;
        size_t o = 0;  // (a slot past the step's data: the blob's first bytes, never read)
        if (q < C::STEP_W) {
            if (MODE == 0) {
                const int row = q / C::PPR, j = q - row * C::PPR;  // [256 rows: 128 gate, 128 up][PPR pieces]
                const int f = ti.nt * PF_NF_GU + (row & 127);
                o = ((row < 128 ? 0 : ti.Fx) + f) * rowG + 16 * j;
            } else {
                o = 2 * ti.Fx * rowG + (size_t)ti.nt * PF_NF_DN * bb + 16 * (size_t)q;  // [256 rows][bb bytes]
            }
        }
        woff[i] = (uint32_t)o;
    }
    const size_t wstep = MODE == 0 ? (size_t)KS * bb : (size_t)KS * P.H * bb;  // blob bytes per K step

    // ---- this thread's activation piece (rows past the tile: row 0's, never stored) ----
    int ap_part, ap_m, ap_blk, ap_g, ap_n;
    a_piece<KS>(tid, ap_part, ap_m, ap_blk, ap_g, ap_n);
    const int a_row = 16 * ap_m + ap_n;
    const bool a_in = ap_m < MT && a_row < ti.nrows;
    const uint8_t *a_src;
    size_t a_step;
    if (MODE == 0) {
        int tok = 0;
        if (ti.shared_slot) tok = ti.r0 + (a_in ? a_row : 0);
        else tok = a_in ? ti.a_pair / P.k : 0;
        const size_t el = (size_t)tok * P.H + 32 * ap_blk + 8 * ap_g;
        a_src = XF32 ? (const uint8_t *)((const float *)P.x + el) : (const uint8_t *)((const uint16_t *)P.x + el);
        a_step = (size_t)32 * KS * (XF32 ? 4 : 2);
    } else {
        const size_t row = (size_t)ti.hrow0 + ti.r0 + (a_in ? a_row : 0);
        a_src = (const uint8_t *)((const uint16_t *)P.hbuf + row * (2 * hs) + (size_t)ap_part * hs + 8 * ap_g);
        a_step = (size_t)32 * KS * 2;
    }

    const int lw_step = nw + (XF32 ? 0 : 1);  // direct-to-LDS loads of this wave per step
    // gate/up: step s's runs start (s * wstep) & 15 bytes into their first piece
    auto issue = [&](int s) {
        lds_u8 *st = ring + (s % NS) * C::STAGE;
        const uint8_t *wb = ti.blob + (MODE == 0 ? (((size_t)s * wstep) & ~(size_t)15) : (size_t)s * wstep);
#pragma unroll
        for (int i = 0; i < LW; ++i)
            if (MODE == 1 || i * PF_THREADS + 64 * wave < C::STEP_W)
                __builtin_amdgcn_global_load_lds(wb + woff[i], st + 16 * (i * PF_THREADS + 64 * wave), 16, 0, 0);
        if constexpr (!XF32)
            __builtin_amdgcn_global_load_lds(a_src + (size_t)s * a_step, st + C::W_BYTES + 16 * 64 * wave, 16, 0, 0);
    };

    float4v acc[NB][MT];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[a][m] = float4v{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const lds_u8 *st, int s) {
        const lds_u8 *wsl = st, *asl = st + C::W_BYTES;
        constexpr int NRAW = MODE == 0 ? NPASS : KS;  // block pairs this lane reads per step
        uint32_t rw[NRAW][NW];
        if (MODE == 0) {
            const int ph = (int)(((size_t)s * wstep) & 15);  // the step's phase in each row's pieces
#pragma unroll
            for (int p = 0; p < NPASS; ++p)
                lds_dwords<NW>(wsl + (p * 128 + wave * 16 + n_lane) * (16 * C::PPR) + ph, rw[p]);
        } else {
            // rows o, o + 1 (o = 32 w + 2 n) of block b: 2 * bb bytes from o * bb (a multiple of 4)
#pragma unroll
            for (int b = 0; b < KS; ++b) lds_dwords<NW>(wsl + b * 256 * bb + (wave * 32 + 2 * n_lane) * bb, rw[b]);
        }
#pragma unroll
        for (int blk = 0; blk < KS; ++blk) {
            bf16x8 av[MT][XP];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int x = 0; x < XP; ++x)
                    av[m][x] = __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)(asl + a_off<KS>(x, m, blk, g_lane, n_lane)));
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                // fragment f: gate/up pass f, or down n-tile f (row parity f)
                BFields<BITS> fl;
                if (MODE == 0) fl = block_fields<BITS>(rw[f], blk == 1, nib_layout(BITS) ? 4 : 3);
                else fl = block_fields<BITS>(rw[blk], f == 1, nib_layout(BITS) ? 4 : 3);
                const bf16x8 bq = __builtin_bit_cast(bf16x8, deq_group<BITS>(fl, (uint32_t)g_lane, P.nl));
                const float d = half_bits_to_float(fl.d);
                // the m-tiles' MFMAs issue back to back, then their scaling
                float4v dd[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float4v z = {0.f, 0.f, 0.f, 0.f};
                    dd[m] = mfma16bf(av[m][0], bq, z);
                    if (XP == 2) dd[m] = mfma16bf(av[m][XP - 1], bq, dd[m]);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[f][m].x = fmaf(d, dd[m].x, acc[f][m].x);
                    acc[f][m].y = fmaf(d, dd[m].y, acc[f][m].y);
                    acc[f][m].z = fmaf(d, dd[m].z, acc[f][m].z);
                    acc[f][m].w = fmaf(d, dd[m].w, acc[f][m].w);
                }
            }
        }
    };

    // ---- the K loop: NS - 1 steps of loads ahead of the one computed ----
    for (int u = 0; u < NS - 1 && u < nks; ++u) issue(u);
    for (int s = 0; s < nks; ++s) {
        lds_u8 *st = ring + (s % NS) * C::STAGE;
        if constexpr (XF32) {
            // fp32 activations: this thread's 8 values, split into bf16 hi + lo
            // pieces here (the slot's previous reader finished NS - 1 steps ago)
            const u32x4 *src = (const u32x4 *)(a_src + (size_t)s * a_step);
            const u32x4 r0 = src[0], r1 = src[1];
            wait_vm<0>();
            const uint32_t v[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
            uint32_t hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v0 = __builtin_bit_cast(float, v[2 * i]), v1 = __builtin_bit_cast(float, v[2 * i + 1]);
                const uint16_t h0 = f2bf_bits(v0), h1 = f2bf_bits(v1);
                const uint16_t l0 = f2bf_bits(v0 - bf16_bits_to_float(h0));
                const uint16_t l1 = f2bf_bits(v1 - bf16_bits_to_float(h1));
                hv[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lv[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            lds_u8 *asl = st + C::W_BYTES;
            *(lds_u32x4 *)(asl + a_off<KS>(0, ap_m, ap_blk, ap_g, ap_n)) = u32x4{hv[0], hv[1], hv[2], hv[3]};
            *(lds_u32x4 *)(asl + a_off<KS>(1, ap_m, ap_blk, ap_g, ap_n)) = u32x4{lv[0], lv[1], lv[2], lv[3]};
            wait_lgkm0();
        } else {
            wait_vm_n(lw_step * min(NS - 2, nks - 1 - s));
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (s + NS - 1 < nks) issue(s + NS - 1);
        compute(st, s);
    }

    // ---- epilogue ----
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = m * 16 + 4 * g_lane + r;
            if (rr >= ti.nrows) continue;
            if (MODE == 0) {
                const int col = ti.nt * PF_NF_GU + wave * 16 + n_lane;  // feature
                const float g = acc[0][m][r], u = acc[NPASS - 1][m][r];
                const float h = g * u * __frcp_rn(1.0f + __expf(-g));
                const uint16_t hh = f2bf_bits(h);
                const uint16_t hl = f2bf_bits(h - bf16_bits_to_float(hh));
                uint16_t *dst = (uint16_t *)P.hout + (size_t)(ti.hrow0 + ti.r0 + rr) * (2 * hs) + col;
                dst[0] = hh;
                dst[hs] = hl;
            } else {
                const int pr = s_pair[rr];
                const float wgt = s_w[rr];
                float *orow = ti.shared_slot ? P.out_shared + (size_t)(ti.r0 + rr) * P.H
                                             : P.out_pairs + (size_t)pr * P.H;
#pragma unroll
                for (int t = 0; t < NTW; ++t)
                    orow[ti.nt * PF_NF_DN + 32 * wave + 2 * n_lane + t] = wgt * acc[t][m][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM: persistent workgroups walk the tile list (slots by decreasing
// row count; within a slot, m-tiles of one n-tile are consecutive): each takes
// tiles blockIdx.x and blockIdx.x + G, then the next untaken ones from a
// counter in list order (tiles differ in cost: a fixed stride left the last
// workgroups ~20 % behind the mean), each id taken one tile ahead so that the
// atomic's round trip hides behind a tile's work.  Dynamic
// LDS: the slot plan (read once), then the ring.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int pf_plan_bytes(int E) { return (((5 * (E + 1) + 1) * 4) + 15) / 16 * 16; }

template <int MODE, int BITS, int XF32>
// (four waves per SIMD: two workgroups share a CU, so one's loads and
// barriers overlap the other's compute; the register limit this sets spills
// a few per-tile values, none in the K loop)
__global__ __launch_bounds__(PF_THREADS, 4) void k_prefill_gemm(GemmParams P) {
    __shared__ int s_pair[64];   // pair id of each tile row
    __shared__ float s_w[64];    // router weight of each tile row (down tiles)
    // the slot plan, read once: prefix[ns + 1], then per slot exp, cnt, row0, hrow0
    extern __shared__ __align__(16) int s_plan[];
    const int tid = threadIdx.x;
    const int ns = P.prefix[P.E + 2];
    const int total = P.prefix[ns];
    int *s_prefix = s_plan, *s_exp = s_plan + ns + 1, *s_cnt = s_exp + ns, *s_row0 = s_cnt + ns,
        *s_hrow0 = s_row0 + ns;
    lds_u8 *ring = (lds_u8 *)s_plan + pf_plan_bytes(P.E);
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
        const int a_r = 16 * (tid >> 7) + (tid & 15);  // this thread's activation row (gate/up pieces)
        ti.a_pair = (MODE == 0 && !ti.shared_slot && (tid >> 7) < ti.mtl && a_r < ti.nrows) ? P.pairs[row0 + a_r] : -1;
        ti.pr64 = (tid < 64 && tid < ti.nrows && !ti.shared_slot) ? P.pairs[row0 + tid] : -1;
        ti.w64 = (MODE == 1 && ti.pr64 >= 0 && P.pair_w) ? P.pair_w[ti.pr64] : 1.0f;
    };

    const int G = gridDim.x;
    uint32_t *const ctr = (uint32_t *)(P.prefix + P.E + 3);  // zeroed by the plan
    __shared__ int s_grab;  // the tile after the next one (thread 0's take, published at a tile's end)
    int tile = blockIdx.x;
    int nid = tile + G;  // the next tile
    TileInfo cur;
    if (tile < total) tile_info(tile, cur);
    for (bool first = true; tile < total; first = false) {
        // the previous tile is done with the ring, s_pair and s_w, and s_grab
        // holds its take (LDS only: its output stores need not have
        // completed, and this tile's loads go out meanwhile)
        lds_barrier();
        if (!first) nid = s_grab;
        uint32_t grab = 0;  // the tile after nid: its counter round trip overlaps this tile
        if (tid == 0 && nid < total) grab = add_dev(ctr, 1u);
        TileInfo nxt;
        const bool more = nid < total;
        if (more) tile_info(nid, nxt);
        if (tid < 64) {
            s_pair[tid] = cur.pr64;
            s_w[tid] = cur.w64;
        }
        lds_barrier();
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile, __builtin_amdgcn_s_memrealtime());
        // the MFMAs cover the tile's non-empty 16-row m-tiles only (the last
        // 64-row tile of a group may hold 1 to 64 rows)
        const int mact = (cur.nrows + 15) >> 4;
        if (mact == 4) gemm_tile<MODE, BITS, XF32, 4>(P, ring, s_pair, s_w, cur);
        else if (mact == 3) gemm_tile<MODE, BITS, XF32, 3>(P, ring, s_pair, s_w, cur);
        else if (mact == 2) gemm_tile<MODE, BITS, XF32, 2>(P, ring, s_pair, s_w, cur);
        else gemm_tile<MODE, BITS, XF32, 1>(P, ring, s_pair, s_w, cur);
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 1, __builtin_amdgcn_s_memrealtime());
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 2, (uint64_t)cur.mtl);
        PTRACE(((size_t)MODE << 20) + 4 * (size_t)tile + 3, (uint64_t)blockIdx.x);
        if (tid == 0) s_grab = nid < total ? 2 * G + (int)grab : total;
        if (more) cur = nxt;
        tile = nid;
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

// Persistent grid: as many workgroups as are resident at once (cus x
// workgroups per CU for this launch's LDS).
template <int MODE, int BITS, int XF32>
static hipError_t gemm_t(const GemmParams &P, int cus, hipStream_t st) {
    using C = PfCfg<MODE, BITS, XF32>;
    const size_t lds = (size_t)pf_plan_bytes(P.E) + C::RING;
    static int attr_set = 0;
    static int occ_lds[2] = {-1, 0};  // (LDS bytes, workgroups per CU) of the last query
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_prefill_gemm<MODE, BITS, XF32>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           pf_plan_bytes(MOE_MAX_EXPERTS_DEV) + C::RING);
        if (e != hipSuccess) return e;
        attr_set = 1;
    }
    if (occ_lds[0] != (int)lds) {
        int occ = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)k_prefill_gemm<MODE, BITS, XF32>,
                                                                    PF_THREADS, lds);
        if (e != hipSuccess) return e;
        occ_lds[0] = (int)lds;
        occ_lds[1] = occ < 1 ? 1 : occ;
    }
    hipLaunchKernelGGL((k_prefill_gemm<MODE, BITS, XF32>), dim3(cus * occ_lds[1]), dim3(PF_THREADS), lds, st, P);
    return hipGetLastError();
}

hipError_t prefill_gemm_launch(int mode, int bits, const GemmParams &P, int cus, hipStream_t st) {
    if (mode == 0) {
        if (bits == 4) return P.x_f32 ? gemm_t<0, 4, 1>(P, cus, st) : gemm_t<0, 4, 0>(P, cus, st);
        if (bits == MOE_FMT_NL4)
            return P.x_f32 ? gemm_t<0, MOE_FMT_NL4, 1>(P, cus, st) : gemm_t<0, MOE_FMT_NL4, 0>(P, cus, st);
        if (bits == 3) return P.x_f32 ? gemm_t<0, 3, 1>(P, cus, st) : gemm_t<0, 3, 0>(P, cus, st);
        return hipErrorInvalidValue;
    }
    if (bits == 4) return gemm_t<1, 4, 0>(P, cus, st);
    if (bits == MOE_FMT_NL4) return gemm_t<1, MOE_FMT_NL4, 0>(P, cus, st);
    if (bits == 3) return gemm_t<1, 3, 0>(P, cus, st);
    return hipErrorInvalidValue;
}

hipError_t prefill_combine_launch(const CombineParams &P, hipStream_t st) {
    const size_t n = (size_t)P.T * P.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_prefill_combine, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, P);
    return hipGetLastError();
}

}  // namespace moe
