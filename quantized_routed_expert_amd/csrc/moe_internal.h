// moe_internal.h -- structures shared by the host library and its kernels.
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace moe {

// Format code of the non-linear 4-bit block (the 4-bit layout, codes index a
// 16-entry table of signed 8-bit values).
#define MOE_FMT_NL4 20

// A non-linear 4-bit table as two byte tables of 16-bit floats of its
// entries: t[0..3] = low bytes of entries 0..15, t[4..7] = high bytes (fp16
// for the decode kernels, bf16 for the grouped GEMM).
struct NlTab {
    uint32_t t[8];
};

// ---------------------------------------------------------------------------
// Fused decode launch (routing + grouping + gate/up/SwiGLU + down + weighted
// write + combine in one kernel, T <= 16 rows).
// ---------------------------------------------------------------------------
constexpr int DEC_WAVES = 8;                 // waves per workgroup
constexpr int DEC_THREADS = DEC_WAVES * 64;
constexpr int DEC_DN_ROWS = DEC_WAVES * 16;  // down-projection rows per workgroup tile
constexpr int DEC_CB_MAX = 32;               // quant blocks per row in one streamed chunk
constexpr int DEC_MAX_LD = 9;                // 16-byte loads per lane per chunk (16 rows x 32 x 18 B)
constexpr int DEC_MAX_E_FUSED = 1024;        // router fused into the kernel up to this many experts
constexpr int DEC_MAX_F = 1024;              // expert FFN width handled by the fused decode launch
constexpr int DEC_XG_BF16 = 8;              // activation k-groups (8 values) loaded per thread: bf16
constexpr int DEC_XG_F32 = 4;               // ... fp32
constexpr uint32_t DEC_SPIN_LIMIT = 1u << 20;  // bounded waits: a wait that runs out sets err bit 0
constexpr int DEC_COMB_LOADS = 8;           // combine: loads in flight per thread
constexpr int DEC_COMB_PARTS = 8;           // combine items per 128-row slice
constexpr int DEC_CSTRIDE = 64;              // 32-bit words between counters (one 256-byte line each)
constexpr int EPOCH_SLOTS = 1024;            // per-workgroup copies of the call count (grids of <= 1024)
constexpr int DEC_RANK_MAX_KEYS = 2048;      // routing by ranks: T*E up to this ...
constexpr int DEC_RANK_MAX_CMP = 64;         // ... and at most this many comparisons per thread
#define MOE_MAX_EXPERTS_DEV 4096
#define MOE_DECODE_ROWS_DEV 16  // <= 32: the fused grouping keeps a 32-bit token mask per expert
constexpr int DEC_MAX_SLOTS = MOE_DECODE_ROWS_DEV * 32 + 1;  // T*k pairs (k <= 32) + the shared expert
constexpr int DEC_MAX_SLICES = 65536 / DEC_DN_ROWS;

// bits of DecodeParams::mode
constexpr int DEC_MODE_ROUTE = 1;    // route + group from logits (else grouping is given)
constexpr int DEC_MODE_COMBINE = 2;  // sum per-pair rows + shared into y
constexpr int DEC_MODE_SHARED = 4;   // a shared expert is present

// Quant blocks per streamed gate/up chunk for a row of nkb blocks: the K
// chunks of a row number 1, 2, 4 or 8 (so the units of a 16-feature group
// fill a workgroup's 8 waves exactly, in one or two rounds), each chunk a
// multiple of 8 blocks (so chunk segments start 16-byte aligned in both
// formats) and at most DEC_CB_MAX.  0: no such split (the fused decode launch
// does not take the shape).
__host__ __device__ inline int decode_h_chunk_blocks(int nkb) {
    for (int nch = 1; nch <= 8; nch <<= 1) {
        if (nkb % nch) continue;
        const int cb = nkb / nch;
        if (cb <= DEC_CB_MAX && cb % 8 == 0) return cb;
    }
    return 0;
}

// Quant blocks per streamed down chunk (F is a multiple of 256: nkb % 8 == 0).
__host__ __device__ inline int decode_f_chunk_blocks(int nkb) {
    return (nkb % 32 == 0) ? 32 : (nkb % 24 == 0) ? 24 : (nkb % 16 == 0) ? 16 : 8;
}

// LDS bytes between the 16 rows of a staged chunk: a whole number of 16-byte
// granules, made odd so that the 16 rows start in 16 different bank groups.
__host__ __device__ inline int decode_chunk_rstride(int seg_bytes) {
    const int gr = (seg_bytes + 15) >> 4;
    return 16 * (gr | 1);
}

// The tag of the call that follows `completed` calls on a workspace: a
// bijection of the count (so consecutive calls never share a tag), never 0
// (the value a zeroed workspace holds).
__host__ __device__ inline uint32_t decode_tag(uint32_t completed) {
    const uint32_t t = ((completed + 1u) * 0x9E3779B1u) ^ 0xA5A5A5A5u;
    return t ? t : 0x5A5A5A5Au;
}

struct DecodeParams {
    const void *x;             // [T][H] fp32 or bf16
    const float *logits;       // [T][E] (ROUTE mode)
    const int32_t *g_offsets;  // given grouping (not ROUTE mode)
    const int32_t *g_pairs;
    const int32_t *g_active;
    const float *g_pair_w;     // may be null: weight 1
    const uint8_t *w_routed;   // E expert blobs
    const uint8_t *w_shared;   // 1 blob or null
    float *y;                  // [T][H] (COMBINE mode)
    float *out_pairs;          // [T*k][H]
    float *out_shared;         // [T][H]
    int32_t *topk_idx_out;     // may be null
    float *topk_w_out;         // may be null
    int32_t *heat;             // [E] routing heat, += pairs per expert (ROUTE mode; may be null)
    // Data handed between workgroups is written as 64-bit words (fp32 value in
    // the low half, the call's tag in the high half), so a reader can tell a
    // word of this call from an older one and the writer never has to wait for
    // its stores to complete.
    uint64_t *hll;             // [(T*k + T)][Fmax] SwiGLU outputs, in the down projection's k order
    uint64_t *oll;             // [(T*k + T)][H] weighted pair rows, then shared rows (COMBINE mode)
    uint32_t *gu_count;        // [DEC_MAX_SLOTS * DEC_CSTRIDE]: finished gate/up tasks per slot
    uint32_t *dn_count;        // [DEC_MAX_SLOTS * DEC_CSTRIDE]: finished down tiles per slot
    uint32_t *slice_count;     // [DEC_MAX_SLICES * DEC_CSTRIDE]: finished slots per 128-row slice
    uint32_t *err;             // error word (bit 0: a wait hit its spin limit; bit 1: bad given grouping);
                               // err[1]: tag of the last call whose wait ran out
    uint32_t *epoch;           // [EPOCH_SLOTS] calls completed on this workspace (the tag source)
    int T, E, k, H, F, Fs;     // Fs = shared ffn (0 = none)
    int bits, x_f32, mode, max_slots;  // bits: gate and up projections
    int dbits;                 // bit width of the down projection
    NlTab nl;                  // fp16 tables of the non-linear format (when a width is MOE_FMT_NL4)
    size_t eb;                 // bytes of one routed expert blob
    int h_stride;              // words per hll row (Fmax)
    int x_rs, h_rs;            // LDS bytes per token row: activations (one part), staged h (hi + lo)
    // geometry, computed on the host (divisions by values that are not powers
    // of two use m_* = ceil(2^32 / d): n / d = umulhi(n, m_d) for n < 2^20)
    int nkbH, cbH, segH, rowH, rsH, perH;  // gate/up rows: blocks, blocks per chunk, chunk bytes per row,
                                           // row bytes, LDS row stride, 16-byte pieces per chunk row
    uint32_t invH;                         // 65536 / perH + 1
    int lg_nchH, lg_upt, lg_nfgT, rounds;  // K chunks, units per 16-feature group, groups per task (log2)
    int tasks_sh, tasks_rt;                // gate/up tasks of the shared expert / of a routed expert
    uint32_t m_tasks_rt;
    int tps;                               // down tiles per slot (H / 128)
    uint32_t m_tps;
    // down geometry per kind of slot: [0] routed (F), [1] shared (Fs).  Down
    // is column-block-major, so a wave's chunk (16 rows x cbF blocks) is cbF
    // runs of 16*bb bytes: segF = bytes between chunks, rowF = between runs,
    // rsF = LDS bytes between runs, perF = 16-byte pieces per run
    int fx[2], cbF[2], nchF[2], segF[2], rowF[2], rsF[2], perF[2];
    uint32_t invF[2], m_ngrp[2];           // m_ngrp: 1 / (fx / 8)
    uint32_t m_k;                          // 1 / k
    int xgrp;                              // activation k-groups per token (H / 8)
    uint32_t m_xgrp;
    // routing by ranks (all threads; small T*E): lg_tpi = log2 threads per logit
    int route_rank, lg_tpi;
    uint32_t m_E;
    // dynamic LDS layout (byte offsets)
    int lds_idx, lds_w, lds_sorted, lds_hist, lds_slot_start, lds_slot_exp, lds_slot_cnt,
        lds_tsc, lds_hsc, lds_xmax, lds_misc, lds_xa, lds_chunk, chunk_stride, lds_total;
};

// ---------------------------------------------------------------------------
// Column-split decode launch (windows of one to four rows): each workgroup item
// is (expert, 32-column slice of its FFN): gate/up rows of the slice, SwiGLU
// and the slice's partial down projection, reduced over the slices at the end.
// ---------------------------------------------------------------------------
constexpr int SPL_MAX_T = 4;
constexpr int SPL_MAX_SLOTS = SPL_MAX_T * 32 + 1;  // T*k pairs (k <= 32) + the shared expert

struct SplitSmall {  // fixed part of the launch's LDS
    int idx[SPL_MAX_T * 32];
    float w[SPL_MAX_T * 32];
    int slot_exp[SPL_MAX_SLOTS];
    int slot_pair[SPL_MAX_SLOTS][SPL_MAX_T];  // pair id of each row in the slot, -1: none
    int plist[SPL_MAX_SLOTS * SPL_MAX_T];     // pairs present (output rows of the per-pair mode)
    uint32_t wmax[8][SPL_MAX_T];  // per wave and row: largest |x| (as bits)
    int tsc[SPL_MAX_T], hsc[SPL_MAX_T];  // per row: the powers of two sc of its integer x and h
    int Sh[SPL_MAX_T];
    int n_slots, n_pl, pad[2];
};

struct SplitParams {
    const void *x;             // [T][H] fp32 or bf16
    const float *logits;       // [T][E] (ROUTE mode)
    const int32_t *g_offsets;  // given grouping (not ROUTE mode)
    const int32_t *g_pairs;
    const int32_t *g_active;
    const float *g_pair_w;     // may be null: weight 1
    const uint8_t *w_routed;   // E prepared expert blobs
    const uint8_t *w_shared;   // 1 prepared blob or null
    float *y;                  // [T][H] (COMBINE mode)
    float *out_pairs;          // [T*k][H]
    float *out_shared;         // [T][H]
    int32_t *topk_idx_out;     // may be null
    float *topk_w_out;         // may be null
    int32_t *heat;             // [E] routing heat, += pairs per expert (ROUTE mode; may be null)
    uint64_t *part;            // [T*k + T][ncmax][H] tagged partial down rows per (pair, slice)
    uint32_t *err, *epoch;     // error word (as DecodeParams::err); [EPOCH_SLOTS] calls completed (the tag source)
    int T, E, k, H, F, Fs, bits, mode, x_f32;
    int dbits;                 // bit width of the down projection (bits: gate and up)
    uint32_t nl8[4];           // the non-linear format's table, 16 signed bytes (when a width is MOE_FMT_NL4)
    size_t eb;                 // bytes of one routed expert blob
    int nc, ncs, ncmax;        // 32-column slices of F and Fs; the partial buffer's stride
    uint32_t m_nc;             // ceil(2^32 / nc) (0 when nc = 1)
    int rowH;                  // bytes of one gate/up row (H/32 blocks of the gate/up format)
    int lg_qpr;                // log2 of the 4-pair pieces per gate/up row (H / 256)
    int units;                 // reduction outputs per workgroup
    // LDS byte offsets
    int lds_small, lds_wt, lds_a, lds_S, lds_xd, lds_gu, lds_ah, lds_hd, lds_total;
};

// ---------------------------------------------------------------------------
// Prefill / general path.
// ---------------------------------------------------------------------------
constexpr int GRP_CHUNK_TOKENS = 16;  // tokens per grouping chunk
#define MOE_TOPK_MAX_LDS 32               // k <= 32
#define MOE_SCAN_PER_MAX 4                // experts per thread in the 1024-thread scan (E <= 4096)

struct RouteParams {
    const float *logits;
    int T, E, k;
    int32_t *idx;
    float *w;
};

// Router projection: logits [T][E] = x [T][H] . W^T, W bf16 [E][H].
struct RouterParams {
    const void *x;          // [T][H] fp32 or bf16
    const uint16_t *w;      // [E][H] bf16
    float *logits;          // [T][E]
    int T, H, E, x_f32;
};

struct GroupParams {
    const int32_t *idx;  // [T][k]
    int T, E, k, nchunks;
    uint32_t *chunk_counts;  // [nchunks][E]
    int32_t *offsets;        // [E+1]
    int32_t *pairs;          // [T*k]
    int32_t *active;         // [E+1]
    int32_t *heat;           // [E] routing heat, += pairs per expert (may be null)
};

struct PlanParams {
    const int32_t *offsets;  // [E+1]
    const int32_t *active;   // [E+1]
    int T, E, k, has_shared, F, Fs, H;
    int32_t *slot_exp;       // [E+1]  expert id, -1 = shared
    int32_t *slot_row0;      // [E+1]  first entry in pairs[] (routed) / 0 (shared)
    int32_t *slot_cnt;       // [E+1]
    int32_t *slot_hrow0;     // [E+1]  first row in the h buffer
    int32_t *prefix_gu;      // [E+4]: tile prefix per slot; [E+2] = number of slots; [E+3] = tile counter
    int32_t *prefix_dn;      // [E+4]
};

struct GemmParams {
    const void *x;          // [T][H] fp32/bf16 (gate/up)
    const float *hbuf;      // h rows, fp32 (down input)
    float *hout;            // h rows (gate/up output)
    const uint8_t *w_routed, *w_shared;
    const int32_t *pairs;   // sorted pair ids
    const float *pair_w;    // [T*k] or null (weight 1)
    float *out_pairs;       // [T*k][H]
    float *out_shared;      // [T][H]
    const int32_t *slot_exp, *slot_row0, *slot_cnt, *slot_hrow0, *prefix;  // prefix[E+2] = #slots
    int T, E, k, H, F, Fs, h_stride, x_f32;
    int rowG;               // bytes of one gate/up row (H/32 blocks of the gate/up format)
    size_t eb;              // bytes of one routed expert blob
    NlTab nl;               // bf16 tables of the non-linear format (when a width is MOE_FMT_NL4)
};

struct CombineParams {
    const float *out_pairs, *out_shared;
    float *y;
    int T, k, H;
};

// Weight preparation (row-by-row block order -> down column-block-major).
struct PrepareParams {
    size_t expert_bytes;  // one blob
    size_t gu_bytes;      // gate + up bytes of one blob (2 * F * H/32 * bb)
    int n_experts, H, nc, bb;  // nc = F / 32 (down blocks per row), bb = bytes per block
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
