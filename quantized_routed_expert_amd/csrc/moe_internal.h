// moe_internal.h -- structures shared by the host library and its kernels.
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace moe {

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
constexpr int DEC_X_BLOCKS_PER_THREAD = 4;   // activation blocks staged per thread (bf16; 2 for fp32)
constexpr uint32_t DEC_SPIN_LIMIT = 1u << 20;  // bounded waits: a wait that runs out sets err bit 0
#define MOE_MAX_EXPERTS_DEV 4096
#define MOE_DECODE_ROWS_DEV 16

// bits of DecodeParams::mode
constexpr int DEC_MODE_ROUTE = 1;    // route + group from logits (else grouping is given)
constexpr int DEC_MODE_COMBINE = 2;  // sum per-pair rows + shared into y
constexpr int DEC_MODE_SHARED = 4;   // a shared expert is present

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
    float *gu_part;            // [(T*k + T)][2][nch][Fmax] fp32 partial gate/up sums per K chunk
    uint32_t *gu_count;        // [max_slots]
    uint32_t *dn_count;        // [max_slots]
    uint32_t *slice_count;     // [H / DEC_DN_ROWS]
    uint32_t *err;             // error word (bit 0: a wait hit its spin limit)
    int T, E, k, H, F, Fs;     // Fs = shared ffn (0 = none)
    int bits, x_f32, mode, max_slots;
    int part_stride;           // floats per gu_part row = 2 * nch * Fmax
    int nch;                   // K chunks of the gate/up rows
    // dynamic LDS layout (byte offsets)
    int lds_idx, lds_w, lds_sorted, lds_hist, lds_slot_start, lds_slot_exp, lds_slot_cnt,
        lds_tinv, lds_hinv, lds_xmax, lds_misc, lds_xa, lds_chunk, chunk_stride, lds_total;
};

// ---------------------------------------------------------------------------
// Prefill / general path.
// ---------------------------------------------------------------------------
constexpr int GRP_CHUNK_TOKENS = 64;  // tokens per grouping chunk
#define MOE_TOPK_MAX_LDS 32               // k <= 32
#define MOE_SCAN_PER_MAX 4                // experts per thread in the 1024-thread scan (E <= 4096)

struct RouteParams {
    const float *logits;
    int T, E, k;
    int32_t *idx;
    float *w;
};

struct GroupParams {
    const int32_t *idx;  // [T][k]
    int T, E, k, nchunks;
    uint32_t *chunk_counts;  // [nchunks][E]
    int32_t *offsets;        // [E+1]
    int32_t *pairs;          // [T*k]
    int32_t *active;         // [E+1]
};

struct PlanParams {
    const int32_t *offsets;  // [E+1]
    const int32_t *active;   // [E+1]
    int T, E, k, has_shared, F, Fs, H;
    int32_t *slot_exp;       // [E+1]  expert id, -1 = shared
    int32_t *slot_row0;      // [E+1]  first entry in pairs[] (routed) / 0 (shared)
    int32_t *slot_cnt;       // [E+1]
    int32_t *slot_hrow0;     // [E+1]  first row in the h buffer
    int32_t *prefix_gu;      // [E+3]: tile prefix per slot; [E+2] = number of slots
    int32_t *prefix_dn;      // [E+3]
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
};

struct CombineParams {
    const float *out_pairs, *out_shared;
    float *y;
    int T, k, H;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
