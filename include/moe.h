/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts layer over
 * block-quantized expert weights.
 *
 * The layer (what the calls below compute, in order):
 *   1. router: per token, the k experts with the largest router logits and a
 *      softmax over those k logits (forum thread "把 Strata 搬上 SGLang 引擎
 *      的嘗試", TL;DR and §三: top-10 of 512 experts; extended-strata-moe
 *      "Reference", section "Routing trace format": k expert ids and k
 *      weights per token and layer);
 *   2. grouping: the (token, expert) pairs bucketed per expert, so each
 *      expert computes only the rows routed to it (thread §二, the
 *      expert-scoped layout);
 *   3. per expert: gather of its rows, dequantization inside the kernel,
 *      gate/up projection, SwiGLU, down projection, weighted scatter-add back
 *      to the tokens, all in one grouped call per layer (thread TL;DR and §三,
 *      the grouped expert kernel and its one-call-per-layer timing);
 *   4. the shared expert, applied to every row of the window (Strata "Several
 *      requests at once (batch slots)", opening section: the shared expert is
 *      read once per window for all rows).
 *
 * Weight format.  Block of 32 weights with an fp16 scale d (thread §四: the
 * 4-bit block of 32 values in 18 bytes):
 *   bits = 4: 18 bytes = d (2 bytes, little-endian binary16) + 16 bytes;
 *             byte 2+i holds code i in its low nibble, code i+16 in its high
 *             nibble; weight = d * (code - 8).
 *   bits = 3: 14 bytes = d + 8 bytes of low parts (code i's two low bits at
 *             bit 2*(i/8) of byte 2+(i%8)) + a 32-bit little-endian word at
 *             bytes 10..13 whose bit i is code i's third bit;
 *             weight = d * (code - 4).
 *   bits = MOE_BITS_NL4 (20), non-linear 4-bit: the 4-bit block's 18 bytes
 *             and nibble order; weight = d * codebook[code], codebook the
 *             16 signed 8-bit values the weights come with (moe_qweights).
 *             The thread's §四 names this block (32 values in 18 bytes) and
 *             §三 pairs it as the down format with 3-bit gate/up formats;
 *             the pages print no table, so the table is the caller's.
 * A matrix [rows][cols] is stored row by row, cols/32 blocks per row, with
 * no padding.  One expert's blob is gate [F][H] | up [F][H] | down [H][F]
 * (gate, up and down concatenated per expert, thread §三); experts follow
 * each other with no padding.  This is MOE_LAYOUT_ROWS.  The nibble order
 * and the whole 3-bit layout are readings of points the pages leave open.
 * Gate and up share one bit width (`bits`); down may have its own
 * (`down_bits`), as the thread's §三 decode table pairs each gate/up format
 * with a down format (a 2- or 3-bit gate/up with a 4-bit down).
 * The grouped GEMM (MOE_PATH_PREFILL) takes every pair of these formats;
 * the decode path takes pairs of the 3- and 4-bit formats, the non-linear
 * format throughout, and a 3-bit gate/up with a non-linear down.  For other
 * pairs MOE_PATH_AUTO serves a decode window with the grouped GEMM and
 * MOE_PATH_DECODE returns MOE_ERR_UNSUPPORTED.
 *
 * The compute calls read MOE_LAYOUT_PREPARED, written once per weight set by
 * moe_prepare_qweights: the same blocks and sizes, gate and up unchanged,
 * the down projection's blocks reordered column-block-major (block (h, c) of
 * down, row h, FFN columns 32c..32c+31, at index c*H + h), so a 32-column
 * slice of down for all H rows is one contiguous run.  (The thread feeds its
 * blob to the kernel without conversion; this library converts once at load
 * time instead, so a decode split over FFN slices streams contiguous bytes.)
 *
 * Conventions for every call:
 *  - Pointers marked (device) point to GPU memory on the current HIP device;
 *    (host) to host memory.  The caller owns every buffer and the stream.
 *    The library allocates nothing, frees nothing and never synchronizes;
 *    all work is enqueued on `stream` (a hipStream_t passed as int64_t,
 *    0 = the null stream), so calls can be captured into a hipGraph.
 *  - Row-major, contiguous tensors; device pointers 16-byte aligned.
 *  - Errors: 0 (MOE_OK) or a negative MOE_ERR_* code.  Arguments are
 *    validated on the host before anything is launched; on an error nothing
 *    is launched and no output is touched.  MOE_ERR_LAUNCH reports a failed
 *    kernel launch (hipGetLastError after the launch).  Device-side input
 *    checks are not made: logits must be finite.
 *  - The workspace (device) must be at least moe_workspace_bytes(...) bytes
 *    and zero-filled before its first use.  Every call leaves its counters
 *    at zero again, so a workspace can be reused by later calls (and graph
 *    replays) without clearing.  Two calls that run at the same time must
 *    not share a workspace.
 *  - Co-residency.  The decode path (MOE_PATH_DECODE, and AUTO for T <= 16)
 *    is one launch whose workgroups hand partial results to each other; it
 *    launches as many workgroups as the device holds at once and assumes
 *    that all of them are resident together.  Every wait in it is bounded:
 *    if other work on the device keeps some workgroup from starting, the
 *    waits run out, the call ends with wrong outputs and the workspace's
 *    error word records it (moe_workspace_error).  Run decode calls without
 *    other kernels competing for the device when the outputs matter.
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, negative or inconsistent size */
#define MOE_ERR_UNSUPPORTED (-2)  /* bits not 3/4/20, H or F not a multiple of 256, weights not prepared, ... */
#define MOE_ERR_WORKSPACE (-3)    /* workspace smaller than moe_workspace_bytes */
#define MOE_ERR_LAUNCH (-4)       /* a kernel launch failed */
#define MOE_ERR_DEVICE (-5)       /* no usable gfx950 device / device query failed */

/* activation dtypes */
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* which kernels run the expert FFN */
#define MOE_PATH_AUTO 0     /* DECODE when T <= MOE_DECODE_MAX_ROWS, else PREFILL */
#define MOE_PATH_DECODE 1   /* one fused launch per layer, T <= MOE_DECODE_MAX_ROWS */
#define MOE_PATH_PREFILL 2  /* grouped GEMM over per-expert row tiles, any T */

/* Rows per decode window: one token per batch slot plus its MTP proposal,
 * up to 16 rows (Strata "Several requests at once", section "Windows of 16
 * rows": HIP builds take windows of 16 rows). */
#define MOE_DECODE_MAX_ROWS 16

/* Limits of this build. */
#define MOE_MAX_EXPERTS 4096
#define MOE_MAX_TOPK 32

/* block orders of a weight set (see "Weight format" above) */
#define MOE_LAYOUT_ROWS 0      /* every matrix row by row, as stored on the pages */
#define MOE_LAYOUT_PREPARED 1  /* down column-block-major: what the compute calls read */

/* the non-linear 4-bit format (see "Weight format" above) */
#define MOE_BITS_NL4 20

/* Quantized expert weights (host struct; `data` is a device pointer). */
typedef struct moe_qweights {
    const void *data;   /* (device) n_experts blobs back to back, see above */
    int32_t bits;       /* 3, 4 or MOE_BITS_NL4: the gate and up projections */
    int32_t n_experts;  /* routed: E; shared: 1 */
    int32_t hidden;     /* H, multiple of 256 */
    int32_t ffn;        /* F, multiple of 256 */
    int32_t layout;     /* MOE_LAYOUT_*; the compute calls take MOE_LAYOUT_PREPARED only */
    int32_t down_bits;  /* 3, 4 or MOE_BITS_NL4: the down projection; 0 = the same as bits */
    int8_t codebook[16]; /* MOE_BITS_NL4: the values codes 0..15 stand for (ignored otherwise);
                            a shared expert must carry the routed experts' table */
} moe_qweights;

/* Library version (major*100 + minor). */
int moe_version(void);

/* Text for a status code; never NULL. */
const char *moe_status_string(int status);

/* Bytes of one expert blob: hidden * ffn/32 * (2 * B(bits) + B(down_bits)),
 * B = 18 (4-bit, non-linear 4-bit) or 14 (3-bit) bytes per block, down_bits 0 = bits; -1 if
 * the arguments are not a valid format and shape (pure host function). */
int64_t moe_expert_bytes(int32_t bits, int32_t down_bits, int32_t hidden, int32_t ffn);

/* Workspace bytes needed by moe_layer_forward / moe_expert_ffn for these
 * shapes on `path` (AUTO resolves as the calls do).  shared_ffn = 0 when
 * there is no shared expert.  Returns a negative MOE_ERR_* for invalid
 * shapes.  Pure host function. */
int64_t moe_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t hidden, int32_t ffn,
                            int32_t shared_ffn, int32_t path);

/*
 * Weight preparation (once per weight set, before any compute call).  src
 * (host struct) describes weights in MOE_LAYOUT_ROWS; dst (device) receives
 * the same n_experts blobs in MOE_LAYOUT_PREPARED (src->n_experts *
 * moe_expert_bytes(...) bytes; describe it with layout = MOE_LAYOUT_PREPARED
 * afterwards).  src and dst must not overlap, and src must stay valid until
 * the copy, enqueued on `stream`, has run.  Errors: MOE_ERR_INVALID_ARG for
 * a null pointer, overlapping buffers or src->layout != MOE_LAYOUT_ROWS,
 * MOE_ERR_UNSUPPORTED for bits or shapes the compute calls do not take.
 */
int moe_prepare_qweights(const moe_qweights *src, void *dst, int64_t stream);

/*
 * Device-side errors of the calls that used a workspace.  Synchronizes
 * `stream`, copies the workspace's error word to *err_out (host) and, if
 * clear != 0, sets it back to zero.  Bits: 1 = a bounded wait of a decode
 * launch ran out (see "Co-residency" above; that call's outputs are wrong);
 * 2 = moe_expert_ffn on the decode path was given a malformed grouping
 * (its outputs are wrong; no access went out of bounds).  0 after correct
 * calls.  The bits stay set until cleared; a later call is not affected by
 * an earlier call's timeout.  Unlike the compute calls, this one waits for
 * the stream and must not be called during graph capture.
 */
int moe_workspace_error(void *ws, int64_t ws_bytes, uint32_t *err_out, int32_t clear, int64_t stream);

/*
 * Router projection (the step before step 1): logits (device) fp32 [T][E]
 * = x (device) [T][hidden] (fp32 or bf16, x_dtype) times the transpose of
 * w_router (device) bf16 [E][hidden] (row e: expert e's router vector):
 *     logits[t][e] = sum_h x[t][h] * w_router[e][h]
 * bf16 products exact, fp32 sums (fp32 x enters as bf16 hi + lo, 16
 * significant bits).  A row's logits do not depend on the other rows, and
 * the same inputs give the same bits on every run.  The extended-strata-moe
 * "Reference", section "Tools" (route_dump / route_predict read a layer's
 * router from its hidden state); in the forum thread's post "prefill 36.8
 * -> 334", the decode wall is met with one captured graph per window over
 * all 48 layers: this launch and moe_layer_forward's per layer.
 * hidden a multiple of 256, at most 4096; E <= MOE_MAX_EXPERTS.
 */
int moe_router_logits(const void *x, int32_t x_dtype, int32_t T, int32_t hidden,
                      const void *w_router, int32_t E, float *logits, int64_t stream);

/*
 * Router (step 1).  logits (device) fp32 [T][E]; writes topk_idx (device)
 * int32 [T][k] and topk_w (device) fp32 [T][k].  Per token the k experts are
 * listed by decreasing logit, an equal logit going to the lower expert id
 * (selection compares the fp32 logits themselves); topk_w[t][j] =
 * exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected, so a row's
 * weights sum to one.  1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS.
 */
int moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_idx,
              float *topk_w, int64_t stream);

/*
 * Grouping (step 2).  topk_idx (device) int32 [T][k], every id in [0, E).
 * Pair id p = t*k + j.  Writes (device): offsets int32 [E+1] (exclusive
 * prefix sum of the per-expert pair counts, offsets[E] = T*k); pairs int32
 * [T*k] (the pair ids of expert 0, then expert 1, ..., each expert's in
 * increasing p, i.e. ordered by (expert, token, slot)); active int32 [E+1]
 * (active[0] = number of experts with at least one pair, then their ids in
 * ascending order; the tail is not written).  The placement is stable and
 * deterministic.  ws (device) is scratch of at least
 * moe_workspace_bytes(T, E, k, ...) bytes (any path).
 */
int moe_group(const int32_t *topk_idx, int32_t T, int32_t E, int32_t k, int32_t *offsets,
              int32_t *pairs, int32_t *active, void *ws, int64_t ws_bytes, int64_t stream);

/*
 * Routed expert FFN (step 3) on a given grouping.  x (device) [T][H] fp32 or
 * bf16 (x_dtype).  offsets/pairs/active (device) as written by moe_group for
 * w->n_experts experts and top-k = k.  pair_w (device) fp32 [T*k] or NULL
 * (weight 1).  For every listed pair p (token t = p/k) of every active
 * expert e:
 *     out_pairs[p][:] = pair_w[p] * down_e( silu(gate_e x_t) * (up_e x_t) )
 * out_pairs (device) fp32 [T*k][H]; rows of pairs that are not listed are
 * not written.  path selects the kernels (DECODE needs T <= 16).
 */
int moe_expert_ffn(const void *x, int32_t x_dtype, int32_t T, const moe_qweights *w,
                   const int32_t *offsets, const int32_t *pairs, const int32_t *active,
                   const float *pair_w, int32_t k, float *out_pairs, int32_t path, void *ws,
                   int64_t ws_bytes, int64_t stream);

/*
 * The whole layer (steps 1-4).  x (device) [T][H] fp32 or bf16; logits
 * (device) fp32 [T][E] with E = routed->n_experts; shared (host struct, may
 * be NULL) with n_experts = 1, the same hidden and the same bits and
 * down_bits as the routed experts (its ffn may differ; other widths:
 * MOE_ERR_UNSUPPORTED, since every launch reads it as one more slot of the
 * routed format).
 * Writes y (device) fp32
 * [T][H]:
 *     y_t = (((w_t0 o_t0 + w_t1 o_t1) + ...) + w_t,k-1 o_t,k-1) + s_t
 * with o_tj the output of token t's j-th expert, w_tj its router weight and
 * s_t the shared expert's output, summed in that fixed order (the result
 * does not depend on launch geometry or timing).  topk_idx_out / topk_w_out
 * (device, may be NULL) receive the routing ([T][k] int32 / fp32).
 *
 * heat (device, may be NULL): int32 [E] routing heat of this layer.  The call
 * adds to heat[e] the number of its (token, slot) pairs routed to expert e
 * (the counts of step 2; they sum to T*k), so a caller keeping one [E] row
 * per layer accumulates the per-(layer, expert) heat over calls (Strata
 * "Several requests at once (batch slots)", section "The VRAM expert tier
 * keeps adapting in batch windows"; extended-strata-moe "Reference",
 * section "The adaptive cache": a heat per layer and expert).  Integer
 * atomic adds, so the counts are exact whatever the order; calls running
 * at the same time may share the buffer.
 */
int moe_layer_forward(const void *x, int32_t x_dtype, const float *logits, int32_t T,
                      int32_t k, const moe_qweights *routed, const moe_qweights *shared,
                      float *y, int32_t *topk_idx_out, float *topk_w_out, int32_t *heat,
                      int32_t path, void *ws, int64_t ws_bytes, int64_t stream);

/*
 * moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments and results are those of
 * moe_layer_forward; the scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES, one per device, held until the process ends
 * and found once per device (hipGetSymbolAddress on the first call made
 * with that device current).  The call allocates and frees nothing.
 * Limit: a call whose workspace (moe_workspace_bytes for its shapes and
 * path) exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE and
 * launches nothing; every decode window of the five reference shapes fits
 * (at most about 24 MiB), a 2048-token prefill chunk does not.  Every call
 * on a device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads) race and give wrong results; calls
 * in one stream's order are safe.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int moe_layer_forward_noalloc(const void *x, int32_t x_dtype, const float *logits, int32_t T,
                              int32_t k, const moe_qweights *routed, const moe_qweights *shared,
                              float *y, int32_t *topk_idx_out, float *topk_w_out, int32_t *heat,
                              int32_t path, int64_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
