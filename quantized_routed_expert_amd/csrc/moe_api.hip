// moe_api.hip -- the C ABI (include/moe.h): host-side validation, workspace
// layout and dispatch.  Arguments follow the statement of the layer on the
// pages (hidden states, router logits, top-k, quantized expert tensors, the
// shared expert); conventions on errors and sizing follow the
// extended-strata-moe "Reference", section "C API" (a query that does not
// apply reports it and leaves its outputs untouched).  The stream is taken as
// an int64 so no HIP type appears in the interface (the forum thread
// "把 Strata 搬上 SGLang 引擎 的嘗試", §三, passes its stream the same way).
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
hipError_t decode_launch(const DecodeParams &P, int grid, hipStream_t st);
int decode_occupancy(int bg, int bd, int x_f32, int lds);
hipError_t decode_set_lds(int bg, int bd, int x_f32, int lds);
bool decode_format_ok(int bg, int bd);
hipError_t split_launch(const SplitParams &P, int grid, hipStream_t st);
hipError_t split_set_lds(int bg, int bd, int T, int xf, int lds);
hipError_t route_launch(const RouteParams &P, hipStream_t st);
hipError_t router_logits_launch(const RouterParams &P, hipStream_t st);
hipError_t group_launch(const GroupParams &P, hipStream_t st);
}  // namespace moe

namespace moe {
hipError_t prefill_plan_launch(const PlanParams &P, hipStream_t st);
hipError_t prefill_gemm_launch(int mode, int bits, const GemmParams &P, int cus, hipStream_t st);
hipError_t prefill_combine_launch(const CombineParams &P, hipStream_t st);
hipError_t prepare_launch(const uint8_t *src, uint8_t *dst, const PrepareParams &P, hipStream_t st);
}  // namespace moe

using namespace moe;

namespace {

// ----------------------------------------------------------------------------
// Device facts (cached per device)
// ----------------------------------------------------------------------------
struct DevInfo {
    int ok = 0;
    int cus = 0;
    int lds_max = 0;
};
std::mutex g_mu;
DevInfo g_dev[64];

int dev_info(DevInfo &out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    DevInfo &d = g_dev[dev];
    if (!d.ok) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MOE_ERR_DEVICE;
        if (strncmp(p.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
        d.cus = p.multiProcessorCount;
        d.lds_max = (int)p.maxSharedMemoryPerMultiProcessor;
        d.ok = 1;
    }
    out = d;
    return MOE_OK;
}

// ----------------------------------------------------------------------------
// Workspace layout
// ----------------------------------------------------------------------------
struct Layout {
    size_t counters = 0, n_counters = 0;       // decode: gu[MS] dn[MS] slice[H/128] err epoch[EPOCH_SLOTS]
    size_t harr = 0, oll = 0, part = 0, out_pairs = 0, out_shared = 0;
    size_t idx = 0, w = 0, offsets = 0, pairs = 0, active = 0, chunk_counts = 0;
    size_t slot_exp = 0, slot_row0 = 0, slot_cnt = 0, slot_hrow0 = 0, prefix_gu = 0, prefix_dn = 0;
    size_t hbuf = 0;
    size_t total = 0;
    int max_slots = 0, nchunks = 0;
};

// The counters sit at offset 0 with a size that depends on no shape, in every
// layout, so a workspace that is zero before its first use stays valid for
// calls of any shape and path (each call returns the counters to zero).  Each
// counter has a 256-byte line of its own.
// after the slot and slice counters: the error word (a line of its own),
// then the per-workgroup epochs
constexpr size_t COUNTER_WORDS = (size_t)(2 * DEC_MAX_SLOTS + DEC_MAX_SLICES + 1) * DEC_CSTRIDE + EPOCH_SLOTS;
// byte offset of the error word (and, after it, the tag of the last call whose wait ran out)
constexpr size_t ERR_OFFSET = (size_t)(2 * DEC_MAX_SLOTS + DEC_MAX_SLICES) * DEC_CSTRIDE * 4;
Layout make_layout(int T, int E, int k, int H, int F, int Fs, int path) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t TK = (size_t)T * k;
    const int Fmax = F > Fs ? F : Fs;
    L.nchunks = (T + GRP_CHUNK_TOKENS - 1) / GRP_CHUNK_TOKENS;
    L.max_slots = DEC_MAX_SLOTS;
    L.n_counters = COUNTER_WORDS;
    L.counters = take(COUNTER_WORDS * 4);
    // routing and grouping (all paths; moe_group uses chunk_counts)
    L.idx = take(TK * 4);
    L.w = take(TK * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.pairs = take(TK * 4);
    L.active = take((size_t)(E + 1) * 4);
    L.chunk_counts = take((size_t)L.nchunks * E * 4);
    L.out_pairs = take(TK * H * 4);
    L.out_shared = take((size_t)T * H * 4);
    if (path == MOE_PATH_DECODE) {
        L.harr = take((TK + T) * (size_t)Fmax * 8);  // tagged SwiGLU outputs per pair row (+ shared rows)
        L.oll = take((TK + T) * (size_t)H * 8);      // tagged weighted pair rows (+ shared rows)
        // tagged partial rows per (pair, 32-column slice) of the column-split
        // launch, sized for its largest window so that a workspace sized for
        // T rows also serves every smaller window
        const size_t Ts = T < SPL_MAX_T ? (size_t)T : (size_t)SPL_MAX_T;
        L.part = take((Ts * k + Ts) * (size_t)(Fmax / 32) * H * 8);
    } else {
        L.slot_exp = take((size_t)(E + 1) * 4);
        L.slot_row0 = take((size_t)(E + 1) * 4);
        L.slot_cnt = take((size_t)(E + 1) * 4);
        L.slot_hrow0 = take((size_t)(E + 1) * 4);
        L.prefix_gu = take((size_t)(E + 4) * 4);  // [E+2] slots, [E+3] the GEMM's tile counter
        L.prefix_dn = take((size_t)(E + 4) * 4);
        L.hbuf = take((TK + T) * (size_t)Fmax * 4);
    }
    L.total = off;
    return L;
}

template <class Tp>
Tp *at(void *ws, size_t off) {
    return (Tp *)((uint8_t *)ws + off);
}

// ----------------------------------------------------------------------------
// Validation helpers
// ----------------------------------------------------------------------------
int check_shape(int32_t T, int32_t E, int32_t k, int32_t H, int32_t F) {
    if (T < 0 || E <= 0 || k <= 0 || H <= 0 || F <= 0) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if (H % 256 || F % 256 || H > 65536 || F > 65536) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int down_bits_of(const moe_qweights *w) { return w->down_bits ? w->down_bits : w->bits; }
// the block formats: 3-bit, 4-bit and the non-linear 4-bit (the 4-bit layout)
bool valid_bits(int b) { return b == 3 || b == 4 || b == MOE_BITS_NL4; }
bool valid_down_bits(int b) { return b == 0 || valid_bits(b); }
bool uses_table(const moe_qweights *w) { return w->bits == MOE_BITS_NL4 || down_bits_of(w) == MOE_BITS_NL4; }
int block_bytes_of(int bits) { return (bits == 4 || bits == MOE_BITS_NL4) ? 18 : 14; }
// index of a format in the per-format launch caches
int fmt_index(int bits) { return bits == 3 ? 0 : bits == 4 ? 1 : 2; }

// The non-linear table as the kernels take it: byte tables of a 16-bit
// float of each entry (fp16 for the decode kernel, bf16 for the grouped
// GEMM), both exact for 8-bit integers.
NlTab nl_tables(const int8_t *cb, bool bf16) {
    NlTab t;
    memset(&t, 0, sizeof(t));
    for (int c = 0; c < 16; ++c) {
        uint16_t h;
        if (bf16) {
            const float f = (float)cb[c];
            uint32_t u;
            memcpy(&u, &f, 4);
            h = (uint16_t)(u >> 16);  // exact: an 8-bit integer needs no rounding
        } else {
            const _Float16 f = (_Float16)cb[c];
            memcpy(&h, &f, 2);
        }
        t.t[c >> 2] |= (uint32_t)(h & 0xFF) << (8 * (c & 3));
        t.t[4 + (c >> 2)] |= (uint32_t)(h >> 8) << (8 * (c & 3));
    }
    return t;
}
// bytes of one expert blob: gate and up [F][H] in `bits`, down [H][F] in `dbits`
size_t expert_bytes_of(int bits, int dbits, int H, int F) {
    return (size_t)H * (F / 32) * (2 * block_bytes_of(bits) + block_bytes_of(dbits));
}

int check_weights(const moe_qweights *w, int H, int n_experts) {
    if (!w || !w->data) return MOE_ERR_INVALID_ARG;
    if (!valid_bits(w->bits) || !valid_down_bits(w->down_bits)) return MOE_ERR_UNSUPPORTED;
    if (w->layout != MOE_LAYOUT_PREPARED) return MOE_ERR_UNSUPPORTED;
    if (w->hidden != H) return MOE_ERR_INVALID_ARG;
    if (n_experts >= 0 && w->n_experts != n_experts) return MOE_ERR_INVALID_ARG;
    if (w->ffn <= 0) return MOE_ERR_INVALID_ARG;
    if (w->ffn % 256) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int resolve_path(int path, int T) {
    if (path == MOE_PATH_AUTO) return T <= MOE_DECODE_MAX_ROWS ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
    return path;
}

inline hipStream_t S(int64_t s) { return (hipStream_t)(intptr_t)s; }

// ceil(2^32 / d) for d >= 2 (n / d == umulhi(n, magic) for n < 2^20); 0 for d = 1
uint32_t magic_div(uint32_t d) { return d < 2 ? 0u : (uint32_t)((((uint64_t)1 << 32) + d - 1) / d); }
int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Geometry of the fused decode launch (see DecodeParams); needs T, E, k, H,
// F, Fs, bits.
void decode_geometry(DecodeParams &P) {
    const int bb = block_bytes_of(P.bits);    // gate/up blocks
    const int bbd = block_bytes_of(P.dbits);  // down blocks
    P.nkbH = P.H / 32;
    P.cbH = decode_h_chunk_blocks(P.nkbH);
    const int nchH = P.nkbH / P.cbH;
    P.segH = P.cbH * bb;
    P.rowH = P.nkbH * bb;
    P.rsH = decode_chunk_rstride(P.segH);
    P.perH = P.segH / 16;
    P.invH = 65536u / (uint32_t)P.perH + 1u;
    P.lg_nchH = ilog2(nchH);
    const int upt = 2 * nchH;
    P.lg_upt = ilog2(upt);
    const int nfgT = upt >= 8 ? 1 : 8 / upt;
    P.lg_nfgT = ilog2(nfgT);
    P.rounds = upt > 8 ? upt / 8 : 1;
    P.tasks_sh = P.Fs / (16 * nfgT);
    P.tasks_rt = P.F / (16 * nfgT);
    P.m_tasks_rt = magic_div(P.tasks_rt);
    P.tps = P.H / DEC_DN_ROWS;
    P.m_tps = magic_div(P.tps);
    for (int i = 0; i < 2; ++i) {
        const int fx = i == 0 ? P.F : (P.Fs ? P.Fs : P.F);
        const int nkb = fx / 32;
        P.fx[i] = fx;
        P.cbF[i] = decode_f_chunk_blocks(nkb);
        P.nchF[i] = nkb / P.cbF[i];
        // down is column-block-major: a chunk is cbF runs of 16 rows x bbd
        // bytes (one run per 32-column block), H*bbd bytes apart
        P.segF[i] = P.cbF[i] * P.H * bbd;  // bytes from one chunk to the next
        P.rowF[i] = P.H * bbd;             // bytes between the runs of a chunk
        P.rsF[i] = decode_chunk_rstride(16 * bbd);
        P.perF[i] = bbd;                   // 16-byte pieces per run
        P.invF[i] = 65536u / (uint32_t)P.perF[i] + 1u;
        P.m_ngrp[i] = magic_div(fx / 8);
    }
    P.m_k = magic_div(P.k);
    P.xgrp = P.H / 8;
    P.m_xgrp = magic_div(P.xgrp);
    // routing by ranks when every thread compares few keys: threads per logit
    // = 512 / (T*E), a power of two from 1 to 16
    const long long nkeys = (long long)P.T * P.E;
    int tpi = 1;
    while (tpi < 16 && nkeys * tpi * 2 <= DEC_THREADS) tpi *= 2;
    const long long cmp = (nkeys + DEC_THREADS / tpi - 1) / (DEC_THREADS / tpi) * ((P.E + tpi - 1) / tpi);
    P.route_rank = nkeys <= DEC_RANK_MAX_KEYS && cmp <= DEC_RANK_MAX_CMP && P.E % (4 * tpi) == 0;
    P.lg_tpi = ilog2(tpi);
    P.m_E = magic_div(P.E);
}

// Fill the decode kernel's LDS layout; returns the byte total.
int decode_lds_layout(DecodeParams &P, int xparts) {
    const int TK = P.T * P.k;
    const int Fmax = P.F > P.Fs ? P.F : P.Fs;
    const int bb = block_bytes_of(P.bits), bbd = block_bytes_of(P.dbits);
    int off = 0;
    auto take = [&](int bytes) {
        int a = off;
        off = (int)align_up((size_t)(off + bytes), 16);
        return a;
    };
    P.lds_idx = take(TK * 4);
    P.lds_w = take(TK * 4);
    P.lds_sorted = take((TK + P.E) * 4);  // sorted pairs, then (fused routing) each expert's first position
    P.lds_hist = take((P.E + 1) * 4);
    P.lds_slot_start = take(P.max_slots * 4);
    P.lds_slot_exp = take(P.max_slots * 4);
    P.lds_slot_cnt = take(P.max_slots * 4);
    P.lds_tsc = take(P.T * 4);
    P.lds_hsc = take(P.T * 4);
    P.lds_xmax = take(P.T * 4);
    P.lds_misc = take(64);
    // activations (one 16-byte pad per token row keeps the 16 rows of an
    // MFMA operand read in distinct banks); later the staged h
    P.x_rs = (P.H / 32) * 64 + 16;
    P.h_rs = Fmax * 4 + 16;
    const int xa_bytes = xparts * P.T * P.x_rs;
    const int ha_bytes = P.T * P.h_rs;
    P.lds_xa = take(xa_bytes > ha_bytes ? xa_bytes : ha_bytes);
    // wave-private chunk buffers (also the gate/up unit partials: 2 x 16 x 16 floats)
    int cmax = 16 * decode_chunk_rstride(P.cbH * bb);
    const int cf = decode_f_chunk_blocks(P.F / 32) * decode_chunk_rstride(16 * bbd);
    cmax = cf > cmax ? cf : cmax;
    if (P.Fs) {
        const int cs = decode_f_chunk_blocks(P.Fs / 32) * decode_chunk_rstride(16 * bbd);
        cmax = cs > cmax ? cs : cmax;
    }
    cmax = cmax > 2048 ? cmax : 2048;
    // (phase A also keeps the rank keys and the selected logits there)
    const int rank_bytes = (P.T * P.E + TK) * 4;
    if (DEC_WAVES * cmax < rank_bytes) cmax = (rank_bytes + DEC_WAVES - 1) / DEC_WAVES;
    P.chunk_stride = (int)align_up((size_t)cmax, 16);
    P.lds_chunk = take(DEC_WAVES * P.chunk_stride);
    P.lds_total = off;
    return off;
}

int launch_err(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Shapes the fused decode launch takes: every thread stages at most
// DEC_X_BLOCKS_PER_THREAD activation blocks (half for fp32), an expert's FFN
// width is at most DEC_MAX_F, the gate/up rows split into 1, 2, 4 or 8 K
// chunks, and the LDS layout fits one workgroup per CU.
constexpr int DEC_LDS_BUDGET = 160 * 1024;
bool decode_fits(int T, int E, int k, int H, int F, int Fs, int bits, int dbits, int x_dtype) {
    if (!decode_format_ok(bits, dbits)) return false;
    const int xf = x_dtype == MOE_DTYPE_F32;
    const int per = xf ? DEC_XG_F32 : DEC_XG_BF16;
    if ((long long)T * (H / 8) > (long long)per * DEC_THREADS) return false;
    if (F > DEC_MAX_F || Fs > DEC_MAX_F) return false;
    if (decode_h_chunk_blocks(H / 32) == 0) return false;
    DecodeParams P;
    memset(&P, 0, sizeof(P));
    P.T = T;
    P.E = E;
    P.k = k;
    P.H = H;
    P.F = F;
    P.Fs = Fs;
    P.bits = bits;
    P.dbits = dbits;
    P.max_slots = ((T * k < E) ? T * k : E) + 1;
    decode_geometry(P);
    return decode_lds_layout(P, xf ? 2 : 1) <= DEC_LDS_BUDGET;
}

// ---- column-split decode launch (windows of one to four rows, T*k <= 64) ----
int split_xps(int /*bits*/) { return 36; }  // digit dwords per pair slot in LDS (both formats)
// 16-byte loads per lane of a wave's 8 gate/up rows at H = 2048 (the most)
int split_gu_loads(int bits) { return block_bytes_of(bits) == 18 ? 9 : 7; }
// 16-byte loads per lane of a wave's H/8 down rows of one column block at H = 2048
int split_dn_loads(int bits) { return block_bytes_of(bits) == 18 ? 5 : 4; }

int split_lds_layout(SplitParams &P) {
    const int bb = block_bytes_of(P.bits), bbd = block_bytes_of(P.dbits), xps = split_xps(P.bits);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t a = off;
        off = align_up(off + bytes, 16);
        return (int)a;
    };
    P.lds_small = take(sizeof(SplitSmall));
    // an item's gate and up rows, then its down column block: each wave's
    // share in its own run of 1 KB loads (split_gu_loads, split_dn_loads)
    P.lds_wt = take((size_t)8 * (split_gu_loads(P.bits) + split_dn_loads(P.dbits)) * 1024);
    P.lds_a = take((size_t)P.T * P.H * 2);  // the integer activations
    P.lds_S = take((size_t)P.T * (P.H / 32) * 4);
    P.lds_xd = take((size_t)P.T * (P.H / 64) * xps * 4);
    P.lds_gu = take((size_t)P.T * 64 * 4);
    P.lds_ah = take((size_t)P.T * 32 * 2);
    P.lds_hd = take((size_t)P.T * xps * 4);
    P.lds_total = (int)off;
    return P.lds_total;
}

// Reduction outputs per workgroup for a grid of G (whole chunks of 8).
int split_units(int T, int k, int H, int combine, int G) {
    const long long n = combine ? (long long)T * H : (long long)T * k * H;
    return (int)(((n + G - 1) / G + 7) / 8 * 8);
}

bool split_fits(int T, int E, int k, int H, int F, int Fs, int bits, int dbits, int combine, int G) {
    (void)E;
    // the pairs the launch is built for (as decode_format_ok)
    if (!decode_format_ok(bits, dbits)) return false;
    if (T < 1 || T > SPL_MAX_T || k > 32 || T * k > 64) return false;
    if (H != 256 && H != 512 && H != 1024 && H != 2048) return false;
    if (F > 4096 || Fs > 4096) return false;
    SplitParams P;
    memset(&P, 0, sizeof(P));
    P.T = T;
    P.H = H;
    P.bits = bits;
    P.dbits = dbits;
    if (split_lds_layout(P) > DEC_LDS_BUDGET) return false;
    // the reduction stages (outputs x terms x (slices + 1)) floats in the item weight area
    const int units = split_units(T, k, H, combine, G);
    const int nterm = combine ? k + 1 : 1;
    const int ncmax = (F > Fs ? F : Fs) / 32;
    return (long long)units * nterm * (ncmax + 1) * 4 <=
           (long long)8 * (split_gu_loads(bits) + split_dn_loads(dbits)) * 1024;
}

}  // namespace

extern "C" {

int moe_version(void) { return 100; }

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, negative or inconsistent size)";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration (bits, shape or path)";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
        case MOE_ERR_LAUNCH: return "kernel launch failed";
        case MOE_ERR_DEVICE: return "no usable gfx950 device";
        default: return "unknown status";
    }
}

int64_t moe_expert_bytes(int32_t bits, int32_t down_bits, int32_t hidden, int32_t ffn) {
    if (!valid_bits(bits) || !valid_down_bits(down_bits)) return -1;
    if (hidden <= 0 || ffn <= 0 || hidden % 32 || ffn % 32) return -1;
    return (int64_t)expert_bytes_of(bits, down_bits ? down_bits : bits, hidden, ffn);
}

int64_t moe_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t hidden, int32_t ffn,
                            int32_t shared_ffn, int32_t path) {
    int rc = check_shape(T, E, k, hidden, ffn);
    if (rc) return rc;
    if (shared_ffn < 0 || shared_ffn % 256) return MOE_ERR_UNSUPPORTED;
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
    // a decode request may be served by the prefill kernels (mixed bit widths,
    // shapes beyond the fused launch), so size for both
    const int p = resolve_path(path, T);
    size_t n = make_layout(T, E, k, hidden, ffn, shared_ffn, p).total;
    if (p == MOE_PATH_DECODE) {
        const size_t n2 = make_layout(T, E, k, hidden, ffn, shared_ffn, MOE_PATH_PREFILL).total;
        n = n > n2 ? n : n2;
    }
    return (int64_t)n;
}

int moe_prepare_qweights(const moe_qweights *src, void *dst, int64_t stream) {
    if (!src || !src->data || !dst) return MOE_ERR_INVALID_ARG;
    if (src->layout != MOE_LAYOUT_ROWS) return MOE_ERR_INVALID_ARG;
    if (!valid_bits(src->bits) || !valid_down_bits(src->down_bits)) return MOE_ERR_UNSUPPORTED;
    if (src->n_experts <= 0 || src->hidden <= 0 || src->ffn <= 0) return MOE_ERR_INVALID_ARG;
    if (src->n_experts > MOE_MAX_EXPERTS || src->hidden % 256 || src->ffn % 256 || src->hidden > 65536 ||
        src->ffn > 65536)
        return MOE_ERR_UNSUPPORTED;
    const int64_t eb = (int64_t)expert_bytes_of(src->bits, down_bits_of(src), src->hidden, src->ffn);
    const uintptr_t s0 = (uintptr_t)src->data, d0 = (uintptr_t)dst;
    const uintptr_t n = (uintptr_t)eb * (uintptr_t)src->n_experts;
    if (s0 < d0 + n && d0 < s0 + n) return MOE_ERR_INVALID_ARG;  // overlap
    PrepareParams P;
    P.expert_bytes = (size_t)eb;
    P.gu_bytes = (size_t)2 * src->ffn * (src->hidden / 32) * block_bytes_of(src->bits);
    P.n_experts = src->n_experts;
    P.H = src->hidden;
    P.nc = src->ffn / 32;
    P.bb = block_bytes_of(down_bits_of(src));  // the down blocks are what moves
    return launch_err(prepare_launch((const uint8_t *)src->data, (uint8_t *)dst, P, S(stream)));
}

int moe_workspace_error(void *ws, int64_t ws_bytes, uint32_t *err_out, int32_t clear, int64_t stream) {
    if (!ws || !err_out) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < (int64_t)(ERR_OFFSET + 8)) return MOE_ERR_WORKSPACE;
    uint8_t *w = (uint8_t *)ws + ERR_OFFSET;
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, w, 4, hipMemcpyDeviceToHost, S(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
    if (hipStreamSynchronize(S(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
    if (clear) {
        if (hipMemsetAsync(w, 0, 8, S(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
        if (hipStreamSynchronize(S(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
    }
    *err_out = v;
    return MOE_OK;
}

int moe_router_logits(const void *x, int32_t x_dtype, int32_t T, int32_t hidden, const void *w_router,
                      int32_t E, float *logits, int64_t stream) {
    if (T < 0 || hidden <= 0 || E <= 0) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (E > MOE_MAX_EXPERTS || hidden % 256 || hidden > 4096) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T > 65535 * 16) return MOE_ERR_UNSUPPORTED;
    DevInfo dv;
    const int rc = dev_info(dv);
    if (rc) return rc;
    RouterParams P{x, (const uint16_t *)w_router, logits, T, hidden, E, x_dtype == MOE_DTYPE_F32 ? 1 : 0};
    return launch_err(router_logits_launch(P, S(stream)));
}

int moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_idx, float *topk_w,
              int64_t stream) {
    int rc = check_shape(T, E, k, 256, 256);
    if (rc) return rc;
    if (T == 0) return MOE_OK;  // nothing to read or write
    if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    RouteParams P{logits, T, E, k, topk_idx, topk_w};
    return launch_err(route_launch(P, S(stream)));
}

int moe_group(const int32_t *topk_idx, int32_t T, int32_t E, int32_t k, int32_t *offsets, int32_t *pairs,
              int32_t *active, void *ws, int64_t ws_bytes, int64_t stream) {
    if (!topk_idx || !offsets || !pairs || !active || !ws) return MOE_ERR_INVALID_ARG;
    int rc = check_shape(T, E, k, 256, 256);
    if (rc) return rc;
    Layout L = make_layout(T, E, k, 256, 256, 0, MOE_PATH_PREFILL);
    if (ws_bytes < (int64_t)(L.chunk_counts + (size_t)L.nchunks * E * 4)) return MOE_ERR_WORKSPACE;
    GroupParams G{topk_idx, T, E, k, L.nchunks, at<uint32_t>(ws, L.chunk_counts), offsets, pairs, active, nullptr};
    return launch_err(group_launch(G, S(stream)));
}

}  // extern "C"

namespace {

// Fused decode launch (routing in-kernel when logits != nullptr).
int run_decode(const void *x, int x_f32, const float *logits, const int32_t *g_off, const int32_t *g_pairs,
               const int32_t *g_act, const float *g_pw, int T, int E, int k, const moe_qweights *routed,
               const moe_qweights *shared, float *y, float *out_pairs, int32_t *tidx, float *tw, int32_t *heat,
               const Layout &L, void *ws, int mode, hipStream_t st) {
    DevInfo dv;
    int rc = dev_info(dv);
    if (rc) return rc;
    const int Fs_ = shared ? shared->ffn : 0;
    const int dbits = down_bits_of(routed);
    if (split_fits(T, E, k, routed->hidden, routed->ffn, Fs_, routed->bits, dbits, (mode & DEC_MODE_COMBINE) ? 1 : 0,
                   dv.cus)) {
        SplitParams S_;
        memset(&S_, 0, sizeof(S_));
        S_.x = x;
        S_.logits = logits;
        S_.g_offsets = g_off;
        S_.g_pairs = g_pairs;
        S_.g_active = g_act;
        S_.g_pair_w = g_pw;
        S_.w_routed = (const uint8_t *)routed->data;
        S_.w_shared = shared ? (const uint8_t *)shared->data : nullptr;
        S_.y = y;
        S_.out_pairs = out_pairs;
        S_.out_shared = at<float>(ws, L.out_shared);
        S_.topk_idx_out = tidx;
        S_.topk_w_out = tw;
        S_.heat = heat;
        S_.part = at<uint64_t>(ws, L.part);
        uint32_t *cnt = at<uint32_t>(ws, L.counters);
        S_.err = cnt + (size_t)(2 * DEC_MAX_SLOTS + DEC_MAX_SLICES) * DEC_CSTRIDE;
        S_.epoch = S_.err + DEC_CSTRIDE;
        S_.T = T;
        S_.E = E;
        S_.k = k;
        S_.H = routed->hidden;
        S_.F = routed->ffn;
        S_.Fs = Fs_;
        S_.bits = routed->bits;
        S_.dbits = dbits;
        memcpy(S_.nl8, routed->codebook, 16);
        S_.eb = expert_bytes_of(routed->bits, dbits, routed->hidden, routed->ffn);
        S_.mode = mode | (shared ? DEC_MODE_SHARED : 0);
        S_.x_f32 = x_f32;
        S_.nc = S_.F / 32;
        S_.ncs = Fs_ / 32;
        S_.ncmax = S_.nc > S_.ncs ? S_.nc : S_.ncs;
        S_.m_nc = magic_div(S_.nc);
        S_.rowH = (S_.H / 32) * block_bytes_of(S_.bits);
        S_.lg_qpr = ilog2(S_.H / 256);
        const int grid = dv.cus;  // one workgroup per CU, all resident
        if (grid > EPOCH_SLOTS) return MOE_ERR_UNSUPPORTED;
        S_.units = split_units(T, k, S_.H, (mode & DEC_MODE_COMBINE) ? 1 : 0, grid);
        const int lds = split_lds_layout(S_);
        if (lds > dv.lds_max) return MOE_ERR_UNSUPPORTED;
        static std::mutex smu;
        static int s_lds_set[3][3][SPL_MAX_T][2] = {};
        {
            std::lock_guard<std::mutex> lk(smu);
            int &cur = s_lds_set[fmt_index(S_.bits)][fmt_index(dbits)][T - 1][x_f32 ? 1 : 0];
            if (lds > cur) {
                if (split_set_lds(S_.bits, dbits, T, x_f32, lds) != hipSuccess) return MOE_ERR_LAUNCH;
                cur = lds;
            }
        }
        return launch_err(split_launch(S_, grid, st));
    }
    DecodeParams P;
    memset(&P, 0, sizeof(P));
    P.x = x;
    P.logits = logits;
    P.g_offsets = g_off;
    P.g_pairs = g_pairs;
    P.g_active = g_act;
    P.g_pair_w = g_pw;
    P.w_routed = (const uint8_t *)routed->data;
    P.w_shared = shared ? (const uint8_t *)shared->data : nullptr;
    P.y = y;
    P.out_pairs = out_pairs;
    P.out_shared = at<float>(ws, L.out_shared);
    P.topk_idx_out = tidx;
    P.topk_w_out = tw;
    P.heat = heat;
    P.hll = at<uint64_t>(ws, L.harr);
    P.oll = at<uint64_t>(ws, L.oll);
    uint32_t *cnt = at<uint32_t>(ws, L.counters);
    P.gu_count = cnt;
    P.dn_count = cnt + (size_t)DEC_MAX_SLOTS * DEC_CSTRIDE;
    P.slice_count = cnt + (size_t)2 * DEC_MAX_SLOTS * DEC_CSTRIDE;
    P.err = cnt + (size_t)(2 * DEC_MAX_SLOTS + DEC_MAX_SLICES) * DEC_CSTRIDE;
    P.epoch = P.err + DEC_CSTRIDE;
    P.T = T;
    P.E = E;
    P.k = k;
    P.H = routed->hidden;
    P.F = routed->ffn;
    P.Fs = shared ? shared->ffn : 0;
    P.bits = routed->bits;
    P.dbits = dbits;
    P.nl = nl_tables(routed->codebook, false);
    P.eb = expert_bytes_of(routed->bits, dbits, routed->hidden, routed->ffn);
    P.x_f32 = x_f32;
    P.mode = mode | (shared ? DEC_MODE_SHARED : 0);
    P.max_slots = ((T * k < E) ? T * k : E) + 1;  // LDS slot tables (counters use the fixed stride)
    P.h_stride = P.F > P.Fs ? P.F : P.Fs;
    decode_geometry(P);
    const int lds = decode_lds_layout(P, x_f32 ? 2 : 1);
    if (lds > dv.lds_max) return MOE_ERR_UNSUPPORTED;
    static std::mutex mu;
    static int lds_set[3][3][2] = {};
    int occ;
    {
        std::lock_guard<std::mutex> lk(mu);
        int &cur = lds_set[fmt_index(P.bits)][fmt_index(dbits)][x_f32 ? 1 : 0];
        if (lds > cur) {
            if (decode_set_lds(P.bits, dbits, x_f32, lds) != hipSuccess) return MOE_ERR_LAUNCH;
            cur = lds;
        }
        occ = decode_occupancy(P.bits, dbits, x_f32, lds);
    }
    if (occ <= 0) return MOE_ERR_UNSUPPORTED;
    // persistent grid: every workgroup resident (the down tiles wait on
    // counters written by other workgroups' gate/up items)
    const int grid = dv.cus * occ;
    if (grid > EPOCH_SLOTS) return MOE_ERR_UNSUPPORTED;
    return launch_err(decode_launch(P, grid, st));
}

int prefill_gemms(const void *x, int x_f32, int T, int E, int k, const moe_qweights *routed,
                  const moe_qweights *shared, const int32_t *pairs, const float *pair_w, float *out_pairs,
                  float *out_shared, const Layout &L, void *ws, hipStream_t st) {
    DevInfo dv;
    int rc = dev_info(dv);
    if (rc) return rc;
    const int Fs = shared ? shared->ffn : 0;
    const int Fmax = routed->ffn > Fs ? routed->ffn : Fs;
    GemmParams G;
    memset(&G, 0, sizeof(G));
    G.x = x;
    G.hbuf = at<float>(ws, L.hbuf);
    G.hout = at<float>(ws, L.hbuf);
    G.w_routed = (const uint8_t *)routed->data;
    G.w_shared = shared ? (const uint8_t *)shared->data : nullptr;
    G.pairs = pairs;
    G.pair_w = pair_w;
    G.out_pairs = out_pairs;
    G.out_shared = out_shared;
    G.slot_exp = at<int32_t>(ws, L.slot_exp);
    G.slot_row0 = at<int32_t>(ws, L.slot_row0);
    G.slot_cnt = at<int32_t>(ws, L.slot_cnt);
    G.slot_hrow0 = at<int32_t>(ws, L.slot_hrow0);
    G.T = T;
    G.E = E;
    G.k = k;
    G.H = routed->hidden;
    G.F = routed->ffn;
    G.Fs = Fs;
    G.h_stride = Fmax;
    G.x_f32 = x_f32;
    const int dbits = down_bits_of(routed);
    G.rowG = (G.H / 32) * block_bytes_of(routed->bits);
    G.eb = expert_bytes_of(routed->bits, dbits, routed->hidden, routed->ffn);
    G.nl = nl_tables(routed->codebook, true);
    G.prefix = at<int32_t>(ws, L.prefix_gu);
    hipError_t e = prefill_gemm_launch(0, routed->bits, G, dv.cus, st);  // gate/up in their format
    if (e != hipSuccess) return MOE_ERR_LAUNCH;
    G.prefix = at<int32_t>(ws, L.prefix_dn);
    e = prefill_gemm_launch(1, dbits, G, dv.cus, st);  // down in its own
    return launch_err(e);
}

}  // namespace

extern "C" {

int moe_expert_ffn(const void *x, int32_t x_dtype, int32_t T, const moe_qweights *w, const int32_t *offsets,
                   const int32_t *pairs, const int32_t *active, const float *pair_w, int32_t k, float *out_pairs,
                   int32_t path, void *ws, int64_t ws_bytes, int64_t stream) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (T != 0 && (!x || !offsets || !pairs || !active || !out_pairs || !ws)) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
    int rc = check_weights(w, w->hidden, -1);
    if (rc) return rc;
    rc = check_shape(T, w->n_experts, k, w->hidden, w->ffn);
    if (rc) return rc;
    int p = resolve_path(path, T);
    if (p == MOE_PATH_DECODE &&
        (T > MOE_DECODE_MAX_ROWS ||
         !(split_fits(T, w->n_experts, k, w->hidden, w->ffn, 0, w->bits, down_bits_of(w), 0, 256) ||
           decode_fits(T, w->n_experts, k, w->hidden, w->ffn, 0, w->bits, down_bits_of(w), x_dtype)))) {
        if (path == MOE_PATH_DECODE) return MOE_ERR_UNSUPPORTED;
        p = MOE_PATH_PREFILL;
    }
    Layout L = make_layout(T, w->n_experts, k, w->hidden, w->ffn, 0, p);
    if (ws_bytes < (int64_t)L.total) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    const int xf = x_dtype == MOE_DTYPE_F32;
    if (p == MOE_PATH_DECODE)
        return run_decode(x, xf, nullptr, offsets, pairs, active, pair_w, T, w->n_experts, k, w, nullptr, nullptr,
                          out_pairs, nullptr, nullptr, nullptr, L, ws, 0, S(stream));
    PlanParams PP{offsets, active, T, w->n_experts, k, 0, w->ffn, 0, w->hidden,
                  at<int32_t>(ws, L.slot_exp), at<int32_t>(ws, L.slot_row0), at<int32_t>(ws, L.slot_cnt),
                  at<int32_t>(ws, L.slot_hrow0), at<int32_t>(ws, L.prefix_gu), at<int32_t>(ws, L.prefix_dn)};
    if (prefill_plan_launch(PP, S(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
    return prefill_gemms(x, xf, T, w->n_experts, k, w, nullptr, pairs, pair_w, out_pairs, nullptr, L, ws,
                         S(stream));
}

int moe_layer_forward(const void *x, int32_t x_dtype, const float *logits, int32_t T, int32_t k,
                      const moe_qweights *routed, const moe_qweights *shared, float *y, int32_t *topk_idx_out,
                      float *topk_w_out, int32_t *heat, int32_t path, void *ws, int64_t ws_bytes,
                      int64_t stream) {
    if (!routed) return MOE_ERR_INVALID_ARG;
    if (T != 0 && (!x || !logits || !y || !ws)) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
    int rc = check_weights(routed, routed->hidden, -1);
    if (rc) return rc;
    if (shared) {
        rc = check_weights(shared, routed->hidden, 1);
        if (rc) return rc;
    }
    const int E = routed->n_experts, H = routed->hidden;
    rc = check_shape(T, E, k, H, routed->ffn);
    if (rc) return rc;
    // every launch reads the shared expert as one more slot in the routed
    // experts' format (and table)
    if (shared && (shared->bits != routed->bits || down_bits_of(shared) != down_bits_of(routed)))
        return MOE_ERR_UNSUPPORTED;
    if (shared && uses_table(routed) && memcmp(shared->codebook, routed->codebook, 16) != 0)
        return MOE_ERR_UNSUPPORTED;
    const int Fs = shared ? shared->ffn : 0;
    int p = resolve_path(path, T);
    if (p == MOE_PATH_DECODE && (T > MOE_DECODE_MAX_ROWS ||
                                 !(split_fits(T, E, k, H, routed->ffn, Fs, routed->bits, down_bits_of(routed), 1, 256) ||
                                   decode_fits(T, E, k, H, routed->ffn, Fs, routed->bits, down_bits_of(routed),
                                               x_dtype)))) {
        if (path == MOE_PATH_DECODE) return MOE_ERR_UNSUPPORTED;
        p = MOE_PATH_PREFILL;
    }
    Layout L = make_layout(T, E, k, H, routed->ffn, Fs, p);
    if (ws_bytes < (int64_t)L.total) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    const int xf = x_dtype == MOE_DTYPE_F32;
    hipStream_t st = S(stream);
    int32_t *idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
    float *wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
    if (p == MOE_PATH_DECODE) {
        if (E <= DEC_MAX_E_FUSED)
            return run_decode(x, xf, logits, nullptr, nullptr, nullptr, nullptr, T, E, k, routed, shared, y,
                              at<float>(ws, L.out_pairs), topk_idx_out, topk_w_out, heat, L, ws,
                              DEC_MODE_ROUTE | DEC_MODE_COMBINE, st);
        RouteParams R{logits, T, E, k, idx, wts};
        if (route_launch(R, st) != hipSuccess) return MOE_ERR_LAUNCH;
        GroupParams G{idx, T, E, k, L.nchunks, at<uint32_t>(ws, L.chunk_counts), at<int32_t>(ws, L.offsets),
                      at<int32_t>(ws, L.pairs), at<int32_t>(ws, L.active), heat};
        if (group_launch(G, st) != hipSuccess) return MOE_ERR_LAUNCH;
        return run_decode(x, xf, nullptr, at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.pairs),
                          at<int32_t>(ws, L.active), wts, T, E, k, routed, shared, y, at<float>(ws, L.out_pairs),
                          nullptr, nullptr, nullptr, L, ws, DEC_MODE_COMBINE, st);
    }
    // prefill: route, group, plan, gate/up GEMM, down GEMM, combine
    RouteParams R{logits, T, E, k, idx, wts};
    if (route_launch(R, st) != hipSuccess) return MOE_ERR_LAUNCH;
    GroupParams G{idx, T, E, k, L.nchunks, at<uint32_t>(ws, L.chunk_counts), at<int32_t>(ws, L.offsets),
                  at<int32_t>(ws, L.pairs), at<int32_t>(ws, L.active), heat};
    if (group_launch(G, st) != hipSuccess) return MOE_ERR_LAUNCH;
    PlanParams PP{at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.active), T, E, k, shared ? 1 : 0, routed->ffn,
                  Fs, H, at<int32_t>(ws, L.slot_exp), at<int32_t>(ws, L.slot_row0), at<int32_t>(ws, L.slot_cnt),
                  at<int32_t>(ws, L.slot_hrow0), at<int32_t>(ws, L.prefix_gu), at<int32_t>(ws, L.prefix_dn)};
    if (prefill_plan_launch(PP, st) != hipSuccess) return MOE_ERR_LAUNCH;
    rc = prefill_gemms(x, xf, T, E, k, routed, shared, at<int32_t>(ws, L.pairs), wts, at<float>(ws, L.out_pairs),
                       shared ? at<float>(ws, L.out_shared) : nullptr, L, ws, st);
    if (rc) return rc;
    CombineParams C{at<float>(ws, L.out_pairs), shared ? at<float>(ws, L.out_shared) : nullptr, y, T, k, H};
    return launch_err(prefill_combine_launch(C, st));
}

}  // extern "C"

// ----------------------------------------------------------------------------
// The layer without a caller workspace: its scratch is this array, one copy
// per device, held until the process ends.  Like every object of static
// storage duration it starts zeroed, which is what the workspace protocol
// needs before a first call; every call leaves its counters at zero again.
// In host code `scratch` names a host-side stand-in: the device address is
// taken with hipGetSymbolAddress, once per device, and only that is used.
// ----------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
void *g_scratch_dev[64];  // per device: the device address of `scratch`

int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}
}  // namespace

extern "C" int moe_layer_forward_noalloc(const void *x, int32_t x_dtype, const float *logits, int32_t T, int32_t k,
                                         const moe_qweights *routed, const moe_qweights *shared, float *y,
                                         int32_t *topk_idx_out, float *topk_w_out, int32_t *heat, int32_t path,
                                         int64_t stream) {
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    // a call whose workspace would exceed the array is refused (MOE_ERR_WORKSPACE) before any launch
    return moe_layer_forward(x, x_dtype, logits, T, k, routed, shared, y, topk_idx_out, topk_w_out, heat, path, ws,
                             (int64_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
