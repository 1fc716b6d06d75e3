/*
 * oracle.c -- plain, slow, obviously-correct CPU reference of the routed
 * mixture-of-experts FFN layer over block-quantized expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the GPU library; the two meet only in the bytes of the seeded inputs.
 *
 * Arithmetic is IEEE binary64 throughout.  Dequantized weights are exact in
 * binary64 (an fp16 scale times a small integer), so the only rounding is
 * in the dot products, the exponentials and the sums.
 *
 * What each function follows (the pages are the forum thread "把 Strata 搬上
 * SGLang 引擎 的嘗試" (lcz.me post 31686), the Strata "Several requests at
 * once (batch slots)" document, and the extended-strata-moe "Reference"):
 *
 *  - orc_half_to_double: IEEE 754 binary16 by its definition (sign, 5-bit
 *    exponent with bias 15, 10-bit fraction, subnormals, inf/NaN).
 *  - orc_dequant_block: the quantized block of 32 weights.  The thread's
 *    §四 names the 4-bit block as 32 values in 18 bytes (an fp16 scale and
 *    16 bytes of 4-bit codes); a 3-bit block of 14 bytes follows the same
 *    plan with 12 bytes of codes.  The byte order of codes inside a block
 *    is not on the pages; the readings taken are written below and in the
 *    repository's design notes.
 *  - orc_route: router softmax and top-k (thread, §TL;DR and §三: top-10 of
 *    512 experts; extended-strata-moe Reference, "Routing trace format":
 *    k expert ids and k weights per token and layer).
 *  - orc_group: grouping of (token, expert) pairs so each expert computes
 *    only its routed rows (thread §二, the expert-scoped layout).
 *  - orc_expert_ffn / orc_layer_forward: per expert gather, dequant,
 *    gate/up projection, SwiGLU, down projection, weighted scatter-add
 *    (thread §TL;DR, the grouped expert call), plus the always-on shared
 *    expert that every row of a window reads (batch-slots document,
 *    opening section).
 *
 * Parity pins live in tests/ (closed forms, brute force, golden blocks,
 * invariants).  No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_MEM (-2)

int orc_version(void) { return 1; }

/*
 * Threads.  Built with OpenMP, the loops over rows (tokens, or the pairs of
 * one expert) and over matrix rows in the dequantization run in parallel.
 * Every row's arithmetic is the same sequence of operations as in the serial
 * build (each row is computed start to end by one thread), so the results
 * are bitwise those of the serial build whatever the thread count.
 */
int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Scalar formats                                                       */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16 -> binary64, from the definition. */
double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Quantized blocks                                                     */
/* ------------------------------------------------------------------ */

/* the non-linear 4-bit format (code 20): the 4-bit block's layout, each code
 * indexing a 16-entry table of signed 8-bit values (thread §四 names a
 * non-linear 4-bit block of 32 values in 18 bytes; the pages print no table,
 * so the table is an input, set with orc_set_codebook) */
#define ORC_BITS_NL4 20
static int8_t orc_cb[16];

void orc_set_codebook(const int8_t *cb) { memcpy(orc_cb, cb, 16); }

int orc_block_bytes(int bits) {
    if (bits == 4 || bits == ORC_BITS_NL4) return 18;
    if (bits == 3) return 14;
    return -1;
}

/*
 * A weight format: the bit width of the gate and up projections in bits
 * 0..7, that of the down projection in bits 8..15, 0 there meaning the same
 * width as gate/up (so a plain 3 or 4 is a uniform format).  The thread's §三
 * decode table pairs each gate/up format with a down format of its own (a
 * 2- or 3-bit gate/up with a 4-bit down); here the same per-projection choice
 * is made between the 3-bit, 4-bit and non-linear 4-bit (20) blocks above.
 * -1 for anything else.
 */
int orc_format_bits(int fmt, int down) {
    int gu = fmt & 0xFF, dn = (fmt >> 8) & 0xFF;
    if (fmt < 0 || (fmt >> 16) != 0) return -1;
    if (dn == 0) dn = gu;
    if (orc_block_bytes(gu) < 0 || orc_block_bytes(dn) < 0) return -1;
    return down ? dn : gu;
}

int64_t orc_expert_bytes(int fmt, int hidden, int ffn) {
    int bg = orc_format_bits(fmt, 0), bd = orc_format_bits(fmt, 1);
    if (bg < 0 || bd < 0 || hidden <= 0 || ffn <= 0 || hidden % 32 || ffn % 32) return -1;
    /* gate [ffn][hidden] + up [ffn][hidden] + down [hidden][ffn] */
    return (int64_t)hidden * (ffn / 32) * (2 * orc_block_bytes(bg) + orc_block_bytes(bd));
}

/*
 * One block of 32 weights.  Bytes 0..1 hold the scale d as little-endian
 * binary16.  The integer code c_i of weight i (0 <= i < 32) is read as:
 *   4-bit (18 bytes): byte 2+(i mod 16), low nibble for i < 16, high nibble
 *                     for i >= 16; value d * (c_i - 8).
 *   3-bit (14 bytes): low two bits = bits 2*(i div 8).. of byte 2+(i mod 8);
 *                     third bit = bit i of the little-endian 32-bit word at
 *                     bytes 10..13; value d * (c_i - 4).
 *   non-linear 4-bit (18 bytes, code 20): c_i as for 4-bit; value
 *                     d * codebook[c_i] (the table set by orc_set_codebook).
 * Symmetric codes: no zero point, only the fixed bias 2^(bits-1).
 */
void orc_dequant_block(int bits, const uint8_t *blk, double *out) {
    double d = orc_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    int i;
    if (bits == 4 || bits == ORC_BITS_NL4) {
        for (i = 0; i < 32; ++i) {
            int c = (i < 16) ? (blk[2 + i] & 0x0F) : (blk[2 + (i - 16)] >> 4);
            out[i] = (bits == ORC_BITS_NL4) ? d * (double)orc_cb[c] : d * (double)(c - 8);
        }
    } else {
        uint32_t qh = (uint32_t)blk[10] | ((uint32_t)blk[11] << 8) |
                      ((uint32_t)blk[12] << 16) | ((uint32_t)blk[13] << 24);
        for (i = 0; i < 32; ++i) {
            int lo = (blk[2 + (i % 8)] >> (2 * (i / 8))) & 3;
            int hi = (int)((qh >> i) & 1u);
            int c = lo | (hi << 2);
            out[i] = d * (double)(c - 4);
        }
    }
}

/* A [rows][cols] matrix stored row by row, cols/32 blocks per row. */
int orc_dequant_matrix(int bits, const uint8_t *m, int rows, int cols, double *out) {
    int bb = orc_block_bytes(bits);
    int r, b;
    if (bb < 0 || cols % 32) return ORC_ERR_ARG;
#pragma omp parallel for private(b) schedule(static)
    for (r = 0; r < rows; ++r)
        for (b = 0; b < cols / 32; ++b)
            orc_dequant_block(bits, m + ((int64_t)r * (cols / 32) + b) * bb,
                              out + (int64_t)r * cols + (int64_t)b * 32);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Router projection: the logits the router ranks                      */
/* ------------------------------------------------------------------ */

/*
 * logits[t][e] = sum over h of x[t][h] * W[e][h], W the router matrix
 * [E][H] in bfloat16 (row e is expert e's router vector), x fp32 or bf16.
 * Products and the sum in binary64, h ascending.  The step that precedes
 * the routed path: the extended-strata-moe "Reference", section "Tools"
 * (route_dump / route_predict read a layer's router from its hidden state),
 * and the forum thread's post "prefill 36.8 -> 334", section on the decode
 * wall (one captured graph per window over all 48 layers).
 */
int orc_router_logits(const void *x, int x_dtype, int T, int H, const uint16_t *w, int E,
                      double *logits) {
    int t;
    if (T < 0 || H <= 0 || E <= 0 || (x_dtype != 0 && x_dtype != 1)) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        int e, h;
        for (e = 0; e < E; ++e) {
            const uint16_t *we = w + (int64_t)e * H;
            double acc = 0.0;
            for (h = 0; h < H; ++h) {
                double xv = x_dtype == 0 ? (double)((const float *)x)[(int64_t)t * H + h]
                                         : orc_bf16_to_double(((const uint16_t *)x)[(int64_t)t * H + h]);
                acc += xv * orc_bf16_to_double(we[h]);
            }
            logits[(int64_t)t * E + e] = acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Router: top-k over raw logits, softmax over the k selected           */
/* ------------------------------------------------------------------ */

/*
 * Per row t: k rounds, each taking the largest logit not yet taken; a tie
 * goes to the lower expert id (scan in ascending id, replace only on a
 * strictly greater value).  The selection compares the fp32 logits
 * themselves.  Weights: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over
 * the k selected, l_0 being the largest, so the k weights sum to one.
 */
int orc_route(const float *logits, int T, int E, int k, int32_t *idx, double *w) {
    int t, j, e;
    char *taken;
    if (T < 0 || E <= 0 || k <= 0 || k > E) return ORC_ERR_ARG;
    taken = (char *)malloc((size_t)E);
    if (!taken) return ORC_ERR_MEM;
    for (t = 0; t < T; ++t) {
        const float *l = logits + (int64_t)t * E;
        double lmax, sum;
        memset(taken, 0, (size_t)E);
        for (j = 0; j < k; ++j) {
            int best = -1;
            for (e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[(int64_t)t * k + j] = best;
        }
        lmax = (double)l[idx[(int64_t)t * k]];
        sum = 0.0;
        for (j = 0; j < k; ++j) sum += exp((double)l[idx[(int64_t)t * k + j]] - lmax);
        for (j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = exp((double)l[idx[(int64_t)t * k + j]] - lmax) / sum;
    }
    free(taken);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Grouping of (token, expert) pairs                                    */
/* ------------------------------------------------------------------ */

/*
 * Pair id p = t*k + j.  counts[e] = number of pairs routed to e;
 * offsets = exclusive prefix sum (E+1 entries); pairs[] lists the pair ids
 * of expert 0, then expert 1, ..., each in increasing p, i.e. ordered by
 * (expert, token, slot).  active[0] = number of experts with a nonzero
 * count, active[1..] = those ids in ascending order.
 */
int orc_group(const int32_t *idx, int T, int E, int k, int32_t *offsets, int32_t *pairs,
              int32_t *active) {
    int64_t p, n = (int64_t)T * k;
    int e, na = 0;
    int32_t *fill;
    if (T < 0 || E <= 0 || k <= 0) return ORC_ERR_ARG;
    for (p = 0; p < n; ++p)
        if (idx[p] < 0 || idx[p] >= E) return ORC_ERR_ARG;
    fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return ORC_ERR_MEM;
    for (e = 0; e <= E; ++e) offsets[e] = 0;
    for (p = 0; p < n; ++p) offsets[idx[p] + 1] += 1;
    for (e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (p = 0; p < n; ++p) {
        e = idx[p];
        pairs[offsets[e] + fill[e]] = (int32_t)p;
        fill[e] += 1;
    }
    for (e = 0; e < E; ++e)
        if (offsets[e + 1] > offsets[e]) active[1 + na++] = e;
    active[0] = na;
    free(fill);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* One expert: SwiGLU FFN                                                */
/* ------------------------------------------------------------------ */

/* Dequantized expert: gate [F][H], up [F][H], down [H][F]. */
typedef struct {
    double *gate, *up, *down;
    int H, F;
} orc_expert;

static int orc_load_expert(int fmt, const uint8_t *blob, int H, int F, orc_expert *ex) {
    int bg = orc_format_bits(fmt, 0), bd = orc_format_bits(fmt, 1);
    int64_t mat = (int64_t)H * (F / 32) * orc_block_bytes(bg); /* bytes of the gate (and the up) matrix */
    ex->H = H;
    ex->F = F;
    ex->gate = (double *)malloc(sizeof(double) * (size_t)H * F);
    ex->up = (double *)malloc(sizeof(double) * (size_t)H * F);
    ex->down = (double *)malloc(sizeof(double) * (size_t)H * F);
    if (!ex->gate || !ex->up || !ex->down) return ORC_ERR_MEM;
    orc_dequant_matrix(bg, blob, F, H, ex->gate);
    orc_dequant_matrix(bg, blob + mat, F, H, ex->up);
    orc_dequant_matrix(bd, blob + 2 * mat, H, F, ex->down);
    return ORC_OK;
}

static void orc_free_expert(orc_expert *ex) {
    free(ex->gate);
    free(ex->up);
    free(ex->down);
    ex->gate = ex->up = ex->down = NULL;
}

/* o = W_down * (silu(W_gate x) * (W_up x)); hid is scratch of F doubles. */
static void orc_ffn_row(const orc_expert *ex, const double *x, double *hid, double *o) {
    int f, h, H = ex->H, F = ex->F;
    for (f = 0; f < F; ++f) {
        const double *gr = ex->gate + (int64_t)f * H;
        const double *ur = ex->up + (int64_t)f * H;
        double g = 0.0, u = 0.0;
        for (h = 0; h < H; ++h) {
            g += gr[h] * x[h];
            u += ur[h] * x[h];
        }
        hid[f] = g / (1.0 + exp(-g)) * u;
    }
    for (h = 0; h < H; ++h) {
        const double *dr = ex->down + (int64_t)h * F;
        double acc = 0.0;
        for (f = 0; f < F; ++f) acc += dr[f] * hid[f];
        o[h] = acc;
    }
}

/* x as doubles: dtype 0 = fp32, 1 = bf16 */
static void orc_load_x_row(const void *x, int x_dtype, int H, int t, double *out) {
    int h;
    if (x_dtype == 0) {
        const float *xf = (const float *)x + (int64_t)t * H;
        for (h = 0; h < H; ++h) out[h] = (double)xf[h];
    } else {
        const uint16_t *xb = (const uint16_t *)x + (int64_t)t * H;
        for (h = 0; h < H; ++h) out[h] = orc_bf16_to_double(xb[h]);
    }
}

/*
 * Routed experts on a given grouping: out_pairs[p][:] = w_p * FFN_e(x_t) for
 * every pair p = t*k + j listed in pairs[offsets[e]..offsets[e+1]) of every
 * active expert e.  pair_w == NULL means weight 1.  Rows of out_pairs for
 * pairs not listed are left untouched.
 */
int orc_expert_ffn(const void *x, int x_dtype, int T, int k, int fmt, int E, int H, int F,
                   const uint8_t *blobs, const int32_t *offsets, const int32_t *pairs,
                   const int32_t *active, const double *pair_w, double *out_pairs) {
    int64_t eb = orc_expert_bytes(fmt, H, F);
    int a, rc = ORC_OK;
    if (eb < 0 || T < 0 || k <= 0 || E <= 0 || (x_dtype != 0 && x_dtype != 1)) return ORC_ERR_ARG;
    for (a = 0; a < active[0]; ++a) {
        int e = active[1 + a], q, h;
        orc_expert ex;
        if (e < 0 || e >= E) { rc = ORC_ERR_ARG; goto done; }
        if (orc_load_expert(fmt, blobs + (int64_t)e * eb, H, F, &ex) != ORC_OK) {
            orc_free_expert(&ex);
            rc = ORC_ERR_MEM;
            goto done;
        }
#pragma omp parallel private(q, h)
        {
            double *xr_t = (double *)malloc(sizeof(double) * (size_t)H);
            double *hid_t = (double *)malloc(sizeof(double) * (size_t)F);
            double *o_t = (double *)malloc(sizeof(double) * (size_t)H);
            if (!xr_t || !hid_t || !o_t) abort();
#pragma omp for schedule(dynamic, 1)
            for (q = offsets[e]; q < offsets[e + 1]; ++q) {
                int p = pairs[q];
                double wp = pair_w ? pair_w[p] : 1.0;
                orc_load_x_row(x, x_dtype, H, p / k, xr_t);
                orc_ffn_row(&ex, xr_t, hid_t, o_t);
                for (h = 0; h < H; ++h) out_pairs[(int64_t)p * H + h] = wp * o_t[h];
            }
            free(xr_t);
            free(hid_t);
            free(o_t);
        }
        orc_free_expert(&ex);
    }
done:
    return rc;
}

/*
 * The whole layer.  rows == NULL computes every token; otherwise only the
 * n_rows tokens listed (routing and grouping are always done for all T).
 * y is [n_rows][H] in the order of rows (or [T][H]).  idx/w receive the
 * routing of all T tokens.  shared == NULL means no shared expert.
 *
 * Combine order per token: (((w_0 o_0 + w_1 o_1) + ...) + w_{k-1} o_{k-1}) + s.
 */
int orc_layer_forward(const void *x, int x_dtype, const float *logits, int T, int E, int k,
                      int H, int fmt, int F, const uint8_t *routed, int s_fmt, int s_F,
                      const uint8_t *shared, int n_rows, const int32_t *rows, double *y,
                      int32_t *idx, double *w) {
    int64_t eb = orc_expert_bytes(fmt, H, F), n = (int64_t)T * k;
    int32_t *offsets = NULL, *pairs = NULL, *active = NULL, *row_of = NULL;
    double *pair_o = NULL;
    int rc = ORC_OK, nr = rows ? n_rows : T, i, a, h;
    if (eb < 0 || T < 0 || E <= 0 || k <= 0 || k > E || (x_dtype != 0 && x_dtype != 1)) return ORC_ERR_ARG;
    if (shared && orc_expert_bytes(s_fmt, H, s_F) < 0) return ORC_ERR_ARG;
    offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    pairs = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    active = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    row_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T ? T : 1));
    pair_o = (double *)calloc((size_t)nr * k * H + 1, sizeof(double));
    if (!offsets || !pairs || !active || !row_of || !pair_o) { rc = ORC_ERR_MEM; goto done; }

    rc = orc_route(logits, T, E, k, idx, w);
    if (rc) goto done;
    rc = orc_group(idx, T, E, k, offsets, pairs, active);
    if (rc) goto done;

    /* which output row (if any) each token feeds */
    for (i = 0; i < T; ++i) row_of[i] = rows ? -1 : i;
    if (rows)
        for (i = 0; i < n_rows; ++i) {
            if (rows[i] < 0 || rows[i] >= T) { rc = ORC_ERR_ARG; goto done; }
            row_of[rows[i]] = i;
        }

    /* routed experts, ascending id; each dequantized once */
    for (a = 0; a < active[0]; ++a) {
        int e = active[1 + a], q, need = 0;
        orc_expert ex;
        for (q = offsets[e]; q < offsets[e + 1]; ++q)
            if (row_of[pairs[q] / k] >= 0) need = 1;
        if (!need) continue;
        if (orc_load_expert(fmt, routed + (int64_t)e * eb, H, F, &ex) != ORC_OK) {
            orc_free_expert(&ex);
            rc = ORC_ERR_MEM;
            goto done;
        }
#pragma omp parallel private(q, h)
        {
            double *xr_t = (double *)malloc(sizeof(double) * (size_t)H);
            double *hid_t = (double *)malloc(sizeof(double) * (size_t)F);
            double *o_t = (double *)malloc(sizeof(double) * (size_t)H);
            if (!xr_t || !hid_t || !o_t) abort();
#pragma omp for schedule(dynamic, 1)
            for (q = offsets[e]; q < offsets[e + 1]; ++q) {
                int p = pairs[q], t = p / k, j = p % k;
                if (row_of[t] < 0) continue;
                orc_load_x_row(x, x_dtype, H, t, xr_t);
                orc_ffn_row(&ex, xr_t, hid_t, o_t);
                for (h = 0; h < H; ++h) pair_o[((int64_t)row_of[t] * k + j) * H + h] = o_t[h];
            }
            free(xr_t);
            free(hid_t);
            free(o_t);
        }
        orc_free_expert(&ex);
    }

    /* combine in slot order, then the shared expert */
#pragma omp parallel for private(h) schedule(static)
    for (i = 0; i < nr; ++i) {
        int t = rows ? rows[i] : i, j;
        for (h = 0; h < H; ++h) {
            double acc = w[(int64_t)t * k] * pair_o[((int64_t)i * k) * H + h];
            for (j = 1; j < k; ++j) acc += w[(int64_t)t * k + j] * pair_o[((int64_t)i * k + j) * H + h];
            y[(int64_t)i * H + h] = acc;
        }
    }
    if (shared) {
        orc_expert sx;
        if (orc_load_expert(s_fmt, shared, H, s_F, &sx) != ORC_OK) {
            orc_free_expert(&sx);
            rc = ORC_ERR_MEM;
            goto done;
        }
#pragma omp parallel private(i, h)
        {
            double *xr_t = (double *)malloc(sizeof(double) * (size_t)H);
            double *hid_t = (double *)malloc(sizeof(double) * (size_t)s_F);
            double *o_t = (double *)malloc(sizeof(double) * (size_t)H);
            if (!xr_t || !hid_t || !o_t) abort();
#pragma omp for schedule(dynamic, 1)
            for (i = 0; i < nr; ++i) {
                int t = rows ? rows[i] : i;
                orc_load_x_row(x, x_dtype, H, t, xr_t);
                orc_ffn_row(&sx, xr_t, hid_t, o_t);
                for (h = 0; h < H; ++h) y[(int64_t)i * H + h] += o_t[h];
            }
            free(xr_t);
            free(hid_t);
            free(o_t);
        }
        orc_free_expert(&sx);
    }
done:
    free(offsets);
    free(pairs);
    free(active);
    free(row_of);
    free(pair_o);
    return rc;
}
