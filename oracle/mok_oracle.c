/*
 * mok_oracle.c -- plain, slow CPU oracle for one GPU's share of the
 * Mixture-of-Kittens (MoK) forward MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the HIP library; it is written from the
 * pages' description of the method:
 *   - tahou.com MoK article: routing assigns each token to experts; the
 *     receiver counts tokens per expert, plans positions so one expert's
 *     tokens are contiguous, then runs a grouped GEMM (paragraphs on MoE
 *     routing and on layout planning); the forward pass pulls tokens by
 *     (source, offset) and pushes results back, ending in a weighted merge
 *     (pull-dispatch and benchmark-scope paragraphs); minibatches sized to
 *     fill at least two full waves (minibatch paragraph); a fixed ring token
 *     buffer (ring-buffer paragraph); MXFP8 activations fused into dispatch,
 *     grouped GEMM and SwiGLU (state-machine paragraph).
 *   - PyTorchKR wiki summary, "key points": {src_rank, src_index} pull
 *     schedule built on the device without sorting.
 * Where the pages are silent the plainest reading is taken: top-k with ties
 * to the lower expert id and softmax over the k picks; stable slot order by
 * assignment id a = t*k + j; SwiGLU a = SiLU(g)*u with gate rows first and no
 * biases; OCP MX v1.0 E4M3 blocks of 32 along the contraction dimension.
 *
 * Arithmetic: fp64 throughout.  Each stored value (the SwiGLU activation,
 * the expert output, the merged output) is rounded once, from its fp64
 * value, to the storage format (bf16 round-to-nearest-even, or the MX
 * quantiser).  The fp64 values before that rounding can be returned too
 * (a_exact, y_exact, out_exact): tests use them to tell where a rounding
 * decision is close enough to a tie that an independently accumulated value
 * may legitimately land on the neighbouring code.
 *
 * Parity pins: every function below is pinned by tests/test_oracle_*.py
 * against brute force, library routines (numpy/torch) or closed forms.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* Number formats, from their definitions.                             */
/* ------------------------------------------------------------------ */

/* Round v to a binary floating-point format with p significant bits
 * (implicit bit included), smallest normal exponent emin, largest finite
 * magnitude maxv.  Round to nearest, ties to even (nearbyint in the default
 * rounding mode).  Values beyond maxv saturate when sat != 0, else become
 * +-inf.  The result is exactly representable in the format. */
static double round_to_format(double v, int p, int emin, double maxv, int sat)
{
    if (v == 0.0 || isnan(v)) return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) -> floor(log2 a) = e-1 */
    int ex = e - 1;
    if (ex < emin) ex = emin; /* subnormal range: fixed quantum 2^(emin-p+1) */
    double q = ldexp(1.0, ex - (p - 1));      /* spacing of the format at a */
    double r = nearbyint(a / q) * q;
    if (r > maxv) r = sat ? maxv : INFINITY;
    return copysign(r, v);
}

/* bf16: 8 significant bits, emin -126, max (2 - 2^-7) * 2^127 */
static double round_bf16(double v)
{
    return round_to_format(v, 8, -126, ldexp(255.0, 120), 0);
}

static uint16_t bf16_bits(double v_exact_bf16)
{
    float f = (float)v_exact_bf16;   /* exact: bf16 values are fp32 values */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit E4M3 (the "FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa,
 * no infinities, 0x7F / 0xFF are NaN, largest finite 448 = 1.75 * 2^8,
 * smallest normal 2^-6, subnormals m/8 * 2^-6. */
static double round_e4m3_sat(double v)
{
    return round_to_format(v, 4, -6, 448.0, 1);
}

ORC_API double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    if (E == 15 && m == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, E - 10);
    return s ? -mag : mag;
}

/* Code of an exactly representable E4M3 value q; sign from sgn (so -0 and
 * negative values that round to zero keep the sign bit). */
static uint8_t e4m3_code(double q, int sgn)
{
    double a = fabs(q);
    uint8_t s = (uint8_t)(sgn ? 0x80 : 0);
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -6)) {                      /* subnormal */
        return (uint8_t)(s | (uint8_t)(a / ldexp(1.0, -9)));
    }
    int e;
    frexp(a, &e);
    int ex = e - 1;                                 /* a in [2^ex, 2^(ex+1)) */
    int m = (int)((a / ldexp(1.0, ex) - 1.0) * 8.0);
    return (uint8_t)(s | (uint8_t)((ex + 7) << 3) | (uint8_t)m);
}

ORC_API uint8_t orc_e4m3_encode(double v)
{
    return e4m3_code(round_e4m3_sat(v), signbit(v) != 0);
}

ORC_API uint16_t orc_bf16_round(double v)
{
    return bf16_bits(round_bf16(v));
}

/* OCP Microscaling v1.0, MXFP8 (E4M3) block of 32 values v[0..31]:
 * shared scale X = 2^E with E = floor(log2(max|v|)) - 8 (8 = exponent of the
 * largest E4M3 normal), clamped to the E8M0 range [-127, 127]; an all-zero
 * block takes E = -127.  Element codes: v / X rounded to E4M3 with ties to
 * even, saturating at +-448.  Scale byte = E + 127. */
ORC_API void orc_mx_block(const double* v, uint8_t* codes, uint8_t* scale_byte)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int E;
    if (amax == 0.0) {
        E = -127;
    } else {
        int e;
        frexp(amax, &e);
        E = (e - 1) - 8;
        if (E < -127) E = -127;
        if (E > 127) E = 127;
    }
    for (int i = 0; i < 32; ++i) codes[i] = orc_e4m3_encode(ldexp(v[i], -E));
    *scale_byte = (uint8_t)(E + 127);
}

ORC_API void orc_mx_quantize(const double* v, int64_t n, uint8_t* codes, uint8_t* scales)
{
    for (int64_t b = 0; b < n / 32; ++b) orc_mx_block(v + 32 * b, codes + 32 * b, scales + b);
}

ORC_API void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ldexp(orc_e4m3_decode(codes[i]), (int)scales[i / 32] - 127);
}

/* ------------------------------------------------------------------ */
/* Route: per-token top-k over E logits with softmax over the k picks.   */
/* (tahou.com article, routing paragraph: the router picks experts per   */
/* token.  The pages fix neither k, the gate form nor ties; reading:     */
/* k largest, ties to the lower expert id, ordered by descending logit,  */
/* gates = softmax over the k picks, which equals the full softmax        */
/* renormalised over the top-k.)                                         */
/* ------------------------------------------------------------------ */
ORC_API int orc_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                           int32_t* topk_idx, float* topk_gate)
{
    if (k < 1 || k > E) return 1;
    char* taken = (char*)malloc((size_t)E);
    if (!taken) return 2;
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                /* strict '>' while scanning upward keeps the lower id on ties */
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            topk_idx[t * k + j] = best;
        }
        double l0 = (double)l[topk_idx[t * k]];
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += exp((double)l[topk_idx[t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            topk_gate[t * k + j] = (float)(exp((double)l[topk_idx[t * k + j]] - l0) / s);
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Schedule: count per local expert, exclusive offsets, then place each   */
/* local assignment at the next free slot of its expert in assignment     */
/* order.  (tahou.com article, layout-planning paragraph: count first,    */
/* then plan positions so one expert's tokens are contiguous; wiki        */
/* summary: the pull table {src_rank, src_index} is made without a sort.) */
/* slot_of_assign[a] = -1 for assignments to non-local experts.           */
/* ------------------------------------------------------------------ */
ORC_API int orc_build_schedule(const int32_t* topk_idx, int64_t T, int32_t k,
                               int32_t expert_base, int32_t n_local,
                               int32_t* counts, int32_t* offsets,
                               int32_t* slot_of_assign, int32_t* assign_of_slot)
{
    int64_t A = T * k;
    for (int e = 0; e < n_local; ++e) counts[e] = 0;
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = topk_idx[a] - expert_base;
        if (e >= 0 && e < n_local) counts[e]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < n_local; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_local > 0 ? n_local : 1));
    if (!cursor) return 2;
    for (int e = 0; e < n_local; ++e) cursor[e] = offsets[e];
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = topk_idx[a] - expert_base;
        if (e >= 0 && e < n_local) {
            int32_t s = cursor[e]++;
            slot_of_assign[a] = s;
            assign_of_slot[s] = (int32_t)a;
        } else {
            slot_of_assign[a] = -1;
        }
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Minibatch windows.  (tahou.com article, minibatch paragraph: a         */
/* minibatch is what is handed to expert compute at once and should fill */
/* at least two full waves of the compute units; ring-buffer paragraph:  */
/* a fixed buffer reused per minibatch.)  Window b covers schedule slots  */
/* [bM, min(R, (b+1)M)); its expert segments are the offsets clipped to   */
/* that range: win_seg[b][e] = clamp(offsets[e], lo_b, hi_b).             */
/* ------------------------------------------------------------------ */
ORC_API void orc_windows(const int32_t* offsets, int32_t n_local, int32_t M, int32_t nwin,
                         int32_t* win_seg)
{
    int64_t R = offsets[n_local];
    for (int64_t b = 0; b < nwin; ++b) {
        int64_t lo = b * (int64_t)M, hi = (b + 1) * (int64_t)M;
        if (hi > R) hi = R;
        if (lo > R) lo = R;
        for (int e = 0; e <= n_local; ++e) {
            int64_t v = offsets[e];
            if (v < lo) v = lo;
            if (v > hi) v = hi;
            win_seg[b * (n_local + 1) + e] = (int32_t)v;
        }
    }
}

/* Two-wave rule for the minibatch: a grouped GEMM with output width n_out,
 * tiles tile_m x tile_n and n_cus compute units forms one full wave every
 * n_cus tiles; two waves need M = 2 * n_cus * tile_m * tile_n / n_out rows,
 * rounded up to a multiple of 64 rows and clipped to the rows available. */
ORC_API int32_t orc_choose_minibatch(int32_t n_cus, int32_t tile_m, int32_t tile_n,
                                     int32_t n_out, int64_t rows)
{
    int64_t need = 2LL * n_cus * tile_m * tile_n;
    int64_t m = (need + n_out - 1) / n_out;
    m = ((m + 63) / 64) * 64;
    if (rows > 0 && m > rows) m = rows;
    return (int32_t)m;
}

/* ------------------------------------------------------------------ */
/* Dispatch (pull): the row of slot s is the token of assignment          */
/* assign_of_slot[s], a bit copy (tahou.com article, pull paragraph: the  */
/* receiver reads by source and offset).  With MXFP8 the row is quantised */
/* in blocks of 32 along the hidden dimension on the way (state-machine   */
/* paragraph: MXFP8 fused into dispatch).                                 */
/* x is the pool flattened to [T][H]; token t is row t.                   */
/* ------------------------------------------------------------------ */
ORC_API void orc_gather_rows(const uint16_t* x, int32_t H, int32_t k,
                             const int32_t* assign_of_slot, const int64_t* slots, int64_t n,
                             int32_t mxfp8, uint16_t* out_bf16, uint8_t* out_codes,
                             uint8_t* out_scales)
{
    double* v = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t r = 0; r < n; ++r) {
        int64_t t = assign_of_slot[slots[r]] / k;
        const uint16_t* src = x + t * (int64_t)H;
        if (!mxfp8) {
            memcpy(out_bf16 + r * (int64_t)H, src, sizeof(uint16_t) * (size_t)H);
        } else {
            for (int h = 0; h < H; ++h) v[h] = bf16_value(src[h]);
            orc_mx_quantize(v, H, out_codes + r * (int64_t)H, out_scales + r * (int64_t)(H / 32));
        }
    }
    free(v);
}

/* MXFP8 weights (a wider reading of the article's MXFP8 datapath: the    */
/* weights in the same OCP MX format as the activations, quantised per    */
/* row in blocks of 32 along the contraction dimension K).  w: bf16 bits  */
/* [rows][K]; codes [rows][K], scales [rows][K/32].                        */
ORC_API void orc_mx_quantize_rows_bf16(const uint16_t* w, int64_t rows, int32_t K, uint8_t* codes,
                                       uint8_t* scales)
{
    #pragma omp parallel
    {
        double* v = (double*)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int32_t k = 0; k < K; ++k) v[k] = bf16_value(w[r * (int64_t)K + k]);
            orc_mx_quantize(v, K, codes + r * (int64_t)K, scales + r * (int64_t)(K / 32));
        }
        free(v);
    }
}

/* Weight element k of row r: bf16 value, or the MXFP8 code times 2^E of its block. */
static double w_value(const uint16_t* wb, const uint8_t* wc, const uint8_t* ws, int64_t r, int32_t K,
                      int32_t k)
{
    if (!wc) return bf16_value(wb[r * (int64_t)K + k]);
    return ldexp(orc_e4m3_decode(wc[r * (int64_t)K + k]), (int)ws[r * (int64_t)(K / 32) + k / 32] - 127);
}

/* ------------------------------------------------------------------ */
/* Expert SwiGLU FFN for a list of dispatched rows (tahou.com article:    */
/* grouped GEMM over the expert-contiguous layout; SwiGLU named in the    */
/* MXFP8 datapath).  Row r belongs to local expert expert_of_row[r]:      */
/*   h = W_gu[e] . x   (W_gu rows 0..I-1 = gate, I..2I-1 = up; no bias)   */
/*   a_i = SiLU(h_i) * h_{I+i},  SiLU(z) = z / (1 + exp(-z))              */
/*   a -> bf16 (or MXFP8 blocks of 32 along I, then dequantised)          */
/*   y = W_d[e] . a  -> bf16                                               */
/* a_exact [n][I] / y_exact [n][H] (optional, may be NULL): the fp64      */
/* values of a and y before their rounding.                                */
/* x rows are bf16 bits (xb) or MXFP8 codes + scales (xc, xs).  Weights   */
/* are bf16 (w_gu, w_d) or, when gu_c is not null, MXFP8 codes + scales   */
/* of the same matrices (gu_c/gu_s [n_local*2I][H], d_c/d_s [n_local*H][I]).*/
/* ------------------------------------------------------------------ */
ORC_API void orc_ffn_rows(const uint16_t* xb, const uint8_t* xc, const uint8_t* xs,
                          const int32_t* expert_of_row, int64_t n, int32_t H, int32_t I,
                          const uint16_t* w_gu, const uint16_t* w_d, int32_t mxfp8,
                          const uint8_t* gu_c, const uint8_t* gu_s, const uint8_t* d_c,
                          const uint8_t* d_s, uint16_t* y, double* a_exact, double* y_exact)
{
    #pragma omp parallel
    {
        double* xv = (double*)malloc(sizeof(double) * (size_t)H);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        uint8_t* ac = (uint8_t*)malloc((size_t)I);
        uint8_t* as = (uint8_t*)malloc((size_t)(I / 32 + 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            int64_t e = expert_of_row[r];
            if (!mxfp8) {
                for (int h = 0; h < H; ++h) xv[h] = bf16_value(xb[r * (int64_t)H + h]);
            } else {
                orc_mx_dequantize(xc + r * (int64_t)H, xs + r * (int64_t)(H / 32), H, xv);
            }
            const int64_t gbase = e * 2 * (int64_t)I;     /* first W_gu row of expert e */
            for (int i = 0; i < I; ++i) {
                double g = 0.0, u = 0.0;
                for (int h = 0; h < H; ++h) {
                    g += w_value(w_gu, gu_c, gu_s, gbase + i, H, h) * xv[h];
                    u += w_value(w_gu, gu_c, gu_s, gbase + I + i, H, h) * xv[h];
                }
                double silu = g / (1.0 + exp(-g));
                a[i] = silu * u;
            }
            if (a_exact) memcpy(a_exact + r * (int64_t)I, a, sizeof(double) * (size_t)I);
            if (!mxfp8) {
                for (int i = 0; i < I; ++i) a[i] = round_bf16(a[i]);
            } else {
                orc_mx_quantize(a, I, ac, as);
                orc_mx_dequantize(ac, as, I, a);
            }
            const int64_t dbase = e * (int64_t)H;         /* first W_d row of expert e */
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int i = 0; i < I; ++i) acc += w_value(w_d, d_c, d_s, dbase + h, I, i) * a[i];
                if (y_exact) y_exact[r * (int64_t)H + h] = acc;
                y[r * (int64_t)H + h] = bf16_bits(round_bf16(acc));
            }
        }
        free(xv); free(a); free(ac); free(as);
    }
}

/* ------------------------------------------------------------------ */
/* Combine (push) and final weighted merge (tahou.com article: results    */
/* are pushed back to their token; the benchmark scope ends with the      */
/* weighted merge).  For each listed token with at least one local        */
/* assignment: out = bf16( sum over local j ascending of gate_tj * y[slot]*/
/* ).  y_of_slot(s) is row y_row_of_slot[s] of y (so callers may pass     */
/* only sampled rows).  Tokens without a local assignment are skipped     */
/* (written[r] = 0) and their rows are left untouched.  out_exact         */
/* (optional) receives the fp64 sums before rounding.                     */
/* ------------------------------------------------------------------ */
ORC_API void orc_combine_tokens(const uint16_t* y, const int64_t* y_row_of_slot,
                                const int32_t* slot_of_assign, const float* topk_gate,
                                const int64_t* tokens, int64_t n, int32_t k, int32_t H,
                                uint16_t* out, uint8_t* written, double* out_exact)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        int64_t t = tokens[r];
        int any = 0;
        for (int j = 0; j < k; ++j) any |= slot_of_assign[t * k + j] >= 0;
        written[r] = (uint8_t)any;
        if (!any) continue;
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t s = slot_of_assign[t * k + j];
                if (s < 0) continue;
                acc += (double)topk_gate[t * k + j] * bf16_value(y[y_row_of_slot[s] * H + h]);
            }
            if (out_exact) out_exact[r * (int64_t)H + h] = acc;
            out[r * (int64_t)H + h] = bf16_bits(round_bf16(acc));
        }
    }
}

/* Array forms of the scalar format helpers (for the pins). */
ORC_API void orc_e4m3_encode_n(const double* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

ORC_API void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

ORC_API void orc_bf16_round_n(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(v[i]);
}

/* Threads the OpenMP loops above run on. */
#include <omp.h>
ORC_API int orc_max_threads(void) { return omp_get_max_threads(); }
