/*
 * moe_oracle.c -- plain, slow CPU oracle for the grouped top-k W4A16 MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Its only callers are the tests, the smoke check and the
 * benchmark's CPU-baseline leg.  It shares no code, header, table or
 * constant with the HIP library: every definition below is written out
 * again from the pages.
 *
 * Sources (web pages, cited by title and section):
 *  [MXFP4 card]  "LFM2.5-24B-A2B -- Packed MXFP4 Inference" (Hugging Face model
 *                card FP8Enjoyer/LFM2.5-24B-A2B-MXFP4), sections "Model and
 *                quantization" and "What was optimized / Grouped top-4 expert
 *                execution".
 *  [NVFP4 card]  "primitive-ai/LFM2.5-24B-A2B-NVFP4A16", section "What's
 *                quantized to what".
 *  [Budget art.] "LFM2.5-24B-A2B on Your Own Hardware: The RAM, KV Cache and
 *                Bandwidth Budget", section "Where do the 2.45B active
 *                parameters actually go?" (hidden 2048, expert intermediate
 *                1536, 64 experts, top-4, SwiGLU gate/up/down).
 *
 * What it computes, per token t and routing slot j (expert e = ids[t][j]):
 *   u      = x[t]                        (or the weightless RMS pre-norm of x[t])
 *   g[n]   = bf16( sum_k u[k] * Wg_e[n,k] )           n < I
 *   v[n]   = bf16( sum_k u[k] * Wu_e[n,k] )
 *   h[n]   = bf16( silu(g[n]) * v[n] )
 *   y_j[m] = bf16( sum_n h[n] * Wd_e[m,n] )           m < H
 *   acc    = +0;  for j = 0..k-1: acc = bf16(acc + bf16(w[t][j] * y_j[m]))
 *   out    = acc, or bf16(residual + acc) when a residual is given.
 * Dequantised weight W[n,k] = E2M1(q) * S * g_tensor, where S is the E8M0
 * block scale 2^(e-127) per 32 values along k ([MXFP4 card], "Model and
 * quantization") or the E4M3FN scale per 16 values, and g_tensor is the FP32
 * per-expert tensor scale of the NVFP4 variant ([NVFP4 card], "What's
 * quantized to what": gate and up share one global scale, down has its own).
 * g_tensor = 1 for MXFP4.
 *
 * Every bf16() is round-to-nearest-even applied once, directly from the fp64
 * value.  Sums run sequentially in fp64 with k ascending.  Build with
 * -O2 -ffp-contract=off and no fast-math, so no FMA changes any rounding.
 *
 * W4A4 variant ([NVFP4 card], "Why this quant": the W4A4 builds quantise the
 * expert activations to 4 bits as well, for FP4 matrix hardware): u and every
 * h are replaced by their MXFP4 quantisation (see oracle_quant_mxfp4) before
 * the GEMV that consumes them; everything else is unchanged.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): low nibble = even k; scale blocks aligned at k = 0 along a
 * row; matrices stored [out][in] row-major; one rounding inside silu*up;
 * the combine multiplies and adds with separate BF16 roundings (no fused
 * multiply-add), in slot order, starting from +0; the residual add is a
 * separate rounding after the combine; the pre-norm is
 * u = bf16(x / sqrt(mean(x^2) + eps)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* scale-format selectors of this oracle's own interface */
#define ORC_FMT_E8M0_G32 0
#define ORC_FMT_E4M3_G16 1

/* ---------------------------------------------------------------------- */
/* Formats                                                                 */
/* ---------------------------------------------------------------------- */

/* E2M1 value table, indexed by the 4-bit code: bit 3 = sign, bits 2..1 =
 * exponent (bias 1), bit 0 = mantissa; exponent 0 is subnormal (0 or 0.5).
 * [MXFP4 card], "Model and quantization": packed E2M1 FP4 weight values. */
static const double E2M1_TABLE[16] = {
    0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double oracle_e2m1(int code) { return E2M1_TABLE[code & 15]; }

/* E8M0 block scale: 2^(e-127); e = 255 encodes NaN.
 * [MXFP4 card], "Model and quantization": one E8M0 scale per 32 values. */
double oracle_e8m0(int e)
{
    e &= 255;
    if (e == 255) return NAN;
    return ldexp(1.0, e - 127);
}

/* OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN.  Used by the NVFP4 variant's per-16 scales. */
double oracle_e4m3fn(int c)
{
    c &= 255;
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    double v;
    if (E == 15 && m == 7) return NAN;
    if (E == 0) v = ldexp((double)m, -9);          /* m/8 * 2^-6 */
    else v = ldexp(8.0 + m, E - 10);                /* (1 + m/8) * 2^(E-7) */
    return s ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* BF16                                                                    */
/* ---------------------------------------------------------------------- */

static double round_half_even(double q)
{
    double f = floor(q), d = q - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Round an fp64 value once to BF16 (8 significant bits, fp32 exponent range,
 * subnormals kept), nearest-even; returns the BF16 bit pattern. */
uint16_t oracle_bf16_from_f64(double v)
{
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0 : 0x7FC0);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e;
    frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -126) E = -126;  /* below the normal range the step is fixed */
    double quantum = ldexp(1.0, E - 7);
    double r = round_half_even(a / quantum) * quantum;   /* both exact */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)r;      /* exact: r has at most 9 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

double oracle_f64_from_bf16(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

void oracle_bf16_round_array(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f64(in[i]);
}

/* ---------------------------------------------------------------------- */
/* Dequantisation                                                          */
/* ---------------------------------------------------------------------- */

static int group_of(int fmt) { return fmt == ORC_FMT_E4M3_G16 ? 16 : 32; }

static double scale_value(int fmt, uint8_t code)
{
    return fmt == ORC_FMT_E4M3_G16 ? oracle_e4m3fn(code) : oracle_e8m0(code);
}

/* Weight element (n, k) of a row-major [rows][cols] packed matrix: byte k/2
 * of row n holds element k in its low nibble when k is even, in its high
 * nibble when k is odd; the scale of (n, k) is scales[n][k / group]. */
static double weight_at(const uint8_t* nib, const uint8_t* sc, int cols,
                        int fmt, int n, int k)
{
    uint8_t byte = nib[(size_t)n * (cols / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    int G = group_of(fmt);
    return E2M1_TABLE[code] * scale_value(fmt, sc[(size_t)n * (cols / G) + k / G]);
}

/* Full dequantisation of one packed matrix to fp64 (E2M1 * block scale). */
int oracle_dequant(const uint8_t* nib, const uint8_t* sc, int rows, int cols,
                   int fmt, double* out)
{
    if (rows < 0 || cols <= 0 || cols % group_of(fmt) != 0) return -1;
    for (int n = 0; n < rows; ++n)
        for (int k = 0; k < cols; ++k)
            out[(size_t)n * cols + k] = weight_at(nib, sc, cols, fmt, n, k);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* GEMV, activation, combine                                               */
/* ---------------------------------------------------------------------- */

/* sum_k v[k] * W[n,k] * tscale, fp64, k ascending */
static double row_dot(const double* v, const uint8_t* nib, const uint8_t* sc,
                      int cols, int fmt, int n, double tscale)
{
    double acc = 0.0;
    for (int k = 0; k < cols; ++k) {
        double w = weight_at(nib, sc, cols, fmt, n, k) * tscale;  /* exact */
        acc += v[k] * w;
    }
    return acc;
}

/* SiLU(g) * u with one final rounding: silu(z) = z / (1 + e^-z). */
static double silu_mul(double g, double u) { return (g / (1.0 + exp(-g))) * u; }

/* Routing-weighted combine in slot order with sequential BF16 rounding.
 * [MXFP4 card], "Grouped top-4 expert execution": the fused combination keeps
 * the sequential BF16 multiply/add rounding of the per-expert engine.
 * y: [T][K][H] bf16, w: [T][K] bf16, residual: [T][H] bf16 or NULL. */
void oracle_combine(const uint16_t* y, const uint16_t* w, const uint16_t* residual,
                    uint16_t* out, int T, int K, int H)
{
    for (int t = 0; t < T; ++t)
        for (int m = 0; m < H; ++m) {
            uint16_t acc = 0;  /* +0 */
            for (int j = 0; j < K; ++j) {
                double p = oracle_f64_from_bf16(w[(size_t)t * K + j]) *
                           oracle_f64_from_bf16(y[((size_t)t * K + j) * H + m]);
                uint16_t pb = oracle_bf16_from_f64(p);
                acc = oracle_bf16_from_f64(oracle_f64_from_bf16(acc) +
                                           oracle_f64_from_bf16(pb));
            }
            if (residual)
                acc = oracle_bf16_from_f64(oracle_f64_from_bf16(residual[(size_t)t * H + m]) +
                                           oracle_f64_from_bf16(acc));
            out[(size_t)t * H + m] = acc;
        }
}

/* Weightless RMS pre-norm: u = bf16(x / sqrt(mean(x^2) + eps)). */
void oracle_prenorm(const uint16_t* x, uint16_t* u, int H, double eps)
{
    double ss = 0.0;
    for (int k = 0; k < H; ++k) {
        double v = oracle_f64_from_bf16(x[k]);
        ss += v * v;
    }
    double d = sqrt(ss / H + eps);
    for (int k = 0; k < H; ++k) u[k] = oracle_bf16_from_f64(oracle_f64_from_bf16(x[k]) / d);
}

/* Stable counting sort of the T*K (token, slot) pairs by expert id: the
 * batched path's grouping (pairs of one expert are contiguous, in token-major
 * order).  counts[E], offsets[E+1], perm[T*K] = t*K + j. */
int oracle_sort_pairs(const int32_t* ids, int T, int K, int E,
                      int32_t* counts, int32_t* offsets, int32_t* perm)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < T * K; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return -1;
        counts[ids[p]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!fill) return -2;
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int p = 0; p < T * K; ++p) perm[fill[ids[p]]++] = p;
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* 4-bit activations (W4A4)                                                */
/* ---------------------------------------------------------------------- */

/* MXFP4 quantisation of activations.  [NVFP4 card], "Why this quant", says
 * only that the W4A4 builds make the expert activations 4-bit; it gives no
 * format.  Reading: the weights' own format ([MXFP4 card], "Model and
 * quantization": E2M1 values, two per byte, one E8M0 scale per 32 values
 * along k), with the shared-scale rule and element conversion of the OCP
 * Microscaling (MX) Formats specification v1.0, section "Conversion":
 *   X   = 2^(floor(log2(max |v|)) - 2) per block of 32 (2 is the largest
 *         E2M1 exponent), the exponent clamped to -127..127; a block of zeros
 *         takes X = 2^-127 (E8M0 code 0);
 *   q_i = v_i / X rounded to E2M1, nearest with ties to the even code,
 *         magnitudes beyond 6 saturating to 6; the sign bit is the input's.
 * The quantised activation is q_i * X.  E2M1 keeps one mantissa bit, so the
 * step is 0.5 below 2, 1 in [2, 4) and 2 from 4 up.
 * v [rows][cols] bf16; codes [rows][cols/2] (low nibble = even k, as the
 * weights); scales [rows][cols/32] E8M0.  Returns -1 unless cols % 32 == 0. */
int oracle_quant_mxfp4(const uint16_t* v, int rows, int cols, uint8_t* codes, uint8_t* scales)
{
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return -1;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < cols / 32; ++b) {
            const uint16_t* blk = v + (size_t)r * cols + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(oracle_f64_from_bf16(blk[i])));
            int x = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);          /* amax in [2^(ex-1), 2^ex) */
                x = (ex - 1) - 2;
                if (x < -127) x = -127;
                if (x > 127) x = 127;
            }
            scales[(size_t)r * (cols / 32) + b] = (uint8_t)(x + 127);
            for (int i = 0; i < 32; ++i) {
                double val = oracle_f64_from_bf16(blk[i]);
                double a = ldexp(fabs(val), -x);                 /* exact */
                double step = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
                double q = round_half_even(a / step) * step;
                if (q > 6.0) q = 6.0;
                int code = 0;
                while (E2M1_TABLE[code] != q) ++code;            /* q is on the grid */
                if (signbit(val)) code |= 8;
                const int k = 32 * b + i;
                uint8_t* byte = codes + (size_t)r * (cols / 2) + k / 2;
                if (k & 1) *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                else *byte = (uint8_t)((*byte & 0xF0) | code);
            }
        }
    return 0;
}

/* The quantised values of one row as fp64: q_i * X (exact). */
static void quant_row_values(const uint16_t* v, int cols, double* out)
{
    uint8_t* c = (uint8_t*)calloc((size_t)cols / 2, 1);
    uint8_t* s = (uint8_t*)malloc((size_t)cols / 32);
    oracle_quant_mxfp4(v, 1, cols, c, s);
    for (int k = 0; k < cols; ++k) {
        int code = (k & 1) ? (c[k / 2] >> 4) : (c[k / 2] & 15);
        out[k] = E2M1_TABLE[code] * oracle_e8m0(s[k / 32]);
    }
    free(c);
    free(s);
}

/* ---------------------------------------------------------------------- */
/* The whole layer                                                         */
/* ---------------------------------------------------------------------- */

/*
 * x        [T][H] bf16        ids [T][K] int32     route_w [T][K] bf16
 * nib[e]   gate [I][H/2] | up [I][H/2] | down [H][I/2]   (host pointers)
 * scl[e]   gate [I][H/G] | up [I][H/G] | down [H][I/G]
 * tscales  [E][2] fp32 {gate/up, down} or NULL (then 1.0)
 * residual [T][H] bf16 or NULL
 * out      [T][H] bf16
 * dump_*   optional: u [T][H], g/v/h [T][K][I], y [T][K][H] (bf16)
 * Returns 0, or -1 on a bad argument.
 */
static int moe_forward_impl(int T, int H, int I, int E, int K, int fmt,
                            const uint16_t* x, const int32_t* ids, const uint16_t* route_w,
                            const uint8_t* const* nib, const uint8_t* const* scl,
                            const float* tscales, const uint16_t* residual,
                            int prenorm, double eps, uint16_t* out,
                            uint16_t* dump_u, uint16_t* dump_g, uint16_t* dump_v,
                            uint16_t* dump_h, uint16_t* dump_y, int nthreads, int a4)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0) return -1;
    if (fmt != ORC_FMT_E8M0_G32 && fmt != ORC_FMT_E4M3_G16) return -1;
    int G = group_of(fmt);
    if (H % G || I % G || H % 2 || I % 2) return -1;
    if (a4 && (fmt != ORC_FMT_E8M0_G32 || H % 32 || I % 32)) return -1;
    for (int p = 0; p < T * K; ++p)
        if (ids[p] < 0 || ids[p] >= E) return -1;
    /* the thread count applies to this call only (no process-wide setting) */
#ifdef _OPENMP
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    const int nth = 1;
    (void)nthreads;
#endif
    (void)nth;
    const size_t gate_n = 0, up_n = (size_t)I * H / 2, down_n = (size_t)I * H;  /* bytes */
    const size_t gate_s = 0, up_s = (size_t)I * H / G, down_s = 2 * (size_t)I * H / G;

    uint16_t* ub = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
    double* uv = (double*)malloc(sizeof(double) * (size_t)H);
    uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)K * I);
    double* hv = (double*)malloc(sizeof(double) * (size_t)K * I);
    uint16_t* yb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)K * H);
    if (!ub || !uv || !hb || !hv || !yb) {
        free(ub); free(uv); free(hb); free(hv); free(yb);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (size_t)t * H;
        if (prenorm) oracle_prenorm(xt, ub, H, eps);
        else memcpy(ub, xt, sizeof(uint16_t) * (size_t)H);
        if (a4) quant_row_values(ub, H, uv);
        else
            for (int k = 0; k < H; ++k) uv[k] = oracle_f64_from_bf16(ub[k]);
        if (dump_u) memcpy(dump_u + (size_t)t * H, ub, sizeof(uint16_t) * (size_t)H);

        /* gate, up, silu*up for every slot */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nth)
        for (int j = 0; j < K; ++j)
            for (int n = 0; n < I; ++n) {
                int e = ids[(size_t)t * K + j];
                double tg = tscales ? (double)tscales[2 * e] : 1.0;
                double g = row_dot(uv, nib[e] + gate_n, scl[e] + gate_s, H, fmt, n, tg);
                double v = row_dot(uv, nib[e] + up_n, scl[e] + up_s, H, fmt, n, tg);
                uint16_t gb = oracle_bf16_from_f64(g), vb = oracle_bf16_from_f64(v);
                uint16_t h = oracle_bf16_from_f64(
                    silu_mul(oracle_f64_from_bf16(gb), oracle_f64_from_bf16(vb)));
                hb[(size_t)j * I + n] = h;
                hv[(size_t)j * I + n] = oracle_f64_from_bf16(h);
                size_t d = ((size_t)t * K + j) * I + n;
                if (dump_g) dump_g[d] = gb;
                if (dump_v) dump_v[d] = vb;
                if (dump_h) dump_h[d] = h;
            }
        if (a4)
            for (int j = 0; j < K; ++j) quant_row_values(hb + (size_t)j * I, I, hv + (size_t)j * I);
        /* down */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nth)
        for (int j = 0; j < K; ++j)
            for (int m = 0; m < H; ++m) {
                int e = ids[(size_t)t * K + j];
                double td = tscales ? (double)tscales[2 * e + 1] : 1.0;
                double y = row_dot(hv + (size_t)j * I, nib[e] + down_n, scl[e] + down_s,
                                   I, fmt, m, td);
                yb[(size_t)j * H + m] = oracle_bf16_from_f64(y);
            }
        if (dump_y) memcpy(dump_y + (size_t)t * K * H, yb, sizeof(uint16_t) * (size_t)K * H);
        oracle_combine(yb, route_w + (size_t)t * K, residual ? residual + (size_t)t * H : NULL,
                       out + (size_t)t * H, 1, K, H);
    }
    free(ub); free(uv); free(hb); free(hv); free(yb);
    return 0;
}

int oracle_moe_forward(int T, int H, int I, int E, int K, int fmt,
                       const uint16_t* x, const int32_t* ids, const uint16_t* route_w,
                       const uint8_t* const* nib, const uint8_t* const* scl,
                       const float* tscales, const uint16_t* residual,
                       int prenorm, double eps, uint16_t* out,
                       uint16_t* dump_u, uint16_t* dump_g, uint16_t* dump_v,
                       uint16_t* dump_h, uint16_t* dump_y, int nthreads)
{
    return moe_forward_impl(T, H, I, E, K, fmt, x, ids, route_w, nib, scl, tscales, residual,
                            prenorm, eps, out, dump_u, dump_g, dump_v, dump_h, dump_y,
                            nthreads, 0);
}

/* The W4A4 layer: as oracle_moe_forward, with u and every h replaced by their
 * MXFP4 quantisation before the GEMV that reads them.  MXFP4 weights only
 * (the E8M0 block scale of the activations and the weights must agree in
 * kind for FP4 matrix hardware); returns -1 for the E4M3 format. */
int oracle_moe_forward_w4a4(int T, int H, int I, int E, int K, int fmt,
                            const uint16_t* x, const int32_t* ids, const uint16_t* route_w,
                            const uint8_t* const* nib, const uint8_t* const* scl,
                            const float* tscales, const uint16_t* residual,
                            int prenorm, double eps, uint16_t* out,
                            uint16_t* dump_u, uint16_t* dump_g, uint16_t* dump_v,
                            uint16_t* dump_h, uint16_t* dump_y, int nthreads)
{
    return moe_forward_impl(T, H, I, E, K, fmt, x, ids, route_w, nib, scl, tscales, residual,
                            prenorm, eps, out, dump_u, dump_g, dump_v, dump_h, dump_y,
                            nthreads, 1);
}

/* ---------------------------------------------------------------------- */
/* Router                                                                  */
/* ---------------------------------------------------------------------- */

/* The router of a fully GPU-resident layer ([MXFP4 card], "GPU routing
 * inside resident-layer graphs"): router projection, sigmoid scores, expert
 * bias where configured, dynamic top-k selection, routing coefficients.
 * Readings where the card is silent:
 *   u         = x[t], or the weightless RMS pre-norm of x[t] (as the layer)
 *   logit[e]  = sum_k u[k] * Wr[e][k]     (BF16 router rows [E][H], fp64, k ascending)
 *   s[e]      = 1 / (1 + exp(-logit[e]))
 *   c[e]      = s[e] + bias[e]             (bias FP32 [E]; 0 when not configured)
 *   slots     = the k experts of largest c, in descending c; equal c -> smaller e
 *   w[t][j]   = bf16( s[e_j] / sum_j' s[e_j'] )   (coefficients from the scores,
 *               normalised over the selected experts; the bias only selects)
 * logits_out (optional) receives logit[t][e]. */
int oracle_route(int T, int H, int E, int K, const uint16_t* x, const uint16_t* wr,
                 const float* bias, int prenorm, double eps, int32_t* ids, uint16_t* rw,
                 double* logits_out)
{
    if (K < 1 || K > E) return -1;
    uint16_t* u = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    double* c = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (size_t)t * H;
        if (prenorm) oracle_prenorm(xt, u, H, eps);
        else memcpy(u, xt, sizeof(uint16_t) * (size_t)H);
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int k = 0; k < H; ++k)
                acc += oracle_f64_from_bf16(u[k]) * oracle_f64_from_bf16(wr[(size_t)e * H + k]);
            if (logits_out) logits_out[(size_t)t * E + e] = acc;
            s[e] = 1.0 / (1.0 + exp(-acc));
            c[e] = s[e] + (bias ? (double)bias[e] : 0.0);
            taken[e] = 0;
        }
        double sum = 0.0;
        for (int j = 0; j < K; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || c[e] > c[best])) best = e;
            taken[best] = 1;
            ids[(size_t)t * K + j] = best;
            sum += s[best];
        }
        for (int j = 0; j < K; ++j)
            rw[(size_t)t * K + j] = oracle_bf16_from_f64(s[ids[(size_t)t * K + j]] / sum);
    }
    free(u); free(s); free(c); free(taken);
    return 0;
}

int oracle_threads_available(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Hybrid mode: the pinned RAM expert cache                               */
/* ---------------------------------------------------------------------- */

/* [MXFP4 card], "Bounded pinned RAM expert cache" and "Hybrid mode": CPU-backed
 * experts of a partially resident layer are served from a packed RAM cache of
 * contiguous expert triplets with LRU eviction under a memory limit; a miss
 * rebuilds the triplet from the checkpoint.  Only routed CPU experts are
 * requested.  Reading where the card is silent: one call requests its
 * distinct CPU-backed experts in the order of their first appearance in the
 * ids (token-major, slot order); the cache holds `capacity` triplets.
 * Plain definition: a list ordered by last use; a request for a key in the
 * list is a hit and moves it to the front, any other request is a miss that
 * inserts the key at the front and, when the list is longer than capacity,
 * drops the key at the back.  keys[n] -> hit[n] (1 = hit).  Returns the
 * number of hits, or -1 on a bad argument. */
int oracle_lru(const int64_t* keys, int n, int capacity, uint8_t* hit)
{
    if (n < 0 || capacity < 1) return -1;
    int64_t* list = (int64_t*)malloc(sizeof(int64_t) * (size_t)(capacity + 1));
    if (!list) return -2;
    int len = 0, hits = 0;
    for (int i = 0; i < n; ++i) {
        int pos = -1;
        for (int j = 0; j < len; ++j)
            if (list[j] == keys[i]) { pos = j; break; }
        hit[i] = pos >= 0;
        if (pos >= 0) ++hits;
        else pos = len++;                       /* a new entry, at the back for now */
        for (int j = pos; j > 0; --j) list[j] = list[j - 1];
        list[0] = keys[i];                      /* most recently used first */
        if (len > capacity) --len;              /* the least recently used leaves */
    }
    free(list);
    return hits;
}
