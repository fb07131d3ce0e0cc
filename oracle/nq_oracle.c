/*
 * nq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of group-wise affine
 * quantization and of the quantized matrix products built on it.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it;
 * the GPU library never links, includes or calls it, and it shares no code
 * with the GPU library.
 *
 * Source: "Quantization" page of the nuvec documentation
 * (hupe1980.github.io/nuvec/docs/quantization/):
 *   - section "Affine": every row is cut into groups of group_size values
 *     (32, 64 or 128); each group keeps one scale and one bias; each value
 *     becomes a `bits`-bit integer code packed into uint32 words, and the
 *     weight is approximately scale * code + bias;
 *   - section "Affine", example: `x.quantized_matmul(&q, true)` is x times the
 *     transposed weights, `q.dequantize(None)` gives the approximate weights;
 *   - section "Mixture of experts": gather_qmm multiplies each row by the
 *     weights of the expert chosen for that row.
 * The nuvec API index (docs.rs/nuvec, struct `Quantized`) adds that scales
 * are kept in the weights' dtype.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the bias of a group is its minimum and the scale is (max - min) over
 *     the number of steps 2^bits - 1 (min/max affine), computed in fp32;
 *   - scale and bias are rounded to the storage dtype first, and codes are
 *     the nearest level with respect to the STORED scale and bias;
 *   - codes round half to even (rintf) and are clamped to [0, 2^bits - 1];
 *   - a group whose stored scale is zero gets all-zero codes;
 *   - -0 is canonicalised to +0 (x + 0.0f) for min, max and scale;
 *   - codes are laid out as one little-endian bit stream per row, element k
 *     occupying stream bits [k*bits, (k+1)*bits), stream bit i being bit
 *     (i mod 32) of word i/32 (LSB first);
 *   - the stand-alone dequantize contract is one fp32 fused multiply-add
 *     fmaf(scale, code, bias) rounded to nearest-even in the output dtype;
 *   - products use the exact-in-fp64 dequantized weight scale*code + bias
 *     and accumulate in fp64 in natural k order.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 * On x86-64 float arithmetic is SSE single precision, so every fp32 step
 * below rounds exactly once, to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

enum { OR_F32 = 0, OR_BF16 = 1 };

/* ---- storage formats ---------------------------------------------------- */

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;   /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* The value a bf16 bit pattern stands for, in double, with the pattern just
 * above the largest finite one (0x7F80 after a carry) read as 2^128 so that
 * the distance test below also decides overflow. */
static double bf16_magnitude(uint16_t h)
{
    if ((h & 0x7FFFu) == 0x7F80u) return ldexp(1.0, 128);
    return fabs((double)bf16_to_f32(h));
}

/* Round an fp32 value to the nearest bf16 value, ties to the even pattern
 * (IEEE round-to-nearest-even).  Written as its definition: take the two
 * bf16 neighbours of |f| and keep the closer one. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);   /* quiet NaN */
    uint16_t down = (uint16_t)(u >> 16);           /* toward zero */
    if ((u & 0xFFFFu) == 0) return down;           /* already a bf16 value */
    uint16_t up = (uint16_t)(down + 1);            /* away from zero */
    double a = fabs((double)f);
    double d_down = a - bf16_magnitude(down);
    double d_up = bf16_magnitude(up) - a;
    if (d_down < d_up) return down;
    if (d_up < d_down) return up;
    return (down & 1u) ? up : down;                /* tie: even pattern */
}

static float load_f(const void *p, int dt, int64_t i)
{
    if (dt == OR_F32) return ((const float *)p)[i];
    return bf16_to_f32(((const uint16_t *)p)[i]);
}

/* Store v in dtype dt and return the value actually stored. */
static float store_f(void *p, int dt, int64_t i, float v)
{
    if (dt == OR_F32) {
        ((float *)p)[i] = v;
        return v;
    }
    uint16_t h = f32_to_bf16(v);
    ((uint16_t *)p)[i] = h;
    return bf16_to_f32(h);
}

/* ---- code stream -------------------------------------------------------- */

/* Element k of a row is stream bits [k*bits, (k+1)*bits). */
static uint32_t get_code(const uint32_t *row, int64_t k, int bits)
{
    uint32_t q = 0;
    for (int j = 0; j < bits; ++j) {
        int64_t bit = k * bits + j;
        q |= ((row[bit / 32] >> (bit % 32)) & 1u) << j;
    }
    return q;
}

static void put_code(uint32_t *row, int64_t k, int bits, uint32_t q)
{
    for (int j = 0; j < bits; ++j) {
        int64_t bit = k * bits + j;
        if ((q >> j) & 1u) row[bit / 32] |= 1u << (bit % 32);
    }
}

int oracle_bits_supported(int bits)
{
    return bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 5 ||
           bits == 6 || bits == 8;
}

int oracle_group_supported(int gs) { return gs == 32 || gs == 64 || gs == 128; }

/* Threads the OpenMP loops below run on. */
int oracle_threads(void) { return omp_get_max_threads(); }

void oracle_bf16_round(const float *in, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = f32_to_bf16(in[i]);
}

/* ---- quantize ------------------------------------------------------------ */

/* w: [n, k] in w_dt.  codes: [n, k*bits/32] uint32.  scales, biases: [n, k/gs]
 * in w_dt.  Returns 0, or -1 on an unsupported (gs, bits) or k % gs != 0. */
int oracle_quantize(const void *w, int w_dt, int64_t n, int64_t k, int gs, int bits,
                    uint32_t *codes, void *scales, void *biases)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
    const float top = (float)((1u << bits) - 1u);   /* number of steps */
    memset(codes, 0, (size_t)(n * P) * sizeof(uint32_t));

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t k0 = g * gs;
            float mn = INFINITY, mx = -INFINITY;
            for (int j = 0; j < gs; ++j) {
                float v = load_f(w, w_dt, r * k + k0 + j);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            mn = mn + 0.0f;                     /* -0 -> +0 */
            mx = mx + 0.0f;
            float range = mx - mn;
            float scale = range / top;          /* correctly rounded fp32 divide */
            scale = scale + 0.0f;
            float bias = mn;
            float s = store_f(scales, w_dt, r * G + g, scale);
            float b = store_f(biases, w_dt, r * G + g, bias);
            for (int j = 0; j < gs; ++j) {
                float v = load_f(w, w_dt, r * k + k0 + j);
                uint32_t q = 0;
                if (s != 0.0f) {
                    float t = (v - b) / s;      /* two fp32 roundings, no fma */
                    t = rintf(t);               /* nearest, ties to even */
                    t = fminf(fmaxf(t, 0.0f), top);
                    q = (uint32_t)t;
                }
                put_code(codes + r * P, k0 + j, bits, q);
            }
        }
    }
    return 0;
}

/* ---- dequantize ----------------------------------------------------------- */

/* The stand-alone dequantize contract: fmaf(scale, code, bias), then rounded
 * to out_dt.  out: [n, k]. */
int oracle_dequantize(const uint32_t *codes, const void *scales, const void *biases, int sb_dt,
                      int64_t n, int64_t k, int gs, int bits, void *out, int out_dt)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t kk = 0; kk < k; ++kk) {
            float s = load_f(scales, sb_dt, r * G + kk / gs);
            float b = load_f(biases, sb_dt, r * G + kk / gs);
            float q = (float)get_code(codes + r * P, kk, bits);
            store_f(out, out_dt, r * k + kk, fmaf(s, q, b));
        }
    return 0;
}

/* The dequantized weight in fp64: scale*code is exact in double, the bias
 * addition rounds once.  out: [n, k] double. */
int oracle_dequantize_f64(const uint32_t *codes, const void *scales, const void *biases,
                          int sb_dt, int64_t n, int64_t k, int gs, int bits, double *out)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t kk = 0; kk < k; ++kk) {
            double s = load_f(scales, sb_dt, r * G + kk / gs);
            double b = load_f(biases, sb_dt, r * G + kk / gs);
            double q = (double)get_code(codes + r * P, kk, bits);
            out[r * k + kk] = s * q + b;
        }
    return 0;
}

/* ---- products ------------------------------------------------------------- */

static void dequant_row_f64(const uint32_t *codes, const void *scales, const void *biases,
                            int sb_dt, int64_t r, int64_t k, int gs, int bits, double *row)
{
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
    for (int64_t kk = 0; kk < k; ++kk) {
        double s = load_f(scales, sb_dt, r * G + kk / gs);
        double b = load_f(biases, sb_dt, r * G + kk / gs);
        row[kk] = s * (double)get_code(codes + r * P, kk, bits) + b;
    }
}

/* y[m, n] = sum_k x[m, k] * w_hat[n, k]  (x times the transposed weights),
 * fp64, natural k order.  x: [m, k] in x_dt; y: [m, n] double. */
int oracle_qmm_f64(const void *x, int x_dt, int64_t m, int64_t k, const uint32_t *codes,
                   const void *scales, const void *biases, int sb_dt, int64_t n, int gs,
                   int bits, double *y)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *wr = (double *)malloc((size_t)k * sizeof(double));
        if (!wr) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t c = 0; c < n; ++c) {
            if (!wr) continue;
            dequant_row_f64(codes, scales, biases, sb_dt, c, k, gs, bits, wr);
            for (int64_t r = 0; r < m; ++r) {
                double acc = 0.0;
                for (int64_t kk = 0; kk < k; ++kk)
                    acc += (double)load_f(x, x_dt, r * k + kk) * wr[kk];
                y[r * n + c] = acc;
            }
        }
        free(wr);
    }
    return failed ? -2 : 0;
}

/* The same product at chosen output positions only: out[i] = y[ms[i], ns[i]]. */
int oracle_qmm_sample_f64(const void *x, int x_dt, int64_t k, const uint32_t *codes,
                          const void *scales, const void *biases, int sb_dt, int gs, int bits,
                          const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double s = load_f(scales, sb_dt, ns[i] * G + kk / gs);
            double b = load_f(biases, sb_dt, ns[i] * G + kk / gs);
            double wv = s * (double)get_code(codes + ns[i] * P, kk, bits) + b;
            acc += (double)load_f(x, x_dt, ms[i] * k + kk) * wv;
        }
        out[i] = acc;
    }
    return 0;
}

/* Mixture of experts: x [rows, l, k], codes [e, n, k*bits/32], scales and
 * biases [e, n, k/gs], idx [rows].  y[r, j, :] = x[r, j, :] times the
 * transposed weights of expert idx[r]; a row whose id is >= e is all zeros.
 * y: [rows, l, n] double. */
int oracle_gather_qmm_f64(const void *x, int x_dt, int64_t rows, int64_t l, int64_t k,
                          const uint32_t *codes, const void *scales, const void *biases,
                          int sb_dt, int64_t e, int64_t n, int gs, int bits,
                          const uint32_t *idx, double *y)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const uint32_t ex = idx[r];
        for (int64_t j = 0; j < l; ++j)
            for (int64_t c = 0; c < n; ++c) {
                double acc = 0.0;
                if ((int64_t)ex < e) {
                    const int64_t wr = (int64_t)ex * n + c;   /* row of the stacked weights */
                    for (int64_t kk = 0; kk < k; ++kk) {
                        double s = load_f(scales, sb_dt, wr * G + kk / gs);
                        double b = load_f(biases, sb_dt, wr * G + kk / gs);
                        double wv = s * (double)get_code(codes + wr * P, kk, bits) + b;
                        acc += (double)load_f(x, x_dt, (r * l + j) * k + kk) * wv;
                    }
                }
                y[(r * l + j) * n + c] = acc;
            }
    }
    return 0;
}

/* ---- products with the untransposed weights, and derivatives ------------- */

/* y[r, c] = sum_i x[r, i] * w_hat[i, c]: x times the weights as stored, the
 * `transpose = false` product ("Quantization" page, "Affine" example's
 * quantized_matmul flag).  The quantized matrix has rows i (ni of them) and
 * columns c (nc), grouped along c.  fp64, natural i order.  y: [m, nc]. */
int oracle_qmm_nt_f64(const void *x, int x_dt, int64_t m, int64_t ni, const uint32_t *codes,
                      const void *scales, const void *biases, int sb_dt, int64_t nc, int gs,
                      int bits, double *y)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || nc % gs != 0) return -1;
    const int64_t G = nc / gs;
    const int64_t P = nc * bits / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < nc; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < ni; ++i) {
                double s = load_f(scales, sb_dt, i * G + c / gs);
                double b = load_f(biases, sb_dt, i * G + c / gs);
                double wv = s * (double)get_code(codes + i * P, c, bits) + b;
                acc += (double)load_f(x, x_dt, r * ni + i) * wv;
            }
            y[r * nc + c] = acc;
        }
    return 0;
}

/* Derivatives of L = sum_{r,c} dy[r, c] * y[r, c], y = x times the
 * transposed weights (w_hat[c, kk] = s[c, g] * q[c, kk] + b[c, g], g = kk / gs),
 * with respect to the scales and biases ("Quantization" page, "Training
 * through quantized weights"):
 *   ds[c, g] = sum_r dy[r, c] * sum_{kk in g} x[r, kk] * q[c, kk]
 *   db[c, g] = sum_r dy[r, c] * sum_{kk in g} x[r, kk]
 * fp64, r outer and kk inner in natural order.  x: [m, k]; dy: [m, n];
 * codes: [n, k*bits/32]; ds, db: [n, k/gs] double.  (The derivative for x is
 * dy times the weights as stored: oracle_qmm_nt_f64 with ni = n, nc = k.) */
int oracle_qmm_grad_sb_f64(const void *x, int x_dt, const void *dy, int dy_dt, int64_t m, int64_t k,
                           const uint32_t *codes, int64_t n, int gs, int bits, double *ds, double *db)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < n; ++c)
        for (int64_t g = 0; g < G; ++g) {
            double as = 0.0, ab = 0.0;
            for (int64_t r = 0; r < m; ++r) {
                const double d = load_f(dy, dy_dt, r * n + c);
                double xq = 0.0, xs = 0.0;
                for (int64_t kk = g * gs; kk < (g + 1) * gs; ++kk) {
                    const double xv = load_f(x, x_dt, r * k + kk);
                    xq += xv * (double)get_code(codes + c * P, kk, bits);
                    xs += xv;
                }
                as += d * xq;
                ab += d * xs;
            }
            ds[c * G + g] = as;
            db[c * G + g] = ab;
        }
    return 0;
}

/* gather_qmm with both index arrays ("Mixture of experts": the call takes an
 * optional left index and the expert index).  x: [b, l, k]; lhs [rows]
 * selects the x item of each output row (null: item r), rhs [rows] the
 * expert.  y[r, j, :] = x[lhs[r], j, :] times the transposed weights of
 * expert rhs[r]; zero rows for rhs >= e (lhs >= b is outside the contract of
 * the callers and also gives a zero row here).  y: [rows, l, n] double. */
int oracle_gather_qmm_lhs_f64(const void *x, int x_dt, int64_t b, int64_t rows, int64_t l, int64_t k,
                              const uint32_t *codes, const void *scales, const void *biases,
                              int sb_dt, int64_t e, int64_t n, int gs, int bits,
                              const uint32_t *lhs, const uint32_t *rhs, double *y)
{
    if (!oracle_bits_supported(bits) || !oracle_group_supported(gs) || k % gs != 0) return -1;
    const int64_t G = k / gs;
    const int64_t P = k * bits / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t xi = lhs ? (int64_t)lhs[r] : r;
        const uint32_t ex = rhs[r];
        for (int64_t j = 0; j < l; ++j)
            for (int64_t c = 0; c < n; ++c) {
                double acc = 0.0;
                if ((int64_t)ex < e && xi < b) {
                    const int64_t wr = (int64_t)ex * n + c;
                    for (int64_t kk = 0; kk < k; ++kk) {
                        double s = load_f(scales, sb_dt, wr * G + kk / gs);
                        double bb = load_f(biases, sb_dt, wr * G + kk / gs);
                        double wv = s * (double)get_code(codes + wr * P, kk, bits) + bb;
                        acc += (double)load_f(x, x_dt, (xi * l + j) * k + kk) * wv;
                    }
                }
                y[(r * l + j) * n + c] = acc;
            }
    }
    return 0;
}
