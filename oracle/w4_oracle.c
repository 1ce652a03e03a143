/*
 * CPU oracle for the W4A16 decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may call
 * this code.  It shares nothing with the GPU library (no headers, helpers or
 * tables) and must never be used as a fallback for it.
 *
 * What is computed follows these passages:
 *   [P1-S1]  dev.to "Gemma 4 on a 4 GB GPU in Plain PyTorch", section "Step 1 -
 *            Load Google's QAT Weights Without Unpacking Them": W4A16 means 4-bit
 *            weight codes in groups of 32 with 16-bit activations; each group's
 *            step is stored in bf16.
 *   [P1-S2]  same page, "Step 2 - Keep the Vocabulary Tables in 4-Bit": the
 *            vocabulary table is stored as 4-bit codes plus a per-group step and
 *            one copy serves both the input lookup and the output layer.
 *   [P1-S3]  same page, "Step 3 - Multiply Straight From the Packed Weights":
 *            decoding multiplies one vector by every weight matrix, reading the
 *            packed words and never writing a 16-bit copy; a code becomes a float
 *            by OR-ing it into the bits of 2^23 and subtracting 2^23 + 8, i.e. the
 *            stored code c stands for the integer c - 8.
 *   [P3]     anyesh.me "Running a 26B MoE on an 8 GB Jetson by streaming experts
 *            from SSD", section "Streaming without touching a single GPU kernel":
 *            the expert matmul addresses expert id as base + id * stride, a pool
 *            of slots is addressed through slot ids, and every other per-expert
 *            tensor keeps the real expert id.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - nibble j (bits 4j..4j+3) of packed word w of a row is column 8w+j;
 *   - a matrix is [N_out][K_in]; steps are a separate row-major bf16[N][K/32];
 *   - y is produced in full precision here (fp64); the GPU stores fp32;
 *   - every narrowing cast rounds to nearest, ties to even.
 *
 * Everything is plain scalar code in ascending index order with fp64
 * accumulation.  No blocking, no reordering.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define W4O_F16 0
#define W4O_BF16 1

/* ---- 16-bit float formats, decoded from their IEEE definitions ---------- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double w4o_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double w4o_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133); /* subnormal: f * 2^-126 * 2^-7 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
    }
    return sign ? -v : v;
}

double w4o_act_to_f64(uint16_t bits, int dtype) {
    return dtype == W4O_F16 ? w4o_f16_to_f64(bits) : w4o_bf16_to_f64(bits);
}

/*
 * Round a double to a binary format with `prec` significant bits, smallest
 * normal exponent `emin` and largest finite value `maxfin`, nearest-even.
 * Returns the rounded value as a double (exact).
 */
static double round_to_format(double a, int prec, int emin, double maxfin, double *out) {
    /* a > 0, finite */
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int ex = e2 - 1;
    if (ex < emin) ex = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, ex - (prec - 1));
    double q = nearbyint(a / quantum); /* default rounding mode: ties to even */
    double r = q * quantum;
    /* overflow: values at or beyond maxfin + half an ulp of maxfin become inf */
    if (r > maxfin) r = INFINITY;
    *out = r;
    return r;
}

uint16_t w4o_f64_to_f16_rne(double v) {
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r;
    round_to_format(a, 11, -14, 65504.0, &r);
    if (isinf(r)) return sign | 0x7C00;
    if (r < ldexp(1.0, -14)) /* subnormal (or rounded to zero) */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    int e2;
    frexp(r, &e2);
    int ex = e2 - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, ex - 10) - 1024.0);
    return sign | (uint16_t)((ex + 15) << 10) | frac;
}

uint16_t w4o_f64_to_bf16_rne(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r;
    double maxfin = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    round_to_format(a, 8, -126, maxfin, &r);
    if (isinf(r)) return sign | 0x7F80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    int e2;
    frexp(r, &e2);
    int ex = e2 - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, ex - 7) - 128.0);
    return sign | (uint16_t)((ex + 127) << 7) | frac;
}

uint16_t w4o_f64_to_act_rne(double v, int dtype) {
    return dtype == W4O_F16 ? w4o_f64_to_f16_rne(v) : w4o_f64_to_bf16_rne(v);
}

/* ---- the packed format [P1-S1], [P1-S3] ----------------------------------- */

/* Code of weight (n, k): nibble k%8 of word k/8 of row n (low nibble first). */
int w4o_code(const uint32_t *codes, int64_t K, int64_t n, int64_t k) {
    uint32_t word = codes[n * (K / 8) + k / 8];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

/* Step of weight (n, k): the bf16 step of group k/32 of row n. */
double w4o_step(const uint16_t *steps, int64_t K, int64_t n, int64_t k) {
    return w4o_bf16_to_f64(steps[n * (K / 32) + k / 32]);
}

/* Dequantised weight: (c - 8) * step. */
double w4o_weight(const uint32_t *codes, const uint16_t *steps, int64_t K, int64_t n, int64_t k) {
    return (double)(w4o_code(codes, K, n, k) - 8) * w4o_step(steps, K, n, k);
}

/* Dense dequantised matrix W[N][K] (fp64). */
void w4o_dequant(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, double *W) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = w4o_weight(codes, steps, K, n, k);
}

/*
 * Matrix-vector product of one packed matrix with one activation vector
 * [P1-S3]: y[n] = sum_k w(n,k) * x[k], ascending k, fp64.  Alongside it
 * a[n] = sum_k |w(n,k) * x[k]| (the scale of the error bound).
 * Rows [n0, n1) only, so that large matrices can be sampled.
 */
void w4o_gemv_rows(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K,
                   const uint16_t *x, int xdtype, int64_t n0, int64_t n1, double *y, double *a) {
    (void)N;
    for (int64_t n = n0; n < n1; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = w4o_weight(codes, steps, K, n, k) * w4o_act_to_f64(x[k], xdtype);
            acc += p;
            mag += fabs(p);
        }
        y[n - n0] = acc;
        if (a) a[n - n0] = mag;
    }
}

void w4o_gemv(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K,
              const uint16_t *x, int xdtype, double *y, double *a) {
    w4o_gemv_rows(codes, steps, N, K, x, xdtype, 0, N, y, a);
}

/* Multi-threaded variant (rows split across threads; each row unchanged). */
void w4o_gemv_omp(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K,
                  const uint16_t *x, int xdtype, double *y, double *a) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        w4o_gemv_rows(codes, steps, N, K, x, xdtype, n, n + 1, y + n, a ? a + n : 0);
}

/*
 * The same product on an input given exactly as fp64 values (rows n0..n1-1),
 * with the bound's sum of |w x|: the decode chain's input x = u / r, the
 * previous output's leading entries divided by their RMS (the chaining step of
 * the decode sweep), enters the product exactly, not as a 16-bit vector.
 */
void w4o_gemv_x64_rows(const uint32_t *codes, const uint16_t *steps, int64_t K, const double *x,
                       int64_t n0, int64_t n1, double *y, double *a) {
    for (int64_t n = n0; n < n1; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = w4o_weight(codes, steps, K, n, k) * x[k];
            acc += p;
            mag += fabs(p);
        }
        y[n - n0] = acc;
        a[n - n0] = mag;
    }
}

int w4o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Small-M product: every activation row m gets the matrix-vector product
 * above.  X is [M][ldx] (row m starts at X + m*ldx); Y and A are [M][N].
 */
void w4o_gemm(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K,
              const uint16_t *X, int xdtype, int64_t M, int64_t ldx, double *Y, double *A) {
    for (int64_t m = 0; m < M; ++m)
        w4o_gemv_rows(codes, steps, N, K, X + m * ldx, xdtype, 0, N, Y + m * N, A ? A + m * N : 0);
}

/*
 * Row gather from a 4-bit table [P1-S2]: out[i][k] = bf16_RNE((c - 8) * step)
 * of row ids[i].  The product is exact in double, so rounding once to bf16 is
 * the single rounding.  Returns the number of ids outside [0, V) (their rows
 * are left untouched).
 */
int w4o_gather(const uint32_t *codes, const uint16_t *steps, int64_t V, int64_t K,
               const int32_t *ids, int64_t n, uint16_t *out) {
    int bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = ids[i];
        if (r < 0 || r >= V) { ++bad; continue; }
        for (int64_t k = 0; k < K; ++k)
            out[i * K + k] = w4o_f64_to_bf16_rne(w4o_weight(codes, steps, K, r, k));
    }
    return bad;
}

/*
 * Expert-indexed product [P3]: for token t and choice j, expert e = ids[t][j]
 * (a real expert id).  The weights of the expert sit at
 *     codes_base + a * stride_codes,  steps_base + a * stride_steps
 * where a = e (direct addressing) or a = slot_of[e] (pool addressing).
 * The input row is X[t] (x_per_pair = 0) or X[t*topk + j] (x_per_pair = 1),
 * each row ldx elements apart.  The optional per-expert output scale
 * row_scale[e][n] is indexed by the REAL id e in both addressing modes.
 *
 * Without route weights: Y[(t*topk + j)][n] = (W_a x)[n] * row_scale[e][n],
 *                        A the matching sum of |products| * |row_scale|.
 * With route weights r[t][j]: Y[t][n] = sum over j = 0..topk-1, ascending, of
 *                        r[t][j] * (that per-choice value); A likewise with |r|.
 * Returns -1 if an id or slot is out of range, else 0.
 */
int w4o_moe(const uint32_t *codes_base, const uint16_t *steps_base,
            int64_t stride_codes, int64_t stride_steps, int64_t N, int64_t K,
            const uint16_t *X, int xdtype, int x_per_pair, int64_t ldx,
            const int32_t *ids, int64_t T, int64_t topk,
            const int32_t *slot_of, int64_t n_experts, int64_t n_slots,
            const float *row_scale, const float *route_w, double *Y, double *A) {
    for (int64_t t = 0; t < T; ++t) {
        if (route_w) {
            for (int64_t n = 0; n < N; ++n) { Y[t * N + n] = 0.0; if (A) A[t * N + n] = 0.0; }
        }
        for (int64_t j = 0; j < topk; ++j) {
            int64_t e = ids[t * topk + j];
            if (e < 0 || e >= n_experts) return -1;
            int64_t a = e;
            if (slot_of) {
                a = slot_of[e];
                if (a < 0 || a >= n_slots) return -1;
            }
            const uint32_t *cw = codes_base + a * stride_codes;
            const uint16_t *sw = steps_base + a * stride_steps;
            const uint16_t *xr = X + (x_per_pair ? (t * topk + j) : t) * ldx;
            for (int64_t n = 0; n < N; ++n) {
                double v, m;
                w4o_gemv_rows(cw, sw, N, K, xr, xdtype, n, n + 1, &v, &m);
                if (row_scale) {
                    double s = (double)row_scale[e * N + n];
                    v *= s;
                    m *= fabs(s);
                }
                if (route_w) {
                    double r = (double)route_w[t * topk + j];
                    Y[t * N + n] += r * v;
                    if (A) A[t * N + n] += fabs(r) * m;
                } else {
                    Y[(t * topk + j) * N + n] = v;
                    if (A) A[(t * topk + j) * N + n] = m;
                }
            }
        }
    }
    return 0;
}

/*
 * Renormalisation between layers: take the leading K entries u of an output v,
 * r = sqrt(mean(u^2)) in fp64, next input = RNE(u / r) in the activation dtype.
 * A zero vector (r == 0) gives zeros.
 */
void w4o_rms_renorm(const float *v, int64_t K, int out_dtype, uint16_t *out) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) ss += (double)v[k] * (double)v[k];
    double r = sqrt(ss / (double)K);
    for (int64_t k = 0; k < K; ++k)
        out[k] = w4o_f64_to_act_rne(r > 0.0 ? (double)v[k] / r : 0.0, out_dtype);
}

/*
 * Grid packing of a 16-bit table [P1-S2] (the conversion behind the 4-bit
 * tables).  The page reports that the 16-bit tables were trained onto a 4-bit
 * grid -- every group of 32 holds at most 16 distinct values -- and that the
 * 4-bit tables hold codes with each group's step recovered from that grid;
 * nearly every stored value then equals its 16-bit source, and the rest are
 * off by a small fraction of a step.  How the step is recovered is not on the
 * page.  Reading taken, per group of 32 values v (bf16, finite):
 *   an = the largest magnitude among negative values (0 if none),
 *   ap = the largest positive value (0 if none);
 *   all zero: step 0 and code 8 everywhere.
 *   Otherwise the step is the grid's own: the largest bf16 value s > 0 for
 *   which every v is m * s with m an integer in [-8, 7].  Such an s puts the
 *   negative extreme -an at some level -j, j = 1..8 (or, with no negative
 *   value, ap at a level i = 1..7), so the candidates are an / j (ap / i) in
 *   that order, largest first, and each counts only if it is a bf16 value.
 *   When no candidate fits (values not on any such grid), the step comes from
 *   the extreme: s = an / 8 if an > ap (the negative extreme at code 0), else
 *   ap / 7 (the positive extreme at code 15), rounded to bf16 (ties to even).
 *   code = clamp(rint(v / s) + 8, 0, 15), with the exact quotient v / s and
 *   rint rounding halves to even.
 * The quotient is taken in fp64: v and s carry 8 significant bits each, so a
 * quotient that is not a half-integer lies at least 2^-12 of its size away
 * from one, far beyond fp64's rounding, and rint decides as on the exact
 * value.  On exact grid values this returns every value exactly (the codes of
 * the coarsest such grid); elsewhere each value in the grid's range is within
 * half a step.
 */
static double w4o_bf16_round(double x) { return w4o_bf16_to_f64(w4o_f64_to_bf16_rne(x)); }

/* every v[k] equal to m * s with m an integer in [-8, 7] */
static int w4o_on_grid(const double *v, double s) {
    for (int k = 0; k < 32; ++k) {
        const double m = v[k] / s;
        if (m != floor(m) || m < -8.0 || m > 7.0) return 0;
    }
    return 1;
}

void w4o_grid_to_codes(const uint16_t *table, int64_t N, int64_t K, uint32_t *codes,
                       uint16_t *steps) {
    const int64_t G = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            double v[32];
            double an = 0.0, ap = 0.0;
            for (int k = 0; k < 32; ++k) {
                v[k] = w4o_bf16_to_f64(table[n * K + g * 32 + k]);
                if (-v[k] > an) an = -v[k];
                if (v[k] > ap) ap = v[k];
            }
            double step = 0.0;
            if (an > 0.0 || ap > 0.0) {
                const double e = an > 0.0 ? an : ap;
                const int jmax = an > 0.0 ? 8 : 7;
                int found = 0;
                for (int j = 1; j <= jmax && !found; ++j) {
                    const double s = e / j;
                    if (w4o_bf16_round(s) != s || s * j != e) continue;
                    if (w4o_on_grid(v, s)) {
                        step = s;
                        found = 1;
                    }
                }
                if (!found) step = w4o_bf16_round(an > ap ? an / 8.0 : ap / 7.0);
            }
            steps[n * G + g] = w4o_f64_to_bf16_rne(step);
            for (int w = 0; w < 4; ++w) {
                uint32_t word = 0;
                for (int j = 0; j < 8; ++j) {
                    int c = 8;
                    if (step != 0.0) {
                        double q = nearbyint(v[8 * w + j] / step) + 8.0;
                        q = q < 0.0 ? 0.0 : (q > 15.0 ? 15.0 : q);
                        c = (int)q;
                    }
                    word |= (uint32_t)c << (4 * j);
                }
                codes[n * (K / 8) + g * 4 + w] = word;
            }
        }
    }
}
