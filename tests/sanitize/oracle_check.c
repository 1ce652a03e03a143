/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * entry point on small seeded inputs, including the special values and edge
 * shapes the pins use (zero rows, NaN/inf/subnormal activations, out-of-range
 * ids, all-zero and single-level groups for grid packing). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double w4o_f16_to_f64(uint16_t h);
double w4o_bf16_to_f64(uint16_t b);
uint16_t w4o_f64_to_f16_rne(double v);
uint16_t w4o_f64_to_bf16_rne(double v);
void w4o_dequant(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, double *W);
void w4o_gemv_rows(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, const uint16_t *x,
                   int xdtype, int64_t n0, int64_t n1, double *y, double *a);
void w4o_gemv(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, const uint16_t *x, int xdtype,
              double *y, double *a);
void w4o_gemv_omp(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, const uint16_t *x,
                  int xdtype, double *y, double *a);
void w4o_gemv_x64_rows(const uint32_t *codes, const uint16_t *steps, int64_t K, const double *x, int64_t n0,
                       int64_t n1, double *y, double *a);
void w4o_gemm(const uint32_t *codes, const uint16_t *steps, int64_t N, int64_t K, const uint16_t *X, int xdtype,
              int64_t M, int64_t ldx, double *Y, double *A);
int w4o_gather(const uint32_t *codes, const uint16_t *steps, int64_t V, int64_t K, const int32_t *ids, int64_t n,
               uint16_t *out);
int w4o_moe(const uint32_t *codes_base, const uint16_t *steps_base, int64_t stride_codes, int64_t stride_steps,
            int64_t N, int64_t K, const uint16_t *X, int xdtype, int x_per_pair, int64_t ldx, const int32_t *ids,
            int64_t T, int64_t topk, const int32_t *slot_of, int64_t n_experts, int64_t n_slots,
            const float *row_scale, const float *route_w, double *Y, double *A);
void w4o_rms_renorm(const float *v, int64_t K, int out_dtype, uint16_t *out);
void w4o_grid_to_codes(const uint16_t *table, int64_t N, int64_t K, uint32_t *codes, uint16_t *steps);

static uint64_t g_state = 88172645463325252ull;
static uint32_t rnd(void) {
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)g_state;
}

int main(void) {
    enum { N = 24, K = 96, E = 6, T = 3, TOPK = 2 };
    uint32_t *codes = malloc(sizeof(uint32_t) * E * N * K / 8);
    uint16_t *steps = malloc(sizeof(uint16_t) * E * N * K / 32);
    for (int i = 0; i < E * N * K / 8; ++i) codes[i] = rnd();
    for (int i = 0; i < E * N * K / 32; ++i) steps[i] = w4o_f64_to_bf16_rne(0.001 + (rnd() % 1000) * 1e-5);
    uint16_t x[4 * K], xb[4 * K];
    for (int i = 0; i < 4 * K; ++i) {
        x[i] = w4o_f64_to_f16_rne(((int)(rnd() % 2001) - 1000) / 500.0);
        xb[i] = w4o_f64_to_bf16_rne(((int)(rnd() % 2001) - 1000) / 500.0);
    }
    /* special activation values */
    x[3] = 0x7C00;  /* inf */
    x[5] = 0x0001;  /* smallest subnormal */
    xb[7] = 0x7FC0; /* NaN */
    double *W = malloc(sizeof(double) * N * K), y[N], a[N], Y[4 * N], A[4 * N];
    w4o_dequant(codes, steps, N, K, W);
    w4o_gemv(codes, steps, N, K, x, 0, y, a);
    w4o_gemv_omp(codes, steps, N, K, xb, 1, y, a);
    w4o_gemv_rows(codes, steps, N, K, x, 0, 5, 17, y, a);
    double xd[K];
    for (int k = 0; k < K; ++k) xd[k] = (k % 7) - 3.0;
    w4o_gemv_x64_rows(codes, steps, K, xd, 0, N, y, a);
    w4o_gemm(codes, steps, N, K, xb, 1, 3, K, Y, A);
    w4o_gemm(codes, steps, 0, K, xb, 1, 3, K, Y, A);
    /* gather: valid ids and one out of range */
    int32_t ids[5] = {0, N - 1, 3, 3, N};
    uint16_t *g = calloc(5 * K, sizeof(uint16_t));
    int bad = w4o_gather(codes, steps, N, K, ids, 5, g);
    /* expert product: direct, pool, row scales, route weights, a bad id */
    int32_t eids[T * TOPK] = {0, 5, 2, 2, 4, 1};
    int32_t slot_of[E] = {3, 0, 1, 2, 5, 4};
    float rs[E * N], rw[T * TOPK];
    for (int i = 0; i < E * N; ++i) rs[i] = 0.5f + (rnd() % 100) / 100.0f;
    for (int i = 0; i < T * TOPK; ++i) rw[i] = 1.0f / TOPK;
    double MY[T * TOPK * N], MA[T * TOPK * N];
    int rc = 0;
    rc |= w4o_moe(codes, steps, N * K / 8, N * K / 32, N, K, xb, 1, 0, K, eids, T, TOPK, NULL, E, 0, NULL, NULL, MY, MA);
    rc |= w4o_moe(codes, steps, N * K / 8, N * K / 32, N, K, x, 0, 1, K / 2 * 0 + K, eids, 2, TOPK, slot_of, E, E, rs,
                  NULL, MY, MA);
    rc |= w4o_moe(codes, steps, N * K / 8, N * K / 32, N, K, xb, 1, 0, K, eids, T, TOPK, NULL, E, 0, rs, rw, MY, MA);
    eids[1] = E + 2;
    const int rc_bad = w4o_moe(codes, steps, N * K / 8, N * K / 32, N, K, xb, 1, 0, K, eids, T, TOPK, NULL, E, 0, NULL,
                               NULL, MY, MA);
    /* renormalisation: ordinary, zero and huge rows */
    float v[K];
    uint16_t out[K];
    for (int k = 0; k < K; ++k) v[k] = (float)((int)(rnd() % 2001) - 1000) * 0.01f;
    w4o_rms_renorm(v, K, 0, out);
    w4o_rms_renorm(v, K, 1, out);
    memset(v, 0, sizeof(v));
    w4o_rms_renorm(v, K, 0, out);
    for (int k = 0; k < K; ++k) v[k] = 3e38f;
    w4o_rms_renorm(v, K, 1, out);
    /* grid packing: random bf16 values, then special groups */
    enum { GN = 4, GK = 128 };
    uint16_t table[GN * GK];
    for (int i = 0; i < GN * GK; ++i) table[i] = w4o_f64_to_bf16_rne(((int)(rnd() % 31) - 15) * 0.0625);
    for (int i = 0; i < 32; ++i) table[i] = 0;                  /* all-zero group */
    for (int i = 32; i < 64; ++i) table[i] = 0x3F80;            /* one positive level */
    for (int i = 64; i < 96; ++i) table[i] = (i & 1) ? 0x0001 : 0x8001; /* bf16 subnormals */
    for (int i = 96; i < 128; ++i) table[i] = 0x7F7F;           /* largest finite */
    uint32_t gc[GN * GK / 8];
    uint16_t gs[GN * GK / 32];
    w4o_grid_to_codes(table, GN, GK, gc, gs);
    /* conversions of special values */
    double acc = 0.0;
    for (uint32_t h = 0; h < 65536; h += 7) {
        const double f = w4o_f16_to_f64((uint16_t)h), b = w4o_bf16_to_f64((uint16_t)h);
        if (isfinite(f)) acc += w4o_f64_to_f16_rne(f);
        if (isfinite(b)) acc += w4o_f64_to_bf16_rne(b);
    }
    printf("oracle checks: gather bad=%d moe rc=%d bad rc=%d (acc %g)\n", bad, rc, rc_bad, acc);
    free(codes);
    free(steps);
    free(W);
    free(g);
    return (bad == 0 || rc != 0 || rc_bad == 0) ? 1 : 0;
}
