// Small-batch W4A16 product on the matrix cores of gfx950 (M <= 16 rows).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 3 -
// Multiply Straight From the Packed Weights") multiplies packed weights without
// writing a 16-bit copy; its section "Step 5 - Attention for One Token at a
// Time" notes that without matrix units a dot-product instruction lost to a
// plain multiply-and-sum.  Here the M activation rows make the product a real
// (if thin) contraction, so it runs on MFMA (engine in w4_mfma.h).
//
// Grid: x = steps of kSmallMWaves/KW 16-row tiles, y = the K-slice.  With one
// slice the engine stores Y directly; with several, each slice writes its
// partial sums to a workspace [S][M][N] and a second kernel adds them in slice
// order.
#include <cstdio>
#include <cstdlib>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

// Activation row m at X + m*ldx.  S == 1: output Y[m*ldy + n]; otherwise the
// slice's partial to ws[(slice*M + m)*N + n].
template <int R, bool STEPS8>
__global__ __launch_bounds__(64 * kSmallMWaves) void gemm_smallm_kernel(
    const uint4 *__restrict__ codes, const uint16_t *__restrict__ steps, int N, int K,
    const uint16_t *__restrict__ X, long ldx, int dt, int M, float *__restrict__ Y, long ldy,
    float *__restrict__ ws, int Gs, int mp_log2, int KW) {
    __shared__ SmallMShared sh;
    extern __shared__ uint4 smallm_a[];
    const int G = K >> 5;
    const int slice = blockIdx.y;
    const int g_lo = slice * Gs, g_hi = min(G, g_lo + Gs);
    const bool xvec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);
    const bool direct = gridDim.y == 1;
    smallm_engine<R, STEPS8>(
        codes, steps, N, K, g_lo, g_hi,
        [&](int m) __attribute__((always_inline)) { return X + (long)m * ldx; }, xvec, dt, M,
        mp_log2, KW, blockIdx.x, gridDim.x,
        [&](int m, int n, float v) __attribute__((always_inline)) {
            if (direct) Y[(long)m * ldy + n] = v;
            else ws[((long)slice * M + m) * N + n] = v;
        },
        sh, smallm_a);
}

// Y[m][n] = sum over slices s = 0, 1, ... of ws[s][m][n], in that order.
__global__ __launch_bounds__(256) void smallm_slices_kernel(const float *__restrict__ ws, int S,
                                                            int M, int N, float *__restrict__ Y,
                                                            long ldy) {
    const long total = (long)M * N;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long)gridDim.x * blockDim.x) {
        float s = ws[i];
        for (int k = 1; k < S; ++k) s += ws[(long)k * total + i];
        const int m = (int)(i / N), n = (int)(i % N);
        Y[(long)m * ldy + n] = s;
    }
}

namespace {

typedef void (*GemmFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, long, int, int,
                       float *, long, float *, int, int, int);

template <bool S8>
GemmFn pick_gemm_s(int R) {
    switch (R) {
        case 4: return gemm_smallm_kernel<4, S8>;
        case 8: return gemm_smallm_kernel<8, S8>;
        case 16: return gemm_smallm_kernel<16, S8>;
        case 24: return gemm_smallm_kernel<24, S8>;
    }
    return nullptr;
}

}  // namespace

size_t gemm_smallm_workspace(int N, int K, int M) {
    const SmallMPlan p = smallm_plan(N, K, M, 1);
    return p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
}

int smallm_grid_x(int N, int KW) {
    const int ntiles = (N + 15) / 16, tpw = kSmallMWaves / KW;
    int bx = (ntiles + tpw - 1) / tpw;
    if (bx > 2048) bx = 2048;
    return bx < 1 ? 1 : bx;
}

hipError_t launch_gemm_smallm(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              float *ws, hipStream_t stream) {
    const SmallMPlan p = smallm_plan(N, K, M, 1);
    const bool steps8 = (K / 32) % 4 == 0 && (reinterpret_cast<uintptr_t>(steps) & 7) == 0;
    GemmFn fn = steps8 ? pick_gemm_s<true>(p.R) : pick_gemm_s<false>(p.R);
    if (!fn || (p.S > 1 && !ws)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, dim3(smallm_grid_x(N, p.KW), p.S), dim3(64 * kSmallMWaves), p.lds_a,
                       stream, reinterpret_cast<const uint4 *>(codes), steps, N, K, X, ldx, dt, M, Y,
                       ldy, ws, p.Gs, p.mp_log2, p.KW);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    const long total = (long)M * N;
    long blocks = (total + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(smallm_slices_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, p.S,
                       M, N, Y, ldy);
    return hipGetLastError();
}

}  // namespace w4
