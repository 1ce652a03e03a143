// Small-batch W4A16 product on the matrix cores of gfx950 (M <= 16 rows).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 3 -
// Multiply Straight From the Packed Weights") multiplies packed weights without
// writing a 16-bit copy; its section "Step 5 - Attention for One Token at a
// Time" notes that without matrix units a dot-product instruction lost to a
// plain multiply-and-sum.  Here the M activation rows make the product a real
// (if thin) contraction, so it runs on MFMA (engine in w4_mfma.h); a single row
// goes to the batch-1 kernel instead.
//
// Grid: x = steps of kSmallMWaves/KW 16-row tiles, y = the K-slice.  With one
// slice the engine stores Y directly.  With several, each slice stores its
// partial sums to a workspace [S][M][N] (agent-coherent stores) and counts
// itself in on a per-column-of-the-grid counter; the last slice to arrive adds
// the S partials in slice order (so the result does not depend on the order of
// arrival), writes Y and puts the counter back to zero.
#include <cstdio>
#include <cstdlib>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

// Activation row m at X + m*ldx.  S == 1: output Y[m*ldy + n]; otherwise the
// slice's partial to part[(slice*M + m)*N + n], then the last slice of grid
// column blockIdx.x sums them.  cnt: one counter per grid column.
template <int R, bool STEPS8>
__global__ __launch_bounds__(64 * kSmallMWaves) void gemm_smallm_kernel(
    const uint4 *__restrict__ codes, const uint16_t *__restrict__ steps, int N, int K,
    const uint16_t *__restrict__ X, long ldx, int dt, int M, float *__restrict__ Y, long ldy,
    float *__restrict__ part, unsigned *__restrict__ cnt, int Gs, int mp_log2, int KW) {
    __shared__ SmallMShared sh;
    __shared__ int last_s;
    extern __shared__ uint4 smallm_a[];
    const int G = K >> 5;
    const int slice = blockIdx.y, S = gridDim.y;
    const int g_lo = slice * Gs, g_hi = min(G, g_lo + Gs);
    const bool xvec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);
    smallm_engine<R, STEPS8>(
        codes, steps, N, K, g_lo, g_hi,
        [&](int m) __attribute__((always_inline)) { return X + (long)m * ldx; }, xvec, dt, M,
        mp_log2, KW, blockIdx.x, gridDim.x,
        [&](int m, int n, float v) __attribute__((always_inline)) {
            if (S == 1)
                Y[(long)m * ldy + n] = v;
            else
                __hip_atomic_store(part + ((long)slice * M + m) * N + n, v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        },
        sh, smallm_a);
    if (S == 1) return;
    // this slice's partials are stored (every wave waits for its own), then
    // one count per workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        last_s = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)S - 1;
    __syncthreads();
    if (!last_s) return;
    // the last slice of this grid column: its tiles, every (m, n), slices in order
    const int tpw = kSmallMWaves / KW, ntiles = (N + 15) >> 4, cols = tpw * 16;
    const long plane = (long)M * N;
    for (int tg = blockIdx.x; tg * tpw < ntiles; tg += gridDim.x) {
        for (int o = threadIdx.x; o < cols * M; o += blockDim.x) {
            const int m = o / cols, n = tg * cols + o % cols;
            if (n >= N) continue;
            const float *pp = part + (long)m * N + n;
            float v = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int k = 1; k < S; ++k)
                v += __hip_atomic_load(pp + k * plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            Y[(long)m * ldy + n] = v;
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

namespace {

typedef void (*GemmFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, long, int, int,
                       float *, long, float *, unsigned *, int, int, int);

template <bool S8>
GemmFn pick_gemm_s(int R) {
    switch (R) {
        case 3: return gemm_smallm_kernel<3, S8>;
        case 4: return gemm_smallm_kernel<4, S8>;
        case 6: return gemm_smallm_kernel<6, S8>;
        case 8: return gemm_smallm_kernel<8, S8>;
        case 12: return gemm_smallm_kernel<12, S8>;
        case 16: return gemm_smallm_kernel<16, S8>;
        case 24: return gemm_smallm_kernel<24, S8>;
    }
    return nullptr;
}

SmallMPlan gemm_plan(int N, int K, int M) { return smallm_plan(N, K, M, 1, kSmallMLdsFast, true); }

}  // namespace

// Up to four rows: M batch-1 products side by side, their weights read from
// HBM about once (the workgroups of a row block run together); on a set of
// the four sweep shapes 28.1 against 32.3 us at M = 2, 34.3 against 37.9 us at
// M = 4.  From 8 rows the matrix cores win (45.9 against 48.9 us at M = 8).
static bool smallm_by_rows(int M) { return M <= settings().smallm_rows_max; }

size_t gemm_smallm_workspace(int N, int K, int M) {
    if (M == 1 || smallm_by_rows(M)) return 0;  // batch-1 products
    const SmallMPlan p = gemm_plan(N, K, M);
    return p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
}

int smallm_grid_x(int N, int KW) {
    const int ntiles = (N + 15) / 16, tpw = kSmallMWaves / KW;
    int bx = (ntiles + tpw - 1) / tpw;
    if (bx > kMaxGridColumns) bx = kMaxGridColumns;
    return bx < 1 ? 1 : bx;
}

// Grid columns of a small-M launch of S slices: one per step of tiles, but
// no more than `groups` workgroups in all, so that each workgroup stages its
// activations once and then loops over several tiles.
static int gemm_grid_x(int N, const SmallMPlan &p, int groups) {
    int bx = smallm_grid_x(N, p.KW);
    const int cap = (int)((groups + p.S - 1) / p.S);
    return bx < cap ? bx : (cap < 1 ? 1 : cap);
}

hipError_t launch_gemm_smallm(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              void *ws, hipStream_t stream) {
    // one activation row: the batch-1 kernel (no matrix-core padding)
    if (M == 1) return launch_gemv(codes, steps, N, K, X, dt, Y, stream);
    if (smallm_by_rows(M)) return launch_gemv_rows(codes, steps, N, K, X, ldx, dt, M, Y, ldy, stream);
    const SmallMPlan p = gemm_plan(N, K, M);
    const bool steps8 = (K / 32) % 4 == 0 && (reinterpret_cast<uintptr_t>(steps) & 7) == 0;
    GemmFn fn = steps8 ? pick_gemm_s<true>(p.R) : pick_gemm_s<false>(p.R);
    if (!fn || (p.S > 1 && !ws)) return hipErrorInvalidConfiguration;
    unsigned *cnt = static_cast<unsigned *>(ws);
    float *part = ws ? reinterpret_cast<float *>(static_cast<char *>(ws) + kWsCounterBytes) : nullptr;
    const int groups = (int)(p.KW == 1 && M >= 8 ? kSmallMWideGroups : kSmallMTargetGroups);
    hipLaunchKernelGGL(fn, dim3(gemm_grid_x(N, p, groups), p.S),
                       dim3(64 * kSmallMWaves), p.lds_a,
                       stream, reinterpret_cast<const uint4 *>(codes), steps, N, K, X, ldx, dt, M, Y,
                       ldy, part, cnt, p.Gs, p.mp_log2, p.KW);
    return hipGetLastError();
}

}  // namespace w4
