// Small-batch W4A16 product on the matrix cores of gfx950 (M <= 16 rows).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 3 -
// Multiply Straight From the Packed Weights") multiplies packed weights without
// writing a 16-bit copy; its section "Step 5 - Attention for One Token at a
// Time" notes that without matrix units a dot-product instruction lost to a
// plain multiply-and-sum.  Here the M activation rows make the product a real
// (if thin) contraction, so it runs on MFMA.
//
// One v_mfma_f32_16x16x32_f16 covers one group of 32 codes for 16 weight rows
// (B operand) against all 16 (padded) activation rows (A operand), so its fp32
// result can be scaled by that group's bf16 step, per weight row, exactly
// where the step applies.  Operands are exact fp16: the weights are c - 8
// (OR-magic unpack plus one packed subtract/FMA, as in the GEMV) and each
// activation row m is staged as x * 2^s_m with a per-row power of two, undone
// once per output.
//
// Register layout (lane i, 0..63): A holds X[m = i%16][k-slots 8(i/16)..+7],
// B holds W[n = i%16][the same k-slots], D holds rows m = 4(i/16)..+3 of
// column n = i%16.  The k-slots of lane group q = i/16 are word q of the group,
// in the pair order (c0,c4),(c1,c5),(c2,c6),(c3,c7) for both operands.
//
// Loads: lane (n, q) reads the whole 16-byte group g0+q of row n (four lanes
// of a row read 64 contiguous bytes); a 4x4 transpose across the lane groups
// (v_permlane32_swap then v_permlane16_swap) leaves word q of groups g0..g0+3
// in the lane's four registers.
//
// Work split: a workgroup of WK waves owns a 16-row tile at a time; wave w owns
// a contiguous K-slice of GPW groups and keeps its A fragments in registers for
// the whole kernel.  Per-wave partial tiles are summed in LDS in wave order.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

// Plain small-M product: activation row m at X + m*ldx, output Y[m*ldy + n].
template <int GPW, bool STEPS8>
__global__ __launch_bounds__(1024) void gemm_smallm_kernel(const uint4 *__restrict__ codes,
                                                           const uint16_t *__restrict__ steps,
                                                           int N, int K,
                                                           const uint16_t *__restrict__ X,
                                                           long ldx, int dt, int M,
                                                           float *__restrict__ Y, long ldy) {
    __shared__ SmallMShared sh;
    const bool xvec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);
    smallm_engine<GPW, STEPS8>(
        codes, steps, N, K,
        [&](int m) __attribute__((always_inline)) { return X + (long)m * ldx; }, xvec, dt, M,
        blockIdx.x, gridDim.x,
        [&](int m, int n, float v) __attribute__((always_inline)) { Y[(long)m * ldy + n] = v; }, sh);
}

namespace {

typedef void (*GemmFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, long, int, int,
                       float *, long);

template <bool S8>
GemmFn pick_gemm_s(int gpw) {
    switch (gpw) {
        case 4: return gemm_smallm_kernel<4, S8>;
        case 8: return gemm_smallm_kernel<8, S8>;
        case 12: return gemm_smallm_kernel<12, S8>;
        case 16: return gemm_smallm_kernel<16, S8>;
    }
    return nullptr;
}

GemmFn pick_gemm(int gpw, bool steps8) {
    return steps8 ? pick_gemm_s<true>(gpw) : pick_gemm_s<false>(gpw);
}

}  // namespace

GemmTile gemm_tile(int N, int K) {
    // Groups per wave: at most 16 (64 A-fragment registers); waves per
    // workgroup cover K; at most 16 waves.  Grid: one workgroup per 16-row
    // tile, capped so that each loops over a few tiles.
    const int G = K / 32;
    GemmTile t;
    int wk = (G + 15) / 16;
    if (wk < 1) wk = 1;
    int gpw = (G + wk - 1) / wk;
    gpw = (gpw + 3) / 4 * 4;
    if (gpw < 4) gpw = 4;
    t.gpw = gpw;
    t.waves = (G + gpw - 1) / gpw;
    if (t.waves < 1) t.waves = 1;
    const int ntiles = (N + 15) / 16;
    t.blocks = ntiles < 1024 ? (ntiles < 1 ? 1 : ntiles) : 1024;
    return t;
}

hipError_t launch_gemm_smallm(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              hipStream_t stream) {
    const GemmTile t = gemm_tile(N, K);
    const bool steps8 = (K / 32) % 4 == 0 && (reinterpret_cast<uintptr_t>(steps) & 7) == 0;
    GemmFn fn = pick_gemm(t.gpw, steps8);
    if (!fn || t.waves > 16) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, dim3(t.blocks), dim3(64 * t.waves), 0, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, X, ldx, dt, M, Y, ldy);
    return hipGetLastError();
}

}  // namespace w4
