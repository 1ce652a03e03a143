// Batch-1 W4A16 matrix-vector product for gfx950.
//
// The decode step of the dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch"
// (section "Step 3 - Multiply Straight From the Packed Weights") multiplies one
// activation vector by every packed matrix, unpacking in registers and never
// writing a 16-bit weight copy; its speed limit is the weight read.
//
// Mapping.  A wave's 64 lanes are cut into 64/L row slots of L lanes.  Each slot
// owns one row at a time; lane l of a slot owns the groups g = l, l+L, l+2L, ...
// (< K/32) of every row it visits, so one wave-wide 16-byte load instruction
// reads 64/L contiguous runs of 16*L bytes.  The lane's activations for those
// groups stay in registers for the whole kernel (16 fp16 pairs per group), and
// the workgroup loops over rows with a grid stride, R rows per slot in flight.
// Partial row sums are reduced across the L lanes of a slot by lane shuffles
// in a fixed order, so results are bitwise reproducible.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

template <int L, int NG, int R>
__global__ __launch_bounds__(256) void gemv_kernel(const uint4 *__restrict__ codes,
                                                   const uint16_t *__restrict__ steps,
                                                   int N, int K,
                                                   const uint16_t *__restrict__ x, int dt,
                                                   float *__restrict__ y) {
    constexpr int SLOTS = kWave / L;
    extern __shared__ _Float16 xs[];
    __shared__ int red[8];
    const int G = K >> 5;
    const Staging st = stage_activations(x, K, dt, xs, red);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int l = lane % L, slot = lane / L;
    const int rows_per_iter = nwaves * SLOTS * R;

    h2 xr[NG][16];
    const h2 *xs2 = reinterpret_cast<const h2 *>(xs);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = l + i * L;
#pragma unroll
        for (int p = 0; p < 16; ++p) xr[i][p] = (g < G) ? xs2[g * 16 + p] : h2{0, 0};
    }

    for (int row0 = blockIdx.x * rows_per_iter; row0 < N; row0 += gridDim.x * rows_per_iter) {
        uint4 q[R][NG];
        uint32_t sb[R][NG];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + (r * nwaves + wave) * SLOTS + slot;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = l + i * L;
                if (row < N && g < G) {
                    q[r][i] = codes[(size_t)row * G + g];
                    sb[r][i] = steps[(size_t)row * G + g];
                } else {
                    q[r][i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
                    sb[r][i] = 0;
                }
            }
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc[r] = 0.0f;
            const int row = row0 + (r * nwaves + wave) * SLOTS + slot;
            if (!st.fallback) {
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    acc[r] = __builtin_fmaf(group_dot(q[r][i], xr[i]), bf16_to_f32(sb[r][i]), acc[r]);
            } else {
                for (int i = 0; i < NG; ++i) {
                    const int g = l + i * L;
                    if (row < N && g < G)
                        acc[r] = __builtin_fmaf(group_dot_f32(q[r][i], x + g * 32, dt),
                                                bf16_to_f32(sb[r][i]), acc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1) acc[r] += __shfl_xor(acc[r], off, kWave);
            const int row = row0 + (r * nwaves + wave) * SLOTS + slot;
            if (l == 0 && row < N) y[row] = st.fallback ? acc[r] : __builtin_ldexpf(acc[r], -st.scale);
        }
    }
}

// ---- tiling table ------------------------------------------------------------

namespace {

typedef void (*GemvFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, int, float *);

template <int L, int NG>
GemvFn pick_r(int R) {
    return R == 1 ? gemv_kernel<L, NG, 1> : gemv_kernel<L, NG, 2>;
}

template <int L>
GemvFn pick_ng(int NG, int R) {
    switch (NG) {
        case 1: return pick_r<L, 1>(R);
        case 2: return pick_r<L, 2>(R);
        case 3: return pick_r<L, 3>(R);
        case 4: return pick_r<L, 4>(R);
        case 6: return pick_r<L, 6>(R);
        case 8: return pick_r<L, 8>(R);
    }
    return nullptr;
}

GemvFn pick(int L, int NG, int R) {
    switch (L) {
        case 4: return pick_ng<4>(NG, R);
        case 8: return pick_ng<8>(NG, R);
        case 16: return pick_ng<16>(NG, R);
        case 32: return pick_ng<32>(NG, R);
        case 64: return pick_ng<64>(NG, R);
    }
    return nullptr;
}

}  // namespace

GemvTile gemv_tile(int N, int K) {
    // Lanes per row L and groups per lane NG: cover the G = K/32 groups of a
    // row with as few idle lane slots as possible, preferring NG <= 4 (fewer
    // activation registers) and wider L for long rows.
    const int G = K / 32;
    static const int kL[] = {64, 32, 16, 8, 4};
    static const int kNG[] = {1, 2, 3, 4, 6, 8};
    GemvTile best{64, 8, 1, 4, 0};
    double best_cost = 1e30;
    for (int L : kL) {
        for (int NG : kNG) {
            if (L * NG < G) continue;
            const double idle = double(L * NG - G) / double(L * NG);
            double cost = idle + (NG > 4 ? 0.05 * (NG - 4) : 0.0);
            if (L < 16 && G >= 32) cost += 0.2;  // short runs per load
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                best = GemvTile{L, NG, 1, 4, 0};
            }
        }
    }
    if (G == 0) best = GemvTile{64, 1, 1, 4, 0};
    // Rows in flight per slot and waves per workgroup: big matrices keep two
    // rows per slot in flight with four-wave workgroups; small ones use one
    // row and one-wave workgroups so that the rows spread over every CU.
    const int slots = 64 / best.L;
    const long rows_wave = (long)slots;
    if ((long)N >= rows_wave * 2 * 4 * 1024) { best.R = 2; best.waves = 4; }
    else if ((long)N >= rows_wave * 4 * 512) { best.R = 1; best.waves = 4; }
    else { best.R = 1; best.waves = 1; }
    const long rows_per_iter = rows_wave * best.R * best.waves;
    long blocks = (N + rows_per_iter - 1) / rows_per_iter;
    const long cap = 2048;
    best.blocks = (int)(blocks < cap ? (blocks < 1 ? 1 : blocks) : cap);
    return best;
}

hipError_t launch_gemv(const uint32_t *codes, const uint16_t *steps, int N, int K,
                       const uint16_t *x, int dt, float *y, hipStream_t stream) {
    const GemvTile t = gemv_tile(N, K);
    GemvFn fn = pick(t.L, t.NG, t.R);
    if (!fn) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)(K > 0 ? K : 2) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3(t.blocks), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, x, dt, y);
    return hipGetLastError();
}

}  // namespace w4
