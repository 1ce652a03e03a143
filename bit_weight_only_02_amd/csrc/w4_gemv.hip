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
#include <cstdio>
#include <cstdlib>
#include <type_traits>

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
    extern __shared__ _Float16 xs[];  // the raw activations (stage_raw_halves(K))
    const int G = K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int l = lane % L, slot = lane / L;
    const int rows_per_iter = nwaves * SLOTS * R;
    const int gstride = gridDim.x * rows_per_iter;

    if (G == 0) {  // empty sums
        for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < N; n += gridDim.x * blockDim.x)
            y[n] = 0.0f;
        return;
    }

    // Group indices of this lane, clamped so that every load is in bounds and
    // can be issued without a branch; lanes past the row end contribute zero.
    int gc[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) gc[i] = min(l + i * L, G - 1);

    auto load_rows = [&](uint4 (&q)[R][NG], uint32_t (&sv)[R][NG], int r0)
        __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(r0 + (r * nwaves + wave) * SLOTS + slot, N - 1);
            const uint4 *cp = codes + (size_t)row * G;
            const uint16_t *sp = steps + (size_t)row * G;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                q[r][i] = cp[gc[i]];
                sv[r][i] = sp[gc[i]];
            }
        }
    };

    // The activations go to LDS by DMA with the first rows' weights requested
    // right behind them; one barrier later every wave stages its own lanes'
    // activations into registers (wave_scan / convert_group) -- no further
    // workgroup-wide step.  A wave that cannot stage exactly takes the fp32
    // path on its own.
    uint16_t *raw = reinterpret_cast<uint16_t *>(xs);
    stage_issue(x, K, raw);
    int row0 = blockIdx.x * rows_per_iter;
    uint4 qa[R][NG];
    uint32_t sa[R][NG];
    if (row0 < N) load_rows(qa, sa, row0);
    if (!stage_vector_path(x))
        for (int i = threadIdx.x; i < K; i += blockDim.x) raw[i] = x[i];
    wait_vmcnt<0>();
    lds_barrier();

    // fp16: the values are staged as they are (scale 0, never the fp32 path);
    // bf16: scaled into fp16 after a per-wave exponent scan.
    WaveScale ws{0, 0, 0};
    if (dt != 0) ws = wave_scan(raw, K, dt);
    h2 xr[NG][16];
    int lost = ws.bad;
    auto load_xr = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            if (g < G) {
                if (dt == 0)
                    permute_group_f16(raw, g, xr[i]);
                else
                    lost |= convert_group(raw, g, dt, ws, xr[i]);
            } else {
#pragma unroll
                for (int p = 0; p < 16; ++p) xr[i][p] = h2{0, 0};
            }
        }
    };
    if (!ws.bad) load_xr();
    Staging st;
    st.scale = ws.scale;
    st.fallback = wave_or_i32(lost);

    auto compute_rows = [&](const uint4 (&q)[R][NG], const uint32_t (&sv)[R][NG], int r0,
                            auto exact_f32) __attribute__((always_inline)) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = l + i * L;
                float part;
                if constexpr (decltype(exact_f32)::value)
                    part = group_dot_f32(q[r][i], raw + gc[i] * 32, dt);
                else
                    part = group_dot(q[r][i], xr[i]);
                acc[r] = (g < G) ? __builtin_fmaf(part, bf16_to_f32(sv[r][i]), acc[r]) : acc[r];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1) acc[r] += __shfl_xor(acc[r], off, kWave);
            const int row = r0 + (r * nwaves + wave) * SLOTS + slot;
            if (l == 0 && row < N)
                y[row] = decltype(exact_f32)::value ? acc[r] : __builtin_ldexpf(acc[r], -st.scale);
        }
    };

    // Each step issues all R*NG row loads of the lane back to back (clamped,
    // so none sits behind a branch), then does the math; other waves on the
    // CU keep the memory system busy meanwhile.  The first step's loads were
    // issued before the staging.
    auto row_loop = [&](auto exact_f32) __attribute__((always_inline)) {
        if (row0 >= N) return;
        compute_rows(qa, sa, row0, exact_f32);
        for (row0 += gstride; row0 < N; row0 += gstride) {
            load_rows(qa, sa, row0);
            compute_rows(qa, sa, row0, exact_f32);
        }
    };
    // The staging outcome is uniform within the wave: branch on it once, in a
    // scalar register.
    if (__builtin_amdgcn_readfirstlane(st.fallback))
        row_loop(std::true_type{});
    else
        row_loop(std::false_type{});
}

// ---- tiling table ------------------------------------------------------------

namespace {

typedef void (*GemvFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, int, float *);

template <int L, int NG>
GemvFn pick_r(int R) {
    switch (R) {
        case 1: return gemv_kernel<L, NG, 1>;
        case 2: return gemv_kernel<L, NG, 2>;
        case 4: return gemv_kernel<L, NG, 4>;
    }
    return nullptr;
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
    // row with as few idle lane slots as possible; among equal covers prefer
    // 16 lanes per row and three or four groups per lane, which measured best
    // on MI355X (e.g. 262144 x 1536: L=16, NG=3 at 4.8 TB/s against 3.1 TB/s
    // for L=64, NG=1 with a quarter of the lanes idle).
    const int G = K / 32;
    static const int kL[] = {16, 32, 64, 8};
    static const int kNG[] = {3, 4, 2, 6, 1, 8};
    GemvTile best{16, 3, 2, 4, 0};
    double best_cost = 1e30;
    for (int L : kL) {
        for (int NG : kNG) {
            if (L * NG < G) continue;
            double cost = double(L * NG - G) / double(L * NG);
            if (NG > 4) cost += 0.02 * (NG - 4);  // register pressure
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                best = GemvTile{L, NG, 1, 4, 0};
            }
        }
    }
    if (G == 0) best = GemvTile{64, 1, 1, 4, 0};
    // One row per slot in flight and four-wave workgroups (fewer registers,
    // more waves per CU measured faster than two rows per slot); at most four
    // workgroups per CU (1024), each looping over rows with a grid stride.
    const long rows_per_iter = (long)(64 / best.L) * best.R * best.waves;
    const long blocks = (N + rows_per_iter - 1) / rows_per_iter;
    best.blocks = (int)(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
    return best;
}

hipError_t launch_gemv(const uint32_t *codes, const uint16_t *steps, int N, int K,
                       const uint16_t *x, int dt, float *y, hipStream_t stream) {
    GemvTile t = gemv_tile(N, K);
    // W4_GEMV_TILE="L,NG,R,waves,blocks" overrides the table (tile sweeps);
    // it changes only the schedule, never what is computed.
    if (const char *e = getenv("W4_GEMV_TILE")) {
        GemvTile o;
        if (sscanf(e, "%d,%d,%d,%d,%d", &o.L, &o.NG, &o.R, &o.waves, &o.blocks) == 5 &&
            o.L * o.NG * 32 >= K && o.waves >= 1 && o.waves <= 4 && o.blocks >= 1)
            t = o;
    }
    GemvFn fn = pick(t.L, t.NG, t.R);
    if (!fn) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)(stage_raw_halves(K) + 8) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3(t.blocks), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, x, dt, y);
    return hipGetLastError();
}

}  // namespace w4
