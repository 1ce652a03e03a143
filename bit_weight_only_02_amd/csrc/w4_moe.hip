// Expert-indexed W4A16 product for gfx950.
//
// The anyesh.me page "Running a 26B MoE on an 8 GB Jetson by streaming experts
// from SSD" (section "Streaming without touching a single GPU kernel") runs the
// routed-expert matmul as one kernel that takes the expert weight tensor and a
// small tensor of selected ids and addresses each expert as base + id * stride;
// a pool of expert slots is read the same way through slot ids and must give
// exactly the bytes of the full tensor, while every other per-expert tensor
// (scales, biases) keeps the real expert id.
//
// T tokens x topk choices = P pairs.  Up to four tokens, the P choices run as
// P matrix-vector products in one launch of the batch-1 kernel (one pair per
// gridDim.y index): nearly every chosen expert then has a single activation row.
//
// More tokens: each workgroup takes one DISTINCT
// expert (deduplicated on the device, in order of first appearance -- with
// wave ballots for up to 64 pairs), one
// K-slice and a group of 16-row tiles, reads that part of the expert's packed
// weights once, and runs the MFMA small-M engine with one A row per pair that
// chose the expert.  The weight address is the only place where slot_of
// enters, so direct and pool addressing execute identical arithmetic and agree
// bit for bit.  Per-expert side inputs (row_scale) are read with the real id.
//
// With one K-slice and no route weights the engine stores each pair's row,
// times row_scale[e], straight into Y.  Otherwise it stores unscaled per-slice
// rows into a workspace [S][P][N], and a finishing kernel adds the slices in
// order, applies row_scale[e] and, with route weights, sums a token's choices
// in ascending order.
#include <cstdio>
#include <cstdlib>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

constexpr int kMaxPairs = 1024;

template <int R, bool STEPS8>
__global__ __launch_bounds__(64 * kSmallMWaves) void moe_kernel(
    const uint4 *__restrict__ codes_base, const uint16_t *__restrict__ steps_base,
    int64_t stride_c4, int64_t stride_s, int N, int K, const uint16_t *__restrict__ X, long ldx,
    int dt, int x_per_pair, const int32_t *__restrict__ ids, int P, int topk,
    const int32_t *__restrict__ slot_of, int n_experts, int n_slots,
    const float *__restrict__ row_scale, float *__restrict__ out, int direct, int Gs, int KW,
    int32_t *__restrict__ dev_err) {
    __shared__ SmallMShared sh;
    extern __shared__ uint4 smallm_a[];
    __shared__ int ids_s[kMaxPairs];
    __shared__ unsigned char first_s[kMaxPairs];
    __shared__ int pairs_s[kMaxPairs];
    __shared__ int info_s[3];  // expert id, number of pairs, found
    const int u = blockIdx.y, slice = blockIdx.z;
    const int G = K >> 5;
    const int g_lo = slice * Gs, g_hi = min(G, g_lo + Gs);

    // ---- this workgroup's distinct expert and the pairs that chose it
    if (P <= kWave) {
        // one wave, in registers: lane p holds pair p's id; a pair is the first
        // of its expert when no earlier lane holds the same id; ballots give
        // the u-th first pair and the (ordered) pairs of that expert
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            const int e = lane < P ? ids[lane] : 0;
            bool first = lane < P;
            for (int q = 0; q < P; ++q) {
                const int eq = __builtin_amdgcn_readlane(e, q);
                first = first && !(q < lane && eq == e);
            }
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const uint64_t firsts = __builtin_amdgcn_ballot_w64(first);
            const int rank = __builtin_popcountll(firsts & below);
            const uint64_t pick = __builtin_amdgcn_ballot_w64(first && rank == u);
            if (pick == 0) {
                if (lane == 0) info_s[2] = 0;
            } else {
                const int eu = __builtin_amdgcn_readlane(e, __builtin_ctzll(pick));
                const uint64_t mine = __builtin_amdgcn_ballot_w64(lane < P && e == eu);
                if (lane < P && e == eu) pairs_s[__builtin_popcountll(mine & below)] = lane;
                if (lane == 0) {
                    info_s[0] = eu;
                    info_s[1] = __builtin_popcountll(mine);
                    info_s[2] = 1;
                }
            }
        }
        lds_barrier();
    } else {
    for (int p = threadIdx.x; p < P; p += blockDim.x) ids_s[p] = ids[p];
    lds_barrier();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int e = ids_s[p];
        int first = 1;
        for (int p2 = 0; p2 < p; ++p2)
            if (ids_s[p2] == e) { first = 0; break; }
        first_s[p] = (unsigned char)first;
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        int cnt = 0, e = 0, found = 0;
        for (int p = 0; p < P; ++p)
            if (first_s[p]) {
                if (cnt == u) { e = ids_s[p]; found = 1; break; }
                ++cnt;
            }
        int np = 0;
        if (found)
            for (int p = 0; p < P; ++p)
                if (ids_s[p] == e) pairs_s[np++] = p;
        info_s[0] = e;
        info_s[1] = np;
        info_s[2] = found;
    }
    lds_barrier();
    }
    if (!info_s[2]) return;  // fewer distinct experts than this grid row
    const int e = info_s[0], npairs = info_s[1];
    const int ntiles = (N + 15) >> 4;
    // destination of pair p, column n: Y[p][n], or this slice's workspace row
    auto dst = [&](int p, int n) __attribute__((always_inline)) -> float & {
        return out[((long)(direct ? 0 : slice) * P + p) * N + n];
    };

    // ---- addressing: the only use of slot_of
    long a = e;
    bool valid = e >= 0 && e < n_experts;
    if (valid && slot_of) {
        a = slot_of[e];
        valid = a >= 0 && a < n_slots;
    }
    if (!valid) {
        // never leave an untouched row behind: NaN rows and the error flag
        // (the tiles this workgroup owns: kSmallMWaves/KW consecutive ones per step)
        const int tpw = kSmallMWaves / KW, cols = tpw * 16;
        for (int t0 = blockIdx.x * tpw; t0 < ntiles; t0 += gridDim.x * tpw)
            for (int o = threadIdx.x; o < cols * npairs; o += blockDim.x) {
                const int n = t0 * 16 + o % cols;
                if (n < N) dst(pairs_s[o / cols], n) = __builtin_nanf("");
            }
        if (threadIdx.x == 0 && blockIdx.x == 0 && dev_err) *dev_err = 1;
        return;
    }
    const uint4 *codes = codes_base + a * stride_c4;
    const uint16_t *steps = steps_base + a * stride_s;
    const bool xvec = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);

    // up to 16 pairs per engine pass (one A row each)
    for (int c0 = 0; c0 < npairs; c0 += 16) {
        const int M = min(16, npairs - c0);
        int mp_log2 = 0;
        while ((1 << mp_log2) < M) ++mp_log2;
        auto xrow = [&](int m) __attribute__((always_inline)) {
            const int p = pairs_s[c0 + m];
            return X + (long)(x_per_pair ? p : p / topk) * ldx;
        };
        auto store = [&](int m, int n, float v) __attribute__((always_inline)) {
            const int p = pairs_s[c0 + m];
            if (direct && row_scale) v *= row_scale[(long)e * N + n];
            dst(p, n) = v;
        };
        smallm_engine<R, STEPS8>(codes, steps, N, K, g_lo, g_hi, xrow, xvec, dt, M, mp_log2, KW,
                                 blockIdx.x, gridDim.x, store, sh, smallm_a);
        lds_barrier();  // the engine's shared memory is reused by the next pass
    }
}

// Finish: v(p, n) = sum over slices s ascending of ws[s][p][n], times
// row_scale[e_p][n] (real id e_p; rows of an invalid id are already NaN).
// route_w: Y[t][n] = sum over j = 0..topk-1 ascending of route_w[t][j] * v(t*topk + j, n);
// otherwise Y[p][n] = v(p, n).
__global__ __launch_bounds__(256) void moe_finish_kernel(const float *__restrict__ ws, int S, int P,
                                                         int N, const int32_t *__restrict__ ids,
                                                         int n_experts,
                                                         const float *__restrict__ row_scale,
                                                         const float *__restrict__ route_w, int T,
                                                         int topk, float *__restrict__ Y) {
    const int rows = route_w ? T : P;
    const int total = rows * N;  // <= 1024 * N rows of pairs, well inside int
    const long plane = (long)P * N;
    // one pair's value: its slices in order, then row_scale of the real id
    auto pair_value = [&](int p, int n) __attribute__((always_inline)) {
        const long o = (long)p * N + n;
        float v = ws[o];
        for (int s = 1; s < S; ++s) v += ws[(long)s * plane + o];
        const int e = ids[p];
        if (row_scale && e >= 0 && e < n_experts) v *= row_scale[(long)e * N + n];
        return v;
    };
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
        const int r = i / N, n = i - r * N;
        if (route_w && S == 1) {
            // every choice's value and weight requested before any is used
            // (eight at a time), then row_scale, then the sum in ascending j
            float s = 0.0f;
            for (int j0 = 0; j0 < topk; j0 += 8) {
                float v[8], w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int p = r * topk + min(j0 + u, topk - 1);
                    v[u] = ws[(long)p * N + n];
                    w[u] = route_w[p];
                }
                if (row_scale) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int e = ids[r * topk + min(j0 + u, topk - 1)];
                        if (e >= 0 && e < n_experts) v[u] *= row_scale[(long)e * N + n];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (j0 + u < topk) s = __builtin_fmaf(w[u], v[u], s);
            }
            Y[i] = s;
        } else if (route_w) {
            float s = 0.0f;
            for (int j = 0; j < topk; ++j)
                s = __builtin_fmaf(route_w[r * topk + j], pair_value(r * topk + j, n), s);
            Y[i] = s;
        } else {
            Y[i] = pair_value(r, n);
        }
    }
}

namespace {

typedef void (*MoeFn)(const uint4 *, const uint16_t *, int64_t, int64_t, int, int, const uint16_t *,
                      long, int, int, const int32_t *, int, int, const int32_t *, int, int,
                      const float *, float *, int, int, int, int32_t *);

template <bool S8>
MoeFn pick_moe_s(int R) {
    switch (R) {
        case 3: return moe_kernel<3, S8>;
        case 4: return moe_kernel<4, S8>;
        case 6: return moe_kernel<6, S8>;
        case 8: return moe_kernel<8, S8>;
        case 12: return moe_kernel<12, S8>;
        case 16: return moe_kernel<16, S8>;
        case 24: return moe_kernel<24, S8>;
    }
    return nullptr;
}

}  // namespace

// Plan of an expert launch: rows per engine pass are at most min(16, P) (the
// pairs that chose one expert), and up to P experts run side by side.
static SmallMPlan moe_plan(int N, int K, int T, int topk) {
    const int P = T * topk;
    SmallMPlan p = smallm_plan(N, K, P < 16 ? P : 16, P);
    return p;
}

// Up to a few tokens (a setting, 4 by default): every choice runs as its own matrix-vector
// product, side by side in one launch of the batch-1 kernel (gridDim.y =
// pairs).  With few tokens almost every chosen expert serves a single pair,
// and the matrix engine would give it a 16-row MFMA tile with one live row:
// one expert layer at 4 tokens measured 2.6x faster this way although the
// few experts shared by two tokens are read twice.
// (the bound is a setting, 4 by default)
bool moe_by_pairs(int T) { return T <= settings().moe_pairs_max_t; }

size_t moe_workspace(int N, int K, int T, int topk, bool route) {
    if (moe_by_pairs(T)) return route ? (size_t)T * topk * N * sizeof(float) : 0;
    const SmallMPlan p = moe_plan(N, K, T, topk);
    if (p.S == 1 && !route) return 0;
    return (size_t)p.S * T * topk * N * sizeof(float);
}

hipError_t launch_moe(const uint32_t *codes_base, const uint16_t *steps_base,
                      int64_t stride_codes, int64_t stride_steps, int N, int K,
                      const uint16_t *X, long ldx, int dt, int x_per_pair,
                      const int32_t *ids, int T, int topk, const int32_t *slot_of,
                      int n_experts, int n_slots, const float *row_scale, const float *route_w,
                      float *Y, void *wsv, int32_t *dev_err, hipStream_t stream) {
    // partial sums after the workspace's counter area (which this kernel leaves alone)
    float *ws = wsv ? reinterpret_cast<float *>(static_cast<char *>(wsv) + kWsCounterBytes) : nullptr;
    if (moe_by_pairs(T)) {
        // rows straight into Y (times row_scale), or per-choice rows into the
        // workspace for the route-weighted sum of the finishing kernel
        if (route_w && !ws) return hipErrorInvalidConfiguration;
        const int P = T * topk;
        hipError_t e = launch_gemv_pairs(codes_base, steps_base, stride_codes, stride_steps, N, K, X, ldx, dt,
                                         x_per_pair, ids, P, topk, slot_of, n_experts, n_slots,
                                         route_w ? nullptr : row_scale, route_w ? ws : Y, dev_err, stream);
        if (e != hipSuccess || !route_w) return e;
        const long blocks = ((long)T * N + 255) / 256;
        hipLaunchKernelGGL(moe_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, 1, P, N, ids,
                           n_experts, row_scale, route_w, T, topk, Y);
        return hipGetLastError();
    }
    if (dt == 2) return hipErrorInvalidConfiguration;  // fp32 rows are renormalised by the caller here
    const SmallMPlan p = moe_plan(N, K, T, topk);
    const bool steps8 = (K / 32) % 4 == 0 && (reinterpret_cast<uintptr_t>(steps_base) & 7) == 0 &&
                        (stride_steps % 4) == 0;
    MoeFn fn = steps8 ? pick_moe_s<true>(p.R) : pick_moe_s<false>(p.R);
    const int direct = (p.S == 1 && !route_w) ? 1 : 0;
    if (!fn || (!direct && !ws)) return hipErrorInvalidConfiguration;
    const int P = T * topk;
    hipLaunchKernelGGL(fn, dim3(smallm_grid_x(N, p.KW), P, p.S), dim3(64 * kSmallMWaves), p.lds_a,
                       stream, reinterpret_cast<const uint4 *>(codes_base), steps_base,
                       stride_codes / 4, stride_steps, N, K, X, ldx, dt, x_per_pair, ids, P, topk,
                       slot_of, n_experts, n_slots, row_scale, direct ? Y : ws, direct, p.Gs, p.KW,
                       dev_err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    const long total = (long)(route_w ? T : P) * N;
    long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(moe_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, p.S, P,
                       N, ids, n_experts, row_scale, route_w, T, topk, Y);
    return hipGetLastError();
}

}  // namespace w4
