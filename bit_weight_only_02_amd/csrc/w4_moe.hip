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
// Here: T tokens x topk choices = P pairs.  Each workgroup takes one DISTINCT
// expert (deduplicated on the device, in order of first appearance) and a
// range of 16-row tiles, reads that expert's packed weights once, and runs the
// MFMA small-M engine with one A row per pair that chose the expert.  Results
// go to one output row per pair, multiplied by row_scale[e] of the real id e.
// The weight address is the only place where slot_of enters, so direct and
// pool addressing execute identical arithmetic and agree bit for bit.
//
// The route-weighted sum over a token's choices runs as a second kernel over
// the per-pair rows, in ascending choice order.
#include <cstdio>
#include <cstdlib>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

constexpr int kMaxPairs = 1024;

template <int GPW, bool STEPS8>
__global__ __launch_bounds__(1024) void moe_kernel(const uint4 *__restrict__ codes_base,
                                                   const uint16_t *__restrict__ steps_base,
                                                   int64_t stride_c4, int64_t stride_s,
                                                   int N, int K,
                                                   const uint16_t *__restrict__ X, long ldx, int dt,
                                                   int x_per_pair,
                                                   const int32_t *__restrict__ ids, int P, int topk,
                                                   const int32_t *__restrict__ slot_of,
                                                   int n_experts, int n_slots,
                                                   const float *__restrict__ row_scale,
                                                   float *__restrict__ out,
                                                   int32_t *__restrict__ dev_err) {
    __shared__ SmallMShared sh;
    __shared__ int ids_s[kMaxPairs];
    __shared__ unsigned char first_s[kMaxPairs];
    __shared__ int pairs_s[kMaxPairs];
    __shared__ int info_s[3];  // expert id, number of pairs, found
    const int u = blockIdx.y;

    // ---- this workgroup's distinct expert and the pairs that chose it
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
    if (!info_s[2]) return;  // fewer distinct experts than this grid row
    const int e = info_s[0], npairs = info_s[1];
    const int ntiles = (N + 15) >> 4;

    // ---- addressing: the only use of slot_of
    long a = e;
    bool valid = e >= 0 && e < n_experts;
    if (valid && slot_of) {
        a = slot_of[e];
        valid = a >= 0 && a < n_slots;
    }
    if (!valid) {
        // never leave an untouched row behind: NaN rows and the error flag
        for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
            for (int o = threadIdx.x; o < 16 * npairs; o += blockDim.x) {
                const int n = tile * 16 + (o & 15);
                if (n < N) out[(long)pairs_s[o >> 4] * N + n] = __builtin_nanf("");
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
        auto xrow = [&](int m) __attribute__((always_inline)) {
            const int p = pairs_s[c0 + m];
            return X + (long)(x_per_pair ? p : p / topk) * ldx;
        };
        auto store = [&](int m, int n, float v) __attribute__((always_inline)) {
            const int p = pairs_s[c0 + m];
            if (row_scale) v *= row_scale[(long)e * N + n];
            out[(long)p * N + n] = v;
        };
        smallm_engine<GPW, STEPS8>(codes, steps, N, K, xrow, xvec, dt, M, blockIdx.x, gridDim.x,
                                   store, sh);
        lds_barrier();  // the engine's shared memory is reused by the next pass
    }
}

// Y[t][n] = sum over j = 0..topk-1, ascending, of route_w[t][j] * rows[t*topk + j][n].
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *__restrict__ rows,
                                                          const float *__restrict__ route_w,
                                                          int T, int topk, int N,
                                                          float *__restrict__ Y) {
    const long total = (long)T * N;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long)gridDim.x * blockDim.x) {
        const int t = (int)(i / N), n = (int)(i % N);
        float s = 0.0f;
        for (int j = 0; j < topk; ++j)
            s = __builtin_fmaf(route_w[t * topk + j], rows[((long)t * topk + j) * N + n], s);
        Y[i] = s;
    }
}

namespace {

typedef void (*MoeFn)(const uint4 *, const uint16_t *, int64_t, int64_t, int, int, const uint16_t *,
                      long, int, int, const int32_t *, int, int, const int32_t *, int, int,
                      const float *, float *, int32_t *);

template <bool S8>
MoeFn pick_moe_s(int gpw) {
    switch (gpw) {
        case 4: return moe_kernel<4, S8>;
        case 8: return moe_kernel<8, S8>;
        case 12: return moe_kernel<12, S8>;
        case 16: return moe_kernel<16, S8>;
    }
    return nullptr;
}

}  // namespace

hipError_t launch_moe(const uint32_t *codes_base, const uint16_t *steps_base,
                      int64_t stride_codes, int64_t stride_steps, int N, int K,
                      const uint16_t *X, long ldx, int dt, int x_per_pair,
                      const int32_t *ids, int T, int topk, const int32_t *slot_of,
                      int n_experts, int n_slots, const float *row_scale, float *rows_out,
                      int32_t *dev_err, hipStream_t stream) {
    const GemmTile t = gemm_tile(N, K);
    const bool steps8 = (K / 32) % 4 == 0 && (reinterpret_cast<uintptr_t>(steps_base) & 7) == 0 &&
                        (stride_steps % 4) == 0;
    MoeFn fn = steps8 ? pick_moe_s<true>(t.gpw) : pick_moe_s<false>(t.gpw);
    if (!fn || t.waves > 16) return hipErrorInvalidConfiguration;
    const int P = T * topk;
    const int ntiles = (N + 15) / 16;
    // tiles of one expert spread over workgroups; about 1024 workgroups in all
    int per_expert = 1024 / (P > 0 ? P : 1);
    if (per_expert < 16) per_expert = 16;
    const int bx = ntiles < per_expert ? ntiles : per_expert;
    hipLaunchKernelGGL(fn, dim3(bx, P), dim3(64 * t.waves), 0, stream,
                       reinterpret_cast<const uint4 *>(codes_base), steps_base, stride_codes / 4,
                       stride_steps, N, K, X, ldx, dt, x_per_pair, ids, P, topk, slot_of,
                       n_experts, n_slots, row_scale, rows_out, dev_err);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float *rows, const float *route_w, int T, int topk, int N,
                              float *Y, hipStream_t stream) {
    const long total = (long)T * N;
    long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows,
                       route_w, T, topk, N, Y);
    return hipGetLastError();
}

}  // namespace w4
