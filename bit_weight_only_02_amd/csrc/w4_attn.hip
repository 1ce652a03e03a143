// Decode attention for one query token, split over the key/value cache, for
// gfx950.
//
// Source: the dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch", sections
// "Step 5 - Attention for One Token at a Time" (a grouped-query layout: eight
// query heads over a single key/value head, the cache cut into slices whose
// partial softmax results are merged) and "Step 7 - Fit the Full 131,072-Token
// Context" (the cache shape: one head of width 512, a slot per position on the
// full layers, a 512-slot ring on the sliding-window layers).  Here every
// cached row is streamed from memory once and used for all query heads.
//
// attn_split_kernel: workgroup w takes keys [w*C, min(L, (w+1)*C)); its waves
// take kU consecutive keys at a time, in turn.  Lane l holds dims
// [l*DPL, (l+1)*DPL) of q (pre-scaled by scale * log2 e), of the keys and values
// and of the accumulators of all kH heads, so one 16-byte load per lane reads a
// whole 1 KiB key row.  A score is the whole-wave sum of the lanes' partial
// dots (row shifts and broadcasts, then read from the last lane: the same value
// in every lane); each head keeps a running maximum m, a running sum l of
// 2^(s - m) and the accumulated values, rescaled when m grows.  The waves of a
// workgroup are merged in wave order into one partial {m, l, acc} per head.
// attn_merge_kernel: output (h, d) = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M)
// l_w over the partials (a running merge over each quarter of them, then the
// quarters in order), M the largest m_w.
#include <cmath>

#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

constexpr int kAttnH = 8;      // query heads per key/value head handled per pass
constexpr int kAttnWaves = 4;  // waves per workgroup
constexpr int kAttnU = 4;      // keys per wave step

template <int DPL>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K, long ldk,
    const uint16_t *__restrict__ V, long ldv, int H, int L, int C, float scale_log2,
    float *__restrict__ ws) {
    constexpr int D = 64 * DPL;
    __shared__ float sm[kAttnWaves][kAttnH], sl[kAttnWaves][kAttnH];
    __shared__ float sacc[kAttnWaves][kAttnH][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l0 = blockIdx.x * C, l1 = min(L, l0 + C);
    typedef unsigned short us_v __attribute__((ext_vector_type(DPL)));
    float qf[kAttnH][DPL];
#pragma unroll
    for (int h = 0; h < kAttnH; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d)
            qf[h][d] = h < H ? bf16_to_f32(q[h * D + lane * DPL + d]) * scale_log2 : 0.0f;
    float m[kAttnH], l[kAttnH], acc[kAttnH][DPL];
#pragma unroll
    for (int h = 0; h < kAttnH; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] = 0.0f;
    }
    for (int k0 = l0 + wave * kAttnU; k0 < l1; k0 += kAttnWaves * kAttnU) {
        // the step's keys and values, all requested before any is used
        // (keys past the range re-read the last one and get no weight)
        us_v kr[kAttnU], vr[kAttnU];
#pragma unroll
        for (int u = 0; u < kAttnU; ++u) {
            const int key = min(k0 + u, l1 - 1);
            kr[u] = *reinterpret_cast<const us_v *>(K + (long)key * ldk + lane * DPL);
            vr[u] = *reinterpret_cast<const us_v *>(V + (long)key * ldv + lane * DPL);
        }
        float s[kAttnU][kAttnH];
#pragma unroll
        for (int u = 0; u < kAttnU; ++u)
#pragma unroll
            for (int h = 0; h < kAttnH; ++h) {
                float t = 0.0f;
#pragma unroll
                for (int d = 0; d < DPL; ++d) t = __builtin_fmaf(qf[h][d], bf16_to_f32(kr[u][d]), t);
                t = lane_group_sum<64>(t);
                s[u][h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 63));
                if (k0 + u >= l1) s[u][h] = -INFINITY;
            }
#pragma unroll
        for (int h = 0; h < kAttnH; ++h) {
            float mn = m[h];
#pragma unroll
            for (int u = 0; u < kAttnU; ++u) mn = fmaxf(mn, s[u][h]);
            const float corr = exp2f(m[h] - mn);  // 0 on the first step (m = -inf)
            float p[kAttnU], ps = 0.0f;
#pragma unroll
            for (int u = 0; u < kAttnU; ++u) {
                p[u] = exp2f(s[u][h] - mn);  // 0 for keys past the range
                ps += p[u];
            }
            l[h] = l[h] * corr + ps;
#pragma unroll
            for (int d = 0; d < DPL; ++d) {
                float a = acc[h][d] * corr;
#pragma unroll
                for (int u = 0; u < kAttnU; ++u) a = __builtin_fmaf(p[u], bf16_to_f32(vr[u][d]), a);
                acc[h][d] = a;
            }
            m[h] = mn;
        }
    }
    // the waves of this workgroup merged in wave order
#pragma unroll
    for (int h = 0; h < kAttnH; ++h) {
        if (lane == 0) {
            sm[wave][h] = m[h];
            sl[wave][h] = l[h];
        }
#pragma unroll
        for (int d = 0; d < DPL; ++d) sacc[wave][h][lane * DPL + d] = acc[h][d];
    }
    __syncthreads();
    float *out = ws + (long)blockIdx.x * (2 * kAttnH + kAttnH * D);
    for (int i = threadIdx.x; i < kAttnH * D; i += 64 * kAttnWaves) {
        const int h = i / D, d = i % D;
        float M = -INFINITY;
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm[w][h]);
        float a = 0.0f, z = 0.0f;
        for (int w = 0; w < kAttnWaves; ++w) {
            const float c = sm[w][h] == -INFINITY ? 0.0f : exp2f(sm[w][h] - M);
            a += c * sacc[w][h][d];
            z += c * sl[w][h];
        }
        out[2 * kAttnH + i] = a;
        if (d == 0) {
            out[h] = M;
            out[kAttnH + h] = z;
        }
    }
}

// Merge: workgroup (h, 64-dim block) with 256 threads, thread (quarter qt,
// dim d): a running merge over slices qt, qt+4, ... (rescaled when the
// maximum grows), then the four quarters combined in order in LDS.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *__restrict__ ws, int S, int H, int D,
                                                         float *__restrict__ o) {
    __shared__ float pm[4][64], pa[4][64], pz[4][64];
    const int h = blockIdx.y, d = blockIdx.x * 64 + (threadIdx.x & 63), qt = threadIdx.x >> 6;
    const long stride = 2 * kAttnH + (long)kAttnH * D;
    float M = -INFINITY, a = 0.0f, z = 0.0f;
#pragma unroll 4
    for (int sidx = qt; sidx < S; sidx += 4) {
        const float *p = ws + sidx * stride;
        const float ms = p[h];
        if (ms == -INFINITY) continue;  // an empty slice
        const float mn = fmaxf(M, ms);
        const float c0 = exp2f(M - mn), c1 = exp2f(ms - mn);  // exp2(-inf) = 0 at the start
        a = a * c0 + c1 * p[2 * kAttnH + h * D + d];
        z = z * c0 + c1 * p[kAttnH + h];
        M = mn;
    }
    pm[qt][threadIdx.x & 63] = M;
    pa[qt][threadIdx.x & 63] = a;
    pz[qt][threadIdx.x & 63] = z;
    __syncthreads();
    if (qt == 0 && h < H) {
        const int t = threadIdx.x & 63;
        float MM = -INFINITY;
        for (int k = 0; k < 4; ++k) MM = fmaxf(MM, pm[k][t]);
        float A = 0.0f, Z = 0.0f;
        for (int k = 0; k < 4; ++k) {
            const float c = pm[k][t] == -INFINITY ? 0.0f : exp2f(pm[k][t] - MM);
            A += c * pa[k][t];
            Z += c * pz[k][t];
        }
        o[h * D + d] = A / Z;
    }
}

// Splits: about 32 keys each (8 per wave), at most 256 (one per CU): 131072
// positions took 155 us with 256 splits, 203 us with 512, 300 us with 1024; a
// 512-slot ring 21.5 us with 16 splits, 25 us with 64.
static int attn_splits(int L) {
    int S = (L + 31) / 32;
    if (S > 256) S = 256;
    if (S > L) S = L;
    return S < 1 ? 1 : S;
}

size_t attn_workspace(int H, int D, int L) {
    (void)H;
    return (size_t)attn_splits(L) * (2 * kAttnH + (size_t)kAttnH * D) * sizeof(float);
}

hipError_t launch_attn(const uint16_t *q, int H, int D, const uint16_t *K, long ldk, const uint16_t *V,
                       long ldv, int L, float scale, float *o, void *ws, hipStream_t stream) {
    const int S = attn_splits(L);
    const int C = (L + S - 1) / S;
    const float sl2 = scale * 1.4426950408889634f;  // log2 e
    float *w = static_cast<float *>(ws);
    switch (D) {
        case 512:
            hipLaunchKernelGGL(attn_split_kernel<8>, dim3(S), dim3(64 * kAttnWaves), 0, stream, q, K, ldk, V,
                               ldv, H, L, C, sl2, w);
            break;
        case 256:
            hipLaunchKernelGGL(attn_split_kernel<4>, dim3(S), dim3(64 * kAttnWaves), 0, stream, q, K, ldk, V,
                               ldv, H, L, C, sl2, w);
            break;
        default:
            return hipErrorInvalidConfiguration;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(D / 64, H), dim3(256), 0, stream, w, S, H, D, o);
    return hipGetLastError();
}

}  // namespace w4
