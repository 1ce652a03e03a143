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
// attn_split_kernel: workgroup b's wave w takes the keys
// [(4b + w) * KPW, ...) (KPW a multiple of 16, at most L), 16 at a time.  The
// scores of a tile come from the matrix cores: S^T = K_tile Q^T with
// v_mfma_f32_16x16x32_bf16, the tile's 16 key rows as the A operand (one
// 16-byte piece of a key row per lane, straight from memory) and the query
// heads as the B operand (held in registers for the whole range; heads past H
// are zero).  Lane i then holds the scores of keys 4(i/16)..+3 of the tile for
// head i%16, so each head's running maximum is an in-lane maximum and two
// exchanges across lane groups, and its running sum is kept per lane and added
// over the four lane groups at the end.  The weighted sum of the values stays
// on the VALU in fp32 (the matrix cores would need the tile's values
// transposed, and bf16 weights would cost the output precision): lane i holds
// dims [i*DPL, (i+1)*DPL) of all heads' accumulators, reads each key's weights
// for the 8 heads from a small LDS buffer written by the score lanes, and
// multiplies them into the value row it loaded (one 16-byte load per lane per
// key).  The next tile's keys and values are requested while the current one is
// used: each key block right after its matrix instruction, each value row right
// after its multiply-adds (clamped to the last key of the range, which stays
// in the caches, when there is no next tile).  Value rows are read with
// non-temporal loads (each is used once: 155 -> 68 -> 56 us over 131072
// positions with that change); key rows with plain ones (a key line is read by
// two consecutive instructions, 16 rows x 64 bytes each, and non-temporal key
// loads measured slower).  The waves of a workgroup are then
// merged in wave order into one partial {m, l, acc} per head.
// attn_merge_kernel: output (h, d) = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s -
// M) l_s over the partials, M the largest m_s: the weights first (one pass
// over the partials' maxima), then sixteen interleaved sixteenths of the
// partials summed with all their loads in flight, then the sixteenths in
// order.
#include <cmath>

#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

constexpr int kAttnH = 8;      // query heads per key/value head handled per pass
constexpr int kAttnWaves = 4;  // waves per workgroup
constexpr int kAttnT = 16;     // keys per tile (the matrix instruction's rows)

typedef __bf16 attn_bf8 __attribute__((ext_vector_type(8)));
typedef float attn_f4 __attribute__((ext_vector_type(4)));
typedef unsigned attn_u2 __attribute__((ext_vector_type(2)));

// 16 bytes of a bf16 row (two 8-byte loads when rows may be only 8-byte
// aligned)
template <bool A16>
__device__ __forceinline__ u32x4 attn_load16(const uint16_t *p) {
    if constexpr (A16) {
        return *reinterpret_cast<const u32x4 *>(p);
    } else {
        const attn_u2 a = *reinterpret_cast<const attn_u2 *>(p), b = *reinterpret_cast<const attn_u2 *>(p + 4);
        return u32x4{a.x, a.y, b.x, b.y};
    }
}

template <int DPL, bool A16>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K, long ldk,
    const uint16_t *__restrict__ V, long ldv, int H, int L, int KPW, float scale_log2,
    float *__restrict__ ws) {
    constexpr int D = 64 * DPL;
    constexpr int NB = D / 32;  // matrix instructions per score tile
    typedef unsigned short vrow __attribute__((ext_vector_type(DPL)));
    __shared__ float pl[kAttnWaves][kAttnT][kAttnH];  // a tile's weights, [key][head]
    __shared__ float pc[kAttnWaves][kAttnH];           // the tile's rescale per head
    __shared__ float sm[kAttnWaves][kAttnH], sl[kAttnWaves][kAttnH];
    __shared__ float sacc[kAttnWaves][kAttnH][D];
    // (the wave index made uniform, so that the key range and every row
    // address computed from it stay in scalar registers)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const long k_lo = ((long)blockIdx.x * kAttnWaves + wave) * KPW;
    const int k_hi = (int)min((long)L, k_lo + KPW);  // k_lo >= k_hi: an empty wave
    // the heads as the B operand: lane i holds q[i%16][32t + 8(i/16) .. +7]
    u32x4 qb[NB];
    const uint16_t *qrow = q + (long)min(n, H - 1) * D + 8 * g;  // (rows past H read row H-1, then zeroed)
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t v = (uint32_t)qrow[32 * t + 2 * j] | ((uint32_t)qrow[32 * t + 2 * j + 1] << 16);
            qb[t][j] = n < H ? v : 0u;
        }
    float acc[kAttnH][DPL];
#pragma unroll
    for (int h = 0; h < kAttnH; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;  // head n's running maximum and this lane's part of its sum
    // two tiles in flight: slot 0 holds the even tiles of the range, slot 1
    // the odd ones; a slot's next tile is requested as soon as each piece of
    // it is used
    u32x4 ka0[NB], ka1[NB];
    vrow vr0[kAttnT], vr1[kAttnT];
    auto load_k = [&](u32x4 (&ka)[NB], int kt) __attribute__((always_inline)) {
        const uint16_t *kp = K + (long)min(kt + n, k_hi - 1) * ldk + 8 * g;
#pragma unroll
        for (int t = 0; t < NB; ++t) ka[t] = attn_load16<A16>(kp + 32 * t);
    };
    auto load_v = [&](vrow (&vr)[kAttnT], int kt) __attribute__((always_inline)) {
        const uint16_t *vp = V + lane * DPL;
#pragma unroll
        for (int j = 0; j < kAttnT; ++j) vr[j] = __builtin_nontemporal_load(reinterpret_cast<const vrow *>(vp + (long)min(kt + j, k_hi - 1) * ldv));
    };
    // one tile: keys [k0, k0 + 16) from slot (ka, vr), whose loads then move
    // on to the tile at nx (clamped to the range's last key past its end)
    auto tile = [&](u32x4 (&ka)[NB], vrow (&vr)[kAttnT], int k0, int nx) __attribute__((always_inline)) {
        // scores: S^T[key 4g + r][head n] in s[r]
        attn_f4 s = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint16_t *kp = K + (long)min(nx + n, k_hi - 1) * ldk + 8 * g;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(attn_bf8, ka[t]),
                                                        __builtin_bit_cast(attn_bf8, qb[t]), s, 0, 0, 0);
            ka[t] = attn_load16<A16>(kp + 32 * t);
        }
        // the tile's online-softmax step for head n (keys past the range get
        // no weight; the tile holds at least one key of the range)
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = k0 + 4 * g + r < k_hi ? s[r] * scale_log2 : -INFINITY;
        float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        tm = fmaxf(tm, __shfl_xor(tm, 16, kWave));
        tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
        const float mn = fmaxf(m, tm);
        const float corr = exp2f(m - mn);  // 0 on the first tile (m = -inf)
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = exp2f(sc[r] - mn);
        lsum = lsum * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m = mn;
        if (n < kAttnH) {
#pragma unroll
            for (int r = 0; r < 4; ++r) pl[wave][4 * g + r][n] = pr[r];
            if (g == 0) pc[wave][n] = corr;
        }
        // the values: acc[h][.] = acc[h][.] * corr[h] + sum_j p[j][h] V[j][.]
        {
            const float4 c0 = *reinterpret_cast<const float4 *>(&pc[wave][0]);
            const float4 c1 = *reinterpret_cast<const float4 *>(&pc[wave][4]);
            const float cr[kAttnH] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int h = 0; h < kAttnH; ++h)
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[h][d] *= cr[h];
        }
        const uint16_t *vp = V + lane * DPL;
#pragma unroll
        for (int j = 0; j < kAttnT; ++j) {
            const float4 p0 = *reinterpret_cast<const float4 *>(&pl[wave][j][0]);
            const float4 p1 = *reinterpret_cast<const float4 *>(&pl[wave][j][4]);
            const float pj[kAttnH] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            float vf[DPL];
#pragma unroll
            for (int d = 0; d < DPL; ++d) vf[d] = bf16_to_f32(vr[j][d]);
#pragma unroll
            for (int h = 0; h < kAttnH; ++h)
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[h][d] = __builtin_fmaf(pj[h], vf[d], acc[h][d]);
            vr[j] = __builtin_nontemporal_load(reinterpret_cast<const vrow *>(vp + (long)min(nx + j, k_hi - 1) * ldv));
        }
    };
    if (k_lo < k_hi) {
        const int kl = (int)k_lo;
        load_k(ka0, kl);
        load_v(vr0, kl);
        load_k(ka1, kl + kAttnT);
        load_v(vr1, kl + kAttnT);
        for (int k0 = kl; k0 < k_hi; k0 += 2 * kAttnT) {
            tile(ka0, vr0, k0, k0 + 2 * kAttnT);
            if (k0 + kAttnT >= k_hi) break;
            tile(ka1, vr1, k0 + kAttnT, k0 + 3 * kAttnT);
        }
    }
    // head n's sum over the four lane groups; the waves merged in wave order
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    if (lane < kAttnH) {
        sm[wave][lane] = m;
        sl[wave][lane] = lsum;
    }
#pragma unroll
    for (int h = 0; h < kAttnH; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d) sacc[wave][h][lane * DPL + d] = acc[h][d];
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

// Merge: workgroup (64-dim block, head h) of 1024 threads.  Every load is
// issued first: thread (w, d) its sixteenth of the partials' values for
// (h, d) -- s = w, w + 16, ... -- and thread s < S partial s's maximum and sum.
// Then M = the largest m_s, c_s = 2^(m_s - M) (0 for an empty partial), Z =
// sum_s c_s l_s (a fixed-order sum within each wave, then the waves in order),
// each thread's sum of c_s acc_s[h][d], and the sixteen sums in order.
constexpr int kMergeThreads = 1024;
constexpr int kMergeParts = kMergeThreads / 64;
constexpr int kMaxSplits = 256;

__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float *__restrict__ ws, int S, int H,
                                                                   int D, float *__restrict__ o) {
    __shared__ float cs[kMaxSplits];
    __shared__ float pa[kMergeParts][64];
    __shared__ float red[kMergeParts], redz[kMergeParts];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int d = blockIdx.x * 64 + lane;
    const long stride = 2 * kAttnH + (long)kAttnH * D;
    constexpr int kPer = kMaxSplits / kMergeParts;
    float v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int sidx = w + kMergeParts * k;
        v[k] = sidx < S ? ws[sidx * stride + 2 * kAttnH + (long)h * D + d] : 0.0f;
    }
    const float ms = tid < S ? ws[tid * stride + h] : -INFINITY;
    const float ls = tid < S ? ws[tid * stride + kAttnH + h] : 0.0f;
    float mx = ms;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    if (lane == 0) red[w] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int k = 1; k < kMergeParts; ++k) M = fmaxf(M, red[k]);
    const float c = ms == -INFINITY ? 0.0f : exp2f(ms - M);
    if (tid < S) cs[tid] = c;
    const float zw = lane_group_sum<64>(c * ls);  // the wave's sum, complete in its last lane
    if (lane == 63) redz[w] = zw;
    __syncthreads();
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int sidx = w + kMergeParts * k;
        if (sidx < S) a = __builtin_fmaf(cs[sidx], v[k], a);
    }
    pa[w][lane] = a;
    __syncthreads();
    if (w == 0 && h < H) {
        float A = 0.0f, Z = 0.0f;
#pragma unroll
        for (int k = 0; k < kMergeParts; ++k) {
            A += pa[k][lane];
            Z += redz[k];
        }
        o[(long)h * D + d] = A / Z;
    }
}

// Work split: tiles of 16 keys, about L / 1024 keys per wave (so that
// 256 workgroups of 4 waves cover the cache), at most 256 workgroups.
static void attn_plan(int L, int *S, int *kpw) {
    const int waves = kMaxSplits * kAttnWaves;
    const int per = (L + waves - 1) / waves;
    int k = (per + kAttnT - 1) / kAttnT * kAttnT;
    if (k < kAttnT) k = kAttnT;
    *kpw = k;
    *S = (L + kAttnWaves * k - 1) / (kAttnWaves * k);
    if (*S < 1) *S = 1;
}

size_t attn_workspace(int H, int D, int L) {
    (void)H;
    int S = 0, kpw = 0;
    attn_plan(L, &S, &kpw);
    return (size_t)S * (2 * kAttnH + (size_t)kAttnH * D) * sizeof(float);
}

hipError_t launch_attn(const uint16_t *q, int H, int D, const uint16_t *K, long ldk, const uint16_t *V,
                       long ldv, int L, float scale, float *o, void *ws, hipStream_t stream) {
    int S = 0, kpw = 0;
    attn_plan(L, &S, &kpw);
    if (S > kMaxSplits) return hipErrorInvalidConfiguration;
    const float sl2 = scale * 1.4426950408889634f;  // log2 e
    float *w = static_cast<float *>(ws);
    const bool a16 = (reinterpret_cast<uintptr_t>(K) & 15) == 0 && (ldk & 7) == 0;
    switch (D) {
        case 512:
            hipLaunchKernelGGL((attn_split_kernel<8, true>), dim3(S), dim3(64 * kAttnWaves), 0, stream, q, K, ldk,
                               V, ldv, H, L, kpw, sl2, w);
            break;
        case 256:
            if (a16)
                hipLaunchKernelGGL((attn_split_kernel<4, true>), dim3(S), dim3(64 * kAttnWaves), 0, stream, q, K,
                                   ldk, V, ldv, H, L, kpw, sl2, w);
            else
                hipLaunchKernelGGL((attn_split_kernel<4, false>), dim3(S), dim3(64 * kAttnWaves), 0, stream, q,
                                   K, ldk, V, ldv, H, L, kpw, sl2, w);
            break;
        default:
            return hipErrorInvalidConfiguration;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(D / 64, H), dim3(kMergeThreads), 0, stream, w, S, H, D, o);
    return hipGetLastError();
}

}  // namespace w4
