// MFMA engine of the small-M products (gfx950): shared by the plain small-M
// product and the expert-indexed product.
//
// One v_mfma_f32_16x16x32_f16 multiplies one group of 32 codes of 16 weight
// rows (B operand) by the same 32 columns of 16 (padded) activation rows (A
// operand); its fp32 result is then scaled by the group's bf16 step, per weight
// row, exactly where the step applies.  Operands are exact fp16: the weights
// are c - 8 (the OR-into-1024 unpack of w4_device.h), and each activation row
// is fp16 as given, or bf16 staged as x * 2^s with a power of two per row and
// K-slice (undone once per output).
//
// Register layout (lane i, 0..63): A holds X[m = i%16][k-slots 8(i/16)..+7],
// B holds W[n = i%16][the same k-slots], D holds rows m = 4(i/16)..+3 of column
// n = i%16.  The k-slots of lane group q = i/16 are the eight codes of word q
// of the group, in the pair order (c0,c4),(c1,c5),(c2,c6),(c3,c7) that the
// unpack produces; the A operand is stored in LDS in that same order.
//
// Work split.  A workgroup of kSmallMWaves waves owns one K-slice of at most
// kSliceGroups groups.  It stages that slice of the activations once into LDS
// (direct-to-LDS loads, then one in-place conversion pass), and each wave then
// computes whole 16-row tiles over the slice: no reduction across waves.  All
// weight loads of a wave's first tile are issued before the staging starts, so
// their latency overlaps it.  Results of several K-slices are summed by a
// separate pass in slice order (deterministic).
#pragma once

#include "w4_device.h"

namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kSmallMWaves = 4;    // waves per workgroup
constexpr int kSliceGroups = 96;   // largest K-slice, in groups of 32 (96 KB of LDS)

// 4x4 transpose of words across the four 16-lane groups: on entry lane group
// Q holds words 0..3 of group Q in v[0..3]; on exit lane group q holds word q
// of groups 0..3 in v[0..3].
__device__ __forceinline__ void transpose_lane_groups(uint32_t (&v)[4]) {
    auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    v[2] = d[0];
    v[3] = d[1];
}

// Shared memory of one engine instance.  a[]: the staged A operand of the
// K-slice; chunk (gl, q, m) -- activation row m, columns 8q..8q+7 of slice
// group gl, in pair order -- sits at a[gl*64 + q*16 + m], so that lane
// i = 16q + m of a wave reads the chunk of group gl at a[gl*64 + i].
struct SmallMShared {
    uint4 a[kSliceGroups * 64];
    int emax[kSmallMWaves][16];
    int scale[16];
    int flag[2][kSmallMWaves];
};

// Host-side plan of a small-M launch.
struct SmallMPlan {
    int S;   // K-slices
    int Gs;  // groups per slice (a multiple of 4; the last slice may be shorter)
    int R;   // rounds of 4 groups whose loads a wave keeps in flight
};

__host__ __device__ inline SmallMPlan smallm_plan(int K) {
    const int G = K / 32;
    SmallMPlan p;
    p.S = (G + kSliceGroups - 1) / kSliceGroups;
    if (p.S < 1) p.S = 1;
    int gs = (G + p.S - 1) / p.S;
    gs = (gs + 3) / 4 * 4;
    if (gs < 4) gs = 4;
    p.Gs = gs;
    p.S = (G + gs - 1) / gs;
    if (p.S < 1) p.S = 1;
    const int nr = gs / 4;
    p.R = nr <= 4 ? 4 : nr <= 8 ? 8 : nr <= 16 ? 16 : 24;
    return p;
}

// The engine: every thread of the workgroup calls it (it has barriers).
//   R: rounds of 4 groups per batch of loads (template, so the load registers
//      are plain registers); STEPS8: the four steps of a round are read with
//      one 8-byte load (K/32 a multiple of 4, steps 8-byte aligned);
//   [g_lo, g_hi): the K-slice in groups, g_hi - g_lo <= kSliceGroups;
//   xrow(m): activation row m < M, read 8 values at a time at column offsets
//            that are multiples of 8; xvec: those reads are 16-byte aligned;
//   tiles tile_first + wave, + tile_stride, ... (16 rows each) are computed;
//   store(m, n, v): receives the slice's sum for output (m, n), m < M, n < N.
template <int R, bool STEPS8, class XRow, class Store>
__device__ __forceinline__ void smallm_engine(const uint4 *__restrict__ codes,
                                              const uint16_t *__restrict__ steps, int N, int K,
                                              int g_lo, int g_hi, XRow xrow, bool xvec, int dt,
                                              int M, int tile_first, int tile_stride, Store store,
                                              SmallMShared &sh) {
    const int G = K >> 5;
    const int ng = g_hi - g_lo;
    const int nr = (ng + 3) >> 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, q = lane >> 4;
    const int ntiles = (N + 15) >> 4;

    uint4 qr[R];
    uint2 sr[R];
    // Loads of rounds r0 .. r0+R-1 of one tile.  Lane (n, Q) reads the whole
    // 16-byte group g0+Q of row n; rows past N and groups past the slice are
    // clamped to valid addresses (their A operands are zero, their steps 0).
    auto load_rounds = [&](int tile, int r0) __attribute__((always_inline)) {
        const int row = min(tile * 16 + n_l, N - 1);
        const uint4 *crow = codes + (long)row * G;
        const uint16_t *srow = steps + (long)row * G;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r0 + r < nr) {
                const int g0 = g_lo + 4 * (r0 + r);
                qr[r] = crow[min(g0 + q, g_hi - 1)];
                if (STEPS8 && g0 + 3 < g_hi) {
                    sr[r] = *reinterpret_cast<const uint2 *>(srow + g0);
                } else {
                    const uint32_t s0 = srow[g0];
                    const uint32_t s1 = g0 + 1 < g_hi ? srow[g0 + 1] : 0u;
                    const uint32_t s2 = g0 + 2 < g_hi ? srow[g0 + 2] : 0u;
                    const uint32_t s3 = g0 + 3 < g_hi ? srow[g0 + 3] : 0u;
                    sr[r] = make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
                }
            }
        }
    };

    int tile = tile_first + wave;
    if (tile < ntiles) load_rounds(tile, 0);

    // ---- stage the slice of the activations into sh.a -----------------------
    // One direct-to-LDS instruction moves the 64 chunks of one slice group:
    // lane 16q + m brings X[m][8q .. 8q+7] of that group.  Rows m >= M and
    // groups past the slice read valid addresses and are overwritten below.
    const int nchunks = nr * 256;  // 4 groups x 64 chunks per round
    if (xvec) {
        const int mm = min(n_l, M - 1);
        for (int gl = wave; gl < nr * 4; gl += kSmallMWaves) {
            const int g = min(g_lo + gl, g_hi - 1);
            const uint16_t *src = xrow(mm) + g * 32 + 8 * q;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(&sh.a[gl * 64]), 16, 0, 0);
        }
        wait_vmcnt<0>();
    }
    lds_barrier();

    // Thread t owns chunks t, t + 256, ...: always activation row m = t % 16.
    const int m = tid & 15;
    auto raw_chunk = [&](int c) __attribute__((always_inline)) {
        if (xvec) return sh.a[c];
        const uint16_t *src = xrow(m) + (g_lo + (c >> 6)) * 32 + 8 * ((c >> 4) & 3);
        return make_uint4(src[0] | ((uint32_t)src[1] << 16), src[2] | ((uint32_t)src[3] << 16),
                          src[4] | ((uint32_t)src[5] << 16), src[6] | ((uint32_t)src[7] << 16));
    };
    auto chunk_valid = [&](int c) __attribute__((always_inline)) {
        return m < M && (c >> 6) < ng;
    };

    int rowmax = -100000, s_m = 0, bad = 0, lost = 0;
    if (dt != 0) {
        // bf16: largest exponent of row m over the slice, and inf/NaN
        int emax = -100000;
        for (int c = tid; c < nchunks; c += kSmallMWaves * 64) {
            if (!chunk_valid(c)) continue;
            const uint4 v = raw_chunk(c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bf16_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                if (!__builtin_isfinite(f)) bad = 1;
                else if (f != 0.0f) emax = max(emax, f32_exponent(f));
            }
        }
        emax = max_across_lane_groups(emax);
        bad = wave_or_i32(bad);
        if (lane < 16) sh.emax[wave][lane] = emax;
        if (lane == 0) sh.flag[0][wave] = bad;
        lds_barrier();
#pragma unroll
        for (int w = 0; w < kSmallMWaves; ++w) {
            rowmax = max(rowmax, sh.emax[w][m]);
            bad |= sh.flag[0][w];
        }
        s_m = rowmax == -100000 ? 0 : 14 - rowmax;
    }
    // Conversion in place: fp16 chunks are only permuted to pair order; bf16
    // chunks become fp16 x * 2^s_m (exact unless a value lies more than 2^28
    // below the row's largest; then the slice takes the exact fp32 path).
    if (!bad) {
        for (int c = tid; c < nchunks; c += kSmallMWaves * 64) {
            uint4 o = make_uint4(0, 0, 0, 0);
            if (chunk_valid(c)) {
                uint4 v = raw_chunk(c);
                if (dt != 0) {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    uint32_t hw[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        uint32_t h = 0;
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int i = 2 * p + e;
                            const float f = bf16_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
                            if (f != 0.0f && f32_exponent(f) < rowmax - 28) lost = 1;
                            const uint32_t b = __builtin_bit_cast(
                                uint16_t, (_Float16)__builtin_ldexpf(f, s_m));
                            h |= b << (16 * e);
                        }
                        hw[p] = h;
                    }
                    v = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                }
                // words (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
                o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
                o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
                o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
                o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
            }
            sh.a[c] = o;
        }
    }
    lost = wave_or_i32(lost | bad);
    if (lane == 0) sh.flag[1][wave] = lost;
    if (wave == 0 && lane < 16) sh.scale[lane] = s_m;
    lds_barrier();
    int fallback = 0;
#pragma unroll
    for (int w = 0; w < kSmallMWaves; ++w) fallback |= sh.flag[1][w];

    if (__builtin_amdgcn_readfirstlane(fallback)) {
        // Rare exact path: plain fp32 products and sums of the slice, one
        // output per lane of the wave.
        for (; tile < ntiles; tile += tile_stride) {
            for (int o = lane; o < 16 * M; o += 64) {
                const int mm = o >> 4, n = tile * 16 + (o & 15);
                if (n >= N) continue;
                float acc = 0.0f;
                for (int g = g_lo; g < g_hi; ++g)
                    acc = __builtin_fmaf(group_dot_f32(codes[(long)n * G + g], xrow(mm) + g * 32, dt),
                                         bf16_to_f32(steps[(long)n * G + g]), acc);
                store(mm, n, acc);
            }
        }
        return;
    }

    const h2 kSub = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 kInv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 kSub72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const h8 *A = reinterpret_cast<const h8 *>(sh.a);

    for (; tile < ntiles; tile += tile_stride) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int r0 = 0; r0 < nr; r0 += R) {
            if (r0 > 0) load_rounds(tile, r0);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r0 + r < nr) {
                    uint32_t w[4] = {qr[r].x, qr[r].y, qr[r].z, qr[r].w};
                    transpose_lane_groups(w);
                    const uint32_t sw[4] = {sr[r].x & 0xFFFFu, sr[r].x >> 16, sr[r].y & 0xFFFFu,
                                            sr[r].y >> 16};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const h8 a = A[(4 * (r0 + r) + j) * 64 + lane];
                        const uint32_t u = w[j] >> 8;
                        const h2 p0 = as_h2((w[j] & 0x000F000Fu) | 0x64006400u) + kSub;
                        const h2 p1 = as_h2((w[j] & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
                        const h2 p2 = as_h2((u & 0x000F000Fu) | 0x64006400u) + kSub;
                        const h2 p3 = as_h2((u & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
                        h8 b;
                        b[0] = p0[0]; b[1] = p0[1]; b[2] = p1[0]; b[3] = p1[1];
                        b[4] = p2[0]; b[5] = p2[1]; b[6] = p3[0]; b[7] = p3[1];
                        const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                        const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, zero, 0, 0, 0);
                        const float st = bf16_to_f32(sw[j]);
                        acc[0] = __builtin_fmaf(d[0], st, acc[0]);
                        acc[1] = __builtin_fmaf(d[1], st, acc[1]);
                        acc[2] = __builtin_fmaf(d[2], st, acc[2]);
                        acc[3] = __builtin_fmaf(d[3], st, acc[3]);
                    }
                }
            }
        }
        const int n = tile * 16 + n_l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int mm = 4 * q + j;
            if (mm < M && n < N) store(mm, n, __builtin_ldexpf(acc[j], -sh.scale[mm]));
        }
        if (tile + tile_stride < ntiles) load_rounds(tile + tile_stride, 0);
    }
}

}  // namespace w4
