// MFMA engine of the small-M products (gfx950): shared by the plain small-M
// product and the expert-indexed product.  See w4_gemm_smallm.hip for the
// layout and the reasoning.
#pragma once

#include "w4_device.h"

namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ h8 make_h8(h2 a, h2 b, h2 c, h2 d) {
    h8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

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


// Shared memory of one engine instance.
struct SmallMShared {
    float part[2][16][64][4];  // [tile parity][wave][lane][j]
    int emax_s[16][16];        // [wave][row m]
    int flag_s[16];
    int scale_s[16];
};

// The engine: every wave of the workgroup calls it.  GPW: groups per wave
// (multiple of 4); STEPS8: the four steps of a round are read with one 8-byte
// load (K/32 a multiple of 4 and steps 8-byte aligned).  blockDim = 64*WK.
//   xrow(m): pointer to activation row m (m < M), read 8 values at a time at
//            column offsets that are multiples of 8;  xvec: those 16-byte
//            reads are aligned;
//   store(m, n, v): receives output (m, n) for m < M, n < N, already scaled
//            back from the staging power of two;
//   tiles tile_begin, tile_begin + tile_stride, ... of 16 rows are processed.
template <int GPW, bool STEPS8, class XRow, class Store>
__device__ __forceinline__ void smallm_engine(const uint4 *__restrict__ codes,
                                              const uint16_t *__restrict__ steps, int N, int K,
                                              XRow xrow, bool xvec, int dt, int M,
                                              int tile_begin, int tile_stride, Store store,
                                              SmallMShared &sh) {
    constexpr int ROUNDS = GPW / 4;
    auto &part = sh.part;
    auto &emax_s = sh.emax_s;
    auto &flag_s = sh.flag_s;
    auto &scale_s = sh.scale_s;
    const int G = K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int WK = blockDim.x >> 6;
    const int n_l = lane & 15, q = lane >> 4;
    const int g_begin = wave * GPW;
    const int ntiles = (N + 15) >> 4;

    // ---- stage this wave's A fragments: X[m][g*32 + 8q .. +7], m = lane % 16.
    // Two passes over the (L2-resident) activations: first the largest
    // exponent of each row over every wave's slice, then a second read that
    // converts straight into the fragments (one copy of the slice in registers).
    const int m = n_l;
    auto load_x = [&](int g) __attribute__((always_inline)) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < M && g < G) {
            const uint16_t *src = xrow(m) + g * 32 + 8 * q;
            if (xvec)
                v = *reinterpret_cast<const uint4 *>(src);
            else
                v = make_uint4(src[0] | ((uint32_t)src[1] << 16), src[2] | ((uint32_t)src[3] << 16),
                               src[4] | ((uint32_t)src[5] << 16), src[6] | ((uint32_t)src[7] << 16));
        }
        return v;
    };
    auto unpack_x = [&](uint4 v, float (&xv)[8]) __attribute__((always_inline)) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = act_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, dt);
    };
    int emax = -100000, bad = 0;
#pragma unroll 4
    for (int r = 0; r < GPW; ++r) {
        float xv[8];
        unpack_x(load_x(g_begin + r), xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!__builtin_isfinite(xv[e])) bad = 1;
            else if (xv[e] != 0.0f) emax = max(emax, f32_exponent(xv[e]));
        }
    }
    // largest exponent of row m over this wave's slice (lanes m, m+16, m+32, m+48)
    emax = max_across_lane_groups(emax);
    bad = wave_or_i32(bad);
    if (lane < 16) emax_s[wave][lane] = emax;
    if (lane == 0) flag_s[wave] = bad;
    lds_barrier();
    int rowmax = -100000;
    for (int w = 0; w < WK; ++w) rowmax = max(rowmax, emax_s[w][m]);
    const int s_m = (rowmax == -100000) ? 0 : 14 - rowmax;
    int lost = 0;
    h8 afrag[GPW];
#pragma unroll
    for (int r = 0; r < GPW; ++r) {
        float xv[8];
        unpack_x(load_x(g_begin + r), xv);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (xv[e] != 0.0f && f32_exponent(xv[e]) < rowmax - 28) lost = 1;
        // pair order (x0,x4),(x1,x5),(x2,x6),(x3,x7)
        h8 a;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            a[2 * p] = (_Float16)__builtin_ldexpf(xv[p], s_m);
            a[2 * p + 1] = (_Float16)__builtin_ldexpf(xv[p + 4], s_m);
        }
        afrag[r] = a;
        // keep each group's load next to its conversion (hoisting all of them
        // would need a second copy of the slice in registers)
        if (r % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    lost = wave_or_i32(lost);
    if (lane < 16 && wave == 0) scale_s[lane] = s_m;
    lds_barrier();  // everyone has read flag_s/emax_s
    if (lane == 0) flag_s[wave] |= lost;
    lds_barrier();
    int fallback = 0;
    for (int w = 0; w < WK; ++w) fallback |= flag_s[w];

    if (__builtin_amdgcn_readfirstlane(fallback)) {
        // Rare exact path: plain fp32 products and sums, one output per thread.
        for (int tile = tile_begin; tile < ntiles; tile += tile_stride) {
            for (int o = threadIdx.x; o < 16 * M; o += blockDim.x) {
                const int mm = o / 16, n = tile * 16 + (o % 16);
                if (n >= N) continue;
                float acc = 0.0f;
                for (int g = 0; g < G; ++g)
                    acc = __builtin_fmaf(group_dot_f32(codes[(long)n * G + g], xrow(mm) + g * 32, dt),
                                         bf16_to_f32(steps[(long)n * G + g]), acc);
                store(mm, n, acc);
            }
        }
        return;
    }

    // Per-lane constants of the D layout: rows m_j = 4q + j, column n_l.
    const h2 kSub = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 kInv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 kSub72 = {(_Float16)-72.0f, (_Float16)-72.0f};

    int parity = 0;
    for (int tile = tile_begin; tile < ntiles; tile += tile_stride, parity ^= 1) {
        const int row = min(tile * 16 + n_l, N - 1);  // clamped: loads stay in bounds
        const uint4 *crow = codes + (long)row * G;
        const uint16_t *srow = steps + (long)row * G;
        // Rounds of four groups, two deep: the next round's loads are issued
        // before the current one is multiplied.  The four bf16 steps of a round
        // travel packed in two registers.
        auto load_round = [&](int rd, uint4 &qr, uint2 &sr) __attribute__((always_inline)) {
            const int g0 = g_begin + 4 * rd;
            qr = crow[min(g0 + q, G - 1)];
            if (STEPS8 && g0 + 3 < G) {
                sr = *reinterpret_cast<const uint2 *>(srow + g0);
            } else {
                sr.x = srow[min(g0, G - 1)] | ((uint32_t)srow[min(g0 + 1, G - 1)] << 16);
                sr.y = srow[min(g0 + 2, G - 1)] | ((uint32_t)srow[min(g0 + 3, G - 1)] << 16);
            }
        };
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        uint4 qcur, qnext;
        uint2 scur, snext;
        load_round(0, qcur, scur);
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            if (rd + 1 < ROUNDS) load_round(rd + 1, qnext, snext);
            const int g0 = g_begin + 4 * rd;
            uint32_t w[4] = {qcur.x, qcur.y, qcur.z, qcur.w};
            transpose_lane_groups(w);
            const uint32_t sw[4] = {scur.x & 0xFFFFu, scur.x >> 16, scur.y & 0xFFFFu, scur.y >> 16};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int g = g0 + j;
                const uint32_t u = w[j] >> 8;
                const h2 p0 = as_h2((w[j] & 0x000F000Fu) | 0x64006400u) + kSub;
                const h2 p1 = as_h2((w[j] & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
                const h2 p2 = as_h2((u & 0x000F000Fu) | 0x64006400u) + kSub;
                const h2 p3 = as_h2((u & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
                const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag[4 * rd + j],
                                                                     make_h8(p0, p1, p2, p3), zero,
                                                                     0, 0, 0);
                const float st = (g < G) ? bf16_to_f32(sw[j]) : 0.0f;
                acc[0] = __builtin_fmaf(d[0], st, acc[0]);
                acc[1] = __builtin_fmaf(d[1], st, acc[1]);
                acc[2] = __builtin_fmaf(d[2], st, acc[2]);
                acc[3] = __builtin_fmaf(d[3], st, acc[3]);
            }
            if (rd + 1 < ROUNDS) { qcur = qnext; scur = snext; }
        }
        const int n = tile * 16 + n_l;
        if (WK == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 4 * q + j;
                if (mm < M && n < N) store(mm, n, __builtin_ldexpf(acc[j], -scale_s[mm]));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) part[parity][wave][lane][j] = acc[j];
            lds_barrier();
            for (int t = threadIdx.x; t < 256; t += blockDim.x) {
                const int ln = t & 63, j = t >> 6;
                const int mm = 4 * (ln >> 4) + j, nn = tile * 16 + (ln & 15);
                float s = 0.0f;
                for (int w = 0; w < WK; ++w) s += part[parity][w][ln][j];
                if (mm < M && nn < N) store(mm, nn, __builtin_ldexpf(s, -scale_s[mm]));
            }
            // The next tile writes the other half of part[]; the one after that
            // comes behind the next tile's barrier, by which time every thread
            // has finished reading this half.
        }
    }
}


}  // namespace w4
