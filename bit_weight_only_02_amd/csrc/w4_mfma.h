// MFMA engine of the small-M products (gfx950): shared by the plain small-M
// product and the expert-indexed product.
//
// One v_mfma_f32_16x16x32_f16 multiplies one group of 32 codes of 16 weight
// rows (B operand) by the same 32 columns of up to 16 activation rows (A
// operand); its fp32 result is then scaled by the group's bf16 step, per weight
// row, exactly where the step applies.  Operands are exact fp16: the weights
// are (c - 8) * 2^-24 -- each nibble shifted to the low bits and masked is the
// fp16 subnormal c * 2^-24, and one packed subtract of 8 * 2^-24 follows --
// and each activation row is fp16 as given, or bf16 staged as x * 2^s with a
// power of two per row and K-slice; both scalings are undone once per output.
//
// Register layout (lane i, 0..63): A holds X[m = i%16][k-slots 8(i/16)..+7],
// B holds W[n = i%16][the same k-slots], D holds rows m = 4(i/16)..+3 of column
// n = i%16.  The k-slots of lane group q = i/16 are the eight codes of word q
// of the group, in the pair order (c0,c4),(c1,c5),(c2,c6),(c3,c7) that the
// unpack produces; the A operand is stored in LDS in that same order.  Rows
// m >= M of A hold whatever is in LDS: they only reach rows m >= M of D, which
// are never stored.
//
// Work split.  A workgroup of kSmallMWaves waves owns one K-slice.  It stages
// that slice of the activations once into LDS (direct-to-LDS loads, then one
// conversion pass), for Mp = M rounded up to a power of two rows, so that small
// M needs little LDS.  KW waves share a 16-row tile, each taking a contiguous
// run of the slice's rounds (4 groups each), and their partial tiles are added
// in LDS in wave order.  The plan picks KW and the number of K-slices so that
// the chip holds about 16 waves per CU (a thin product is latency-bound: the
// more independent waves, the more weight bytes in flight) without splitting K
// across workgroups unless a wave would otherwise run a long serial chain of
// rounds (the cross-workgroup sum costs a few memory round trips).  All weight
// loads of a wave's first tile are issued before the staging starts, so their
// latency overlaps it.  Results of several K-slices are summed in slice order
// (deterministic) by the caller.
#pragma once

#include "w4_device.h"

namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kSmallMWaves = 4;           // waves per workgroup
constexpr int kSmallMLdsA = 96 * 1024;    // largest staged A operand, bytes
constexpr int kSmallMLdsFast = 48 * 1024; // staged A per workgroup that leaves room for 3 per CU
constexpr long kSmallMTargetWaves = 4096; // 16 waves per CU on 256 CUs
constexpr int kSmallMMaxRounds = 8;       // rounds per wave above which K is split further
constexpr long kSmallMTargetGroups = 768; // workgroups: 3 per CU, each looping over its tiles
constexpr long kSmallMWideGroups = 256;   // the same for 8 or more rows with one wave per tile

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

// Static shared memory of one engine instance; the staged A operand lives in
// dynamic shared memory (smallm_plan().lds_a bytes): chunk (gl, q, m) --
// activation row m, columns 8q..8q+7 of slice group gl, in pair order -- at
// uint4 index (gl*4 + q)*Mp + m.
struct SmallMShared {
    f4 part[kSmallMWaves][64];            // per-wave partial tiles
    uint32_t mx[kSmallMWaves][16];        // per-row largest |x| (bf16 bits)
    uint32_t mn[kSmallMWaves][16];        // per-row smallest nonzero |x| - 1
    int scale[16];
    int flag[kSmallMWaves];
};

// Host-side plan of a small-M launch.
struct SmallMPlan {
    int S;       // K-slices
    int Gs;      // groups per slice (a multiple of 4; the last slice may be shorter)
    int R;       // rounds of 4 groups whose loads a wave keeps in flight
    int KW;      // waves per tile (1, 2 or 4)
    int mp_log2; // log2 of the staged rows Mp
    int lds_a;   // dynamic shared memory bytes
};

// M: activation rows (largest per engine pass); units: independent problems
// (experts) that run in the same launch; lds_budget: bytes of staged A per
// workgroup; split: more K-slices may be used to reach the wave target.
inline SmallMPlan smallm_plan(int N, int K, int M, int units, int lds_budget = kSmallMLdsA,
                              bool split = false) {
    const int G = K / 32;
    SmallMPlan p;
    int mp = 1, lg = 0;
    while (mp < M) { mp <<= 1; ++lg; }
    p.mp_log2 = lg;
    const long U = units > 0 ? units : 1;
    const long ntiles = (N + 15) / 16;
    const int nr_full = (G + 3) / 4;                        // rounds of 4 groups
    const int max_gs = lds_budget / (64 * mp) / 4 * 4;      // one group = 4*Mp chunks of 16 bytes
    // waves per tile: up to 4 while each wave keeps at least one round --
    // except, when splitting is allowed, for 8 or more activation rows over
    // enough tiles to give every wave of the chip its own: each workgroup then
    // stages its (large) activation block once and its waves take separate
    // tiles (measured 1.6x faster for 16 x 16384 x 1536)
    p.KW = 1;
    const bool wide = split && mp >= 8 && ntiles * U >= 4 * 256;
    if (split) {
        while (!wide && p.KW < kSmallMWaves && nr_full >= 2 * p.KW) p.KW *= 2;
    } else {
        // (expert launches: many units, each staging the rows of the largest
        // pass; more waves per tile only while the launch is small)
        while (p.KW < kSmallMWaves && ntiles * U * p.KW < 1024 && nr_full >= 4 * p.KW) p.KW *= 2;
    }
    int S = max_gs > 0 ? (G + max_gs - 1) / max_gs : G;
    if (split && !wide && (nr_full + S * p.KW - 1) / (S * p.KW) > kSmallMMaxRounds &&
        ntiles * U * S * p.KW < kSmallMTargetWaves) {
        // long serial chains on too few waves: more slices, down to about
        // kSmallMMaxRounds / 2 rounds per wave or the wave target
        const long want = (kSmallMTargetWaves + ntiles * U * p.KW - 1) / (ntiles * U * p.KW);
        const int s_rounds = (nr_full + p.KW * kSmallMMaxRounds / 2 - 1) / (p.KW * kSmallMMaxRounds / 2);
        const int s_new = (int)(want < s_rounds ? want : s_rounds);
        if (s_new > S) S = s_new;
    }
    if (S < 1) S = 1;
    int gs = (G + S - 1) / S;
    gs = (gs + 3) / 4 * 4;
    if (gs < 4) gs = 4;
    p.Gs = gs;
    p.S = (G + gs - 1) / gs;
    if (p.S < 1) p.S = 1;
    const int nr = gs / 4;
    while (p.KW > 1 && nr < p.KW) p.KW /= 2;
    const int rpw = (nr + p.KW - 1) / p.KW;
    // rounds per batch of loads: exactly a wave's rounds where an instance
    // exists (straight-line code), else the next larger one
    p.R = rpw <= 3 ? (rpw == 3 ? 3 : 4) : rpw <= 4 ? 4 : rpw <= 6 ? 6 : rpw <= 8 ? 8 : rpw <= 12 ? 12 : rpw <= 16 ? 16 : 24;
    const int chunks = nr * 4 * 4 * mp;
    p.lds_a = (chunks + 63) / 64 * 64 * 16;
    return p;
}

// The engine: every thread of the workgroup calls it (it has barriers).
//   R: rounds of 4 groups per batch of loads (template, so the load registers
//      are plain registers); STEPS8: the four steps of a round are read with
//      one 8-byte load (K/32 a multiple of 4, steps 8-byte aligned);
//   [g_lo, g_hi): the K-slice in groups (4*Mp*ceil4(g_hi-g_lo) chunks must fit
//      the dynamic LDS A, rounded up to 64 chunks);
//   xrow(m): activation row m < M, read 8 values at a time at column offsets
//            that are multiples of 8; xvec: those reads are 16-byte aligned;
//   M <= 2^mp_log2 <= 16; KW divides kSmallMWaves;
//   tile groups tg_first, + tg_stride, ... are computed, kSmallMWaves/KW
//            tiles of 16 rows each;
//   store(m, n, v): receives the slice's sum for output (m, n), m < M, n < N.
template <int R, bool STEPS8, class XRow, class Store>
__device__ __forceinline__ void smallm_engine(const uint4 *__restrict__ codes,
                                              const uint16_t *__restrict__ steps, int N, int K,
                                              int g_lo, int g_hi, XRow xrow, bool xvec, int dt,
                                              int M, int mp_log2, int KW, int tg_first,
                                              int tg_stride, Store store, SmallMShared &sh,
                                              uint4 *__restrict__ A) {
    const int G = K >> 5;
    const int ng = g_hi - g_lo;
    const int nr = (ng + 3) >> 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_l = lane & 15, q = lane >> 4;
    const int ntiles = (N + 15) >> 4;
    const int tpw = kSmallMWaves / KW;             // tiles per step of the workgroup
    const int kp = wave % KW, tsub = wave / KW;    // K-part and tile of this wave
    const int rpw = (nr + KW - 1) / KW;
    const int rb = min(nr, kp * rpw), re = min(nr, rb + rpw);
    const int mmask = (1 << mp_log2) - 1;

    uint4 qr[R];
    uint2 sr[R];
    // Loads of rounds r0 .. r0+R-1 of one tile (r0 < re).  Lane (n, Q) reads
    // the whole 16-byte group g0+Q of row n; rows past N and groups past the
    // slice are clamped to valid addresses (their A operands are zero, their
    // steps 0).  All R rounds are requested, those past re as copies of round
    // re - 1 (never used), with no branch between the loads: the compiler then
    // knows how many loads are in flight and waits for each round alone, not
    // for all of them at the first use.  With STEPS8 every round of a slice is
    // whole (K/32 and the slice length are multiples of 4), so its four steps
    // are one 8-byte load.
    auto load_rounds = [&](int tile, int r0) __attribute__((always_inline)) {
        const int row = min(tile * 16 + n_l, N - 1);
        const uint4 *crow = codes + (long)row * G;
        const uint16_t *srow = steps + (long)row * G;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int g0 = g_lo + 4 * min(r0 + r, re - 1);
            qr[r] = crow[min(g0 + q, g_hi - 1)];
            if constexpr (STEPS8) {
                sr[r] = *reinterpret_cast<const uint2 *>(srow + g0);
            } else {
                const uint32_t s0 = srow[g0];
                const uint32_t t1 = srow[min(g0 + 1, g_hi - 1)];
                const uint32_t t2 = srow[min(g0 + 2, g_hi - 1)];
                const uint32_t t3 = srow[min(g0 + 3, g_hi - 1)];
                const uint32_t s1 = g0 + 1 < g_hi ? t1 : 0u;
                const uint32_t s2 = g0 + 2 < g_hi ? t2 : 0u;
                const uint32_t s3 = g0 + 3 < g_hi ? t3 : 0u;
                sr[r] = make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
            }
        }
        // load instructions issued (wave-uniform)
        return STEPS8 ? 2 * R : 5 * R;
    };

    // ---- stage the slice of the activations into A ------------------------
    // Chunk c = (gl*4 + q)*Mp + m.  Every lane of a direct-to-LDS instruction
    // moves one chunk; chunks of rows >= M, of groups past the slice and past
    // the last chunk read clamped valid addresses (their LDS is either never
    // used, overwritten with zeros below, or padding).  The activations go
    // out first and the first tile's weights right behind them: a wave's
    // loads come back in issue order, so the staging below waits only for
    // its own chunks while the weights are still in flight.
    const int nchunks = nr << (mp_log2 + 4);
    // (A is read and written through an LDS-typed pointer: through the generic
    // one these are flat accesses, which also wait for every outstanding
    // global load, the weights included)
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    lds_u32x4 *AL = (lds_u32x4 *)A;
    const int m = tid & mmask;
    if (!xvec) {
        // rows that are not 16-byte aligned: 16-bit loads, written to LDS as
        // they are before any weight load is requested, so that nothing below
        // waits for the weights (the chunk's row is m: 256 is a multiple of Mp)
        for (int c = tid; c < nchunks; c += kSmallMWaves * 64) {
            const int gl = min(c >> (mp_log2 + 2), ng - 1);
            const uint16_t *src = xrow(min(m, M - 1)) + (g_lo + gl) * 32 + 8 * ((c >> mp_log2) & 3);
            AL[c] = u32x4{src[0] | ((uint32_t)src[1] << 16), src[2] | ((uint32_t)src[3] << 16),
                          src[4] | ((uint32_t)src[5] << 16), src[6] | ((uint32_t)src[7] << 16)};
        }
    } else {
        for (int c0 = wave * 64; c0 < nchunks; c0 += kSmallMWaves * 64) {
            const int c = c0 + lane;
            const int m = min(c & mmask, M - 1);
            const int qq = (c >> mp_log2) & 3;
            const int gl = min(c >> (mp_log2 + 2), ng - 1);
            const uint16_t *src = xrow(m) + (g_lo + gl) * 32 + 8 * qq;
            // (the asm form: the compiler would make every later LDS read wait
            // for all outstanding loads, weights included; the wait for these
            // chunks is the explicit one below)
            lds_dma16(src, A + c0);
        }
    }
    asm volatile("" ::: "memory");  // (the weight loads stay behind the activation loads)
    int tg = tg_first;
    // (the load instructions younger than the activation loads: waiting for at
    // most that many to be outstanding leaves the activation loads complete)
    int wloads = 0;
    if (tg * tpw + tsub < ntiles && rb < re) wloads = load_rounds(tg * tpw + tsub, rb);
    if (xvec) wait_vmcnt_upto(wloads);
    lds_barrier();

    // Thread t visits chunks t, t + 256, ...: always activation row t & mmask.
    // Every chunk is in LDS by now, by either path.
    auto raw_chunk = [&](int c) __attribute__((always_inline)) {
        const u32x4 v = AL[c];
        return make_uint4(v.x, v.y, v.z, v.w);
    };

    int s_m = 0, fallback = 0;
    if (dt != 0) {
        // bf16: per row, the largest magnitude and the smallest nonzero one
        // (bf16 magnitudes order like their values); zero maps to 0xFFFF.
        u16x2 vmx = {0, 0}, vmn = {0xFFFF, 0xFFFF};
        const u16x2 one = {1, 1};
        if (m < M) {
            // four chunks per step, their reads issued together
            for (int c0 = tid; c0 < nchunks; c0 += 4 * kSmallMWaves * 64) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = raw_chunk(min(c0 + u * kSmallMWaves * 64, nchunks - 1));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = c0 + u * kSmallMWaves * 64;
                    const bool ok = c < nchunks && (c >> (mp_log2 + 2)) < ng;
                    const uint32_t w4v[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u16x2 mag = __builtin_bit_cast(u16x2, w4v[i] & 0x7FFF7FFFu);
                        vmx = ok ? __builtin_elementwise_max(vmx, mag) : vmx;
                        vmn = ok ? __builtin_elementwise_min(vmn, mag - one) : vmn;
                    }
                }
            }
        }
        uint32_t mx = max((uint32_t)vmx[0], (uint32_t)vmx[1]);
        uint32_t mn = min((uint32_t)vmn[0], (uint32_t)vmn[1]);
        for (int off = 1 << mp_log2; off < 64; off <<= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, kWave));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, kWave));
        }
        if (lane <= mmask) {
            sh.mx[wave][lane] = mx;
            sh.mn[wave][lane] = mn;
        }
        lds_barrier();
        mx = sh.mx[0][m];
        mn = sh.mn[0][m];
#pragma unroll
        for (int w = 1; w < kSmallMWaves; ++w) {
            mx = max(mx, sh.mx[w][m]);
            mn = min(mn, sh.mn[w][m]);
        }
        // Row m is staged exactly as fp16 x * 2^s with s = 14 - emax when no
        // value is inf/NaN or a bf16 subnormal and every nonzero value lies
        // within 2^31 of the largest (fp16 then holds its 8 significant bits,
        // as a normal or subnormal number).
        if (m < M && mn != 0xFFFFu) {
            const int emax = (int)(mx >> 7), emin = (int)((mn + 1) >> 7);
            const bool bad = mx >= 0x7F80u || emin == 0 || emin + 31 < emax;
            fallback = bad ? 1 : 0;
            s_m = 141 - emax;   // 14 - (emax - 127)
        }
    }
    fallback = wave_or_i32(fallback);
    if (lane == 0) sh.flag[wave] = fallback;
    if (wave == 0 && lane <= mmask) sh.scale[lane] = s_m;
    // Conversion in place: fp16 chunks are only permuted to pair order; bf16
    // chunks become fp16 x * 2^s_m; chunks of groups past the slice become 0.
    if (m < M) {
        // four chunks per step: reads first, then the converted chunks
        for (int c0 = tid; c0 < nchunks; c0 += 4 * kSmallMWaves * 64) {
            uint4 vv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) vv[u] = raw_chunk(min(c0 + u * kSmallMWaves * 64, nchunks - 1));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * kSmallMWaves * 64;
            if (c >= nchunks) break;
            uint4 o = make_uint4(0, 0, 0, 0);
            if ((c >> (mp_log2 + 2)) < ng) {
                const uint4 v = vv[u];
                if (dt != 0) {
                    // x_i is half (i & 1) of word i >> 1; output word p = (x_p, x_{p+4})
                    auto f = [&](uint32_t w, int hi) __attribute__((always_inline)) {
                        return __builtin_ldexpf(__uint_as_float(hi ? (w & 0xFFFF0000u) : (w << 16)),
                                                s_m);
                    };
                    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.x, 0), f(v.z, 0)));
                    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.x, 1), f(v.z, 1)));
                    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.y, 0), f(v.w, 0)));
                    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.y, 1), f(v.w, 1)));
                } else {
                    // words (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
                    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
                    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
                    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
                    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
                }
            }
            AL[c] = u32x4{o.x, o.y, o.z, o.w};
            }
        }
    }
    lds_barrier();
    fallback = 0;
#pragma unroll
    for (int w = 0; w < kSmallMWaves; ++w) fallback |= sh.flag[w];

    if (__builtin_amdgcn_readfirstlane(fallback)) {
        // Rare exact path: plain fp32 products and sums of the slice, one
        // output per lane, by the first wave of each tile.
        if (kp != 0) return;
        for (; tg * tpw < ntiles; tg += tg_stride) {
            const int tile = tg * tpw + tsub;
            if (tile >= ntiles) continue;
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

    const h2 k8 = __builtin_bit_cast(h2, 0x00080008u);  // 8 * 2^-24 in both halves
    const __attribute__((address_space(3))) h8 *Ah = (const __attribute__((address_space(3))) h8 *)A;
    const int arow = (q << mp_log2) + (n_l & mmask);   // this lane's A chunk within a group

    for (; tg * tpw < ntiles; tg += tg_stride) {
        const int tile = tg * tpw + tsub;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (tile < ntiles) {
            // one round: its 4 groups on the matrix cores, the steps applied per group
            auto round = [&](const uint4 &qw, const uint2 &sw, int rr) __attribute__((always_inline)) {
                h8 a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = Ah[((4 * rr + j) << (mp_log2 + 2)) + arow];
                uint32_t w[4] = {qw.x, qw.y, qw.z, qw.w};
                transpose_lane_groups(w);
                h8 b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // (c - 8) * 2^-24 for the pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7)
                    const h2 p0 = as_h2(w[j] & 0x000F000Fu) - k8;
                    const h2 p1 = as_h2((w[j] >> 4) & 0x000F000Fu) - k8;
                    const h2 p2 = as_h2((w[j] >> 8) & 0x000F000Fu) - k8;
                    const h2 p3 = as_h2((w[j] >> 12) & 0x000F000Fu) - k8;
                    b[j][0] = p0[0]; b[j][1] = p0[1]; b[j][2] = p1[0]; b[j][3] = p1[1];
                    b[j][4] = p2[0]; b[j][5] = p2[1]; b[j][6] = p3[0]; b[j][7] = p3[1];
                }
                const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                f4 d[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b[j], zero, 0, 0, 0);
                const float st[4] = {bf16_to_f32(sw.x & 0xFFFFu), bf16_to_f32(sw.x >> 16),
                                     bf16_to_f32(sw.y & 0xFFFFu), bf16_to_f32(sw.y >> 16)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[0] = __builtin_fmaf(d[j][0], st[j], acc[0]);
                    acc[1] = __builtin_fmaf(d[j][1], st[j], acc[1]);
                    acc[2] = __builtin_fmaf(d[j][2], st[j], acc[2]);
                    acc[3] = __builtin_fmaf(d[j][3], st[j], acc[3]);
                }
            };
            if (rb + R == re) {
                // exactly one batch of R rounds: straight-line code, so that the
                // rounds can overlap (a guard per round would cut them apart)
#pragma unroll
                for (int r = 0; r < R; ++r) round(qr[r], sr[r], rb + r);
            } else {
                for (int r0 = rb; r0 < re; r0 += R) {
                    if (r0 > rb) load_rounds(tile, r0);
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (r0 + r < re) round(qr[r], sr[r], r0 + r);
                }
            }
        }
        if (KW > 1) {
            // partial tiles of the KW waves of a tile, added in wave order
            sh.part[wave][lane] = acc;
            lds_barrier();
            if (kp == 0) {
                for (int k = 1; k < KW; ++k) {
                    const f4 o = sh.part[wave + k][lane];
                    acc[0] += o[0];
                    acc[1] += o[1];
                    acc[2] += o[2];
                    acc[3] += o[3];
                }
            }
            lds_barrier();
        }
        const int n = tile * 16 + n_l;
        if (kp == 0 && tile < ntiles) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 4 * q + j;
                if (mm < M && n < N) store(mm, n, __builtin_ldexpf(acc[j], kGroupDotExp - sh.scale[mm]));
            }
        }
        const int next = (tg + tg_stride) * tpw + tsub;
        if (next < ntiles && rb < re) load_rounds(next, rb);
    }
}

}  // namespace w4
