// Prompt-chunk W4A16 product on the matrix cores of gfx950 (M up to
// W4_MAX_M_PROMPT activation rows, e.g. a 256-token chunk).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 6 -
// Read Prompts in 32-Bit on a Card Without Tensor Cores") reads a prompt in
// chunks of 256 tokens, unpacking the weights to a full matrix for each
// multiply, and quotes [256, 1536] x [1536, 24576] in TFLOP/s.  With M = 256
// the product is a real contraction (about 910 flop per weight byte), so here
// it runs on MFMA straight from the packed words: no 16-bit weight matrix is
// ever written.
//
// Exact operands.  Each weight enters v_mfma_f32_16x16x32_f16 as the fp16
// value (c - 8) * step * 2^t_n: (c - 8) has at most 3 significant bits and a
// bf16 step 8, so the product fits fp16's 11 bits exactly whenever it is a
// normal fp16 number.  t_n is a power of two per weight row, chosen from the
// row's largest step so that every product lies in [2^-14, 2^15); a row whose
// steps span more than 2^21 (or hold a bf16 subnormal, inf or NaN) cannot be
// scaled that way, and the 16-row tile holding it instead multiplies (c - 8)
// alone and applies each group's step to the fp32 MFMA result (the small-M
// engine's form: exact, but one VALU multiply-add per output per group).  The
// activations are fp16 as given, or bf16 staged as x * 2^s_m with a power of
// two per row (exact when the row's nonzero magnitudes span at most 2^31); a
// block of rows holding one that cannot be staged so is computed with plain
// fp32 products.  The MFMA sums in fp32; the output is scaled back by
// 2^-(t_n + s_m) once.
//
// Two launches: a staging pass converts X once into fp16 chunks laid out
// plane by plane ([Gp][4][Mp] chunks of 8 values, plane p = 4g + q holding
// columns 32g + 8q .. +7 of every row), so that the product streams each
// round of 4 groups of a row block into LDS with contiguous direct-to-LDS
// loads; the product then gives each workgroup BM = 16*MT activation rows and
// BN = 16*W*NT weight rows, each of its W waves 16*NT weight rows.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

constexpr int kPromptNT = 3;  // 16-row weight tiles per wave

// ---- staging pass ---------------------------------------------------------
// Workgroups 0 .. Mp-1 stage one activation row each; the next Np/16 each
// prepare one 16-row tile of the weight steps.
//
// Activation row m: Xt chunk (p, m) at Xt[p*Mp + m] holds columns 8p..8p+7
// (p = 4g + q) in the pair order (x0,x4)(x1,x5)(x2,x6)(x3,x7) of the weight
// unpack, scaled by 2^xs[m]; rows m >= M and columns >= K are zeros.
// xbad[m] = 1 when the bf16 row cannot be staged exactly (its chunks are then
// zeros and the product reads the row itself).
//
// Weight tile T (rows 16T .. 16T+15, rows >= N as all-zero steps): per row the
// scale t_n = 138 - (largest biased step exponent), so that every |c - 8| *
// step * 2^t_n lies below 2^15; the tile is fast (tfast[T] = 1) when every row
// has no subnormal, inf or NaN step and its nonzero steps span at most 2^21
// (every product then at least 2^-14, a normal fp16 number).  For a fast tile,
// St[(r*Np + n)*4 + j] = fp16(step(n, 4r + j) * 2^t_n), exact (8 significant
// bits in fp16's normal range), and 0 for groups past K.
__global__ __launch_bounds__(256) void prompt_stage_kernel(
    const uint16_t *__restrict__ X, long ldx, int dt, int M, int K, int Gp, int Mp,
    uint4 *__restrict__ Xt, int *__restrict__ xs, int *__restrict__ xbad,
    const uint16_t *__restrict__ steps, int N, int Np, _Float16 *__restrict__ St,
    int *__restrict__ tn, int *__restrict__ tfast) {
    __shared__ uint32_t red_mx[4], red_mn[4];
    __shared__ int red_bad[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = K >> 5;

    if ((int)blockIdx.x >= Mp) {
        // ---- one 16-row tile of weight steps: 16 threads per row ----
        const int T = blockIdx.x - Mp;
        const int r16 = tid >> 4, k = tid & 15;
        const int n = T * 16 + r16;
        const uint16_t *sp = steps + (long)min(n, N - 1) * G;
        int emax = 0, emin = 255, bad = 0;
        if (n < N) {
            for (int g = k; g < G; g += 16) {
                const int mag = sp[g] & 0x7FFF;
                if (mag == 0) continue;
                const int e = mag >> 7;
                if (e == 0 || e == 255) bad = 1;
                emax = max(emax, e);
                emin = min(emin, e);
            }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            emax = max(emax, __shfl_xor(emax, off, kWave));
            emin = min(emin, __shfl_xor(emin, off, kWave));
            bad |= __shfl_xor(bad, off, kWave);
        }
        if (emax > 0 && emax - emin > 21) bad = 1;
        const int t = emax > 0 ? 138 - emax : 0;
        const int wbad = wave_or_i32(bad);
        if (lane == 0) red_bad[wave] = wbad;
        __syncthreads();
        const bool fast = !(red_bad[0] | red_bad[1] | red_bad[2] | red_bad[3]);
        if (k == 0) tn[n] = fast ? t : 0;
        if (tid == 0) tfast[T] = fast ? 1 : 0;
        // scaled steps of every round, 4 per row and round; 0 past K and past N
        for (int gg = k; gg < Gp; gg += 16) {
            _Float16 v = (_Float16)0.0f;
            if (fast && n < N && gg < G) v = (_Float16)__builtin_ldexpf(bf16_to_f32(sp[gg]), t);
            St[((long)(gg >> 2) * Np + n) * 4 + (gg & 3)] = v;
        }
        return;
    }

    // ---- one activation row ----
    const int m = blockIdx.x;
    const int nch = Gp * 4, kch = K >> 3;
    if (m >= M) {
        for (int p = tid; p < nch; p += 256) Xt[(long)p * Mp + m] = make_uint4(0, 0, 0, 0);
        if (tid == 0) {
            xs[m] = 0;
            xbad[m] = 0;
        }
        return;
    }
    const uint16_t *xr = X + (long)m * ldx;
    auto chunk = [&](int p) __attribute__((always_inline)) {
        const uint16_t *s = xr + 8 * p;
        return make_uint4(s[0] | ((uint32_t)s[1] << 16), s[2] | ((uint32_t)s[3] << 16),
                          s[4] | ((uint32_t)s[5] << 16), s[6] | ((uint32_t)s[7] << 16));
    };
    int s_m = 0, bad = 0;
    if (dt != 0) {
        // largest magnitude and smallest nonzero magnitude - 1 (bf16 bits order
        // like the magnitudes; zero wraps to 0xFFFF)
        uint32_t mx = 0, mn = 0xFFFFu;
        for (int p = tid; p < kch; p += 256) {
            const uint4 v = chunk(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
                mx = max(mx, max(lo, hi));
                mn = min(mn, min((lo - 1) & 0xFFFFu, (hi - 1) & 0xFFFFu));
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, kWave));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, kWave));
        }
        if (lane == 0) {
            red_mx[wave] = mx;
            red_mn[wave] = mn;
        }
        __syncthreads();
        mx = max(max(red_mx[0], red_mx[1]), max(red_mx[2], red_mx[3]));
        mn = min(min(red_mn[0], red_mn[1]), min(red_mn[2], red_mn[3]));
        if (mn != 0xFFFFu) {  // some nonzero value
            const int emax = (int)(mx >> 7), emin = (int)((mn + 1) >> 7);
            bad = (mx >= 0x7F80u || emin == 0 || emin + 31 < emax) ? 1 : 0;
            s_m = 141 - emax;  // largest magnitude scaled into [2^14, 2^15)
        }
    }
    for (int p = tid; p < nch; p += 256) {
        uint4 o = make_uint4(0, 0, 0, 0);
        if (p < kch && !bad) {
            const uint4 v = chunk(p);
            if (dt != 0) {
                auto f = [&](uint32_t w, int hi) __attribute__((always_inline)) {
                    return __builtin_ldexpf(__uint_as_float(hi ? (w & 0xFFFF0000u) : (w << 16)), s_m);
                };
                o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.x, 0), f(v.z, 0)));
                o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.x, 1), f(v.z, 1)));
                o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.y, 0), f(v.w, 0)));
                o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f(v.y, 1), f(v.w, 1)));
            } else {
                o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
                o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
                o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
                o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
            }
        }
        Xt[(long)p * Mp + m] = o;
    }
    if (tid == 0) {
        xs[m] = s_m;
        xbad[m] = bad;
    }
}

// ---- the product -------------------------------------------------------------
// Grid: x = blocks of BN = 16*W*NT weight rows, y = blocks of BM = 16*MT
// activation rows.  Every operand goes through a ring of D stages in LDS, each
// holding one round (4 groups) and filled by direct-to-LDS loads D-1 rounds
// ahead of the round computed:
//   A:  16*BM chunks, chunk (p, m) of the round at p*BM + m (p = 4j + q);
//   B:  4*BN chunks of codes, group 4r + Q of block row rl at 4*rl + Q (each
//       row's 64 bytes are read by 4 adjacent lanes);
//   S:  the scaled steps of the round, 4 fp16 per block row (BN*8 bytes,
//       padded to 64 chunks per wave so that every wave issues one full
//       instruction).
// W waves, each with NT 16-row weight tiles and all MT activation tiles.
// Each wave issues the same number of load instructions per round, so "round
// r has landed" is a count of outstanding loads.
template <int MT, int D, int W>
__global__ __launch_bounds__(64 * W) void prompt_kernel(
    const uint4 *__restrict__ codes, const uint16_t *__restrict__ steps, int N, int K,
    const uint4 *__restrict__ Xt, const int *__restrict__ xs, const int *__restrict__ xbad,
    const uint4 *__restrict__ St, const int *__restrict__ tn, const int *__restrict__ tfast,
    const uint16_t *__restrict__ X, long ldx, int dt, int M, int Mp, int Gp, int Np,
    float *__restrict__ Y, long ldy) {
    constexpr int NT = kPromptNT, BM = 16 * MT, BN = 16 * W * NT, TH = 64 * W;
    constexpr int SA = 16 * BM, SB = 4 * BN, SS = TH, STAGE = SA + SB + SS;  // chunks
    constexpr int PER = SA / TH + SB / TH + 1;  // load instructions per wave and round
    static_assert(SA % TH == 0 && SB % TH == 0 && BN * 8 <= SS * 16, "stage layout");
    static_assert((D - 2) * PER < 64, "vmcnt range");
    extern __shared__ uint4 prompt_lds[];
    __shared__ int sh_xs[BM];
    __shared__ int sh_bad;
    const int G = K >> 5;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.y * BM, nb0 = blockIdx.x * BN;

    if (tid == 0) sh_bad = 0;
    __syncthreads();
    for (int i = tid; i < BM; i += TH) {
        sh_xs[i] = xs[m0 + i];
        if (m0 + i < M && xbad[m0 + i]) sh_bad = 1;
    }
    __syncthreads();

    if (sh_bad) {
        // Rare exact path: a row of this block could not be staged as fp16.
        // Plain fp32 products and group sums, one output per thread at a time.
        for (int o = tid; o < BM * BN; o += TH) {
            const int mm = m0 + o / BN, n = nb0 + o % BN;
            if (mm >= M || n >= N) continue;
            float acc = 0.0f;
            for (int g = 0; g < G; ++g)
                acc = __builtin_fmaf(group_dot_f32(codes[(long)n * G + g], X + mm * ldx + g * 32, dt),
                                     bf16_to_f32(steps[(long)n * G + g]), acc);
            Y[(long)mm * ldy + n] = acc;
        }
        return;
    }

    // the wave's tiles: fast when the staging pass found all of them scalable
    int fast_i = 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) fast_i &= tfast[(nb0 >> 4) + wave * NT + t];
    const bool fast = __builtin_amdgcn_readfirstlane(fast_i) != 0;

    // Request round r into stage b.  Per-lane byte offsets are fixed; the
    // round enters through the wave-uniform bases.  Every address is in
    // bounds: codes rows are clamped to N - 1, and in a last round cut by K the
    // groups too; S padding lanes re-read the first chunk.
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)prompt_lds;
    uint32_t offa[SA / TH], offb[SB / TH];
#pragma unroll
    for (int i = 0; i < SA / TH; ++i) {
        const int c = wave * 64 + TH * i + lane;
        offa[i] = (uint32_t)((c / BM) * Mp + c % BM) * 16u;
    }
    int brow[SB / TH], bq[SB / TH];
#pragma unroll
    for (int i = 0; i < SB / TH; ++i) {
        const int c = wave * 64 + TH * i + lane;
        brow[i] = min(nb0 + (c >> 2), N - 1) - nb0;  // a row's 4 groups from 4 adjacent lanes
        bq[i] = c & 3;
        offb[i] = (uint32_t)(brow[i] * G + bq[i]) * 16u;
    }
    const uint32_t offs = (uint32_t)((wave * 64 + lane) < BN / 2 ? (wave * 64 + lane) : 0) * 16u;
    const uint4 *codes_blk = codes + (long)nb0 * G;
    auto issue = [&](int r, int b) __attribute__((always_inline)) {
        const uint32_t st = lds0 + (uint32_t)(b * STAGE) * 16u;
#pragma unroll
        for (int i = 0; i < SA / TH; ++i)
            lds_dma16_so<false>(Xt + (long)16 * r * Mp + m0, offa[i], st + (wave_u * 64 + TH * i) * 16u);
        if (4 * r + 3 < G) {
#pragma unroll
            for (int i = 0; i < SB / TH; ++i)
                lds_dma16_so<true>(codes_blk + 4 * r, offb[i], st + (SA + wave_u * 64 + TH * i) * 16u);
        } else {
#pragma unroll
            for (int i = 0; i < SB / TH; ++i)
                lds_dma16_so<true>(codes_blk, (uint32_t)(brow[i] * G + min(4 * r + bq[i], G - 1)) * 16u,
                                   st + (SA + wave_u * 64 + TH * i) * 16u);
        }
        lds_dma16_so<false>(St + ((long)r * Np + nb0) / 2, offs, st + (SA + SB + wave_u * 64) * 16u);
    };

    const int rounds = Gp >> 2;
    // Unpack: a nibble masked into the low mantissa of an fp16 1024 gives
    // 1024 + c (low nibble of a byte) or 1024 + 16c (high nibble); subtracting
    // 1032 or 1152 leaves (c - 8) or 16 (c - 8), and the step factor (divided
    // by 16 for the high nibbles) follows.  One AND-OR per pair, one shift per
    // word.
    const uint32_t k_or = 0x64006400u, m_lo = 0x000F000Fu, m_hi = 0x00F000F0u;
    const h2 k1032 = __builtin_bit_cast(h2, 0x64086408u);  // 1032 in both halves
    const h2 k1152 = __builtin_bit_cast(h2, 0x64806480u);  // 1152 in both halves
    const h2 k16th = __builtin_bit_cast(h2, 0x2C002C00u);  // 1/16 in both halves
    auto and_or = [](uint32_t x, uint32_t m, uint32_t k) __attribute__((always_inline)) {
        uint32_t r;
        asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(k));
        return r;
    };
    f4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    auto main_loop = [&](auto fast_t) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_t)::value;
#pragma unroll
        for (int s = 0; s < D - 1; ++s)
            if (s < rounds) issue(s, s);
        for (int r = 0; r < rounds; ++r) {
            // round r landed (for this wave; the barrier then for all waves),
            // and every wave is done with round r - 1, whose stage is refilled
            if (r + D - 2 < rounds)
                wait_vmcnt_mem<(D - 2) * PER>();
            else
                wait_vmcnt_mem<0>();
            lds_barrier();
            if (r + D - 1 < rounds) issue(r + D - 1, (r + D - 1) % D);
            const uint4 *st = prompt_lds + (r % D) * STAGE;
            const h8 *Ah = reinterpret_cast<const h8 *>(st);
            const uint4 *Bc = st + SA;
            const uint2 *Sc = reinterpret_cast<const uint2 *>(st + SA + SB);
            // the round's raw words (word q of each of the 4 groups) and steps
            uint32_t w[NT][4];
            h2 sc[NT][4];
            float sf[NT][4];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int rl = (wave * NT + t) * 16 + n_l;
                const uint4 qv = Bc[4 * rl + q];
                w[t][0] = qv.x;
                w[t][1] = qv.y;
                w[t][2] = qv.z;
                w[t][3] = qv.w;
                if constexpr (FAST) {
                    const uint2 sv = Sc[rl];
                    sc[t][0] = as_h2(__builtin_amdgcn_perm(sv.x, sv.x, 0x01000100u));
                    sc[t][1] = as_h2(__builtin_amdgcn_perm(sv.x, sv.x, 0x03020302u));
                    sc[t][2] = as_h2(__builtin_amdgcn_perm(sv.y, sv.y, 0x01000100u));
                    sc[t][3] = as_h2(__builtin_amdgcn_perm(sv.y, sv.y, 0x03020302u));
                } else {
                    const long rowoff = (long)min(nb0 + rl, N - 1) * G;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int g = 4 * r + j;
                        sf[t][j] = g < G ? bf16_to_f32(steps[rowoff + g]) : 0.0f;
                        sc[t][j] = h2{(_Float16)1.0f, (_Float16)1.0f};
                    }
                }
            }
            // Software pipeline over the round's 4 groups: the A fragments of
            // group j + 1 are requested before the MFMAs of group j, and its
            // weight tiles are unpacked between them (one after each
            // activation tile), so the VALU work sits among the MFMAs
            h8 a[2][MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) a[0][i] = Ah[q * BM + 16 * i + n_l];
#pragma unroll
            for (int t = 0; t < NT; ++t) transpose_lane_groups(w[t]);
            auto unpack = [&](int t, int j) __attribute__((always_inline)) {
                const uint32_t wj = w[t][j];
                const uint32_t u = wj >> 8;
                const h2 s16 = sc[t][j] * k16th;
                const h2 p0 = (as_h2(and_or(wj, m_lo, k_or)) - k1032) * sc[t][j];
                const h2 p1 = (as_h2(and_or(wj, m_hi, k_or)) - k1152) * s16;
                const h2 p2 = (as_h2(and_or(u, m_lo, k_or)) - k1032) * sc[t][j];
                const h2 p3 = (as_h2(and_or(u, m_hi, k_or)) - k1152) * s16;
                return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            };
            h8 bf[2][NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) bf[0][t] = unpack(t, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < MT; ++i) a[(j + 1) & 1][i] = Ah[(4 * (j + 1) + q) * BM + 16 * i + n_l];
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if constexpr (FAST) {
                            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j & 1][i], bf[j & 1][t], acc[i][t], 0, 0, 0);
                        } else {
                            const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                a[j & 1][i], bf[j & 1][t], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                            acc[i][t][0] = __builtin_fmaf(d[0], sf[t][j], acc[i][t][0]);
                            acc[i][t][1] = __builtin_fmaf(d[1], sf[t][j], acc[i][t][1]);
                            acc[i][t][2] = __builtin_fmaf(d[2], sf[t][j], acc[i][t][2]);
                            acc[i][t][3] = __builtin_fmaf(d[3], sf[t][j], acc[i][t][3]);
                        }
                    }
                    // the next group's weight tiles, one after each activation tile
                    if (j + 1 < 4 && i < NT) bf[(j + 1) & 1][i] = unpack(i, j + 1);
                }
                if (j + 1 < 4) {
#pragma unroll
                    for (int t = MT; t < NT; ++t) bf[(j + 1) & 1][t] = unpack(t, j + 1);
                }
            }
        }
    };
    if (fast)
        main_loop(std::true_type{});
    else
        main_loop(std::false_type{});

    // Lane (n_l, q) holds rows 4q..4q+3 of column n_l of each 16 x 16 tile.
    // Each value is scaled back first (its column's t_n, its row's s_m); then
    // a 4 x 4 transpose inside each quad of lanes (two exchange stages, lanes
    // 1 and 2 apart) leaves lane (4k + c, q) with row 4q + c, columns 4k..4k+3,
    // stored as one 16-byte non-temporal write when the four columns exist and
    // Y allows it.
    const bool yvec = (reinterpret_cast<uintptr_t>(Y) & 15) == 0 && (ldy & 3) == 0;
    const int c = n_l & 3, k4 = n_l >> 2;
    auto xch = [](float v, auto ctrl) __attribute__((always_inline)) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    using X1 = std::integral_constant<int, 0xB1>;  // quad_perm [1,0,3,2]
    using X2 = std::integral_constant<int, 0x4E>;  // quad_perm [2,3,0,1]
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int nt0 = nb0 + (wave * NT + t) * 16;
        const int n = nt0 + n_l;
        const int e_n = fast && n < N ? tn[n] : 0;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __builtin_ldexpf(acc[i][t][j], -e_n - sh_xs[16 * i + 4 * q + j]);
            {
                const float p0 = xch(v[0], X1{}), p1 = xch(v[1], X1{}), p2 = xch(v[2], X1{}), p3 = xch(v[3], X1{});
                if (c & 1) {
                    v[0] = p1;
                    v[2] = p3;
                } else {
                    v[1] = p0;
                    v[3] = p2;
                }
            }
            {
                const float p0 = xch(v[0], X2{}), p1 = xch(v[1], X2{}), p2 = xch(v[2], X2{}), p3 = xch(v[3], X2{});
                if (c & 2) {
                    v[0] = p2;
                    v[1] = p3;
                } else {
                    v[2] = p0;
                    v[3] = p1;
                }
            }
            const int ml = 16 * i + 4 * q + c, nc = nt0 + 4 * k4;
            if (m0 + ml >= M) continue;
            float *dst = Y + (long)(m0 + ml) * ldy + nc;
            if (yvec && nc + 3 < N) {
                typedef float f4v __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f4v{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4v *>(dst));
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (nc + jj < N) dst[jj] = v[jj];
            }
        }
    }
}

namespace {

typedef void (*PromptFn)(const uint4 *, const uint16_t *, int, int, const uint4 *, const int *,
                         const int *, const uint4 *, const int *, const int *, const uint16_t *, long,
                         int, int, int, int, int, float *, long);

constexpr int kPromptD = 3;  // ring stages

struct PromptPlan {
    int MT;      // 16-row activation tiles per workgroup
    int W;       // waves per workgroup
    int Mp;      // activation rows padded to a multiple of 16*MT
    int Gp;      // groups padded to a multiple of 4
    int Np;      // weight rows padded to a multiple of BN = 16*W*NT
    size_t off_xs, off_st, off_tn, off_tf, bytes;  // workspace layout
};

// Above 64 rows, four waves of 8 activation tiles (each unpacked weight tile
// feeds 8 MFMAs); from 33 to 64 rows eight waves of 4; fewer rows, four waves
// with one tile per 16 rows.
PromptPlan prompt_plan(int N, int K, int M) {
    PromptPlan p;
    if (M > 64) {
        p.MT = 8;
        p.W = 4;
    } else if (M > 32) {
        p.MT = 4;
        p.W = 8;
    } else {
        p.MT = M > 16 ? 2 : 1;
        p.W = 4;
    }
    const int bm = 16 * p.MT, bn = 16 * p.W * kPromptNT;
    p.Mp = (M + bm - 1) / bm * bm;
    p.Gp = ((K / 32) + 3) / 4 * 4;
    p.Np = (N + bn - 1) / bn * bn;
    p.off_xs = (size_t)p.Gp * 4 * p.Mp * 16;          // after Xt
    p.off_st = p.off_xs + (size_t)p.Mp * 8;           // after xs, xbad (16-byte multiple)
    p.off_tn = p.off_st + (size_t)(p.Gp / 4) * p.Np * 8;
    p.off_tf = p.off_tn + (size_t)p.Np * 4;
    p.bytes = p.off_tf + (size_t)(p.Np / 16) * 4;
    return p;
}

template <int D, int W>
PromptFn pick_prompt_dw(int MT) {
    switch (MT) {
        case 1: return W == 4 ? prompt_kernel<1, D, 4> : nullptr;
        case 2: return prompt_kernel<2, D, W>;
        case 4: return prompt_kernel<4, D, W>;
        case 8: return prompt_kernel<8, D, W>;
    }
    return nullptr;
}

PromptFn pick_prompt(int MT, int D, int W) {
    switch (D * 16 + W) {
        case 2 * 16 + 4: return pick_prompt_dw<2, 4>(MT);
        case 3 * 16 + 4: return pick_prompt_dw<3, 4>(MT);
        case 2 * 16 + 8: return pick_prompt_dw<2, 8>(MT);
        case 3 * 16 + 8: return pick_prompt_dw<3, 8>(MT);
    }
    return nullptr;
}

size_t prompt_lds_bytes(int MT, int D, int W) {
    return (size_t)D * (16 * 16 * MT + 4 * 16 * W * kPromptNT + 64 * W) * 16;
}

}  // namespace

size_t gemm_prompt_workspace(int N, int K, int M) { return prompt_plan(N, K, M).bytes; }

hipError_t launch_gemm_prompt(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              void *ws, hipStream_t stream) {
    const PromptPlan p = prompt_plan(N, K, M);
    const int D = kPromptD;
    PromptFn fn = pick_prompt(p.MT, D, p.W);
    if (prompt_lds_bytes(p.MT, D, p.W) > 150 * 1024) return hipErrorInvalidConfiguration;
    if (!fn || !ws || K < 32 || M < 1 || N < 1 || (reinterpret_cast<uintptr_t>(ws) & 15))
        return hipErrorInvalidConfiguration;
    char *base = static_cast<char *>(ws);
    uint4 *Xt = reinterpret_cast<uint4 *>(base);
    int *xs = reinterpret_cast<int *>(base + p.off_xs);
    int *xbad = xs + p.Mp;
    _Float16 *St = reinterpret_cast<_Float16 *>(base + p.off_st);
    int *tn = reinterpret_cast<int *>(base + p.off_tn);
    int *tf = reinterpret_cast<int *>(base + p.off_tf);
    hipLaunchKernelGGL(prompt_stage_kernel, dim3((unsigned)(p.Mp + p.Np / 16)), dim3(256), 0, stream, X,
                       ldx, dt, M, K, p.Gp, p.Mp, Xt, xs, xbad, steps, N, p.Np, St, tn, tf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bn = 16 * p.W * kPromptNT, bm = 16 * p.MT;
    const size_t lds = prompt_lds_bytes(p.MT, D, p.W);
    hipLaunchKernelGGL(fn, dim3((unsigned)(p.Np / bn), (unsigned)(p.Mp / bm)), dim3(64 * p.W), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, Xt, xs, xbad,
                       reinterpret_cast<const uint4 *>(St), tn, tf, X, ldx, dt, M, p.Mp, p.Gp, p.Np, Y,
                       ldy);
    return hipGetLastError();
}

}  // namespace w4
