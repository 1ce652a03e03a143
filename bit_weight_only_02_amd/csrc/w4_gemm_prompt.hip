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
// steps span more than 2^25 (or hold a bf16 subnormal, inf or NaN) cannot be
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
// BN = 64*NT weight rows, each of its four waves 16*NT weight rows.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4_device.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {

constexpr int kPromptNT = 3;  // 16-row weight tiles per wave

// ---- staging pass: one workgroup per (padded) activation row ---------------
// Xt chunk (p, m) at Xt[p*Mp + m]: columns 8p..8p+7 of row m (p = 4g + q), in
// the pair order (x0,x4)(x1,x5)(x2,x6)(x3,x7) of the weight unpack, scaled by
// 2^xs[m]; rows m >= M and columns >= K are zeros.  xbad[m] = 1 when row m
// cannot be staged exactly (bf16 only).
__global__ __launch_bounds__(256) void prompt_stage_kernel(const uint16_t *__restrict__ X, long ldx,
                                                           int dt, int M, int K, int Gp, int Mp,
                                                           uint4 *__restrict__ Xt,
                                                           int *__restrict__ xs,
                                                           int *__restrict__ xbad) {
    __shared__ uint32_t red_mx[4], red_mn[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
// Grid: x = blocks of BN = 64*NT weight rows, y = blocks of BM = 16*MT
// activation rows.  Dynamic LDS: two buffers of one round (4 groups) of the
// staged activations, 16*BM chunks of 16 bytes each, chunk (p, m) of the round
// at p*BM + m.
template <int MT>
__global__ __launch_bounds__(256) void prompt_kernel(const uint4 *__restrict__ codes,
                                                     const uint16_t *__restrict__ steps, int N, int K,
                                                     const uint4 *__restrict__ Xt,
                                                     const int *__restrict__ xs,
                                                     const int *__restrict__ xbad,
                                                     const uint16_t *__restrict__ X, long ldx, int dt,
                                                     int M, int Mp, int Gp, float *__restrict__ Y,
                                                     long ldy) {
    constexpr int NT = kPromptNT, BM = 16 * MT, BN = 64 * NT;
    extern __shared__ uint4 prompt_a[];
    __shared__ int sh_xs[BM];
    __shared__ int sh_bad;
    const int G = K >> 5;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.y * BM, nb0 = blockIdx.x * BN;

    if (tid == 0) sh_bad = 0;
    __syncthreads();
    for (int i = tid; i < BM; i += 256) {
        sh_xs[i] = xs[m0 + i];
        if (m0 + i < M && xbad[m0 + i]) sh_bad = 1;
    }
    __syncthreads();

    if (sh_bad) {
        // Rare exact path: a row of this block could not be staged as fp16.
        // Plain fp32 products and group sums, one output per thread at a time.
        for (int o = tid; o < BM * BN; o += 256) {
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

    // Rows of this wave's NT tiles (clamped for loads; stored only below N).
    int row[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) row[t] = min(nb0 + (wave * NT + t) * 16 + n_l, N - 1);

    // Per-row scale t_n from the exponents of the row's nonzero steps; a row
    // that cannot be scaled makes its wave take the per-group path.
    int tn[NT];
    int wave_bad = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        int emax = 0, emin = 255, bad = 0;
        const uint16_t *sp = steps + (long)row[t] * G;
        for (int g = q; g < G; g += 4) {
            const int mag = sp[g] & 0x7FFF;
            if (mag == 0) continue;
            const int e = mag >> 7;
            if (e == 0 || e == 255) bad = 1;
            emax = max(emax, e);
            emin = min(emin, e);
        }
        emax = max(emax, __shfl_xor(emax, 16, kWave));
        emax = max(emax, __shfl_xor(emax, 32, kWave));
        emin = min(emin, __shfl_xor(emin, 16, kWave));
        emin = min(emin, __shfl_xor(emin, 32, kWave));
        if (emax > 0 && emax - emin > 25) bad = 1;
        tn[t] = emax > 0 ? 138 - emax : 0;  // largest |c - 8| * step * 2^t below 2^15
        wave_bad |= bad;
    }
    const bool fast = !wave_or_i32(wave_bad);

    // Loads of one round (4 groups): lane (n_l, q) reads group 4r + q of its
    // rows (clamped: groups past G multiply zero activations, and their steps
    // read as 0), and the 4 steps of the round.
    uint4 qw[NT];
    uint2 sw[NT];
    const bool steps8 = (G & 3) == 0 && (reinterpret_cast<uintptr_t>(steps) & 7) == 0;
    auto load_b = [&](int r) __attribute__((always_inline)) {
        const int g0 = 4 * r;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            qw[t] = codes[(long)row[t] * G + min(g0 + q, G - 1)];
            const uint16_t *sp = steps + (long)row[t] * G + g0;
            if (steps8) {
                sw[t] = *reinterpret_cast<const uint2 *>(sp);
            } else {
                const uint32_t s0 = g0 < G ? sp[0] : 0u, s1 = g0 + 1 < G ? sp[1] : 0u;
                const uint32_t s2 = g0 + 2 < G ? sp[2] : 0u, s3 = g0 + 3 < G ? sp[3] : 0u;
                sw[t] = make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
            }
        }
    };
    // Direct-to-LDS copy of round r's activations into buffer b: 16*BM chunks,
    // 64 per instruction (BM is a multiple of 16, so every lane has one).
    auto load_a = [&](int r, int b) __attribute__((always_inline)) {
        uint4 *dst = prompt_a + b * 16 * BM;
        for (int c0 = wave * 64; c0 < 16 * BM; c0 += 256) {
            const int c = c0 + lane;
            const int p = c / BM, mm = c % BM;
            const uint4 *src = Xt + (long)(16 * r + p) * Mp + m0 + mm;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(dst + c0), 16,
                                             0, 0);
        }
    };

    const int rounds = Gp >> 2;
    const uint32_t k_or = 0x64006400u;                   // 1024 in both fp16 halves
    const h2 k1032 = __builtin_bit_cast(h2, 0x64086408u);  // 1032 in both halves
    f4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    auto main_loop = [&](auto fast_t) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_t)::value;
        load_a(0, 0);
        load_b(0);
        for (int r = 0; r < rounds; ++r) {
            wait_vmcnt<0>();
            lds_barrier();  // round r staged by every wave; buffer (r+1)&1 free
            // this round's weight fragments, built before the next loads go out
            h8 bf[4][NT];
            float st[4][NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t w[4] = {qw[t].x, qw[t].y, qw[t].z, qw[t].w};
                transpose_lane_groups(w);
                const uint32_t sv[4] = {sw[t].x & 0xFFFFu, sw[t].x >> 16, sw[t].y & 0xFFFFu,
                                        sw[t].y >> 16};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h2 sc = {(_Float16)1.0f, (_Float16)1.0f};
                    if constexpr (FAST) {
                        const _Float16 s = (_Float16)__builtin_ldexpf(bf16_to_f32(sv[j]), tn[t]);
                        sc = h2{s, s};
                    } else {
                        st[j][t] = bf16_to_f32(sv[j]);
                    }
                    // (c - 8) [* step * 2^t_n] for the pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7)
                    const h2 p0 = (as_h2((w[j] & 0x000F000Fu) | k_or) - k1032) * sc;
                    const h2 p1 = (as_h2(((w[j] >> 4) & 0x000F000Fu) | k_or) - k1032) * sc;
                    const h2 p2 = (as_h2(((w[j] >> 8) & 0x000F000Fu) | k_or) - k1032) * sc;
                    const h2 p3 = (as_h2(((w[j] >> 12) & 0x000F000Fu) | k_or) - k1032) * sc;
                    bf[j][t] = h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                }
            }
            if (r + 1 < rounds) {
                load_a(r + 1, (r + 1) & 1);
                load_b(r + 1);
            }
            const h8 *Ah = reinterpret_cast<const h8 *>(prompt_a + (r & 1) * 16 * BM);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const h8 a = Ah[(4 * j + q) * BM + 16 * i + n_l];
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if constexpr (FAST) {
                            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[j][t], acc[i][t], 0, 0, 0);
                        } else {
                            const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                a, bf[j][t], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                            acc[i][t][0] = __builtin_fmaf(d[0], st[j][t], acc[i][t][0]);
                            acc[i][t][1] = __builtin_fmaf(d[1], st[j][t], acc[i][t][1]);
                            acc[i][t][2] = __builtin_fmaf(d[2], st[j][t], acc[i][t][2]);
                            acc[i][t][3] = __builtin_fmaf(d[3], st[j][t], acc[i][t][3]);
                        }
                    }
                }
            }
        }
    };
    if (fast)
        main_loop(std::true_type{});
    else
        main_loop(std::false_type{});

    // lane (n_l, q) holds rows 4q..4q+3 of column n_l of each 16 x 16 tile
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = nb0 + (wave * NT + t) * 16 + n_l;
        if (n >= N) continue;
        const int e_n = fast ? tn[t] : 0;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ml = 16 * i + 4 * q + j;
                if (m0 + ml < M)
                    Y[(long)(m0 + ml) * ldy + n] = __builtin_ldexpf(acc[i][t][j], -e_n - sh_xs[ml]);
            }
        }
    }
}

namespace {

typedef void (*PromptFn)(const uint4 *, const uint16_t *, int, int, const uint4 *, const int *,
                         const int *, const uint16_t *, long, int, int, int, int, float *, long);

struct PromptPlan {
    int MT;      // 16-row activation tiles per workgroup
    int Mp;      // activation rows padded to a multiple of 16*MT
    int Gp;      // groups padded to a multiple of 4
};

PromptPlan prompt_plan(int K, int M) {
    PromptPlan p;
    p.MT = M > 64 ? 8 : M > 32 ? 4 : M > 16 ? 2 : 1;
    const int bm = 16 * p.MT;
    p.Mp = (M + bm - 1) / bm * bm;
    p.Gp = ((K / 32) + 3) / 4 * 4;
    return p;
}

PromptFn pick_prompt(int MT) {
    switch (MT) {
        case 1: return prompt_kernel<1>;
        case 2: return prompt_kernel<2>;
        case 4: return prompt_kernel<4>;
        case 8: return prompt_kernel<8>;
    }
    return nullptr;
}

}  // namespace

size_t gemm_prompt_workspace(int N, int K, int M) {
    (void)N;
    const PromptPlan p = prompt_plan(K, M);
    // staged chunks, then the row scales and the row flags
    return (size_t)p.Gp * 4 * p.Mp * 16 + (size_t)p.Mp * 8;
}

hipError_t launch_gemm_prompt(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              void *ws, hipStream_t stream) {
    const PromptPlan p = prompt_plan(K, M);
    PromptFn fn = pick_prompt(p.MT);
    if (!fn || !ws || K < 32 || M < 1) return hipErrorInvalidConfiguration;
    uint4 *Xt = static_cast<uint4 *>(ws);
    int *xs = reinterpret_cast<int *>(Xt + (size_t)p.Gp * 4 * p.Mp);
    int *xbad = xs + p.Mp;
    hipLaunchKernelGGL(prompt_stage_kernel, dim3((unsigned)p.Mp), dim3(256), 0, stream, X, ldx, dt, M,
                       K, p.Gp, p.Mp, Xt, xs, xbad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bn = 64 * kPromptNT;
    const size_t lds = (size_t)2 * 16 * 16 * p.MT * sizeof(uint4);
    hipLaunchKernelGGL(fn, dim3((unsigned)((N + bn - 1) / bn), (unsigned)(p.Mp / (16 * p.MT))), dim3(256),
                       lds, stream, reinterpret_cast<const uint4 *>(codes), steps, N, K, Xt, xs, xbad, X,
                       ldx, dt, M, p.Mp, p.Gp, Y, ldy);
    return hipGetLastError();
}

}  // namespace w4
