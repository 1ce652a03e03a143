// Device helpers shared by the W4A16 kernels (gfx950 / CDNA4, wave64).
//
// Packed format: codes uint32[N][K/8] (nibble j of word w = column 8w+j), bf16
// steps [N][K/32]; weight = (code - 8) * step.  One 16-byte load (uint4) of a
// row is exactly one group of 32 codes, and it pairs with one bf16 step.
//
// Exact operands.  The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch"
// (section "Step 3 - Multiply Straight From the Packed Weights") turns a code
// into a float by OR-ing it into the bits of 2^23 and subtracting 2^23 + 8.
// The same idea is used here two codes at a time in fp16, one step further:
// with a zero exponent field a masked nibble already IS a float (the subnormal
// c * 2^-24), so a single AND yields two codes and one packed subtract of
// 8 * 2^-24 yields two exact (c - 8) * 2^-24.  The pairs feed v_dot2_f32_f16,
// which multiplies fp16 pairs exactly and accumulates in fp32; the finished
// row is scaled back by 2^24.
//
// Activations are staged as fp16 scaled by a power of two 2^s chosen from the
// vector's largest exponent (so that every staged value is a normal fp16 equal
// to x * 2^s exactly).  Then every product (c - 8) * x * 2^s is exact in fp32,
// and the result is scaled back by 2^-s at the end (also exact).  A vector whose
// values cannot all be staged exactly (a dynamic range above 2^28, or inf/NaN)
// takes a plain fp32 path instead, with the same exact products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also makes
// the wave wait for every outstanding global load (its release fence covers all
// address spaces), which would stall on weight loads that were deliberately
// left in flight across the barrier.
// Written as one asm statement with a memory clobber: the compiler neither
// moves memory accesses across it nor adds waits for loads still in flight.
// LDS written by global_load_lds must be waited for (wait_vmcnt) beforehand.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ float act_to_f32(uint32_t bits, int dt) {
    return dt == 0 ? f16_to_f32(bits) : bf16_to_f32(bits);
}

// Unbiased exponent of a finite nonzero fp32 value that is normal in fp32
// (every fp16 value and every normal bf16 value); -127 for fp32 subnormals.
__device__ __forceinline__ int f32_exponent(float v) {
    return (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;
}

// Unpack.  A nibble masked into the low mantissa bits of an fp16 with a zero
// exponent field is the subnormal c * 2^-24 (or 16c * 2^-24 when it sits four
// bits higher), so one AND turns codes into exact fp16 operands, two per
// 32-bit lane: w & 0x000F000F gives (c0, c4), w & 0x00F000F0 gives 16 (c1, c5),
// and the same masks on w >> 8 give (c2, c6) and 16 (c3, c7).  Every step is
// exact as long as fp16 subnormals are kept (the default floating-point mode
// of these kernels).  The activations are staged in the matching pair order
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) of each 8-value block.

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Group sums come out scaled by 2^-kGroupDotExp; the caller multiplies the
// finished row by 2^kGroupDotExp (exact, a power of two).
constexpr int kGroupDotExp = 24;

// Sum over one group of 32 codes, sum_k (c_k - 8) x_k times 2^-24, with the
// offset taken out of the row loop: sum_k c_k x_k - 8 sum_k x_k.  q holds the
// group's 4 packed words, xr its 16 staged activation pairs.
// group_dot_raw returns the two raw partial sums {even nibbles, odd nibbles
// (times 16)} of c * 2^-24 * x -- every product exact in fp32 -- in a fixed
// order of dot2 steps; group_offset is the same computation on codes that are
// all 8, done once per activation vector.  The difference of the two, taken
// per partial sum and joined with a factor 1/16, is exact whenever the sums
// are (integer or one-hot inputs), and is exactly 0 for a group whose codes
// are all 8.  Per packed word: one shift, four ands and four dot2.
__device__ __forceinline__ float2 group_dot_raw(uint4 q, const h2 *xr) {
    float lo = 0.0f, hi = 0.0f;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t u = w[k] >> 8;
        lo = dot2(as_h2(w[k] & 0x000F000Fu), xr[4 * k + 0], lo);
        hi = dot2(as_h2(w[k] & 0x00F000F0u), xr[4 * k + 1], hi);
        lo = dot2(as_h2(u & 0x000F000Fu), xr[4 * k + 2], lo);
        hi = dot2(as_h2(u & 0x00F000F0u), xr[4 * k + 3], hi);
    }
    return make_float2(lo, hi);
}

__device__ __forceinline__ float2 group_offset(const h2 *xr) {
    // (an opaque all-8 word, so that the compiler emits the very same dot2
    // sequence rather than folding it into something else)
    const uint32_t w8 = __builtin_amdgcn_readfirstlane(0x88888888u);
    return group_dot_raw(make_uint4(w8, w8, w8, w8), xr);
}

__device__ __forceinline__ float group_dot_off(uint4 q, const h2 *xr, float2 off) {
    const float2 s = group_dot_raw(q, xr);
    return __builtin_fmaf(s.y - off.y, 0.0625f, s.x - off.x);
}

// Sum over each group of L consecutive lanes (L = 8, 16, 32 or 64), left in
// the group's last lane: shifted adds within rows of 16 lanes (DPP row_shr),
// then row broadcasts across rows.  A fixed order, so results are reproducible.
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "lanes per group");
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
    if (L >= 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
    if (L >= 32)  // row_bcast:15 into rows 1 and 3
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    if (L == 64)  // row_bcast:31 into rows 2 and 3
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

// Exact fp32 group sum for the fallback path: activations read as fp32 from a
// pointer to the group's 32 raw values.
// (Kept rolled: it is the rare path, and unrolling it would raise the register
// count of the whole kernel.)
__device__ __noinline__ float group_dot_f32(uint4 q, const uint16_t *xg, int dt) {
    float s = 0.0f;
#pragma unroll 1
    for (int k = 0; k < 32; ++k) {
        const uint32_t word = k < 8 ? q.x : k < 16 ? q.y : k < 24 ? q.z : q.w;
        const int c = (int)((word >> (4 * (k & 7))) & 0xFu) - 8;
        s = __builtin_fmaf((float)c, act_to_f32(xg[k], dt), s);
    }
    return s;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ int wave_or_i32(int v) {
    return __builtin_amdgcn_ballot_w64(v != 0) != 0 ? 1 : 0;
}

// Sum of a double over the 64 lanes of a wave, the same bits in every lane:
// a butterfly of exchanges -- lanes 1 apart, 2 apart (quad permutes), the two
// halves of each 8-lane group and of each 16-lane row (mirrors), then pairs of
// rows 16 and 32 apart (permlane swaps) -- each adding the two operands of a
// pair in the same order on both sides.  The exchanges move the two 32-bit
// halves of the double with DPP and permlane instructions, so no LDS traffic.
template <int ctrl>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, ctrl, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    // pair (a, b) is added as min-lane + max-lane in both lanes: a + b is
    // commutative in IEEE arithmetic, so both lanes get the same bits
    v = v + dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v = v + dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v = v + dpp_f64<0x141>(v);  // row_half_mirror
    v = v + dpp_f64<0x140>(v);  // row_mirror
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    auto swap_sum = [](uint64_t x, bool rows32) __attribute__((always_inline)) {
        const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
        uint32_t a_lo, b_lo, a_hi, b_hi;
        if (rows32) {
            const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
            const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
            a_lo = pl[0]; b_lo = pl[1]; a_hi = ph[0]; b_hi = ph[1];
        } else {
            const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
            const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
            a_lo = pl[0]; b_lo = pl[1]; a_hi = ph[0]; b_hi = ph[1];
        }
        // a holds the lower row of each swapped pair in both rows, b the upper
        const double a = __builtin_bit_cast(double, ((uint64_t)a_hi << 32) | a_lo);
        const double b = __builtin_bit_cast(double, ((uint64_t)b_hi << 32) | b_lo);
        return a + b;
    };
    v = swap_sum(u, false);
    v = swap_sum(__builtin_bit_cast(uint64_t, v), true);
    return v;
}

// Sum of squares of v[0..K) (K a multiple of 4) in fp64 with one fixed order,
// shared by every kernel that renormalises (so that they agree bit for bit):
// thread t of a 256-thread workgroup owns the 4-element chunks c = t, t+256,
// ... and adds their squares in ascending (c, element) order; the 64 lanes of
// a wave are combined by wave_sum_f64; the four wave sums are added in wave
// order.  load4(c) returns chunk c as a float4.  Every thread gets the total.
// `red` is 4 doubles of shared scratch.
// (one chunk's squares, in element order: every form of this sum uses it)
__device__ __forceinline__ double add_squares4(double ss, float4 v) {
    ss += (double)v.x * (double)v.x;
    ss += (double)v.y * (double)v.y;
    ss += (double)v.z * (double)v.z;
    ss += (double)v.w * (double)v.w;
    return ss;
}

template <class Load4>
__device__ __forceinline__ double sum_squares_256(int K, Load4 load4, double *red) {
    const int tid = threadIdx.x;
    double ss = 0.0;
    for (int c = tid; c < (K >> 2); c += 256) ss = add_squares4(ss, load4(c));
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const double tot = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return tot;
}

// Buffer resource over `bytes` bytes at p (raw buffer loads, gfx9 format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// 16-byte load that is coherent at agent scope (cache policy SC1): it sees
// stores made with agent scope by workgroups on any XCD.
__device__ __forceinline__ float4 load_coherent_f4(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 16));
}

// Renormalisation of one entry: u / sqrt(ss / K), formed as u times the fp64
// reciprocal 1 / sqrt(ss / K) (computed once per vector), rounded to fp32 and
// then to nearest-even in fp16 (dt 0) or bf16 (dt 1); zero when the vector is
// zero.  Within one unit in the last place of the exactly rounded quotient.
__device__ __forceinline__ double renorm_scale(double ss, int K) {
    const double r = sqrt(ss / (double)K);
    return r > 0.0 ? 1.0 / r : 0.0;
}

__device__ __forceinline__ uint16_t renorm_value(float u, double inv, int dt) {
    // Two separate roundings, fp64 -> fp32 -> 16 bits: with contraction allowed
    // the compiler fuses them into one software fp64 -> fp16 conversion (some
    // forty instructions, and a different rounding).
#pragma clang fp contract(off)
    const float q = (float)((double)u * inv);
    return dt == 0 ? __builtin_bit_cast(uint16_t, (_Float16)q) : __builtin_bit_cast(uint16_t, (__bf16)q);
}

struct Staging {
    int scale;     // s: staged value = x * 2^s
    int fallback;  // 1: the vector cannot be staged exactly; use the fp32 path
};

// Workgroup-wide staging: the raw vector (K halves in LDS, landed and visible
// to every wave) is converted once per workgroup -- every thread takes whole
// 8-value chunks -- into staged[c], chunk c as four fp16 pairs in unpack
// order, (x0,x4) (x1,x5) (x2,x6) (x3,x7).  fp16 values are only permuted; bf16
// values are scaled by 2^s, s = 14 - (largest exponent of the vector), exactly.
// Every thread returns the same {s, fallback}; fallback is set when some value
// cannot be staged exactly (inf/NaN, or a nonzero more than 2^28 below the
// largest), and then staged[] is not to be used.  Up to 16 waves.
__device__ __forceinline__ Staging stage_x_workgroup(const uint16_t *raw, uint4 *staged, int K, int dt) {
    __shared__ int red[48];
    const int tid = threadIdx.x, nthr = blockDim.x, nw = nthr >> 6, wave = tid >> 6;
    const uint4 *r16 = reinterpret_cast<const uint4 *>(raw);
    const int n8 = K >> 3;
    int emax = -100000, bad = 0;
    if (dt != 0) {
        for (int c = tid; c < n8; c += nthr) {
            const uint4 v = r16[c];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = act_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, dt);
                if (!__builtin_isfinite(f)) bad = 1;
                else if (f != 0.0f) emax = max(emax, f32_exponent(f));
            }
        }
        emax = wave_max_i32(emax);
        bad = wave_or_i32(bad);
        if ((tid & 63) == 0) {
            red[wave] = emax;
            red[16 + wave] = bad;
        }
        lds_barrier();
        emax = -100000;
        bad = 0;
        for (int i = 0; i < nw; ++i) {
            emax = max(emax, red[i]);
            bad |= red[16 + i];
        }
    }
    const int scale = (dt == 0 || emax == -100000) ? 0 : 14 - emax;
    int lost = bad;
    if (!bad) {
        for (int c = tid; c < n8; c += nthr) {
            const uint4 v = r16[c];
            if (dt == 0) {
                staged[c] = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                       __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                       __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                       __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
            } else {
                const uint32_t b[4] = {v.x, v.y, v.z, v.w};
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    f[e] = act_to_f32((b[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, dt);
                    if (f[e] != 0.0f && f32_exponent(f[e]) < emax - 28) lost = 1;
                }
                uint32_t o[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    h2 t;
                    t[0] = (_Float16)__builtin_ldexpf(f[p], scale);
                    t[1] = (_Float16)__builtin_ldexpf(f[p + 4], scale);
                    o[p] = __builtin_bit_cast(uint32_t, t);
                }
                staged[c] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
    lost = wave_or_i32(lost);
    if ((tid & 63) == 0) red[32 + wave] = lost;
    lds_barrier();
    int fallback = 0;
    for (int i = 0; i < nw; ++i) fallback |= red[32 + i];
    return Staging{scale, fallback};
}

// The staged pairs of group g (4 chunks) into registers.
__device__ __forceinline__ void load_staged_group(const uint4 *staged, int g, h2 *xr) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint4 v = staged[g * 4 + w];
        xr[w * 4 + 0] = as_h2(v.x);
        xr[w * 4 + 1] = as_h2(v.y);
        xr[w * 4 + 2] = as_h2(v.z);
        xr[w * 4 + 3] = as_h2(v.w);
    }
}

// Staging of a raw activation vector: stage_issue() requests all of x straight
// into LDS (global_load_lds_dwordx4: no registers; each wave moves 64 chunks of
// 16 bytes per instruction); a kernel using it issues its first weight loads
// and waits for every outstanding load (wait_vmcnt<0>) before reading the
// staged bytes, since with the builtin the compiler does not promise to keep
// the weight loads after the activation loads.  stage_issue_ordered() (below)
// makes the same requests as inline assembly, which later loads stay behind,
// so that a wait for the activations alone suffices.
// `raw` needs stage_raw_halves(K) halves.
__device__ __forceinline__ bool stage_vector_path(const uint16_t *x) {
    return (reinterpret_cast<uintptr_t>(x) & 15) == 0;
}

__host__ __device__ constexpr int stage_raw_halves(int K) {
    return ((K / 8 + 63) / 64) * 64 * 8;
}

__device__ __forceinline__ void stage_issue(const uint16_t *__restrict__ x, int K, uint16_t *raw) {
    const int n16 = K >> 3;
    if (!stage_vector_path(x) || n16 == 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint4 *x16 = reinterpret_cast<const uint4 *>(x);
    uint4 *r16 = reinterpret_cast<uint4 *>(raw);
    for (int c0 = wave * 64; c0 < n16; c0 += (int)blockDim.x) {
        const int c = min(c0 + lane, n16 - 1);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(x16 + c),
            (__attribute__((address_space(3))) void *)(r16 + c0), 16, 0, 0);
    }
}


// Direct-to-LDS 16-byte load written as inline assembly, for pipelines that
// keep several such loads in flight and wait for them by count themselves
// (wait_vmcnt_mem).  Given the builtin, the compiler's wait insertion treats
// every later LDS read as possibly reading this load's destination and waits for
// all outstanding loads before it, which would drain the pipeline each step.
// Lane i writes 16 bytes at lds + 16*i; `lds` must be wave-uniform; the loads
// are marked non-temporal (weights are read once).  M0 carries
// the LDS address and is set here; none of the kernels using this keeps a
// compiler-managed M0 value live across it.
__device__ __forceinline__ void lds_dma16(const void *g, void *lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m) : "memory");
}

// The 4-byte form (lane i writes 4 bytes at lds + 4*i).
__device__ __forceinline__ void lds_dma4(const void *g, void *lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt" ::"v"(g), "s"(m) : "memory");
}

// The same load with a wave-uniform 64-bit base in scalar registers and a
// per-lane 32-bit byte offset, marked non-temporal (the data are read once:
// measured on MI355X, streaming reads run markedly faster with this hint).
__device__ __forceinline__ void lds_dma16_nt(const void *sbase, uint32_t voff, void *lds) {
    // (readfirstlane returns a signed int: widen each half as unsigned, or the
    // low half would be sign-extended into the high one)
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    sbase = (const void *)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m)
                 : "memory");
}

// Direct-to-LDS load with a wave-uniform base (scalar registers), a per-lane
// 32-bit byte offset and a wave-uniform LDS byte address (lane i writes 16
// bytes at lds_addr + 16*i); NT marks it non-temporal.
template <bool NT>
__device__ __forceinline__ void lds_dma16_so(const void *sbase, uint32_t voff, uint32_t lds_addr) {
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    sbase = (const void *)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m)
                     : "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m)
                     : "memory");
}

// Wait until at most `pending` vector-memory operations are outstanding, as an
// asm statement with a memory clobber, so that no LDS read is moved above it.
template <int pending>
__device__ __forceinline__ void wait_vmcnt_mem() {
    static_assert(pending >= 0 && pending < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(pending) : "memory");
}

// stage_issue's requests written as inline assembly (with a memory clobber), so
// that loads issued after them stay after them: a wait for at most n
// outstanding loads, n the number of load instructions issued since, then
// covers the activations alone.  Not marked non-temporal: every workgroup
// reads x.
__device__ __forceinline__ void stage_issue_ordered(const uint16_t *__restrict__ x, int K, uint16_t *raw) {
    const int n16 = K >> 3;
    if (n16 == 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint4 *r16 = reinterpret_cast<uint4 *>(raw);
    for (int c0 = wave * 64; c0 < n16; c0 += (int)blockDim.x) {
        const int c = min(c0 + lane, n16 - 1);
        lds_dma16_so<false>(x, (uint32_t)c * 16u,
                            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)(r16 + c0));
    }
}

// Wait until at most n (wave-uniform) vector-memory instructions of this wave
// are outstanding; counts past 63 wait until at most 63 are (a binary search
// down to an immediate).
template <int Lo = 0, int Hi = 63>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    if constexpr (Lo == Hi) {
        wait_vmcnt_mem<Lo>();
    } else {
        constexpr int Mid = (Lo + Hi) / 2;
        if (n <= Mid)
            wait_vmcnt_upto<Lo, Mid>(n);
        else
            wait_vmcnt_upto<Mid + 1, Hi>(n);
    }
}

// Wait until at most `pending` vector-memory loads are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima so they are not waited for).
template <int pending>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(pending >= 0 && pending < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((pending & 15) | ((pending >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace w4
