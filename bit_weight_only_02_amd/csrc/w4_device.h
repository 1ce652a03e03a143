// Device helpers shared by the W4A16 kernels (gfx950 / CDNA4, wave64).
//
// Packed format: codes uint32[N][K/8] (nibble j of word w = column 8w+j), bf16
// steps [N][K/32]; weight = (code - 8) * step.  One 16-byte load (uint4) of a
// row is exactly one group of 32 codes, and it pairs with one bf16 step.
//
// Exact operands.  The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch"
// (section "Step 3 - Multiply Straight From the Packed Weights") turns a code
// into a float by OR-ing it into the bits of 2^23 and subtracting 2^23 + 8.
// Here the same idea runs two lanes at a time in fp16: OR-ing a nibble into
// the mantissa of 1024.0h gives 1024 + c exactly, and one packed subtract of
// 1032 gives c - 8 exactly.  A nibble sitting four bits higher gives 1024 + 16c,
// and one packed FMA (x 1/16, - 72) gives c - 8 exactly.  The packed pairs then
// feed v_dot2_f32_f16, which multiplies fp16 pairs and accumulates in fp32.
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

// Eight codes of one packed word -> four exact fp16 pairs (c - 8), ordered
// (c0,c4), (c1,c5), (c2,c6), (c3,c7).
__device__ __forceinline__ void unpack_word(uint32_t w, h2 &p0, h2 &p1, h2 &p2, h2 &p3) {
    const h2 kSub = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 kInv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 kSub72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t u = w >> 8;
    p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + kSub;
    p1 = as_h2((w & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
    p2 = as_h2((u & 0x000F000Fu) | 0x64006400u) + kSub;
    p3 = as_h2((u & 0x00F000F0u) | 0x64006400u) * kInv16 + kSub72;
}

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Sum over one group of 32 codes: q holds the 4 packed words, xr the 16 staged
// activation pairs of the group in the order unpack_word produces.
__device__ __forceinline__ float group_dot(uint4 q, const h2 *xr) {
    h2 a0, a1, a2, a3;
    float s0 = 0.0f, s1 = 0.0f;
    unpack_word(q.x, a0, a1, a2, a3);
    s0 = dot2(a0, xr[0], s0); s1 = dot2(a1, xr[1], s1);
    s0 = dot2(a2, xr[2], s0); s1 = dot2(a3, xr[3], s1);
    unpack_word(q.y, a0, a1, a2, a3);
    s0 = dot2(a0, xr[4], s0); s1 = dot2(a1, xr[5], s1);
    s0 = dot2(a2, xr[6], s0); s1 = dot2(a3, xr[7], s1);
    unpack_word(q.z, a0, a1, a2, a3);
    s0 = dot2(a0, xr[8], s0); s1 = dot2(a1, xr[9], s1);
    s0 = dot2(a2, xr[10], s0); s1 = dot2(a3, xr[11], s1);
    unpack_word(q.w, a0, a1, a2, a3);
    s0 = dot2(a0, xr[12], s0); s1 = dot2(a1, xr[13], s1);
    s0 = dot2(a2, xr[14], s0); s1 = dot2(a3, xr[15], s1);
    return s0 + s1;
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

// max over the four lanes l, l^16, l^32, l^48 (the 16-lane groups of a wave)
__device__ __forceinline__ int max_across_lane_groups(int v) {
    auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max((int)a[0], (int)a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max((int)b[0], (int)b[1]);
}

// Sum of squares of v[0..K) (K a multiple of 4) in fp64 with one fixed order,
// shared by every kernel that renormalises (so that they agree bit for bit):
// thread t of a 256-thread workgroup owns the 4-element chunks c = t, t+256,
// ... and adds their squares in ascending (c, element) order; the 64 lanes of
// a wave are folded by xor shuffles 32, 16, ..., 1; the four wave sums are
// added in wave order.  load4(c) returns chunk c as a float4.  Every thread
// gets the total.  `red` is 4 doubles of shared scratch.
template <class Load4>
__device__ __forceinline__ double sum_squares_256(int K, Load4 load4, double *red) {
    const int tid = threadIdx.x;
    double ss = 0.0;
    for (int c = tid; c < (K >> 2); c += 256) {
        const float4 v = load4(c);
        ss += (double)v.x * (double)v.x;
        ss += (double)v.y * (double)v.y;
        ss += (double)v.z * (double)v.z;
        ss += (double)v.w * (double)v.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const double tot = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return tot;
}

// The same sum over chunks already in registers: v[j] is chunk tid + 256*j
// (valid while tid + 256*j < K/4), up to J chunks per thread.  Threads with
// `active` false (beyond the first 256 of a larger workgroup) add nothing and
// only take part in the barriers; `red` holds one double per wave.
template <int J>
__device__ __forceinline__ double sum_squares_256_regs(int K, const float4 (&v)[J], double *red,
                                                       bool active = true) {
    const int tid = threadIdx.x;
    double ss = 0.0;
    if (active) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (tid + 256 * j < (K >> 2)) {
                ss += (double)v[j].x * (double)v[j].x;
                ss += (double)v[j].y * (double)v[j].y;
                ss += (double)v[j].z * (double)v[j].z;
                ss += (double)v[j].w * (double)v[j].w;
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if ((tid & 63) == 0 && tid < 256) red[tid >> 6] = ss;
    lds_barrier();
    const double tot = ((red[0] + red[1]) + red[2]) + red[3];
    lds_barrier();
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
    const float q = (float)((double)u * inv);
    return dt == 0 ? __builtin_bit_cast(uint16_t, (_Float16)q) : __builtin_bit_cast(uint16_t, (__bf16)q);
}

// ---- per-wave activation staging -------------------------------------------
// Every wave scans the whole raw vector itself (no cross-wave reduction), then
// each lane converts only the groups it owns, straight from LDS into its
// registers.  The staged value is x * 2^s with s = 14 - (largest exponent):
// every nonzero value must land in the normal fp16 range, i.e. lie within 2^28
// of the largest; otherwise (or with inf/NaN) the wave takes the fp32 path.
struct WaveScale {
    int scale;  // s
    int emax;   // largest exponent (-100000: all zero)
    int bad;    // inf/NaN present
};

// raw: K halves in LDS, 16-byte aligned, K a multiple of 32.
__device__ __forceinline__ WaveScale wave_scan(const uint16_t *raw, int K, int dt) {
    const int lane = threadIdx.x & 63;
    const uint4 *r16 = reinterpret_cast<const uint4 *>(raw);
    int emax = -100000, bad = 0;
    for (int c = lane; c < (K >> 3); c += 64) {
        const uint4 v = r16[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = act_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, dt);
            if (!__builtin_isfinite(f)) bad = 1;
            else if (f != 0.0f) emax = max(emax, f32_exponent(f));
        }
    }
    WaveScale ws;
    ws.emax = wave_max_i32(emax);
    ws.bad = wave_or_i32(bad);
    ws.scale = ws.emax == -100000 ? 0 : 14 - ws.emax;
    return ws;
}

// Group g of raw -> 16 staged pairs in unpack_word order; returns 1 if a value
// cannot be staged exactly.
__device__ __forceinline__ int convert_group(const uint16_t *raw, int g, int dt, const WaveScale &ws,
                                             h2 *xr) {
    const uint4 *r16 = reinterpret_cast<const uint4 *>(raw) + g * 4;
    int lost = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint4 v = r16[w];
        const uint32_t b[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[e] = act_to_f32((b[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, dt);
            if (f[e] != 0.0f && f32_exponent(f[e]) < ws.emax - 28) lost = 1;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            h2 t;
            t[0] = (_Float16)__builtin_ldexpf(f[p], ws.scale);
            t[1] = (_Float16)__builtin_ldexpf(f[p + 4], ws.scale);
            xr[w * 4 + p] = t;
        }
    }
    return lost;
}

// fp16 activations need no scaling: v_dot2_f32_f16 and the f16 MFMA take
// fp16 subnormals as they are (measured on gfx950), so (c - 8) * x is exact in
// fp32 for every fp16 x.  Staging is then only the pair permutation:
// words (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ void permute_group_f16(const uint16_t *raw, int g, h2 *xr) {
    const uint4 *r16 = reinterpret_cast<const uint4 *>(raw) + g * 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint4 v = r16[w];
        // v_perm_b32 selector: bytes 0-3 from src1, 4-7 from src0
        xr[w * 4 + 0] = as_h2(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u));
        xr[w * 4 + 1] = as_h2(__builtin_amdgcn_perm(v.z, v.x, 0x07060302u));
        xr[w * 4 + 2] = as_h2(__builtin_amdgcn_perm(v.w, v.y, 0x05040100u));
        xr[w * 4 + 3] = as_h2(__builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
    }
}

struct Staging {
    int scale;     // s: staged value = x * 2^s
    int fallback;  // 1: the vector cannot be staged exactly; use the fp32 path
};

// Staging of a raw activation vector: stage_issue() requests all of x straight
// into LDS (global_load_lds_dwordx4: no registers; each wave moves 64 chunks of
// 16 bytes per instruction); the kernel then issues its first weight loads and
// waits for every outstanding load (wait_vmcnt<0>) before reading the staged
// bytes.  (Waiting for a partial count would depend on the compiler keeping the
// weight loads after the activation loads, which it does not promise.)
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


// Wait until at most `pending` vector-memory loads are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima so they are not waited for).
template <int pending>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(pending >= 0 && pending < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((pending & 15) | ((pending >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace w4
