// Grid packing of a 16-bit table into 4-bit codes and bf16 steps, for gfx950.
//
// Source: the dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch", section
// "Step 2 - Keep the Vocabulary Tables in 4-Bit".  Its 16-bit tables were
// trained so that each group of 32 takes at most 16 distinct values, and its
// 4-bit tables keep, per group, codes and a step taken from those values.
// The page leaves the recovery open; the rule implemented here, per group:
//   - all zero: step 0, every code 8;
//   - else the coarsest exact grid: the largest bf16 step s such that every
//     value is m * s with m an integer in [-8, 7].  The candidates are the
//     negative extreme an divided by j = 1..8 (with no negative value, the
//     positive extreme ap divided by i = 1..7), largest first, each counting
//     only if it is a bf16 value (checked as s * j == an, an exact product);
//   - else (values on no such grid) the extreme sets it: an / 8 when an > ap,
//     otherwise ap / 7, rounded to bf16 (ties to even);
//   - code = clamp(rint(v / s) + 8, 0, 15) on the exact quotient.
//
// The quotient: q0 = v * r with r = 1/s, the residual e = v - q0 * s (one
// fused multiply-add, exact: v and s carry 8 significant bits, so e needs
// about 10), and q1 = q0 + e * r (a second fused multiply-add) is the quotient
// rounded to fp32 up to a term far below half an ulp.  A quotient that is a
// half-integer is an fp32 value and comes out exactly; any other lies at
// least 2^-12 of its size from a half-integer.  So rint(q1) is rint of the
// exact quotient, ties to even included.  Groups whose values are all below
// 2^-96 are scaled by 2^96 (exactly) first, so that 1/s stays finite, and
// groups above 2^96 by 2^-64, so that the exact products below stay finite.
//
// The search.  Every candidate e / j divides e / 840 (840 = lcm(1..8)), so a
// group on any such grid has every value a multiple of e / 840, of magnitude
// at most 8 e, and no nonzero value below e / 8.  One test of that (with the
// group's single reciprocal 1 / e) passes over the groups of arbitrary tables;
// the candidates of the rest are tested exactly: v is a multiple m of e / j
// when m = rint(v * j / e) gives m * e == v * j, both products exact.
//
// Four adjacent lanes per group, each with 8 values (one 16-byte load) and one
// code word to store; the group's extremes and every group-wide test meet by
// quad exchanges.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// (contraction off: every rounding below is the one written)
#pragma clang fp contract(off)

namespace {

// x rounded to the nearest bf16 value, ties to even (finite x), as an fp32
__device__ __forceinline__ float bf16_round(float x) {
    uint32_t b = __float_as_uint(x);
    b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
    return __uint_as_float(b);
}

// the same value on the four lanes of a quad (a group's lanes)
__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
    return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ bool quad_all(bool p) {
    int x = p ? 1 : 0;
    x &= __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
    x &= __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
    return x != 0;
}

}  // namespace

__global__ __launch_bounds__(256) void grid_pack_kernel(const uint4 *__restrict__ table, long groups,
                                                        uint32_t *__restrict__ codes,
                                                        uint16_t *__restrict__ steps) {
    // four adjacent lanes per group, 8 values (16 bytes) each: loads and code
    // stores are contiguous across the wave.  (4 * groups is a multiple of 4,
    // so the quads of a wave are whole groups and leave the loop together.)
    const int part = threadIdx.x & 3;
    for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < 4 * groups;
         idx += (long)gridDim.x * blockDim.x) {
        const long gi = idx >> 2;
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(table) + idx);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
        float v[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[2 * h] = bf16_to_f32(w[h] & 0xFFFFu);
            v[2 * h + 1] = bf16_to_f32(w[h] >> 16);
        }
        float an = 0.0f, ap = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            an = fmaxf(an, -v[k]);
            ap = fmaxf(ap, v[k]);
        }
        an = quad_max(an);
        ap = quad_max(ap);
        // tiny and huge groups are scaled (exactly) so that reciprocals and the
        // exact products of the search stay finite
        const float mx = fmaxf(an, ap);
        const float sc = mx < 0x1p-96f ? 0x1p96f : (mx > 0x1p96f ? 0x1p-64f : 1.0f);
        float vs[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) vs[k] = v[k] * sc;
        float step = 0.0f, ss = 0.0f;  // the step, and the step times sc
        if (mx > 0.0f) {
            const float eu = an > 0.0f ? an : ap;  // the extreme the candidates divide
            const float e = eu * sc;
            const float re = 1.0f / e;
            // The test every grid group passes (see above), on the lane's first
            // value alone: groups of an arbitrary table nearly always fail it
            // there, and a wave with no group left skips the search (a
            // wave-uniform branch).  A candidate that no group of the wave has
            // is skipped; the others are tested on two values per lane first
            // and on the other six only in waves where some group passed; a
            // candidate's full test is the definition itself, so passing the
            // first test is needed, not trusted.
            auto on840 = [&](int k) __attribute__((always_inline)) {
                const float t = vs[k] * 840.0f;
                const float m = __builtin_rintf(t * re);
                return m * e == t && fabsf(m) <= 6720.0f && (v[k] == 0.0f || fabsf(v[k]) >= eu * 0.125f);
            };
            const bool grid = quad_all(on840(0));
            bool found = false;
            if (__builtin_amdgcn_ballot_w64(grid) != 0) {
                // the coarsest exact grid: candidates e / j, largest first
                const int jmax = an > 0.0f ? 8 : 7;
#pragma unroll
                for (int j = 1; j <= 8; ++j) {
                    const float fj = (float)j;
                    // e / j when that is a bf16 value: a candidate within two
                    // fp32 ulps of it rounds to it, and s * j == e is exact
                    const float s = bf16_round(e * (1.0f / fj));
                    const float u = s * (1.0f / sc);  // the step itself
                    const bool cand = grid && !found && j <= jmax && s * fj == e && u * sc == s &&
                                      (__float_as_uint(u) & 0xFFFFu) == 0u;
                    auto on_grid = [&](int k) __attribute__((always_inline)) {
                        const float t = vs[k] * fj;
                        const float m = __builtin_rintf(t * re);
                        return m * e == t && m >= -8.0f && m <= 7.0f;
                    };
                    bool ok = false;
                    if (__builtin_amdgcn_ballot_w64(cand) != 0) {
                        ok = quad_all(cand && on_grid(0) && on_grid(1));
                        if (__builtin_amdgcn_ballot_w64(ok) != 0) {
#pragma unroll
                            for (int k = 2; k < 8; ++k) ok = ok && on_grid(k);
                            ok = quad_all(ok);
                        }
                    }
                    if (ok) {
                        step = u;
                        ss = s;
                        found = true;
                    }
                }
            }
            if (!found) {
                step = bf16_round(an > ap ? an / 8.0f : ap / 7.0f);
                ss = step * sc;
            }
        }
        const uint16_t sb = (uint16_t)(__float_as_uint(step) >> 16);
        uint32_t wd = 0x88888888u;
        if (ss != 0.0f) {
            const float r = 1.0f / ss;
            wd = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q0 = vs[j] * r;
                const float e = __builtin_fmaf(-q0, ss, vs[j]);
                const float q1 = __builtin_fmaf(e, r, q0);
                // clamp(rint(q1) + 8, 0, 15) as clamp(q1, -8, 7) + (2^23 + 8):
                // the add rounds to an integer (ties to even) and leaves the
                // code in the low mantissa bits; the two orders agree for
                // every finite q1
                const float q = __builtin_amdgcn_fmed3f(q1, -8.0f, 7.0f) + 8388616.0f;
                wd |= (__float_as_uint(q) & 0xFu) << (4 * j);
            }
        }
        codes[idx] = wd;
        if (part == 0) steps[gi] = sb;
    }
}

hipError_t launch_grid_pack(const uint16_t *table, long groups, uint32_t *codes, uint16_t *steps,
                            hipStream_t stream) {
    long blocks = (4 * groups + 255) / 256;
    if (blocks > 8192) blocks = 8192;  // 32 waves per CU, each looping over groups
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(grid_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(table), groups, codes, steps);
    return hipGetLastError();
}

}  // namespace w4
