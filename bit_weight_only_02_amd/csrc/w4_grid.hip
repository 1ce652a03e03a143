// Grid packing of a 16-bit table into 4-bit codes and bf16 steps, for gfx950.
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 2 -
// Keep the Vocabulary Tables in 4-Bit") notes that the 16-bit vocabulary and
// per-layer tables were trained onto a grid of at most 16 levels per group of
// 32, and stores them as 4-bit codes with each group's step recovered from the
// grid.  The page does not say how; the rule here: the group's extreme value
// sets the step -- a negative extreme larger in magnitude than every positive
// value is 8 steps below zero (code 0), otherwise the largest positive value is
// 7 steps above (code 15) -- the step is rounded to bf16, and every value gets
// code clamp(rint(q) + 8, 0, 15) in fp32, q = v times the correctly rounded
// reciprocal of the step (ties to even).  Exact grid values that use code 0 or 15 come back as the
// codes and step they were made from.
//
// Four adjacent lanes per group, each with 8 values (one 16-byte load) and one
// code word to store; the group's extremes meet by quad exchanges.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// (contraction off: every rounding below is the one written)
#pragma clang fp contract(off)
__global__ __launch_bounds__(256) void grid_pack_kernel(const uint4 *__restrict__ table, long groups,
                                                        uint32_t *__restrict__ codes,
                                                        uint16_t *__restrict__ steps) {
    // four adjacent lanes per group, 8 values (16 bytes) each: loads and code
    // stores are contiguous across the wave
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
        // the group's extremes over its 4 lanes (quad exchanges 1 and 2 apart)
        an = fmaxf(an, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(an), 0xB1, 0xF, 0xF, false)));
        ap = fmaxf(ap, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ap), 0xB1, 0xF, 0xF, false)));
        an = fmaxf(an, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(an), 0x4E, 0xF, 0xF, false)));
        ap = fmaxf(ap, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ap), 0x4E, 0xF, 0xF, false)));
        const float s = an > ap ? an / 8.0f : ap / 7.0f;
        const uint16_t sb = __builtin_bit_cast(uint16_t, (__bf16)s);
        const float sf = bf16_to_f32(sb);
        // quotient v / sf as v times the reciprocal (correctly rounded, once
        // per group)
        const float r = sf != 0.0f ? 1.0f / sf : 0.0f;
        // clamp(rint(q) + 8, 0, 15) as clamp(q, -8, 7) + (2^23 + 8): the add
        // rounds to an integer (ties to even) and leaves the code in the low
        // mantissa bits; the two orders agree for every finite q
        uint32_t wd = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = v[j];
            const float q = __builtin_amdgcn_fmed3f(x * r, -8.0f, 7.0f) + 8388616.0f;
            wd |= (__float_as_uint(q) & 0xFu) << (4 * j);
        }
        if (sf == 0.0f) wd = 0x88888888u;
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
