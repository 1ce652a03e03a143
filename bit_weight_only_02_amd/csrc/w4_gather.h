// One wave's share of the 4-bit table row gather (gfx950): output row
// row_out, slice `slice` of kSliceWords packed words.  Shared by the gather
// launch and by the product launch that runs the gather beside the
// vocabulary-table product.
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 2 -
// Keep the Vocabulary Tables in 4-Bit") keeps the embedding table as 4-bit
// codes with one step per group of 32 and looks rows up on the card; the same
// copy is the output layer.  Row id -> bf16 values (c - 8) * step, rounded to
// nearest-even (the fp32 product is exact, so this is the only rounding).
// Lane i handles words i, i+64, ... of the slice (8 codes -> 16 output bytes
// each), all of its loads issued before the first store.
#pragma once

#include "w4_device.h"

namespace w4 {

constexpr int kSliceWords = 256;  // 4 words per lane

__device__ __forceinline__ void gather_row_slice(const uint32_t *__restrict__ codes,
                                                 const uint16_t *__restrict__ steps, int V, int K,
                                                 const int32_t *__restrict__ ids, int row_out, int slice,
                                                 uint16_t *__restrict__ out, int32_t *__restrict__ dev_err) {
    const int lane = threadIdx.x & 63;
    const int id = ids[row_out];
    const int words = K >> 3;
    const int w0 = slice * kSliceWords;
    uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)row_out * K);
    if (id < 0 || id >= V) {
        for (int w = w0 + lane; w < min(words, w0 + kSliceWords); w += kWave)
            dst[w] = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
        if (lane == 0 && dev_err) *dev_err = 1;
        return;
    }
    const uint32_t *src = codes + (size_t)id * words;
    const uint16_t *st = steps + (size_t)id * (K >> 5);
    constexpr int U = kSliceWords / kWave;
    uint32_t word[U];
    float step[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int w = min(w0 + lane + u * kWave, words - 1);  // clamped: in bounds, not stored
        word[u] = src[w];
        step[u] = bf16_to_f32(st[w >> 2]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int w = w0 + lane + u * kWave;
        if (w >= words) break;
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float lo = (float)((int)((word[u] >> (8 * p)) & 0xFu) - 8) * step[u];
            const float hi = (float)((int)((word[u] >> (8 * p + 4)) & 0xFu) - 8) * step[u];
            const uint32_t blo = __builtin_bit_cast(uint16_t, (__bf16)lo);
            const uint32_t bhi = __builtin_bit_cast(uint16_t, (__bf16)hi);
            o[p] = blo | (bhi << 16);
        }
        dst[w] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace w4
