// 4-bit vocabulary-table row gather for gfx950.
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 2 -
// Keep the Vocabulary Tables in 4-Bit") keeps the embedding table as 4-bit
// codes with one step per group of 32 and looks rows up on the card; the same
// copy is the output layer.  Row id -> bf16 values (c - 8) * step, rounded to
// nearest-even (the fp32 product is exact, so this is the only rounding).
//
// One wave per output row and slice of kSliceWords packed words (gridDim.y
// slices): lane i handles words i, i+64, ... of the slice (8 codes -> 16
// output bytes each), all of its loads issued before the first store, so loads
// and stores are contiguous and a wide row is spread over several waves.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

constexpr int kSliceWords = 256;  // 4 words per lane

__global__ __launch_bounds__(256) void gather_kernel(const uint32_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ steps,
                                                     int V, int K,
                                                     const int32_t *__restrict__ ids, int n,
                                                     uint16_t *__restrict__ out,
                                                     int32_t *__restrict__ dev_err) {
    const int row_out = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row_out >= n) return;
    const int id = ids[row_out];
    const int words = K >> 3;
    const int w0 = blockIdx.y * kSliceWords;
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

hipError_t launch_gather(const uint32_t *codes, const uint16_t *steps, int V, int K,
                         const int32_t *ids, int n, uint16_t *out, int32_t *dev_err,
                         hipStream_t stream) {
    const int rows_per_block = 4;
    const int blocks = (n + rows_per_block - 1) / rows_per_block;
    const int slices = ((K >> 3) + kSliceWords - 1) / kSliceWords;
    if (blocks > 2147483647 || slices > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gather_kernel, dim3(blocks, slices), dim3(64 * rows_per_block), 0, stream,
                       codes, steps, V, K, ids, n, out, dev_err);
    return hipGetLastError();
}

}  // namespace w4
