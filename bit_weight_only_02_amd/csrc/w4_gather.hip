// 4-bit vocabulary-table row gather for gfx950.
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 2 -
// Keep the Vocabulary Tables in 4-Bit") keeps the embedding table as 4-bit
// codes with one step per group of 32 and looks rows up on the card; the same
// copy is the output layer.  Row id -> bf16 values (c - 8) * step, rounded to
// nearest-even (the fp32 product is exact, so this is the only rounding).
//
// One wave per output row and slice of kSliceWords packed words (gridDim.y
// slices), so that a wide row is spread over several waves; the wave's work is
// gather_row_slice.
#include "w4_device.h"
#include "w4_gather.h"
#include "w4_internal.h"

namespace w4 {

__global__ __launch_bounds__(256) void gather_kernel(const uint32_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ steps,
                                                     int V, int K,
                                                     const int32_t *__restrict__ ids, int n,
                                                     uint16_t *__restrict__ out,
                                                     int32_t *__restrict__ dev_err) {
    const int row_out = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row_out >= n) return;
    gather_row_slice(codes, steps, V, K, ids, row_out, blockIdx.y, out, dev_err);
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
