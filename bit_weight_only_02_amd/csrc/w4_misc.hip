// Small kernels around the products: the renormalisation between chained
// products, and a plain streaming-read probe.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// Leading K entries u of each row of v -> u / sqrt(mean(u^2)), rounded to
// nearest-even in fp16 (out_dt 0) or bf16 (out_dt 1).  One 256-thread
// workgroup per row, with the canonical sum-of-squares order.
__global__ __launch_bounds__(256) void rms_renorm_kernel(const float *__restrict__ v0, long ldv,
                                                         int K, uint16_t *__restrict__ out0,
                                                         long ldo, int out_dt) {
    __shared__ double red[4];
    const float *v = v0 + (long)blockIdx.x * ldv;
    uint16_t *out = out0 + (long)blockIdx.x * ldo;
    const bool vec = (reinterpret_cast<uintptr_t>(v) & 15) == 0;
    auto load4 = [&](int c) {
        return vec ? reinterpret_cast<const float4 *>(v)[c]
                   : make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
    };
    const double inv = renorm_scale(sum_squares_256(K, load4, red), K);
    for (int k = threadIdx.x; k < K; k += 256) out[k] = renorm_value(v[k], inv, out_dt);
}

hipError_t launch_rms_renorm(const float *v, long ldv, int K, int rows, void *out, long ldo,
                             int out_dt, hipStream_t stream) {
    hipLaunchKernelGGL(rms_renorm_kernel, dim3(rows), dim3(256), 0, stream, v, ldv, K,
                       static_cast<uint16_t *>(out), ldo, out_dt);
    return hipGetLastError();
}

// Streaming read: sum of all 32-bit words (mod 2^32) into *out.  Integer adds
// only, so the result is order independent.  Each workgroup step covers one
// contiguous chunk of 8 * blockDim 16-byte words; every thread has its 8 loads
// in flight at once (indices clamped, so no load sits behind a branch), marked
// non-temporal.  One atomic per workgroup: thousands of atomics on one word
// serialise and would be measured as part of the read.
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void probe_stream_kernel(const uint4 *__restrict__ buf,
                                                           int64_t n16, uint32_t *__restrict__ out) {
    __shared__ uint32_t part[4];
    const int64_t chunk = (int64_t)kProbeUnroll * blockDim.x;
    const u32x4 *b = reinterpret_cast<const u32x4 *>(buf);
    uint32_t s = 0;
    for (int64_t base = (int64_t)blockIdx.x * chunk; base < n16; base += (int64_t)gridDim.x * chunk) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x + threadIdx.x;
            v[u] = __builtin_nontemporal_load(b + (i < n16 ? i : n16 - 1));
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t i = base + (int64_t)u * blockDim.x + threadIdx.x;
            const uint32_t t = v[u].x + v[u].y + v[u].z + v[u].w;
            s += i < n16 ? t : 0u;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(out, part[0] + part[1] + part[2] + part[3]);
}

hipError_t launch_probe_stream(const void *buf, int64_t bytes, uint32_t *out, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    int64_t blocks = (n16 + 256 * kProbeUnroll - 1) / (256 * kProbeUnroll);
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(probe_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4 *>(buf), n16, out);
    return hipGetLastError();
}

}  // namespace w4
