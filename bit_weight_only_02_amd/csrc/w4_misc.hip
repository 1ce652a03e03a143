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

// The same for K <= 8192, with each thread's chunks kept in registers between
// the sum of squares (the same order: chunks t, t+256, ... ascending, then
// wave_sum_f64, then the four wave sums in order) and the writes, and a single
// workgroup barrier.  Bitwise the result of rms_renorm_kernel.
constexpr int kRenormRegJ = 8;  // chunks per thread: K <= 256 * 4 * 8

__global__ __launch_bounds__(256) void rms_renorm_reg_kernel(const float *__restrict__ v0, long ldv,
                                                             int K, uint16_t *__restrict__ out0,
                                                             long ldo, int out_dt) {
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const float *v = v0 + (long)blockIdx.x * ldv;
    uint16_t *out = out0 + (long)blockIdx.x * ldo;
    const bool vec = (reinterpret_cast<uintptr_t>(v) & 15) == 0;
    const bool ovec = (reinterpret_cast<uintptr_t>(out) & 7) == 0;
    const int n4 = K >> 2;
    const int jn = (n4 + 255) >> 8;  // uniform
    float4 x[kRenormRegJ];
#pragma unroll
    for (int j = 0; j < kRenormRegJ; ++j) {
        const int c = tid + 256 * j;
        x[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (j < jn && c < n4)
            x[j] = vec ? reinterpret_cast<const float4 *>(v)[c]
                       : make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
    }
    // (chunks past the end are zeros: adding +0 leaves the sum's bits alone)
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kRenormRegJ; ++j) {
        if (j < jn) {
            ss += (double)x[j].x * (double)x[j].x;
            ss += (double)x[j].y * (double)x[j].y;
            ss += (double)x[j].z * (double)x[j].z;
            ss += (double)x[j].w * (double)x[j].w;
        }
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const double inv = renorm_scale(((red[0] + red[1]) + red[2]) + red[3], K);
#pragma unroll
    for (int j = 0; j < kRenormRegJ; ++j) {
        const int c = tid + 256 * j;
        if (j < jn && c < n4) {
            const uint32_t h0 = renorm_value(x[j].x, inv, out_dt), h1 = renorm_value(x[j].y, inv, out_dt);
            const uint32_t h2 = renorm_value(x[j].z, inv, out_dt), h3 = renorm_value(x[j].w, inv, out_dt);
            if (ovec) {
                reinterpret_cast<uint2 *>(out)[c] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
            } else {
                out[4 * c] = (uint16_t)h0;
                out[4 * c + 1] = (uint16_t)h1;
                out[4 * c + 2] = (uint16_t)h2;
                out[4 * c + 3] = (uint16_t)h3;
            }
        }
    }
}

hipError_t launch_rms_renorm(const float *v, long ldv, int K, int rows, void *out, long ldo,
                             int out_dt, hipStream_t stream) {
    if (K <= 256 * 4 * kRenormRegJ)
        hipLaunchKernelGGL(rms_renorm_reg_kernel, dim3(rows), dim3(256), 0, stream, v, ldv, K,
                           static_cast<uint16_t *>(out), ldo, out_dt);
    else
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
