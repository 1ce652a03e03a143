// A decode-step chain of W4A16 products as one persistent launch (gfx950).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 4 -
// Replay Each Decode Step as One CUDA Graph") notes that a decode step is
// hundreds of small kernels and that launching them one by one costs more than
// running them; its tip "Merge the Small Projections" merges q/k/v and gate/up
// into one matrix each.  Here the whole chain of merged matrices runs inside
// one kernel: every workgroup stays resident, takes its share of the rows of
// matrix i, and a grid-wide barrier separates matrix i from matrix i+1 (whose
// input is the renormalised output of matrix i and so needs all of it).
//
// Per step:
//   1. input: x0 for the first matrix, else the leading K entries of the
//      previous output divided by their RMS and rounded to fp16 (the same
//      arithmetic as w4_rms_renorm, so that results are bitwise those of the
//      separate calls), staged as exactly scaled fp16 like the GEMV;
//   2. the rows of this workgroup (a row mapping chosen from the shape), the
//      results written with agent-scope stores;
//   3. the barrier: every wave waits for its stores, then wave 0 adds to a
//      counter and polls it (agent scope, bounded), while waves 1..3 pull this
//      workgroup's share of the NEXT matrix into L2 with LDS-DMA loads into a
//      scratch LDS area, so that the next step reads its weights from L2.
// Outputs of every step are read back with agent-scope loads, which see the
// stores of workgroups on other XCDs.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4.h"
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

struct ChainMat {
    const uint32_t *codes;
    const uint16_t *steps;
    float *y;
    int32_t N;
    int32_t K;
};
static_assert(sizeof(ChainMat) == sizeof(w4_chain_mat), "descriptor layout");

constexpr int kChainThreads = 256;
constexpr int kChainMaxK = 8192;
constexpr int kPrefetchBytes = 32768;  // LDS scratch for the L2 prefetch
// sync words
constexpr int kSyncArrive = 0, kSyncExit = 1, kSyncError = 2;

__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_agent_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row mapping of one step: lanes per row L and groups per lane NG.
struct ChainVariant {
    int L, NG;
};

__device__ __forceinline__ int chain_variant(int N, int G, int nwg) {
    // Few lane-tasks (one 16-byte group each): spread them, 64 lanes per row.
    // Many: 16 or 32 lanes per row with several groups per lane.
    const long tasks = (long)N * G, lanes = (long)nwg * kChainThreads;
    if (tasks <= 2 * lanes) return G <= 64 ? 0 : (G <= 128 ? 1 : 2);
    if (G <= 48) return 3;
    if (G <= 64) return 4;
    if (G <= 128) return 5;
    return 2;
}

__device__ __forceinline__ ChainVariant variant_shape(int v) {
    switch (v) {
        case 0: return {64, 1};
        case 1: return {64, 2};
        case 2: return {64, 4};
        case 3: return {16, 3};
        case 4: return {16, 4};
        default: return {32, 4};
    }
}

template <int L, int NG>
__device__ __forceinline__ void chain_rows(const uint4 *__restrict__ codes,
                                           const uint16_t *__restrict__ steps, int N, int K,
                                           const _Float16 *xs, const uint16_t *raw,
                                           const Staging &st, float *y) {
    constexpr int SLOTS = kWave / L;
    const int G = K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = lane % L, slot = lane / L;
    const int rows_per_iter = (kChainThreads / 64) * SLOTS;
    int gc[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) gc[i] = min(l + i * L, G - 1);
    h2 xr[NG][16];
    if (!st.fallback) {
        const h2 *xs2 = reinterpret_cast<const h2 *>(xs);
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
#pragma unroll
            for (int p = 0; p < 16; ++p) xr[i][p] = (g < G) ? xs2[g * 16 + p] : h2{0, 0};
        }
    }
    for (int row0 = blockIdx.x * rows_per_iter; row0 < N; row0 += gridDim.x * rows_per_iter) {
        const int row = row0 + wave * SLOTS + slot;
        const int rc = min(row, N - 1);
        uint4 q[NG];
        uint32_t sv[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            q[i] = codes[(size_t)rc * G + gc[i]];
            sv[i] = steps[(size_t)rc * G + gc[i]];
        }
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            const float part = st.fallback ? group_dot_f32(q[i], raw + gc[i] * 32, 0)
                                           : group_dot(q[i], xr[i]);
            acc = (g < G) ? __builtin_fmaf(part, bf16_to_f32(sv[i]), acc) : acc;
        }
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
        if (l == 0 && row < N)
            store_agent(y + row, st.fallback ? acc : __builtin_ldexpf(acc, -st.scale));
    }
}

// Pull this workgroup's rows of the next matrix into L2 (waves 1..3 only; the
// data land in a scratch LDS area that nobody reads).
__device__ __forceinline__ void chain_prefetch(const ChainMat &m, int nwg, uint4 *scratch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave == 0) return;
    const int G = m.K >> 5;
    const ChainVariant vs = variant_shape(chain_variant(m.N, G, nwg));
    const int rows_per_iter = (kChainThreads / 64) * (kWave / vs.L);
    const uint4 *codes = reinterpret_cast<const uint4 *>(m.codes);
    int budget = kPrefetchBytes / 16;  // 16-byte chunks this workgroup may pull
    int dst = 0;
    for (int row0 = blockIdx.x * rows_per_iter; row0 < m.N && budget > 0; row0 += nwg * rows_per_iter) {
        const int nrows = min(rows_per_iter, m.N - row0);
        const long first = (long)row0 * G;
        const int chunks = min(nrows * G, budget);
        for (int c0 = (wave - 1) * 64; c0 < chunks; c0 += 3 * 64) {
            const int c = min(c0 + lane, chunks - 1);
            const int d = (dst + c0) % (kPrefetchBytes / 16 - 63);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(codes + first + c),
                (__attribute__((address_space(3))) void *)(scratch + d), 16, 0, 0);
        }
        budget -= chunks;
        dst += chunks;
    }
}

// Grid barrier number `gen` (1-based).  Stores of every wave complete first;
// wave 0 of each workgroup arrives and polls with a bounded spin; a timeout
// sets the error word.  Returns false if the chain must stop.
__device__ __forceinline__ bool chain_barrier(unsigned *sync, unsigned gen, unsigned spin_limit,
                                              const ChainMat *next, int nwg, uint4 *scratch) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are done
    lds_barrier();
    __shared__ int stop_s;
    if (next) chain_prefetch(*next, nwg, scratch);
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(sync + kSyncArrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned target = gen * (unsigned)nwg;
        unsigned it = 0;
        int stop = 0;
        while (load_agent_u(sync + kSyncArrive) < target) {
            if (++it > spin_limit) {
                __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                stop = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (load_agent_u(sync + kSyncError) != 0) stop = 1;
        stop_s = stop;
    }
    lds_barrier();
    return stop_s == 0;
}

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainMat *__restrict__ desc,
                                                              int n, const uint16_t *__restrict__ x0,
                                                              unsigned *sync, unsigned spin_limit) {
    extern __shared__ uint4 smem[];
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);            // kChainMaxK halves
    uint16_t *raw = reinterpret_cast<uint16_t *>(xs + kChainMaxK);  // kChainMaxK halves
    uint4 *scratch = smem + (2 * kChainMaxK * 2) / 16;              // kPrefetchBytes
    __shared__ double dred[4];
    __shared__ int ired[8];
    const int nwg = gridDim.x;
    const int tid = threadIdx.x;

    // Every workgroup checks the descriptors (same answer everywhere).
    bool ok = n >= 1;
    for (int i = 0; i < n && ok; ++i) {
        const ChainMat m = desc[i];
        if (m.N < 1 || m.K < 32 || (m.K & 31) || m.K > kChainMaxK || !m.codes || !m.steps || !m.y ||
            (reinterpret_cast<uintptr_t>(m.codes) & 15) || (i > 0 && m.K > desc[i - 1].N))
            ok = false;
    }
    if (ok) {
        for (int i = 0; i < n; ++i) {
            const ChainMat m = desc[i];
            const int K = m.K, G = K >> 5;
            // 1. input
            if (i == 0) {
                for (int k = tid; k < K; k += kChainThreads) raw[k] = x0[k];
            } else {
                const float *prev = desc[i - 1].y;
                const double ss = sum_squares_256(K, [&](int k) { return load_agent(prev + k); }, dred);
                for (int k = tid; k < K; k += kChainThreads) raw[k] = renorm_value(load_agent(prev + k), ss, K, 0);
            }
            __syncthreads();
            const Staging st = stage_convert(K, 0, xs, raw, ired);
            // 2. rows
            const uint4 *codes = reinterpret_cast<const uint4 *>(m.codes);
            switch (__builtin_amdgcn_readfirstlane(chain_variant(m.N, G, nwg))) {
                case 0: chain_rows<64, 1>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
                case 1: chain_rows<64, 2>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
                case 2: chain_rows<64, 4>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
                case 3: chain_rows<16, 3>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
                case 4: chain_rows<16, 4>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
                default: chain_rows<32, 4>(codes, m.steps, m.N, K, xs, raw, st, m.y); break;
            }
            // 3. barrier before the next matrix reads this output
            if (i + 1 < n) {
                const ChainMat next = desc[i + 1];
                if (!chain_barrier(sync, (unsigned)(i + 1), spin_limit, &next, nwg, scratch)) break;
            }
        }
    } else if (blockIdx.x == 0 && tid == 0) {
        __hip_atomic_store(sync + kSyncError, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Exit: the last workgroup out (every other one is past its last barrier)
    // returns the counters to zero for the next call.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(sync + kSyncExit, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)nwg - 1) {
            __hip_atomic_store(sync + kSyncArrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + kSyncExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t chain_lds_bytes() { return (size_t)2 * kChainMaxK * 2 + kPrefetchBytes; }

hipError_t launch_chain(const void *desc, int n, const uint16_t *x0, void *sync, unsigned spin_limit,
                        hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const size_t lds = chain_lds_bytes();
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, kChainThreads, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    if (per_cu > 2) per_cu = 2;
    const ChainMat *d = static_cast<const ChainMat *>(desc);
    unsigned *s = static_cast<unsigned *>(sync);
    void *args[] = {&d, &n, &x0, &s, &spin_limit};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(chain_kernel), dim3(cus * per_cu),
                                      dim3(kChainThreads), args, (unsigned)lds, stream);
}

}  // namespace w4
