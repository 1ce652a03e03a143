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
//      arithmetic as w4_rms_renorm, bit for bit), read with agent-coherent
//      16-byte loads all issued at once; fp16 operands are exact as they are,
//      so each wave only permutes them into the pair layout of the GEMV;
//   2. the rows of this workgroup (a row mapping chosen from the shape), the
//      results written with agent-scope stores;
//   3. the barrier: every wave waits for its stores, the workgroup stores its
//      generation into its own flag and wave 0 polls all flags (agent scope,
//      bounded; no contended read-modify-write), while waves 1..3 pull this
//      workgroup's share of the NEXT matrix into L2 with LDS-DMA loads into a
//      scratch LDS area, so that the next step reads its weights from L2.
// Outputs of every step are read back with agent-scope loads, which see the
// stores of workgroups on other XCDs.  One workgroup of eight waves per CU.
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

constexpr int kChainThreads = 512;  // eight waves; the renorm uses the first four
constexpr int kChainMaxK = 8192;
constexpr int kPrefetchBytes = 32768;  // LDS scratch for the L2 prefetch
// sync buffer: word 0 exit counter, word 1 epoch (barrier generations used by
// earlier calls), word 2 error; from word 64 on, one arrival flag per
// workgroup (the generation it last reached).
constexpr int kSyncExit = 0, kSyncEpoch = 1, kSyncError = 2, kSyncFlags = 64;
constexpr int kMaxChainWG = (W4_CHAIN_SYNC_BYTES / 4) - kSyncFlags;

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
                                           const uint16_t *raw, float *y) {
    constexpr int SLOTS = kWave / L;
    const int G = K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = lane % L, slot = lane / L;
    const int rows_per_iter = (kChainThreads / 64) * SLOTS;
    int gc[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) gc[i] = min(l + i * L, G - 1);
    // this wave's activations (fp16, staged as they are), LDS -> registers
    h2 xr[NG][16];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = l + i * L;
        if (g < G) {
            permute_group_f16(raw, g, xr[i]);
        } else {
#pragma unroll
            for (int p = 0; p < 16; ++p) xr[i][p] = h2{0, 0};
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
            acc = (g < G) ? __builtin_fmaf(group_dot(q[i], xr[i]), bf16_to_f32(sv[i]), acc) : acc;
        }
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
        if (l == 0 && row < N) store_agent(y + row, acc);
    }
}

// Pull this workgroup's rows of the next matrix (codes, then steps) into L2
// (waves 1.. only; the data land in a scratch LDS area that nobody reads).
__device__ __forceinline__ void chain_prefetch(const ChainMat &m, int nwg, uint4 *scratch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = kChainThreads / 64 - 1;  // prefetching waves
    if (wave == 0) return;
    const int G = m.K >> 5;
    const ChainVariant vs = variant_shape(chain_variant(m.N, G, nwg));
    const int rows_per_iter = (kChainThreads / 64) * (kWave / vs.L);
    int budget = kPrefetchBytes / 16;  // 16-byte chunks this workgroup may pull
    int dst = 0;
    auto pull = [&](const uint4 *base, long first, int chunks) __attribute__((always_inline)) {
        for (int c0 = (wave - 1) * 64; c0 < chunks; c0 += nw * 64) {
            const int c = min(c0 + lane, chunks - 1);
            const int d = (dst + c0) % (kPrefetchBytes / 16 - 63);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(base + first + c),
                (__attribute__((address_space(3))) void *)(scratch + d), 16, 0, 0);
        }
        dst += chunks;
    };
    for (int row0 = blockIdx.x * rows_per_iter; row0 < m.N && budget > 0; row0 += nwg * rows_per_iter) {
        const int nrows = min(rows_per_iter, m.N - row0);
        const int chunks = min(nrows * G, budget);
        pull(reinterpret_cast<const uint4 *>(m.codes), (long)row0 * G, chunks);
        budget -= chunks;
        // the steps of these rows: the 16-byte chunks lying wholly inside
        // their nrows*G bf16 values (never past the end of the step array)
        const long s_first = ((long)row0 * G * 2 + 15) / 16;
        const long s_end = ((long)(row0 + nrows) * G * 2) / 16;
        const int s_chunks = (int)min((long)budget, s_end - s_first);
        if (s_chunks > 0 && (reinterpret_cast<uintptr_t>(m.steps) & 15) == 0) {
            pull(reinterpret_cast<const uint4 *>(m.steps), s_first, s_chunks);
            budget -= s_chunks;
        }
    }
}

// Grid barrier to generation `gen`.  No read-modify-write on a shared word:
// each workgroup stores `gen` into its own flag, then wave 0 reads every
// workgroup's flag (agent-coherent loads, all issued at once, one or more per
// lane) until all have reached `gen`, with a bounded number of polls; a
// timeout sets the error word.  Meanwhile waves 1..3 pull this workgroup's
// share of the next matrix into L2.  Returns false if the chain must stop.
__device__ __forceinline__ bool chain_barrier(unsigned *sync, unsigned gen, unsigned spin_limit,
                                              const ChainMat *next, int nwg, uint4 *scratch) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are done
    lds_barrier();
    __shared__ int stop_s;
    unsigned *flags = sync + kSyncFlags;
    if (threadIdx.x == 0)
        __hip_atomic_store(flags + blockIdx.x, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (next) chain_prefetch(*next, nwg, scratch);
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const __amdgpu_buffer_rsrc_t fr = buffer_rsrc(flags, nwg * 4);
        unsigned it = 0;
        int stop = 0;
        for (;;) {
            // lane l checks flags l, l+64, ... (four at a time per load)
            int behind = 0;
            for (int f0 = lane * 4; f0 < nwg; f0 += 256) {
                const float4 v = load_coherent_f4(fr, f0 * 4);
                const unsigned a = __float_as_uint(v.x), b = __float_as_uint(v.y);
                const unsigned c = __float_as_uint(v.z), d = __float_as_uint(v.w);
                // generations only grow; compare with wrap-around arithmetic
                behind |= (int)(a - gen) < 0 && f0 + 0 < nwg;
                behind |= (int)(b - gen) < 0 && f0 + 1 < nwg;
                behind |= (int)(c - gen) < 0 && f0 + 2 < nwg;
                behind |= (int)(d - gen) < 0 && f0 + 3 < nwg;
            }
            if (!wave_or_i32(behind)) break;
            if (++it > spin_limit) {
                if (lane == 0)
                    __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                stop = 1;
                break;
            }
        }
        if (lane == 0) stop_s = stop || load_agent_u(sync + kSyncError) != 0;
    }
    lds_barrier();
    return stop_s == 0;
}

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainMat *__restrict__ desc,
                                                              int n, const uint16_t *__restrict__ x0,
                                                              unsigned *sync, unsigned spin_limit) {
    extern __shared__ uint4 smem[];
    uint16_t *raw = reinterpret_cast<uint16_t *>(smem);          // kChainMaxK halves
    uint4 *scratch = smem + (kChainMaxK * 2) / 16;                // kPrefetchBytes
    __shared__ double dred[8];
    const int nwg = gridDim.x;
    const int tid = threadIdx.x;

    // Every workgroup checks the descriptors (same answer everywhere).
    bool ok = n >= 1;
    for (int i = 0; i < n && ok; ++i) {
        const ChainMat m = desc[i];
        if (m.N < 1 || m.K < 32 || (m.K & 31) || m.K > kChainMaxK || !m.codes || !m.steps || !m.y ||
            (reinterpret_cast<uintptr_t>(m.codes) & 15) || (reinterpret_cast<uintptr_t>(m.y) & 15) ||
            (i > 0 && m.K > desc[i - 1].N))
            ok = false;
    }
    if (nwg > kMaxChainWG) ok = false;
    // barrier generations of this call continue from those of earlier calls
    const unsigned epoch = load_agent_u(sync + kSyncEpoch);
    if (ok) {
        for (int i = 0; i < n; ++i) {
            const ChainMat m = desc[i];
            const int K = m.K, G = K >> 5;
            // 1. input into LDS (raw fp16)
            uint4 *r16 = reinterpret_cast<uint4 *>(raw);
            if (i == 0) {
                const uint4 *x16 = reinterpret_cast<const uint4 *>(x0);
                for (int c = tid; c < (K >> 3); c += kChainThreads) r16[c] = x16[c];
            } else {
                // previous output: all of this thread's chunks requested at
                // once with agent-coherent loads, then the canonical sum
                const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(desc[i - 1].y, K * 4);
                constexpr int J = kChainMaxK / 4 / 256;
                float4 v[J];
                const bool rn = tid < 256;  // the canonical 256-thread order
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int c = min((rn ? tid : 0) + 256 * j, (K >> 2) - 1);
                    v[j] = load_coherent_f4(pr, c * 16);
                }
                const double ss = sum_squares_256_regs(K, v, dred, rn);
                if (rn) {
#pragma unroll
                    for (int j = 0; j < J; ++j) {
                        const int c = tid + 256 * j;
                        if (c < (K >> 2)) {
                            const uint32_t lo = renorm_value(v[j].x, ss, K, 0) | ((uint32_t)renorm_value(v[j].y, ss, K, 0) << 16);
                            const uint32_t hi = renorm_value(v[j].z, ss, K, 0) | ((uint32_t)renorm_value(v[j].w, ss, K, 0) << 16);
                            reinterpret_cast<uint2 *>(raw)[c] = make_uint2(lo, hi);
                        }
                    }
                }
            }
            __syncthreads();
            // 2. rows
            const uint4 *codes = reinterpret_cast<const uint4 *>(m.codes);
            switch (__builtin_amdgcn_readfirstlane(chain_variant(m.N, G, nwg))) {
                case 0: chain_rows<64, 1>(codes, m.steps, m.N, K, raw, m.y); break;
                case 1: chain_rows<64, 2>(codes, m.steps, m.N, K, raw, m.y); break;
                case 2: chain_rows<64, 4>(codes, m.steps, m.N, K, raw, m.y); break;
                case 3: chain_rows<16, 3>(codes, m.steps, m.N, K, raw, m.y); break;
                case 4: chain_rows<16, 4>(codes, m.steps, m.N, K, raw, m.y); break;
                default: chain_rows<32, 4>(codes, m.steps, m.N, K, raw, m.y); break;
            }
            // 3. barrier before the next matrix reads this output
            if (i + 1 < n) {
                const ChainMat next = desc[i + 1];
                if (!chain_barrier(sync, epoch + (unsigned)(i + 1), spin_limit, &next, nwg, scratch)) break;
            }
        }
    } else if (blockIdx.x == 0 && tid == 0) {
        __hip_atomic_store(sync + kSyncError, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Exit: the last workgroup out (every other one is past its last barrier
    // and has read the epoch) advances the epoch past this call's generations
    // and returns the exit counter to zero.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(sync + kSyncExit, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)nwg - 1) {
            __hip_atomic_store(sync + kSyncEpoch, epoch + (unsigned)n, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + kSyncExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t chain_lds_bytes() { return (size_t)kChainMaxK * 2 + kPrefetchBytes; }

hipError_t launch_chain(const void *desc, int n, const uint16_t *x0, void *sync, unsigned spin_limit,
                        hipStream_t stream) {
    // One workgroup per CU, all resident together on an otherwise idle device
    // (the occupancy check makes sure one fits per CU).  A plain launch: if
    // some workgroups could not start while others wait, the bounded barrier
    // waits end with the timeout error instead of a hang.
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const size_t lds = chain_lds_bytes();
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, kChainThreads, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus > kMaxChainWG) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chain_kernel, dim3(cus), dim3(kChainThreads), lds, stream,
                       static_cast<const ChainMat *>(desc), n, x0, static_cast<unsigned *>(sync),
                       spin_limit);
    return hipGetLastError();
}

}  // namespace w4
