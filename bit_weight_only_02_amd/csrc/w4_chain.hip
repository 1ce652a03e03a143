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
// Per step i (one workgroup of eight waves per CU; workgroup b owns the
// contiguous row block [b*ceil(N/nwg), ...) of every matrix):
//   1. input: x0 for the first matrix, else the leading K entries of the
//      previous output divided by their RMS and rounded to fp16 (the same
//      arithmetic as w4_rms_renorm, bit for bit), read with agent-coherent
//      16-byte loads all issued at once;
//   2. waves 0..3 compute the block's rows of matrix i from an LDS weight
//      buffer (codes and steps staged there in advance) and store them with
//      agent-scope stores, while waves 4..7 stage the block of matrix i+1 into
//      the other buffer with direct-to-LDS loads, so the weight stream of the
//      next step overlaps this step's compute, the barrier and the next
//      renormalisation;
//   3. the barrier: each workgroup stores its generation into its own flag
//      and wave 0 polls all flags (agent scope, bounded; no contended
//      read-modify-write).
// Outputs of every step are read back with agent-scope loads, which see the
// stores of workgroups on other XCDs.  Rows beyond what one buffer holds are
// read from memory directly.
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

constexpr int kChainThreads = 512;  // eight waves
constexpr int kComputeWaves = 7;    // waves 0..6 compute rows (0..3 also renormalise); 7 copies weights
constexpr int kChainMaxK = 8192;
constexpr int kWeightBuf = 64 * 1024;  // bytes of each of the two LDS weight buffers
constexpr int kCopyEarly = 16;         // copy instructions per wave issued before the rows
// sync buffer: word 0 exit counter, word 1 epoch (barrier generations used by
// earlier calls), word 2 error; from word 64 on, one arrival flag per
// workgroup (the generation it last reached), kFlagStride words apart.
// Each flag has a 256-byte line of its own: the pollers' reads then spread over
// many memory channels instead of queueing on the one or two that would hold
// a packed array (measured: 3.0 against 3.8 us per barrier at 256 workgroups).
constexpr int kSyncExit = 0, kSyncEpoch = 1, kSyncError = 2, kSyncFlags = 64;
constexpr int kFlagStride = 64;  // words
constexpr int kMaxChainWG = (W4_CHAIN_SYNC_BYTES / 4 - kSyncFlags) / kFlagStride;

__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Pointers read from the descriptors are generic; the weights are in global
// memory, and saying so keeps their loads off the flat path.
__device__ __forceinline__ uint4 load_global_u4(const uint4 *p, long i) {
    const u32x4 v = ((const __attribute__((address_space(1))) u32x4 *)p)[i];
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_global_u16(const uint16_t *p, long i) {
    return ((const __attribute__((address_space(1))) uint16_t *)p)[i];
}

// One output, stored so that loads with agent scope on any XCD see it.
__device__ __forceinline__ void store_y(float *y, int n, int row, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), buffer_rsrc(y, n * 4), row * 4, 0, 16);
}
__device__ __forceinline__ unsigned load_agent_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rows of one step that this workgroup computes: a contiguous block
// [rb, re); the first nlds of them are staged in an LDS weight buffer (codes,
// then -- when lds_steps -- their steps), the rest are read from memory.
struct RowBlock {
    int rb, re, nlds;
    int steps_chunk;  // uint4 index of the staged steps inside the buffer
    bool lds_steps;
};

__device__ __forceinline__ RowBlock chain_block(const ChainMat &m, int nwg) {
    const int G = m.K >> 5;
    const int rpw = (m.N + nwg - 1) / nwg;
    RowBlock b;
    b.rb = min(m.N, (int)blockIdx.x * rpw);
    b.re = min(m.N, b.rb + rpw);
    // steps travel as 4-byte words: the block's steps must start on one
    b.lds_steps = (G % 2) == 0 && (reinterpret_cast<uintptr_t>(m.steps) & 3) == 0;
    auto bytes = [&](int rows) {
        const int chunks = (rows * G + 63) / 64 * 64;
        const int words = b.lds_steps ? (rows * G / 2 + 63) / 64 * 64 : 0;
        return chunks * 16 + words * 4;
    };
    int n = min(b.re - b.rb, kWeightBuf / (G * 18));
    while (n > 0 && bytes(n) > kWeightBuf) --n;
    b.nlds = n;
    b.steps_chunk = (n * G + 63) / 64 * 64;
    return b;
}

// Copy waves: request the staged part of a block into `buf` (direct-to-LDS
// loads; every lane moves 16 bytes of codes or 4 bytes of steps, and the last
// instruction of each run lands its surplus lanes in the rounding padding).
// Instructions [first, last) of the run are issued (codes first, then steps),
// so that the copy can be split around a barrier.
__device__ __forceinline__ void chain_copy(const ChainMat &m, const RowBlock &b, uint4 *buf,
                                           int first, int last) {
    const int w = (threadIdx.x >> 6) - kComputeWaves, lane = threadIdx.x & 63;
    constexpr int nw = kChainThreads / 64 - kComputeWaves;
    const int G = m.K >> 5;
    const int n = b.nlds * G;
    if (n == 0) return;
    int k = 0;  // this wave's instruction count over the whole run
    const uint4 *src = reinterpret_cast<const uint4 *>(m.codes) + (long)b.rb * G;
    for (int c0 = w * 64; c0 < n; c0 += nw * 64, ++k) {
        if (k < first) continue;
        if (k >= last) return;
        const int c = min(c0 + lane, n - 1);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(src + c),
            (__attribute__((address_space(3))) void *)(buf + c0), 16, 0, 0);
    }
    if (b.lds_steps) {
        const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(m.steps + (long)b.rb * G);
        uint32_t *sdst = reinterpret_cast<uint32_t *>(buf + b.steps_chunk);
        const int nd = n / 2;
        for (int d0 = w * 64; d0 < nd; d0 += nw * 64, ++k) {
            if (k < first) continue;
            if (k >= last) return;
            const int d = min(d0 + lane, nd - 1);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(ssrc + d),
                (__attribute__((address_space(3))) void *)(sdst + d0), 4, 0, 0);
        }
    }
}

// Compute waves: the rows of the block, L lanes per row, NG groups per lane;
// codes and steps from the LDS buffer for staged rows, else from memory.
template <int L, int NG>
__device__ __forceinline__ void chain_rows(const ChainMat &m, const RowBlock &b, const uint4 *buf,
                                           const uint16_t *raw) {
    constexpr int SLOTS = kWave / L;
    const int G = m.K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = lane % L, slot = lane / L;
    const uint4 *codes = reinterpret_cast<const uint4 *>(m.codes);
    const uint16_t *lsteps = reinterpret_cast<const uint16_t *>(buf + b.steps_chunk);
    // this wave's activations, already in pair order in LDS -> registers
    h2 xr[NG][16];
    const uint4 *r16 = reinterpret_cast<const uint4 *>(raw);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = l + i * L;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint4 v = g < G ? r16[g * 4 + w] : make_uint4(0, 0, 0, 0);
            xr[i][w * 4 + 0] = as_h2(v.x);
            xr[i][w * 4 + 1] = as_h2(v.y);
            xr[i][w * 4 + 2] = as_h2(v.z);
            xr[i][w * 4 + 3] = as_h2(v.w);
        }
    }
    // Rows [rb, rb + nlds) from the buffer, the rest from memory (two loops,
    // so that every load has a known address space).
    auto finish = [&](int row, const uint4 (&q)[NG], const uint32_t (&sv)[NG]) __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            acc = (g < G) ? __builtin_fmaf(group_dot(q[i], xr[i]), bf16_to_f32(sv[i]), acc) : acc;
        }
        acc = lane_group_sum<L>(acc);
        if (l == L - 1 && row < b.re) store_y(m.y, m.N, row, __builtin_ldexpf(acc, kGroupDotExp));
    };
    const int staged_end = b.rb + b.nlds;
    for (int r0 = b.rb; r0 < staged_end; r0 += kComputeWaves * SLOTS) {
        const int row = r0 + wave * SLOTS + slot;
        const int rl = min(row, staged_end - 1) - b.rb;
        uint4 q[NG];
        uint32_t sv[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) q[i] = buf[rl * G + min(l + i * L, G - 1)];
        if (b.lds_steps) {
#pragma unroll
            for (int i = 0; i < NG; ++i) sv[i] = lsteps[rl * G + min(l + i * L, G - 1)];
        } else {
#pragma unroll
            for (int i = 0; i < NG; ++i) sv[i] = load_global_u16(m.steps, (long)(b.rb + rl) * G + min(l + i * L, G - 1));
        }
        finish(row < staged_end ? row : b.re, q, sv);
    }
    for (int r0 = staged_end; r0 < b.re; r0 += kComputeWaves * SLOTS) {
        const int row = r0 + wave * SLOTS + slot;
        const int rc = min(row, b.re - 1);
        uint4 q[NG];
        uint32_t sv[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = min(l + i * L, G - 1);
            q[i] = load_global_u4(codes, (long)rc * G + g);
            sv[i] = load_global_u16(m.steps, (long)rc * G + g);
        }
        finish(row, q, sv);
    }
}

__device__ __forceinline__ void chain_rows_any(const ChainMat &m, const RowBlock &b, const uint4 *buf,
                                               const uint16_t *raw) {
    const int G = m.K >> 5;
    const int L = G <= 64 ? 16 : (G <= 128 ? 32 : 64);
    const int NG = (G + L - 1) / L;
    switch (__builtin_amdgcn_readfirstlane(L * 8 + NG)) {
        case 16 * 8 + 1: chain_rows<16, 1>(m, b, buf, raw); break;
        case 16 * 8 + 2: chain_rows<16, 2>(m, b, buf, raw); break;
        case 16 * 8 + 3: chain_rows<16, 3>(m, b, buf, raw); break;
        case 16 * 8 + 4: chain_rows<16, 4>(m, b, buf, raw); break;
        case 32 * 8 + 3: chain_rows<32, 3>(m, b, buf, raw); break;
        case 32 * 8 + 4: chain_rows<32, 4>(m, b, buf, raw); break;
        case 64 * 8 + 3: chain_rows<64, 3>(m, b, buf, raw); break;
        default: chain_rows<64, 4>(m, b, buf, raw); break;
    }
}

// Wave 0: wait until every workgroup's flag has reached generation `gen`
// (agent-coherent loads, all issued at once, one or more per lane), with a
// bounded number of polls; a timeout sets the error word.  Returns 1 if the
// chain must stop.
__device__ __forceinline__ int chain_poll(unsigned *sync, unsigned gen, unsigned spin_limit, int nwg) {
    const int lane = threadIdx.x;
    const __amdgpu_buffer_rsrc_t fr = buffer_rsrc(sync + kSyncFlags, nwg * kFlagStride * 4);
    unsigned it = 0;
    int stop = 0;
    for (;;) {
        // lane l checks the flags of workgroups l, l+64, ... (one load each)
        int behind = 0;
        for (int f = lane; f < nwg; f += 64) {
            const unsigned a = __builtin_amdgcn_raw_buffer_load_b32(fr, f * kFlagStride * 4, 0, 16);
            // generations only grow; compare with wrap-around arithmetic
            behind |= (int)(a - gen) < 0;
        }
        if (!wave_or_i32(behind)) break;
        if (++it > spin_limit) {
            if (lane == 0)
                __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            stop = 1;
            break;
        }
    }
    return stop || load_agent_u(sync + kSyncError) != 0;
}

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainMat *__restrict__ desc,
                                                              int n, const uint16_t *__restrict__ x0,
                                                              unsigned *sync, unsigned spin_limit) {
    extern __shared__ uint4 smem[];
    uint16_t *raw = reinterpret_cast<uint16_t *>(smem);   // kChainMaxK halves
    uint4 *bufs = smem + (kChainMaxK * 2) / 16;            // two weight buffers
    __shared__ double dred[8];
    __shared__ int stop_s;
    const int nwg = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6;
    const bool copier = wave >= kComputeWaves;

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
        if (copier) chain_copy(desc[0], chain_block(desc[0], nwg), bufs, 0, 1 << 30);
        for (int i = 0; i < n; ++i) {
            const ChainMat m = desc[i];
            const int K = m.K;
            // 1. input into LDS (raw fp16)
            uint4 *r16 = reinterpret_cast<uint4 *>(raw);
            // (both paths leave each 8-value block in the pair order
            // (x0,x4)(x1,x5)(x2,x6)(x3,x7) that the unpack of a packed word uses)
            if (i == 0) {
                const uint4 *x16 = reinterpret_cast<const uint4 *>(x0);
                for (int c = tid; c < (K >> 3); c += kChainThreads) {
                    const uint4 v = x16[c];
                    r16[c] = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                        __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                        __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                        __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
                }
            } else {
                // previous output: the chunks of the canonical 256-thread
                // order, all requested at once with agent-coherent loads
                const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(desc[i - 1].y, K * 4);
                constexpr int J = kChainMaxK / 4 / 256;
                float4 v[J];
                const bool rn = tid < 256;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int c = tid + 256 * j;
                    v[j] = (rn && c < (K >> 2)) ? load_coherent_f4(pr, c * 16)
                                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
                const double inv = renorm_scale(sum_squares_256_regs(K, v, dred, rn), K);
                if (rn) {
#pragma unroll
                    for (int j = 0; j < J; ++j) {
                        const int c = tid + 256 * j;
                        if (c < (K >> 2)) {
                            // chunk c holds values 4(c&1)..+3 of block c>>1:
                            // value e of a block sits at position 2(e&3) + (e>>2)
                            uint16_t *blk = raw + (c >> 1) * 8 + (c & 1);
                            blk[0] = renorm_value(v[j].x, inv, 0);
                            blk[2] = renorm_value(v[j].y, inv, 0);
                            blk[4] = renorm_value(v[j].z, inv, 0);
                            blk[6] = renorm_value(v[j].w, inv, 0);
                        }
                    }
                }
            }
            // input staged, and this step's weights landed (the copy waves
            // have no loads outstanding past this point)
            __syncthreads();
            // 2. copy waves fetch the next step's block; compute waves run this one
            // (the copy wave issues the first kCopyEarly instructions of the next
            // block now and the rest after the pre-flag barrier below, so that
            // it reaches that barrier without delay)
            uint4 *next_buf = bufs + ((i + 1) & 1) * (kWeightBuf / 16);
            if (copier) {
                if (i + 1 < n) chain_copy(desc[i + 1], chain_block(desc[i + 1], nwg), next_buf, 0, kCopyEarly);
            } else {
                chain_rows_any(m, chain_block(m, nwg), bufs + (i & 1) * (kWeightBuf / 16), raw);
            }
            if (i + 1 == n) break;
            // 3. grid barrier before the next step reads this output
            if (!copier) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // outputs stored
            lds_barrier();
            if (tid == 0)
                __hip_atomic_store(sync + kSyncFlags + blockIdx.x * kFlagStride, epoch + (unsigned)(i + 1),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (copier) {
                chain_copy(desc[i + 1], chain_block(desc[i + 1], nwg), next_buf, kCopyEarly, 1 << 30);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // next block landed
            }
            if (wave == 0) {
                const int stop = chain_poll(sync, epoch + (unsigned)(i + 1), spin_limit, nwg);
                if (tid == 0) stop_s = stop;
            }
            lds_barrier();
            if (stop_s) break;
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

size_t chain_lds_bytes() { return (size_t)kChainMaxK * 2 + 2 * (size_t)kWeightBuf; }

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
