// A decode-step chain of W4A16 products as one persistent launch (gfx950).
//
// The dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch" (section "Step 4 -
// Replay Each Decode Step as One CUDA Graph") notes that a decode step is
// hundreds of small kernels and that launching them one by one costs more than
// running them; its tip "Merge the Small Projections" merges q/k/v and gate/up
// into one matrix each.  Here the whole chain of merged matrices runs inside
// one kernel: every workgroup stays resident and takes its share of the rows
// of matrix i; matrix i+1 needs all of the renormalised output of matrix i.
//
// Exchange.  There is no separate grid barrier: every output that the next
// matrix needs is published as one 4-byte cell holding the bitwise complement
// of the value (NaNs stored as one quiet NaN, so no written cell is zero),
// and a cell that is still zero has not been written.  A consumer reads the
// cells it needs until none is zero (bounded; a timeout sets the error word):
// one round trip through memory both waits for the producers and brings
// their values.  Each step has its own cell region, so a fast workgroup never
// overwrites values that a slow one has yet to read.  Regions go back to zero
// within the call: once a workgroup has read all of step s-1's cells, every
// workgroup has finished reading step s-2's (each wrote its step s-1 cells
// only after that), so it clears its own cells of step s-2; the last
// workgroup out clears the last region that was read.
//
// Per step i (one workgroup of eight waves per CU; workgroup b owns the
// contiguous row block [b*ceil(N/nwg), ...) of every matrix):
//   1. input: x0 for the first matrix; else waves 0..3 read the leading K
//      cells of step i-1 (agent-coherent loads), the workgroup takes their sum
//      of squares in fp64 in the fixed order of w4_rms_renorm and writes
//      u / rms rounded to fp16 into LDS (bit for bit what w4_rms_renorm gives);
//      meanwhile waves 6..7 wait for their copy of this step's weights;
//   2. waves 6..7 request the next step's weight block into the other LDS
//      buffer (direct-to-LDS loads that only they wait for, at the start of
//      the next step: neither the exchange loads of waves 0..3 nor any row
//      computation queue behind weight traffic);
//   3. waves 0..3 compute the block's rows from LDS and store y, and the
//      cells of the rows the next step needs.  Wave w runs on SIMD w mod 4,
//      so these are one wave per SIMD; a second computing wave on a SIMD
//      (waves 4 and 5 did so) measured slower over the decode sweep: its
//      rows finish last and hold up the next exchange.  Waves 4..5 only
//      join the workgroup barriers.
// The descriptors are copied into LDS once (the first kDescCache of them).
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
constexpr int kChainWaves = kChainThreads / 64;
constexpr int kPollThreads = 256;   // waves 0..3 read the exchange cells and renormalise
constexpr int kCopyWave0 = 6;       // waves 6..7 copy weight blocks and compute nothing
constexpr int kComputeWaves = 4;    // waves 0..3 compute rows (one per SIMD); waves 4..5 only join barriers
constexpr int kDescCache = 128;     // descriptors kept in LDS
constexpr int kChainMaxK = 8192;

// The staged input is kept as four planes: plane w holds uint4 w (pair-order
// fp16 values 8w..8w+7) of every group, so that lanes reading the same plane
// for consecutive groups touch consecutive LDS banks.  The plane stride is
// the group count rounded up to 8 modulo 16 uint4, which puts planes 1 and 3
// on the other half of the banks from planes 0 and 2 when they are written.
__device__ __forceinline__ int chain_plane(int G) { return ((G + 7) >> 4) * 16 + 8; }
constexpr int kXinBytes = 4 * (((kChainMaxK / 32 + 7) >> 4) * 16 + 8) * 16;
constexpr int kWeightBuf = 64 * 1024;  // bytes of each of the two LDS weight buffers
// sync buffer: bytes [0, 256) a header (word 0 exit counter, word 2 error);
// from byte 256, one region of kChainMaxK 4-byte cells per matrix.
constexpr int kSyncExit = 0, kSyncError = 2;
constexpr long kExchOffset = 256, kExchBytes = (long)kChainMaxK * 4;
static_assert(W4_CHAIN_SYNC_BYTES(1) == kExchOffset + kExchBytes, "sync layout");

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
__device__ __forceinline__ unsigned load_agent_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This workgroup's plan for one step.  Its rows are range A, [ra, ra + na),
// then range B, [rb2, rb2 + nb).  When the next step reads only the leading
// k_next < N outputs (the gate half of gate/up), A is this workgroup's share of
// those rows and B its share of the rest, so every workgroup publishes the
// exchanged rows first and computes the others while they travel; otherwise A
// is a contiguous block and B is empty.  The first nlds rows of A ++ B are
// staged in an LDS weight buffer -- A's codes at 0, B's at offb, then the
// steps (A's, then B's at sbo words) -- and the rest are read from memory.
// Worked out once per descriptor, when the descriptor enters the LDS table.
struct RowBlock {
    int ra, na, rb2, nb;
    int nlds;
    int sel;     // row kernel: lanes per row * 8 + groups per lane
    int k_next;  // K of the next step (the cells it reads), 0 after the last
    int pad;
};
static_assert(sizeof(RowBlock) == 32, "plan entry");

__device__ __forceinline__ int round64(int v) { return (v + 63) & ~63; }

// LDS layout of a plan's staged rows (uint4 chunks for codes, 4-byte words
// for steps; every run rounded to 64, so that the surplus lanes of a copy
// instruction land in padding)
struct StagedLayout {
    int na_st, nb_st;  // staged rows of A and B
    int offb;          // chunk offset of B's codes
    int sc;            // chunk offset of the steps
    int sbo;           // word offset of B's steps inside the steps
};
__device__ __forceinline__ StagedLayout staged_layout(const RowBlock &b, int G) {
    StagedLayout s;
    s.na_st = min(b.na, b.nlds);
    s.nb_st = b.nlds - s.na_st;
    s.offb = round64(s.na_st * G);
    s.sc = s.offb + round64(s.nb_st * G);
    s.sbo = round64(s.na_st * G / 2);
    return s;
}

__device__ __forceinline__ RowBlock chain_plan(const ChainMat &m, int k_next, int nwg) {
    const int G = m.K >> 5;
    const int b = blockIdx.x;
    RowBlock p;
    const int kn = (k_next > 0 && k_next < m.N) ? k_next : 0;
    if (kn) {
        const int ra_w = (kn + nwg - 1) / nwg, rb_w = (m.N - kn + nwg - 1) / nwg;
        p.ra = min(kn, b * ra_w);
        p.na = min(kn, p.ra + ra_w) - p.ra;
        p.rb2 = kn + min(m.N - kn, b * rb_w);
        p.nb = min(m.N, p.rb2 + rb_w) - p.rb2;
    } else {
        const int rpw = (m.N + nwg - 1) / nwg;
        p.ra = min(m.N, b * rpw);
        p.na = min(m.N, p.ra + rpw) - p.ra;
        p.rb2 = m.N;
        p.nb = 0;
    }
    // steps travel as 4-byte words: every row's steps must start on one
    const bool lds_steps = (G % 2) == 0 && (reinterpret_cast<uintptr_t>(m.steps) & 3) == 0;
    auto bytes = [&](int rows) {
        const int a = min(p.na, rows), c = rows - a;
        return (round64(a * G) + round64(c * G)) * 16 + (round64(a * G / 2) + round64(c * G / 2)) * 4;
    };
    // (rows are staged only together with their steps)
    int n = lds_steps ? min(p.na + p.nb, kWeightBuf / (G * 18)) : 0;
    while (n > 0 && bytes(n) > kWeightBuf) --n;
    p.nlds = n;
    // lanes per row from the row length alone: 16 lanes up to 64 groups, 32
    // up to 128, else 64.  (Choosing by the least work per lane -- 64 lanes
    // for a block of six 64-group rows, say -- measured slower over the whole
    // decode sweep: passes are latency-bound, not arithmetic-bound.)
    const int L = G <= 64 ? 16 : (G <= 128 ? 32 : 64);
    p.sel = L * 8 + (G + L - 1) / L;
    p.k_next = k_next;
    p.pad = 0;
    return p;
}

// Copy waves: request the staged rows into `buf` with direct-to-LDS loads
// (every lane moves 16 bytes of codes or 4 bytes of steps; the last
// instruction of each run lands its surplus lanes in the run's padding).
// Written with the asm form of the load, so that the compiler adds no waits
// for it; the copy waves wait for it themselves (vmcnt 0) before the workgroup
// barrier that precedes the block's use.
__device__ __forceinline__ void chain_copy(const ChainMat &m, const RowBlock &b, uint4 *buf) {
    const int w = (threadIdx.x >> 6) - kCopyWave0, lane = threadIdx.x & 63;
    constexpr int nw = kChainWaves - kCopyWave0;
    const int G = m.K >> 5;
    if (b.nlds == 0) return;
    const StagedLayout sl = staged_layout(b, G);
    auto codes_run = [&](int row0, int rows, uint4 *dst) __attribute__((always_inline)) {
        const int n = rows * G;
        const uint4 *src = reinterpret_cast<const uint4 *>(m.codes) + (long)row0 * G;
        for (int c0 = w * 64; c0 < n; c0 += nw * 64) lds_dma16(src + min(c0 + lane, n - 1), dst + c0);
    };
    auto steps_run = [&](int row0, int rows, uint32_t *dst) __attribute__((always_inline)) {
        const int nd = rows * G / 2;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(m.steps + (long)row0 * G);
        for (int d0 = w * 64; d0 < nd; d0 += nw * 64) lds_dma4(src + min(d0 + lane, nd - 1), dst + d0);
    };
    uint32_t *sdst = reinterpret_cast<uint32_t *>(buf + sl.sc);
    codes_run(b.ra, sl.na_st, buf);
    steps_run(b.ra, sl.na_st, sdst);
    if (sl.nb_st > 0) {
        codes_run(b.rb2, sl.nb_st, buf + sl.offb);
        steps_run(b.rb2, sl.nb_st, sdst + sl.sbo);
    }
}

// One exchange cell: the complement of the value's bits, published with a
// single 4-byte store that agent-scope loads on any XCD see.
__device__ __forceinline__ void store_cell(uint32_t *cells, int row, float v) {
    const uint32_t bits = v == v ? __float_as_uint(v) : 0x7FC00000u;
    __hip_atomic_store(cells + row, ~bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void clear_cell(uint32_t *cells, int row) {
    __hip_atomic_store(cells + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where the rows of one step go: y, and the cells of rows < k_next (the
// leading entries the next step reads; k_next 0 for the last step).
struct RowSink {
    uint32_t *cells;
};

// Computing waves: the rows of the block, L lanes per row, NG groups per lane;
// rows staged in the LDS buffer first (a loop with no global loads), then any
// rows read from memory.
template <int L, int NG>
__device__ __forceinline__ void chain_rows(const ChainMat &m, const RowBlock &b, const uint4 *buf,
                                           const uint16_t *xin, const RowSink &sink) {
    constexpr int SLOTS = kWave / L;
    const int G = m.K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = lane % L, slot = lane / L;
    const StagedLayout sl = staged_layout(b, G);
    const uint16_t *lsteps = reinterpret_cast<const uint16_t *>(buf + sl.sc);
    const int nrows = b.na + b.nb;
    // local row lr of A ++ B -> its global row
    auto global_row = [&](int lr) __attribute__((always_inline)) { return lr < b.na ? b.ra + lr : b.rb2 + (lr - b.na); };
    // the activations, already in pair order in LDS -> registers
    h2 xr[NG][16];
    const uint4 *r16 = reinterpret_cast<const uint4 *>(xin);
    const int Gs = chain_plane(G);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = l + i * L;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint4 v = g < G ? r16[w * Gs + g] : make_uint4(0, 0, 0, 0);
            xr[i][w * 4 + 0] = as_h2(v.x);
            xr[i][w * 4 + 1] = as_h2(v.y);
            xr[i][w * 4 + 2] = as_h2(v.z);
            xr[i][w * 4 + 3] = as_h2(v.w);
        }
    }
    float2 xo[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) xo[i] = group_offset(xr[i]);
    auto finish = [&](int row, const uint4 (&q)[NG], const uint32_t (&sv)[NG]) __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            acc = (g < G) ? __builtin_fmaf(group_dot_off(q[i], xr[i], xo[i]), bf16_to_f32(sv[i]), acc) : acc;
        }
        acc = lane_group_sum<L>(acc);
        if (l == L - 1 && row >= 0) {
            const float v = __builtin_ldexpf(acc, kGroupDotExp);
            // (a global store: through the generic pointer it would be a flat
            // store, which every later LDS read would have to wait for)
            ((__attribute__((address_space(1))) float *)m.y)[row] = v;
            if (row < b.k_next) store_cell(sink.cells, row, v);
        }
    };
    // A pass gives each computing wave SLOTS rows.  Waves whose rows are all
    // past the end still run the pass on clamped rows and store nothing:
    // skipping it (and giving the idle SIMD time to the wave beside it)
    // measured slower over the decode sweep.
    for (int l0 = 0; l0 < b.nlds; l0 += kComputeWaves * SLOTS) {
        const int lr = l0 + wave * SLOTS + slot;
        const int lc = min(lr, b.nlds - 1);
        // staged position: A's rows from 0, B's from offb (codes) / 2 sbo (steps)
        const int cbase = lc < sl.na_st ? lc * G : sl.offb + (lc - sl.na_st) * G;
        const int sbase = lc < sl.na_st ? lc * G : 2 * sl.sbo + (lc - sl.na_st) * G;
        uint4 q[NG];
        uint32_t sv[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = min(l + i * L, G - 1);
            q[i] = buf[cbase + g];
            sv[i] = lsteps[sbase + g];
        }
        finish(lr < b.nlds ? global_row(lr) : -1, q, sv);
    }
    if (b.nlds < nrows) {
        const uint4 *codes = reinterpret_cast<const uint4 *>(m.codes);
        for (int l0 = b.nlds; l0 < nrows; l0 += kComputeWaves * SLOTS) {
            const int lr = l0 + wave * SLOTS + slot;
            const int rc = global_row(min(lr, nrows - 1));
            uint4 q[NG];
            uint32_t sv[NG];
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = min(l + i * L, G - 1);
                q[i] = load_global_u4(codes, (long)rc * G + g);
                sv[i] = load_global_u16(m.steps, (long)rc * G + g);
            }
            finish(lr < nrows ? global_row(lr) : -1, q, sv);
        }
    }
}

__device__ __forceinline__ void chain_rows_any(const ChainMat &m, const RowBlock &b, const uint4 *buf,
                                               const uint16_t *xin, const RowSink &sink) {
    if (b.na + b.nb == 0) return;
    switch (__builtin_amdgcn_readfirstlane(b.sel)) {
        case 16 * 8 + 1: chain_rows<16, 1>(m, b, buf, xin, sink); break;
        case 16 * 8 + 2: chain_rows<16, 2>(m, b, buf, xin, sink); break;
        case 16 * 8 + 3: chain_rows<16, 3>(m, b, buf, xin, sink); break;
        case 16 * 8 + 4: chain_rows<16, 4>(m, b, buf, xin, sink); break;
        case 32 * 8 + 3: chain_rows<32, 3>(m, b, buf, xin, sink); break;
        case 32 * 8 + 4: chain_rows<32, 4>(m, b, buf, xin, sink); break;
        case 64 * 8 + 3: chain_rows<64, 3>(m, b, buf, xin, sink); break;
        default: chain_rows<64, 4>(m, b, buf, xin, sink); break;
    }
}

// Waves 0..3: read the K cells of one region until none is zero.  Thread t
// owns the 4-value chunks c = t, t+256, ... (the order of the sum of squares)
// and re-reads only chunks not yet complete.  A bounded number of rounds; a
// timeout (or an error raised elsewhere) returns 1.
constexpr int kPollJ = kChainMaxK / 4 / kPollThreads;

__device__ __forceinline__ int chain_read_cells(const uint32_t *cells, int K, unsigned spin_limit,
                                                unsigned *sync, float4 (&v)[kPollJ]) {
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(cells, K * 4);
    unsigned pend = 0;
#pragma unroll
    for (int j = 0; j < kPollJ; ++j) {
        v[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (tid + kPollThreads * j < (K >> 2)) pend |= 1u << j;
    }
    for (unsigned it = 0;; ++it) {
        uint4 a[kPollJ];
#pragma unroll
        for (int j = 0; j < kPollJ; ++j)
            if (pend & (1u << j))
                a[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     r, (tid + kPollThreads * j) * 16, 0, 16));
#pragma unroll
        for (int j = 0; j < kPollJ; ++j) {
            if ((pend & (1u << j)) && a[j].x != 0u && a[j].y != 0u && a[j].z != 0u && a[j].w != 0u) {
                v[j] = make_float4(__uint_as_float(~a[j].x), __uint_as_float(~a[j].y),
                                   __uint_as_float(~a[j].z), __uint_as_float(~a[j].w));
                pend &= ~(1u << j);
            }
        }
        if (!wave_or_i32(pend != 0)) return 0;
        if (it >= spin_limit || ((it & 63) == 63 && load_agent_u(sync + kSyncError) != 0)) {
            if ((tid & 63) == 0)
                __hip_atomic_store(sync + kSyncError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return 1;
        }
    }
}

// Sum of squares over the poll waves' values, in the fixed order of
// sum_squares_256 (thread t: chunks t, t+256, ... ascending; wave_sum_f64;
// wave sums added in wave order) -- bit for bit the w4_rms_renorm value --
// with a single workgroup barrier: the wave sums go to one of two LDS slots,
// alternating from step to step, so a slot is rewritten only two barriers
// after it was read.
__device__ __forceinline__ double chain_sum_squares(int K, const float4 (&v)[kPollJ], double *red,
                                                    bool active, int parity) {
    const int tid = threadIdx.x;
    double ss = 0.0;
    if (active) {
        // chunks past the end hold zeros, and adding +0 leaves the sum's bits
        // unchanged: the bound is the wave-uniform chunk count, no lane test
        const int jn = ((K >> 2) + kPollThreads - 1) / kPollThreads;
#pragma unroll
        for (int j = 0; j < kPollJ; ++j) {
            if (j < jn) {
                ss += (double)v[j].x * (double)v[j].x;
                ss += (double)v[j].y * (double)v[j].y;
                ss += (double)v[j].z * (double)v[j].z;
                ss += (double)v[j].w * (double)v[j].w;
            }
        }
    }
    ss = wave_sum_f64(ss);
    double *r = red + parity * 4;
    if ((tid & 63) == 0 && tid < kPollThreads) r[tid >> 6] = ss;
    lds_barrier();
    return ((r[0] + r[1]) + r[2]) + r[3];
}

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainMat *__restrict__ desc,
                                                              int n, const uint16_t *__restrict__ x0,
                                                              unsigned *sync, unsigned spin_limit) {
    extern __shared__ uint4 smem[];
    uint16_t *xin = reinterpret_cast<uint16_t *>(smem);   // the staged input, four planes
    uint4 *bufs = smem + kXinBytes / 16;                   // two weight buffers
    ChainMat *dtab = reinterpret_cast<ChainMat *>(bufs + 2 * (kWeightBuf / 16));
    RowBlock *ptab = reinterpret_cast<RowBlock *>(dtab + kDescCache);  // this workgroup's plans
    __shared__ double dred[8];
    __shared__ int stop_s, bad_s;
    const int nwg = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6;
    const bool copier = wave >= kCopyWave0;
    uint32_t *regions = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(sync) + kExchOffset);

    // Descriptors: the first kDescCache into an LDS table (entry i in slot
    // i % kDescCache); later ones are brought in kDescCache/2 steps ahead of
    // use (see the end of the step loop).  Every workgroup checks them all
    // (same answer everywhere).
    typedef const __attribute__((address_space(1))) uint32_t gword;
    constexpr int kWords = sizeof(ChainMat) / 4;
    gword *dsrc = (gword *)desc;
    uint32_t *dwords = reinterpret_cast<uint32_t *>(dtab);
    for (int k = tid; k < min(n, kDescCache) * kWords; k += kChainThreads) dwords[k] = dsrc[k];
    if (tid == 0) {
        stop_s = 0;
        bad_s = n < 1;
    }
    auto load_desc = [&](int i) __attribute__((always_inline)) {
        uint32_t w[kWords];
#pragma unroll
        for (int k = 0; k < kWords; ++k) w[k] = dsrc[(long)i * kWords + k];
        ChainMat m;
        __builtin_memcpy(&m, w, sizeof(m));
        return m;
    };
    auto load_plan = [&](int i) __attribute__((always_inline)) {
        return chain_plan(load_desc(i), i + 1 < n ? (int)dsrc[(long)(i + 1) * kWords + 7] : 0, nwg);
    };
    static_assert(offsetof(ChainMat, K) == 28, "K is word 7 of a descriptor");
    for (int i = tid; i < n; i += kChainThreads) {
        const ChainMat m = load_desc(i);
        const int prevN = i > 0 ? load_desc(i - 1).N : 0;
        if (m.N < 1 || m.K < 32 || (m.K & 31) || m.K > kChainMaxK || !m.codes || !m.steps || !m.y ||
            (reinterpret_cast<uintptr_t>(m.codes) & 15) || (reinterpret_cast<uintptr_t>(m.y) & 15) ||
            (i > 0 && m.K > prevN))
            bad_s = 1;
    }
    __syncthreads();
    auto get = [&](int i) __attribute__((always_inline)) { return dtab[i % kDescCache]; };
    auto plan = [&](int i) __attribute__((always_inline)) { return ptab[i % kDescCache]; };
    if (!bad_s) {
        // (plans only of checked descriptors)
        for (int i = tid; i < min(n, kDescCache); i += kChainThreads) ptab[i] = load_plan(i);
        lds_barrier();
        if (copier) chain_copy(get(0), plan(0), bufs);
        for (int i = 0; i < n; ++i) {
            const ChainMat m = get(i);
            const int K = m.K;
            // 1. input into LDS, in the pair order (x0,x4)(x1,x5)(x2,x6)(x3,x7)
            // of each 8-value block that the unpack of a packed word uses
            if (i == 0) {
                const uint4 *x16 = reinterpret_cast<const uint4 *>(x0);
                uint4 *r16 = reinterpret_cast<uint4 *>(xin);
                const int Gs = chain_plane(K >> 5);
                for (int c = tid; c < (K >> 3); c += kChainThreads) {
                    const uint4 v = x16[c];
                    r16[(c & 3) * Gs + (c >> 2)] = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                        __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                        __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                        __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
                }
                if (copier) wait_vmcnt_mem<0>();  // block 0 landed
            } else {
                float4 v[kPollJ];
                const bool rn = tid < kPollThreads;
                if (rn) {
                    const int stop = chain_read_cells(regions + (long)(i - 1) * kChainMaxK, K,
                                                      spin_limit, sync, v);
                    if (stop) stop_s = 1;
                } else {
#pragma unroll
                    for (int j = 0; j < kPollJ; ++j) v[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (copier) wait_vmcnt_mem<0>();  // this step's block landed
                }
                // (its barriers also publish stop_s)
                const double inv = renorm_scale(chain_sum_squares(K, v, dred, rn, i & 1), K);
                if (stop_s) break;
                if (rn) {
                    const int Gs = chain_plane(K >> 5);
                    const int jn = ((K >> 2) + kPollThreads - 1) / kPollThreads;
                    uint2 *x8 = reinterpret_cast<uint2 *>(xin);
#pragma unroll
                    for (int j = 0; j < kPollJ; ++j) {
                        if (j < jn) {
                            // chunk c holds values 4(c&1)..+3 of block u = c>>1
                            // (uint4 u & 3 of group u >> 2), whose pair order is
                            // (x0,x4)(x1,x5)(x2,x6)(x3,x7): the even lane of a
                            // pair writes the first two words, the odd lane the
                            // last two, each taking two halves from the other
                            const int c = tid + kPollThreads * j;
                            const uint32_t h0 = renorm_value(v[j].x, inv, 0), h1 = renorm_value(v[j].y, inv, 0);
                            const uint32_t h2 = renorm_value(v[j].z, inv, 0), h3 = renorm_value(v[j].w, inv, 0);
                            const bool odd = c & 1;
                            const uint32_t give = odd ? (h0 | (h1 << 16)) : (h2 | (h3 << 16));
                            const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
                            const uint2 w = odd ? make_uint2((got & 0xFFFFu) | (h2 << 16), (got >> 16) | (h3 << 16))
                                                : make_uint2(h0 | (got << 16), h1 | (got & 0xFFFF0000u));
                            const int u = c >> 1;
                            if (c < (K >> 2)) x8[((u & 3) * Gs + (u >> 2)) * 2 + (c & 1)] = w;
                        }
                    }
                }
            }
            // input staged, and this step's weights landed
            lds_barrier();
            if (copier) {
                // 2. the copy waves request the next step's block
                if (i + 1 < n)
                    chain_copy(get(i + 1), plan(i + 1), bufs + ((i + 1) & 1) * (kWeightBuf / 16));
            } else if (wave < kComputeWaves) {
                // 3. this step's rows
                RowSink sink;
                sink.cells = regions + (long)i * kChainMaxK;
                chain_rows_any(m, plan(i), bufs + (i & 1) * (kWeightBuf / 16), xin, sink);
                // step i-1's cells are all in: every workgroup is done with
                // step i-2's, so this one clears its own
                if (wave == kComputeWaves - 1 && i >= 2) {
                    const RowBlock q = plan(i - 2);
                    uint32_t *cells = regions + (long)(i - 2) * kChainMaxK;
                    for (int r = q.ra + (tid & 63); r < min(q.ra + q.na, q.k_next); r += 64) clear_cell(cells, r);
                }
                // refill: descriptor i + kDescCache/2 (and its plan) into the
                // slot of i - kDescCache/2
                const int j = i + kDescCache / 2;
                if (wave == kComputeWaves - 1 && j >= kDescCache && j < n) {
                    if ((tid & 63) < kWords)
                        dwords[(j % kDescCache) * kWords + (tid & 63)] = dsrc[(long)j * kWords + (tid & 63)];
                    if ((tid & 63) == kWords) ptab[j % kDescCache] = load_plan(j);
                }
            }
        }
    } else if (blockIdx.x == 0 && tid == 0) {
        __hip_atomic_store(sync + kSyncError, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Exit: the last workgroup out (every other one has finished, so all
    // reading is over) clears the cells of the last step that were read and
    // returns the exit counter to zero.
    __shared__ int last_s;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(sync + kSyncExit, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_s = prev == (unsigned)nwg - 1;
        if (last_s) __hip_atomic_store(sync + kSyncExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_barrier();
    if (last_s && !bad_s && n >= 2) {
        const int kl = (int)dsrc[(long)(n - 1) * kWords + 7];
        uint32_t *cells = regions + (long)(n - 2) * kChainMaxK;
        for (int r = tid; r < kl; r += kChainThreads) clear_cell(cells, r);
    }
}

static_assert(kXinBytes + 2 * kWeightBuf + kDescCache * 64 + 256 <= 160 * 1024, "LDS of one workgroup");

size_t chain_lds_bytes() {
    return (size_t)kXinBytes + 2 * (size_t)kWeightBuf + kDescCache * (sizeof(ChainMat) + sizeof(RowBlock));
}

hipError_t launch_chain(const void *desc, int n, const uint16_t *x0, void *sync, unsigned spin_limit,
                        hipStream_t stream) {
    // One workgroup per CU, all resident together on an otherwise idle device
    // (the occupancy check makes sure one fits per CU).  A plain launch: if
    // some workgroups could not start while others wait, the bounded waits for
    // their cells end with the timeout error instead of a hang.
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
    hipLaunchKernelGGL(chain_kernel, dim3(cus), dim3(kChainThreads), lds, stream,
                       static_cast<const ChainMat *>(desc), n, x0, static_cast<unsigned *>(sync),
                       spin_limit);
    return hipGetLastError();
}

}  // namespace w4
