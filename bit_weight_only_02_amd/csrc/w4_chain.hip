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
// Renormalisation as an output scale.  Matrix i > 0 multiplies the leading K
// entries u of the previous output divided by their RMS r; since
// W (u / r) = (W u) / r, the products run on u itself and each finished
// output is multiplied by 1/r, so no step waits for r before its dot
// products.  u goes to fp16 one group of 32 at a time, each group scaled by
// its own power of two (its largest magnitude lands in [2^14, 2^15)), and the
// group's partial sums are scaled back by the inverse power of two with the
// group's step.  r comes from the sum of squares of u: per chunk of four in
// fp32 on the group-scaled values (which are below 2^15, so no overflow), each
// chunk's sum scaled back into fp64, then added in a fixed order (a thread's
// chunks ascending, a butterfly over the wave, the waves in order).
//
// Per step i (one workgroup of ten waves per CU; workgroup b owns the
// contiguous row block [b*ceil(N/nwg), ...) of every matrix):
//   1. input: x0 for the first matrix; else the eight computing waves read
//      the leading K cells of step i-1 (agent-coherent loads), write each
//      group as fp16 into LDS with its scale and its offset sums, and one sum
//      of squares per wave; meanwhile the two copy waves wait for their copy
//      of this step's weights;
//   2. the copy waves request the next step's weight block into the other
//      LDS buffer (direct-to-LDS loads that only they wait for, at the start
//      of the next step: neither the exchange loads nor any row computation
//      queue behind weight traffic), then clear this workgroup's cells of
//      step i-2 and bring in a later descriptor and its plan;
//   3. the eight computing waves (two per SIMD: wave w runs on SIMD w mod 4,
//      so one wave's waits are filled by the other's work) compute the
//      block's rows from LDS, scale them by 1/r, and store y and the cells of
//      the rows the next step needs.
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

// Waves 0..7 read the exchange cells, stage the input and compute rows (two
// per SIMD: wave w runs on SIMD w mod 4, so each SIMD interleaves two of them
// and one's waits are filled by the other's work); waves 8..9 copy weight
// blocks (both, each block: a block of 72 copy instructions would overrun one
// wave's limit of outstanding loads) and keep the step's bookkeeping.
constexpr int kComputeWaves = 8;
constexpr int kPollThreads = kComputeWaves * 64;
constexpr int kCopyWave0 = kComputeWaves;
constexpr int kChainWaves = kComputeWaves + 2;
constexpr int kChainThreads = kChainWaves * 64;
constexpr int kDescCache = 128;     // descriptors kept in LDS
constexpr int kChainMaxK = 8192;

// The staged input is kept as four planes: plane w holds uint4 w (pair-order
// fp16 values 8w..8w+7) of every group, so that lanes reading the same plane
// for consecutive groups touch consecutive LDS banks.  The plane stride is
// the group count rounded up to 8 modulo 16 uint4, which puts planes 1 and 3
// on the other half of the banks from planes 0 and 2 when they are written.
__device__ __forceinline__ int chain_plane(int G) { return ((G + 7) >> 4) * 16 + 8; }
constexpr int kXinBytes = 4 * (((kChainMaxK / 32 + 7) >> 4) * 16 + 8) * 16;
constexpr int kWeightBuf = 56 * 1024;  // bytes of each of the two LDS weight buffers
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
    // lanes per row: the least work per lane, passes x groups per lane (every
    // computing wave runs every pass, on clamped rows where the block has
    // none), at most 4 groups per lane; ties go to fewer lanes per row.
    // Blocks of a few long rows take 64 lanes per row, one row per wave.
    const int nr = max(p.na + p.nb, 1);
    int L = 64, best = 1 << 30;
    for (int l = 16; l <= 64; l <<= 1) {
        const int ng = (G + l - 1) / l;
        if (ng > 4) continue;
        const int passes = (nr + kComputeWaves * (64 / l) - 1) / (kComputeWaves * (64 / l));
        if (passes * ng < best) {
            best = passes * ng;
            L = l;
        }
    }
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
                                           const uint16_t *xin, const float *xf, const float2 *xos,
                                           float oscale, const RowSink &sink) {
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
    // the groups' offset sums (staged with the input, or computed here for
    // the first matrix) and input scales 2^-s
    float2 xo[NG];
    float fx[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = l + i * L;
        xo[i] = xos ? (g < G ? xos[g] : make_float2(0.0f, 0.0f)) : group_offset(xr[i]);
        fx[i] = g < G ? xf[g] : 0.0f;
    }
    auto finish = [&](int row, const uint4 (&q)[NG], const uint32_t (&sv)[NG]) __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            acc = (g < G) ? __builtin_fmaf(group_dot_off(q[i], xr[i], xo[i]), bf16_to_f32(sv[i]) * fx[i], acc)
                          : acc;
        }
        acc = lane_group_sum<L>(acc);
        if (l == L - 1 && row >= 0) {
            const float v = __builtin_ldexpf(acc, kGroupDotExp) * oscale;
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
                                               const uint16_t *xin, const float *xf, const float2 *xos,
                                               float oscale, const RowSink &sink) {
    if (b.na + b.nb == 0) return;
    switch (__builtin_amdgcn_readfirstlane(b.sel)) {
        case 16 * 8 + 1: chain_rows<16, 1>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 16 * 8 + 2: chain_rows<16, 2>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 16 * 8 + 3: chain_rows<16, 3>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 16 * 8 + 4: chain_rows<16, 4>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 32 * 8 + 1: chain_rows<32, 1>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 32 * 8 + 2: chain_rows<32, 2>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 32 * 8 + 3: chain_rows<32, 3>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 32 * 8 + 4: chain_rows<32, 4>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 64 * 8 + 1: chain_rows<64, 1>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 64 * 8 + 2: chain_rows<64, 2>(m, b, buf, xin, xf, xos, oscale, sink); break;
        case 64 * 8 + 3: chain_rows<64, 3>(m, b, buf, xin, xf, xos, oscale, sink); break;
        default: chain_rows<64, 4>(m, b, buf, xin, xf, xos, oscale, sink); break;
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

// The largest of v over the 8 lanes of a group (lanes 8k..8k+7): quad
// exchanges, then the mirror within each half row.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
}

// The power of two that puts a group's largest magnitude m in [2^14, 2^15)
// (0 for an all-zero group), kept within fp32's range of powers of two.
__device__ __forceinline__ int group_scale_exp(float m) {
    if (!(m > 0.0f)) return 0;
    const int s = 14 - f32_exponent(m);
    return s > 149 ? 149 : s;
}

// Sum over the 64 lanes of a wave in a fixed order (row shifts within rows of
// 16, then row broadcasts), left in lane 63.
__device__ __forceinline__ float wave_sum_f32(float v) { return lane_group_sum<64>(v); }

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainMat *__restrict__ desc,
                                                              int n, const uint16_t *__restrict__ x0,
                                                              unsigned *sync, unsigned spin_limit) {
    extern __shared__ uint4 smem[];
    // the staged input (four planes) of even and odd steps: a wave may stage
    // step i+1's input while another still reads step i's
    uint16_t *xins = reinterpret_cast<uint16_t *>(smem);
    uint4 *bufs = smem + 2 * (kXinBytes / 16);             // two weight buffers
    ChainMat *dtab = reinterpret_cast<ChainMat *>(bufs + 2 * (kWeightBuf / 16));
    RowBlock *ptab = reinterpret_cast<RowBlock *>(dtab + kDescCache);  // this workgroup's plans
    __shared__ float xfs[2][kChainMaxK / 32];  // per input group: 2^-(its fp16 scale), by parity
    __shared__ float2 xoss[2][kChainMaxK / 32];  // per input group: its offset sums, by parity
    __shared__ double ssp[2][kComputeWaves];  // sums of squares of the poll waves, by step parity
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
            uint16_t *xin = xins + (i & 1) * (kXinBytes / 2);
            float *xf = xfs[i & 1];
            float2 *xos = xoss[i & 1];
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
                for (int g = tid; g < (K >> 5); g += kChainThreads) xf[g] = 1.0f;
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
                if (rn) {
                    const int jn = ((K >> 2) + kPollThreads - 1) / kPollThreads;
                    // the sum of squares: each chunk's on its group-scaled
                    // values in fp32 (no overflow: they are below 2^15), then
                    // scaled back exactly into fp64, over this thread's chunks
                    // in ascending order, then over the wave in a fixed order
                    double ss = 0.0;
                    // each group to fp16 with its own power of two, in the
                    // pair order (x0,x4)(x1,x5)(x2,x6)(x3,x7) of each
                    // 8-value block: chunk c holds values 4(c&1)..+3 of block
                    // u = c>>1 (uint4 u & 3 of group u >> 2); the even lane of
                    // a pair writes the first two words, the odd lane the
                    // last two, each taking two halves from the other
                    const int Gs = chain_plane(K >> 5);
                    uint2 *x8 = reinterpret_cast<uint2 *>(xin);
#pragma unroll
                    for (int j = 0; j < kPollJ; ++j) {
                        if (j < jn) {
                            const int c = tid + kPollThreads * j;
                            const float m = group8_max(fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)),
                                                             fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
                            const int se = group_scale_exp(m);
                            const float s0 = __builtin_ldexpf(v[j].x, se), s1 = __builtin_ldexpf(v[j].y, se);
                            const float s2 = __builtin_ldexpf(v[j].z, se), s3 = __builtin_ldexpf(v[j].w, se);
                            float q = s0 * s0;
                            q = __builtin_fmaf(s1, s1, q);
                            q = __builtin_fmaf(s2, s2, q);
                            q = __builtin_fmaf(s3, s3, q);
                            ss += __builtin_ldexp((double)q, -2 * se);
                            const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)s0);
                            const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)s1);
                            const uint32_t h2v = __builtin_bit_cast(uint16_t, (_Float16)s2);
                            const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)s3);
                            const bool odd = c & 1;
                            const uint32_t give = odd ? (h0 | (h1 << 16)) : (h2v | (h3 << 16));
                            const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
                            const uint2 w = odd ? make_uint2((got & 0xFFFFu) | (h2v << 16), (got >> 16) | (h3 << 16))
                                                : make_uint2(h0 | (got << 16), h1 | (got & 0xFFFF0000u));
                            const int u = c >> 1;
                            if (c < (K >> 2)) {
                                x8[((u & 3) * Gs + (u >> 2)) * 2 + (c & 1)] = w;
                                if ((c & 7) == 0) xf[c >> 3] = __builtin_ldexpf(1.0f, -se);
                            }
                        }
                    }
                    ss = wave_sum_f64(ss);
                    if ((tid & 63) == 0) ssp[i & 1][tid >> 6] = ss;
                    // each group's offset sums, once, by the wave that staged
                    // it (its 8 chunks sit on 8 neighbouring lanes of this
                    // wave, and a wave's LDS accesses complete in order)
                    asm volatile("" ::: "memory");
                    const uint4 *x16 = reinterpret_cast<const uint4 *>(xin);
                    for (int j = 0; j < jn; ++j) {
                        const int c = tid + kPollThreads * j;
                        if ((c & 7) == 0 && c < (K >> 2)) {
                            const int g = c >> 3;
                            h2 xg[16];
#pragma unroll
                            for (int w4 = 0; w4 < 4; ++w4) {
                                const uint4 q = x16[w4 * Gs + g];
                                xg[w4 * 4 + 0] = as_h2(q.x);
                                xg[w4 * 4 + 1] = as_h2(q.y);
                                xg[w4 * 4 + 2] = as_h2(q.z);
                                xg[w4 * 4 + 3] = as_h2(q.w);
                            }
                            xos[g] = group_offset(xg);
                        }
                    }
                }
            }
            // input staged, and this step's weights landed
            lds_barrier();
            if (stop_s) break;
            if (copier) {
                // 2. the copy waves request the next step's block
                if (i + 1 < n)
                    chain_copy(get(i + 1), plan(i + 1), bufs + ((i + 1) & 1) * (kWeightBuf / 16));
                // the step's bookkeeping, off the computing waves' path:
                // step i-1's cells are all in, so every workgroup is done
                // with step i-2's and this one clears its own; descriptor
                // i + kDescCache/2 and its plan go into the slot of
                // i - kDescCache/2
                if (wave == kCopyWave0) {
                    if (i >= 2) {
                        const RowBlock q = plan(i - 2);
                        uint32_t *cells = regions + (long)(i - 2) * kChainMaxK;
                        for (int r = q.ra + (tid & 63); r < min(q.ra + q.na, q.k_next); r += 64) clear_cell(cells, r);
                    }
                    const int j = i + kDescCache / 2;
                    if (j >= kDescCache && j < n) {
                        if ((tid & 63) < kWords)
                            dwords[(j % kDescCache) * kWords + (tid & 63)] = dsrc[(long)j * kWords + (tid & 63)];
                        if ((tid & 63) == kWords) ptab[j % kDescCache] = load_plan(j);
                    }
                }
            } else if (wave < kComputeWaves) {
                // 3. this step's rows
                RowSink sink;
                sink.cells = regions + (long)i * kChainMaxK;
                // the output scale 1/r, from the poll waves' sums of squares
                // (ss = m 2^e with e even and m in [1/4, 1): 1/r =
                // rsq(m / K) 2^(-e/2), each factor within an ulp or two)
                float oscale = 1.0f;
                if (i > 0) {
                    double ss = ssp[i & 1][0];
#pragma unroll
                    for (int w = 1; w < kComputeWaves; ++w) ss += ssp[i & 1][w];
                    if (ss > 0.0) {
                        const int e = __builtin_amdgcn_frexp_exp(ss) & ~1;
                        const float mk = (float)__builtin_ldexp(ss, -e) * __builtin_amdgcn_rcpf((float)K);
                        oscale = __builtin_ldexpf(__builtin_amdgcn_rsqf(mk), -(e >> 1));
                    } else {
                        oscale = 0.0f;
                    }
                }
                chain_rows_any(m, plan(i), bufs + (i & 1) * (kWeightBuf / 16), xin, xf, i > 0 ? xos : nullptr,
                               oscale, sink);
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

static_assert(2 * kXinBytes + 2 * kWeightBuf + kDescCache * 64 + 2 * kChainMaxK / 32 * 12 + 512 <= 160 * 1024,
              "LDS of one workgroup");

size_t chain_lds_bytes() {
    return 2 * (size_t)kXinBytes + 2 * (size_t)kWeightBuf + kDescCache * (sizeof(ChainMat) + sizeof(RowBlock));
}

hipError_t launch_chain(const void *desc, int n, const uint16_t *x0, void *sync, unsigned spin_limit,
                        hipStream_t stream) {
    // One workgroup per CU, all of which must be resident together (each
    // waits for the others' cells): a cooperative launch, which the runtime
    // starts only when the whole grid can be resident and refuses when it
    // never can (the occupancy check makes sure one fits per CU).  The bounded
    // waits for cells stay, for a producer that does not finish.  (A plain
    // launch measured about 10 us faster over the 35-layer sweep, without the
    // guarantee.)
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
    const ChainMat *d = static_cast<const ChainMat *>(desc);
    unsigned *sy = static_cast<unsigned *>(sync);
    void *args[] = {(void *)&d, (void *)&n, (void *)&x0, (void *)&sy, (void *)&spin_limit};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(chain_kernel), dim3(cus), dim3(kChainThreads),
                                   args, (unsigned)lds, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace w4
