// Batch-1 W4A16 matrix-vector product for gfx950.
//
// The decode step of the dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch"
// (section "Step 3 - Multiply Straight From the Packed Weights") multiplies one
// activation vector by every packed matrix, unpacking in registers and never
// writing a 16-bit weight copy; its speed limit is the weight read.
//
// Mapping.  A wave's 64 lanes are cut into 64/L row slots of L lanes.  Each slot
// owns one row at a time; lane l of a slot owns the groups g = l, l+L, l+2L, ...
// (< K/32) of every row it visits, so one wave-wide 16-byte load instruction
// reads 64/L contiguous runs of 16*L bytes.  The lane's activations for those
// groups stay in registers for the whole kernel (16 fp16 pairs per group), and
// the workgroup loops over rows with a grid stride, R rows per slot in flight.
// Partial row sums are reduced across the L lanes of a slot by lane shuffles
// in a fixed order, so results are bitwise reproducible.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4_device.h"
#include "w4_gather.h"
#include "w4_internal.h"

namespace w4 {

// Expert-indexed use of the same kernel (see launch_gemv_pairs): pair
// p = blockIdx.y reads the matrix of expert a = ids[p] (slot_of[ids[p]] with a
// slot pool) at codes + a*stride_c4, steps + a*stride_s, multiplies the
// activation row p (x_per_pair) or p / topk, and writes row p of the output
// (times row_scale[ids[p]] when given).  ids == nullptr: a plain product.
struct GemvPairs {
    const int32_t *ids;
    const int32_t *slot_of;
    const float *row_scale;
    int32_t *dev_err;
    int64_t stride_c4, stride_s;
    long ldx;
    int n_experts, n_slots, x_per_pair, topk;
    long ldy;  // ids == nullptr and ldy != 0: gridDim.y activation rows (X ldx, Y ldy apart)
    // The row gather from the same table, run by the last g_wgs workgroups of
    // the grid (one wave per output row and slice of g_slices): rows g_ids[i]
    // of the matrix, dequantised to bf16 into g_out (see gather_row_slice).
    const int32_t *g_ids;
    uint16_t *g_out;
    int32_t *g_err;
    int g_n, g_slices, g_wgs;
};

// RN: the activations are fp32 rows (x points at floats; the pair's row is
// ldx floats apart), renormalised on load: the leading K entries divided by
// their RMS, with the sum of squares in the order of w4_rms_renorm and the
// same two roundings, so the staged fp16 values are bitwise that kernel's.
// Rows renormalised on load of up to this many 4-value chunks per thread
// (K <= 4096) are held in registers between the sum of squares and the staging.
constexpr int kRnRegChunks = 4;

template <int L, int NG, int R, int PF, bool RN = false>
__global__ __launch_bounds__(256) void gemv_kernel(const uint4 *__restrict__ codes,
                                                   const uint16_t *__restrict__ steps,
                                                   int N, int K,
                                                   const uint16_t *__restrict__ x, int dt,
                                                   float *__restrict__ y, const GemvPairs bp) {
    constexpr int SLOTS = kWave / L;
    extern __shared__ _Float16 xs[];  // the raw activations (stage_raw_halves(K))
    // the gather workgroups (none unless asked for); the product uses the rest
    const int gx = (int)gridDim.x - bp.g_wgs;
    if ((int)blockIdx.x >= gx) {
        const int idx = ((int)blockIdx.x - gx) * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
        if (idx < bp.g_n * bp.g_slices)
            gather_row_slice(reinterpret_cast<const uint32_t *>(codes), steps, N, K, bp.g_ids, idx / bp.g_slices,
                             idx % bp.g_slices, bp.g_out, bp.g_err);
        return;
    }
    // This workgroup's expert (uniform: scalar loads).  An id or slot out of
    // range leaves no row untouched: the pair's rows become NaN and the error
    // word is set.  The weight address is the only place the slot enters.
    const float *rs = nullptr;
    if (bp.ids) {
        const int p = blockIdx.y;
        const int e = bp.ids[p];
        int a = e;
        bool bad = e < 0 || e >= bp.n_experts;
        if (!bad && bp.slot_of) {
            a = bp.slot_of[e];
            bad = a < 0 || a >= bp.n_slots;
        }
        y += (long)p * N;
        if (bad) {
            for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < N; n += gx * blockDim.x)
                y[n] = __builtin_nanf("");
            if (blockIdx.x == 0 && threadIdx.x == 0 && bp.dev_err) *bp.dev_err = 1;
            return;
        }
        codes += a * bp.stride_c4;
        steps += a * bp.stride_s;
        if constexpr (RN)
            x = reinterpret_cast<const uint16_t *>(reinterpret_cast<const float *>(x) +
                                                   (long)(bp.x_per_pair ? p : p / bp.topk) * bp.ldx);
        else
            x += (long)(bp.x_per_pair ? p : p / bp.topk) * bp.ldx;
        if (bp.row_scale) rs = bp.row_scale + (long)e * N;
    } else if (bp.ldy) {
        // several activation rows against one matrix: row blockIdx.y
        x += (long)blockIdx.y * bp.ldx;
        y += (long)blockIdx.y * bp.ldy;
    }
    const int G = K >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int l = lane % L, slot = lane / L;
    const int rows_per_iter = nwaves * SLOTS * R;
    const int gstride = gx * rows_per_iter;

    if (G == 0) {  // empty sums
        for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < N; n += gx * blockDim.x)
            y[n] = 0.0f;
        return;
    }

    // Group indices of this lane, clamped so that every load is in bounds and
    // can be issued without a branch; lanes past the row end contribute zero.
    int gc[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) gc[i] = min(l + i * L, G - 1);

    auto load_rows = [&](uint4 (&q)[R][NG], uint32_t (&sv)[R][NG], int r0)
        __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(r0 + (r * nwaves + wave) * SLOTS + slot, N - 1);
            const uint4 *cp = codes + (size_t)row * G;
            const uint16_t *sp = steps + (size_t)row * G;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                // read once: non-temporal loads
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp) + gc[i]);
                q[r][i] = make_uint4(v.x, v.y, v.z, v.w);
                sv[r][i] = __builtin_nontemporal_load(sp + gc[i]);
            }
        }
    };

    // The activations are requested first and the first rows' weights right
    // behind them (every load issued without a branch, rows clamped), so that
    // the staging waits for the activations alone while the weights are in
    // flight; the workgroup stages them once (exact fp16 pairs, or the fp32
    // path for the whole workgroup when they cannot be staged exactly) and
    // every lane copies its own groups into registers.
    uint16_t *raw = reinterpret_cast<uint16_t *>(xs);
    uint4 *staged = reinterpret_cast<uint4 *>(raw + stage_raw_halves(K));
    int row0 = blockIdx.x * rows_per_iter;
    uint4 qa[R][NG];
    uint32_t sa[R][NG];
    Staging st;
    st.scale = 0;  // (RN: fp16 values staged as they are)
    st.fallback = 0;
    if constexpr (RN) {
        __shared__ double red_rn[4];
        const float *xf = reinterpret_cast<const float *>(x);
        const bool vec = (reinterpret_cast<uintptr_t>(xf) & 15) == 0;
        auto load4 = [&](int c) __attribute__((always_inline)) {
            return vec ? reinterpret_cast<const float4 *>(xf)[c]
                       : make_float4(xf[4 * c], xf[4 * c + 1], xf[4 * c + 2], xf[4 * c + 3]);
        };
        const int nc = K >> 2;  // 4-value chunks of the row
        if (nc <= kRnRegChunks * 256) {
            // Thread t holds chunks t, t + 256, ... in registers: the row is
            // read once, for the sum of squares (in sum_squares_256's order)
            // and the staged fp16 pairs.
            float4 xv[kRnRegChunks];
#pragma unroll
            for (int j = 0; j < kRnRegChunks; ++j) xv[j] = load4(min((int)threadIdx.x + 256 * j, nc - 1));
            asm volatile("" ::: "memory");  // (the weight loads stay behind the row's)
            load_rows(qa, sa, row0);
            double ss = 0.0;
#pragma unroll
            for (int j = 0; j < kRnRegChunks; ++j)
                if ((int)threadIdx.x + 256 * j < nc) ss = add_squares4(ss, xv[j]);
            ss = wave_sum_f64(ss);
            if ((threadIdx.x & 63) == 0) red_rn[threadIdx.x >> 6] = ss;
            lds_barrier();
            const double inv = renorm_scale(((red_rn[0] + red_rn[1]) + red_rn[2]) + red_rn[3], K);
            // chunk c holds values 4c..4c+3: the low (c even) or high (c odd)
            // halves of the four words of staged[c / 2]
            uint16_t *sh = reinterpret_cast<uint16_t *>(staged);
#pragma unroll
            for (int j = 0; j < kRnRegChunks; ++j) {
                const int c = (int)threadIdx.x + 256 * j;
                if (c < nc) {
                    uint16_t *o = sh + (c >> 1) * 8 + (c & 1);
                    o[0] = renorm_value(xv[j].x, inv, 0);
                    o[2] = renorm_value(xv[j].y, inv, 0);
                    o[4] = renorm_value(xv[j].z, inv, 0);
                    o[6] = renorm_value(xv[j].w, inv, 0);
                }
            }
        } else {
            // a long row: read twice (for the sum of squares, then for the
            // staged pairs)
            load_rows(qa, sa, row0);
            const double inv = renorm_scale(sum_squares_256(K, load4, red_rn), K);
            for (int c = threadIdx.x; c < (K >> 3); c += blockDim.x) {
                const float4 a = load4(2 * c), b = load4(2 * c + 1);
                const uint32_t h0 = renorm_value(a.x, inv, 0), h1 = renorm_value(a.y, inv, 0);
                const uint32_t h2v = renorm_value(a.z, inv, 0), h3 = renorm_value(a.w, inv, 0);
                const uint32_t h4 = renorm_value(b.x, inv, 0), h5 = renorm_value(b.y, inv, 0);
                const uint32_t h6 = renorm_value(b.z, inv, 0), h7 = renorm_value(b.w, inv, 0);
                staged[c] = make_uint4(h0 | (h4 << 16), h1 | (h5 << 16), h2v | (h6 << 16), h3 | (h7 << 16));
            }
        }
        lds_barrier();
    } else {
        // (rows that are not 16-byte aligned: 16-bit loads, written to LDS
        // before any weight load is requested)
        const bool xvec = stage_vector_path(x);
        if (xvec)
            stage_issue_ordered(x, K, raw);
        else
            for (int i = threadIdx.x; i < K; i += blockDim.x) raw[i] = x[i];
        asm volatile("" ::: "memory");  // (the weight loads stay behind the activations)
        load_rows(qa, sa, row0);
        // each (row, group) takes one 16-byte and one 2-byte load instruction
        if (xvec) wait_vmcnt_upto(2 * R * NG);
        lds_barrier();
        // x staged once per workgroup, then each lane takes its own groups
        st = stage_x_workgroup(raw, staged, K, dt);
    }
    h2 xr[NG][16];
    float2 xo[NG];
    if (!st.fallback) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            if (g < G) {
                load_staged_group(staged, g, xr[i]);
            } else {
#pragma unroll
                for (int p = 0; p < 16; ++p) xr[i][p] = h2{0, 0};
            }
            xo[i] = group_offset(xr[i]);
        }
    }

    // dot_rows: the lane's partial sums of its R rows; store_rows: reduce them
    // over the row's lanes and store.  (The next rows' loads go out between
    // the two: the weight registers are free once the partial sums exist.)
    auto dot_rows = [&](const uint4 (&q)[R][NG], const uint32_t (&sv)[R][NG], float (&acc)[R],
                        auto exact_f32) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = l + i * L;
                float part;
                if constexpr (decltype(exact_f32)::value)
                    part = group_dot_f32(q[r][i], raw + gc[i] * 32, dt);
                else
                    part = group_dot_off(q[r][i], xr[i], xo[i]);
                acc[r] = (g < G) ? __builtin_fmaf(part, bf16_to_f32(sv[r][i]), acc[r]) : acc[r];
            }
        }
    };
    auto store_rows = [&](float (&acc)[R], int r0, auto exact_f32) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc[r] = lane_group_sum<L>(acc[r]);
            const int row = r0 + (r * nwaves + wave) * SLOTS + slot;
            if (l == L - 1 && row < N) {
                const float v = decltype(exact_f32)::value ? acc[r] : __builtin_ldexpf(acc[r], kGroupDotExp - st.scale);
                y[row] = rs ? v * rs[row] : v;
            }
        }
    };

    // Each step issues all R*NG row loads of the lane back to back (clamped,
    // so none sits behind a branch), then does the math; other waves on the
    // CU keep the memory system busy meanwhile.  The first step's loads were
    // issued before the staging.
    // With PF, the loads of the next step are issued before the math of this
    // one (two register sets, alternating), so that each wave keeps a step of
    // weights in flight while it computes.
    auto compute_rows = [&](const uint4 (&q)[R][NG], const uint32_t (&sv)[R][NG], int r0,
                            auto exact_f32) __attribute__((always_inline)) {
        float acc[R];
        dot_rows(q, sv, acc, exact_f32);
        store_rows(acc, r0, exact_f32);
    };
    auto row_loop = [&](auto exact_f32) __attribute__((always_inline)) {
        if (row0 >= N) return;
        if constexpr (PF == 0) {
            for (;;) {
                float acc[R];
                dot_rows(qa, sa, acc, exact_f32);
                const int nxt = row0 + gstride;
                if (nxt < N) load_rows(qa, sa, nxt);
                store_rows(acc, row0, exact_f32);
                row0 = nxt;
                if (row0 >= N) break;
            }
        } else {
            uint4 qb[R][NG];
            uint32_t sb[R][NG];
            for (;;) {
                int nxt = row0 + gstride;
                if (nxt < N) load_rows(qb, sb, nxt);
                compute_rows(qa, sa, row0, exact_f32);
                row0 = nxt;
                if (row0 >= N) break;
                nxt = row0 + gstride;
                if (nxt < N) load_rows(qa, sa, nxt);
                compute_rows(qb, sb, row0, exact_f32);
                row0 = nxt;
                if (row0 >= N) break;
            }
        }
    };
    // The staging outcome is uniform within the wave: branch on it once, in a
    // scalar register.
    if (__builtin_amdgcn_readfirstlane(st.fallback))
        row_loop(std::true_type{});
    else
        row_loop(std::false_type{});
}

// ---- streaming variant -------------------------------------------------------
//
// The same row mapping, fed through LDS.  A tile is SLOTS consecutive rows (one
// per row slot of a wave): their codes, SLOTS*G 16-byte groups, and their steps,
// SLOTS*G bf16 values, are contiguous in memory.  Tiles are dealt to waves
// round-robin over the whole grid, and every wave keeps a private ring of D tile
// buffers in LDS that it fills with direct-to-LDS loads (no registers held while
// the data are in flight) D-1 tiles ahead of the tile it computes.  One
// workgroup of eight waves per CU then keeps about 100 KB of weights in flight
// per CU, which the plain register loads of gemv_kernel cannot.  No workgroup
// barrier is needed after the staging of x: each wave waits only for its own
// loads (vmcnt; loads complete in issue order), and the output stores issued
// between tiles are younger than the tile being waited for.
//
// Preconditions (checked by the host): G = K/32 is a multiple of 8 (every row's
// steps are whole 16-byte chunks), the steps are 16-byte aligned, NG = ceil(G/L),
// so that a tile takes exactly NG code instructions and one step instruction.
template <int L, int NG, int D>
__global__ __launch_bounds__(512) void gemv_ring_kernel(const uint4 *__restrict__ codes,
                                                        const uint16_t *__restrict__ steps,
                                                        int N, int K,
                                                        const uint16_t *__restrict__ x, int dt,
                                                        float *__restrict__ y) {
    constexpr int SLOTS = kWave / L;
    constexpr int kPerTile = NG + 1;  // load instructions per tile
    static_assert((D - 1) * kPerTile <= 63, "vmcnt range");
    extern __shared__ uint4 smem[];
    const int G = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar tile loop
    const int nwaves = blockDim.x >> 6;
    const int l = lane % L, slot = lane / L;

    uint16_t *raw = reinterpret_cast<uint16_t *>(smem);
    const int cchunks = SLOTS * G;      // code chunks of a tile
    const int schunks = SLOTS * G / 8;  // step chunks of a tile (<= 64)
    const int tile_chunks = cchunks + schunks;
    uint4 *staged = smem + stage_raw_halves(K) / 8;
    uint4 *ring = staged + stage_raw_halves(K) / 8 + (long)wave * D * tile_chunks;

    const long ntiles = ((long)N + SLOTS - 1) / SLOTS;
    const long tstride = (long)gridDim.x * nwaves;
    const long last_c = (long)N * G - 1, last_s = (long)N * G / 8 - 1;
    const uint4 *steps16 = reinterpret_cast<const uint4 *>(steps);

    // Request tile t into ring buffer b: NG code instructions (lanes past the
    // tile's chunks idle) and one step instruction; rows past N are clamped to
    // the last row (their results are not stored).
    auto issue = [&](long t, int b) __attribute__((always_inline)) {
        uint4 *dst = ring + b * tile_chunks;
        const long c_base = t * cchunks;
        if (c_base + cchunks - 1 <= last_c) {
            // a whole tile: scalar base, fixed lane offsets
            const uint4 *cb = codes + c_base;
#pragma unroll
            for (int i = 0; i < NG; ++i)
                if (i * 64 + lane < cchunks) lds_dma16_nt(cb, (uint32_t)(i * 64 + lane) * 16u, dst + i * 64);
            if (lane < schunks) lds_dma16_nt(steps16 + c_base / 8, (uint32_t)lane * 16u, dst + cchunks);
        } else {
            // the last tile, cut by N: chunks past the end are clamped
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int c = i * 64 + lane;
                if (c < cchunks) lds_dma16(codes + min(c_base + c, last_c), dst + i * 64);
            }
            if (lane < schunks) lds_dma16(steps16 + min(c_base / 8 + lane, last_s), dst + cchunks);
        }
    };

    // x to LDS first, then the first D-1 tiles of this wave.
    stage_issue(x, K, raw);
    if (!stage_vector_path(x))
        for (int i = threadIdx.x; i < K; i += blockDim.x) raw[i] = x[i];
    long t = (long)blockIdx.x * nwaves + wave;
#pragma unroll
    for (int p = 0; p < D - 1; ++p)
        if (t + p * tstride < ntiles) issue(t + p * tstride, p);
    // x has landed once at most the tiles' loads are outstanding
    if (t + (long)(D - 2) * tstride < ntiles)
        wait_vmcnt_mem<(D - 1) * kPerTile>();
    else
        wait_vmcnt_mem<0>();
    wait_vmcnt<0>();  // (no-op by now; tells the compiler that x has landed)
    lds_barrier();

    const Staging st = stage_x_workgroup(raw, staged, K, dt);
    h2 xr[NG][16];
    float2 xo[NG];
    if (!st.fallback) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            const int g = l + i * L;
            if (g < G) {
                load_staged_group(staged, g, xr[i]);
            } else {
#pragma unroll
                for (int p = 0; p < 16; ++p) xr[i][p] = h2{0, 0};
            }
            xo[i] = group_offset(xr[i]);
        }
    }
    const int scale = st.scale;
    const int fallback = st.fallback;

    auto tile_loop = [&](auto exact_f32) __attribute__((always_inline)) {
        int b = 0, bn = D - 1;  // ring buffers of the tile computed and of the one requested
        for (; t < ntiles; t += tstride) {
            const long tn = t + (long)(D - 1) * tstride;
            if (tn < ntiles) {
                issue(tn, bn);
                wait_vmcnt_mem<(D - 1) * kPerTile>();
            } else {
                wait_vmcnt_mem<0>();
            }
            const uint4 *tc = ring + b * tile_chunks + slot * G;
            const uint16_t *ts = reinterpret_cast<const uint16_t *>(ring + b * tile_chunks + cchunks) + slot * G;
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = l + i * L;
                const int gc = min(g, G - 1);
                const uint4 q = tc[gc];
                const uint32_t sv = ts[gc];
                float part;
                if constexpr (decltype(exact_f32)::value)
                    part = group_dot_f32(q, raw + gc * 32, dt);
                else
                    part = group_dot_off(q, xr[i], xo[i]);
                acc = (g < G) ? __builtin_fmaf(part, bf16_to_f32(sv), acc) : acc;
            }
            acc = lane_group_sum<L>(acc);
            const long row = t * SLOTS + slot;
            if (l == L - 1 && row < N)
                y[row] = decltype(exact_f32)::value ? acc : __builtin_ldexpf(acc, kGroupDotExp - scale);
            b = b + 1 == D ? 0 : b + 1;
            bn = bn + 1 == D ? 0 : bn + 1;
        }
    };
    if (__builtin_amdgcn_readfirstlane(fallback))
        tile_loop(std::true_type{});
    else
        tile_loop(std::false_type{});
}

// ---- tiling table ------------------------------------------------------------

namespace {

typedef void (*GemvFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, int, float *,
                       const GemvPairs);
template <int L, int R>
GemvFn pick_rn_ng(int NG) {
    switch (NG) {
        case 1: return gemv_kernel<L, 1, R, 0, true>;
        case 2: return gemv_kernel<L, 2, R, 0, true>;
        case 3: return gemv_kernel<L, 3, R, 0, true>;
        case 4: return gemv_kernel<L, 4, R, 0, true>;
        case 6: return gemv_kernel<L, 6, R, 0, true>;
        case 8: return gemv_kernel<L, 8, R, 0, true>;
    }
    return nullptr;
}

// the kernels that renormalise fp32 rows on load (R = 1 or 3 rows per slot in
// flight, no prefetch)
template <int R>
GemvFn pick_rn(int L, int NG) {
    switch (L) {
        case 8: return pick_rn_ng<8, R>(NG);
        case 16: return pick_rn_ng<16, R>(NG);
        case 32: return pick_rn_ng<32, R>(NG);
        case 64: return pick_rn_ng<64, R>(NG);
    }
    return nullptr;
}

typedef void (*RingFn)(const uint4 *, const uint16_t *, int, int, const uint16_t *, int, float *);

template <int L, int NG>
GemvFn pick_r(int R, int pf) {
    switch (R * 2 + (pf ? 1 : 0)) {
        case 2: return gemv_kernel<L, NG, 1, 0>;
        case 3: return gemv_kernel<L, NG, 1, 1>;
        case 4: return gemv_kernel<L, NG, 2, 0>;
    }
    return nullptr;
}

template <int L>
GemvFn pick_ng(int NG, int R, int pf) {
    switch (NG) {
        case 1: return pick_r<L, 1>(R, pf);
        case 2: return pick_r<L, 2>(R, pf);
        case 3: return pick_r<L, 3>(R, pf);
        case 4: return pick_r<L, 4>(R, pf);
        case 6: return pick_r<L, 6>(R, pf);
        case 8: return pick_r<L, 8>(R, pf);
    }
    return nullptr;
}

GemvFn pick(int L, int NG, int R, int pf) {
    switch (L) {
        case 8: return pick_ng<8>(NG, R, pf);
        case 16: return pick_ng<16>(NG, R, pf);
        case 32: return pick_ng<32>(NG, R, pf);
        case 64: return pick_ng<64>(NG, R, pf);
    }
    return nullptr;
}

template <int L, int NG>
RingFn pick_ring_d(int D) {
    switch (D) {
        case 2: return gemv_ring_kernel<L, NG, 2>;
        case 3: return gemv_ring_kernel<L, NG, 3>;
        case 4: return gemv_ring_kernel<L, NG, 4>;
        case 5: return gemv_ring_kernel<L, NG, 5>;
        case 6: return gemv_ring_kernel<L, NG, 6>;
    }
    return nullptr;
}

RingFn pick_ring(int L, int NG, int D) {
    switch (L * 16 + NG) {
        case 16 * 16 + 3: return pick_ring_d<16, 3>(D);
        case 16 * 16 + 4: return pick_ring_d<16, 4>(D);
        case 32 * 16 + 3: return pick_ring_d<32, 3>(D);
        case 32 * 16 + 4: return pick_ring_d<32, 4>(D);
        case 64 * 16 + 3: return pick_ring_d<64, 3>(D);
        case 64 * 16 + 4: return pick_ring_d<64, 4>(D);
    }
    return nullptr;
}

constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU (gfx950)
constexpr int kRingMaxD = 6;

// Bytes of one ring buffer (a tile of 64/L rows: codes then steps).
int ring_tile_bytes(int L, int K) {
    const int G = K / 32;
    return (64 / L) * G * 16 + (64 / L) * G * 2;
}

}  // namespace

GemvTile gemv_tile(int N, int K) {
    // Lanes per row L and groups per lane NG: cover the G = K/32 groups of a
    // row with as few idle lane slots as possible; among equal covers prefer
    // 16 lanes per row and three or four groups per lane, which measured best
    // on MI355X (e.g. 262144 x 1536: L=16, NG=3 at 4.8 TB/s against 3.1 TB/s
    // for L=64, NG=1 with a quarter of the lanes idle).
    const int G = K / 32;
    static const int kL[] = {16, 32, 64, 8};
    static const int kNG[] = {3, 4, 2, 6, 1, 8};
    GemvTile best{16, 3, 2, 4, 0};
    double best_cost = 1e30;
    for (int L : kL) {
        for (int NG : kNG) {
            if (L * NG < G) continue;
            double cost = double(L * NG - G) / double(L * NG);
            if (NG > 4) cost += 0.02 * (NG - 4);  // register pressure
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                best = GemvTile{L, NG, 1, 4, 0};
            }
        }
    }
    if (G == 0) best = GemvTile{64, 1, 1, 4, 0};
    // One row per slot in flight and four-wave workgroups (fewer registers,
    // more waves per CU measured faster than two rows per slot); at most four
    // workgroups per CU (1024), each looping over rows with a grid stride.
    const long rows_per_iter = (long)(64 / best.L) * best.R * best.waves;
    const long blocks = (N + rows_per_iter - 1) / rows_per_iter;
    best.blocks = (int)(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
    // (the streaming ring variant measured no faster than this kernel; it is
    // chosen only by the tile override)
    best.ring = 0;
    return best;
}

// The schedule of a batch-1 product: the per-shape table, the wide-row form
// for products too small to fill the chip, then the settings' override.
static GemvTile choose_gemv_tile(int N, int K) {
    GemvTile t = gemv_tile(N, K);
    // A product too small to give every CU a workgroup is latency-bound: 64
    // lanes per row (four rows per workgroup) spread it over more workgroups
    // even with idle lanes (2048 x 1536: 3.3 against 3.6 us per call).
    {
        const int G = K / 32;
        const long rpi = (long)(64 / t.L) * t.R * t.waves;
        const int ng64 = (G + 63) / 64;
        if (!t.ring && t.L < 64 && G > 0 && ng64 <= 8 && (N + rpi - 1) / rpi < 256 &&
            pick(64, ng64, 1, 0) != nullptr) {
            const long b64 = ((long)N + 3) / 4;
            t = GemvTile{64, ng64, 1, 4, (int)(b64 > 1024 ? 1024 : b64), 0, 0};
        }
    }
    // The tile override of the settings (W4_GEMV_TILE, read once per process)
    // changes only the schedule, never what is computed.
    {
        const Settings &cfg = settings();
        const GemvTile &o = cfg.gemv_tile;
        if (cfg.gemv_tile_set && o.L * o.NG * 32 >= K && o.waves >= 1 && o.waves <= (o.ring ? 8 : 4) &&
            o.blocks >= 1 && o.ring >= 0 && o.ring <= kRingMaxD)
            t = o;
    }
    return t;
}

hipError_t launch_gemv(const uint32_t *codes, const uint16_t *steps, int N, int K,
                       const uint16_t *x, int dt, float *y, hipStream_t stream) {
    const GemvTile t = choose_gemv_tile(N, K);
    if (t.ring) {
        // the ring kernel's preconditions (a bad override is refused)
        const int G = K / 32;
        RingFn fn = pick_ring(t.L, t.NG, t.ring);
        if (!fn || G == 0 || G % 8 != 0 || t.NG != (G + t.L - 1) / t.L ||
            (reinterpret_cast<uintptr_t>(steps) & 15) != 0 || t.waves < 1 || t.waves > 8)
            return hipErrorInvalidConfiguration;
        const size_t lds = (size_t)stage_raw_halves(K) * 4 +
                           (size_t)t.waves * t.ring * ring_tile_bytes(t.L, K);
        if (lds > (size_t)kLdsBytes) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(fn, dim3(t.blocks), dim3(64 * t.waves), lds, stream,
                           reinterpret_cast<const uint4 *>(codes), steps, N, K, x, dt, y);
        return hipGetLastError();
    }
    GemvFn fn = pick(t.L, t.NG, t.R, t.pf);
    if (!fn) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)2 * stage_raw_halves(K) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3(t.blocks), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, x, dt, y, GemvPairs{});
    return hipGetLastError();
}

// The product and the row gather from the same table in one launch: the
// product's grid as launch_gemv would run it, plus one workgroup per
// (waves per workgroup) gather rows and slices after it.  The two share no
// memory but the table they read, so each output is bitwise what the separate
// launches give.  (Under a ring-kernel override the two run as two launches.)
hipError_t launch_gemv_gather(const uint32_t *codes, const uint16_t *steps, int N, int K, const uint16_t *x,
                              int dt, float *y, const int32_t *ids, int n, uint16_t *out, int32_t *dev_err,
                              hipStream_t stream) {
    const GemvTile t = choose_gemv_tile(N, K);
    const int slices = ((K >> 3) + kSliceWords - 1) / kSliceWords;
    if (t.ring || n == 0 || K == 0) {
        hipError_t e = launch_gemv(codes, steps, N, K, x, dt, y, stream);
        if (e != hipSuccess || n == 0 || K == 0) return e;
        return launch_gather(codes, steps, N, K, ids, n, out, dev_err, stream);
    }
    GemvFn fn = pick(t.L, t.NG, t.R, t.pf);
    const long gwaves = (long)n * slices, gwgs = (gwaves + t.waves - 1) / t.waves;
    if (!fn || gwgs > 65535 || (long)t.blocks + gwgs > 2147483647L) return hipErrorInvalidConfiguration;
    GemvPairs bp{};
    bp.g_ids = ids;
    bp.g_out = out;
    bp.g_err = dev_err;
    bp.g_n = n;
    bp.g_slices = slices;
    bp.g_wgs = (int)gwgs;
    const size_t lds = (size_t)2 * stage_raw_halves(K) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3((unsigned)(t.blocks + gwgs)), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, x, dt, y, bp);
    return hipGetLastError();
}

// M activation rows against one matrix, as M batch-1 products side by side
// (gridDim.y = M): the M workgroups of a row block run together, so the
// weights come from HBM about once and from the caches for the other rows.
hipError_t launch_gemv_rows(const uint32_t *codes, const uint16_t *steps, int N, int K, const uint16_t *X,
                            long ldx, int dt, int M, float *Y, long ldy, hipStream_t stream) {
    const GemvTile t = gemv_tile(N, K);
    GemvFn fn = pick(t.L, t.NG, 1, 0);
    if (!fn || M < 1 || M > 65535 || ldy < 1) return hipErrorInvalidConfiguration;
    const long rows_per_iter = (long)(64 / t.L) * t.waves;
    const long need = (N + rows_per_iter - 1) / rows_per_iter;
    long bx = (512 + M - 1) / M;  // 512 in all: measured best at M = 2 and 4
    if (bx > need) bx = need;
    if (bx < 1) bx = 1;
    GemvPairs bp{};
    bp.ldx = ldx;
    bp.ldy = ldy;
    const size_t lds = (size_t)2 * stage_raw_halves(K) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3((unsigned)bx, (unsigned)M), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes), steps, N, K, X, dt, Y, bp);
    return hipGetLastError();
}

// Expert-indexed products with one activation row per pair: P products of
// [N][K] matrices in one launch, gridDim.y = P, the tile of a single [N][K]
// product; 512 workgroups in all up to 8 pairs, 768 beyond, so that each
// loops over a few row steps (the activation staging is paid once per
// workgroup).  Measured over an expert token: at 8 pairs (one token) 64 per
// pair gave 566-579 us against 625 us with 72 and 629 us with 128; at 32
// pairs 24 per pair gave 976-982 us against 999 with 32 and 1013 with 16.
hipError_t launch_gemv_pairs(const uint32_t *codes_base, const uint16_t *steps_base, int64_t stride_codes,
                             int64_t stride_steps, int N, int K, const uint16_t *X, long ldx, int dt,
                             int x_per_pair, const int32_t *ids, int P, int topk, const int32_t *slot_of,
                             int n_experts, int n_slots, const float *row_scale, float *out,
                             int32_t *dev_err, hipStream_t stream) {
    const GemvTile t = gemv_tile(N, K);
    // dt 2: fp32 rows renormalised on load.  Up to 8 pairs (one token) those
    // launches keep three rows per slot in flight, so that a workgroup's rows
    // are requested at once (an expert token 441-445 against 455-458 us);
    // with more pairs one row per slot stays (at 32 pairs three measured
    // 932-938 against 851-884 us).
    const int R = (dt == 2 && P <= 8) ? 3 : 1, pf = 0;
    GemvFn fn = dt == 2 ? (t.waves == 4 ? (R == 3 ? pick_rn<3>(t.L, t.NG) : pick_rn<1>(t.L, t.NG)) : nullptr)
                        : pick(t.L, t.NG, R, pf);
    if (!fn || P < 1 || P > 65535) return hipErrorInvalidConfiguration;
    const long rows_per_iter = (long)(64 / t.L) * t.waves * R;
    const long need = (N + rows_per_iter - 1) / rows_per_iter;
    long bx = ((P <= 8 ? 512 : 768) + P - 1) / P;
    if (bx > need) bx = need;
    if (bx < 1) bx = 1;
    GemvPairs bp{};
    bp.ids = ids;
    bp.slot_of = slot_of;
    bp.row_scale = row_scale;
    bp.dev_err = dev_err;
    bp.stride_c4 = stride_codes / 4;
    bp.stride_s = stride_steps;
    bp.ldx = ldx;
    bp.n_experts = n_experts;
    bp.n_slots = n_slots;
    bp.x_per_pair = x_per_pair;
    bp.topk = topk;
    const size_t lds = (size_t)2 * stage_raw_halves(K) * sizeof(_Float16);
    hipLaunchKernelGGL(fn, dim3((unsigned)bx, (unsigned)P), dim3(64 * t.waves), lds, stream,
                       reinterpret_cast<const uint4 *>(codes_base), steps_base, N, K, X, dt, out, bp);
    return hipGetLastError();
}

}  // namespace w4
