// Internal launchers of libw4 (host side).  Every launcher enqueues on `stream`
// and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

struct GemvTile {
    int L;       // lanes per row slot
    int NG;      // groups per lane
    int R;       // rows per slot in flight
    int waves;   // waves per workgroup
    int blocks;  // workgroups
    int ring;    // streaming variant: ring depth in tiles (0: register variant)
    int pf;      // register variant: next step's loads issued before this step's math
};

GemvTile gemv_tile(int N, int K);

// Settings read from the environment once per process (again on
// w4_reload_settings): the batch-1 tile override (W4_GEMV_TILE =
// "L,NG,R,waves,blocks[,ring depth[,prefetch]]"), the bounds below which the
// small-M and expert products run as side-by-side batch-1 products, and two
// test hooks.  Each changes only the schedule, never what is computed.
struct Settings {
    bool force_launch_error;    // W4_FORCE_LAUNCH_ERROR=1
    unsigned chain_spin_limit;  // W4_CHAIN_SPIN_LIMIT (read rounds of a chain wait)
    bool gemv_tile_set;
    GemvTile gemv_tile;
    int smallm_rows_max;        // W4_SMALLM_ROWS_MAX (default 4; 0: always the matrix cores)
    int moe_pairs_max_t;        // W4_MOE_PAIRS_MAX_T (default 4; 0: always the matrix engine)
};
const Settings &settings();

hipError_t launch_gemv(const uint32_t *codes, const uint16_t *steps, int N, int K,
                       const uint16_t *x, int dt, float *y, hipStream_t stream);
hipError_t launch_gemv_gather(const uint32_t *codes, const uint16_t *steps, int N, int K, const uint16_t *x,
                              int dt, float *y, const int32_t *ids, int n, uint16_t *out, int32_t *dev_err,
                              hipStream_t stream);

// Small-M products (w4_mfma.h engine).  A workspace is needed when the plan
// splits K (and, for the expert product, when route weights are given);
// *_workspace() returns the bytes of partial sums it needs (0: none).  The
// workspace handed to the launchers starts with kWsCounterBytes of counters
// (one per grid column, at most kMaxGridColumns; zero between calls: the
// caller zeroes a new workspace, and every kernel that uses them leaves them
// at zero); the partial sums follow.
constexpr int kMaxGridColumns = 2048;
constexpr size_t kWsCounterBytes = 16384;
static_assert(kMaxGridColumns * 4 <= (int)kWsCounterBytes, "counter area");
size_t gemm_smallm_workspace(int N, int K, int M);
// decode attention (w4_attn.hip): split partials in the workspace
size_t attn_workspace(int H, int D, int L);
hipError_t launch_attn(const uint16_t *q, int H, int D, const uint16_t *K, long ldk, const uint16_t *V,
                       long ldv, int L, float scale, float *o, void *ws, hipStream_t stream);
// grid packing of a bf16 table (w4_grid.hip): groups = N*K/32
hipError_t launch_grid_pack(const uint16_t *table, long groups, uint32_t *codes, uint16_t *steps,
                            hipStream_t stream);
// prompt-chunk product (w4_gemm_prompt.hip): staged activations, row scales and flags
size_t gemm_prompt_workspace(int N, int K, int M);
hipError_t launch_gemm_prompt(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              void *ws, hipStream_t stream);
int smallm_grid_x(int N, int KW);

hipError_t launch_gemm_smallm(const uint32_t *codes, const uint16_t *steps, int N, int K,
                              const uint16_t *X, long ldx, int dt, int M, float *Y, long ldy,
                              void *ws, hipStream_t stream);

hipError_t launch_gather(const uint32_t *codes, const uint16_t *steps, int V, int K,
                         const int32_t *ids, int n, uint16_t *out, int32_t *dev_err,
                         hipStream_t stream);

hipError_t launch_rms_renorm(const float *v, long ldv, int K, int rows, void *out, long ldo,
                             int out_dt, hipStream_t stream);

size_t moe_workspace(int N, int K, int T, int topk, bool route);

hipError_t launch_gemv_rows(const uint32_t *codes, const uint16_t *steps, int N, int K, const uint16_t *X,
                            long ldx, int dt, int M, float *Y, long ldy, hipStream_t stream);
hipError_t launch_gemv_pairs(const uint32_t *codes_base, const uint16_t *steps_base, int64_t stride_codes,
                             int64_t stride_steps, int N, int K, const uint16_t *X, long ldx, int dt,
                             int x_per_pair, const int32_t *ids, int P, int topk, const int32_t *slot_of,
                             int n_experts, int n_slots, const float *row_scale, float *out,
                             int32_t *dev_err, hipStream_t stream);
bool moe_by_pairs(int T);
hipError_t launch_moe(const uint32_t *codes_base, const uint16_t *steps_base,
                      int64_t stride_codes, int64_t stride_steps, int N, int K,
                      const uint16_t *X, long ldx, int dt, int x_per_pair,
                      const int32_t *ids, int T, int topk, const int32_t *slot_of,
                      int n_experts, int n_slots, const float *row_scale, const float *route_w,
                      float *Y, void *ws, int32_t *dev_err, hipStream_t stream);

size_t chain_lds_bytes();
hipError_t launch_chain(const void *desc, int n, const uint16_t *x0, void *sync, unsigned spin_limit,
                        hipStream_t stream);

hipError_t launch_probe_stream(const void *buf, int64_t bytes, uint32_t *out,
                               hipStream_t stream);

}  // namespace w4
