// C ABI of libw4: argument checks on the host, then launches on the caller's
// stream.  Declarations and the contract of every entry point are in w4.h.
//
// A failed call never reports success over untouched outputs (the ardana.ai
// page "Fixing Gemma 4's oversized KV cache", section "A failed decode must not
// look uncertain"): argument errors return before anything is enqueued, launch
// errors are read back with hipGetLastError and returned as W4_ERR_HIP.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>

#include "w4.h"
#include "w4_internal.h"

namespace {

thread_local char g_detail[256] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool forced_launch_error() { return w4::settings().force_launch_error; }

int device_ready() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4_ERR_NODEV, "hipGetDevice: %s", hipGetErrorString(e));
    return W4_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_detail[0] = 0;
    return W4_OK;
}

int check_matrix(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K) {
    if (N < 0 || K < 0) return fail(W4_ERR_INVALID_ARG, "negative size N=%d K=%d", N, K);
    if (K % 32) return fail(W4_ERR_INVALID_ARG, "K=%d is not a multiple of 32", K);
    if (K > W4_MAX_K) return fail(W4_ERR_UNSUPPORTED, "K=%d exceeds %d", K, W4_MAX_K);
    if (N > 0 && K > 0 && (!codes || !steps)) return fail(W4_ERR_INVALID_ARG, "null codes/steps");
    if (codes && !aligned(codes, 16)) return fail(W4_ERR_ALIGNMENT, "codes not 16-byte aligned");
    if (steps && !aligned(steps, 2)) return fail(W4_ERR_ALIGNMENT, "steps not 2-byte aligned");
    return W4_OK;
}

int check_dtype(int32_t dt) {
    if (dt != W4_F16 && dt != W4_BF16) return fail(W4_ERR_DTYPE, "unknown dtype %d", dt);
    return W4_OK;
}

// A caller-owned workspace: at least `need` bytes, 256-byte aligned (NULL is
// allowed when nothing is needed).
int check_workspace(const void *ws, int64_t ws_bytes, size_t need) {
    if (ws_bytes < 0) return fail(W4_ERR_INVALID_ARG, "negative workspace_bytes");
    if (need == 0) return W4_OK;
    if (!ws) return fail(W4_ERR_INVALID_ARG, "a workspace of %zu bytes is needed", need);
    if ((uint64_t)ws_bytes < need)
        return fail(W4_ERR_INVALID_ARG, "workspace of %lld bytes, %zu needed", (long long)ws_bytes, need);
    if (!aligned(ws, 256)) return fail(W4_ERR_ALIGNMENT, "workspace not 256-byte aligned");
    return W4_OK;
}

// Bytes of the expert product's workspace: the counter area and the engine's
// partial sums or per-choice rows, then (fp32 rows on the matrix engine) the
// renormalised fp16 rows, 16-byte aligned.  *xoff gets the offset of those
// rows after the counter area.
size_t moe_ws_bytes(int32_t N, int32_t K, int32_t T, int32_t topk, int32_t xdt, int32_t x_per_pair,
                    bool combined, size_t *xoff) {
    size_t b = w4::moe_workspace(N, K, T, topk, combined);
    const size_t off = (b + 15) / 16 * 16;
    if (xoff) *xoff = off;
    if (xdt == W4_F32_RMS && !w4::moe_by_pairs(T)) b = off + (size_t)(x_per_pair ? T * topk : T) * K * 2;
    return b ? w4::kWsCounterBytes + b : 0;
}

// Scratch of w4_moe_gemv_ids_noalloc: a fixed array in the library's device
// image.  Each GPU the library runs on holds its own copy, at its own address,
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device, with
// that device current, and only that address is ever handed to a kernel.
// Calls that share the array on one GPU must not overlap.
static __device__ __align__(256) unsigned char scratch[W4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4_ERR_NODEV, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(W4_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(W4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4_OK;
}

// Settings: two copies, the current one published through an atomic pointer.
std::mutex g_settings_mu;
w4::Settings g_settings_buf[2];
std::atomic<const w4::Settings *> g_settings{nullptr};
int g_settings_next = 0;

const w4::Settings *read_settings() {
    std::lock_guard<std::mutex> lock(g_settings_mu);
    w4::Settings &s = g_settings_buf[g_settings_next];
    g_settings_next ^= 1;
    s = w4::Settings{};
    const char *e = getenv("W4_FORCE_LAUNCH_ERROR");
    s.force_launch_error = e && e[0] == '1';
    s.chain_spin_limit = 1u << 22;
    s.smallm_rows_max = 4;
    s.moe_pairs_max_t = 4;
    if ((e = getenv("W4_SMALLM_ROWS_MAX"))) s.smallm_rows_max = atoi(e);
    if ((e = getenv("W4_MOE_PAIRS_MAX_T"))) s.moe_pairs_max_t = atoi(e);
    if ((e = getenv("W4_CHAIN_SPIN_LIMIT"))) s.chain_spin_limit = (unsigned)strtoul(e, nullptr, 10);
    if ((e = getenv("W4_GEMV_TILE"))) {
        w4::GemvTile &o = s.gemv_tile;
        o.ring = 0;
        o.pf = 0;
        s.gemv_tile_set = sscanf(e, "%d,%d,%d,%d,%d,%d,%d", &o.L, &o.NG, &o.R, &o.waves, &o.blocks, &o.ring,
                                 &o.pf) >= 5;
    }
    g_settings.store(&s, std::memory_order_release);
    return &s;
}

}  // namespace

namespace w4 {
const Settings &settings() {
    const Settings *s = g_settings.load(std::memory_order_acquire);
    return s ? *s : *read_settings();
}
}  // namespace w4

extern "C" {

void w4_reload_settings(void) { (void)read_settings(); }

int64_t w4_gemm_smallM_workspace_bytes(int32_t N, int32_t K, int32_t M) {
    if (N < 0 || K < 0 || (K % 32) || M < 1 || M > W4_MAX_M || K > W4_MAX_K_SMALLM) return W4_ERR_INVALID_ARG;
    if (N == 0 || K == 0) return 0;
    const size_t b = w4::gemm_smallm_workspace(N, K, M);
    return b ? (int64_t)(w4::kWsCounterBytes + b) : 0;
}

int64_t w4_gemm_prompt_workspace_bytes(int32_t N, int32_t K, int32_t M) {
    if (N < 0 || K < 0 || (K % 32) || M < 1 || M > W4_MAX_M_PROMPT || K > W4_MAX_K_SMALLM)
        return W4_ERR_INVALID_ARG;
    if (N == 0 || K == 0) return 0;
    return (int64_t)(w4::kWsCounterBytes + w4::gemm_prompt_workspace(N, K, M));
}

int64_t w4_decode_attention_workspace_bytes(int32_t H, int32_t D, int32_t L) {
    if (H < 1 || H > 8 || (D != 256 && D != 512) || L < 1) return W4_ERR_INVALID_ARG;
    return (int64_t)(w4::kWsCounterBytes + w4::attn_workspace(H, D, L));
}

int64_t w4_moe_gemv_ids_workspace_bytes(int32_t N, int32_t K, int32_t T, int32_t topk, int32_t xdt,
                                        int32_t x_per_pair, int32_t combined) {
    if (N < 0 || K < 0 || (K % 32) || K > W4_MAX_K_SMALLM || T < 0 || topk < 1 || topk > W4_MAX_TOPK ||
        (int64_t)T * topk > 1024 || (xdt != W4_F16 && xdt != W4_BF16 && xdt != W4_F32_RMS) ||
        (x_per_pair != 0 && x_per_pair != 1))
        return W4_ERR_INVALID_ARG;
    if (N == 0 || K == 0 || T == 0) return 0;
    return (int64_t)moe_ws_bytes(N, K, T, topk, xdt, x_per_pair, combined != 0, nullptr);
}

int w4_gemv(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
            const void *x, int32_t xdt, float *y, void *stream) {
    int st;
    if ((st = check_matrix(codes, steps, N, K))) return st;
    if ((st = check_dtype(xdt))) return st;
    if (N > 0 && (!y || (K > 0 && !x))) return fail(W4_ERR_INVALID_ARG, "null x/y");
    if (x && !aligned(x, 2)) return fail(W4_ERR_ALIGNMENT, "x not 2-byte aligned");
    if (y && !aligned(y, 4)) return fail(W4_ERR_ALIGNMENT, "y not 4-byte aligned");
    if (N == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_gemv(codes, steps, N, K, static_cast<const uint16_t *>(x), xdt, y,
                                    static_cast<hipStream_t>(stream)),
                    "w4_gemv");
}

int w4_gemm_smallM(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
                   const void *X, int32_t xdt, int32_t M, int64_t ldx,
                   float *Y, int64_t ldy, void *workspace, int64_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_matrix(codes, steps, N, K))) return st;
    if ((st = check_dtype(xdt))) return st;
    if (M < 1 || M > W4_MAX_M) return fail(W4_ERR_INVALID_ARG, "M=%d outside 1..%d", M, W4_MAX_M);
    if (K > W4_MAX_K_SMALLM) return fail(W4_ERR_UNSUPPORTED, "K=%d exceeds %d", K, W4_MAX_K_SMALLM);
    if (ldx < K || ldy < N) return fail(W4_ERR_INVALID_ARG, "ldx < K or ldy < N");
    if (N > 0 && (!Y || (K > 0 && !X))) return fail(W4_ERR_INVALID_ARG, "null X/Y");
    if (X && !aligned(X, 2)) return fail(W4_ERR_ALIGNMENT, "X not 2-byte aligned");
    if (Y && !aligned(Y, 4)) return fail(W4_ERR_ALIGNMENT, "Y not 4-byte aligned");
    const size_t ws_need = (N > 0 && K > 0) ? (size_t)w4_gemm_smallM_workspace_bytes(N, K, M) : 0;
    if ((st = check_workspace(workspace, workspace_bytes, ws_need))) return st;
    if (N == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    if (K == 0) {
        // empty sums: write zeros through the product kernel path of the GEMV
        for (int m = 0; m < M; ++m) {
            hipError_t e = w4::launch_gemv(codes, steps, N, 0, static_cast<const uint16_t *>(X), xdt,
                                           Y + (int64_t)m * ldy, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return launched(e, "w4_gemm_smallM");
        }
        return launched(hipSuccess, "w4_gemm_smallM");
    }
    return launched(w4::launch_gemm_smallm(codes, steps, N, K, static_cast<const uint16_t *>(X), ldx,
                                           xdt, M, Y, ldy, ws_need ? workspace : nullptr,
                                           static_cast<hipStream_t>(stream)),
                    "w4_gemm_smallM");
}

int w4_gemm_prompt(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
                   const void *X, int32_t xdt, int32_t M, int64_t ldx,
                   float *Y, int64_t ldy, void *workspace, int64_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_matrix(codes, steps, N, K))) return st;
    if ((st = check_dtype(xdt))) return st;
    if (M < 1 || M > W4_MAX_M_PROMPT) return fail(W4_ERR_INVALID_ARG, "M=%d outside 1..%d", M, W4_MAX_M_PROMPT);
    if (K > W4_MAX_K_SMALLM) return fail(W4_ERR_UNSUPPORTED, "K=%d exceeds %d", K, W4_MAX_K_SMALLM);
    if (ldx < K || ldy < N) return fail(W4_ERR_INVALID_ARG, "ldx < K or ldy < N");
    if (N > 0 && (!Y || (K > 0 && !X))) return fail(W4_ERR_INVALID_ARG, "null X/Y");
    if (X && !aligned(X, 2)) return fail(W4_ERR_ALIGNMENT, "X not 2-byte aligned");
    if (Y && !aligned(Y, 4)) return fail(W4_ERR_ALIGNMENT, "Y not 4-byte aligned");
    const size_t ws_need = (N > 0 && K > 0) ? (size_t)w4_gemm_prompt_workspace_bytes(N, K, M) : 0;
    if ((st = check_workspace(workspace, workspace_bytes, ws_need))) return st;
    if (N == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    if (K == 0) {
        // empty sums: zeros through the batch-1 kernel, row by row
        for (int m = 0; m < M; ++m) {
            hipError_t e = w4::launch_gemv(codes, steps, N, 0, static_cast<const uint16_t *>(X), xdt,
                                           Y + (int64_t)m * ldy, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return launched(e, "w4_gemm_prompt");
        }
        return launched(hipSuccess, "w4_gemm_prompt");
    }
    // the staged rows go after the counter area, which must stay zero
    return launched(w4::launch_gemm_prompt(codes, steps, N, K, static_cast<const uint16_t *>(X), ldx, xdt, M,
                                           Y, ldy, static_cast<char *>(workspace) + w4::kWsCounterBytes,
                                           static_cast<hipStream_t>(stream)),
                    "w4_gemm_prompt");
}

int w4_grid_to_codes(const uint16_t *table, int32_t N, int32_t K, uint32_t *codes,
                     uint16_t *steps, void *stream) {
    if (N < 0 || K < 0) return fail(W4_ERR_INVALID_ARG, "negative N or K");
    if (K % 32) return fail(W4_ERR_INVALID_ARG, "K=%d is not a multiple of 32", K);
    if (K > W4_MAX_K) return fail(W4_ERR_UNSUPPORTED, "K=%d exceeds %d", K, W4_MAX_K);
    if ((long)N * K == 0) return W4_OK;
    if (!table || !codes || !steps) return fail(W4_ERR_INVALID_ARG, "null table/codes/steps");
    if (!aligned(table, 16)) return fail(W4_ERR_ALIGNMENT, "table not 16-byte aligned");
    if (!aligned(codes, 16)) return fail(W4_ERR_ALIGNMENT, "codes not 16-byte aligned");
    if (!aligned(steps, 2)) return fail(W4_ERR_ALIGNMENT, "steps not 2-byte aligned");
    int st;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_grid_pack(table, (long)N * (K / 32), codes, steps,
                                         static_cast<hipStream_t>(stream)),
                    "w4_grid_to_codes");
}

int w4_decode_attention(const uint16_t *q, int32_t H, int32_t D, const uint16_t *k, int64_t ldk,
                        const uint16_t *v, int64_t ldv, int32_t L, float scale, float *o,
                        void *workspace, int64_t workspace_bytes, void *stream) {
    if (H < 1 || H > 8) return fail(W4_ERR_INVALID_ARG, "H=%d outside 1..8", H);
    if (D != 256 && D != 512) return fail(W4_ERR_UNSUPPORTED, "D=%d (256 or 512)", D);
    if (L < 1) return fail(W4_ERR_INVALID_ARG, "L=%d", L);
    if (ldk < D || ldv < D) return fail(W4_ERR_INVALID_ARG, "ldk or ldv < D");
    if (!q || !k || !v || !o) return fail(W4_ERR_INVALID_ARG, "null q/k/v/o");
    const int va = D == 512 ? 16 : 8, vl = D == 512 ? 8 : 4;
    if (!aligned(k, va) || !aligned(v, va) || ldk % vl || ldv % vl)
        return fail(W4_ERR_ALIGNMENT, "k/v rows not %d-byte aligned", va);
    if (!aligned(q, 2) || !aligned(o, 4)) return fail(W4_ERR_ALIGNMENT, "q or o misaligned");
    int st;
    if ((st = check_workspace(workspace, workspace_bytes, w4::kWsCounterBytes + w4::attn_workspace(H, D, L))))
        return st;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_attn(q, H, D, k, ldk, v, ldv, L, scale, o,
                                    static_cast<char *>(workspace) + w4::kWsCounterBytes,
                                    static_cast<hipStream_t>(stream)),
                    "w4_decode_attention");
}

int w4_embed_gather(const uint32_t *codes, const uint16_t *steps, int32_t V, int32_t K,
                    const int32_t *ids, int32_t n, uint16_t *out_bf16, int32_t *dev_err,
                    void *stream) {
    int st;
    if ((st = check_matrix(codes, steps, V, K))) return st;
    if (n < 0) return fail(W4_ERR_INVALID_ARG, "negative n");
    if (n > 0 && (!ids || !out_bf16)) return fail(W4_ERR_INVALID_ARG, "null ids/out");
    if (n > 0 && K > 0 && (!codes || !steps)) return fail(W4_ERR_INVALID_ARG, "null codes/steps");
    if (ids && !aligned(ids, 4)) return fail(W4_ERR_ALIGNMENT, "ids not 4-byte aligned");
    if (out_bf16 && !aligned(out_bf16, 16)) return fail(W4_ERR_ALIGNMENT, "out not 16-byte aligned");
    if (dev_err && !aligned(dev_err, 4)) return fail(W4_ERR_ALIGNMENT, "dev_err not aligned");
    if (n == 0 || K == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_gather(codes, steps, V, K, ids, n, out_bf16, dev_err,
                                      static_cast<hipStream_t>(stream)),
                    "w4_embed_gather");
}

int w4_gemv_gather(const uint32_t *codes, const uint16_t *steps, int32_t V, int32_t K,
                   const void *x, int32_t xdt, float *y, const int32_t *ids, int32_t n,
                   uint16_t *out_bf16, int32_t *dev_err, void *stream) {
    int st;
    if ((st = check_matrix(codes, steps, V, K))) return st;
    if ((st = check_dtype(xdt))) return st;
    if (V > 0 && (!y || (K > 0 && !x))) return fail(W4_ERR_INVALID_ARG, "null x/y");
    if (x && !aligned(x, 2)) return fail(W4_ERR_ALIGNMENT, "x not 2-byte aligned");
    if (y && !aligned(y, 4)) return fail(W4_ERR_ALIGNMENT, "y not 4-byte aligned");
    if (n < 0) return fail(W4_ERR_INVALID_ARG, "negative n");
    if (n > 0 && (!ids || !out_bf16)) return fail(W4_ERR_INVALID_ARG, "null ids/out");
    if (ids && !aligned(ids, 4)) return fail(W4_ERR_ALIGNMENT, "ids not 4-byte aligned");
    if (out_bf16 && !aligned(out_bf16, 16)) return fail(W4_ERR_ALIGNMENT, "out not 16-byte aligned");
    if (dev_err && !aligned(dev_err, 4)) return fail(W4_ERR_ALIGNMENT, "dev_err not aligned");
    if (V == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_gemv_gather(codes, steps, V, K, static_cast<const uint16_t *>(x), xdt, y, ids,
                                           K > 0 ? n : 0, out_bf16, dev_err, static_cast<hipStream_t>(stream)),
                    "w4_gemv_gather");
}

int w4_rms_renorm(const float *v, int64_t ldv, int32_t K, int32_t rows, void *out, int64_t ldo,
                  int32_t out_dt, void *stream) {
    int st;
    if ((st = check_dtype(out_dt))) return st;
    if (K < 0 || rows < 0) return fail(W4_ERR_INVALID_ARG, "negative K or rows");
    if (K % 4) return fail(W4_ERR_INVALID_ARG, "K=%d is not a multiple of 4", K);
    if (rows > 65535) return fail(W4_ERR_UNSUPPORTED, "rows=%d exceeds 65535", rows);
    if (rows > 1 && (ldv < K || ldo < K)) return fail(W4_ERR_INVALID_ARG, "ldv or ldo < K");
    if (K > 0 && rows > 0 && (!v || !out)) return fail(W4_ERR_INVALID_ARG, "null v/out");
    if (v && !aligned(v, 4)) return fail(W4_ERR_ALIGNMENT, "v not 4-byte aligned");
    if (out && !aligned(out, 2)) return fail(W4_ERR_ALIGNMENT, "out not 2-byte aligned");
    if (K == 0 || rows == 0) return W4_OK;
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_rms_renorm(v, ldv, K, rows, out, ldo, out_dt,
                                          static_cast<hipStream_t>(stream)),
                    "w4_rms_renorm");
}

}  // extern "C"

namespace {

// The expert product behind both of its entry points.  `noalloc`: the scratch
// is the library's fixed per-device array (`workspace` is ignored).
int moe_call(const uint32_t *codes_base, const uint16_t *steps_base, int64_t expert_stride_codes,
             int64_t expert_stride_steps, int32_t N, int32_t K, const void *X, int32_t xdt, int32_t x_per_pair,
             int64_t ldx, const int32_t *ids, int32_t T, int32_t topk, const int32_t *slot_of,
             int32_t n_experts, int32_t n_slots, const float *row_scale, const float *route_w, float *Y,
             int32_t *dev_err, void *workspace, int64_t workspace_bytes, bool noalloc, void *stream) {
    const char *name = noalloc ? "w4_moe_gemv_ids_noalloc" : "w4_moe_gemv_ids";
    int st;
    if ((st = check_matrix(codes_base, steps_base, N, K))) return st;
    if (xdt != W4_F32_RMS && (st = check_dtype(xdt))) return st;
    if (K > W4_MAX_K_SMALLM) return fail(W4_ERR_UNSUPPORTED, "K=%d exceeds %d", K, W4_MAX_K_SMALLM);
    if (T < 0 || topk < 1 || topk > W4_MAX_TOPK)
        return fail(W4_ERR_INVALID_ARG, "T=%d topk=%d (topk must be 1..%d)", T, topk, W4_MAX_TOPK);
    if ((int64_t)T * topk > 1024) return fail(W4_ERR_UNSUPPORTED, "T*topk exceeds 1024");
    if (x_per_pair != 0 && x_per_pair != 1) return fail(W4_ERR_INVALID_ARG, "x_per_pair must be 0 or 1");
    if (n_experts < 1) return fail(W4_ERR_INVALID_ARG, "n_experts must be >= 1");
    if (slot_of && n_slots < 1) return fail(W4_ERR_INVALID_ARG, "n_slots must be >= 1 with slot_of");
    if (expert_stride_codes < 0 || expert_stride_steps < 0 || expert_stride_codes % 4)
        return fail(W4_ERR_ALIGNMENT, "expert_stride_codes must be a non-negative multiple of 4");
    if (expert_stride_codes < (int64_t)N * (K / 8) || expert_stride_steps < (int64_t)N * (K / 32))
        return fail(W4_ERR_INVALID_ARG, "expert strides smaller than one expert matrix");
    if (ldx < K) return fail(W4_ERR_INVALID_ARG, "ldx < K");
    if (T > 0 && N > 0 && (!ids || !Y || (K > 0 && !X))) return fail(W4_ERR_INVALID_ARG, "null ids/X/Y");
    if (X && !aligned(X, xdt == W4_F32_RMS ? 4 : 2)) return fail(W4_ERR_ALIGNMENT, "X misaligned");
    if (xdt == W4_F32_RMS && K % 4) return fail(W4_ERR_INVALID_ARG, "K must be a multiple of 4");
    if (Y && !aligned(Y, 4)) return fail(W4_ERR_ALIGNMENT, "Y not 4-byte aligned");
    if (ids && !aligned(ids, 4)) return fail(W4_ERR_ALIGNMENT, "ids not 4-byte aligned");
    if (T == 0 || N == 0) return W4_OK;
    if (K == 0) return fail(W4_ERR_UNSUPPORTED, "K == 0");
    // fp32 rows on the matrix engine: renormalised into the workspace, after
    // the engine's part, as fp16 rows of K (16-byte aligned)
    size_t xoff = 0;
    const size_t ws_need = moe_ws_bytes(N, K, T, topk, xdt, x_per_pair, route_w != nullptr, &xoff);
    if (noalloc) {
        if (ws_need > (size_t)W4_NOALLOC_SCRATCH_BYTES)
            return fail(W4_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch, beyond the fixed %d of %s",
                        ws_need, (int)W4_NOALLOC_SCRATCH_BYTES, name);
    } else if ((st = check_workspace(workspace, workspace_bytes, ws_need))) {
        return st;
    }
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    void *ws = nullptr;
    if (ws_need) {
        if (!noalloc)
            ws = workspace;
        else if ((st = scratch_address(&ws)))
            return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int xrows = x_per_pair ? T * topk : T;
    const bool pre_rms = xdt == W4_F32_RMS && !w4::moe_by_pairs(T);
    const void *Xk = X;
    int64_t ldk = ldx;
    int dtk = xdt;
    if (pre_rms) {
        uint16_t *xr = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + w4::kWsCounterBytes + xoff);
        hipError_t e = w4::launch_rms_renorm(static_cast<const float *>(X), ldx, K, xrows, xr, K, W4_F16, s);
        if (e != hipSuccess) return launched(e, name);
        Xk = xr;
        ldk = K;
        dtk = W4_F16;
    }
    return launched(w4::launch_moe(codes_base, steps_base, expert_stride_codes, expert_stride_steps,
                                   N, K, static_cast<const uint16_t *>(Xk), ldk, dtk, x_per_pair, ids,
                                   T, topk, slot_of, n_experts, n_slots, row_scale, route_w, Y,
                                   ws, dev_err, s),
                    name);
}

}  // namespace

extern "C" {

int w4_moe_gemv_ids(const uint32_t *codes_base, const uint16_t *steps_base,
                    int64_t expert_stride_codes, int64_t expert_stride_steps,
                    int32_t N, int32_t K,
                    const void *X, int32_t xdt, int32_t x_per_pair, int64_t ldx,
                    const int32_t *ids, int32_t T, int32_t topk,
                    const int32_t *slot_of, int32_t n_experts, int32_t n_slots,
                    const float *row_scale, const float *route_w,
                    float *Y, int32_t *dev_err, void *workspace, int64_t workspace_bytes, void *stream) {
    return moe_call(codes_base, steps_base, expert_stride_codes, expert_stride_steps, N, K, X, xdt, x_per_pair,
                    ldx, ids, T, topk, slot_of, n_experts, n_slots, row_scale, route_w, Y, dev_err, workspace,
                    workspace_bytes, false, stream);
}

int w4_moe_gemv_ids_noalloc(const uint32_t *codes_base, const uint16_t *steps_base,
                            int64_t expert_stride_codes, int64_t expert_stride_steps,
                            int32_t N, int32_t K,
                            const void *X, int32_t xdt, int32_t x_per_pair, int64_t ldx,
                            const int32_t *ids, int32_t T, int32_t topk,
                            const int32_t *slot_of, int32_t n_experts, int32_t n_slots,
                            const float *row_scale, const float *route_w,
                            float *Y, int32_t *dev_err, void *stream) {
    return moe_call(codes_base, steps_base, expert_stride_codes, expert_stride_steps, N, K, X, xdt, x_per_pair,
                    ldx, ids, T, topk, slot_of, n_experts, n_slots, row_scale, route_w, Y, dev_err, nullptr, 0,
                    true, stream);
}

int w4_gemv_chain(const w4_chain_mat *desc, int32_t n_mats, const uint16_t *x0, void *sync,
                  int64_t sync_bytes, void *stream) {
    int st;
    if (n_mats < 1) return fail(W4_ERR_INVALID_ARG, "n_mats must be >= 1");
    if (!desc || !x0 || !sync) return fail(W4_ERR_INVALID_ARG, "null desc/x0/sync");
    if (sync_bytes < W4_CHAIN_SYNC_BYTES(n_mats))
        return fail(W4_ERR_INVALID_ARG, "sync buffer of %lld bytes, %lld needed", (long long)sync_bytes,
                    (long long)W4_CHAIN_SYNC_BYTES(n_mats));
    if (!aligned(desc, 8) || !aligned(x0, 16) || !aligned(sync, 16))
        return fail(W4_ERR_ALIGNMENT, "desc, x0 or sync misaligned");
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    // the settings' spin limit bounds each wait for exchange cells (read
    // rounds); tests set it tiny to exercise the timeout path without a hang
    return launched(w4::launch_chain(desc, n_mats, x0, sync, w4::settings().chain_spin_limit,
                                     static_cast<hipStream_t>(stream)),
                    "w4_gemv_chain");
}

int w4_probe_stream(const void *buf, int64_t bytes, uint32_t *out, void *stream) {
    int st;
    if (bytes < 0 || bytes % 16) return fail(W4_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    if (!out || (bytes > 0 && !buf)) return fail(W4_ERR_INVALID_ARG, "null buf/out");
    if ((buf && !aligned(buf, 16)) || !aligned(out, 4)) return fail(W4_ERR_ALIGNMENT, "misaligned");
    if ((st = device_ready())) return st;
    if (forced_launch_error()) return fail(W4_ERR_HIP, "forced launch error (test hook)");
    return launched(w4::launch_probe_stream(buf, bytes, out, static_cast<hipStream_t>(stream)),
                    "w4_probe_stream");
}

const char *w4_strerror(int status) {
    switch (status) {
        case W4_OK: return "ok";
        case W4_ERR_INVALID_ARG: return "invalid argument";
        case W4_ERR_ALIGNMENT: return "misaligned pointer";
        case W4_ERR_DTYPE: return "unknown activation dtype";
        case W4_ERR_UNSUPPORTED: return "unsupported size";
        case W4_ERR_NODEV: return "no HIP device";
        case W4_ERR_HIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

const char *w4_last_error_detail(void) { return g_detail; }

}  // extern "C"
