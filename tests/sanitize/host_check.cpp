// Host-side checks of libw4 under AddressSanitizer and UndefinedBehaviorSanitizer:
// every entry point's argument validation, the workspace-size arithmetic over
// a grid of shapes (including sizes at and past the limits), the slot-pool
// planner over many steps, settings parsing and the status strings.  It runs
// with no HIP device visible: calls whose arguments are valid stop at the
// device check (W4_ERR_NODEV), so nothing is ever launched.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "w4.h"

static int g_fails = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fails;                                                            \
        }                                                                         \
    } while (0)

int main() {
    // status strings
    for (int s = -20; s <= 5; ++s) EXPECT(w4_strerror(s) != nullptr);
    EXPECT(w4_last_error_detail() != nullptr);

    // workspace sizes: never negative for valid shapes, negative for invalid ones
    const int32_t Ns[] = {1, 15, 16, 17, 33, 1408, 1536, 2816, 16384, 262144, 1 << 24};
    const int32_t Ks[] = {32, 64, 96, 704, 1536, 2048, 2816, 3200, 8192, 16384};
    for (int32_t N : Ns)
        for (int32_t K : Ks) {
            for (int32_t M = 1; M <= W4_MAX_M; ++M) EXPECT(w4_gemm_smallM_workspace_bytes(N, K, M) >= 0);
            EXPECT(w4_gemm_smallM_workspace_bytes(N, K, W4_MAX_M + 1) < 0);
            for (int32_t M : {1, 2, 17, 256, 1000, W4_MAX_M_PROMPT}) EXPECT(w4_gemm_prompt_workspace_bytes(N, K, M) >= 0);
            EXPECT(w4_gemm_prompt_workspace_bytes(N, K, W4_MAX_M_PROMPT + 1) < 0);
            for (int32_t T : {1, 2, 4, 5, 16, 32})
                for (int32_t topk : {1, 4, 8, 32})
                    for (int32_t xdt : {W4_F16, W4_BF16, W4_F32_RMS})
                        for (int32_t xpp : {0, 1})
                            for (int32_t comb : {0, 1})
                                EXPECT(w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, xdt, xpp, comb) >= 0);
        }
    EXPECT(w4_gemm_smallM_workspace_bytes(16, 33, 4) < 0);
    EXPECT(w4_gemm_smallM_workspace_bytes(-1, 32, 4) < 0);
    EXPECT(w4_moe_gemv_ids_workspace_bytes(16, 32, 1, W4_MAX_TOPK + 1, W4_F16, 0, 0) < 0);
    EXPECT(w4_moe_gemv_ids_workspace_bytes(16, 32, 1, 8, 7, 0, 0) < 0);
    for (int32_t H : {1, 8})
        for (int32_t D : {256, 512})
            for (int32_t L : {1, 511, 512, 4099, 131072, 1 << 22}) EXPECT(w4_decode_attention_workspace_bytes(H, D, L) >= 0);
    EXPECT(w4_decode_attention_workspace_bytes(9, 512, 16) < 0);
    EXPECT(w4_decode_attention_workspace_bytes(8, 384, 16) < 0);
    EXPECT(w4_decode_attention_workspace_bytes(8, 512, 0) < 0);

    // host buffers (16-byte aligned), never touched by a device
    const int32_t N = 64, K = 96;
    std::vector<uint32_t> codes(N * K / 8 + 8, 0x88888888u);
    std::vector<uint16_t> steps(N * K / 32 + 8, 0x3F80);
    std::vector<uint16_t> x(16 * K + 8, 0x3C00);
    std::vector<float> xf(16 * K + 8, 1.0f), y(16 * N + 8);
    std::vector<int32_t> ids(64, 1), slot(64, 0);
    std::vector<uint8_t> ws(1 << 20);
    void *wsp = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws.data()) + 255) & ~uintptr_t(255));
    const uint32_t *c = codes.data();
    const uint16_t *s = steps.data();
    const char *odd = reinterpret_cast<const char *>(x.data()) + 1;

    // batch-1 product
    EXPECT(w4_gemv(nullptr, s, N, K, x.data(), W4_F16, y.data(), nullptr) == W4_ERR_INVALID_ARG);
    EXPECT(w4_gemv(c, s, N, 33, x.data(), W4_F16, y.data(), nullptr) == W4_ERR_INVALID_ARG);
    EXPECT(w4_gemv(c, s, N, K, x.data(), 9, y.data(), nullptr) == W4_ERR_DTYPE);
    EXPECT(w4_gemv(c, s, N, K, odd, W4_F16, y.data(), nullptr) == W4_ERR_ALIGNMENT);
    EXPECT(w4_gemv(c, s, N, W4_MAX_K + 32, x.data(), W4_F16, y.data(), nullptr) != W4_OK);
    EXPECT(w4_gemv(c, s, N, K, x.data(), W4_BF16, y.data(), nullptr) == W4_ERR_NODEV);
    EXPECT(w4_gemv(c, s, 0, K, x.data(), W4_BF16, y.data(), nullptr) == W4_OK);
    // small-M
    const int64_t need_m = w4_gemm_smallM_workspace_bytes(N, K, 8);
    EXPECT(w4_gemm_smallM(c, s, N, K, x.data(), W4_F16, 17, K, y.data(), N, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_gemm_smallM(c, s, N, K, x.data(), W4_F16, 8, K - 1, y.data(), N, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_gemm_smallM(c, s, N, K, x.data(), W4_F16, 8, K, y.data(), N - 1, wsp, 1 << 19, nullptr) != W4_OK);
    if (need_m > 0) EXPECT(w4_gemm_smallM(c, s, N, K, x.data(), W4_F16, 8, K, y.data(), N, wsp, need_m - 1, nullptr) != W4_OK);
    EXPECT(w4_gemm_smallM(c, s, N, K, x.data(), W4_F16, 8, K, y.data(), N, wsp, 1 << 19, nullptr) == W4_ERR_NODEV);
    // prompt chunk
    const int64_t need_p = w4_gemm_prompt_workspace_bytes(N, K, 32);
    EXPECT(need_p > 0 && need_p < (1 << 19));
    EXPECT(w4_gemm_prompt(c, s, N, K, x.data(), W4_F16, 32, K, y.data(), N, nullptr, 0, nullptr) != W4_OK);
    EXPECT(w4_gemm_prompt(c, s, N, K, x.data(), W4_F16, 16, K, y.data(), N, wsp, need_p, nullptr) == W4_ERR_NODEV);
    EXPECT(w4_gemm_prompt(c, s, N, K, x.data(), W4_F16, W4_MAX_M_PROMPT + 1, K, y.data(), N, wsp, need_p, nullptr) != W4_OK);
    // grid packing
    std::vector<uint32_t> gc(N * K / 8);
    std::vector<uint16_t> gs(N * K / 32);
    EXPECT(w4_grid_to_codes(x.data(), N, 33, gc.data(), gs.data(), nullptr) != W4_OK);
    EXPECT(w4_grid_to_codes(nullptr, N, K, gc.data(), gs.data(), nullptr) != W4_OK);
    EXPECT(w4_grid_to_codes(x.data(), 16, K, gc.data(), gs.data(), nullptr) == W4_ERR_NODEV);
    // decode attention
    const int64_t need_a = w4_decode_attention_workspace_bytes(8, 256, 8);
    EXPECT(w4_decode_attention(x.data(), 9, 256, x.data(), 256, x.data(), 256, 8, 1.0f, y.data(), wsp, need_a, nullptr) != W4_OK);
    EXPECT(w4_decode_attention(x.data(), 1, 256, x.data(), 255, x.data(), 256, 1, 1.0f, y.data(), wsp, need_a, nullptr) != W4_OK);
    EXPECT(w4_decode_attention(x.data(), 1, 256, x.data(), 256, x.data(), 256, 1, 1.0f, y.data(), wsp, need_a, nullptr) == W4_ERR_NODEV);
    // expert-indexed product
    const int64_t sc = (int64_t)N * K / 8, ss = (int64_t)N * K / 32;
    EXPECT(w4_moe_gemv_ids(c, s, sc, ss, N, K, x.data(), W4_F16, 0, K, ids.data(), 2, W4_MAX_TOPK + 1, nullptr, 2, 0,
                           nullptr, nullptr, y.data(), nullptr, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_moe_gemv_ids(c, s, sc - 1, ss, N, K, x.data(), W4_F16, 0, K, ids.data(), 1, 2, nullptr, 2, 0,
                           nullptr, nullptr, y.data(), nullptr, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_moe_gemv_ids(c, s, sc, ss, N, K, x.data(), W4_F16, 2, K, ids.data(), 1, 2, nullptr, 2, 0,
                           nullptr, nullptr, y.data(), nullptr, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_moe_gemv_ids(c, s, sc, ss, N, K, x.data(), W4_F16, 0, K, ids.data(), 1, 2, slot.data(), 2, 0,
                           nullptr, nullptr, y.data(), nullptr, wsp, 1 << 19, nullptr) != W4_OK);
    EXPECT(w4_moe_gemv_ids(c, s, sc, ss, N, K, xf.data(), W4_F32_RMS, 0, K, ids.data(), 1, 2, nullptr, 2, 0,
                           nullptr, nullptr, y.data(), nullptr, wsp, 1 << 19, nullptr) == W4_ERR_NODEV);
    EXPECT(w4_moe_gemv_ids_noalloc(c, s, sc, ss, N, K, x.data(), W4_BF16, 1, K, ids.data(), 2, 2, nullptr, 2, 0,
                                   nullptr, nullptr, y.data(), nullptr, nullptr) == W4_ERR_NODEV);
    // gather, renormalisation, chain, probe
    EXPECT(w4_embed_gather(c, s, N, K, ids.data(), -1, x.data(), nullptr, nullptr) != W4_OK);
    EXPECT(w4_embed_gather(c, s, N, K, ids.data(), 4, x.data(), nullptr, nullptr) == W4_ERR_NODEV);
    EXPECT(w4_gemv_gather(c, s, N, K, x.data(), W4_BF16, y.data(), ids.data(), -1, x.data(), nullptr, nullptr) != W4_OK);
    EXPECT(w4_gemv_gather(c, s, N, K, x.data(), 9, y.data(), ids.data(), 4, x.data(), nullptr, nullptr) != W4_OK);
    EXPECT(w4_gemv_gather(c, s, N, K, x.data(), W4_BF16, y.data(), ids.data(), 4, x.data(), nullptr, nullptr) == W4_ERR_NODEV);
    EXPECT(w4_gemv_gather(c, s, N, K, x.data(), W4_F16, y.data(), nullptr, 0, nullptr, nullptr, nullptr) == W4_ERR_NODEV);
    EXPECT(w4_rms_renorm(xf.data(), K, K, 2, x.data(), K, 7, nullptr) != W4_OK);
    EXPECT(w4_rms_renorm(xf.data(), K - 1, K, 2, x.data(), K, W4_F16, nullptr) != W4_OK);
    EXPECT(w4_rms_renorm(xf.data(), K, K, 2, x.data(), K, W4_F16, nullptr) == W4_ERR_NODEV);
    w4_chain_mat m[2] = {{c, s, y.data(), N, K}, {c, s, y.data(), N, N}};
    EXPECT(w4_gemv_chain(m, 0, x.data(), wsp, W4_CHAIN_SYNC_BYTES(2), nullptr) != W4_OK);
    EXPECT(w4_gemv_chain(m, 2, x.data(), wsp, W4_CHAIN_SYNC_BYTES(2) - 1, nullptr) != W4_OK);
    EXPECT(w4_probe_stream(nullptr, 1024, nullptr, nullptr) != W4_OK);

    // slot pools: argument checks, then the planner over many steps
    w4_pool *pool = nullptr;
    const int64_t parts[2] = {1024, 256}, bad_parts[2] = {1024, 250};
    EXPECT(w4_pool_create(0, 8, 4, 2, parts, &pool) == W4_ERR_INVALID_ARG);
    EXPECT(w4_pool_create(2, 8, 4, 2, bad_parts, &pool) == W4_ERR_ALIGNMENT);
    EXPECT(w4_pool_create(2, 8, 4, W4_POOL_MAX_PARTS + 1, parts, &pool) == W4_ERR_INVALID_ARG);
    EXPECT(w4_pool_create(3, 48, 16, 2, parts, &pool) == W4_OK && pool != nullptr);
    std::mt19937 rng(5);
    std::vector<int32_t> pids(8), so(48), me(16), ms(16);
    for (int step = 0; step < 2000; ++step) {
        const int layer = step % 3;
        for (int i = 0; i < 8; ++i) pids[i] = (int32_t)(rng() % 48);
        const int st = w4_pool_plan(pool, layer, pids.data(), 8, so.data(), me.data(), ms.data());
        EXPECT(st >= 0 && st <= 8);
        for (int i = 0; i < 8; ++i) EXPECT(so[pids[i]] >= 0 && so[pids[i]] < 16);
    }
    EXPECT(w4_pool_plan(pool, 3, pids.data(), 8, so.data(), me.data(), ms.data()) < 0);
    pids[0] = 48;
    EXPECT(w4_pool_plan(pool, 0, pids.data(), 8, so.data(), me.data(), ms.data()) < 0);
    std::vector<int32_t> many(17);
    for (int i = 0; i < 17; ++i) many[i] = i;  // more distinct experts than slots
    EXPECT(w4_pool_plan(pool, 0, many.data(), 17, so.data(), me.data(), ms.data()) < 0);
    int64_t hits = -1, misses = -1, bytes = -1;
    EXPECT(w4_pool_stats(pool, &hits, &misses, &bytes) == W4_OK && hits >= 0 && misses >= 0);
    w4_pool_destroy(pool);
    w4_pool_destroy(nullptr);

    // settings: odd values are parsed without harm
    setenv("W4_GEMV_TILE", "32,3,1,4,256", 1);
    setenv("W4_SMALLM_ROWS_MAX", "nonsense", 1);
    setenv("W4_MOE_PAIRS_MAX_T", "-7", 1);
    w4_reload_settings();
    setenv("W4_GEMV_TILE", "1,2", 1);
    w4_reload_settings();
    unsetenv("W4_GEMV_TILE");
    unsetenv("W4_SMALLM_ROWS_MAX");
    unsetenv("W4_MOE_PAIRS_MAX_T");
    w4_reload_settings();

    std::printf("host checks: %d failed\n", g_fails);
    return g_fails ? 1 : 0;
}
