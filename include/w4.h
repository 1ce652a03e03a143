/*
 * w4.h -- C ABI of the MI355X (gfx950) W4A16 decode library (libw4.so).
 *
 * The operation throughout is the decode-time product of a 4-bit weight-only
 * quantised matrix with a 16-bit activation vector, computed straight from the
 * packed weights without ever writing a 16-bit copy of them.
 *
 * Sources of the operations (web pages; cited by title and section):
 *   [P1-S1] dev.to, "Gemma 4 on a 4 GB GPU in Plain PyTorch: From Out of Memory
 *           to Faster Than llama.cpp", section "Step 1 - Load Google's QAT
 *           Weights Without Unpacking Them": the W4A16 format -- 4-bit codes in
 *           groups of 32, one bf16 step per group, 16-bit activations.
 *   [P1-S2] same page, "Step 2 - Keep the Vocabulary Tables in 4-Bit": the
 *           vocabulary table kept as 4-bit codes; one copy serves as the input
 *           embedding (a row lookup) and as the output layer (a GEMV).
 *   [P1-S3] same page, "Step 3 - Multiply Straight From the Packed Weights":
 *           a decode step multiplies one vector by every weight matrix, reading
 *           packed words and unpacking in registers; code c stands for c - 8.
 *   [P1-S4] same page, "Step 4 - Replay Each Decode Step as One CUDA Graph" and
 *           the tip "Merge the Small Projections": a decode step is a long chain
 *           of small products, run without host launches in between.
 *   [P1-S6] same page, "Step 6 - Read Prompts in 32-Bit on a Card Without Tensor
 *           Cores": a prompt is read in chunks of 256 tokens, each chunk a
 *           product of many activation rows with every weight matrix.
 *   [P1-S5] same page, "Step 5 - Attention for One Token at a Time": grouped
 *           query heads over one key/value head; the cache in slices whose
 *           partial softmax results are merged.
 *   [P1-S7] same page, "Step 7 - Fit the Full 131,072-Token Context": the
 *           cache is one head of width 512 per layer.
 *   [P3]    anyesh.me, "Running a 26B MoE on an 8 GB Jetson by streaming experts
 *           from SSD", section "Streaming without touching a single GPU kernel":
 *           the expert matmul addresses expert id as base + id * stride; a pool
 *           of slots is read through slot ids and must give bitwise the same
 *           result; per-expert side tensors keep the real expert id.
 *   [P2]    ardana.ai, "Fixing Gemma 4's oversized KV cache", section "A failed
 *           decode must not look uncertain": a failed GPU call must never
 *           leave an untouched output that looks like a valid result.
 *
 * Storage format (shared by every entry point):
 *   codes  uint32[N][K/8], row-major; nibble j (bits 4j..4j+3) of word w of a
 *          row is the code of column 8w+j.  Must be 16-byte aligned.
 *   steps  bf16[N][K/32] (raw uint16 bits), row-major; step of group g of row n
 *          at steps[n*(K/32) + g].
 *   weight w(n,k) = (code(n,k) - 8) * step(n, k/32).
 *   K must be a multiple of 32 and at most W4_MAX_K.
 *   Activations are fp16 or bf16 (raw uint16 bits).  Outputs of products are
 *   fp32; the row gather writes bf16.
 *
 * Conventions:
 *   - All array pointers are DEVICE pointers owned by the caller (the slot
 *     pools' host store excepted).  The compute entry points allocate, free
 *     and synchronise nothing (w4_moe_gemv_ids_noalloc keeps its scratch in a
 *     fixed array of the library's device image); the slot-pool object owns
 *     host state, events and a small pinned staging area (see w4_pool_*).
 *   - Workspaces.  w4_gemm_smallM, w4_gemm_prompt, w4_decode_attention and
 *     w4_moe_gemv_ids need device memory beyond their inputs and outputs
 *     (partial sums, staged activations, per-split partials).  The caller owns
 *     it: the matching *_workspace_bytes call gives the size for a shape (0:
 *     none needed, NULL may be passed); the caller allocates at least that
 *     many bytes, 256-byte aligned, sets them all to zero once before the
 *     workspace's first use, and passes it with every call.  Every workspace
 *     starts with a 16 KiB area of counters; every call that completes leaves
 *     them at zero again, so one workspace serves any number of later calls
 *     (of any of the four entry points, with the largest size they need)
 *     without clearing.  Two calls that may run at the same time (different
 *     streams or host threads) need different workspaces; the rest of their
 *     contents is scratch.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     enqueue and return; the caller synchronises.
 *   - Return value: W4_OK (0) or a negative w4_status.  Argument errors are
 *     detected on the host before any launch (nothing is enqueued, outputs are
 *     untouched).  A failed launch returns W4_ERR_HIP; W4_OK is returned only
 *     after every kernel of the call has been enqueued.
 *   - Results do not depend on pointer values, alignment or the stream: the
 *     kernel configuration is chosen from the shape alone, and no float atomics
 *     are used, so every call is bitwise reproducible.
 *   - Numerics: each product c-8 times an activation is exact; sums run in fp32.
 *     Every product output satisfies |y - y_exact| <= 1e-3 * sum_k |w(n,k) x_k|.
 *   - Thread safety: entry points may be called from several host threads and
 *     streams at once, each call with its own workspace (see above); a chain's
 *     sync buffer and w4_moe_gemv_ids_noalloc's scratch are shared by the
 *     calls that use them, which must not overlap.
 *   - Settings: five environment variables are read once per process (and
 *     again by w4_reload_settings): W4_GEMV_TILE (a tile override of the
 *     batch-1 product), W4_SMALLM_ROWS_MAX and W4_MOE_PAIRS_MAX_T (up to how
 *     many rows / tokens the small-M and expert products run as side-by-side
 *     batch-1 products; 4 by default), all three schedule only;
 *     W4_CHAIN_SPIN_LIMIT (the bound of the chain's waits) and
 *     W4_FORCE_LAUNCH_ERROR=1 (every entry point returns W4_ERR_HIP after
 *     validation without enqueuing anything), two test hooks.
 */
#ifndef W4_H
#define W4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4_OK = 0,
    W4_ERR_INVALID_ARG = -1, /* null pointer, bad size, K % 32 != 0, ... */
    W4_ERR_ALIGNMENT = -2,   /* a pointer is not aligned as documented */
    W4_ERR_DTYPE = -3,       /* unknown activation dtype */
    W4_ERR_UNSUPPORTED = -4, /* valid but beyond the library's limits */
    W4_ERR_NODEV = -5,       /* no usable HIP device */
    W4_ERR_HIP = -6          /* a HIP call or kernel launch failed */
} w4_status;

typedef enum { W4_F16 = 0, W4_BF16 = 1, W4_F32_RMS = 2 } w4_dtype;
/* W4_F32_RMS (w4_moe_gemv_ids only): the activation rows are fp32, and each
 * row's leading K entries are renormalised as part of the product -- divided
 * by their RMS and rounded to fp16 bit for bit as w4_rms_renorm(..., W4_F16)
 * would -- so no separate renormalisation pass runs between two products. */

#define W4_MAX_K 16384       /* largest K of w4_gemv and w4_embed_gather */
#define W4_MAX_K_SMALLM 16384 /* largest K of w4_gemm_smallM and w4_moe_gemv_ids */
#define W4_MAX_K_CHAIN 8192   /* largest K of a w4_gemv_chain record */
#define W4_MAX_M 16     /* largest M of w4_gemm_smallM */
#define W4_MAX_TOPK 32  /* largest experts per token of w4_moe_gemv_ids */
#define W4_MAX_M_PROMPT 4096 /* largest M of w4_gemm_prompt */

/*
 * Batch-1 product [P1-S3]:  y[n] = sum_k w(n,k) * x[k]  for n in [0, N).
 *   codes, steps: one packed matrix [N][K] (see above).
 *   x:   K activations of dtype xdt (W4_F16 or W4_BF16), 2-byte aligned.
 *   y:   N floats (written, never read).
 * N == 0 is a no-op; K == 0 writes zeros.
 */
int w4_gemv(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
            const void *x, int32_t xdt, float *y, void *stream);

/*
 * Small-batch product [P1-S3] with M activation rows, 1 <= M <= W4_MAX_M:
 *   Y[m*ldy + n] = sum_k w(n,k) * X[m*ldx + k]   for m < M, n < N.
 * ldx >= K, ldy >= N, K <= W4_MAX_K_SMALLM (larger K: W4_ERR_UNSUPPORTED).
 * M <= 4 runs M batch-1 products of w4_gemv's kernel side by side in one
 * launch (row m has the bits w4_gemv gives for that row with the same tile;
 * the workgroups of a row block run together, so the weights come from memory
 * about once).  M >= 5 runs on the matrix cores, each weight read from memory
 * once for all M rows; when the plan splits K into slices (to give the chip
 * enough independent work, or to fit the staged activations), the slices are
 * summed in a fixed order inside the same launch, through the workspace
 * (w4_gemm_smallM_workspace_bytes; 0 bytes for the plans that do not split).
 */
int64_t w4_gemm_smallM_workspace_bytes(int32_t N, int32_t K, int32_t M);
int w4_gemm_smallM(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
                   const void *X, int32_t xdt, int32_t M, int64_t ldx,
                   float *Y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                   void *stream);

/*
 * Prompt-chunk product [P1-S6] with M activation rows, 1 <= M <= W4_MAX_M_PROMPT
 * (a chunk of prompt tokens, e.g. 256):
 *   Y[m*ldy + n] = sum_k w(n,k) * X[m*ldx + k]   for m < M, n < N.
 * [P1-S6] is the same page's "Step 6 - Read Prompts in 32-Bit on a Card
 * Without Tensor Cores": prompts are read in chunks of 256 tokens, and the
 * product [256, 1536] x [1536, 24576] is quoted in TFLOP/s.  Here it runs on
 * the matrix cores straight from the packed words (no 16-bit weight matrix).
 *   X: fp16 or bf16 (xdt), 2-byte aligned, ldx >= K.  Y: fp32, ldy >= N,
 *      4-byte aligned; written, never read.  K <= W4_MAX_K_SMALLM.
 * Each weight (c - 8) * step, scaled by a power of two per weight row, and
 * each activation, scaled by a power of two per activation row, is an exact
 * fp16 operand; the products sum in fp32.  Rows outside those exponent ranges
 * (weight steps spanning more than 2^21, or a bf16 subnormal/inf/NaN step;
 * bf16 activation rows spanning more than 2^31, or holding inf/NaN or a
 * subnormal) take slower exact paths, so the bound above holds for all inputs.
 * Two kernels run: the activations are first staged as fp16 into the
 * workspace (w4_gemm_prompt_workspace_bytes: about 2*K*M + N*K/16 bytes, with
 * the scaled steps and per-row flags), then the product.
 */
int64_t w4_gemm_prompt_workspace_bytes(int32_t N, int32_t K, int32_t M);
int w4_gemm_prompt(const uint32_t *codes, const uint16_t *steps, int32_t N, int32_t K,
                   const void *X, int32_t xdt, int32_t M, int64_t ldx,
                   float *Y, int64_t ldy, void *workspace, int64_t workspace_bytes,
                   void *stream);

/*
 * Grid packing of a 16-bit table [P1-S2] (the conversion behind the 4-bit
 * tables): table is bf16 [N][K] (raw uint16 bits, finite values, 16-byte
 * aligned) whose groups of 32 are meant to lie on a 4-bit grid; writes
 * codes [N][K/8] (16-byte aligned) and bf16 steps [N][K/32] in the storage
 * format above.  Per group, in fp32: an = largest magnitude among negative
 * values, ap = largest positive value (0 if none); step = bf16_RNE(an > ap ?
 * an / 8 : ap / 7); code = clamp(rint(v * r) + 8, 0, 15) with r = 1 / step
 * (correctly rounded; all fp32, ties to even), or 8 everywhere when step is 0.  A group of exact
 * grid values (c - 8) * step that uses code 0 or 15 packs back into those codes
 * and that step; other values land within half a step (within about one step
 * for a positive extreme clamped to code 15).  K % 32 == 0, K <= W4_MAX_K.
 */
int w4_grid_to_codes(const uint16_t *table, int32_t N, int32_t K, uint32_t *codes,
                     uint16_t *steps, void *stream);

/*
 * Decode attention for one query token [P1-S5, P1-S7]: H <= 8 query heads over
 * one key/value head of width 256 or 512; the cache is a slot per position or
 * a ring of slots (the page's sliding layers use 512).  Every cached row is
 * streamed once for all heads, in slices whose partial results are merged.
 *   o[h][d] = sum_j p[h][j] * V[j][d],  p[h][.] = softmax_j(scale * q[h] . K[j])
 * over the L cached positions j given (a ring passes its valid slots: the
 * result does not depend on their order).
 *   q: bf16 [H][D] contiguous.  K, V: bf16 rows ldk / ldv elements apart.
 *   D is 256 or 512; K, V 16-byte aligned (8-byte for D = 256) and ldk, ldv
 *   multiples of 8 (of 4).  o: fp32 [H][D], written.  1 <= L.
 * The split partials live in the workspace
 * (w4_decode_attention_workspace_bytes).  Accumulation in fp32 with base-2
 * exponentials.
 */
int64_t w4_decode_attention_workspace_bytes(int32_t H, int32_t D, int32_t L);
int w4_decode_attention(const uint16_t *q, int32_t H, int32_t D, const uint16_t *k, int64_t ldk,
                        const uint16_t *v, int64_t ldv, int32_t L, float scale, float *o,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Expert-indexed product [P3].  T tokens each select topk experts:
 * ids[t*topk + j] is a REAL expert id in [0, n_experts).  The weights used for
 * that choice are the packed matrix [N][K] at
 *     codes_base + a * expert_stride_codes   (uint32 units, multiple of 4)
 *     steps_base + a * expert_stride_steps   (uint16 units)
 * with a = ids[...] (slot_of == NULL: direct addressing) or a = slot_of[id]
 * (pool addressing; slot_of is int32[n_experts] on the device, values in
 * [0, n_slots), -1 for "not resident").  Both addressings run the same kernels
 * with the same reduction order, so equal bytes give bitwise equal results.
 *
 *   X: activation rows, ldx apart: row t (x_per_pair == 0, the same input for
 *      all choices of a token) or row t*topk + j (x_per_pair == 1).  xdt
 *      W4_F16 or W4_BF16 (2-byte aligned), or W4_F32_RMS (fp32 rows, 4-byte
 *      aligned, ldx in floats, renormalised on load; from 5 tokens the rows
 *      are renormalised into the workspace first).
 *   row_scale: optional float[n_experts][N] per-expert output scale, ALWAYS
 *      indexed by the real id (only the weight read goes through slot_of).
 *   route_w: optional float[T][topk].  NULL: Y is float[T*topk][N], one row per
 *      choice.  Non-NULL: Y is float[T][N] = sum over j = 0..topk-1 (ascending)
 *      of route_w[t][j] * (choice j's row).
 *   Up to 4 tokens every choice is its own matrix-vector product (an expert
 *   chosen by several tokens is read once per token); with more tokens the
 *   matrix engine reads each distinct expert once for all its tokens.
 *   dev_err: optional device int32; an id or slot out of range sets it to 1 and
 *      fills the affected output rows with NaN (never leaves them untouched).
 *   The combined form (route_w != NULL), and from 5 tokens any K > 3072
 *   (summed over K-slices in a fixed order), stage per-choice rows in the
 *   workspace (w4_moe_gemv_ids_workspace_bytes, with combined = route_w !=
 *   NULL; 0 bytes when nothing is staged).
 * Limits: T*topk <= 1024, topk <= W4_MAX_TOPK, K <= W4_MAX_K_SMALLM.
 */
int64_t w4_moe_gemv_ids_workspace_bytes(int32_t N, int32_t K, int32_t T, int32_t topk, int32_t xdt,
                                        int32_t x_per_pair, int32_t combined);
int w4_moe_gemv_ids(const uint32_t *codes_base, const uint16_t *steps_base,
                    int64_t expert_stride_codes, int64_t expert_stride_steps,
                    int32_t N, int32_t K,
                    const void *X, int32_t xdt, int32_t x_per_pair, int64_t ldx,
                    const int32_t *ids, int32_t T, int32_t topk,
                    const int32_t *slot_of, int32_t n_experts, int32_t n_slots,
                    const float *row_scale, const float *route_w,
                    float *Y, int32_t *dev_err, void *workspace, int64_t workspace_bytes,
                    void *stream);

/*
 * The expert-indexed product for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): w4_moe_gemv_ids with the same arguments and results (the same
 * kernels, bit for bit), but its scratch is a fixed array of
 * W4_NOALLOC_SCRATCH_BYTES in the library's device image, one per GPU, held
 * until the process ends; no call allocates, frees or synchronises.  A call
 * whose shape needs more scratch than that (w4_moe_gemv_ids_workspace_bytes)
 * returns W4_ERR_UNSUPPORTED before enqueuing anything.  Every call on a GPU
 * shares that GPU's array, so calls on one GPU that may overlap (several
 * streams or host threads) race and must be serialised by the caller.  No
 * part of the array needs to start at zero: the kernels write every value
 * they later read within the same call.
 */
#define W4_NOALLOC_SCRATCH_BYTES (8 << 20)
int w4_moe_gemv_ids_noalloc(const uint32_t *codes_base, const uint16_t *steps_base,
                            int64_t expert_stride_codes, int64_t expert_stride_steps,
                            int32_t N, int32_t K,
                            const void *X, int32_t xdt, int32_t x_per_pair, int64_t ldx,
                            const int32_t *ids, int32_t T, int32_t topk,
                            const int32_t *slot_of, int32_t n_experts, int32_t n_slots,
                            const float *row_scale, const float *route_w,
                            float *Y, int32_t *dev_err, void *stream);

/*
 * Expert slot pools [P3, "Streaming without touching a single GPU kernel" and
 * "Numbers from the actual machine"]: routed experts are kept in a host store
 * and streamed into a small per-layer pool of device slots; the expert
 * product reads the pool through slot ids (w4_moe_gemv_ids with slot_of).
 * A w4_pool holds the host-side state of n_layers layers of n_experts experts
 * and n_slots slots; an expert is n_parts contiguous parts (for example gate/
 * up codes, gate/up steps, down codes, down steps) of part_bytes[p] bytes each
 * (multiples of 16).  Per layer, the caller owns:
 *   a host store: part p of expert e at host_parts[p] + e * part_bytes[p],
 *     in pinned host memory allocated as such (hipHostMalloc or torch's
 *     pin_memory), so that the copies are asynchronous;
 *   a device pool: part p of slot s at dev_parts[p] + s * part_bytes[p] (the
 *     stride w4_moe_gemv_ids takes), and the device slot map int32[n_experts].
 * Per layer and decode step, in order:
 *   w4_pool_prepare(layer, ids)  as soon as the router's choices are known (ids
 *     are real expert ids, host int32, duplicates allowed): the per-layer LFU
 *     -- hits stay; each miss takes the lowest empty slot, else the slot whose
 *     expert this call does not request with the fewest uses (one use per call
 *     that requests it), then the least recently used, then the lowest index
 *     -- and, on copy_stream (a second stream of default priority): a wait for
 *     the layer's last release, the copies of the misses, the upload of the
 *     slot map (-1 for experts not resident) and the layer's event.  More
 *     distinct ids than slots, or an id outside [0, n_experts): an error, no
 *     state changed.  The host blocks only if the slot-map staging of two calls
 *     earlier on this layer is still being read.
 *   (the layer's dense work on the compute stream, overlapping the copies)
 *   w4_pool_join(layer, stream)  the one join: stream waits for the copies.
 *   (the expert products on stream, with slot_of = the device slot map)
 *   w4_pool_release(layer, stream)  after the layer's last read of its pool.
 * w4_pool_plan is the host-side LFU decision alone (no device work; the same
 * state change as prepare): it writes the slot map to slot_of_out
 * (int32[n_experts]) and the misses' experts and slots (in request order) to
 * miss_expert / miss_slot (room for n_ids each), and returns the miss count.
 * One host thread at a time per pool.  w4_pool_stats: hits, misses and bytes
 * copied since creation.
 */
#define W4_POOL_MAX_PARTS 8
typedef struct w4_pool w4_pool;
int w4_pool_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t n_parts,
                   const int64_t *part_bytes, w4_pool **pool);
void w4_pool_destroy(w4_pool *pool);
int w4_pool_plan(w4_pool *pool, int32_t layer, const int32_t *ids, int32_t n_ids, int32_t *slot_of_out,
                 int32_t *miss_expert, int32_t *miss_slot);
int w4_pool_prepare(w4_pool *pool, int32_t layer, const int32_t *ids, int32_t n_ids,
                    const void *const *host_parts, void *const *dev_parts, int32_t *dev_slot_of,
                    void *copy_stream);
int w4_pool_join(w4_pool *pool, int32_t layer, void *stream);
int w4_pool_release(w4_pool *pool, int32_t layer, void *stream);
int w4_pool_stats(const w4_pool *pool, int64_t *hits, int64_t *misses, int64_t *bytes);

/*
 * Row gather from a 4-bit table [P1-S2] (the input-embedding use of the same
 * table that w4_gemv multiplies as the output layer):
 *   out[i*K + k] = bf16_round_nearest_even((code(ids[i], k) - 8) * step)
 * for i < n.  The product is exact in fp32, so the result is bit-exact.
 *   ids: int32[n] on the device; an id outside [0, V) sets *dev_err (if given)
 *   to 1 and fills that output row with bf16 NaN.
 */
int w4_embed_gather(const uint32_t *codes, const uint16_t *steps, int32_t V, int32_t K,
                    const int32_t *ids, int32_t n, uint16_t *out_bf16,
                    int32_t *dev_err, void *stream);

/*
 * The two uses of one 4-bit vocabulary table in a decode step [P1-S2, P1-S3],
 * in a single launch: y = W x as w4_gemv computes it (W the [V][K] table) and
 * the rows ids[0..n) of W dequantised to bf16 as w4_embed_gather computes it.
 * The launch's last workgroups do the gather while the others run the
 * product; both results are bitwise those of the two separate calls.
 * Arguments, layouts, limits and errors are those of w4_gemv (codes, steps,
 * V, K, x, xdt, y) and of w4_embed_gather (ids, n, out_bf16, dev_err); n may
 * be 0 (the product alone).
 */
int w4_gemv_gather(const uint32_t *codes, const uint16_t *steps, int32_t V, int32_t K,
                   const void *x, int32_t xdt, float *y, const int32_t *ids, int32_t n,
                   uint16_t *out_bf16, int32_t *dev_err, void *stream);

/*
 * Renormalisation between chained products [P1-S4], for `rows` vectors at
 * once (K a multiple of 4): for each row r, take the leading K entries u of
 * the fp32 vector
 * v + r*ldv, r_rms = sqrt(mean(u^2)), and write (out + r*ldo)[k] = u[k] / r_rms
 * in dtype out_dt (zeros if r_rms == 0): u[k] times the fp64 reciprocal of
 * r_rms, rounded to fp32 and then to nearest-even in out_dt, which is within
 * one unit in the last place of the exactly rounded quotient.  The sum of
 * squares is taken in fp64 in one fixed order.  One workgroup per row.
 */
int w4_rms_renorm(const float *v, int64_t ldv, int32_t K, int32_t rows, void *out, int64_t ldo,
                  int32_t out_dt, void *stream);

/*
 * One decode-step chain as a single launch [P1-S4]: n_mats packed matrices
 * applied in sequence.  Matrix i (a w4_chain_mat record) has shape [N][K] at
 * codes/steps and writes fp32 y[0..N).  Its input is x0 (fp16, K of matrix 0
 * long, 16-byte aligned) for i == 0, else x = u / r: u the leading K entries
 * of the previous matrix's y, r = sqrt(mean(u^2)) (x = 0 when r = 0).  Each
 * output satisfies |y[n] - sum_k w(n,k) x[k]| <= 1e-3 * sum_k |w(n,k) x[k]| on
 * that exact x: the products run on u, rounded to fp16 one group of 32 at a
 * time with the group's own power-of-two scale, and each finished output is
 * multiplied by 1/r (r from sums of squares taken four values at a time in
 * fp32 and added in fp64 in a fixed order), so no
 * product waits for r before its dot products.  Results are bitwise
 * reproducible from call to call.
 *   desc: DEVICE array of n_mats records (it is read by the kernel).
 *   sync: device buffer of sync_bytes >= W4_CHAIN_SYNC_BYTES(n_mats) bytes,
 *         16-byte aligned, all zero before the first call and then owned by
 *         the chain (a header and one region of exchange cells per matrix; a
 *         call that ends without error leaves it all zero again, so it can be
 *         reused by chains run one after another on one stream).  Word 2 is
 *         an error word written by the kernel: 1 if a wait for another
 *         workgroup's outputs timed out (results incomplete), 2 if a record
 *         was invalid (N < 1, K not a multiple of 32, K larger than
 *         W4_MAX_K_CHAIN or than the previous N, a null or misaligned pointer;
 *         nothing computed).  After an error the caller zeroes the whole
 *         buffer before the next call.
 * One workgroup per CU, all resident at once: the kernel is launched
 * cooperatively, so the runtime starts it only when the whole grid can be
 * resident and the call fails with W4_ERR_HIP when it never can; a wait for a
 * producer that does not finish still ends with error 1 rather than a hang.
 * Concurrent chains must use different sync buffers.
 */
#define W4_CHAIN_SYNC_BYTES(n_mats) (256 + (int64_t)(n_mats) * 32768)
typedef struct {
    const uint32_t *codes; /* device, 16-byte aligned */
    const uint16_t *steps; /* device */
    float *y;              /* device, N floats, 16-byte aligned */
    int32_t N;
    int32_t K;
} w4_chain_mat;
int w4_gemv_chain(const w4_chain_mat *desc, int32_t n_mats, const uint16_t *x0, void *sync,
                  int64_t sync_bytes, void *stream);

/*
 * Plain streaming read of `bytes` bytes (a multiple of 16, buf 16-byte aligned):
 * every 32-bit word is added into *out (device uint32, mod 2^32; the caller
 * zeroes it).  This is the memory-read ceiling that product bandwidths are
 * quoted against ([P1-S3] compares its kernel with a plain sum over memory).
 */
int w4_probe_stream(const void *buf, int64_t bytes, uint32_t *out, void *stream);

/* Re-reads the settings variables (see Conventions); not to be called while
 * another host thread is inside an entry point. */
void w4_reload_settings(void);

/* Static description of a status code. */
const char *w4_strerror(int status);

/* Detail of the last error returned on this host thread ("" if none). */
const char *w4_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
