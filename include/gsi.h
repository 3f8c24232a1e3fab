/*
 * gsi.h - C ABI of libgsi: Gated Subspace Inference (GSI) linear layers on AMD Instinct MI355X
 * (gfx950).
 *
 * The method is the one described in the technical summary "Gated Subspace Inference for
 * transformer acceleration" (gist.science, arXiv 2605.03109), cited as [GSI §n]:
 *
 *   For a linear layer y = W x, W in R^{d_out x d}, and an orthonormal basis V_k in R^{d x k}
 *   of the activation subspace, the input decomposes exactly as x = V_k V_k^T x + r [GSI §2.1].
 *   M = W V_k (d_out x k) is precomputed once and cached; g = V_k^T x. A per-token gate compares
 *   the residual ratio rho = |r| / |x| with a threshold eps [GSI §2.2]:
 *     rho <  eps  -> fast path, y = M g   (reads M instead of W)
 *     rho >= eps  -> slow path, y = W x   (the exact product)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers (memory of the current HIP device) unless a
 *    parameter says "host". The caller allocates and owns every device buffer; the library
 *    only borrows them. W, V, M and aux must stay valid and unmodified for a layer's lifetime.
 *  - Layouts are row-major and dense:
 *      W    [d_out, d]   weight dtype          V   [d, k]   weight dtype
 *      M    [d_out, k]   weight dtype          x   [T, d]   weight dtype (token-major)
 *      y    [T, d_out]   weight dtype          gate[T] uint8, 1 = slow (residual passed through)
 *      rho  [T] float32 (optional, may be NULL): sqrt(|r|^2 / |x|^2), NaN when x = 0.
 *  - dtype is one of GSI_F32, GSI_F16, GSI_BF16 and applies to W, V, M, x and y alike. All
 *    accumulation is float32. g is kept in float32.
 *  - d must be a multiple of 8 with 8 <= d <= 65536; k must be a power of two with
 *    8 <= k <= min(d, 512); 1 <= d_out <= 262144.
 *    Device pointers must be 16-byte aligned.
 *  - The gate is evaluated in float32 as  nr2 < fl(fl(eps*eps) * nx2),  with nx2 = |x|^2 and
 *    nr2 = |x - V g|^2 of the *stored* V (formed exactly through the identity
 *    |x - Vg|^2 = |x|^2 - |g|^2 + g^T (V^T V - I) g with g = V^T x). Ties (rho = eps) go slow,
 *    x = 0 goes slow with y = 0, and NaN/Inf in x go slow and propagate into y.
 *  - `stream` is a hipStream_t passed as void*. Every call only enqueues work on it and returns;
 *    nothing synchronises the host. Validation happens before anything is enqueued: a call that
 *    returns an error code has enqueued nothing. Faults inside kernels surface at the caller's
 *    next synchronisation; a wait inside a kernel that exceeds its time bound records
 *    GSI_ERR_TIMEOUT in the workspace (see gsi_workspace_status).
 *  - Calls on one workspace must not overlap (use one workspace per stream). The workspace keeps
 *    a 64-bit launch counter that tags the in-kernel exchange words; no tag repeats within the
 *    life of a workspace, so it never needs clearing after the first zero fill.
 */
#ifndef GSI_H
#define GSI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gsi_dtype { GSI_F32 = 0, GSI_F16 = 1, GSI_BF16 = 2 };

/*
 * What one site of a stack computes for every token.
 *   GSI_SITE_GATED   the method: gate on rho < eps, y = M g (fast) or W x (slow) [GSI §2.2].
 *   GSI_SITE_STATIC  static projection: y = M g for every token, with no residual norm and no
 *                    gate (the limit eps > 1 of the gate for x != 0) [GSI §2.2, closing remark
 *                    on static projection; §4 negative control]. gate = 0, rho = NaN.
 *   GSI_SITE_DENSE   y = W x for every token: a linear map left outside the method, e.g. the
 *                    attention maps of a stack that gates only its MLP maps (the MLP-only
 *                    predecessor named in [GSI §2]). gate = 1, rho = NaN.
 */
enum gsi_site_mode { GSI_SITE_GATED = 0, GSI_SITE_STATIC = 1, GSI_SITE_DENSE = 2 };

enum gsi_status {
  GSI_OK = 0,
  GSI_ERR_NULL = -1,       /* a required pointer is NULL */
  GSI_ERR_SHAPE = -2,      /* a dimension is out of range (see conventions) */
  GSI_ERR_DTYPE = -3,      /* unknown dtype, or mixed dtypes in one stack */
  GSI_ERR_EPS = -4,        /* eps < 0 or NaN */
  GSI_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required */
  GSI_ERR_ALIGN = -6,      /* a device pointer is not 16-byte aligned */
  GSI_ERR_DEVICE = -7,     /* the current device is not gfx950, or too few co-resident blocks */
  GSI_ERR_HIP = -8,        /* a HIP runtime call or launch failed */
  GSI_ERR_TIMEOUT = -9     /* recorded in a workspace: an in-kernel wait exceeded its bound */
};

typedef struct gsi_layer gsi_layer;
typedef struct gsi_stack gsi_stack;

/* Static text for a status code; never NULL. */
const char* gsi_status_string(int code);

/* GSI_OK if the current HIP device is gfx950 (MI355X), GSI_ERR_DEVICE otherwise. */
int gsi_device_check(void);

/*
 * Bytes of per-layer derived data ("aux") that gsi_layer_create fills: V^T [k, d] in the weight
 * dtype, then V^T V - I [k, k] in float32, then the work split of the batch-1 kernel (256 rows of
 * 80 bytes), then, for 16-bit weights, (V (V^T V - I))^T [k, d] in the weight dtype (the rows
 * whose products with x give h = (V^T V - I) g, the gate's second term [GSI §2.2], for the
 * batched path), each part 256-byte aligned. k = 0 gives the size for gsi_layer_create_dense (the
 * work split only). 0 for invalid arguments.
 */
size_t gsi_layer_aux_bytes(int dtype, int d_out, int d, int k);

/*
 * Scratch bytes gsi_layer_create can use for this shape (0 when it has no use for any). With at
 * least this much, the precomputation runs its products split over K across the chip (float32
 * partial sums added in a fixed order, so the result does not depend on scheduling); without it
 * a single-pass kernel runs. 0 also for invalid arguments.
 */
size_t gsi_layer_create_workspace_bytes(int dtype, int d_out, int d, int k);

/*
 * Create a GSI layer [GSI §2.1]: enqueue on `stream` the precomputation of the cached low-rank
 * weight image M = W V (written to the caller's buffer M, [d_out, k], weight dtype, float32
 * accumulation, rounded to nearest even) and of aux (V^T, V^T V - I and, for 16-bit weights,
 * (V (V^T V - I))^T from V^T V - I split into two parts of the weight dtype). Returns after
 * enqueueing;
 * *out receives a small host handle that borrows W, M and aux (V is not used after the
 * precomputation has run). On error *out is left NULL.
 * ws / ws_bytes: optional device scratch (NULL, or at least gsi_layer_create_workspace_bytes;
 * GSI_ERR_WORKSPACE if smaller), used only by the work this call enqueues: it may be reused for
 * the next call on the same stream, or freed once the stream has passed this call.
 */
int gsi_layer_create(gsi_layer** out, int dtype, int d_out, int d, int k, const void* W, const void* V,
                     void* M, void* aux, size_t aux_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * Create a dense layer (no basis): every token takes y = W x, gate = 1, rho = NaN. Used for the
 * linear maps a stack leaves outside the method (GSI_SITE_DENSE). aux: gsi_layer_aux_bytes with
 * k = 0. Same shape rules as gsi_layer_create without k; same ownership and errors.
 */
int gsi_layer_create_dense(gsi_layer** out, int dtype, int d_out, int d, const void* W, void* aux, size_t aux_bytes,
                           void* stream);

/* Free the host handle (device buffers remain the caller's). NULL is accepted. */
int gsi_layer_destroy(gsi_layer* L);

/* Workspace bytes gsi_forward needs for up to T_max tokens on a layer of this shape (k = 0 for a
 * dense layer). */
size_t gsi_workspace_bytes(int dtype, int d_out, int d, int k, int T_max);

/*
 * Run one GSI layer over T tokens [GSI §2.1-§2.2]: y[t] = M g_t if rho_t < eps else W x_t,
 * gate[t] = 0 (fast) or 1 (slow), rho[t] if rho != NULL. T = 0 returns GSI_OK with nothing
 * enqueued. T < 16 runs the per-token persistent path; T >= 16 the batched path in chunks of at
 * most 64 tokens (16-bit weights: a projection, then one launch that forms every gate and lists
 * the fast and slow tokens on the device and runs the two products, the next chunk's projection
 * beside them; float32 weights: projection, gate, compaction and products in their own
 * launches), with no host synchronisation in either. x must not overlap y, gate or rho. The
 * workspace must be zero-filled before its first use and is kept consistent by the library
 * afterwards.
 */
int gsi_forward(const gsi_layer* L, const void* x, int T, float eps, void* y, uint8_t* gate, float* rho,
                void* ws, size_t ws_bytes, void* stream);

/*
 * A stack of layers ("sites") run in order, as every linear map of a transformer block
 * (QKV, output, MLP in and out) and block after block [GSI §3]. `sites` is a HOST array of
 * n_sites layer handles, all of one dtype; the stack borrows them. The library allocates the
 * work split of every (site, block) of the batch-1 kernel on the device (128 bytes each, freed by
 * gsi_stack_destroy); creation synchronises with the device once.
 * gsi_stack_create runs every layer in its own mode (gated, or dense for a dense layer);
 * gsi_stack_create_modes takes a HOST array of n_sites gsi_site_mode values instead (NULL: the
 * layers' own modes). A dense layer only accepts GSI_SITE_DENSE (GSI_ERR_SHAPE otherwise, as for
 * an unknown mode).
 */
int gsi_stack_create(gsi_stack** out, gsi_layer* const* sites, int n_sites);
int gsi_stack_create_modes(gsi_stack** out, gsi_layer* const* sites, const int* modes, int n_sites);
int gsi_stack_destroy(gsi_stack* S);

/* Workspace bytes gsi_stack_decode needs for steps of T_step tokens. */
size_t gsi_stack_workspace_bytes(const gsi_stack* S, int T_step);

/*
 * Decode n_steps steps of T_step tokens through the stack. Token-major stacked layouts:
 *   X     [n_steps * T_step, sum_s d_s]      row n holds site 0's input, then site 1's, ...
 *   Y     [n_steps * T_step, sum_s d_out_s]  same stacking for the outputs
 *   gates [n_steps * T_step, n_sites] uint8  (1 = slow)
 *   rho   [n_steps * T_step, n_sites] float32, optional (NULL)
 * Sites run in order within a step and steps run in order. Site inputs are read from X (they are
 * not chained from the previous site's output), so a site's input may be read before the
 * previous site's output is complete; X must not overlap Y, gates or rho. T_step < 16 runs one
 * persistent kernel for the whole call, one token at a time (inside a step: each site for each of
 * the step's tokens in turn) on the vector ALU; n_steps * T_step * n_sites must then be below
 * 2^28 (GSI_ERR_SHAPE). T_step >= 16 runs the batched path per (step, site) in chunks of at most
 * 64 tokens, whose products use the matrix cores; a chunk's projection (g, ||x||^2 and the gate
 * pieces, from X and the site's basis only) runs in the same launch as the previous chunk's
 * products, and its gate and products start after those products are complete.
 */
int gsi_stack_decode(gsi_stack* S, const void* X, int n_steps, int T_step, float eps, void* Y, uint8_t* gates,
                     float* rho, void* ws, size_t ws_bytes, void* stream);

/*
 * The batch-1 stack decode for callers that cannot allocate device memory or pass a workspace
 * (code under stream capture, serving loops, harnesses that forbid allocation): gsi_stack_decode
 * with T_step < 16, whose in-kernel exchange state (65,792 bytes) lives in a device array inside
 * the library, one per GPU for the life of the process, instead of in a caller workspace.
 * Arguments as for gsi_stack_decode without ws / ws_bytes. T_step >= 16 (the batched path, whose
 * scratch grows with T_step and d_out) returns GSI_ERR_WORKSPACE; the other checks and errors are
 * those of gsi_stack_decode. Calls share the array of their GPU: calls on one GPU must not overlap
 * (their exchanges would race), and a wait timeout inside the kernel cannot be read back (the
 * launch leaves early with incomplete outputs). The call allocates nothing: its first call on a
 * device only looks up the array's address.
 */
int gsi_stack_decode_noalloc(gsi_stack* S, const void* X, int n_steps, int T_step, float eps, void* Y, uint8_t* gates,
                             float* rho, void* stream);

/*
 * Copy the workspace's status word to *host_status (host pointer) after synchronising `stream`:
 * GSI_OK, or GSI_ERR_TIMEOUT if an in-kernel wait of an earlier call ran past its bound.
 * Resets the word to GSI_OK.
 */
int gsi_workspace_status(void* ws, size_t ws_bytes, int* host_status, void* stream);

/*
 * Calibration of a layer's activation basis with the depth cascade [GSI §2.3]: the basis is
 * computed once from calibration activations (one forward pass over a representative sequence);
 * the basis of layer l + 1 starts from the basis of layer l and is corrected by a few rank-1
 * (DGKS) updates instead of a full SVD per layer.
 *
 * gsi_calibrate runs n_iter (1..64) steps of subspace iteration  Q <- orth(A^T (A Q))  from the
 * start Q0, where orth is Gram-Schmidt over the columns in order (each column projected against
 * the orthonormal columns before it, and a second time when the first projection leaves less
 * than 1/sqrt(2) of its norm: the Daniel-Gragg-Kaufman-Stewart criterion). All float32:
 *   A    [n, d]  calibration activations, one token per row (device)
 *   Q0t  [k, d]  start basis BY ROWS (row j = column j of Q0): a Gaussian draw for the first
 *                layer, the previous layer's calibrated basis for the cascade (device)
 *   Qt   [k, d]  result by rows, orthonormal rows spanning the k-dimensional leading subspace of
 *                A^T A as far as n_iter steps reach it (device). Qt may be Q0t itself; it must
 *                not overlap A or the workspace otherwise (GSI_ERR_SHAPE).
 * Shapes: 8 <= k <= 512, k <= d <= 16384 with d a multiple of 8, k <= n <= 2^20 with n a multiple
 * of 8. The basis is used by the layer as V = transpose(Qt), rounded to the weight dtype by the
 * caller. The workspace (gsi_calibrate_workspace_bytes, no zero-fill needed) holds A^T and the
 * two products; calls on one workspace must not overlap. Enqueues on `stream` and returns.
 */
size_t gsi_calibrate_workspace_bytes(int n, int d, int k);
int gsi_calibrate(int n, int d, int k, const float* A, const float* Q0t, int n_iter, float* Qt, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * One block of a batch-1 decode step with the GSI sites embedded in an unchanged plain attention
 * [GSI §3 item 4, §5 last bullet]: the pages run every linear map as a GSI site and leave
 * attention as it is; the block around the sites is the GPT-J-shaped parallel form (one
 * LayerNorm feeding both branches). For a token x (one row of d, updated in place):
 *   a = LayerNorm(x; gamma, beta), eps_ln 1e-5, statistics in float32
 *   [q | k | v] = site QKV(a), f = site fc_in(a)               stack A: [QKV, fc_in], input [a | a]
 *   K[pos] = k, V[pos] = v; per head h (dh = d / n_heads): o_h = softmax(q_h K_h^T / sqrt(dh)) V_h
 *   over cache rows 0 .. pos (plain softmax, no positional rotation, float32)
 *   u = gelu(f), tanh form
 *   y_out = site out(o), y_mlp = site fc_out(u)                stack B: [out, fc_out], input [o | u]
 *   x += y_out + y_mlp
 * A and B are stacks of one 16-bit dtype with those shapes (A: d -> 3 d and d -> dff; B: d -> d
 * and dff -> d; any site mode), n_heads divides d with d / n_heads in {64, 128, 256},
 * d <= 16384; otherwise GSI_ERR_SHAPE / GSI_ERR_DTYPE. A may instead be one shared-input site
 * d -> 3 d + dff: QKV and fc_in read the same a, so one basis serves both and the site forms one
 * g and decides one gate for both (W rows [q | k | v | f], written to ya as they are); its gate
 * and ratio are then reported in entries 0 and 1 alike. Each stack runs with gate
 * threshold eps through the batch-1 kernel for one token, as an ordinary launch of its co-resident
 * grid (a cooperative launch would add a queue switch before and after each of the two).
 * Buffers (device, 16-byte aligned, the caller's): gamma, beta [d]; x [d]; k_cache, v_cache
 * [>= pos + 1, d] row-major, 0 <= pos < 2^24 (rows 0 .. pos - 1 are read, row pos is written); the step's
 * intermediates, readable after the call: xa [2 d] = [a | a], ya [3 d + dff] = [q | k | v | f],
 * xb [d + dff] = [o | u], yb [2 d] = [y_out | y_mlp]; gates [4] uint8 = QKV, fc_in, out, fc_out
 * (1 = slow); rho [4] float32 in the same order, optional (NULL). None of them may overlap.
 * Workspace: gsi_block_step_workspace_bytes, zero-filled before its first use (it holds the
 * batch-1 kernel's exchange state and the attention's partial sums and per-head arrival counters,
 * kept consistent by the library afterwards); calls on one workspace must not overlap. Arguments are checked before anything
 * is enqueued; the call enqueues five launches on `stream` (LayerNorm, stack A, attention with
 * GELU, stack B, residual add) and returns.
 */
size_t gsi_block_step_workspace_bytes(const gsi_stack* A, const gsi_stack* B, int n_heads);
int gsi_block_step(gsi_stack* A, gsi_stack* B, const void* gamma, const void* beta, void* x, void* k_cache,
                   void* v_cache, int pos, int n_heads, float eps, void* xa, void* ya, void* xb, void* yb,
                   uint8_t* gates, float* rho, void* ws, size_t ws_bytes, void* stream);

/*
 * A whole batch-1 decode step: gsi_block_step for blocks 0 .. n_blocks - 1 in order on the one
 * token row x (each block's output is the next block's input), at cache position pos. A, B, gamma,
 * beta, k_cache and v_cache are HOST arrays of n_blocks per-block arguments as in gsi_block_step;
 * every block must have the same d, d_ff and dtype. xa, ya, xb, yb are shared by the blocks (they
 * hold the last block's intermediates afterwards); gates [n_blocks * 4] and rho [n_blocks * 4]
 * (optional) take each block's four entries in turn. One workspace of
 * gsi_block_step_workspace_bytes of block 0's stacks. Every block's arguments are checked before
 * anything is enqueued; the call enqueues 4 n_blocks + 1 launches on `stream` (a block's residual
 * add and the next block's LayerNorm share one) and returns.
 */
int gsi_decode_step(int n_blocks, gsi_stack* const* A, gsi_stack* const* B, const void* const* gamma,
                    const void* const* beta, void* const* k_cache, void* const* v_cache, int pos, int n_heads,
                    float eps, void* x, void* xa, void* ya, void* xb, void* yb, uint8_t* gates, float* rho, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * gsi_decode_step with the cache position in device memory, so that one captured graph of the call
 * replays token after token [GSI §3 item 4, §5: every linear map a GSI site, attention unchanged].
 * `pos` is a device int32 (4-byte aligned), read by the step's kernels when they run; the call's
 * last launch adds one to it. cache_rows (1 .. 2^24) is the number of rows of every k_cache and
 * v_cache. A step whose *pos lies outside [0, cache_rows) runs no attention and writes no cache
 * row (its outputs are then unspecified). Other arguments, checks and launches as gsi_decode_step
 * (one more launch, the advance); the attention launch always has the grid of the longest cache.
 */
int gsi_decode_step_devpos(int n_blocks, gsi_stack* const* A, gsi_stack* const* B, const void* const* gamma,
                           const void* const* beta, void* const* k_cache, void* const* v_cache, int* pos,
                           int cache_rows, int n_heads, float eps, void* x, void* xa, void* ya, void* xb, void* yb,
                           uint8_t* gates, float* rho, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GSI_H */
