/*
 * flint_moe.h -- C ABI of the Flint routed-expert MoE layer for AMD MI355X (gfx950).
 *
 * The layer (pages on the Flint release):
 *   - "Recursive Flint serving kit" review (asivanadi0.github.io), section
 *     "The architecture, from the config": 256 routed experts per MoE layer,
 *     6 selected per token, plus an always-on shared expert; expert intermediate
 *     size 512, shared expert 1024; sigmoid router scores with normalised top-k,
 *     not softmax.  The same section's parameter count fits gated three-matrix
 *     (gate, up, down) experts.
 *   - "Recursive opens Flint, a 40B coding model with 2.5B active" (promtime.net),
 *     section "What runs on each token": a router picks 6 of 256 expert
 *     sub-networks for each token and one shared expert runs every time.
 *
 * For each token x (length H):
 *   z_e   = x . router[e] (+ router_bias[e])            e = 0..E-1, float32
 *   s_e   = sigmoid(z_e)                                 float32 (a subnormal for
 *           logits between about -103.3 and -87.3, 0 below, 1 above about 17)
 *   S     = the K experts with the largest s_e (equal scores: lower index first),
 *           reported in ascending expert order
 *   w_e   = s_e / sum_{j in S} s_j                       float32, e in S
 *           (1/K each when every selected s_e is 0: the quotient is 0/0 there,
 *           and 1/K is what equal scores give)
 *   h_e   = silu(gate[e] x) * (up[e] x),  silu(g) = g * sigmoid(g), stored in the
 *           layer's dtype
 *   out   = sum_{e in S} w_e * down[e] h_e  +  shared_down (silu(shared_gate x) * (shared_up x))
 *
 * Conventions (all entry points):
 *   - Every pointer except `dims`/`weights` structs is a DEVICE pointer owned by
 *     the caller (for example the storage of a torch tensor).  The library never
 *     allocates, frees or synchronises; it enqueues kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream) and returns.
 *   - Layouts are row-major with the reduction dimension contiguous:
 *       x [T][H]; router [E][H]; router_bias [E] float32 or NULL;
 *       gate, up [E][I][H]; down [E][H][I];
 *       shared_gate, shared_up [Is][H]; shared_down [H][Is].
 *     Element type of x and of every weight except router_bias: dims.dtype.
 *   - Supported set (anything else is refused with FLINT_UNSUPPORTED, never
 *     served by a fallback -- the serving-kit review, section "What isn't
 *     validated, and what the kit refuses to do", praises refusing unsupported
 *     configurations loudly rather than running a path that ignores the sigmoid
 *     routing):
 *       dtype F32 or BF16; 1 <= K <= 8; K <= E <= 256; H, I, Is multiples of 64
 *       (Is = 0 means no shared expert); H <= 8192; I, Is <= 4096;
 *       T * K < 2^31; every device pointer 16-byte aligned.
 *   - T = 0 is a valid no-op.  T < 0 or a NULL required pointer is
 *     FLINT_INVALID_ARG.  Argument errors are detected on the host before any
 *     launch and leave every output untouched.  FLINT_DEVICE_ERROR reports an
 *     immediate launch failure; faults during execution surface at the
 *     caller's next synchronisation.
 *   - Non-finite inputs give undefined results.
 *   - The calls keep no state between calls and may be issued from several
 *     threads on different streams, each with its own workspace.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t flint_status;
#define FLINT_OK 0
#define FLINT_INVALID_ARG 1
#define FLINT_UNSUPPORTED 2
#define FLINT_WORKSPACE_TOO_SMALL 3
#define FLINT_DEVICE_ERROR 4

typedef int32_t flint_dtype;
#define FLINT_F32 0
#define FLINT_BF16 1

/* Layer shape: hidden size H, routed experts E, experts per token K, routed
 * expert width I, shared expert width Is (0: none), element type. */
typedef struct {
    int32_t hidden;
    int32_t n_experts;
    int32_t top_k;
    int32_t inter;
    int32_t shared_inter;
    flint_dtype dtype;
} flint_moe_dims;

/* Device pointers to one layer's weights (layouts above).  The shared_* pointers
 * are ignored when dims.shared_inter == 0. */
typedef struct {
    const void *router;
    const float *router_bias;
    const void *gate;
    const void *up;
    const void *down;
    const void *shared_gate;
    const void *shared_up;
    const void *shared_down;
} flint_moe_weights;

/* Static, NUL-terminated description of a status code. */
const char *flint_status_string(flint_status status);

/* Bytes of device workspace that flint_moe_route, flint_moe_dispatch and
 * flint_moe_forward need for T tokens of this shape (an upper bound valid for
 * all three).  Returns 0 for an unsupported shape or T < 0.  The workspace is
 * scratch: its contents on entry do not matter and are not preserved. */
size_t flint_moe_workspace_bytes(const flint_moe_dims *dims, int32_t T);

/* Router (serving-kit review, "The architecture, from the config": sigmoid
 * scoring with normalised top-k).
 *   x [T][H] (dims.dtype), router [E][H] (dims.dtype), router_bias [E] float32
 *   or NULL (added to the logit before the sigmoid).
 *   topk_idx [T][K] int32 out: the K selected experts, distinct, ascending.
 *   topk_w   [T][K] float32 out: their weights s_e / sum of the selected s,
 *            in the same order; each row sums to 1 up to float32 rounding.
 *   ws / ws_bytes: device workspace of at least flint_moe_workspace_bytes. */
flint_status flint_moe_route(const flint_moe_dims *dims, int32_t T, const void *x,
                             const void *router, const float *router_bias,
                             int32_t *topk_idx, float *topk_w,
                             void *ws, size_t ws_bytes, void *stream);

/* Dispatch: the token -> expert assignment grouped by expert (release news page,
 * "What runs on each token": a router picks 6 of 256 expert sub-networks for
 * each token).
 *   topk_idx [T][K] int32 in: each row K distinct experts in [0, E).  Rows need
 *            not be sorted.  Out-of-range ids give undefined results.
 *   expert_counts  [E]   out: tokens routed to each expert.
 *   expert_offsets [E+1] out: exclusive prefix sum of the counts; [E] = T*K.
 *   sorted_token [T*K] out: expert-major, token-ascending within an expert.
 *   slot_of      [T*K] out: slot_of[t*K+k] is the position of the pair
 *                (t, topk_idx[t][k]) in sorted_token.
 *   The result is unique, so it is bit-exact and deterministic. */
flint_status flint_moe_dispatch(const flint_moe_dims *dims, int32_t T, const int32_t *topk_idx,
                                int32_t *expert_counts, int32_t *expert_offsets,
                                int32_t *sorted_token, int32_t *slot_of,
                                void *ws, size_t ws_bytes, void *stream);

/* The whole layer: router, dispatch, routed experts, shared expert, weighted
 * combine (both pages cited above).
 *   x [T][H] (dims.dtype); weights: device pointers, layouts above.
 *   out [T][H]: out_dtype FLINT_F32 (float32) or FLINT_BF16 (rounded to
 *               nearest even from the float32 sum).
 *   topk_idx_out [T][K], topk_w_out [T][K]: optional (NULL to skip); the routing
 *               used, as flint_moe_route defines it.
 *   The result is deterministic: the same inputs give the same bits.
 *   Precision: h is stored in dims.dtype, every sum is float32.  At batch
 *   sizes served by the LDS-tiled kernels (bf16, T > 384) each routed
 *   expert's output row, and the shared expert's, travels from the down
 *   product to the combine as fp16 scaled by a power of two per 64 columns
 *   (the scale keeps every finite value in range), which adds at most 2^-11
 *   of each term's magnitude: with routed weights summing to 1, at most 2^-11
 *   of the largest routed output of the token plus 2^-11 of the shared one. */
flint_status flint_moe_forward(const flint_moe_dims *dims, int32_t T, const void *x,
                               const flint_moe_weights *weights, void *out,
                               flint_dtype out_dtype, int32_t *topk_idx_out,
                               float *topk_w_out, void *ws, size_t ws_bytes, void *stream);

/* flint_moe_forward with stage timing: identical arguments, results and
 * kernels, plus `events`, an array of 10 hipEvent_t handles (created by the
 * caller, passed as void*): a start and a stop event for each of the five
 * stages, in the order router logits, top-k + dispatch, gate/up + SwiGLU, down
 * projection, combine ([2i] start, [2i+1] stop of stage i).  The kernels are
 * launched with hipExtLaunchKernel, so a stage's start is stamped when its
 * first kernel begins and its stop when its last kernel ends: the interval is
 * kernel execution time, as a kernel trace reports it.  The caller reads them
 * with hipEventElapsedTime.  NULL `events` makes it flint_moe_forward. */
flint_status flint_moe_forward_profiled(const flint_moe_dims *dims, int32_t T, const void *x,
                                        const flint_moe_weights *weights, void *out,
                                        flint_dtype out_dtype, int32_t *topk_idx_out,
                                        float *topk_w_out, void *ws, size_t ws_bytes, void *stream,
                                        void *const *events);

/* ---- Persistent fused decode ------------------------------------------------
 * The layer with top-k, dispatch, gate/up + SwiGLU and down in one persistent
 * launch between the router and the combine (release news page, "Built with
 * the Eureka Machine": a megakernel that fuses the decode forward pass; the
 * same idea for this layer).  The expert work runs as data flow: a unit's down
 * items wait only for that unit's gate/up items, through completion counters
 * in the workspace; no wait can deadlock (items are claimed in dependency
 * order), and every wait is bounded: one that gives up makes every output NaN.
 * Same arguments, workspace size and results as flint_moe_forward_profiled
 * (the same bits: the expert items are those flint_moe_forward runs at these
 * sizes); in `events` stage 1 covers the fused kernel and stages 2 and 3 are
 * empty.  Supported: dims.dtype BF16, 1 <= T <= 64, H and I multiples of 256,
 * Is a multiple of I with Is / I <= 8; anything else is FLINT_UNSUPPORTED.
 * flint_moe_forward does not use it: measured on one MI355X at T = 32 (the
 * Flint layer), the separate kernels take 178 us a layer and this path
 * 196-203 us (its top-k -> dispatch chain costs ~16 us before routed weights
 * stream, with only the shared expert to overlap it). */
flint_status flint_moe_forward_fused(const flint_moe_dims *dims, int32_t T, const void *x,
                                     const flint_moe_weights *weights, void *out, flint_dtype out_dtype,
                                     int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                                     void *stream, void *const *events);

/* ---- Expert weights in MXFP4 (block-scaled 4-bit) --------------------------
 * The pages' low-bit builds store weights in 4 bits ("Recursive launches
 * Flint: open-weight coding model with 39.8 billion parameters for local
 * execution", section "What Flint is, and how it is built": 4-bit weights take
 * roughly 23 GB) without a format for these
 * kernels; this library defines one: OCP Microscaling MXFP4 values in a tiled
 * byte order.  The values: FP4 E2M1 elements (sign, 2 exponent bits with bias
 * 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E8M0 scale
 * 2^(s - 127) per 32 consecutive elements of a row (255 is NaN); a weight is
 * element x scale.  The matrices are the bf16 layout's (gate/up [E][I][H],
 * down [E][H][I], shared [Is][H], [Is][H], [H][Is]), rows x cols each, with
 * rows a multiple of 16 and cols a multiple of 32.  Storage: a tile is 16
 * consecutive rows x one 32-element block;
 *   codes  [rows/16][cols/32][16][16] bytes: per tile, row r's 16 bytes (two
 *          elements per byte, the lower-indexed in the low nibble), rows in
 *          order, tiles along the columns, then down the rows;
 *   scales [rows/16][cols/32][16] bytes: per tile, row r's scale byte;
 * each expert's arrays follow the previous expert's ([E] outermost).  The byte
 * for element (row, col) is at codes[row/16][col/32][row%16][(col%32)/2], its
 * scale at scales[row/16][col/32][row%16].  (This order makes the 64 lanes of
 * one GPU load read one contiguous stretch.)  The router stays in dims.dtype
 * (BF16), activations are bf16, and everything after the weight decoding is as
 * in flint_moe_forward. */
typedef struct {
    const void *router;        /* [E][H] bf16 */
    const float *router_bias;  /* [E] or NULL */
    const uint8_t *gate_q, *gate_s;
    const uint8_t *up_q, *up_s;
    const uint8_t *down_q, *down_s;
    const uint8_t *shared_gate_q, *shared_gate_s;  /* NULL when shared_inter == 0 */
    const uint8_t *shared_up_q, *shared_up_s;
    const uint8_t *shared_down_q, *shared_down_s;
} flint_moe_weights_mx4;

/* flint_moe_forward with MXFP4 expert weights.  Same arguments and results as
 * flint_moe_forward otherwise; the workspace is flint_moe_workspace_bytes(dims,
 * T).  Supported: dims.dtype == FLINT_BF16, T <= 512, H a multiple of 1024, I
 * and Is multiples of 256 (Is may be 0), 16-byte aligned code arrays; anything
 * else is refused with FLINT_UNSUPPORTED.  The weight arrays are read only.  `events` as in
 * flint_moe_forward_profiled (10 handles) or NULL. */
flint_status flint_moe_forward_mx4(const flint_moe_dims *dims, int32_t T, const void *x,
                                   const flint_moe_weights_mx4 *weights, void *out,
                                   flint_dtype out_dtype, int32_t *topk_idx_out,
                                   float *topk_w_out, void *ws, size_t ws_bytes, void *stream,
                                   void *const *events);

/* ---- Dense MLP layer -------------------------------------------------------
 * The model's first two layers are dense MLPs (serving-kit review, "The
 * architecture, from the config": two dense layers, about 75M parameters
 * together; no width is given).  Same gated three-matrix form as an expert,
 * width `inter` (6144 fits the page's count at hidden 2048):
 *   out[t] = W_down (silu(W_gate x_t) * (W_up x_t)),
 * h rounded to dtype, float32 accumulation (the shared expert's kernels).
 *   dims.hidden H: multiple of 64, at most 8192; dims.inter I: multiple of 64,
 *   at most 16384; dims.dtype F32 or BF16.
 *   x [T][H] dtype; gate, up [I][H] dtype; down [H][I] dtype; out [T][H]
 *   out_dtype (F32, or BF16 rounded to nearest even) -- device pointers,
 *   16-byte aligned, caller-owned; weights and x are read only.
 *   ws: caller-owned device scratch of flint_dense_workspace_bytes(dims, T)
 *   bytes, 256-byte aligned.
 *   events: NULL or 6 hipEvent_t handles: start/stop of the gate/up, down and
 *   output stages (the output stage is empty, its events stamped at the down
 *   stage's end, when out_dtype is F32: the down stage writes out directly).
 * Errors as for flint_moe_forward; T = 0 is a no-op. */
typedef struct {
    int32_t hidden;    /* H */
    int32_t inter;     /* I */
    flint_dtype dtype; /* x, weights and h */
} flint_dense_dims;

size_t flint_dense_workspace_bytes(const flint_dense_dims *dims, int32_t T);

flint_status flint_dense_mlp(const flint_dense_dims *dims, int32_t T, const void *x, const void *gate,
                             const void *up, const void *down, void *out, flint_dtype out_dtype, void *ws,
                             size_t ws_bytes, void *stream, void *const *events);

/* ---- Allocation-free variant ----------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * flint_moe_forward with the same arguments except the workspace: the scratch
 * lives in a file-scope device array of FLINT_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (looked up with
 * hipGetSymbolAddress at the first call on each device; no call allocates).
 * Results are those of flint_moe_forward, bit for bit.
 *   - A shape whose flint_moe_workspace_bytes(dims, T) exceeds
 *     FLINT_STATIC_SCRATCH_BYTES is refused with FLINT_WORKSPACE_TOO_SMALL
 *     (48 MiB: the Flint layer up to T = 751 tokens), before any launch.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on a
 *     GPU (several streams or threads at once) race and give undefined results;
 *     serialise them, or use flint_moe_forward with a workspace per stream.
 *   - Other errors as for flint_moe_forward; FLINT_DEVICE_ERROR also when the
 *     array's address cannot be looked up. */
#define FLINT_STATIC_SCRATCH_BYTES ((size_t)48 << 20)

flint_status flint_moe_forward_static(const flint_moe_dims *dims, int32_t T, const void *x,
                                      const flint_moe_weights *weights, void *out, flint_dtype out_dtype,
                                      int32_t *topk_idx_out, float *topk_w_out, void *stream);

/* RMSNorm between stacked MoE layers (unit gain): out = bf16(in / sqrt(mean(in^2) + eps)),
 * the mean over each row of H values.  in [T][H] float32, out [T][H] bf16.
 * H must be a multiple of 64 and at most 8192.  This joins consecutive layers in
 * the stacked workload; the pages use RMSNorm on attention heads, not here. */
flint_status flint_rmsnorm(int32_t T, int32_t H, const float *in, void *out_bf16, float eps,
                           void *stream);

/* The layer followed by that RMSNorm, for a stack of layers: flint_moe_forward_profiled
 * (same arguments, workspace and results, and `out` as it writes it), and
 * norm_out_bf16 [T][H] bf16 receives flint_rmsnorm(T, H, y, norm_out_bf16, eps)
 * of the layer's float32 output y, bit for bit, whatever out_dtype is.  The
 * norm runs inside the layer's last kernel, its combine (a work-group per
 * token sums the row's squares in the order flint_rmsnorm does), so a stack
 * makes one launch fewer per layer.  norm_out_bf16: device pointer, 16-byte
 * aligned, caller-owned; it must not overlap out, and it may be x itself (x is
 * not read after the expert products).  H must be a multiple of 64 and at most
 * 8192, eps >= 0, else FLINT_UNSUPPORTED / FLINT_INVALID_ARG; a null
 * norm_out_bf16 with T > 0 is FLINT_INVALID_ARG.  In `events` the combine
 * stage covers the norm too. */
flint_status flint_moe_forward_rmsnorm(const flint_moe_dims *dims, int32_t T, const void *x,
                                       const flint_moe_weights *weights, void *out, flint_dtype out_dtype,
                                       void *norm_out_bf16, float eps, int32_t *topk_idx_out,
                                       float *topk_w_out, void *ws, size_t ws_bytes, void *stream,
                                       void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MOE_H */
