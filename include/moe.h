/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts layer library.
 *
 * One MoE layer's forward pass on one GPU: route (top-k + renormalised
 * softmax), permute (group the (token, expert) pairs by expert and copy the
 * token rows into expert-contiguous order), grouped feed-forward (each
 * expert's SwiGLU MLP over its own rows) and combine (routing-weighted sum
 * back to token order).  The operations follow the Hugging Face Transformers
 * docs, "Expert parallelism" (sections "Adding an implementation" and "Token
 * dispatch") and "Tensor parallelism for inference" (section "Packed
 * strategies"); each entry point names its passage.
 *
 * Conventions for every entry point:
 *  - Array arguments are DEVICE pointers (for example a torch tensor's
 *    data_ptr()).  The caller owns every buffer; the library allocates and
 *    frees nothing and never synchronises with the host.
 *  - `stream` is a hipStream_t (NULL = the default stream).  On success the
 *    work is enqueued on it and MOE_OK is returned at once.  Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Scalars and pointers are validated on the host FIRST: on any error a
 *    status is returned and nothing is enqueued.
 *  - Rows are row-major and dense (stride = row length).  Element type
 *    `moe_dtype`: MOE_F32 (IEEE float) or MOE_BF16 (bfloat16).
 *  - Limits: 1 <= E <= 256; k >= 1, and k <= E where the call routes; d and
 *    I multiples of 64; T*k*max(d, I) and every activation array below 2^31
 *    elements; one expert's weights (4*d*I bytes for gate/up) below 2 GiB.
 *    T == 0 (or no rows) is valid: nothing is enqueued.
 *  - Device-side values that the host cannot see (expert ids, offsets, row
 *    indices) are clamped to the buffers they index: an expert id outside
 *    [0, E) drops its pair, a row index outside the capacity is skipped.
 *    Garbage in such arrays gives garbage results, never an out-of-bounds
 *    access.
 *  - Calls are reentrant; concurrent calls need separate workspaces.
 *  - No call reads device memory from the host, so a sequence of calls can
 *    be captured into a HIP graph.
 */
#ifndef TRE_MOE_H
#define TRE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,         /* invalid argument: bad size, NULL pointer, k > E ... */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside the library's limits (E > 256, d % 64 ...) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace_size() */
  MOE_ERR_HIP = 4          /* the HIP runtime refused a launch */
} moe_status;

/* Static, never NULL. */
const char* moe_status_string(moe_status s);

/* ---- route ----------------------------------------------------------------
 * "Expert parallelism", "Adding an implementation": the expert path receives
 * each token's selected expert ids (top_k_index) and routing weights
 * (top_k_weights).  Selection rule (softmax top-k): the k largest logits,
 * equal logits ordered by the lower expert index (-0.0 equals +0.0); slot 0
 * holds the largest.  Weight of slot j: exp(l_j - l_0) / sum over the k
 * selected of exp(l_i - l_0), i.e. the softmax probability renormalised over
 * the selection.
 *   logits    [T, E] float32, finite
 *   topk_idx  [T, k] int32  (output)
 *   topk_w    [T, k] float32 (output)                                        */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                          int32_t* topk_idx, float* topk_w, void* stream);

/* Router projection fused with the routing above.  "Expert parallelism",
 * introduction: a router sends each token to its experts; the router module
 * is the model's gate linear layer (mlp.gate or mlp.router, "Token
 * dispatch"), read here as bias-free:
 *   logits[t, e] = sum_c x[t, c] * w_router[e, c]      (float32 accumulation)
 * then topk_idx / topk_w exactly as moe_route_topk computes them from those
 * logits.
 *   x         [T, d] dt        (d a multiple of 64)
 *   w_router  [E, d] dt        (the linear layer's weight)
 *   logits    [T, E] float32   (output; NULL: not written)
 *   topk_idx  [T, k] int32, topk_w [T, k] float32 (outputs)
 * Errors: MOE_ERR_ARG for k > E, bad dtype or NULL outputs; MOE_ERR_UNSUPPORTED
 * for E > 256, d not a multiple of 64 or d >= 2^22; T == 0 returns MOE_OK. */
moe_status moe_route_project(const void* x, const void* w_router, moe_dtype dt, int32_t T, int32_t d,
                             int32_t E, int32_t k, float* logits, int32_t* topk_idx, float* topk_w,
                             void* stream);

/* ---- permute --------------------------------------------------------------
 * "Expert parallelism", "Token dispatch": every (token, expert) pair goes to
 * the expert's owner, which runs the expert on the rows it receives.  Here:
 * pair p = t*k + j with expert pair_expert[p] (-1, or any id outside [0, E):
 * not handled here, dropped).  Pairs are grouped by expert, stable in p:
 * expert e owns rows [expert_offsets[e], expert_offsets[e+1]).
 *   x               [T, d] dt
 *   pair_expert     [T*k] int32
 *   x_perm          [T*k, d] dt   (output; rows >= expert_offsets[E] untouched;
 *                   NULL: only the index arrays are built, no rows move, and
 *                   x may be NULL too)
 *   row_token       [T*k] int32   (output; row r holds token row_token[r])
 *   pair_row        [T*k] int32   (output; row of pair p, -1 when dropped)
 *   expert_offsets  [E+1] int32   (output)
 *   workspace       >= moe_permute_workspace_size(T, k, E) bytes, 256-aligned */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);
moe_status moe_permute(const void* x, moe_dtype dt, int32_t T, int32_t d, int32_t k,
                       const int32_t* pair_expert, int32_t E, void* x_perm, int32_t* row_token,
                       int32_t* pair_row, int32_t* expert_offsets, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---- grouped feed-forward ---------------------------------------------------
 * "Tensor parallelism for inference", "Packed strategies": gate and up
 * projections packed as one [E, d, 2I] weight applied as x @ W and split with
 * the gate half first; down projection [E, I, d] (down_proj, "Expert
 * parallelism", "Overriding plans"), same orientation.  For each expert e and
 * each row r in [expert_offsets[e], expert_offsets[e+1]):
 *   h      = silu(x_perm[r] @ Wgu[e][:, :I]) * (x_perm[r] @ Wgu[e][:, I:])
 *   y[r]   = h @ Wd[e]
 * float32 accumulation; h is rounded to dt before the down projection.
 * Offsets are read on the device only.
 *   x_perm      [max_rows, d] dt
 *   w_gate_up   [E, d, 2I] dt;  w_down [E, I, d] dt
 *   y_perm      [max_rows, d] dt (output; rows >= expert_offsets[E] untouched)
 *   workspace   >= moe_grouped_ffn_workspace_size(max_rows, E, d, I, dt) bytes */
size_t moe_grouped_ffn_workspace_size(int32_t max_rows, int32_t E, int32_t d, int32_t I, moe_dtype dt);
moe_status moe_grouped_ffn(const void* x_perm, const int32_t* expert_offsets, int32_t max_rows,
                           int32_t E, int32_t d, int32_t I, const void* w_gate_up,
                           const void* w_down, moe_dtype dt, void* y_perm, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The two halves of moe_grouped_ffn, for callers that schedule or time them
 * separately.  Same operands, layouts and row ranges as moe_grouped_ffn:
 *   moe_gate_up_swiglu:  h[r] = silu(a_r @ Wgu[e][:, :I]) * (a_r @ Wgu[e][:, I:])
 *                        h [max_rows, I] dt (output)
 *     row_token == NULL: a_r = x[r], x is the expert-ordered x_perm [max_rows, d];
 *     row_token != NULL: a_r = x[row_token[r]], x is the token batch [x_rows, d]
 *       (the row move of moe_permute done inside the projection's loads;
 *       bf16 only, and x_rows * d below 2^30; row_token as moe_permute
 *       writes it).
 *   moe_down_proj:       y_perm[r] = h[r] @ Wd[e]
 * Neither needs a workspace.  Without one, the down projection computes every
 * tile whole; moe_grouped_ffn and moe_forward use their workspace to cut the
 * k-range of a last, partial round of 256-row tiles into pieces whose float32
 * partial sums are added in a fixed order -- deterministic, but those rows
 * can differ from moe_down_proj's in the last bit.                          */
moe_status moe_gate_up_swiglu(const void* x, const int32_t* expert_offsets, int32_t max_rows,
                              int32_t E, int32_t d, int32_t I, const void* w_gate_up, moe_dtype dt,
                              const int32_t* row_token, int32_t x_rows, void* h, void* stream);
moe_status moe_down_proj(const void* h, const int32_t* expert_offsets, int32_t max_rows, int32_t E,
                         int32_t d, int32_t I, const void* w_down, moe_dtype dt, void* y_perm,
                         void* stream);

/* ---- combine ----------------------------------------------------------------
 * "Expert parallelism", "Token dispatch" / "Adding an implementation": the
 * expert outputs are combined with the routing weights into the weighted
 * expert output of each token:
 *   out[t] = sum over j < k with 0 <= pair_row[t*k+j] < max_rows of
 *            pair_w[t*k+j] * y_perm[pair_row[t*k+j]]
 * float32 accumulation in ascending j, rounded to dt.
 *   y_perm [max_rows, d] dt; pair_row, pair_w [T*k]; out [T, d] dt (output)  */
moe_status moe_combine(const void* y_perm, int32_t max_rows, const int32_t* pair_row,
                       const float* pair_w, int32_t T, int32_t k, int32_t d, moe_dtype dt,
                       void* out, void* stream);

/* ---- the whole layer ----------------------------------------------------------
 * "Expert parallelism", "Adding an implementation": called with the batch
 * this device holds and returns the weighted expert output of each token.
 * logits != NULL: route first (topk_idx / topk_w are outputs).
 * logits == NULL: topk_idx / topk_w are INPUTS (already-routed pairs, e.g.
 *   the rows one expert-parallel rank received, ids local to this device).
 * expert_offsets [E+1], row_token [T*k], pair_row [T*k] are optional outputs
 * (NULL: kept in the workspace).
 *   x [T, d] dt; out [T, d] dt (output)
 *   workspace >= moe_forward_workspace_size(T, d, E, k, I, dt) bytes          */
size_t moe_forward_workspace_size(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, moe_dtype dt);
moe_status moe_forward(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                       int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                       int32_t* pair_row, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- column-tiled expert weights (inference) ---------------------------------
 * The expert weights in the layout the grouped products stream them in: each
 * expert's weight is stored as one block per 256-column tile of its product,
 * so that a tile's k-stage is one contiguous run of memory (the pages' layout
 * puts it in K separate pieces of a row).  A permutation of the elements: the
 * tiled arrays have the sizes of the originals.  For expert e:
 *   gate/up, tile c = 0 .. ceil(I/128)-1, n0 = 128 c, w = min(128, I - n0):
 *     block [d][2w] at element e*d*2I + d*2*n0, row r =
 *     Wgu[e][r][n0 .. n0+w) followed by Wgu[e][r][I+n0 .. I+n0+w);
 *   down, tile c = 0 .. ceil(d/256)-1, n0 = 256 c, w = min(256, d - n0):
 *     block [I][w] at element e*I*d + I*n0, row r = Wd[e][r][n0 .. n0+w).
 * moe_tile_weights writes them (once, e.g. when a model is loaded: a read and
 * a write of every weight); moe_forward_tiled is moe_forward on them, with
 * results bit-identical to moe_forward on the original weights.  bf16 only.
 *   w_gate_up [E, d, 2I], w_down [E, I, d] bf16 (inputs, unchanged)
 *   w_gate_up_tiled, w_down_tiled: outputs of the same sizes
 * Errors: as moe_forward's shape checks; MOE_ERR_UNSUPPORTED for MOE_F32;
 * MOE_ERR_ARG for NULL pointers.  The forward's arguments and workspace are
 * moe_forward's.                                                            */
moe_status moe_tile_weights(const void* w_gate_up, const void* w_down, int32_t E, int32_t d, int32_t I, moe_dtype dt,
                            void* w_gate_up_tiled, void* w_down_tiled, void* stream);
moe_status moe_forward_tiled(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                             int32_t I, const void* w_gate_up_tiled, const void* w_down_tiled, moe_dtype dt,
                             int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                             int32_t* pair_row, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* The layer as moe_forward computes it (same kernels, same results bit for
 * bit), for callers that cannot allocate memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  There is
 * no workspace argument: the scratch lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * until the process ends; its device address is looked up on the first call
 * on each device (with that device current).  The call allocates nothing.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (concurrent streams, or host
 * threads) race and give wrong results.  Serialise them.
 *   arguments as moe_forward, without workspace / workspace_bytes
 * Errors: as moe_forward; MOE_ERR_WORKSPACE when the layer needs more
 * scratch than MOE_NOALLOC_SCRATCH_BYTES (moe_forward_workspace_size()
 * tells how much it needs), with nothing enqueued; MOE_ERR_HIP when the
 * array's address cannot be looked up.                                      */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                               int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                               int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                               int32_t* pair_row, void* out, void* stream);

/* ---- the layer's backward pass ----------------------------------------------
 * "Expert parallelism", "Adding an implementation": gradients, the routing
 * weights' included, must reach the rank that holds the tokens; "Combining
 * with FSDP2": an expert's weight gradient sums over every row it served (an
 * expert without rows gets a zero gradient).  Gradients of <dout, out> with
 * out = moe_forward(x, ...) on the same arguments, by the chain rule:
 *   pair p = (t, j) with expert e, weight w_p, x row x_t:
 *     g = x_t Wg[e], u = x_t Wu[e], s = sigmoid(g), h = g s u, y_p = h Wd[e]
 *     dtopk_w[p] = <dout_t, y_p>;   dy_p = w_p dout_t
 *     dW_down[e] = sum_p h^T dy_p;  dh = dy_p Wd[e]^T
 *     dg = dh u s (1 + g (1 - s));  du = dh g s
 *     dW_gate_up[e] = sum_p x_t^T [dg | du];  dx_t = sum_j [dg | du] Wgu[e]^T
 *     with logits: dlogits[t, e_j] = w_j (dtopk_w_j - sum_i w_i dtopk_w_i),
 *     zero for experts not selected (the selection passes no gradient).
 * recompute = 1: the forward is recomputed inside (routing when logits are
 * given, the grouping, both projections).  recompute = 0: the workspace
 * holds what moe_forward_train left there for these same arguments (and
 * topk_idx / topk_w are the arrays that call filled or read), untouched since;
 * only the gradients are computed.  dt = MOE_BF16: bf16 operands and stored
 * intermediates (the pre-activations g, u, h, y and the row gradients),
 * float32 accumulation, gradients rounded to bf16; dt = MOE_F32: float32
 * throughout (dtopk_w and dlogits are float32 for both).
 *   x, dout [T, d] dt; w_gate_up [E, d, 2I], w_down [E, I, d] dt
 *   logits [T, E] float32 or NULL, and topk_idx / topk_w [T, k], as for
 *     moe_forward (outputs with logits, inputs without; -1 ids are skipped)
 *   dx [T, d], dw_gate_up [E, d, 2I], dw_down [E, I, d] dt (outputs,
 *     overwritten); dtopk_w [T, k] float32 (output, 0 for skipped pairs);
 *     dlogits [T, E] float32 (output; NULL to skip; only with logits)
 *   workspace >= moe_backward_workspace_size(T, d, E, k, I, dt) bytes
 *     (the size depends on dt; 0 for an unknown dt)
 * Errors: as moe_forward; MOE_ERR_ARG for dlogits without logits or
 * recompute not 0 or 1.  T == 0 zeroes the weight gradients only.          */
size_t moe_backward_workspace_size(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, moe_dtype dt);
moe_status moe_backward(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                        int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                        int32_t* topk_idx, float* topk_w, const void* dout, void* dx, void* dw_gate_up,
                        void* dw_down, float* dtopk_w, float* dlogits, int32_t recompute, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The forward of a training step: out exactly as moe_forward computes it
 * (same kernels, same order of every sum), and the intermediates the
 * backward needs -- the routing, the grouping, the grouped rows of x, the
 * pre-activations g | u, h and the expert outputs y -- kept in the workspace
 * for moe_backward(..., recompute = 0, same workspace).  bf16 or float32.
 *   arguments as moe_forward (the expert_offsets / row_token / pair_row
 *   outputs live in the workspace);
 *   workspace >= moe_backward_workspace_size(T, d, E, k, I, dt) bytes        */
moe_status moe_forward_train(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                             int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                             int32_t* topk_idx, float* topk_w, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TRE_MOE_H */
