/*
 * ttt.h -- C ABI of the chunk-wise test-time-training fast-weight layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the In-Place TTT form of a gated MLP (source: the review of
 * "In-Place Test-Time Training", Method §1-§3, eq. (1)-(6)): the MLP's
 * down-projection W_down is a fast weight.  The sequence is cut into chunks
 * of C tokens; chunk c is first applied with the state left by chunks
 * 0..c-1, O_c = Z_c W_c^T (eq. (3)), then one gradient step is folded into
 * the state (eq. (4)).  Two objectives are provided:
 *   dot -- negative Frobenius inner product with the target V^ (eq. (6)):
 *          W_{c+1} = W_c + eta V^_c^T Z_c.  The deltas do not depend on W, so
 *          all chunks are computed in parallel and combined by an exclusive
 *          prefix sum (Method §3, three-step form).
 *   mse -- squared error (1/(2C))||Z_c W^T - V^_c||^2 at the pre-update state:
 *          W_{c+1} = W_c - (eta/C)(Z_c W_c^T - V^_c)^T Z_c, an in-order scan.
 * with Z = silu(H W_gate^T) * (H W_up^T) (eq. (2)) and the target
 * V^ = CausalDepthwiseConv1D(X0) W_target (eq. (5), causal padding of §3).
 * A LaCT SwiGLU fast weight (review of "Test-Time Training Done Right",
 * LaCT Model Architecture §1, eq. (3)-(4)) is the second layer family.
 *
 * Conventions common to every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller (e.g.
 *     torch.Tensor.data_ptr()), row-major and contiguous, 16-byte aligned.
 *     The library allocates no device memory and creates no streams or
 *     events; scratch comes from the caller's workspace, whose size the
 *     matching *_workspace_bytes call returns.
 *   - Inputs are read only.  Outputs and workspace must not alias inputs or
 *     each other.  W_down0 is never written: "in place" names the reuse of
 *     the MLP's own weight as the fast weight, not memory aliasing.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the default stream).  The call returns once the work is enqueued.  It
 *     enqueues kernels only (no copy or memset; ttt_lact_swiglu_ex given a
 *     side stream adds an event fork and join), so a call can be captured
 *     into a HIP graph and replayed with the same buffers.
 *   - Every argument is validated before any device work is enqueued; on an
 *     error status nothing has been enqueued and outputs are untouched.  A
 *     launch failure reported by the runtime returns TTT_ERR_DEVICE, in which
 *     case outputs are undefined.
 *   - dtype selects the element type of every activation, weight, Z, V^ and
 *     O buffer (TTT_F32: fp32 end to end; TTT_BF16: bf16 storage, fp32
 *     accumulation).  Fast-weight states W_final and dW are always fp32.
 *   - Each batch row is an independent document whose state starts at
 *     W_down0 (document-boundary reset, Method §3).
 *   - Supported sizes: d_model, d_ff and chunk multiples of 8, conv_k in
 *     1..8, seq_len <= 2^22 (else TTT_ERR_UNSUPPORTED); seq_len a multiple
 *     of chunk (else TTT_ERR_SHAPE).  seq_len == 0 or batch == 0 is valid: no output rows,
 *     W_final rows (if any) equal W_down0.
 *   - The library keeps no global state (except the static scratch of
 *     ttt_chunk_apply_update_noalloc, below); calls with distinct outputs and
 *     workspaces may run concurrently on different streams.
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TTT_OK = 0,
  TTT_ERR_ARG = 1,          /* null pointer, misaligned pointer, unknown mode/order, non-finite eta */
  TTT_ERR_SHAPE = 2,        /* negative or zero size, seq_len % chunk != 0 */
  TTT_ERR_DTYPE = 3,        /* dtype not TTT_F32 / TTT_BF16 */
  TTT_ERR_WORKSPACE = 4,    /* workspace smaller than the query returned, or NULL when needed */
  TTT_ERR_DEVICE = 5,       /* the HIP runtime rejected a launch */
  TTT_ERR_UNSUPPORTED = 6,  /* valid but outside the sizes this build handles */
  TTT_ERR_SCRATCH_LIMIT = 7 /* ttt_chunk_apply_update_noalloc: the call needs more scratch than
                               TTT_NOALLOC_SCRATCH_BYTES */
};

enum { TTT_F32 = 0, TTT_BF16 = 1 };

enum {
  TTT_MODE_DOT = 0,         /* dot objective; delta + prefix sum fused in one MFMA pass when chunk % 64 == 0 */
  TTT_MODE_MSE = 1,         /* mse objective, in-order chunk scan */
  TTT_MODE_DOT_SCAN = 2     /* dot objective; every chunk delta materialised, then a device-wide prefix scan */
};

enum { TTT_UPDATE_THEN_APPLY = 0, TTT_APPLY_THEN_UPDATE = 1 };

/* Sizes of one In-Place layer call.  n = seq_len, d = d_model, f = d_ff,
 * C = chunk, K = conv_k; k = n / C chunks. */
typedef struct {
  int64_t batch, seq_len, d_model, d_ff, chunk, conv_k;
} ttt_inplace_shape;

/* Sizes of one LaCT layer call: m = hidden (fast MLP width), dh = head_dim. */
typedef struct {
  int64_t batch, heads, seq_len, head_dim, hidden, chunk;
} ttt_lact_shape;

/* Human-readable name of a status code (static storage, never NULL). */
const char* ttt_status_string(int status);

/* ------------------------------------------------------------------ In-Place TTT layer */

/* Workspace bytes needed by ttt_chunk_apply_update (with_producers = 1) or
 * ttt_core_apply_update (with_producers = 0) for this shape, dtype and mode.
 * Writes *bytes; returns a status (same validation as the call itself). */
int ttt_inplace_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int mode, int with_producers,
                                size_t* bytes);

/* The whole layer (In-Place TTT review, Method §1-§3):
 *   Z   = silu(H W_gate^T) * (H W_up^T)                      (eq. (2))
 *   V^  = CausalDepthwiseConv1D_K(X0) W_target               (eq. (5))
 *   for each chunk c: O_c = Z_c W_c^T, then the mode's update (eq. (3), (4)/(6)).
 *
 *   H, X0     [B, n, d]    dtype   hidden states / token embeddings
 *   W_gate    [f, d]       dtype   slow weight
 *   W_up      [f, d]       dtype   slow weight
 *   W_down0   [d, f]       dtype   pretrained down projection = initial fast weight
 *   W_target  [d, d]       dtype   indexed [d_in][d_out]: V^ = Y W_target
 *   conv_w    [d, K]       dtype   depthwise taps, no bias; tap K-1 multiplies the
 *                                  current token, tap j the token K-1-j steps back,
 *                                  tokens before the sequence start are zero
 *   O         [B, n, d]    dtype   output (written)
 *   W_final   [B, d, f]    fp32    state after the last chunk (written)
 *   workspace                      >= ttt_inplace_workspace_bytes(..., 1, ...) bytes
 */
int ttt_chunk_apply_update(const ttt_inplace_shape* shape, int dtype, int mode, float eta,
                           const void* H, const void* X0, const void* W_gate, const void* W_up,
                           const void* W_down0, const void* W_target, const void* conv_w,
                           void* O, float* W_final, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Size of the static device scratch of ttt_chunk_apply_update_noalloc. */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ttt_chunk_apply_update for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, arguments, outputs and errors, with no workspace
 * argument.  The scratch the layer needs (the ttt_inplace_workspace_bytes(...,
 * with_producers = 1, ...) of this shape, dtype and mode) comes from a static
 * device array of TTT_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one
 * per device: the device of `stream` holds its copy from its first call until
 * the process ends, and that first call looks up the array's device address
 * (with the stream's device made current for the lookup).  The call itself
 * allocates nothing.
 *   - A shape whose scratch exceeds TTT_NOALLOC_SCRATCH_BYTES returns
 *     TTT_ERR_SCRATCH_LIMIT before any device work (e.g. the fp32 layer of 2048
 *     tokens, d_model 256, d_ff 512, chunk 256 needs 16.75 MiB; the bf16 layer
 *     of 4096 x 2 tokens, d_model 512, d_ff 1024, chunk 512, 72.5 MiB, does not
 *     fit).
 *   - Every call on a device shares that device's array and leaves its last
 *     contents there; nothing in it needs to start at zero.  Calls that may
 *     overlap on one device (several streams, several host threads) race on
 *     it: the caller orders them, e.g. on one stream.
 *   - The first call on a device must not be under graph capture if the
 *     lookup would be refused there; later calls enqueue kernels only. */
int ttt_chunk_apply_update_noalloc(const ttt_inplace_shape* shape, int dtype, int mode, float eta,
                                   const void* H, const void* X0, const void* W_gate, const void* W_up,
                                   const void* W_down0, const void* W_target, const void* conv_w,
                                   void* O, float* W_final, void* stream);

/* Options of ttt_chunk_apply_update_ex; a NULL options pointer, or all fields
 * zero, gives ttt_chunk_apply_update's results. */
typedef struct {
  /* Rows that pack several documents (In-Place TTT review, Method §3: the
   * fast weight is reset to the pretrained state at document boundaries, so
   * that no context leaks between independent sequences).  [B, k] uint8,
   * DEVICE, k = seq_len / chunk: a nonzero entry marks chunk c as the first
   * chunk of a document (entry 0 of a row is implied), so documents start at
   * chunk boundaries.  At a document start the state is W_down0 again (chunk
   * c is applied with W_down0 and updates it) and the convolution restarts:
   * rows before the chunk's first token read as zero.  W_final is the state
   * after the row's last chunk, i.e. the last document's.  Read on the
   * device; any byte value is valid.  NULL: one document per row.  (Entry 0
   * matters only for resumed rows, below.) */
  const unsigned char* doc_starts;
  /* 0: the causal convolution of ttt_chunk_apply_update.  1: the forward-
   * looking in-chunk reading of the review's next-token example (Method §2):
   * tap j multiplies the token j steps ahead and tokens past the end of the
   * token's chunk are zero, so a chunk's targets come from its own tokens and
   * its update stays causal at chunk level; with W_target = I and
   * conv_w[:, 1] = 1 the target of a token is the next token (zero at a
   * chunk's last token).  Other values: TTT_ERR_ARG. */
  int conv_forward;
  /* Resuming rows that continue a sequence from an earlier call (e.g. a long
   * document processed in pieces): W_init [B, d, f] fp32 (DEVICE, 16-byte
   * aligned) is each row's state before chunk 0 -- the earlier call's
   * W_final -- and x0_halo [B, K-1, d] dtype (DEVICE, 16-byte aligned) holds
   * the K-1 rows of X0 before the first token, which the causal convolution
   * reads instead of zeros.  Either may be NULL (W_down0, resp. zeros).  With
   * either given, chunk 0 starts a new document only where doc_starts flags
   * it (then W_down0 and zeros, as at any document start).  Two calls on the
   * halves of a sequence, the second resumed this way, give the single call's
   * results up to rounding order. */
  const float* W_init;
  const void* x0_halo;
  /* Keeping the states for a backward pass: W_states [B, k, d, f] dtype
   * (DEVICE, 16-byte aligned) receives the state each chunk was applied
   * with, W_states[b, c] = W_c.  Dot objective: in place of the workspace copy
   * the call keeps anyway, so keeping them costs nothing; ttt_core_backward
   * takes them.  MSE objective: one copy per chunk (2 B d f dtype bytes of
   * traffic); ttt_core_backward_mse takes them.  Either backward then skips
   * recomputing the states.  NULL: not kept. */
  void* W_states;
  /* Strided updates (the block-wise mask of the LaCT review's section on the
   * order of the apply and update operations, read onto this layer):
   * [B, k] uint8, DEVICE; a zero entry means chunk c of that row is applied
   * but does not update the state (its update adds exact zeros: the dot
   * objective's target, or the MSE residual, is multiplied by zero), so the
   * next chunk sees the same state.  A document start still resets to
   * W_down0.  NULL: every chunk updates. */
  const unsigned char* update_mask;
  /* 0: apply then update (Method §3: chunk c is applied with the state before
   * its own step).  1: update then apply (the other order of the LaCT
   * review's section on the order of the two operations): chunk c's step is
   * taken first and the chunk is applied with the state after it, so its
   * outputs see its own targets -- the layer is then not causal inside a
   * chunk, for non-causal uses.  W_final is the same in both orders.  Dot
   * objective: the scans write the state after each chunk's step instead of
   * the one before it (TTT_MODE_DOT runs its fused scan in one or two
   * sequence segments then, never four), with the mode's usual workspace.
   * The MSE objective applies each chunk a second time, after its step (one
   * more apply's work).  Not with W_states (TTT_ERR_UNSUPPORTED): the
   * backward passes take the apply-then-update order.  Other values:
   * TTT_ERR_ARG. */
  int update_first;
} ttt_layer_options;

/* The layer of ttt_chunk_apply_update with options (above); same arguments,
 * workspace and errors otherwise. */
int ttt_chunk_apply_update_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta,
                              const void* H, const void* X0, const void* W_gate, const void* W_up,
                              const void* W_down0, const void* W_target, const void* conv_w,
                              const ttt_layer_options* options, void* O, float* W_final,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The chunk loop alone, given Z [B, n, f] and Vhat [B, n, d] (dtype) instead
 * of the producers' inputs.  Same outputs and rules as above; workspace from
 * ttt_inplace_workspace_bytes(..., with_producers = 0, ...). */
int ttt_core_apply_update(const ttt_inplace_shape* shape, int dtype, int mode, float eta,
                          const void* Z, const void* Vhat, const void* W_down0,
                          void* O, float* W_final, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The chunk loop with options: doc_starts, W_init, W_states and update_mask
 * as for the layer (conv_forward and x0_halo concern the target producer and
 * are not read). */
int ttt_core_apply_update_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta,
                             const void* Z, const void* Vhat, const void* W_down0,
                             const ttt_layer_options* options, void* O, float* W_final,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- backward passes ---- */

/* Options of the backward entry points with an _ex suffix; a NULL options
 * pointer, or all fields zero, gives the plain call's results. */
typedef struct {
  /* The per-chunk states the forward call kept (ttt_layer_options.W_states,
   * [B, k, d, f] dtype, DEVICE, 16-byte aligned), or NULL: recomputed. */
  const void* W_states;
  /* Packed documents as in ttt_layer_options.doc_starts (each document is
   * differentiated as the independent sequence the forward call makes of it),
   * or NULL. */
  const unsigned char* doc_starts;
  /* The update mask of the forward call (ttt_layer_options.update_mask, [B, k]
   * uint8, DEVICE), or NULL: every chunk updated.  A masked chunk is applied
   * but adds nothing to the state, so its target gets no gradient (dVhat rows
   * of the chunk are zero) and, for the MSE objective, its residual none. */
  const unsigned char* update_mask;
  /* The whole layer only: 1 when the forward call took the forward-looking
   * in-chunk convolution (ttt_layer_options.conv_forward), 0 for the causal
   * one; other values TTT_ERR_ARG. */
  int conv_forward;
  /* Resumed rows, as the forward call took them (ttt_layer_options.W_init and
   * x0_halo): a row continues its sequence -- its first document starts from
   * W_init[b] and its causal convolution reads x0_halo[b] before the first
   * token -- unless doc_starts flags its chunk 0.  W_init [B, d, f] fp32
   * (DEVICE, 16-byte aligned) or NULL; then dW_init [B, d, f] fp32 (DEVICE,
   * 16-byte aligned) is required and receives each row's initial-state
   * gradient (zero for rows flagged at chunk 0), and dW_down0 sums only the
   * documents that start from W_down0.  With packed documents the dot
   * objective takes a continuing row's first document off the sum of all of
   * them, in fp32, so dW_down0 carries rounding of order 1e-7 of that
   * document's gradient.  x0_halo [B, K-1, d] dtype (DEVICE, 16-byte aligned,
   * whole layer only; the chunk loop's backward reads neither halo field) or
   * NULL; then dx0_halo [B, K-1, d] dtype is required and receives the halo
   * rows' gradient (zero for rows flagged at chunk 0, and everywhere with the
   * forward-looking convolution, which never reads it).  A gradient pointer
   * without its input, or a missing one: TTT_ERR_ARG. */
  const float* W_init;
  const void* x0_halo;
  float* dW_init;
  void* dx0_halo;
} ttt_backward_options;

/* ---- backward of the dot chunk loop ---- */

/* Workspace bytes for ttt_core_backward, with the states given (saved_states
 * = 1) or recomputed (0): about B (2 k d f + n d) dtype elements plus B d f
 * fp32 (the recomputed states, the suffix states, eta V^), one k d f less
 * with saved states; with a chunk length the fused scan does not take (see
 * ttt_chunk_update_scan), token-contiguous copies and fp32 deltas besides. */
int ttt_core_backward_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                      size_t* bytes);

/* Gradients through the dot-objective chunk loop (ttt_core_apply_update with
 * TTT_MODE_DOT), for a loss that depends on O alone, given its gradient
 * dO = dLoss/dO [B, n, d] (dtype).  By the chain rule through
 * O_c = Z_c W_c^T (eq. (3)) and W_c = W_down0 + eta sum_{j<c} V^_j^T Z_j
 * (eq. (6), prefix form of Method §3), with the exclusive suffix
 * S_c = sum_{j>c} dO_j^T Z_j of each row:
 *   dZ       [B, n, f] dtype:  dZ_c = dO_c W_c + eta V^_c S_c
 *   dVhat    [B, n, d] dtype:  dV^_c = eta Z_c S_c^T
 *   dW_down0 [d, f]    fp32:   sum over rows and chunks of dO_c^T Z_c
 *                              (W_down0 is shared by the rows, so their
 *                              gradients add).
 * The states W_c are W_states [B, k, d, f] dtype when given (kept by the
 * forward call through ttt_layer_options.W_states; DEVICE, 16-byte aligned),
 * else recomputed by the chunk scan (NULL).  The suffixes come from the same
 * scan run over the chunks in reverse order on (Z, dO) from a zero state, so
 * each S_c is a sum of its own terms, never a difference of prefix sums.
 * With bf16 the states W_c and S_c are held in bf16 (fp32 accumulation), as in
 * the forward call.  doc_starts [B, k] (DEVICE, as ttt_layer_options.
 * doc_starts; NULL: one document per row) packs documents: the states
 * restart from W_down0 at each start, each suffix S_c runs to the end of c's
 * document (the reversed scan restarts from zero where the forward order's
 * documents end), and dW_down0 receives every document's sum, formed by one
 * more contraction over all chunks (2 d f flop per token).  Update masks:
 * ttt_core_backward_ex (which also takes resumed rows).  Inputs as in
 * ttt_core_apply_update; conv_k is not used.  seq_len == 0 or batch == 0
 * gives dW_down0 = 0 and touches nothing else.  Errors as for every entry
 * point (a too small workspace: TTT_ERR_WORKSPACE). */
int ttt_core_backward(const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                      const void* W_down0, const void* dO, const void* W_states, const unsigned char* doc_starts,
                      void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes for ttt_core_backward_mse, with the states given
 * (saved_states = 1) or recomputed (0): about B (k d f + 2 n d) dtype
 * elements plus 2 B d f fp32, without the k d f and one B d f fp32 when the
 * states are given. */
int ttt_core_backward_mse_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                          size_t* bytes);

/* Gradients through the MSE chunk loop (ttt_core_apply_update with
 * TTT_MODE_MSE), for a loss that depends on O alone, given dO = dLoss/dO
 * [B, n, d] (dtype).  Per chunk (eq. (3)-(4)): O_c = Z_c W_c^T, R_c = Z_c W_c^T
 * - V^_c, W_{c+1} = W_c - (eta/C) R_c^T Z_c.  With G = dLoss/dW_{c+1} (zero
 * after the last chunk), taken from the last chunk back:
 *   T_c = dO_c - (eta/C) Z_c G^T
 *   dZ_c = T_c W_c - (eta/C) R_c G          [B, n, f] dtype
 *   dVhat_c = (eta/C) Z_c G^T               [B, n, d] dtype
 *   dLoss/dW_c = G + T_c^T Z_c;  dW_down0 = its sum over the rows at c = 0
 *                                           [d, f] fp32
 * The states W_c are W_states [B, k, d, f] dtype when given (kept by the
 * forward call through ttt_layer_options.W_states; DEVICE, 16-byte aligned),
 * else the call first runs the forward scan again and keeps them (bf16 copies
 * with bf16).  Then the reverse recursion: per
 * chunk the MSE apply twice (for R_c, and for T_c with dVhat_c), the
 * two-contraction dZ kernel, and the MSE update seeded with G.  doc_starts
 * [B, k] (DEVICE, as ttt_layer_options.doc_starts; NULL: one document per
 * row) packs documents: at a document's first chunk G goes to dW_down0 and
 * restarts from zero for the chunk before.  Update masks:
 * ttt_core_backward_ex (which also takes resumed rows).
 * seq_len == 0 or batch == 0 gives dW_down0 = 0.  Errors as for every entry
 * point. */
int ttt_core_backward_mse(const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                          const void* W_down0, const void* dO, const void* W_states, const unsigned char* doc_starts,
                          void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- backward of the whole dot layer ---- */

/* Workspace bytes for ttt_layer_backward (saved_states as for
 * ttt_core_backward_workspace_bytes).  About B n (5 f + 5 d) dtype elements
 * beside the chunk loop's own (ttt_core_backward_workspace_bytes), plus the
 * weight-gradient scans' scratch, a few times 2 f d. */
int ttt_layer_backward_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                       size_t* bytes);

/* Gradients of a loss that depends on the output O of the dot-objective layer
 * (ttt_chunk_apply_update with TTT_MODE_DOT and the causal convolution),
 * given dO = dLoss/dO [B, n, d] (dtype), with respect to
 * every input (Method §1-§3, eq. (1)-(6), by the chain rule):
 *   dH, dX0            [B, n, d] dtype
 *   dW_gate, dW_up     [f, d] fp32      (sums over the batch rows, as for
 *   dW_down0           [d, f] fp32       every weight: the rows share them)
 *   dW_target          [d, d] fp32      ([d_in, d_out], as W_target)
 *   dconv_w            [d, K] fp32
 * The call recomputes the forward's activations (Z, the convolution Y and
 * V^ = Y W_target), runs the chunk loop's backward (ttt_core_backward; the
 * states are W_states when the forward call kept them through
 * ttt_layer_options.W_states, else recomputed), then, with A = H W_gate^T,
 * U = H W_up^T, Z = silu(A) U: dA = dZ U silu'(A), dU = dZ silu(A),
 * dW_gate = sum dA^T H, dW_up = sum dU^T H, dH = dA W_gate + dU W_up;
 * dW_target = sum Y^T dV^, dY = dV^ W_target^T; dconv_w[i, j] = sum_t dY[t, i]
 * X0[t - (K-1) + j, i] and dX0[s, i] = sum_j conv_w[i, j] dY[s + K-1-j, i].
 * doc_starts [B, k] (DEVICE, as ttt_layer_options.doc_starts; NULL: one
 * document per row) packs documents: each is differentiated as the
 * independent sequence the forward call makes of it (the convolution and the
 * states restart at its first chunk), and the weight gradients add over
 * documents as over rows.
 * Token sums run in the fused scan's K steps, so chunk must be a multiple of
 * 64 (bf16) or 32 (fp32), else TTT_ERR_UNSUPPORTED.  batch == 0 or
 * seq_len == 0: every weight gradient is 0 and nothing else is touched.
 * Other rules as for every entry point. */
int ttt_layer_backward(const ttt_inplace_shape* shape, int dtype, float eta, const void* H, const void* X0,
                       const void* W_gate, const void* W_up, const void* W_down0, const void* W_target,
                       const void* conv_w, const void* dO, const void* W_states, const unsigned char* doc_starts,
                       void* dH, void* dX0, float* dW_gate, float* dW_up, float* dW_down0, float* dW_target,
                       float* dconv_w, void* workspace, size_t workspace_bytes, void* stream);

/* The chunk loop's backward for either objective with options:
 * mode TTT_MODE_DOT (or TTT_MODE_DOT_SCAN) as ttt_core_backward, TTT_MODE_MSE as
 * ttt_core_backward_mse; W_states and doc_starts as there, update_mask,
 * W_init and dW_init as in ttt_backward_options (conv_forward, x0_halo and
 * dx0_halo are not read).  Workspace: the matching
 * ttt_core_backward_workspace_bytes or ttt_core_backward_mse_workspace_bytes.
 * Other arguments, rules and errors as for those calls. */
int ttt_core_backward_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* Z,
                         const void* Vhat, const void* W_down0, const void* dO, const ttt_backward_options* options,
                         void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- backward of the whole MSE layer ---- */

/* Workspace bytes for ttt_layer_backward_mse (saved_states as for
 * ttt_core_backward_mse_workspace_bytes): the layer backward's own buffers
 * (as for ttt_layer_backward_workspace_bytes, plus V^ [B, n, d] dtype) beside
 * the MSE chunk loop's (ttt_core_backward_mse_workspace_bytes). */
int ttt_layer_backward_mse_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                           size_t* bytes);

/* ttt_layer_backward for the MSE objective (ttt_chunk_apply_update with
 * TTT_MODE_MSE and the causal convolution; In-Place TTT review, Method §1-§3,
 * eq. (1)-(5), the update of eq. (4) on the squared error (1/(2C))||Z_c W^T -
 * V^_c||^2): the same arguments, outputs, rules and errors.  The chunk loop's
 * gradients dZ, dV^ and dW_down0 come from the reverse recursion of
 * ttt_core_backward_mse (its states W_states [B, k, d, f] dtype when the
 * forward MSE call kept them, else recomputed); the producers', the target's
 * and the convolution's gradients follow as for the dot layer.  With packed
 * documents each is differentiated as an independent sequence. */
int ttt_layer_backward_mse(const ttt_inplace_shape* shape, int dtype, float eta, const void* H, const void* X0,
                           const void* W_gate, const void* W_up, const void* W_down0, const void* W_target,
                           const void* conv_w, const void* dO, const void* W_states, const unsigned char* doc_starts,
                           void* dH, void* dX0, float* dW_gate, float* dW_up, float* dW_down0, float* dW_target,
                           float* dconv_w, void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer's backward for either objective with options: mode
 * TTT_MODE_DOT (or TTT_MODE_DOT_SCAN) as ttt_layer_backward, TTT_MODE_MSE as
 * ttt_layer_backward_mse, and every field of ttt_backward_options (the update
 * mask, the convolution's direction and the resumed rows' W_init and
 * x0_halo as the forward call took them, with their gradients; the
 * forward-looking convolution's gradient stays inside each chunk, as its
 * window does).  Workspace: ttt_layer_backward_workspace_bytes or
 * ttt_layer_backward_mse_workspace_bytes.  Other arguments, rules and errors
 * as for those calls. */
int ttt_layer_backward_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H,
                          const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
                          const void* W_target, const void* conv_w, const void* dO,
                          const ttt_backward_options* options, void* dH, void* dX0, float* dW_gate, float* dW_up,
                          float* dW_down0, float* dW_target, float* dconv_w, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- the individual steps (each is one stage of the call above; they compose
 *      into it and exist for composition and per-step checks).  The updates
 *      contract over tokens, so they read token-contiguous (transposed) copies:
 *      Zt [B, f, n] and Vt [B, d, n]. ---- */

/* Slow producer (eq. (2)): Z = silu(H W_gate^T) * (H W_up^T), written as
 * Zt [B, f, n] (required) and Z [B, n, f] (may be NULL).  conv_k and chunk of
 * the shape are not used (chunk must still divide seq_len). */
int ttt_produce_z(const ttt_inplace_shape* shape, int dtype, const void* H, const void* W_gate,
                  const void* W_up, void* Z, void* Zt, void* stream);

/* Workspace bytes for ttt_produce_vhat (the convolved embeddings and a
 * transposed copy of W_target). */
int ttt_vhat_workspace_bytes(const ttt_inplace_shape* shape, int dtype, size_t* bytes);

/* Target producer (eq. (5), causal padding of Method §3):
 * Vt [B, d, n] = scale * (CausalDepthwiseConv1D_K(X0) W_target)^T (conventions
 * above).  scale = 1 gives the target itself; scale = eta gives the form the
 * fused update takes. */
int ttt_produce_vhat(const ttt_inplace_shape* shape, int dtype, float scale, const void* X0, const void* conv_w,
                     const void* W_target, void* Vt, void* workspace, size_t workspace_bytes, void* stream);

/* Per-chunk deltas of the dot objective (Method §3 step 1, eq. (6)):
 * dW [B, k, d, f] fp32, dW[b, c] = Vhat_c^T Z_c over the chunk's C tokens,
 * read from Zt [B, f, n] and Vt [B, d, n]. */
int ttt_chunk_delta(const ttt_inplace_shape* shape, int dtype, const void* Zt, const void* Vt,
                    float* dW, void* stream);

/* Exclusive prefix scan over chunks (Method §3 steps 2-3):
 * Wc [B, k, d, f] dtype, Wc[b, c] = W_down0 + eta * sum_{j<c} dW[b, j];
 * W_final [B, d, f] fp32 = W_down0 + eta * sum_{j<k} dW[b, j]. */
int ttt_chunk_scan(const ttt_inplace_shape* shape, int dtype, float eta, const void* W_down0,
                   const float* dW, void* Wc, float* W_final, void* stream);

/* Scratch of ttt_chunk_update_scan for these sizes: 0 when the sequence runs
 * as one segment, else the partial states (dtype) and segment totals (fp32)
 * below. */
int ttt_update_scan_workspace_bytes(const ttt_inplace_shape* shape, int dtype, size_t* bytes);

/* Deltas and scan fused (chunk % 64 == 0 for bf16, % 32 for fp32, else
 * TTT_ERR_UNSUPPORTED), with eta carried by the target: Vt = eta * V^^T (from
 * ttt_produce_vhat with scale = eta), since eta V^_c^T Z_c = (eta V^_c)^T Z_c.
 * The deltas do not depend on the state (eq. (6)), so the scan is the running
 * value of one contraction over the tokens: one MFMA pass per output tile,
 * whose fp32 accumulator starts at W_down0 and holds W_c after the tokens of
 * chunks 0..c-1; at each chunk boundary the tile writes Wc[b, c], after the
 * last chunk W_final.  When the state has too few tiles to fill the GPU, the
 * sequence may run as S side-by-side segments (S in {1, 2, 4} dividing the
 * chunk count, chosen from d_model, d_ff, chunk and the chunk count alone by
 * weighing the rounds of tiles against the cost of joining the segments).
 * S = 2: each second-segment tile takes the first segment's end state (fp32)
 * of the same state tile inside the kernel, one chunk into its K loop, so
 * every state is rounded once.  That wait is bounded (20 ms, or
 * TTT_UPDATE_SCAN_WAIT_US microseconds read from the environment at each call;
 * negative: no wait); a tile that does not receive the end state in time keeps
 * partial states, which a short pass after the kernel completes (rounding
 * them twice in bf16).  S = 4: a short elementwise pass adds the earlier
 * segments' totals (fp32) to the later segments' partial states (kept in
 * dtype; with bf16 a state of a later segment is thus rounded twice).
 * `workspace` (device, at least ttt_update_scan_workspace_bytes) holds the
 * partial states (S = 4; with S = 2 two flag words per state tile in their
 * place) and the totals, and may be NULL when that query returns 0.
 * Same outputs as ttt_chunk_delta (on the unscaled target) followed by
 * ttt_chunk_scan with eta, without dW. */
int ttt_chunk_update_scan(const ttt_inplace_shape* shape, int dtype, const void* W_down0, const void* Zt,
                          const void* Vt, void* Wc, float* W_final, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Apply (eq. (3)): O [B, n, d], O_c = Z_c Wc[b, c]^T, with Z given as its
 * token-contiguous copy Zt [B, f, n] (the one the updates read; the kernel
 * contracts over f by transposing tiles in LDS) and Wc [B, k, d, f] dtype. */
int ttt_chunk_apply(const ttt_inplace_shape* shape, int dtype, const void* Zt, const void* Wc, void* O,
                    void* stream);

/* ------------------------------------------------------------------ LaCT SwiGLU layer */

/* Workspace bytes for ttt_lact_swiglu. */
int ttt_lact_workspace_bytes(const ttt_lact_shape* shape, int dtype, size_t* bytes);

/* LaCT fast-weight layer (review of "Test-Time Training Done Right", LaCT
 * Model Architecture §1, eq. (3)-(4); plain GD, one full-chunk step per chunk):
 *   f_W(x) = W2 [silu(W1 x) * (W3 x)], loss per chunk sum_i (1/2)||f_W(k_i) - v_i||^2,
 *   W <- W - eta * grad (W1, W2, W3 updated together), o_i = f_W(q_i),
 *   order: TTT_UPDATE_THEN_APPLY (queries of chunk c see the step taken on
 *   chunk c) or TTT_APPLY_THEN_UPDATE (they see the state before it).
 *
 *   q, k, v   [B, H, n, dh]   dtype
 *   W1, W3    [H, m, dh]      dtype   initial fast weights (shared by batch rows)
 *   W2        [H, dh, m]      dtype
 *   O         [B, H, n, dh]   dtype   (written)
 *   W1_f, W3_f [B, H, m, dh]  fp32    final states (written)
 *   W2_f      [B, H, dh, m]   fp32
 * Supported: head_dim, hidden, chunk multiples of 8; seq_len % chunk == 0.
 * Every launch is enqueued on `stream` (ttt_lact_swiglu_ex can split the rows
 * over a second stream the caller provides). */
int ttt_lact_swiglu(const ttt_lact_shape* shape, int dtype, int order, float eta,
                    const void* q, const void* k, const void* v,
                    const void* W1, const void* W3, const void* W2,
                    void* O, float* W1_f, float* W3_f, float* W2_f,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Options of ttt_lact_swiglu_ex (zero-initialise, then set what is needed). */
typedef struct {
  /* TTT_UPDATE_THEN_APPLY (0) or TTT_APPLY_THEN_UPDATE (1), as in ttt_lact_swiglu. */
  int order;
  /* Strided update (review of "Test-Time Training Done Right", LaCT Model
   * Architecture §1 on the order of the apply and update operations: updating
   * on some chunks only while applying all of them gives a strided
   * block-wise causal mask; its video use updates on clean chunks).
   * [n / chunk] uint8, HOST memory read during the call, shared by every
   * (batch, head) row: chunk c's keys and values take the gradient step only
   * where update_mask[c] != 0; every chunk's queries are applied.  NULL:
   * every chunk updates.  The mask decides which launches are enqueued, so a
   * captured graph keeps the mask it was captured with. */
  const unsigned char* update_mask;
  /* Per-token learning rates eta_i weighting each token's loss in the
   * gradient (§1, eq. (3)), on top of the scalar eta: [B, H, n] fp32, DEVICE,
   * 16-byte aligned.  NULL: all 1. */
  const float* eta_tok;
  /* 0: the squared error (1/2)||f_W(k) - v||^2 of ttt_lact_swiglu; 1: the
   * dot-product loss -f_W(k)^T v (§1).  Other values: TTT_ERR_ARG. */
  int loss;
  /* 1: after every update, L2-normalise each row of W1, W3 (over head_dim)
   * and of W2 (over hidden) -- the input dimension of each matrix (§2,
   * fast-weight normalisation); the final states are normalised too.  0: no
   * normalisation.  Other values: TTT_ERR_ARG. */
  int weight_norm;
  /* 1: the Muon update rule (§2): each gradient g is replaced by Muon(g) ~
   * U V^T before the step (and before weight_norm).  The page names the
   * Newton-Schulz iteration without its polynomial; this is the quintic one
   * published with the Muon optimizer (coefficients 3.4445, -4.7750, 2.0315,
   * five steps on g / ||g||_F taken as [min(m, dh), max(m, dh)]), run in the
   * layer's dtype with fp32 accumulation.  0: plain gradient.  Other values:
   * TTT_ERR_ARG. */
  int muon;
  /* Two chains: side_stream (a hipStream_t of the same device as `stream`)
   * runs the second half of the (batch, head) rows while `stream` runs the
   * first half, so that one chain's epilogues and short launches overlap the
   * other's contractions.  fork_event and join_event (hipEvent_t, e.g. created
   * with hipEventDisableTiming) order it: the side work starts after
   * everything enqueued on `stream` before the call, and everything enqueued
   * on `stream` after the call waits for it, so the call is ordered on
   * `stream` like one kernel.  All three belong to the caller (created,
   * destroyed, and not shared by calls that may be enqueued concurrently).
   * NULL side_stream: every row runs in one chain on `stream` (the events are
   * not read).  A side stream without both events: TTT_ERR_ARG.  With a
   * single row the side stream is not used. */
  void* side_stream;
  void* fork_event;
  void* join_event;
  /* Keeping the states for a backward pass: W_states (DEVICE, 16-byte
   * aligned, dtype) receives, for every chunk c = 0 .. n / chunk and every
   * (batch, head) row bh, the operand copies of the state chunk c's update
   * starts from (slot n / chunk: the final state) -- W1 [m, dh], W3 [m, dh],
   * W2 [dh, m] one after the other at W_states + ((c B H + bh) 3 + i) m dh,
   * i = 0, 1, 2: (n / chunk + 1) B H 3 m dh elements.  A masked chunk's slot
   * repeats the state it passes on.  One copy per chunk (3 B H m dh dtype
   * elements of traffic).  ttt_lact_swiglu_backward_ex takes them and skips
   * recomputing them.  NULL: not kept. */
  void* W_states;
} ttt_lact_options;

/* The LaCT layer of ttt_lact_swiglu with options (above; NULL options:
 * TTT_ERR_ARG); same arguments, workspace and errors otherwise. */
int ttt_lact_swiglu_ex(const ttt_lact_shape* shape, int dtype, float eta,
                       const void* q, const void* k, const void* v,
                       const void* W1, const void* W3, const void* W2,
                       const ttt_lact_options* options,
                       void* O, float* W1_f, float* W3_f, float* W2_f,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for ttt_lact_swiglu_backward: the forward's own
 * (ttt_lact_workspace_bytes), every chunk's state ((n / chunk + 1) B H 3 m dh
 * dtype), the state gradient (3 B H m dh fp32 and a dtype copy) and the
 * per-chunk intermediates (16 B H chunk m and 2 B H chunk dh dtype, B H chunk
 * dh fp32). */
int ttt_lact_backward_workspace_bytes(const ttt_lact_shape* shape, int dtype, size_t* bytes);

/* Gradients of a loss that depends on the output O of ttt_lact_swiglu (the
 * squared error, plain GD; an update mask through ttt_lact_swiglu_backward_ex,
 * no per-token rates, dot loss, normalisation or Muon) with respect to every
 * input, given dO = dLoss/dO [B, H, n, dh] (dtype)
 * (review of "Test-Time Training Done Right", LaCT Model Architecture §1,
 * eq. (3)-(4), by the chain rule through the chunk loop):
 *   dq, dk, dv   [B, H, n, dh] dtype
 *   dW1, dW3     [H, m, dh] fp32    gradients of the initial weights, summed
 *   dW2          [H, dh, m] fp32    over the batch rows (they share them)
 * Each update W' = W - eta G(W; k, v) is differentiated through G itself, so
 * the second derivatives of the SwiGLU loss enter (through silu'' among
 * others).  The call first recomputes every chunk's state with the forward
 * kernels (keys only) and keeps them in the workspace, then runs the chunks
 * from the last back: the query apply's backward with the state it saw (after
 * the chunk's update, or before it in TTT_APPLY_THEN_UPDATE order) and the
 * update's backward: the forward's gate and residual kernels on the chunk's
 * rows, then batched engine GEMMs over the (batch, head) rows whose epilogues
 * form the gate terms, and one elementwise pass.  dtype, sizes and errors as for
 * ttt_lact_swiglu; batch == 0 gives zero weight gradients, seq_len == 0 zero
 * weight gradients and nothing else. */
int ttt_lact_swiglu_backward(const ttt_lact_shape* shape, int dtype, int order, float eta,
                             const void* q, const void* k, const void* v,
                             const void* W1, const void* W3, const void* W2, const void* dO,
                             void* dq, void* dk, void* dv, float* dW1, float* dW3, float* dW2,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for ttt_lact_swiglu_backward_ex: with saved_states = 1 (the
 * forward call kept its states, ttt_lact_options.W_states) the forward's
 * workspace and the state slots are not needed; saved_states = 0 gives
 * ttt_lact_backward_workspace_bytes.  Other values: TTT_ERR_ARG. */
int ttt_lact_backward_workspace_bytes_ex(const ttt_lact_shape* shape, int dtype, int saved_states, size_t* bytes);

/* ttt_lact_swiglu_backward with the forward call's ttt_lact_options (NULL:
 * TTT_ERR_ARG): `order` and `update_mask` (HOST, [n / chunk], as for
 * ttt_lact_swiglu_ex) are taken -- a chunk whose flag is zero was applied but
 * took no step, so the state gradient passes it unchanged and its dk and dv
 * rows are zero.  W_states, if not NULL, holds the states the forward call
 * kept (same options, same inputs): the call reads them instead of
 * recomputing them, with the workspace of
 * ttt_lact_backward_workspace_bytes_ex(..., saved_states = 1, ...).  The update's variants have no backward here: eta_tok, the
 * dot loss, weight_norm or muon give TTT_ERR_UNSUPPORTED (invalid values of
 * the flags TTT_ERR_ARG).  side_stream and its events are not read (the
 * backward runs as one chain on `stream`).  Other arguments, workspace and
 * errors as for ttt_lact_swiglu_backward. */
int ttt_lact_swiglu_backward_ex(const ttt_lact_shape* shape, int dtype, float eta,
                                const void* q, const void* k, const void* v,
                                const void* W1, const void* W3, const void* W2, const void* dO,
                                const ttt_lact_options* options,
                                void* dq, void* dk, void* dv, float* dW1, float* dW3, float* dW2,
                                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */
