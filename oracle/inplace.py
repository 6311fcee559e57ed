"""Float64 oracle of the In-Place TTT layer (test infrastructure only).

Sources (page titles and sections; the pages are web reviews of the paper):
  * "In-Place Test-Time Training" review, Method §1 *Overall Framework*:
    eq. (1) the gated MLP, eq. (2) the intermediate Z, the chunk split, and
    the two per-chunk operations in order -- apply, eq. (3), then a gradient
    step on the fast weight, eq. (4).
  * same page, Method §2 *LM-Aligned Objective*: eq. (5) the target
    V^ = Conv1D(X0) W_target, and eq. (6) the closed-form step under the
    negative Frobenius inner-product loss.
  * same page, Method §3 *Implementation Details*: the three-step parallel
    form (all per-chunk deltas, one exclusive prefix sum, all applies), causal
    padding of the convolution, and the reset of the fast weight at each
    document boundary.
  * "In-Place Test-Time Training" notes (gitcode), *implementation details*:
    the same prefix-sum restatement.
  * TTT-E2E summary, *mini-batch TTT*: the 1/b mean over a mini-batch, which
    is the 1/C of the MSE objective here.

Readings where the pages are open (each is listed with its reason in the
design notes of the repository):
  * phi is SiLU, silu(x) = x / (1 + exp(-x)).
  * Conv1D is depthwise with weights conv_w[d, K] and no bias, left
    zero-padded by K-1 ("causal padding"): tap K-1 multiplies the current
    token, tap j multiplies the token K-1-j steps back.
  * V^ = Y @ W_target with W_target indexed [d_in, d_out] (eq. (5) has no
    transpose).
  * Chunk c (0-based) is applied with the state left by chunks 0..c-1; chunk 0
    uses W_down0; W_final includes the last chunk's update.
  * dot objective: L = -<Z W^T, V^>_F, so the step is W + eta V^_c^T Z_c
    (eq. (6), no 1/C).
  * mse objective: L = (1/(2C)) ||Z_c W^T - V^_c||_F^2 at the pre-update W,
    so the step is W - (eta/C)(Z_c W^T - V^_c)^T Z_c, with C the number of
    tokens in that chunk.
  * each batch row is one document with its own state starting at W_down0,
    unless document starts are given (a packed row): a document may then
    start at any chunk boundary, where the state is reset to W_down0 and the
    convolution restarts (left zero padding at the document's first token),
    so that nothing of the previous document reaches it (Method §3, document
    boundaries).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu", "causal_depthwise_conv1d", "forward_chunk_conv1d", "target_values", "gated_intermediate",
    "gated_mlp", "loss_dot", "loss_mse", "grad_dot", "grad_mse",
    "chunk_apply_update", "chunk_core_backward", "mse_core_backward", "chunk_prefix_form", "inplace_layer",
    "layer_backward", "resumed_core_backward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(x):
    """SiLU (the reading of phi in eq. (1)): x * sigmoid(x)."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def causal_depthwise_conv1d(X0, conv_w):
    """Causal depthwise 1-D convolution along the token axis (eq. (5), with the
    causal padding of Method §3).

    X0: [..., n, d]; conv_w: [d, K].  Y[t, ch] = sum_j conv_w[ch, j] *
    X0[t - (K-1) + j, ch], where rows before the first token are zero.
    """
    X0 = _f64(X0)
    conv_w = _f64(conv_w)
    n = X0.shape[-2]
    K = conv_w.shape[1]
    Y = np.zeros_like(X0)
    for j in range(K):
        back = K - 1 - j          # tap j looks this many tokens back
        if back >= n:
            continue
        Y[..., back:, :] += conv_w[:, j] * X0[..., : n - back, :]
    return Y


def forward_chunk_conv1d(X0, conv_w, chunk):
    """The forward-looking reading of the convolution (the review's next-token
    example, Method §2): within each chunk, tap j multiplies the token j steps
    ahead, and tokens past the chunk's end are zero, so a chunk's targets come
    from its own tokens only and the per-chunk step stays causal at chunk level.
    With W_target = I and conv_w[:, 1] = 1 (all other taps 0) the target of a
    token is the next token's embedding, except at a chunk's last token.

    X0: [..., n, d]; conv_w: [d, K].  Y[t, ch] = sum_j conv_w[ch, j] *
    X0[t + j, ch] for t + j inside t's chunk.
    """
    X0 = _f64(X0)
    conv_w = _f64(conv_w)
    n = X0.shape[-2]
    K = conv_w.shape[1]
    Y = np.zeros_like(X0)
    for s in range(0, n, chunk):
        e = min(s + chunk, n)
        for j in range(K):
            if j >= e - s:
                continue
            Y[..., s: e - j, :] += conv_w[:, j] * X0[..., s + j: e, :]
    return Y


def target_values(X0, conv_w, W_target):
    """V^ = Conv1D(X0) W_target (eq. (5)); W_target is [d_in, d_out]."""
    return causal_depthwise_conv1d(X0, conv_w) @ _f64(W_target)


def gated_intermediate(H, W_gate, W_up):
    """Z = phi(H W_gate^T) * (H W_up^T) (eq. (2)); H [n, d], W_gate/W_up [f, d]."""
    H = _f64(H)
    return silu(H @ _f64(W_gate).T) * (H @ _f64(W_up).T)


def gated_mlp(H, W_gate, W_up, W_down):
    """The unmodified gated MLP of eq. (1): O = Z W_down^T, W_down [d, f]."""
    return gated_intermediate(H, W_gate, W_up) @ _f64(W_down).T


# --- the two objectives, as losses and as their gradients with respect to W ---

def loss_dot(W, Zc, Vc):
    """Negative Frobenius inner product between the chunk's output Z W^T and
    its target (Method §2)."""
    return -float(np.sum((_f64(Zc) @ _f64(W).T) * _f64(Vc)))


def loss_mse(W, Zc, Vc):
    """Mean-over-the-chunk squared reconstruction error, (1/(2C))||Z W^T - V||^2."""
    Zc = _f64(Zc)
    E = Zc @ _f64(W).T - _f64(Vc)
    return float(0.5 * np.sum(E * E) / Zc.shape[0])


def grad_dot(W, Zc, Vc):
    """Gradient of loss_dot with respect to W [d, f]; independent of W."""
    return -(_f64(Vc).T @ _f64(Zc))


def grad_mse(W, Zc, Vc):
    """Gradient of loss_mse with respect to W [d, f], at the given W."""
    Zc = _f64(Zc)
    return ((Zc @ _f64(W).T - _f64(Vc)).T @ Zc) / Zc.shape[0]


_GRADS = {"dot": grad_dot, "mse": grad_mse}


def chunk_apply_update(Z, Vhat, W0, chunk, eta, mode, update_first=False):
    """The sequential definition (Method §1): for each chunk in order, apply the
    current state (eq. (3)), then take one gradient step on it (eq. (4)).
    `update_first` takes the step first and applies the updated state (the
    update-then-apply order of the LaCT review's section on the order of the
    two operations); W_final is the same in both orders.

    Z [n, f], Vhat [n, d], W0 [d, f].  A last chunk shorter than `chunk` is
    allowed here (it is simply the remaining tokens).
    Returns (O [n, d], W_final [d, f]).
    """
    Z, Vhat = _f64(Z), _f64(Vhat)
    W = _f64(W0).copy()
    grad = _GRADS[mode]
    n = Z.shape[0]
    O = np.empty((n, W.shape[0]))
    for start in range(0, n, chunk):
        rows = slice(start, min(start + chunk, n))
        if not update_first:
            O[rows] = Z[rows] @ W.T                   # apply: state before this chunk
        W = W - eta * grad(W, Z[rows], Vhat[rows])     # update: gradient at that state
        if update_first:
            O[rows] = Z[rows] @ W.T                   # apply: the state after this chunk's step
    return O, W


def chunk_core_backward(Z, Vhat, W0, chunk, eta, dO, doc_starts=None, update_mask=None):
    """Gradients of a loss through the dot-objective chunk loop (chunk_apply_update
    with mode "dot"), given dO = dLoss/dO: returns (dZ [n, f], dVhat [n, d],
    dW0 [d, f]).  The chain rule through O_c = Z_c W_c^T (eq. (3)) and
    W_c = W0 + eta sum_{j<c} Vhat_j^T Z_j (eq. (6), Method §3): chunk c's output
    gives the state gradient dW_c = dO_c^T Z_c; each delta j reaches every later
    state, so with the exclusive suffix S_j = sum_{c>j} dW_c,
      dZ_j    = dO_j W_j + eta Vhat_j S_j,
      dVhat_j = eta Z_j S_j^T,
      dW0     = sum_c dW_c.
    `doc_starts` [n_chunks] (truthy entries; chunk 0 always starts one) packs
    documents as in inplace_layer: the state restarts from W0 at each start, so
    a delta reaches only the later states of its own document, the suffix
    sums run to the end of the document, and W0 receives every document's sum.
    `update_mask` [n_chunks] (truthy entries update) as in inplace_layer: a
    masked chunk's delta is not added, which is the same loop with that chunk's
    targets zero; its targets then reach nothing, so their gradient is zero.
    The loss is taken to depend on O only (not on W_final)."""
    Z, Vhat, W0, dO = _f64(Z), _f64(Vhat), _f64(W0), _f64(dO)
    n = Z.shape[0]
    bounds = [(s, min(s + chunk, n)) for s in range(0, n, chunk)]
    if update_mask is not None:
        Vhat = Vhat.copy()
        for c, (s, e) in enumerate(bounds):
            if not update_mask[c]:
                Vhat[s:e] = 0.0
    starts = [c == 0 or (doc_starts is not None and bool(doc_starts[c])) for c in range(len(bounds))]
    states = []                                   # W_c, the state chunk c is applied with
    W = W0.copy()
    for c, (s, e) in enumerate(bounds):
        if starts[c]:
            W = W0.copy()
        states.append(W)
        W = W + eta * (Vhat[s:e].T @ Z[s:e])
    dWc = [dO[s:e].T @ Z[s:e] for (s, e) in bounds]
    dZ = np.empty_like(Z)
    dV = np.empty_like(Vhat)
    dW0 = np.zeros_like(W0)
    S = np.zeros_like(W0)                         # sum of dW_c over the later chunks of the current document
    for c in range(len(bounds) - 1, -1, -1):
        s, e = bounds[c]
        dZ[s:e] = dO[s:e] @ states[c] + eta * (Vhat[s:e] @ S)
        dV[s:e] = eta * (Z[s:e] @ S.T)
        S = S + dWc[c]
        if starts[c]:                             # the document's first chunk: its sum reaches W0
            dW0 = dW0 + S
            S = np.zeros_like(W0)
    if update_mask is not None:
        for c, (s, e) in enumerate(bounds):
            if not update_mask[c]:
                dV[s:e] = 0.0
    return dZ, dV, dW0


def mse_core_backward(Z, Vhat, W0, chunk, eta, dO, doc_starts=None, update_mask=None):
    """Gradients of a loss through the MSE chunk loop (chunk_apply_update with
    mode "mse"), given dO = dLoss/dO: returns (dZ [n, f], dVhat [n, d],
    dW0 [d, f]).  Per chunk (eq. (3)-(4)): O_c = Z_c W_c^T, R_c = Z_c W_c^T -
    Vhat_c, W_{c+1} = W_c - (eta/C) R_c^T Z_c with C the chunk's tokens.  With
    G = dLoss/dW_{c+1}, taken from the last chunk back (zero after it):
      T_c      = dO_c - (eta/C) Z_c G^T
      dZ_c     = T_c W_c - (eta/C) R_c G
      dVhat_c  = (eta/C) Z_c G^T
      dLoss/dW_c = G + T_c^T Z_c,
    and dW0 is dLoss/dW_0.  The loss is taken to depend on O only.
    `doc_starts` [n_chunks] packs documents as in inplace_layer; they are
    independent sequences, so the gradients are those of each document taken
    alone, dW0 summed over them.  `update_mask` [n_chunks]: a masked chunk
    takes no step (W_{c+1} = W_c), i.e. its eta/C is zero in the formulas above."""
    if doc_starts is not None:
        cuts = [c * chunk for c in range(len(doc_starts)) if c == 0 or doc_starts[c]] + [len(Z)]
        um = lambda a, e: None if update_mask is None else update_mask[a // chunk: (e + chunk - 1) // chunk]
        parts = [mse_core_backward(Z[a:e], Vhat[a:e], W0, chunk, eta, dO[a:e], update_mask=um(a, e))
                 for a, e in zip(cuts[:-1], cuts[1:])]
        return (np.concatenate([q[0] for q in parts]), np.concatenate([q[1] for q in parts]),
                sum(q[2] for q in parts))
    Z, Vhat, W0, dO = _f64(Z), _f64(Vhat), _f64(W0), _f64(dO)
    n = Z.shape[0]
    bounds = [(s, min(s + chunk, n)) for s in range(0, n, chunk)]
    flag = lambda c: 1.0 if update_mask is None or update_mask[c] else 0.0
    states = []
    W = W0.copy()
    for c, (s, e) in enumerate(bounds):           # the forward scan, keeping the state each chunk saw
        states.append(W)
        W = W - flag(c) * eta * grad_mse(W, Z[s:e], Vhat[s:e])
    dZ = np.empty_like(Z)
    dV = np.empty_like(Vhat)
    G = np.zeros_like(W0)
    for c in range(len(bounds) - 1, -1, -1):
        s, e = bounds[c]
        Zc, Wc, a = Z[s:e], states[c], flag(c) * eta / (e - s)
        R = Zc @ Wc.T - Vhat[s:e]
        Q = Zc @ G.T
        T = dO[s:e] - a * Q
        dZ[s:e] = T @ Wc - a * (R @ G)
        dV[s:e] = a * Q
        G = G + T.T @ Zc
    return dZ, dV, G


def resumed_core_backward(Z, Vhat, W0, W_init, chunk, eta, dO, mode, doc_starts=None, update_mask=None):
    """The chunk loop's backward for a resumed row (inplace_layer's W_init): its
    first document continues from W_init unless doc_starts flags chunk 0, and
    every later document starts from W0.  The documents are independent
    sequences, so the first one's gradients are the plain backward with W_init
    in place of W0, whose initial-state gradient is the row's dW_init.
    Returns (dZ, dVhat, dW0, dW_init)."""
    back = {"dot": chunk_core_backward, "mse": mse_core_backward}[mode]
    n = len(Z)
    k = -(-n // chunk)
    flags = [bool(doc_starts[c]) if doc_starts is not None else False for c in range(k)]
    if flags[0]:                                  # a document starts at the resume point: nothing continues
        out = back(Z, Vhat, W0, chunk, eta, dO, doc_starts=doc_starts, update_mask=update_mask)
        return out[0], out[1], out[2], np.zeros_like(_f64(W_init))
    cut = next((c for c in range(1, k) if flags[c]), k)
    e = min(cut * chunk, n)
    um = lambda a, b: None if update_mask is None else update_mask[a:b]
    first = back(Z[:e], Vhat[:e], W_init, chunk, eta, dO[:e], update_mask=um(0, cut))
    if e == n:
        return first[0], first[1], np.zeros_like(_f64(W0)), first[2]
    rest = back(Z[e:], Vhat[e:], W0, chunk, eta, dO[e:], doc_starts=flags[cut:], update_mask=um(cut, k))
    return (np.concatenate([first[0], rest[0]]), np.concatenate([first[1], rest[1]]), rest[2], first[2])


def chunk_prefix_form(Z, Vhat, W0, chunk, eta):
    """The three-step parallel form of the dot-product update (Method §3):
    (1) every chunk's delta V^_c^T Z_c, (2) one exclusive prefix sum over the
    deltas, (3) every chunk applied with W0 + eta * (its prefix).
    Returns (O [n, d], W_final [d, f])."""
    Z, Vhat, W0 = _f64(Z), _f64(Vhat), _f64(W0)
    n = Z.shape[0]
    bounds = [(s, min(s + chunk, n)) for s in range(0, n, chunk)]
    deltas = [Vhat[s:e].T @ Z[s:e] for (s, e) in bounds]           # step 1
    prefix = [np.zeros_like(W0)]                                     # step 2
    for dW in deltas:
        prefix.append(prefix[-1] + dW)
    O = np.empty((n, W0.shape[0]))
    for c, (s, e) in enumerate(bounds):                              # step 3
        O[s:e] = Z[s:e] @ (W0 + eta * prefix[c]).T
    return O, W0 + eta * prefix[-1]


def inplace_layer(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk, eta,
                  mode, max_chunks=None, x0_halo=None, doc_starts=None, conv_forward=False, W_init=None,
                  update_mask=None, update_first=False):
    """The whole In-Place TTT layer, one document per batch row.

    H, X0 [B, n, d]; W_gate, W_up [f, d]; W_down0 [d, f]; W_target [d, d];
    conv_w [d, K].  Streams chunk by chunk: Z_c and V^_c are formed for the
    chunk only (the convolution reads the K-1 previous rows of X0, or
    `x0_halo` [B, K-1, d] before the first row, else zeros).

    `doc_starts` [B, n_chunks] (truthy entries) packs several documents into a
    row: a document starts at every flagged chunk c > 0 (chunk 0 always starts
    one), where the state is reset to W_down0 and the convolution restarts
    with zeros before the chunk's first row (Method §3, document boundaries).

    `W_init` [B, d, f], if given, is each row's state before its first chunk
    (resuming a sequence: the previous call's W_final, with `x0_halo` its last
    K-1 rows of X0); a document start flagged at chunk 0 still resets to
    W_down0 and the convolution to zeros.

    `conv_forward` takes the forward-looking in-chunk convolution
    (forward_chunk_conv1d) for the target; it reads no row outside the chunk,
    so `x0_halo` and document starts do not change it.

    `update_mask` [B, n_chunks] (truthy entries), if given, takes the update
    step on the flagged chunks only; every chunk is applied (the strided
    update of the LaCT review's section on the order of the apply and update
    operations, read onto this layer).

    `update_first` takes each chunk's step before its apply (as in
    chunk_apply_update): chunk c's outputs then see its own targets, so the
    layer is no longer causal inside a chunk -- for non-causal uses.

    `max_chunks` stops after that many chunks (O then covers only those rows
    and W_final is the state after them) -- used to time a bounded sample.

    Returns (O [B, n', d], W_final [B, d, f]).
    """
    H, X0 = _f64(H), _f64(X0)
    W_gate, W_up, W_target, conv_w = map(_f64, (W_gate, W_up, W_target, conv_w))
    B, n, d = H.shape
    K = conv_w.shape[1]
    grad = _GRADS[mode]
    n_chunks = -(-n // chunk) if n else 0
    if max_chunks is not None:
        n_chunks = min(n_chunks, max_chunks)
    n_out = min(n, n_chunks * chunk)
    O = np.empty((B, n_out, d))
    W_final = np.empty((B, d, W_gate.shape[0]))
    for b in range(B):
        if x0_halo is not None:
            Xfull = np.concatenate([_f64(x0_halo[b]), X0[b]], axis=0)
            off = K - 1
        else:
            Xfull, off = X0[b], 0
        W = _f64(W_down0).copy()       # document boundary: reset to the pretrained state
        if W_init is not None:
            W = _f64(W_init[b]).copy()  # a resumed row continues from its state
        doc_row = 0                    # first row of the current document in Xfull (the halo serves the first)
        for c in range(n_chunks):
            s, e = c * chunk, min((c + 1) * chunk, n)
            if (c > 0 or W_init is not None or x0_halo is not None) and doc_starts is not None and doc_starts[b][c]:
                W = _f64(W_down0).copy()   # a packed document starts here
                doc_row = s + off
            lo = max(doc_row, s + off - (K - 1))
            if conv_forward:
                Y = forward_chunk_conv1d(Xfull[s + off: e + off], conv_w, e - s)
            else:
                Y = causal_depthwise_conv1d(Xfull[lo: e + off], conv_w)[-(e - s):]
            Vc = Y @ W_target
            Zc = gated_intermediate(H[b, s:e], W_gate, W_up)
            if not update_first:
                O[b, s:e] = Zc @ W.T
            if update_mask is None or update_mask[b][c]:
                W = W - eta * grad(W, Zc, Vc)
            if update_first:
                O[b, s:e] = Zc @ W.T
        W_final[b] = W
    return O, W_final


def layer_backward(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk, eta, dO, doc_starts=None, mode="dot",
                   update_mask=None, conv_forward=False, W_init=None, x0_halo=None):
    """Gradients of a loss that depends on the output O of the layer
    (inplace_layer with the causal convolution, one document per row, and the
    objective `mode`, "dot" or "mse"), given dO = dLoss/dO [B, n, d].  Returns
    (dH, dX0 [B, n, d], dW_gate, dW_up [f, d], dW_down0 [d, f],
    dW_target [d, d], dconv_w [d, K]).

    The chain rule through the layer's definitions, one step at a time:
      * the chunk loop (chunk_core_backward for the dot objective,
        mse_core_backward for the MSE one, per row) gives dZ, dVhat and the
        row's part of dW_down0;
      * Z = silu(A) * U with A = H W_gate^T and U = H W_up^T (eq. (2)):
        dA = dZ * U * silu'(A) and dU = dZ * silu(A), where
        silu'(a) = s(a) (1 + a (1 - s(a))) with s the logistic function;
        dW_gate = dA^T H, dW_up = dU^T H, dH = dA W_gate + dU W_up;
      * Vhat = Y W_target with Y the causal convolution of X0 (eq. (5)):
        dW_target = Y^T dVhat and dY = dVhat W_target^T;
      * Y[t, i] = sum_j conv_w[i, j] X0[t - (K-1) + j, i]:
        dconv_w[i, j] = sum_t dY[t, i] X0[t - (K-1) + j, i] and
        dX0[s, i] = sum_j conv_w[i, j] dY[s + (K-1) - j, i] (rows outside
        the sequence contribute nothing).
    The weights are shared by the batch rows, so their gradients add over rows.

    `doc_starts` [B, n_chunks] packs documents as in inplace_layer.  The
    documents of a row are independent sequences (the state restarts from
    W_down0 and the convolution from zeros at each start), so the row's
    gradients are those of its documents taken one at a time: the activation
    gradients side by side, the weight gradients added.

    `update_mask` [B, n_chunks] as in inplace_layer (passed to the chunk
    loop's backward).  `conv_forward`: the forward-looking in-chunk
    convolution (forward_chunk_conv1d), Y[t, i] = sum_j conv_w[i, j]
    X0[t + j, i] inside t's chunk, whose gradients are
    dconv_w[i, j] = sum_t dY[t, i] X0[t + j, i] and
    dX0[s, i] = sum_j conv_w[i, j] dY[s - j, i], both over pairs inside one
    chunk.

    `W_init` [B, d, f] and `x0_halo` [B, K-1, d] (either may be None) resume
    rows as in inplace_layer: a row's first document continues from W_init
    and reads the halo before its first token unless doc_starts flags chunk
    0.  Then two more gradients are returned, dW_init [B, d, f] (the initial
    states') and dx0_halo [B, K-1, d] (the halo rows'), both zero for rows
    that start a document at chunk 0: the returned tuple has nine entries.
    """
    if W_init is not None or x0_halo is not None:
        return _resumed_layer_backward(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk, eta, dO, doc_starts,
                                       mode, update_mask, conv_forward, W_init, x0_halo)
    if doc_starts is not None:
        outs = []
        for b in range(len(H)):
            k = len(doc_starts[b])
            cuts = [c * chunk for c in range(k) if c == 0 or doc_starts[b][c]] + [min(k * chunk, len(H[b]))]
            um = lambda a, e: None if update_mask is None else [update_mask[b][a // chunk: (e + chunk - 1) // chunk]]
            parts = [layer_backward(H[b:b + 1, a:e], X0[b:b + 1, a:e], W_gate, W_up, W_down0, W_target, conv_w,
                                    chunk, eta, dO[b:b + 1, a:e], mode=mode, update_mask=um(a, e),
                                    conv_forward=conv_forward) for a, e in zip(cuts[:-1], cuts[1:])]
            outs.append((np.concatenate([q[0] for q in parts], axis=1), np.concatenate([q[1] for q in parts], axis=1),
                         *[sum(q[i] for q in parts) for i in range(2, 7)]))
        return (np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs]),
                *[sum(o[i] for o in outs) for i in range(2, 7)])
    H, X0, Wg, Wu, W0, Wt, cw, dO = map(_f64, (H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO))
    B, n, d = H.shape
    K = cw.shape[1]
    dH, dX0 = np.zeros_like(H), np.zeros_like(X0)
    dWg, dWu = np.zeros_like(Wg), np.zeros_like(Wu)
    dW0, dWt, dcw = np.zeros_like(W0), np.zeros_like(Wt), np.zeros_like(cw)
    for b in range(B):
        A = H[b] @ Wg.T
        U = H[b] @ Wu.T
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-A))
        Z = A * sg * U
        Y = forward_chunk_conv1d(X0[b], cw, chunk) if conv_forward else causal_depthwise_conv1d(X0[b], cw)
        V = Y @ Wt
        core = {"dot": chunk_core_backward, "mse": mse_core_backward}[mode]
        dZ, dV, dW0_b = core(Z, V, W0, chunk, eta, dO[b],
                             update_mask=None if update_mask is None else update_mask[b])
        dW0 += dW0_b
        dA = dZ * U * (sg * (1.0 + A * (1.0 - sg)))
        dU = dZ * (A * sg)
        dWg += dA.T @ H[b]
        dWu += dU.T @ H[b]
        dH[b] = dA @ Wg + dU @ Wu
        dWt += Y.T @ dV
        dY = dV @ Wt.T
        if conv_forward:
            for s0 in range(0, n, chunk):
                e0 = min(s0 + chunk, n)
                for j in range(min(K, e0 - s0)):      # tap j reads the token j steps ahead, inside the chunk
                    dcw[:, j] += np.sum(dY[s0: e0 - j] * X0[b, s0 + j: e0], axis=0)
                    dX0[b, s0 + j: e0] += cw[:, j] * dY[s0: e0 - j]
            continue
        for j in range(K):
            back = K - 1 - j              # tap j reads the token this many steps back
            if back >= n:
                continue
            dcw[:, j] += np.sum(dY[back:] * X0[b, : n - back], axis=0)
            dX0[b, : n - back] += cw[:, j] * dY[back:]
    return dH, dX0, dWg, dWu, dW0, dWt, dcw


def _resumed_layer_backward(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk, eta, dO, doc_starts, mode,
                            update_mask, conv_forward, W_init, x0_halo):
    """layer_backward for resumed rows (see there), one row at a time: a row
    that starts a document at chunk 0 is the plain backward; otherwise its
    first document is differentiated with the halo rows joined in front of
    X0 (the causal convolution reads them) and W_init as the chunk loop's
    initial state, and its later documents as independent rows."""
    H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO = map(
        _f64, (H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO))
    B, n, d = H.shape
    f, K = W_gate.shape[0], conv_w.shape[1]
    k = -(-n // chunk) if n else 0
    out = [np.zeros_like(H), np.zeros_like(X0), np.zeros_like(W_gate), np.zeros_like(W_up),
           np.zeros_like(W_down0), np.zeros_like(W_target), np.zeros_like(conv_w),
           np.zeros((B, d, f)), np.zeros((B, K - 1, d))]
    for b in range(B):
        flags = [bool(doc_starts[b][c]) if doc_starts is not None else False for c in range(k)]
        um = None if update_mask is None else update_mask[b]
        if k == 0:
            continue
        if flags[0]:
            g = layer_backward(H[b:b + 1], X0[b:b + 1], W_gate, W_up, W_down0, W_target, conv_w, chunk, eta,
                               dO[b:b + 1], doc_starts=[flags], mode=mode, update_mask=None if um is None else [um],
                               conv_forward=conv_forward)
            out[0][b], out[1][b] = g[0][0], g[1][0]
            for i in range(2, 7):
                out[i] += g[i]
            continue
        cut = next((c for c in range(1, k) if flags[c]), k)
        e = min(cut * chunk, n)
        # the first document: the halo in front of X0, W_init as the initial state
        halo = np.zeros((K - 1, d)) if x0_halo is None else _f64(x0_halo[b])
        Xf = np.concatenate([halo, X0[b, :e]])
        Hb, dOb = H[b, :e], dO[b, :e]
        A = Hb @ W_gate.T
        U = Hb @ W_up.T
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-A))
        Z = A * sg * U
        if conv_forward:
            Y = forward_chunk_conv1d(X0[b, :e], conv_w, chunk)
        else:
            Y = causal_depthwise_conv1d(Xf, conv_w)[K - 1:]
        V = Y @ W_target
        Wi = W_down0 if W_init is None else _f64(W_init[b])
        back = {"dot": chunk_core_backward, "mse": mse_core_backward}[mode]
        dZ, dV, dWi = back(Z, V, Wi, chunk, eta, dOb, update_mask=None if um is None else um[:cut])
        if W_init is not None:
            out[7][b] = dWi
        else:
            out[4] += dWi
        dA = dZ * U * (sg * (1.0 + A * (1.0 - sg)))
        dU = dZ * (A * sg)
        out[2] += dA.T @ Hb
        out[3] += dU.T @ Hb
        out[0][b, :e] = dA @ W_gate + dU @ W_up
        out[5] += Y.T @ dV
        dY = dV @ W_target.T
        if conv_forward:              # the window stays inside the chunk: the halo is never read
            for s0 in range(0, e, chunk):
                e0 = min(s0 + chunk, e)
                for j in range(min(K, e0 - s0)):
                    out[6][:, j] += np.sum(dY[s0: e0 - j] * X0[b, s0 + j: e0], axis=0)
                    out[1][b, s0 + j: e0] += conv_w[:, j] * dY[s0: e0 - j]
        else:                         # over the joined rows: row r of Xf is position r - (K-1)
            dXf = np.zeros_like(Xf)
            for j in range(K):
                out[6][:, j] += np.sum(dY * Xf[j: j + e], axis=0)
                dXf[j: j + e] += conv_w[:, j] * dY
            out[1][b, :e] = dXf[K - 1:]
            if x0_halo is not None:
                out[8][b] = dXf[:K - 1]
        if e < n:                     # the later documents: independent rows
            g = layer_backward(H[b:b + 1, e:], X0[b:b + 1, e:], W_gate, W_up, W_down0, W_target, conv_w, chunk,
                               eta, dO[b:b + 1, e:], doc_starts=[flags[cut:]], mode=mode,
                               update_mask=None if um is None else [um[cut:]], conv_forward=conv_forward)
            out[0][b, e:] = g[0][0]
            out[1][b, e:] = g[1][0]
            for i in range(2, 7):
                out[i] += g[i]
    return tuple(out)
