"""Float64 oracle of the LaCT SwiGLU fast-weight layer (test infrastructure only).

Sources: "Test-Time Training Done Right" review --
  * Preliminary §1, eq. (1): the update W <- W - eta grad L(f_W(k), v) and
    the apply o = f_W(q), with L usually the squared error;
  * LaCT Model Architecture §1, eq. (3): one gradient per chunk, of the loss
    summed over the chunk's tokens; all queries of the chunk share the
    updated weights; eq. (4): f_W(x) = W2 [SiLU(W1 x) * (W3 x)], no bias;
  * the same section, on ordering: update-then-apply within a chunk versus
    apply-then-update.
"ViT^3" review, Insight 2 and 3: one full-batch GD step per chunk, eta = 1.

Readings: the per-token loss is (1/2)||f_W(k_i) - v_i||^2, summed (no mean)
over the chunk; scalar eta; plain simultaneous GD on W1, W3, W2; layout
q, k, v [B, H, n, dh], W1, W3 [H, m, dh], W2 [H, dh, m], every (batch row,
head) with its own state.

Variants (LaCT Model Architecture §1, eq. (3) and the dot-product loss; §2,
fast-weight normalisation), each off by default:
  * per-token learning rates eta_i weighting each token's loss inside the
    gradient (eq. (3)), on top of the scalar eta;
  * the dot-product loss L = -f_W(k)^T v, whose gradient with respect to the
    output is -v in place of the residual f_W(k) - v;
  * L2 weight normalisation after each update, along each matrix's input
    dimension: every row of W1, W3 (over d_h) and of W2 (over the hidden
    width) is scaled to unit norm;
  * the Muon update rule (§2): each gradient replaced by Muon(g) ~ U V^T
    before the step.  The page names the Newton-Schulz iteration without its
    polynomial; the quintic iteration and its coefficients are those
    published with the Muon optimizer (K. Jordan et al., "Muon: An optimizer
    for hidden layers in neural networks", 2024): X = g / ||g||_F on the wide
    orientation, five times X <- a X + (b A + c A^2) X with A = X X^T.
"""
from __future__ import annotations

import numpy as np

from .inplace import silu

__all__ = ["swiglu_apply", "swiglu_loss", "swiglu_grads", "muon", "l2_normalize_rows", "lact_layer",
           "lact_backward"]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def swiglu_apply(x, W1, W3, W2):
    """f_W(x) row-wise (eq. (4)): x [C, dh] -> [C, dh]."""
    x = _f64(x)
    return (silu(x @ _f64(W1).T) * (x @ _f64(W3).T)) @ _f64(W2).T


def swiglu_loss(kc, vc, W1, W3, W2):
    """Chunk loss: sum over tokens of (1/2)||f_W(k_i) - v_i||^2."""
    R = swiglu_apply(kc, W1, W3, W2) - _f64(vc)
    return float(0.5 * np.sum(R * R))


def swiglu_grads(kc, vc, W1, W3, W2, eta_tok=None, loss="mse"):
    """Gradients (G1, G3, G2) of the chunk loss with respect to W1, W3, W2, by
    the chain rule written out by hand: swiglu_loss ("mse") or the dot-product
    loss sum_i -f_W(k_i)^T v_i ("dot"), each token's term weighted by
    eta_tok[i] when given (eq. (3))."""
    kc, vc, W1, W3, W2 = map(_f64, (kc, vc, W1, W3, W2))
    A = kc @ W1.T                     # [C, m]
    U = kc @ W3.T                     # [C, m]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-A))
    S = A * sig                       # silu(A)
    Hh = S * U                        # hidden [C, m]
    if loss == "mse":
        R = Hh @ W2.T - vc            # d loss / d output: the residual [C, dh]
    elif loss == "dot":
        R = -vc                       # d(-f^T v) / d f
    else:
        raise ValueError(f"unknown loss {loss!r}")
    if eta_tok is not None:
        R = R * _f64(eta_tok)[:, None]   # per-token learning rates weight each token's term
    G2 = R.T @ Hh                     # [dh, m]
    dH = R @ W2                       # [C, m]
    dU = dH * S
    dA = dH * U * (sig * (1.0 + A * (1.0 - sig)))   # silu'(a) = sig(a)(1 + a(1 - sig(a)))
    G3 = dU.T @ kc                    # [m, dh]
    G1 = dA.T @ kc                    # [m, dh]
    return G1, G3, G2


MUON_COEFFS = (3.4445, -4.7750, 2.0315)
MUON_STEPS = 5


def muon(g):
    """Newton-Schulz orthogonalisation of a gradient (see the module notes):
    g [r, c] is scaled to unit Frobenius norm, taken as [min, max] (transposed
    when r > c), iterated MUON_STEPS times X <- a X + (b A + c A^2) X with
    A = X X^T, and returned in g's orientation.  It approximates the polar
    factor U V^T of g = U S V^T."""
    g = _f64(g)
    a, b, c = MUON_COEFFS
    X = g / (np.linalg.norm(g) + 1e-7)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(MUON_STEPS):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T if tall else X


def l2_normalize_rows(W):
    """Each row of W scaled to unit L2 norm (the fast-weight normalisation of
    LaCT Model Architecture §2, along the input dimension of W [out, in])."""
    W = _f64(W)
    return W / np.linalg.norm(W, axis=-1, keepdims=True)


def lact_layer(q, k, v, W1, W3, W2, chunk, eta, order="update_then_apply", update_mask=None, eta_tok=None,
               loss="mse", weight_norm=False, use_muon=False):
    """LaCT layer over chunks.  q, k, v [B, H, n, dh]; W1, W3 [H, m, dh];
    W2 [H, dh, m].  Returns (O [B, H, n, dh], W1_f, W3_f [B, H, m, dh],
    W2_f [B, H, dh, m]).

    `update_mask` [n_chunks] (truthy entries), if given, takes the update step
    on the flagged chunks only; every chunk is applied.  With update-then-apply
    this is the strided block-wise causal mask of the review's section on the
    order of the apply and update operations (its video use updates on the
    clean chunks only).

    `eta_tok` [B, H, n] gives per-token learning rates, `loss` is "mse" or
    "dot", `weight_norm` L2-normalises the rows of each matrix after every
    update, and `use_muon` steps along Muon(g) instead of g (see the module
    notes)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    B, Hn, n, dh = q.shape
    O = np.empty_like(q)
    W1f = np.empty((B,) + W1.shape)
    W3f = np.empty((B,) + W3.shape)
    W2f = np.empty((B,) + W2.shape)
    for b in range(B):
        for h in range(Hn):
            w1, w3, w2 = W1[h].copy(), W3[h].copy(), W2[h].copy()
            for c, s in enumerate(range(0, n, chunk)):
                r = slice(s, min(s + chunk, n))
                if order == "apply_then_update":
                    O[b, h, r] = swiglu_apply(q[b, h, r], w1, w3, w2)
                if update_mask is None or update_mask[c]:
                    et = None if eta_tok is None else _f64(eta_tok)[b, h, r]
                    g1, g3, g2 = swiglu_grads(k[b, h, r], v[b, h, r], w1, w3, w2, et, loss)
                    if use_muon:
                        g1, g3, g2 = muon(g1), muon(g3), muon(g2)
                    w1, w3, w2 = w1 - eta * g1, w3 - eta * g3, w2 - eta * g2
                    if weight_norm:
                        w1, w3, w2 = l2_normalize_rows(w1), l2_normalize_rows(w3), l2_normalize_rows(w2)
                if order == "update_then_apply":
                    O[b, h, r] = swiglu_apply(q[b, h, r], w1, w3, w2)
                elif order != "apply_then_update":
                    raise ValueError(f"unknown order {order!r}")
            W1f[b, h], W3f[b, h], W2f[b, h] = w1, w3, w2
    return O, W1f, W3f, W2f


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _apply_backward(x, W1, W3, W2, dO):
    """Backward of o = f_W(x) (eq. (4)) for a chunk of rows x [C, dh] given
    dO [C, dh]: returns (dx [C, dh], dW1 [m, dh], dW3 [m, dh], dW2 [dh, m])."""
    A = x @ W1.T
    U = x @ W3.T
    sg = _sigmoid(A)
    S = A * sg                                 # silu(A)
    Hq = S * U
    dW2 = dO.T @ Hq
    dH = dO @ W2
    dA = dH * U * (sg * (1.0 + A * (1.0 - sg)))   # silu'(A)
    dU = dH * S
    return dA @ W1 + dU @ W3, dA.T @ x, dU.T @ x, dW2


def _update_backward(kc, vc, W1, W3, W2, gG1, gG3, gG2):
    """Backward of the chunk gradient (G1, G3, G2) = swiglu_grads(kc, vc, W)
    (the squared error summed over the chunk) given upstream gradients
    (gG1, gG3, gG2) of the same shapes: returns (dk [C, dh], dv [C, dh],
    dW1, dW3, dW2), the second-order terms through W included.  The forward
    it differentiates, in the order written in swiglu_grads:
      A = k W1^T, U = k W3^T, S = silu(A), Hh = S U, Y = Hh W2^T, R = Y - v,
      dH = R W2, dU = dH S, dA = dH U silu'(A),
      G2 = R^T Hh, G3 = dU^T k, G1 = dA^T k,
    with silu'(a) = s(a)(1 + a(1 - s(a))) and
    silu''(a) = s(a)(1 - s(a))(2 + a(1 - 2 s(a))), s the logistic function."""
    A = kc @ W1.T
    U = kc @ W3.T
    sg = _sigmoid(A)
    S = A * sg
    s1 = sg * (1.0 + A * (1.0 - sg))
    s2 = sg * (1.0 - sg) * (2.0 + A * (1.0 - 2.0 * sg))
    Hh = S * U
    R = Hh @ W2.T - vc
    dH = R @ W2
    dU = dH * S
    dA = dH * U * s1
    # G1 = dA^T k, G3 = dU^T k, G2 = R^T Hh
    ddA = kc @ gG1.T
    ddU = kc @ gG3.T
    dk = dA @ gG1 + dU @ gG3
    dR = Hh @ gG2.T
    dHh = R @ gG2
    # dA = dH U silu'(A); dU = dH S
    ddH = ddA * U * s1 + ddU * S
    dU_f = ddA * dH * s1
    dA_f = ddA * dH * U * s2
    dS = ddU * dH
    # dH = R W2
    dR = dR + ddH @ W2.T
    dW2 = R.T @ ddH
    # R = Y - v, Y = Hh W2^T
    dv = -dR
    dHh = dHh + dR @ W2
    dW2 = dW2 + dR.T @ Hh
    # Hh = S U, S = silu(A)
    dS = dS + dHh * U
    dU_f = dU_f + dHh * S
    dA_f = dA_f + dS * s1
    # A = k W1^T, U = k W3^T
    dk = dk + dA_f @ W1 + dU_f @ W3
    return dk, dv, dA_f.T @ kc, dU_f.T @ kc, dW2


def lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO, order="update_then_apply", update_mask=None):
    """Gradients of a loss that depends on the output O of lact_layer (the
    squared error, plain GD, optionally an update mask; no other variant) with
    respect to every input, given dO = dLoss/dO [B, H, n, dh]: returns (dq,
    dk, dv [B, H, n, dh], dW1, dW3 [H, m, dh], dW2 [H, dh, m]); the initial
    weights are shared by the batch rows, so their gradients add over rows.

    `update_mask` [n_chunks] as in lact_layer: a chunk whose flag is zero is
    applied but takes no step, so the state passes it unchanged and its keys
    and values reach nothing (their gradients are zero).

    The chain rule through the chunk loop (LaCT Model Architecture §1, eq.
    (3)-(4)), from the last chunk back.  With W_c the state chunk c's update
    starts from and W_{c+1} = W_c - eta G(W_c; k_c, v_c), let gW be the
    gradient with respect to the state after chunk c (zero after the last
    chunk).  Chunk c's queries are applied with W_{c+1} (update-then-apply) or
    W_c (apply-then-update): that apply's backward (_apply_backward) gives dq_c
    and adds its weight gradients to gW or to the result.  The update gives
    dLoss/dW_c = gW + (terms of G's backward with upstream -eta gW)
    (_update_backward), and dk_c, dv_c from the same backward."""
    q, k, v, dO = map(_f64, (q, k, v, dO))
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    B, Hn, n, dh = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dW1, dW3, dW2 = np.zeros_like(W1), np.zeros_like(W3), np.zeros_like(W2)
    bounds = [(s, min(s + chunk, n)) for s in range(0, n, chunk)]
    if order not in ("update_then_apply", "apply_then_update"):
        raise ValueError(f"unknown order {order!r}")
    for b in range(B):
        for h in range(Hn):
            states = []                          # the state each chunk's update starts from
            w = (W1[h].copy(), W3[h].copy(), W2[h].copy())
            for c, (s, e) in enumerate(bounds):
                states.append(w)
                if update_mask is None or update_mask[c]:
                    g1, g3, g2 = swiglu_grads(k[b, h, s:e], v[b, h, s:e], *w)
                    w = (w[0] - eta * g1, w[1] - eta * g3, w[2] - eta * g2)
            states.append(w)
            g = [np.zeros_like(W1[h]), np.zeros_like(W3[h]), np.zeros_like(W2[h])]   # gradient after the last chunk
            for c in range(len(bounds) - 1, -1, -1):
                s, e = bounds[c]
                if order == "update_then_apply":       # the queries see the updated state
                    dqc, a1, a3, a2 = _apply_backward(q[b, h, s:e], *states[c + 1], dO[b, h, s:e])
                    g = [g[0] + a1, g[1] + a3, g[2] + a2]
                if update_mask is None or update_mask[c]:
                    dkc, dvc, u1, u3, u2 = _update_backward(k[b, h, s:e], v[b, h, s:e], *states[c],
                                                            -eta * g[0], -eta * g[1], -eta * g[2])
                    g = [g[0] + u1, g[1] + u3, g[2] + u2]
                else:                                  # no step: the state passes through
                    dkc, dvc = np.zeros((e - s, dh)), np.zeros((e - s, dh))
                if order == "apply_then_update":       # the queries see the state before the update
                    dqc, a1, a3, a2 = _apply_backward(q[b, h, s:e], *states[c], dO[b, h, s:e])
                    g = [g[0] + a1, g[1] + a3, g[2] + a2]
                dq[b, h, s:e], dk[b, h, s:e], dv[b, h, s:e] = dqc, dkc, dvc
            dW1[h] += g[0]
            dW3[h] += g[1]
            dW2[h] += g[2]
    return dq, dk, dv, dW1, dW3, dW2
