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

__all__ = ["swiglu_apply", "swiglu_loss", "swiglu_grads", "muon", "l2_normalize_rows", "lact_layer"]


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
