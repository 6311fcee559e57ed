"""Pins of the In-Place TTT oracle against things other than itself.

Each test fixes the oracle to a library routine, a hand-derived fixture, a
closed form, a brute force written a different way, finite differences of
the loss definitions, or an invariant the pages state.  All run on the CPU.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import inplace as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(rng, n, d, f, K=4):
    H = rng.standard_normal((n, d))
    X0 = rng.standard_normal((n, d))
    Wg = rng.standard_normal((f, d)) / np.sqrt(d)
    Wu = rng.standard_normal((f, d)) / np.sqrt(d)
    W0 = rng.standard_normal((d, f)) / np.sqrt(f)
    Wt = rng.standard_normal((d, d)) / np.sqrt(d)
    cw = rng.standard_normal((d, K)) * 0.5
    return H, X0, Wg, Wu, W0, Wt, cw


# ---------------------------------------------------------------- conv / producers

def test_conv_golden_hand_derived():
    g = _golden("conv_tiny.json")
    Y = orc.causal_depthwise_conv1d(np.array(g["X0"]), np.array(g["conv_w"]))
    np.testing.assert_array_equal(Y, np.array(g["Y"], dtype=np.float64))


@pytest.mark.parametrize("n,d,K", [(17, 5, 4), (3, 4, 4), (9, 3, 1), (6, 2, 7)])
def test_conv_matches_torch_conv1d(n, d, K):
    rng = _rng(n * 100 + K)
    X0 = rng.standard_normal((2, n, d))
    w = rng.standard_normal((d, K))
    ref = F.conv1d(torch.from_numpy(X0).transpose(1, 2), torch.from_numpy(w)[:, None, :],
                   groups=d, padding=K - 1)[..., :n].transpose(1, 2).numpy()
    np.testing.assert_allclose(orc.causal_depthwise_conv1d(X0, w), ref, rtol=1e-13, atol=1e-13)


def test_conv_identity_tap_reduces_to_x0():
    # a one-hot kernel on the current-token tap with W_target = I gives V^ = X0
    rng = _rng(3)
    X0 = rng.standard_normal((11, 6))
    w = np.zeros((6, 4))
    w[:, 3] = 1.0
    np.testing.assert_array_equal(orc.target_values(X0, w, np.eye(6)), X0)
    # one-hot one step back: the previous token (zero at t = 0)
    w = np.zeros((6, 4))
    w[:, 2] = 1.0
    V = orc.target_values(X0, w, np.eye(6))
    np.testing.assert_array_equal(V[1:], X0[:-1])
    np.testing.assert_array_equal(V[0], 0.0)


def test_target_orientation_is_din_dout():
    rng = _rng(4)
    X0 = rng.standard_normal((5, 3))
    w = np.zeros((3, 4))
    w[:, 3] = 1.0
    Wt = rng.standard_normal((3, 7))         # non-square: only Y @ Wt is defined
    assert orc.target_values(X0, w, Wt).shape == (5, 7)
    np.testing.assert_allclose(orc.target_values(X0, w, Wt), X0 @ Wt, rtol=1e-14)


def test_gated_intermediate_matches_torch():
    rng = _rng(5)
    H = rng.standard_normal((13, 8))
    Wg = rng.standard_normal((11, 8))
    Wu = rng.standard_normal((11, 8))
    Ht = torch.from_numpy(H)
    ref = (F.silu(F.linear(Ht, torch.from_numpy(Wg))) * F.linear(Ht, torch.from_numpy(Wu))).numpy()
    np.testing.assert_allclose(orc.gated_intermediate(H, Wg, Wu), ref, rtol=1e-13, atol=1e-14)


def test_silu_special_values():
    np.testing.assert_array_equal(orc.silu(np.array([0.0])), [0.0])
    np.testing.assert_allclose(orc.silu(np.array([50.0, -50.0])), [50.0, -50.0 * np.exp(-50.0)], rtol=1e-12)
    np.testing.assert_allclose(orc.silu(np.array([1.0])), [1.0 / (1.0 + np.exp(-1.0))], rtol=1e-15)
    assert np.isfinite(orc.silu(np.array([-1000.0]))).all()


# ---------------------------------------------------------------- hand-derived recursions

@pytest.mark.parametrize("name", ["scalar_dot.json", "scalar_mse.json", "matrix_dot.json"])
def test_chunk_loop_golden(name):
    g = _golden(name)
    O, W = orc.chunk_apply_update(np.array(g["Z"], float), np.array(g["Vhat"], float),
                                  np.array(g["W0"], float), g["chunk"], g["eta"], g["mode"])
    np.testing.assert_allclose(O, np.array(g["O"], float), rtol=0, atol=1e-14)
    np.testing.assert_allclose(W, np.array(g["W_final"], float), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- brute force

def _dual_form_dot(Z, V, W0, C, eta):
    """Token-by-token dual form written with explicit loops: the output of token
    t is Z_t W0^T plus eta times the sum over every token s of an earlier chunk
    of (Z_t . Z_s) V_s.  No prefix sums, no matrix state."""
    n, f = Z.shape
    d = V.shape[1]
    O = np.zeros((n, d))
    for t in range(n):
        for i in range(d):
            acc = 0.0
            for j in range(f):
                acc += Z[t, j] * W0[i, j]
            O[t, i] = acc
        for s in range(n):
            if s // C < t // C:
                dot = sum(Z[t, j] * Z[s, j] for j in range(f))
                for i in range(d):
                    O[t, i] += eta * dot * V[s, i]
    Wf = W0.copy()
    for s in range(n):
        for i in range(d):
            for j in range(f):
                Wf[i, j] += eta * V[s, i] * Z[s, j]
    return O, Wf


@pytest.mark.parametrize("n,C", [(12, 4), (12, 1), (12, 12), (10, 4), (7, 3)])
def test_dot_equals_block_causal_dual_brute_force(n, C):
    rng = _rng(n * 31 + C)
    d, f = 3, 5
    Z = rng.standard_normal((n, f))
    V = rng.standard_normal((n, d))
    W0 = rng.standard_normal((d, f))
    O, W = orc.chunk_apply_update(Z, V, W0, C, 0.3, "dot")
    Ob, Wb = _dual_form_dot(Z, V, W0, C, 0.3)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Wb, rtol=1e-12, atol=1e-12)


def _online_gd_mse(Z, V, W0, eta):
    """Per-token TTT with the squared error (chunk of one token), scalar loops."""
    n, f = Z.shape
    d = V.shape[1]
    W = W0.copy()
    O = np.zeros((n, d))
    for t in range(n):
        for i in range(d):
            O[t, i] = sum(W[i, j] * Z[t, j] for j in range(f))
        for i in range(d):
            e = O[t, i] - V[t, i]
            for j in range(f):
                W[i, j] -= eta * e * Z[t, j]
    return O, W


def test_mse_chunk_one_is_per_token_online_gd():
    rng = _rng(7)
    Z = rng.standard_normal((9, 4)) * 0.5
    V = rng.standard_normal((9, 3))
    W0 = rng.standard_normal((3, 4))
    O, W = orc.chunk_apply_update(Z, V, W0, 1, 0.2, "mse")
    Ob, Wb = _online_gd_mse(Z, V, W0, 0.2)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Wb, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- gradients by finite differences

@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_gradients_match_finite_differences(mode):
    rng = _rng(11)
    C, d, f = 6, 3, 4
    Z = rng.standard_normal((C, f))
    V = rng.standard_normal((C, d))
    W = rng.standard_normal((d, f))
    loss = {"dot": orc.loss_dot, "mse": orc.loss_mse}[mode]
    grad = {"dot": orc.grad_dot, "mse": orc.grad_mse}[mode](W, Z, V)
    h = 1e-6
    fd = np.zeros_like(W)
    for i in range(d):
        for j in range(f):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            fd[i, j] = (loss(Wp, Z, V) - loss(Wm, Z, V)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-8)


def test_gradients_match_autograd():
    rng = _rng(12)
    C, d, f = 5, 4, 6
    Z = torch.from_numpy(rng.standard_normal((C, f)))
    V = torch.from_numpy(rng.standard_normal((C, d)))
    W = torch.from_numpy(rng.standard_normal((d, f))).requires_grad_(True)
    (-(Z @ W.T * V).sum()).backward()
    np.testing.assert_allclose(orc.grad_dot(W.detach().numpy(), Z.numpy(), V.numpy()), W.grad.numpy(), rtol=1e-13)
    W.grad = None
    (((Z @ W.T - V) ** 2).sum() / (2 * C)).backward()
    np.testing.assert_allclose(orc.grad_mse(W.detach().numpy(), Z.numpy(), V.numpy()), W.grad.numpy(), rtol=1e-12)


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_eta_zero_is_plain_gated_mlp(mode):
    rng = _rng(13)
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, 24, 6, 10)
    O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, 8, 0.0, mode)
    ref = (F.silu(torch.from_numpy(H) @ torch.from_numpy(Wg).T) * (torch.from_numpy(H) @ torch.from_numpy(Wu).T)) \
        @ torch.from_numpy(W0).T
    np.testing.assert_allclose(O[0], ref.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(Wf[0], W0)


def test_chunk_equal_sequence_is_one_full_batch_step():
    rng = _rng(14)
    n, d, f = 16, 4, 7
    Z = rng.standard_normal((n, f))
    V = rng.standard_normal((n, d))
    W0 = rng.standard_normal((d, f))
    O, W = orc.chunk_apply_update(Z, V, W0, n, 0.25, "dot")
    np.testing.assert_allclose(O, np.einsum("tf,df->td", Z, W0), rtol=1e-13)
    np.testing.assert_allclose(W, W0 + 0.25 * np.einsum("ti,tj->ij", V, Z), rtol=1e-13)
    O, W = orc.chunk_apply_update(Z, V, W0, n, 0.25, "mse")
    E = np.einsum("tf,df->td", Z, W0) - V
    np.testing.assert_allclose(O, np.einsum("tf,df->td", Z, W0), rtol=1e-13)
    np.testing.assert_allclose(W, W0 - 0.25 / n * np.einsum("ti,tj->ij", E, Z), rtol=1e-13)


def test_mse_orthogonal_keys_reach_target_in_one_step():
    # chunk = d_ff, Z = sqrt(C) Q with Q orthogonal, V^ = Z W*^T, eta = 1:
    # W - (1/C)(W - W*) Z^T Z = W*
    rng = _rng(15)
    f, d = 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((f, f)))
    Z = np.sqrt(f) * Q
    Wstar = rng.standard_normal((d, f))
    V = Z @ Wstar.T
    W0 = rng.standard_normal((d, f))
    _, W = orc.chunk_apply_update(Z, V, W0, f, 1.0, "mse")
    np.testing.assert_allclose(W, Wstar, rtol=1e-12, atol=1e-12)


def test_mse_eta_scaling_identity():
    # eta * K^T (K W - V) = K~^T (K~ W - V~) with K~ = sqrt(eta) K, V~ = sqrt(eta) V
    rng = _rng(16)
    Z = rng.standard_normal((12, 5))
    V = rng.standard_normal((12, 3))
    W0 = rng.standard_normal((3, 5))
    eta = 0.37
    O1, W1 = orc.chunk_apply_update(Z, V, W0, 4, eta, "mse")
    O2, W2 = orc.chunk_apply_update(np.sqrt(eta) * Z, np.sqrt(eta) * V, W0, 4, 1.0, "mse")
    np.testing.assert_allclose(W1, W2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O1 * np.sqrt(eta), O2, rtol=1e-12, atol=1e-13)


def test_prefix_form_equals_sequential():
    rng = _rng(17)
    for n, C in [(32, 8), (30, 8), (5, 5), (9, 1)]:
        Z = rng.standard_normal((n, 6))
        V = rng.standard_normal((n, 4))
        W0 = rng.standard_normal((4, 6))
        O1, W1 = orc.chunk_apply_update(Z, V, W0, C, 0.05, "dot")
        O2, W2 = orc.chunk_prefix_form(Z, V, W0, C, 0.05)
        np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(W1, W2, rtol=1e-12, atol=1e-12)


def test_dot_is_affine_in_eta():
    rng = _rng(18)
    Z = rng.standard_normal((20, 6))
    V = rng.standard_normal((20, 4))
    W0 = rng.standard_normal((4, 6))
    O0, _ = orc.chunk_apply_update(Z, V, W0, 5, 0.0, "dot")
    O1, _ = orc.chunk_apply_update(Z, V, W0, 5, 0.1, "dot")
    O2, _ = orc.chunk_apply_update(Z, V, W0, 5, 0.2, "dot")
    np.testing.assert_allclose(O2 - 2 * O1 + O0, 0.0, atol=1e-12)


# ---------------------------------------------------------------- causality, batch, resume

@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_causality_future_targets_do_not_reach_past_chunks(mode):
    rng = _rng(19)
    n, C, d, f = 32, 8, 4, 6
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f)
    O, _ = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    for c in range(n // C):
        X0p = X0.copy()
        X0p[c * C:] += rng.standard_normal(X0p[c * C:].shape)     # changes V^ of chunks >= c
        Hp = H.copy()
        Hp[(c + 1) * C:] += rng.standard_normal(Hp[(c + 1) * C:].shape)  # changes Z of chunks > c
        Op, _ = orc.inplace_layer(Hp[None], X0p[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
        np.testing.assert_array_equal(Op[0, : (c + 1) * C], O[0, : (c + 1) * C])
        if c + 1 < n // C:
            assert not np.array_equal(Op[0, (c + 1) * C:], O[0, (c + 1) * C:])


def test_layer_batch_rows_are_independent_documents():
    rng = _rng(20)
    n, C, d, f = 16, 4, 3, 5
    H = rng.standard_normal((3, n, d))
    X0 = rng.standard_normal((3, n, d))
    _, _, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f)
    O, Wf = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, 0.2, "dot")
    for b in range(3):
        Ob, Wb = orc.inplace_layer(H[b:b + 1], X0[b:b + 1], Wg, Wu, W0, Wt, cw, C, 0.2, "dot")
        np.testing.assert_array_equal(O[b], Ob[0])
        np.testing.assert_array_equal(Wf[b], Wb[0])


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_resume_at_chunk_boundary_with_conv_halo(mode):
    rng = _rng(21)
    n, C, d, f, K = 24, 6, 4, 5, 4
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f, K)
    O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    s = 2 * C
    O1, W1 = orc.inplace_layer(H[None, :s], X0[None, :s], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    O2, W2 = orc.inplace_layer(H[None, s:], X0[None, s:], Wg, Wu, W1[0], Wt, cw, C, 0.1, mode,
                               x0_halo=X0[None, s - (K - 1): s])
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=1), O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W2, Wf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_packed_documents_equal_separate_runs(mode):
    """Documents packed into one row (Method §3: the fast weight resets at document boundaries, and
    nothing of one document reaches the next) give exactly what separate rows give: outputs of each
    document, and the last document's final state."""
    rng = _rng(25)
    C, d, f, K = 4, 3, 5, 4
    docs = [3, 1, 2]                                    # chunks per document
    n = C * sum(docs)
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f, K)
    starts = np.zeros((1, n // C), dtype=bool)
    starts[0, np.cumsum([0] + docs[:-1])] = True
    O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode, doc_starts=starts)
    row = 0
    for nc in docs:
        r = slice(row, row + nc * C)
        Od, Wd = orc.inplace_layer(H[None, r], X0[None, r], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
        np.testing.assert_allclose(O[0, r], Od[0], rtol=1e-12, atol=1e-12)
        row += nc * C
    np.testing.assert_allclose(Wf, Wd, rtol=1e-12, atol=1e-12)
    # flags only at chunk 0 (or none) are the single-document row
    first = np.zeros_like(starts)
    first[0, 0] = True
    O1, W1 = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode, doc_starts=first)
    O2, W2 = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(W1, W2)


def test_document_at_every_chunk_is_the_plain_mlp():
    """A document starting at every chunk: each chunk sees W_down0 (the plain gated MLP of eq. (1)), and the
    final state is one dot step on the last chunk alone, with its convolution zero-padded at its own start."""
    rng = _rng(26)
    n, C, d, f, K = 12, 4, 3, 5, 3
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f, K)
    starts = np.ones((1, n // C), dtype=bool)
    O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.3, "dot", doc_starts=starts)
    Zfull = F.silu(torch.from_numpy(H @ Wg.T)).numpy() * (H @ Wu.T)
    np.testing.assert_allclose(O[0], Zfull @ W0.T, rtol=1e-12, atol=1e-12)
    last = slice(n - C, n)
    Ylast = np.zeros((C, d))                            # conv of the last chunk alone, by hand
    for t in range(C):
        for j in range(K):
            src = t - (K - 1) + j
            if src >= 0:
                Ylast[t] += cw[:, j] * X0[n - C + src]
    np.testing.assert_allclose(Wf[0], W0 + 0.3 * (Ylast @ Wt).T @ Zfull[last], rtol=1e-12, atol=1e-12)


def test_layer_matches_whole_sequence_composition():
    # streaming per chunk must equal forming Z and V^ over the whole sequence first
    rng = _rng(22)
    n, C, d, f = 40, 8, 5, 7
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f)
    Z = orc.gated_intermediate(H, Wg, Wu)
    V = orc.target_values(X0, cw, Wt)
    for mode in ("dot", "mse"):
        O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.05, mode)
        O2, W2 = orc.chunk_apply_update(Z, V, W0, C, 0.05, mode)
        np.testing.assert_allclose(O[0], O2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Wf[0], W2, rtol=1e-12, atol=1e-12)


def test_max_chunks_gives_the_prefix_of_the_run():
    rng = _rng(23)
    n, C, d, f = 32, 8, 3, 4
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f)
    O, _ = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, "mse")
    Op, Wp = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, "mse", max_chunks=2)
    _, W2 = orc.inplace_layer(H[None, : 2 * C], X0[None, : 2 * C], Wg, Wu, W0, Wt, cw, C, 0.1, "mse")
    np.testing.assert_array_equal(Op[0], O[0, : 2 * C])
    np.testing.assert_array_equal(Wp, W2)


def test_empty_sequence():
    rng = _rng(24)
    _, _, Wg, Wu, W0, Wt, cw = _problem(rng, 4, 3, 5)
    O, Wf = orc.inplace_layer(np.zeros((2, 0, 3)), np.zeros((2, 0, 3)), Wg, Wu, W0, Wt, cw, 4, 0.1, "dot")
    assert O.shape == (2, 0, 3)
    np.testing.assert_array_equal(Wf, np.broadcast_to(W0, (2, 3, 5)))


# ---------------------------------------------------------------- planted mistakes must be caught

def test_planted_mistakes_fail_the_pins(monkeypatch):
    """Each plausible mistake (inclusive prefix, wrong sign, missing 1/C,
    transposed target) makes at least one pin fail."""
    g = _golden("matrix_dot.json")
    Z, V, W0 = (np.array(g[k], float) for k in ("Z", "Vhat", "W0"))

    def inclusive(Z, V, W0, chunk, eta, mode):
        W = W0.copy()
        O = np.empty((Z.shape[0], W0.shape[0]))
        for s in range(0, Z.shape[0], chunk):
            r = slice(s, s + chunk)
            W = W + eta * V[r].T @ Z[r]
            O[r] = Z[r] @ W.T
        return O, W
    O, _ = inclusive(Z, V, W0, g["chunk"], g["eta"], "dot")
    assert not np.allclose(O, np.array(g["O"], float))

    O, W = orc.chunk_apply_update(Z, -V, W0, g["chunk"], g["eta"], "dot")   # wrong sign
    assert not np.allclose(W, np.array(g["W_final"], float))

    gm = _golden("scalar_mse.json")
    Zs, Vs, Ws = (np.array(gm[k], float) for k in ("Z", "Vhat", "W0"))
    monkeypatch.setitem(orc._GRADS, "mse", lambda W, Zc, Vc: (Zc @ W.T - Vc).T @ Zc)  # no 1/C
    _, W = orc.chunk_apply_update(Zs, Vs, Ws, gm["chunk"], gm["eta"], "mse")
    assert not np.allclose(W, np.array(gm["W_final"], float))


def test_forward_conv_next_token_example():
    """The review's next-token target (Method §2): W_target = I and a kernel that weights only the next token give
    each token the next token's embedding; with the forward-looking in-chunk reading, a chunk's last token gets
    zero (the next token belongs to the next chunk)."""
    rng = _rng(30)
    n, C, d, K = 12, 4, 3, 4
    X0 = rng.standard_normal((n, d))
    cw = np.zeros((d, K))
    cw[:, 1] = 1.0
    V = orc.forward_chunk_conv1d(X0, cw, C) @ np.eye(d)
    want = np.zeros((n, d))
    for t in range(n):
        if (t + 1) % C:
            want[t] = X0[t + 1]
    np.testing.assert_array_equal(V, want)


@pytest.mark.parametrize("n,C,d,K", [(12, 4, 3, 4), (10, 5, 2, 3), (8, 8, 4, 1)])
def test_forward_conv_matches_torch_per_chunk(n, C, d, K):
    """Per chunk, torch's depthwise conv1d (a cross-correlation) with K-1 zeros appended on the right."""
    rng = _rng(31)
    X0 = rng.standard_normal((n, d))
    cw = rng.standard_normal((d, K))
    Y = orc.forward_chunk_conv1d(X0, cw, C)
    for s in range(0, n, C):
        x = torch.from_numpy(X0[s:s + C].T.copy())[None]                      # [1, d, C]
        ref = F.conv1d(F.pad(x, (0, K - 1)), torch.from_numpy(cw)[:, None, :], groups=d)[0].T.numpy()
        np.testing.assert_allclose(Y[s:s + C], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_forward_conv_layer_is_causal_per_chunk_and_composes(mode):
    """With the forward-looking target, chunk c's update reads chunk c's tokens only: changing X0 in chunks >= c
    leaves the outputs of chunks <= c unchanged.  The streamed layer equals the chunk loop on the whole-sequence
    target."""
    rng = _rng(32)
    n, C, d, f, K = 24, 6, 4, 5, 4
    H, X0, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f, K)
    O, Wf = orc.inplace_layer(H[None], X0[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode, conv_forward=True)
    Z = orc.gated_intermediate(H, Wg, Wu)
    V = orc.forward_chunk_conv1d(X0, cw, C) @ Wt
    O2, W2 = orc.chunk_apply_update(Z, V, W0, C, 0.1, mode)
    np.testing.assert_allclose(O[0], O2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wf[0], W2, rtol=1e-12, atol=1e-12)
    for c in range(n // C):
        X0p = X0.copy()
        X0p[c * C:] += rng.standard_normal(X0p[c * C:].shape)
        Op, _ = orc.inplace_layer(H[None], X0p[None], Wg, Wu, W0, Wt, cw, C, 0.1, mode, conv_forward=True)
        np.testing.assert_array_equal(Op[0, : (c + 1) * C], O[0, : (c + 1) * C])


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_resume_rows_with_their_own_states(mode):
    """Two rows resumed at a chunk boundary, each from its own state (W_init, the first call's W_final) and its
    own last K-1 rows of X0 (x0_halo): the two calls equal the single call.  A document flagged at the resume
    point ignores both and starts from W_down0 with zeros."""
    rng = _rng(33)
    B, n, C, d, f, K = 2, 24, 6, 4, 5, 4
    H = rng.standard_normal((B, n, d))
    X0 = rng.standard_normal((B, n, d))
    _, _, Wg, Wu, W0, Wt, cw = _problem(rng, n, d, f, K)
    O, Wf = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    s = 2 * C
    O1, W1 = orc.inplace_layer(H[:, :s], X0[:, :s], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    O2, W2 = orc.inplace_layer(H[:, s:], X0[:, s:], Wg, Wu, W0, Wt, cw, C, 0.1, mode, W_init=W1,
                               x0_halo=X0[:, s - (K - 1): s])
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=1), O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W2, Wf, rtol=1e-12, atol=1e-12)
    starts = np.zeros((B, (n - s) // C), dtype=bool)
    starts[1, 0] = True
    O3, W3 = orc.inplace_layer(H[:, s:], X0[:, s:], Wg, Wu, W0, Wt, cw, C, 0.1, mode, W_init=W1,
                               x0_halo=X0[:, s - (K - 1): s], doc_starts=starts)
    O4, W4 = orc.inplace_layer(H[1:, s:], X0[1:, s:], Wg, Wu, W0, Wt, cw, C, 0.1, mode)
    np.testing.assert_array_equal(O3[0], O2[0])
    np.testing.assert_allclose(O3[1], O4[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W3[1], W4[0], rtol=1e-12, atol=1e-12)


def _torch_dot_chunk_loop(Z, V, W0, C, eta):
    """The dot-objective chunk loop in torch float64 (apply, then update), for autograd."""
    W = W0
    outs = []
    for s in range(0, Z.shape[0], C):
        outs.append(Z[s:s + C] @ W.T)
        W = W + eta * (V[s:s + C].T @ Z[s:s + C])
    return torch.cat(outs)


@pytest.mark.parametrize("n,C", [(12, 4), (10, 3), (8, 8)])
def test_core_backward_matches_autograd(n, C):
    """The backward of the dot chunk loop against torch autograd of the same loop in float64, for a random
    upstream dO; includes a ragged last chunk and a single chunk."""
    rng = _rng(50)
    d, f, eta = 3, 5, 0.3
    Z, V, W0, dO = (rng.standard_normal(s) for s in ((n, f), (n, d), (d, f), (n, d)))
    dZ, dV, dW0 = orc.chunk_core_backward(Z, V, W0, C, eta, dO)
    tz, tv, tw = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0))
    (_torch_dot_chunk_loop(tz, tv, tw, C, eta) * torch.from_numpy(dO)).sum().backward()
    grad = lambda t: np.zeros(t.shape) if t.grad is None else t.grad.numpy()   # one chunk: V^ reaches no output
    np.testing.assert_allclose(dZ, grad(tz), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dV, grad(tv), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW0, grad(tw), rtol=1e-12, atol=1e-12)


def test_core_backward_finite_differences():
    """Central differences of <O, dO> for a few entries of Z, V^ and W0."""
    rng = _rng(51)
    n, C, d, f, eta = 9, 3, 2, 3, 0.4
    Z, V, W0, dO = (rng.standard_normal(s) for s in ((n, f), (n, d), (d, f), (n, d)))
    dZ, dV, dW0 = orc.chunk_core_backward(Z, V, W0, C, eta, dO)
    L = lambda Z_, V_, W_: float(np.sum(orc.chunk_apply_update(Z_, V_, W_, C, eta, "dot")[0] * dO))
    h = 1e-6
    for arr, grad, which in ((Z, dZ, 0), (V, dV, 1), (W0, dW0, 2)):
        for idx in [(0, 0), tuple(s - 1 for s in arr.shape), (arr.shape[0] // 2, 1)]:
            p, m = [Z.copy(), V.copy(), W0.copy()], [Z.copy(), V.copy(), W0.copy()]
            p[which][idx] += h
            m[which][idx] -= h
            assert abs((L(*p) - L(*m)) / (2 * h) - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx]))


def _torch_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta):
    """The dot-objective layer written with torch float64 primitives (F.silu, grouped conv1d with left padding,
    the chunk loop), for autograd."""
    import torch.nn.functional as F
    B, n, d = H.shape
    K = cw.shape[1]
    Z = F.silu(H @ Wg.T) * (H @ Wu.T)
    Y = F.conv1d(F.pad(X0.transpose(1, 2), (K - 1, 0)), cw[:, None, :], groups=d).transpose(1, 2)
    V = Y @ Wt
    return torch.stack([_torch_dot_chunk_loop(Z[b], V[b], W0, C, eta) for b in range(B)])


@pytest.mark.parametrize("n,C,K", [(12, 4, 3), (10, 5, 1), (9, 3, 4)])
def test_layer_backward_matches_autograd(n, C, K):
    """Every gradient of the whole dot layer (producers, causal conv, target projection, chunk loop) against torch
    autograd of the same layer built from torch's own silu and grouped conv1d, two batch rows sharing the weights."""
    rng = _rng(52)
    B, d, f, eta = 2, 3, 5, 0.2
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    H, X0, Wg, Wu, W0, Wt, cw = (rng.standard_normal(s) * 0.7 for s in shapes)
    dO = rng.standard_normal((B, n, d))
    ours = orc.layer_backward(H, X0, Wg, Wu, W0, Wt, cw, C, eta, dO)
    ts = [torch.tensor(a, requires_grad=True) for a in (H, X0, Wg, Wu, W0, Wt, cw)]
    (_torch_layer(*ts, C, eta) * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-11)
    # the forward it differentiates is the oracle's own layer
    O, _ = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "dot")
    np.testing.assert_allclose(O, _torch_layer(*[t.detach() for t in ts], C, eta).numpy(), rtol=1e-12, atol=1e-12)


def test_layer_backward_finite_differences():
    """Central differences of <O, dO> through the oracle's layer for entries of the conv taps, W_target, W_gate and
    X0 (the entries reached only through the producers and the convolution)."""
    rng = _rng(53)
    B, n, C, d, f, K, eta = 1, 8, 4, 2, 3, 3, 0.3
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(s) * 0.7 for s in shapes]
    dO = rng.standard_normal((B, n, d))
    grads = orc.layer_backward(*args, C, eta, dO)
    L = lambda a: float(np.sum(orc.inplace_layer(*a, C, eta, "dot")[0] * dO))
    h = 1e-6
    for which, idx in ((6, (1, 0)), (6, (0, 2)), (5, (1, 0)), (2, (2, 1)), (1, (0, 2, 1)), (1, (0, 7, 0))):
        p = [a.copy() for a in args]
        m = [a.copy() for a in args]
        p[which][idx] += h
        m[which][idx] -= h
        g = grads[which][idx]
        assert abs((L(p) - L(m)) / (2 * h) - g) < 1e-6 * max(1.0, abs(g)), (which, idx)


def _torch_mse_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta):
    """The MSE-objective layer written with torch float64 primitives (F.silu, grouped conv1d with left padding, the
    MSE chunk loop), for autograd."""
    import torch.nn.functional as F
    B, n, d = H.shape
    K = cw.shape[1]
    Z = F.silu(H @ Wg.T) * (H @ Wu.T)
    Y = F.conv1d(F.pad(X0.transpose(1, 2), (K - 1, 0)), cw[:, None, :], groups=d).transpose(1, 2)
    V = Y @ Wt
    return torch.stack([_torch_mse_chunk_loop(Z[b], V[b], W0, C, eta) for b in range(B)])


@pytest.mark.parametrize("n,C,K", [(12, 4, 3), (10, 5, 1), (9, 3, 4), (8, 8, 2)])
def test_mse_layer_backward_matches_autograd(n, C, K):
    """Every gradient of the whole MSE-objective layer (producers, causal conv, target projection, the in-order
    MSE scan) against torch autograd of the same layer built from torch's own silu and grouped conv1d, two batch
    rows sharing the weights; one case is a single chunk, where the targets reach no output (dX0, dW_target and
    the conv taps' gradients are exactly zero)."""
    rng = _rng(56)
    B, d, f, eta = 2, 3, 5, 0.6
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    H, X0, Wg, Wu, W0, Wt, cw = (rng.standard_normal(s) * 0.7 for s in shapes)
    dO = rng.standard_normal((B, n, d))
    ours = orc.layer_backward(H, X0, Wg, Wu, W0, Wt, cw, C, eta, dO, mode="mse")
    ts = [torch.tensor(a, requires_grad=True) for a in (H, X0, Wg, Wu, W0, Wt, cw)]
    (_torch_mse_layer(*ts, C, eta) * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        want = np.zeros(t.shape) if t.grad is None else t.grad.numpy()
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    if n == C:
        assert not ours[1].any() and not ours[5].any() and not ours[6].any()
    O, _ = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "mse")
    np.testing.assert_allclose(O, _torch_mse_layer(*[t.detach() for t in ts], C, eta).numpy(), rtol=1e-12,
                               atol=1e-12)


def test_mse_layer_backward_finite_differences_and_documents():
    """Central differences of <O, dO> through the oracle's MSE layer for entries of the conv taps, W_target,
    W_gate, W_down0 and X0; and with packed documents, the row's gradients equal those of its documents taken as
    separate rows (activation gradients side by side, weight gradients added)."""
    rng = _rng(57)
    B, n, C, d, f, K, eta = 1, 8, 4, 2, 3, 3, 0.5
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(s) * 0.7 for s in shapes]
    dO = rng.standard_normal((B, n, d))
    grads = orc.layer_backward(*args, C, eta, dO, mode="mse")
    L = lambda a: float(np.sum(orc.inplace_layer(*a, C, eta, "mse")[0] * dO))
    h = 1e-6
    for which, idx in ((6, (1, 0)), (6, (0, 2)), (5, (1, 0)), (2, (2, 1)), (4, (1, 2)), (1, (0, 2, 1))):
        p = [a.copy() for a in args]
        m = [a.copy() for a in args]
        p[which][idx] += h
        m[which][idx] -= h
        g = grads[which][idx]
        assert abs((L(p) - L(m)) / (2 * h) - g) < 1e-6 * max(1.0, abs(g)), (which, idx)
    # documents of 2 and 1 chunks in one row of 3 chunks
    n2 = 12
    shapes = ((1, n2, d), (1, n2, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(s) * 0.7 for s in shapes]
    dO = rng.standard_normal((1, n2, d))
    packed = orc.layer_backward(*args, C, eta, dO, doc_starts=np.array([[1, 0, 1]]), mode="mse")
    first = orc.layer_backward(args[0][:, :8], args[1][:, :8], *args[2:], C, eta, dO[:, :8], mode="mse")
    second = orc.layer_backward(args[0][:, 8:], args[1][:, 8:], *args[2:], C, eta, dO[:, 8:], mode="mse")
    for i in (0, 1):
        np.testing.assert_allclose(packed[i], np.concatenate([first[i], second[i]], axis=1), rtol=1e-12,
                                   atol=1e-12)
    for i in range(2, 7):
        np.testing.assert_allclose(packed[i], first[i] + second[i], rtol=1e-12, atol=1e-12)


def _masked_dual_form_dot(Z, V, W0, C, eta, mask):
    """The dual form above with the update mask: token s of an earlier chunk contributes only if its chunk is
    flagged."""
    n, f = Z.shape
    d = V.shape[1]
    O = np.zeros((n, d))
    for t in range(n):
        for i in range(d):
            O[t, i] = sum(Z[t, j] * W0[i, j] for j in range(f))
        for s in range(n):
            if s // C < t // C and mask[s // C]:
                dot = sum(Z[t, j] * Z[s, j] for j in range(f))
                for i in range(d):
                    O[t, i] += eta * dot * V[s, i]
    return O


def test_update_mask_dot_equals_masked_brute_force():
    """The layer with an update mask (dot objective) against the token-level dual form in which only flagged
    chunks' tokens reach later outputs; an all-ones mask is the unmasked layer."""
    rng = _rng(60)
    B, n, C, d, f, K, eta = 2, 12, 3, 3, 4, 2, 0.2
    H, X0 = rng.standard_normal((B, n, d)), rng.standard_normal((B, n, d))
    Wg, Wu = rng.standard_normal((f, d)) * 0.5, rng.standard_normal((f, d)) * 0.5
    W0, Wt, cw = rng.standard_normal((d, f)), rng.standard_normal((d, d)), rng.standard_normal((d, K))
    mask = np.array([[1, 0, 1, 0], [0, 1, 1, 0]], dtype=np.uint8)
    O, _ = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "dot", update_mask=mask)
    for b in range(B):
        Z = orc.gated_intermediate(H[b], Wg, Wu)
        V = orc.target_values(X0[b], cw, Wt)
        np.testing.assert_allclose(O[b], _masked_dual_form_dot(Z, V, W0, C, eta, mask[b]), rtol=1e-12, atol=1e-12)
    O1, W1 = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "dot", update_mask=np.ones((B, 4)))
    O2, W2 = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "dot")
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(W1, W2)


def test_update_mask_mse_equals_resumed_calls_with_a_frozen_chunk():
    """A masked chunk of the MSE layer is the same as resuming the sequence at that chunk with eta = 0 for one chunk
    and then resuming again with the original eta (resumed calls are pinned separately)."""
    rng = _rng(61)
    B, C, d, f, K, eta = 1, 4, 3, 4, 3, 0.3
    n = 3 * C
    H, X0 = rng.standard_normal((B, n, d)), rng.standard_normal((B, n, d))
    Wg, Wu = rng.standard_normal((f, d)) * 0.5, rng.standard_normal((f, d)) * 0.5
    W0, Wt, cw = rng.standard_normal((d, f)), rng.standard_normal((d, d)), rng.standard_normal((d, K))
    O, W = orc.inplace_layer(H, X0, Wg, Wu, W0, Wt, cw, C, eta, "mse", update_mask=np.array([[1, 0, 1]]))
    piece = lambda a, c0, c1: a[:, c0 * C: c1 * C]
    halo = lambda c0: X0[:, c0 * C - (K - 1): c0 * C]
    Oa, Wa = orc.inplace_layer(piece(H, 0, 1), piece(X0, 0, 1), Wg, Wu, W0, Wt, cw, C, eta, "mse")
    Ob, Wb = orc.inplace_layer(piece(H, 1, 2), piece(X0, 1, 2), Wg, Wu, W0, Wt, cw, C, 0.0, "mse", W_init=Wa,
                               x0_halo=halo(1))
    Oc, Wc = orc.inplace_layer(piece(H, 2, 3), piece(X0, 2, 3), Wg, Wu, W0, Wt, cw, C, eta, "mse", W_init=Wb,
                               x0_halo=halo(2))
    np.testing.assert_allclose(O, np.concatenate([Oa, Ob, Oc], axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Wc, rtol=1e-12, atol=1e-12)


def test_core_backward_with_documents_matches_autograd():
    """Packed documents: autograd of the chunk loop that restarts from W0 at every flagged chunk."""
    rng = _rng(54)
    n, C, d, f, eta = 15, 3, 3, 4, 0.3
    starts = np.array([1, 0, 1, 1, 0])
    Z, V, W0, dO = (rng.standard_normal(s) for s in ((n, f), (n, d), (d, f), (n, d)))
    dZ, dV, dW0 = orc.chunk_core_backward(Z, V, W0, C, eta, dO, doc_starts=starts)
    tz, tv, tw = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0))
    W, outs = tw, []
    for c, s in enumerate(range(0, n, C)):
        if starts[c]:
            W = tw
        outs.append(tz[s:s + C] @ W.T)
        W = W + eta * (tv[s:s + C].T @ tz[s:s + C])
    (torch.cat(outs) * torch.from_numpy(dO)).sum().backward()
    np.testing.assert_allclose(dZ, tz.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW0, tw.grad.numpy(), rtol=1e-12, atol=1e-12)
    # and the forward it differentiates is the layer's packed-document chunk loop
    O_loop = torch.cat(outs).detach().numpy()
    O_docs = np.concatenate([orc.chunk_apply_update(Z[a:b], V[a:b], W0, C, eta, "dot")[0]
                             for a, b in ((0, 6), (6, 9), (9, 15))])
    np.testing.assert_allclose(O_loop, O_docs, rtol=1e-12, atol=1e-12)


def test_layer_backward_with_documents_matches_autograd():
    """Packed documents in the whole layer: autograd of the layer whose convolution restarts with zeros and whose
    chunk loop restarts from W0 at each flagged chunk (torch's grouped conv1d per document)."""
    import torch.nn.functional as F
    rng = _rng(55)
    B, n, C, d, f, K, eta = 2, 12, 3, 3, 4, 3, 0.2
    starts = np.array([[1, 0, 1, 0], [1, 1, 0, 1]])
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(s) * 0.7 for s in shapes]
    dO = rng.standard_normal((B, n, d))
    ours = orc.layer_backward(*args, C, eta, dO, doc_starts=starts)
    ts = [torch.tensor(a, requires_grad=True) for a in args]
    H, X0, Wg, Wu, W0, Wt, cw = ts
    rows = []
    for b in range(B):
        outs, W = [], W0
        cuts = [c * C for c in range(4) if starts[b][c]] + [n]
        for a, e in zip(cuts[:-1], cuts[1:]):
            Z = F.silu(H[b, a:e] @ Wg.T) * (H[b, a:e] @ Wu.T)
            Y = F.conv1d(F.pad(X0[b, a:e].T[None], (K - 1, 0)), cw[:, None, :], groups=d)[0].T
            outs.append(_torch_dot_chunk_loop(Z, Y @ Wt, W0, C, eta))
        rows.append(torch.cat(outs))
    (torch.stack(rows) * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-11)
    O, _ = orc.inplace_layer(*args, C, eta, "dot", doc_starts=starts)
    np.testing.assert_allclose(O, torch.stack(rows).detach().numpy(), rtol=1e-12, atol=1e-12)


def _torch_mse_chunk_loop(Z, V, W0, C, eta):
    """The MSE chunk loop in torch float64 (apply, then the step on the chunk's mean squared error), for autograd."""
    W = W0
    outs = []
    for s in range(0, Z.shape[0], C):
        Zc, Vc = Z[s:s + C], V[s:s + C]
        O = Zc @ W.T
        outs.append(O)
        W = W - (eta / Zc.shape[0]) * ((O - Vc).T @ Zc)
    return torch.cat(outs)


@pytest.mark.parametrize("n,C", [(12, 4), (10, 3), (8, 8)])
def test_mse_core_backward_matches_autograd(n, C):
    """The MSE chunk loop's backward against torch autograd of the same loop (ragged last chunk, one chunk)."""
    rng = _rng(56)
    d, f, eta = 3, 5, 0.4
    Z, V, W0, dO = (rng.standard_normal(s) for s in ((n, f), (n, d), (d, f), (n, d)))
    dZ, dV, dW0 = orc.mse_core_backward(Z, V, W0, C, eta, dO)
    tz, tv, tw = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0))
    (_torch_mse_chunk_loop(tz, tv, tw, C, eta) * torch.from_numpy(dO)).sum().backward()
    grad = lambda t: np.zeros(t.shape) if t.grad is None else t.grad.numpy()
    np.testing.assert_allclose(dZ, grad(tz), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dV, grad(tv), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dW0, grad(tw), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(_torch_mse_chunk_loop(tz, tv, tw, C, eta).detach().numpy(),
                               orc.chunk_apply_update(Z, V, W0, C, eta, "mse")[0], rtol=1e-12, atol=1e-12)


def test_mse_core_backward_with_documents_matches_autograd():
    """Packed documents in the MSE loop: autograd of the loop restarting from W0 at every flagged chunk."""
    rng = _rng(57)
    n, C, d, f, eta = 15, 3, 3, 4, 0.4
    starts = np.array([1, 0, 1, 1, 0])
    Z, V, W0, dO = (rng.standard_normal(s) for s in ((n, f), (n, d), (d, f), (n, d)))
    dZ, dV, dW0 = orc.mse_core_backward(Z, V, W0, C, eta, dO, doc_starts=starts)
    tz, tv, tw = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0))
    W, outs = tw, []
    for c, s in enumerate(range(0, n, C)):
        if starts[c]:
            W = tw
        Zc, Vc = tz[s:s + C], tv[s:s + C]
        O = Zc @ W.T
        outs.append(O)
        W = W - (eta / C) * ((O - Vc).T @ Zc)
    (torch.cat(outs) * torch.from_numpy(dO)).sum().backward()
    np.testing.assert_allclose(dZ, tz.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dW0, tw.grad.numpy(), rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- backward with update masks and the forward conv

def _torch_loop(Z, V, W0, C, eta, mode, mask):
    """The chunk loop (either objective) in torch float64 with an update mask: a masked chunk is applied and takes
    no step."""
    W = W0
    outs = []
    for c, s in enumerate(range(0, Z.shape[0], C)):
        Zc, Vc = Z[s:s + C], V[s:s + C]
        O = Zc @ W.T
        outs.append(O)
        if mask[c]:
            W = W + eta * (Vc.T @ Zc) if mode == "dot" else W - (eta / Zc.shape[0]) * ((O - Vc).T @ Zc)
    return torch.cat(outs)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_core_backward_with_update_mask_matches_autograd(mode):
    """A masked chunk is applied with the state it finds and leaves it unchanged: autograd of that loop gives the
    oracle's gradients, the masked chunks' target gradient zero; an all-ones mask is the unmasked backward."""
    rng = _rng(58)
    n, C, d, f, eta = 15, 3, 3, 4, 0.4
    Z, V, W0, dO = (rng.standard_normal(sh) for sh in ((n, f), (n, d), (d, f), (n, d)))
    mask = [1, 0, 1, 0, 1]
    back = orc.chunk_core_backward if mode == "dot" else orc.mse_core_backward
    ours = back(Z, V, W0, C, eta, dO, update_mask=mask)
    tz, tv, tw = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0))
    (_torch_loop(tz, tv, tw, C, eta, mode, mask) * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, (tz, tv, tw)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert not ours[1][3:6].any() and not ours[1][9:12].any()
    plain = back(Z, V, W0, C, eta, dO)
    for a, b in zip(back(Z, V, W0, C, eta, dO, update_mask=[1] * 5), plain):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_layer_backward_forward_conv_and_mask_match_autograd(mode):
    """The whole layer with the forward-looking in-chunk convolution (torch's grouped conv1d on each chunk, right
    padded) and an update mask, two rows with different masks: every gradient against autograd; the forward it
    differentiates is the oracle's layer."""
    import torch.nn.functional as F
    rng = _rng(59)
    B, n, C, d, f, K, eta = 2, 12, 4, 3, 4, 3, 0.3
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(sh) * 0.7 for sh in shapes]
    dO = rng.standard_normal((B, n, d))
    mask = np.array([[1, 0, 1], [0, 1, 1]])
    ours = orc.layer_backward(*args, C, eta, dO, mode=mode, update_mask=mask, conv_forward=True)
    ts = [torch.tensor(a, requires_grad=True) for a in args]
    H, X0, Wg, Wu, W0, Wt, cw = ts
    rows = []
    for b in range(B):
        Z = F.silu(H[b] @ Wg.T) * (H[b] @ Wu.T)
        Y = torch.cat([F.conv1d(F.pad(X0[b, s:s + C].T[None], (0, K - 1)), cw[:, None, :], groups=d)[0].T
                       for s in range(0, n, C)])
        rows.append(_torch_loop(Z, Y @ Wt, W0, C, eta, mode, mask[b]))
    (torch.stack(rows) * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-11)
    O, _ = orc.inplace_layer(*args, C, eta, mode, update_mask=mask, conv_forward=True)
    np.testing.assert_allclose(O, torch.stack(rows).detach().numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward of resumed rows

def _torch_resumed_layer(ts, C, eta, mode, docs, mask, conv_forward):
    """The layer over resumed rows written per document in torch float64: a row's documents are cut at its flagged
    chunks; the first one continues (reads the halo, starts from W_init) unless chunk 0 is flagged; every other
    document starts from W_down0 with zeros before its first row."""
    import torch.nn.functional as F
    H, X0, Wg, Wu, W0, Wt, cw, Wi, halo = ts
    B, n, d = H.shape
    K = cw.shape[1]
    k = -(-n // C)
    rows = []
    for b in range(B):
        starts = [0] + [c for c in range(1, k) if docs[b][c]] + [k]
        outs = []
        for j in range(len(starts) - 1):
            s, e = starts[j] * C, min(starts[j + 1] * C, n)
            cont = j == 0 and not docs[b][0]
            Z = F.silu(H[b, s:e] @ Wg.T) * (H[b, s:e] @ Wu.T)
            if conv_forward:
                Y = torch.cat([F.conv1d(F.pad(X0[b, t:min(t + C, e)].T[None], (0, K - 1)), cw[:, None, :],
                                        groups=d)[0].T for t in range(s, e, C)])
            else:
                pre = halo[b] if (cont and halo is not None) else torch.zeros(K - 1, d, dtype=H.dtype)
                Y = F.conv1d(torch.cat([pre, X0[b, s:e]]).T[None], cw[:, None, :], groups=d)[0].T
            Ws = Wi[b] if (cont and Wi is not None) else W0
            m = [1] * (e // C + 1) if mask is None else mask[b]
            outs.append(_torch_loop(Z, Y @ Wt, Ws, C, eta, mode, m[starts[j]:]))
        rows.append(torch.cat(outs))
    return torch.stack(rows)


@pytest.mark.parametrize("mode", ["dot", "mse"])
@pytest.mark.parametrize("case", ["both", "state_only", "halo_only", "mask", "forward_conv"])
def test_layer_backward_resumed_rows_match_autograd(mode, case):
    """Resumed rows (W_init and the halo of the previous call's last K-1 rows), three rows: one continuing with a
    second document at chunk 2, one flagged at chunk 0 (nothing continues: zero dW_init and dx0_halo), one
    continuing to its end.  Every gradient, dW_init and dx0_halo included, against autograd of the per-document
    torch layer, whose output is also the oracle's forward."""
    rng = _rng(60)
    B, n, C, d, f, K, eta = 3, 14, 4, 3, 4, 3, 0.3
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K), (B, d, f), (B, K - 1, d))
    args = [rng.standard_normal(sh) * 0.7 for sh in shapes]
    dO = rng.standard_normal((B, n, d))
    docs = np.array([[0, 0, 1, 0], [1, 0, 0, 1], [0, 0, 0, 0]])
    mask = np.array([[1, 0, 1, 1], [0, 1, 1, 1], [1, 1, 0, 1]]) if case == "mask" else None
    if case == "state_only":
        args[8] = None
    if case == "halo_only":
        args[7] = None
    fwd = case == "forward_conv"
    ours = orc.layer_backward(*args[:7], C, eta, dO, doc_starts=docs, mode=mode, update_mask=mask,
                              conv_forward=fwd, W_init=args[7], x0_halo=args[8])
    assert len(ours) == 9
    ts = [None if a is None else torch.tensor(a, requires_grad=True) for a in args]
    O = _torch_resumed_layer(ts, C, eta, mode, docs, mask, fwd)
    (O * torch.from_numpy(dO)).sum().backward()
    for i, t in enumerate(ts):
        want = np.zeros_like(ours[i]) if t is None or t.grad is None else t.grad.numpy()
        np.testing.assert_allclose(ours[i], want, rtol=1e-10, atol=1e-11, err_msg=f"gradient {i}")
    assert not ours[7][1].any() and not ours[8][1].any()
    if fwd:
        assert not ours[8].any()
    Of, _ = orc.inplace_layer(*args[:7], C, eta, mode, x0_halo=args[8], doc_starts=docs, conv_forward=fwd,
                              W_init=args[7], update_mask=mask)
    np.testing.assert_allclose(Of, O.detach().numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_resumed_core_backward_matches_autograd(mode):
    """The chunk loop of a resumed row with a second document at chunk 3: autograd of the two documents (the first
    from W_init, the second from W_down0) gives dZ, dV^, dW_down0 (second document only) and dW_init (first only);
    a row flagged at chunk 0 is the plain backward with a zero dW_init."""
    rng = _rng(61)
    n, C, d, f, eta = 17, 3, 3, 4, 0.35
    Z, V, W0, Wi, dO = (rng.standard_normal(sh) for sh in ((n, f), (n, d), (d, f), (d, f), (n, d)))
    docs = [0, 0, 0, 1, 0, 0]
    ours = orc.resumed_core_backward(Z, V, W0, Wi, C, eta, dO, mode, doc_starts=docs)
    tz, tv, tw, ti = (torch.tensor(a, requires_grad=True) for a in (Z, V, W0, Wi))
    ones = [1] * 6
    O = torch.cat([_torch_loop(tz[:9], tv[:9], ti, C, eta, mode, ones), _torch_loop(tz[9:], tv[9:], tw, C, eta,
                                                                                   mode, ones)])
    (O * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, (tz, tv, tw, ti)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)
    back = orc.chunk_core_backward if mode == "dot" else orc.mse_core_backward
    flagged = [1, 0, 0, 1, 0, 0]
    r = orc.resumed_core_backward(Z, V, W0, Wi, C, eta, dO, mode, doc_starts=flagged)
    for a, b in zip(r[:3], back(Z, V, W0, C, eta, dO, doc_starts=flagged)):
        np.testing.assert_array_equal(a, b)
    assert not r[3].any()


# ---------------------------------------------------------------- update-then-apply order

def test_update_first_dot_closed_form():
    """Dot objective, update first: O_c = Z_c (W_c + eta V^_c^T Z_c)^T = the apply-then-update output plus
    eta (Z_c Z_c^T) V^_c, the chunk's own targets through its token Gram matrix; W_final is the same in both
    orders."""
    rng = _rng(90)
    n, C, d, f, eta = 13, 4, 3, 5, 0.3
    Z, V, W0 = rng.standard_normal((n, f)), rng.standard_normal((n, d)), rng.standard_normal((d, f))
    Oa, Wa = orc.chunk_apply_update(Z, V, W0, C, eta, "dot")
    Ou, Wu = orc.chunk_apply_update(Z, V, W0, C, eta, "dot", update_first=True)
    want = Oa.copy()
    for s in range(0, n, C):
        Zc, Vc = Z[s:s + C], V[s:s + C]
        want[s:s + C] += eta * (Zc @ Zc.T) @ Vc
    np.testing.assert_allclose(Ou, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(Wu, Wa)


def test_update_first_mse_closed_form():
    """MSE objective, update first: W_{c+1} = W_c - (eta/C) R_c^T Z_c with R_c = Z_c W_c^T - V^_c, so
    O_c = Z_c W_{c+1}^T = (apply-then-update output) - (eta/C) (Z_c Z_c^T) R_c: the chunk's own residual through its
    token Gram matrix.  R_c is formed here from the apply-then-update outputs, which are Z_c W_c^T; W_final is the
    same in both orders.  The ragged last chunk divides by its own length."""
    rng = _rng(92)
    n, C, d, f, eta = 14, 4, 3, 5, 0.7
    Z, V = rng.standard_normal((n, f)) * 0.5, rng.standard_normal((n, d))
    W0 = rng.standard_normal((d, f)) * 0.4
    Oa, Wa = orc.chunk_apply_update(Z, V, W0, C, eta, "mse")
    Ou, Wu = orc.chunk_apply_update(Z, V, W0, C, eta, "mse", update_first=True)
    want = Oa.copy()
    for s0 in range(0, n, C):
        Zc, Vc = Z[s0:s0 + C], V[s0:s0 + C]
        Rc = Oa[s0:s0 + C] - Vc
        want[s0:s0 + C] -= eta / len(Zc) * (Zc @ Zc.T) @ Rc
    np.testing.assert_allclose(Ou, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(Wu, Wa)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_update_first_layer_equals_truncated_final_states(mode):
    """The layer with update_first: chunk c's outputs are Z_c times the W_final of the apply-then-update layer
    stopped after chunk c (max_chunks = c + 1), for every row of a packed, masked, resumed batch; the final states
    equal the apply-then-update layer's."""
    rng = _rng(91)
    B, n, C, d, f, K, eta = 2, 12, 4, 3, 4, 3, 0.4
    shapes = ((B, n, d), (B, n, d), (f, d), (f, d), (d, f), (d, d), (d, K))
    args = [rng.standard_normal(sh) * 0.7 for sh in shapes]
    docs = [[0, 1, 0], [0, 0, 0]]
    mask = [[1, 1, 0], [0, 1, 1]]
    Wi = rng.standard_normal((B, d, f)) * 0.5
    halo = rng.standard_normal((B, K - 1, d))
    kw = dict(doc_starts=docs, update_mask=mask, W_init=Wi, x0_halo=halo)
    Ou, Wu = orc.inplace_layer(*args, C, eta, mode, update_first=True, **kw)
    Oa, Wa = orc.inplace_layer(*args, C, eta, mode, **kw)
    np.testing.assert_array_equal(Wu, Wa)
    for c in range(n // C):
        _, Wc = orc.inplace_layer(*args, C, eta, mode, max_chunks=c + 1, **kw)
        for b in range(B):
            Zc = orc.gated_intermediate(args[0][b, c * C:(c + 1) * C], args[2], args[3])
            np.testing.assert_allclose(Ou[b, c * C:(c + 1) * C], Zc @ Wc[b].T, rtol=1e-12, atol=1e-12)
    # a masked chunk takes no step, so both orders apply it with the same state
    np.testing.assert_array_equal(Ou[0, 8:12], Oa[0, 8:12])
