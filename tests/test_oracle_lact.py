"""Pins of the LaCT SwiGLU oracle: autograd, finite differences, a hand-derived
scalar case, eta = 0, chunk = sequence, and causality of the ordering."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lact as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, B=1, H=2, n=12, dh=3, m=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, n, dh))
    k = rng.standard_normal((B, H, n, dh))
    v = rng.standard_normal((B, H, n, dh))
    W1 = rng.standard_normal((H, m, dh)) / np.sqrt(dh)
    W3 = rng.standard_normal((H, m, dh)) / np.sqrt(dh)
    W2 = rng.standard_normal((H, dh, m)) / np.sqrt(m)
    return q, k, v, W1, W3, W2


def _torch_swiglu(x, W1, W3, W2):
    return F.linear(F.silu(F.linear(x, W1)) * F.linear(x, W3), W2)


def test_grads_match_autograd():
    q, k, v, W1, W3, W2 = _problem(1, n=9, dh=4, m=6)
    kc, vc = k[0, 0], v[0, 0]
    w1, w3, w2 = (torch.from_numpy(a[0].copy()).requires_grad_(True) for a in (W1, W3, W2))
    out = _torch_swiglu(torch.from_numpy(kc), w1, w3, w2)
    (0.5 * ((out - torch.from_numpy(vc)) ** 2).sum()).backward()
    G1, G3, G2 = orc.swiglu_grads(kc, vc, W1[0], W3[0], W2[0])
    np.testing.assert_allclose(G1, w1.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(G3, w3.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(G2, w2.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_grads_match_finite_differences():
    q, k, v, W1, W3, W2 = _problem(2, n=5, dh=2, m=3)
    kc, vc = k[0, 0], v[0, 0]
    Ws = [W1[0].copy(), W3[0].copy(), W2[0].copy()]
    grads = orc.swiglu_grads(kc, vc, *Ws)
    h = 1e-6
    for which in range(3):
        fd = np.zeros_like(Ws[which])
        for idx in np.ndindex(*Ws[which].shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[which][idx] += h
            Wm[which][idx] -= h
            fd[idx] = (orc.swiglu_loss(kc, vc, *Wp) - orc.swiglu_loss(kc, vc, *Wm)) / (2 * h)
        np.testing.assert_allclose(grads[which], fd, rtol=1e-6, atol=1e-8)


def test_scalar_golden_hand_derived():
    with open(os.path.join(GOLDEN, "lact_scalar.json")) as fh:
        g = json.load(fh)
    a = lambda x: np.array([[x]], dtype=np.float64)
    G1, G3, G2 = orc.swiglu_grads(a(g["k"]), a(g["v"]), a(g["w1"]), a(g["w3"]), a(g["w2"]))
    assert G1.item() == g["G1"] and G3.item() == g["G3"] and G2.item() == g["G2"]
    q = np.array(g["q"]).reshape(1, 1, 1, 1)
    k = np.array(g["k"]).reshape(1, 1, 1, 1)
    v = np.array(g["v"]).reshape(1, 1, 1, 1)
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, a(g["w1"])[None], a(g["w3"])[None], a(g["w2"])[None],
                                      1, g["eta"], "update_then_apply")
    assert W1f.item() == g["w1_after"] and W3f.item() == g["w3_after"] and W2f.item() == g["w2_after"]
    np.testing.assert_allclose(O.item(), 144.0 / (1.0 + math.exp(-12.0)), rtol=1e-15)


@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_eta_zero_is_plain_swiglu(order):
    q, k, v, W1, W3, W2 = _problem(3)
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.0, order)
    for h in range(W1.shape[0]):
        ref = _torch_swiglu(torch.from_numpy(q[0, h]), torch.from_numpy(W1[h]), torch.from_numpy(W3[h]),
                            torch.from_numpy(W2[h])).numpy()
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(W1f[0], W1)
    np.testing.assert_array_equal(W2f[0], W2)


def test_chunk_equal_sequence_is_one_full_batch_gd_step():
    q, k, v, W1, W3, W2 = _problem(4, H=1, n=10)
    eta = 0.7
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 10, eta, "update_then_apply")
    w1, w3, w2 = (torch.from_numpy(a[0].copy()).requires_grad_(True) for a in (W1, W3, W2))
    loss = 0.5 * ((_torch_swiglu(torch.from_numpy(k[0, 0]), w1, w3, w2) - torch.from_numpy(v[0, 0])) ** 2).sum()
    loss.backward()
    n1, n3, n2 = (w.detach() - eta * w.grad for w in (w1, w3, w2))
    np.testing.assert_allclose(W1f[0, 0], n1.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(W3f[0, 0], n3.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(W2f[0, 0], n2.numpy(), rtol=1e-12, atol=1e-14)
    ref = _torch_swiglu(torch.from_numpy(q[0, 0]), n1, n3, n2).numpy()
    np.testing.assert_allclose(O[0, 0], ref, rtol=1e-12, atol=1e-14)


def test_update_then_apply_causality():
    q, k, v, W1, W3, W2 = _problem(5, n=16)
    C = 4
    O, *_ = orc.lact_layer(q, k, v, W1, W3, W2, C, 0.5, "update_then_apply")
    rng = np.random.default_rng(50)
    for c in range(4):
        kp, vp, qp = k.copy(), v.copy(), q.copy()
        kp[:, :, (c + 1) * C:] += rng.standard_normal(kp[:, :, (c + 1) * C:].shape)
        vp[:, :, (c + 1) * C:] += rng.standard_normal(vp[:, :, (c + 1) * C:].shape)
        qp[:, :, (c + 1) * C:] += rng.standard_normal(qp[:, :, (c + 1) * C:].shape)
        Op, *_ = orc.lact_layer(qp, kp, vp, W1, W3, W2, C, 0.5, "update_then_apply")
        np.testing.assert_array_equal(Op[:, :, : (c + 1) * C], O[:, :, : (c + 1) * C])
    # within a chunk, the chunk's own keys reach its queries (update first)
    kp = k.copy()
    kp[:, :, 0] += 1.0
    Op, *_ = orc.lact_layer(q, kp, v, W1, W3, W2, C, 0.5, "update_then_apply")
    assert not np.allclose(Op[:, :, :C], O[:, :, :C])


def test_apply_then_update_first_chunk_uses_initial_weights():
    q, k, v, W1, W3, W2 = _problem(6, n=8)
    O, *_ = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.5, "apply_then_update")
    for h in range(2):
        np.testing.assert_allclose(O[0, h, :4], orc.swiglu_apply(q[0, h, :4], W1[h], W3[h], W2[h]), rtol=1e-14)


def test_heads_and_batch_rows_are_independent():
    q, k, v, W1, W3, W2 = _problem(7, B=2, H=2, n=8)
    O, W1f, _, _ = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.3)
    for b in range(2):
        for h in range(2):
            Ob, W1b, _, _ = orc.lact_layer(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                           W1[h:h + 1], W3[h:h + 1], W2[h:h + 1], 4, 0.3)
            np.testing.assert_array_equal(O[b, h], Ob[0, 0])
            np.testing.assert_array_equal(W1f[b, h], W1b[0, 0])


def test_update_mask_all_off_is_plain_swiglu():
    """No chunk updates: every chunk is applied with the initial weights, which stay as they are."""
    q, k, v, W1, W3, W2 = _problem(11)
    n_chunks = q.shape[2] // 4
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.9, "update_then_apply",
                                      update_mask=np.zeros(n_chunks, dtype=bool))
    for h in range(W1.shape[0]):
        ref = _torch_swiglu(torch.from_numpy(q[0, h]), torch.from_numpy(W1[h]), torch.from_numpy(W3[h]),
                            torch.from_numpy(W2[h])).numpy()
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(W1f[0], W1)
    np.testing.assert_array_equal(W3f[0], W3)
    np.testing.assert_array_equal(W2f[0], W2)


@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_update_mask_composes_from_unmasked_runs(order):
    """Mask [1, 0, 1]: chunk 0 as an unmasked run, chunk 1 only applied (torch SwiGLU) with the weights chunk 0
    left, chunk 2 as an unmasked run from those weights."""
    q, k, v, W1, W3, W2 = _problem(12, H=1, n=12)
    C, eta = 4, 0.6
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, C, eta, order, update_mask=[1, 0, 1])
    r0, r1, r2 = slice(0, C), slice(C, 2 * C), slice(2 * C, 3 * C)
    O0, a1, a3, a2 = orc.lact_layer(q[..., r0, :], k[..., r0, :], v[..., r0, :], W1, W3, W2, C, eta, order)
    np.testing.assert_allclose(O[..., r0, :], O0, rtol=1e-12, atol=1e-14)
    O1 = _torch_swiglu(torch.from_numpy(q[0, 0, r1]), torch.from_numpy(a1[0, 0]), torch.from_numpy(a3[0, 0]),
                       torch.from_numpy(a2[0, 0])).numpy()
    np.testing.assert_allclose(O[0, 0, r1], O1, rtol=1e-12, atol=1e-14)
    O2, b1, b3, b2 = orc.lact_layer(q[..., r2, :], k[..., r2, :], v[..., r2, :], a1[0], a3[0], a2[0], C, eta, order)
    np.testing.assert_allclose(O[..., r2, :], O2, rtol=1e-12, atol=1e-14)
    for got, want in ((W1f, b1), (W3f, b3), (W2f, b2)):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_token_rates_and_losses_match_autograd(loss):
    """One chunk spanning the sequence: the step on sum_i eta_i L_i (eq. (3)), with the squared error or the
    dot-product loss -f(k)^T v, equals torch autograd's; the queries then see the stepped weights."""
    q, k, v, W1, W3, W2 = _problem(13, H=1, n=10)
    eta = 0.4
    et = np.random.default_rng(14).uniform(0.2, 1.5, size=(1, 1, 10))
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 10, eta, "update_then_apply", eta_tok=et, loss=loss)
    w1, w3, w2 = (torch.from_numpy(a[0].copy()).requires_grad_(True) for a in (W1, W3, W2))
    y = _torch_swiglu(torch.from_numpy(k[0, 0]), w1, w3, w2)
    vt, e = torch.from_numpy(v[0, 0]), torch.from_numpy(et[0, 0])
    per_tok = 0.5 * ((y - vt) ** 2).sum(dim=1) if loss == "mse" else -(y * vt).sum(dim=1)
    (e * per_tok).sum().backward()
    n1, n3, n2 = (w.detach() - eta * w.grad for w in (w1, w3, w2))
    for got, want in ((W1f[0, 0], n1), (W3f[0, 0], n3), (W2f[0, 0], n2)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-13)
    ref = _torch_swiglu(torch.from_numpy(q[0, 0]), n1, n3, n2).numpy()
    np.testing.assert_allclose(O[0, 0], ref, rtol=1e-11, atol=1e-13)


def test_constant_token_rate_is_a_scaled_eta():
    q, k, v, W1, W3, W2 = _problem(15)
    a = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.5, eta_tok=np.full(q.shape[:3], 0.3))
    b = orc.lact_layer(q, k, v, W1, W3, W2, 4, 0.15)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_weight_norm_matches_torch_normalize():
    """LaCT Model Architecture §2: after the step, every row of each matrix (its input dimension) is scaled to
    unit L2 norm -- torch's F.normalize of the autograd step on one chunk; after several chunks every row still
    has unit norm."""
    q, k, v, W1, W3, W2 = _problem(16, H=1, n=10)
    eta = 0.8
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 10, eta, weight_norm=True)
    w1, w3, w2 = (torch.from_numpy(a[0].copy()).requires_grad_(True) for a in (W1, W3, W2))
    (0.5 * ((_torch_swiglu(torch.from_numpy(k[0, 0]), w1, w3, w2) - torch.from_numpy(v[0, 0])) ** 2).sum()).backward()
    n1, n3, n2 = (F.normalize(w.detach() - eta * w.grad, dim=-1) for w in (w1, w3, w2))
    for got, want in ((W1f[0, 0], n1), (W3f[0, 0], n3), (W2f[0, 0], n2)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(O[0, 0], _torch_swiglu(torch.from_numpy(q[0, 0]), n1, n3, n2).numpy(), rtol=1e-11,
                               atol=1e-13)
    q, k, v, W1, W3, W2 = _problem(17)
    _, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 3, eta, weight_norm=True)
    for W in (W1f, W3f, W2f):
        np.testing.assert_allclose(np.linalg.norm(W, axis=-1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("shape", [(6, 4), (4, 6), (5, 5)])
def test_muon_acts_on_singular_values(shape):
    """An odd matrix polynomial acts on each singular value alone, so the Newton-Schulz iteration equals
    U p(...p(s / ||g||_F)) V^T from numpy's SVD of g, with p the quintic a x + b x^3 + c x^5; and it lands near
    the polar factor U V^T (every singular value of the result within [0.6, 1.25])."""
    g = np.random.default_rng(40).standard_normal(shape)
    U, S, Vt = np.linalg.svd(g, full_matrices=False)
    a, b, c = orc.MUON_COEFFS
    x = S / (np.linalg.norm(g) + 1e-7)
    for _ in range(orc.MUON_STEPS):
        x = a * x + b * x ** 3 + c * x ** 5
    want = (U * x) @ Vt
    got = orc.muon(g)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    sv = np.linalg.svd(got, compute_uv=False)
    assert sv.min() > 0.6 and sv.max() < 1.25, sv


# The quintic Newton-Schulz iteration published with the Muon optimizer (K. Jordan et al., "Muon: An optimizer for
# hidden layers in neural networks", 2024), which the LaCT review's section 2 names without its polynomial: the
# coefficients and the step count typed here from that publication, independently of the oracle's constants.
PUBLISHED_ABC = (3.4445, -4.7750, 2.0315)
PUBLISHED_STEPS = 5


def test_muon_coefficients_are_the_published_ones():
    assert tuple(orc.MUON_COEFFS) == PUBLISHED_ABC
    assert orc.MUON_STEPS == PUBLISHED_STEPS


def test_muon_rank_one_and_small_singular_values_follow_the_published_quintic():
    """A rank-one gradient has one singular value, 1 after the Frobenius scaling: the first step maps it to
    p(1) = a + b + c = 0.701 and five steps to 0.6964 (the published polynomial iterated by hand below).  A
    singular value far below the largest one grows by p'(0) = a per step, a^5 = 484.9 over five steps: the
    publication's steep slope at zero."""
    a, b, c = PUBLISHED_ABC
    x = 1.0
    traj = []
    for _ in range(PUBLISHED_STEPS):
        x = a * x + b * x ** 3 + c * x ** 5
        traj.append(x)
    np.testing.assert_allclose(traj[0], 0.701, rtol=1e-12)
    np.testing.assert_allclose(traj, [0.701, 1.113620, 0.720706, 1.089974, 0.696436], atol=1e-6)
    rng = np.random.default_rng(42)
    u = rng.standard_normal(6)
    v = rng.standard_normal(4)
    got = orc.muon(7.0 * np.outer(u, v))
    np.testing.assert_allclose(got, traj[-1] * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v)), rtol=1e-6,
                               atol=1e-9)
    # diag(1, eps): the small value is multiplied by a at every step (its cubic and quintic terms vanish)
    eps = 1e-7
    got = orc.muon(np.diag([1.0, eps]))
    np.testing.assert_allclose(got[0, 0], traj[-1], rtol=1e-6)
    np.testing.assert_allclose(got[1, 1], a ** 5 * eps, rtol=1e-5)
    np.testing.assert_allclose(a ** 5, 484.876, rtol=1e-5)


def test_muon_update_in_the_layer():
    """One chunk: W_final = W - eta Muon(g) with g from torch autograd; the queries see it."""
    q, k, v, W1, W3, W2 = _problem(41, H=1, n=10)
    eta = 0.05
    O, W1f, W3f, W2f = orc.lact_layer(q, k, v, W1, W3, W2, 10, eta, use_muon=True)
    w1, w3, w2 = (torch.from_numpy(a[0].copy()).requires_grad_(True) for a in (W1, W3, W2))
    (0.5 * ((_torch_swiglu(torch.from_numpy(k[0, 0]), w1, w3, w2) - torch.from_numpy(v[0, 0])) ** 2).sum()).backward()
    n1, n3, n2 = (w.detach().numpy() - eta * orc.muon(w.grad.numpy()) for w in (w1, w3, w2))
    for got, want in ((W1f[0, 0], n1), (W3f[0, 0], n3), (W2f[0, 0], n2)):
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)
    ref = _torch_swiglu(*(torch.from_numpy(a) for a in (q[0, 0], n1, n3, n2))).numpy()
    np.testing.assert_allclose(O[0, 0], ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- backward of the layer

def _torch_lact_layer(q, k, v, W1, W3, W2, chunk, eta, order, update_mask=None):
    """The LaCT layer in torch float64 with the inner gradient taken by autograd itself (create_graph, so that an
    outer backward differentiates through it), for the backward's pin."""
    B, Hn, n, dh = q.shape
    rows = []
    for b in range(B):
        heads = []
        for h in range(Hn):
            w = [W1[h], W3[h], W2[h]]
            outs = []
            for c, s in enumerate(range(0, n, chunk)):
                qc, kc, vc = q[b, h, s:s + chunk], k[b, h, s:s + chunk], v[b, h, s:s + chunk]
                if order == "apply_then_update":
                    outs.append(_torch_swiglu(qc, *w))
                if update_mask is None or update_mask[c]:
                    loss = 0.5 * ((_torch_swiglu(kc, *w) - vc) ** 2).sum()
                    grads = torch.autograd.grad(loss, w, create_graph=True)
                    w = [wi - eta * gi for wi, gi in zip(w, grads)]
                if order == "update_then_apply":
                    outs.append(_torch_swiglu(qc, *w))
            heads.append(torch.cat(outs))
        rows.append(torch.stack(heads))
    return torch.stack(rows)


@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
@pytest.mark.parametrize("n,chunk", [(12, 4), (10, 4), (6, 6)])
def test_lact_backward_matches_autograd(order, n, chunk):
    """Every gradient of the layer (q, k, v and the three initial weights, shared by two batch rows) against torch
    autograd of the layer whose inner chunk gradient autograd also takes (second-order terms through the update
    included); a ragged last chunk and a single chunk."""
    q, k, v, W1, W3, W2 = _problem(70, B=2, H=2, n=n, dh=3, m=5)
    eta = 0.7
    dO = np.random.default_rng(71).standard_normal(q.shape)
    ours = orc.lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO, order)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, W1, W3, W2)]
    out = _torch_lact_layer(*ts, chunk, eta, order)
    (out * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        # (one chunk applied before its update: k and v reach no output, autograd gives no gradient)
        want = np.zeros(t.shape) if t.grad is None else t.grad.numpy()
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # the forward it differentiates is the oracle's layer
    O, *_ = orc.lact_layer(q, k, v, W1, W3, W2, chunk, eta, order)
    np.testing.assert_allclose(O, out.detach().numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_lact_backward_with_update_mask_matches_autograd(order):
    """A masked chunk is applied but takes no step: autograd of the layer that skips those steps gives every
    gradient, the masked chunks' dk and dv are exactly zero, and the forward differentiated is the oracle's masked
    layer; an all-ones mask is the unmasked backward."""
    q, k, v, W1, W3, W2 = _problem(74, B=2, H=2, n=16, dh=3, m=5)
    eta, chunk = 0.7, 4
    mask = [1, 0, 0, 1]
    dO = np.random.default_rng(75).standard_normal(q.shape)
    ours = orc.lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO, order, update_mask=mask)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, W1, W3, W2)]
    out = _torch_lact_layer(*ts, chunk, eta, order, update_mask=mask)
    (out * torch.from_numpy(dO)).sum().backward()
    for got, t in zip(ours, ts):
        want = np.zeros(t.shape) if t.grad is None else t.grad.numpy()
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    for g in ours[1:3]:
        assert not g[:, :, 4:12].any()
    O, *_ = orc.lact_layer(q, k, v, W1, W3, W2, chunk, eta, order, update_mask=mask)
    np.testing.assert_allclose(O, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    plain = orc.lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO, order)
    for a, b in zip(orc.lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO, order, update_mask=[1] * 4), plain):
        np.testing.assert_array_equal(a, b)


def test_lact_backward_finite_differences_and_eta_zero():
    """Central differences of <O, dO> through the oracle's layer for entries of q, k, v and each initial weight;
    with eta = 0 the layer is the plain SwiGLU on the queries: dk = dv = 0 and the weight gradients are the
    apply's alone."""
    q, k, v, W1, W3, W2 = _problem(72, B=1, H=1, n=8, dh=3, m=4)
    eta, chunk = 0.6, 4
    dO = np.random.default_rng(73).standard_normal(q.shape)
    grads = orc.lact_backward(q, k, v, W1, W3, W2, chunk, eta, dO)
    args = [q, k, v, W1, W3, W2]
    L = lambda a: float(np.sum(orc.lact_layer(*a, chunk, eta)[0] * dO))
    h = 1e-6
    for which, idx in ((0, (0, 0, 5, 1)), (1, (0, 0, 2, 0)), (1, (0, 0, 6, 2)), (2, (0, 0, 1, 1)), (3, (0, 2, 1)),
                       (4, (0, 1, 0)), (5, (0, 2, 3))):
        p = [a.copy() for a in args]
        m = [a.copy() for a in args]
        p[which][idx] += h
        m[which][idx] -= h
        g = grads[which][idx]
        assert abs((L(p) - L(m)) / (2 * h) - g) < 1e-6 * max(1.0, abs(g)), (which, idx)
    dq, dk, dv, dW1, dW3, dW2 = orc.lact_backward(q, k, v, W1, W3, W2, chunk, 0.0, dO)
    assert not dk.any() and not dv.any()
    qt = torch.tensor(q[0, 0], requires_grad=True)
    ws = [torch.tensor(a[0], requires_grad=True) for a in (W1, W3, W2)]
    (_torch_swiglu(qt, *ws) * torch.from_numpy(dO[0, 0])).sum().backward()
    np.testing.assert_allclose(dq[0, 0], qt.grad.numpy(), rtol=1e-12, atol=1e-13)
    for got, t in zip((dW1[0], dW3[0], dW2[0]), ws):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-12, atol=1e-13)
