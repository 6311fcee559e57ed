"""GPU parity of the LaCT layer's backward (ttt_lact_swiglu_backward) against the float64 oracle.

The oracle's lact_backward is pinned on the CPU by torch autograd through the inner gradient step (create_graph)
and by central differences.  Tolerances (relative Frobenius) as for the forward: 1e-4 for fp32; 2e-2 for bf16
storage with fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti
from oracle import lact as olact

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dW1", "dW3", "dW2")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def case(dtype, order="update_then_apply", B=2, H=2, n=384, dh=72, m=136, C=128, eta=0.7, seed=81):
    cfg = ti.LactConfig("lbwd", B, H, n, dh, m, C, eta, order, dtype, seed=seed)
    x = ti.lact_inputs(cfg)
    gen = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn(B, H, n, dh, generator=gen).to(x["q"].dtype)
    return cfg, x, dO


def run(cfg, x, dO):
    print(f"lact backward case: {cfg.dtype} {cfg.order} B={cfg.batch} H={cfg.heads} n={cfg.seq_len} "
          f"dh={cfg.head_dim} m={cfg.hidden} C={cfg.chunk}", flush=True)
    g = {k: v.cuda() for k, v in x.items()}
    grads = cw.ttt_lact_swiglu_backward(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO.cuda(), cfg.chunk,
                                        cfg.eta, cfg.order)
    torch.cuda.synchronize()
    return grads


def oracle(cfg, x, dO):
    return olact.lact_backward(*(ti.to_f64(x[k]) for k in ("q", "k", "v", "W1", "W3", "W2")), cfg.chunk, cfg.eta,
                               ti.to_f64(dO), cfg.order)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_lact_backward_matches_oracle(dtype, order):
    """Every gradient on 2 x 2 (batch, head) rows (the weights' gradients summed over the two batch rows of each
    head), ragged head_dim 72 and hidden 136 (partial 256-tiles), three chunks."""
    cfg, x, dO = case(dtype, order)
    grads = run(cfg, x, dO)
    errs = {name: rel(f64(got), want) for name, got, want in zip(NAMES, grads, oracle(cfg, x, dO))}
    assert all(e < TOL[dtype] for e in errs.values()), errs


def test_lact_backward_single_chunk_and_eta_zero():
    # one chunk applied before its update: k and v reach no output, so dk = dv = 0 exactly
    cfg, x, dO = case("bf16", "apply_then_update", n=128)
    grads = run(cfg, x, dO)
    assert not torch.any(grads[1]) and not torch.any(grads[2])
    ref = oracle(cfg, x, dO)
    for i in (0, 3, 4, 5):
        assert rel(f64(grads[i]), ref[i]) < TOL["bf16"], NAMES[i]
    # eta = 0: the plain SwiGLU on the queries; dk = dv = 0
    cfg, x, dO = case("f32", eta=0.0)
    grads = run(cfg, x, dO)
    assert not torch.any(grads[1]) and not torch.any(grads[2])
    ref = oracle(cfg, x, dO)
    for i in (0, 3, 4, 5):
        assert rel(f64(grads[i]), ref[i]) < TOL["f32"], NAMES[i]


def test_lact_backward_empty_batch():
    cfg, x, dO = case("bf16", B=0)
    grads = run(cfg, x, dO)
    assert all(not torch.any(t) for t in grads[3:])


def test_lact_backward_workload_shape():
    """The workload's head_dim 512, hidden 1024, chunk 4096 and eta 1, on three chunks of two heads."""
    cfg = ti.workload("lact_bf16_256k").with_(heads=2, seq_len=3 * 4096)
    x = ti.lact_inputs(cfg)
    gen = torch.Generator().manual_seed(91)
    dO = torch.randn(*x["q"].shape, generator=gen).to(x["q"].dtype)
    grads = run(cfg, x, dO)
    errs = {name: rel(f64(got), want) for name, got, want in zip(NAMES, grads, oracle(cfg, x, dO))}
    print("  rel err " + "  ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    assert all(e < TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_lact_backward_with_update_mask(dtype, order):
    """The backward with an update mask (ttt_lact_swiglu_backward_ex): chunks 1 and 2 of four are applied without
    taking a step, so the recompute keeps their unchanged state and the reverse pass lets the state gradient through
    them; their dk and dv rows are exactly zero, and every gradient matches the oracle's masked backward."""
    cfg, x, dO = case(dtype, order, n=512, seed=83)
    mask = [1, 0, 0, 1]
    g = {k: v.cuda() for k, v in x.items()}
    print(f"lact backward mask case: {dtype} {order} mask={mask}", flush=True)
    grads = cw.ttt_lact_swiglu_backward(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO.cuda(), cfg.chunk,
                                        cfg.eta, order, update_mask=mask)
    torch.cuda.synchronize()
    ref = olact.lact_backward(*(ti.to_f64(x[k]) for k in ("q", "k", "v", "W1", "W3", "W2")), cfg.chunk, cfg.eta,
                              ti.to_f64(dO), order, update_mask=mask)
    errs = {name: rel(f64(got), want) for name, got, want in zip(NAMES, grads, ref)}
    assert all(e < TOL[dtype] for e in errs.values()), errs
    for gt in grads[1:3]:
        assert not torch.any(gt[:, :, cfg.chunk:3 * cfg.chunk])
    # an all-ones mask is the plain backward, bit for bit
    ones = cw.ttt_lact_swiglu_backward(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO.cuda(), cfg.chunk,
                                       cfg.eta, order, update_mask=[1] * 4)
    plain = run(cfg, x, dO)
    for a, b in zip(ones, plain):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["plain", "side", "mask", "apply_then_update"])
def test_lact_backward_with_kept_states(dtype, variant):
    """States kept by the forward call (ttt_lact_options.W_states; on two streams, with an update mask, or in
    apply-then-update order) give the backward that recomputes them, bit for bit; slot 0 holds the initial weights
    and the last slot the final state in the layer's dtype."""
    order = "apply_then_update" if variant == "apply_then_update" else "update_then_apply"
    cfg, x, dO = case(dtype, order, n=512, seed=85)
    mask = [1, 0, 1, 1] if variant == "mask" else None
    g = {k: v.cuda() for k, v in x.items()}
    B, H, n, dh = g["q"].shape
    m = g["W1"].shape[1]
    k = n // cfg.chunk
    print(f"lact kept-states case: {dtype} {variant}", flush=True)
    Ws = torch.full((k + 1, B, H, 3, m * dh), float("nan"), dtype=g["q"].dtype, device="cuda")
    side = cw.LactSideStream() if variant == "side" else None
    O, W1f, W3f, W2f = cw.ttt_lact_swiglu(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta, order,
                                          update_mask=mask, side=side, W_states=Ws)
    torch.cuda.synchronize()
    assert not torch.isnan(Ws).any()
    for h in range(H):
        assert torch.equal(Ws[0, :, h, 0], g["W1"][h].reshape(-1).expand(B, -1))
        assert torch.equal(Ws[0, :, h, 2], g["W2"][h].reshape(-1).expand(B, -1))
    assert torch.equal(Ws[k, :, :, 0].float(), W1f.reshape(B, H, -1).to(Ws.dtype).float())
    assert torch.equal(Ws[k, :, :, 2].float(), W2f.reshape(B, H, -1).to(Ws.dtype).float())
    args = (g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO.cuda(), cfg.chunk, cfg.eta, order)
    kept = cw.ttt_lact_swiglu_backward(*args, update_mask=mask, W_states=Ws)
    again = cw.ttt_lact_swiglu_backward(*args, update_mask=mask)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, kept, again):
        assert torch.equal(a, b), name
