"""GPU parity of the LaCT SwiGLU fast-weight layer against the float64 oracle.

Calls go through the C ABI (ttt_lact_swiglu).  Tolerances as for the
In-Place layer: relative Frobenius <= 1e-4 (fp32), <= 2e-2 (bf16 storage,
fp32 accumulation and fp32 states); the update W_final - W0 is compared on its
own as well so that the learned part is pinned, not just the initial weights.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti
from oracle import lact as olact

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def cfg_small(dtype="f32", order="update_then_apply", B=1, H=2, n=512, dh=64, m=128, C=128, eta=1.0, seed=5):
    return ti.LactConfig("small", B, H, n, dh, m, C, eta, order, dtype, seed=seed)


def run(cfg):
    x = ti.lact_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    O, W1f, W3f, W2f = cw.ttt_lact_swiglu(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta,
                                          cfg.order)
    torch.cuda.synchronize()
    return x, O, W1f, W3f, W2f


def check(cfg, x, O, W1f, W3f, W2f, tol=None):
    tol = tol or TOL[cfg.dtype]
    ref = olact.lact_layer(*(ti.to_f64(x[k]) for k in ("q", "k", "v", "W1", "W3", "W2")), cfg.chunk, cfg.eta,
                           cfg.order)
    Oref, W1r, W3r, W2r = ref
    errs = {"O": rel(f64(O), Oref)}
    for name, got, want, init in (("W1", W1f, W1r, x["W1"]), ("W3", W3f, W3r, x["W3"]), ("W2", W2f, W2r, x["W2"])):
        w0 = ti.to_f64(init)[None]
        errs[name] = rel(f64(got), want)
        errs[name + "_delta"] = rel(f64(got) - w0, want - w0)
    assert all(v < tol for v in errs.values()), errs
    return errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_lact_small(dtype, order):
    cfg = cfg_small(dtype, order)
    check(cfg, *run(cfg))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lact_ragged_dims_and_batch(dtype):
    # head_dim and hidden not multiples of the 64-element K step or the tiles; 2 x 2 (batch, head) states
    cfg = cfg_small(dtype, B=2, H=2, n=384, dh=72, m=136, C=96, eta=0.7, seed=9)
    check(cfg, *run(cfg))


def test_lact_eta_zero_is_plain_swiglu():
    cfg = cfg_small("bf16", eta=0.0)
    x, O, W1f, W3f, W2f = run(cfg)
    for h in range(cfg.heads):
        ref = olact.swiglu_apply(ti.to_f64(x["q"])[0, h], ti.to_f64(x["W1"])[h], ti.to_f64(x["W3"])[h],
                                 ti.to_f64(x["W2"])[h])
        assert rel(f64(O[0, h]), ref) < TOL["bf16"]
    assert np.array_equal(f64(W1f[0]), ti.to_f64(x["W1"]))
    assert np.array_equal(f64(W2f[0]), ti.to_f64(x["W2"]))


@pytest.mark.parametrize("two_chains", [False, True])
@pytest.mark.parametrize("B,H", [(1, 3), (3, 1), (2, 2)])
def test_lact_rows_equal_single_row_calls(B, H, two_chains):
    """Every (batch, head) row is an independent fast weight.  A call on B x H rows (in one chain, or split into
    two groups whose chains run on the caller's stream and a side stream, unevenly for 3 rows) gives each row bit
    for bit what a call on that row alone gives, and a repeated call gives the same bits."""
    cfg = cfg_small("bf16", B=B, H=H, n=384, dh=64, m=128, C=128, eta=0.7, seed=11)
    x = ti.lact_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    side = cw.LactSideStream() if two_chains else None
    call = lambda q, k, v, W1, W3, W2: cw.ttt_lact_swiglu(q, k, v, W1, W3, W2, cfg.chunk, cfg.eta, cfg.order,
                                                          side=side)
    full = call(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"])
    again = call(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"])
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(full, again))
    for b in range(B):
        for h in range(H):
            row = lambda t: t[b:b + 1, h:h + 1].contiguous()
            head = lambda t: t[h:h + 1].contiguous()
            one = call(row(g["q"]), row(g["k"]), row(g["v"]), head(g["W1"]), head(g["W3"]), head(g["W2"]))
            torch.cuda.synchronize()
            for got, want in zip(one, full):
                assert torch.equal(got[0, 0], want[b, h]), (b, h)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
def test_lact_update_mask(dtype, order):
    """Strided update (ttt_lact_swiglu_ex, option update_mask): only the flagged chunks take the gradient step, every chunk is
    applied, against the oracle with the same mask on 2 x 2 rows (run as two chains with a side stream); the first
    chunk is masked, which leaves the first update-then-apply step with nothing to do.  An all-on mask gives the
    unmasked call's bits, and one chain the two chains' bits."""
    cfg = cfg_small(dtype, order, B=2, H=2, n=768, dh=64, m=128, C=128, eta=0.8, seed=21)
    mask = [0, 1, 1, 0, 1, 0]
    x = ti.lact_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    args = (g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta, cfg.order)
    got = cw.ttt_lact_swiglu(*args, update_mask=mask, side=cw.LactSideStream())
    one_chain = cw.ttt_lact_swiglu(*args, update_mask=mask)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, one_chain))
    plain = cw.ttt_lact_swiglu(*args)
    all_on = cw.ttt_lact_swiglu(*args, update_mask=[1] * len(mask))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(all_on, plain))
    Oref, W1r, W3r, W2r = olact.lact_layer(*(ti.to_f64(x[k]) for k in ("q", "k", "v", "W1", "W3", "W2")), cfg.chunk,
                                           cfg.eta, cfg.order, update_mask=mask)
    tol = TOL[dtype]
    errs = {"O": rel(f64(got[0]), Oref)}
    for name, t, want, init in (("W1", got[1], W1r, x["W1"]), ("W3", got[2], W3r, x["W3"]), ("W2", got[3], W2r, x["W2"])):
        w0 = ti.to_f64(init)[None]
        errs[name] = rel(f64(t), want)
        errs[name + "_delta"] = rel(f64(t) - w0, want - w0)
    assert all(e < tol for e in errs.values()), errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
@pytest.mark.parametrize("variant", ["eta_tok", "dot", "weight_norm", "all", "muon", "muon_weight_norm"])
def test_lact_update_variants(dtype, order, variant):
    """LaCT's update variants (ttt_lact_swiglu_ex): per-token learning rates, the dot-product loss, L2 weight
    normalisation after each update, all three with an update mask, and the Muon rule (Newton-Schulz on the
    gradients, dh 64 < m 128 so W1 and W3's gradients are iterated transposed) with and without normalisation,
    against the oracle on 2 heads."""
    cfg = cfg_small(dtype, order, B=1, H=2, n=512, dh=64, m=128, C=128, seed=23,
                    eta={"dot": 0.1, "all": 0.1, "muon": 0.05, "muon_weight_norm": 0.05}.get(variant, 0.6))
    x = ti.lact_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    rates = np.random.default_rng(24).uniform(0.2, 1.2, size=(cfg.batch, cfg.heads, cfg.seq_len))
    kw, okw = {}, {}
    if variant in ("eta_tok", "all"):
        kw["eta_tok"] = torch.from_numpy(rates).float().cuda()
        okw["eta_tok"] = kw["eta_tok"].double().cpu().numpy()      # the rates the kernel sees (fp32)
    if variant in ("dot", "all"):
        kw["loss"] = okw["loss"] = "dot"
    if variant in ("weight_norm", "all", "muon_weight_norm"):
        kw["weight_norm"] = okw["weight_norm"] = True
    if variant.startswith("muon"):
        kw["muon"] = okw["use_muon"] = True
    if variant == "all":
        kw["update_mask"] = okw["update_mask"] = [1, 0, 1, 1]
    got = cw.ttt_lact_swiglu(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta, cfg.order, **kw)
    torch.cuda.synchronize()
    Oref, W1r, W3r, W2r = olact.lact_layer(*(ti.to_f64(x[k]) for k in ("q", "k", "v", "W1", "W3", "W2")), cfg.chunk,
                                           cfg.eta, cfg.order, **okw)
    tol = TOL[dtype]
    errs = {"O": rel(f64(got[0]), Oref)}
    for name, t, want, init in (("W1", got[1], W1r, x["W1"]), ("W3", got[2], W3r, x["W3"]),
                                ("W2", got[3], W2r, x["W2"])):
        w0 = ti.to_f64(init)[None]
        errs[name] = rel(f64(t), want)
        errs[name + "_delta"] = rel(f64(t) - w0, want - w0)
    assert all(e < tol for e in errs.values()), errs
    if variant in ("weight_norm", "all", "muon_weight_norm"):
        for t in got[1:]:
            assert torch.allclose(t.norm(dim=-1), torch.ones((), device=t.device), atol=1e-5)


def test_lact_single_chunk_full_batch_step():
    cfg = cfg_small("f32", n=256, C=256)
    check(cfg, *run(cfg))


def test_lact_causality_update_then_apply():
    cfg = cfg_small("bf16", n=512, C=128)
    x = ti.lact_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    args = lambda gg: (gg["q"], gg["k"], gg["v"], gg["W1"], gg["W3"], gg["W2"], cfg.chunk, cfg.eta, cfg.order)
    O = cw.ttt_lact_swiglu(*args(g))[0]
    g2 = dict(g)
    for name in ("q", "k", "v"):
        g2[name] = g[name].clone()
        g2[name][:, :, 2 * cfg.chunk:] = g[name][:, :, 2 * cfg.chunk:].flip(2)
    O2 = cw.ttt_lact_swiglu(*args(g2))[0]
    torch.cuda.synchronize()
    assert torch.equal(O[:, :, : 2 * cfg.chunk], O2[:, :, : 2 * cfg.chunk])
    assert not torch.equal(O[:, :, 2 * cfg.chunk:], O2[:, :, 2 * cfg.chunk:])


def test_lact_workload_shapes_two_chunks():
    """The workload's head_dim 512, hidden 1024, chunk 4096, eta 1, on two chunks of one head."""
    cfg = ti.workload("lact_bf16_256k").with_(heads=1, seq_len=8192)
    check(cfg, *run(cfg))


@pytest.mark.slow
def test_lact_full_size():
    """The full 256K workload (4 heads, head_dim 512, hidden 1024, chunk 4096, 64 chunks, eta 1), called as the
    bench calls it, against the oracle on every element of O, the three final states and their updates
    W_final - W0.  The oracle runs one head at a time (LaCT Model Architecture §1, eq. (3)-(4))."""
    cfg = ti.workload("lact_bf16_256k")
    print(f"full-size case: lact B={cfg.batch} H={cfg.heads} n={cfg.seq_len} dh={cfg.head_dim} m={cfg.hidden} "
          f"C={cfg.chunk}", flush=True)
    x, O, W1f, W3f, W2f = run(cfg)
    O, W1f, W3f, W2f = O.cpu(), W1f.cpu(), W3f.cpu(), W2f.cpu()
    torch.cuda.empty_cache()
    C = cfg.chunk
    acc = {k: [0.0, 0.0] for k in ("O", "W1", "W3", "W2", "dW1", "dW3", "dW2")}

    def add(key, got, want):
        acc[key][0] += float(np.sum((got - want) ** 2))
        acc[key][1] += float(np.sum(want ** 2))

    for h in range(cfg.heads):
        sub = {k: ti.to_f64(v[:, h:h + 1]) if k in ("q", "k", "v") else ti.to_f64(v[h:h + 1])
               for k, v in x.items()}
        Oref, W1r, W3r, W2r = olact.lact_layer(sub["q"], sub["k"], sub["v"], sub["W1"], sub["W3"], sub["W2"], C,
                                               cfg.eta, cfg.order)
        add("O", f64(O[:, h:h + 1]), Oref)
        for key, got, ref, w0 in (("W1", W1f, W1r, sub["W1"]), ("W3", W3f, W3r, sub["W3"]),
                                  ("W2", W2f, W2r, sub["W2"])):
            gh = f64(got[:, h:h + 1])
            add(key, gh, ref)
            add("d" + key, gh - w0[None], ref - w0[None])
        print(f"  head {h}: done", flush=True)
    errs = {k: float(np.sqrt(a / b)) for k, (a, b) in acc.items()}
    print("  rel err " + "  ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) < TOL["bf16"], errs
