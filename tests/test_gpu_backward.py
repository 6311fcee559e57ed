"""GPU parity of the backward of the dot chunk loop (ttt_core_backward) against the float64 oracle.

The oracle's chunk_core_backward is pinned on the CPU by torch autograd and central differences.  Every call goes
through the C ABI; inputs come from the seeded generator and the oracle sees the same rounded values.  Tolerances
(relative Frobenius): 1e-4 for fp32; 2e-2 for bf16, whose path rounds the transposed operands' scale, the recomputed
states W_c and the suffix states S_c once each (about 2^-9 relative apiece) before the final contractions.
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti
from oracle import inplace as orc

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def cfg_of(dtype, B, k, C, d=264, f=392, eta=0.05, seed=31):
    return ti.InplaceConfig("bwd", B, k * C, d, f, C, eta, "dot", dtype, seed=seed, backward=True)


def run(cfg):
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    dZ, dV, dW0 = cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    return x, f64(dZ), f64(dV), f64(dW0)


def oracle(x, cfg):
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    outs = [orc.chunk_core_backward(Z[b], V[b], W0, cfg.chunk, cfg.eta, dO[b]) for b in range(cfg.batch)]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]), sum(o[2] for o in outs))


# fused scan with four segments (k = 4), one segment (k = 3), and the delta + scan path (chunk not a multiple
# of the fused scan's K step: 40 for fp32, 72 for bf16); every case has ragged 256-tiles in d and f
@pytest.mark.parametrize("dtype,C,k", [("f32", 96, 4), ("f32", 40, 3), ("bf16", 128, 4), ("bf16", 128, 3),
                                       ("bf16", 72, 2)])
def test_backward_matches_oracle(dtype, C, k):
    cfg = cfg_of(dtype, 2, k, C)
    x, dZ, dV, dW0 = run(cfg)
    rZ, rV, rW = oracle(x, cfg)
    assert rel(dZ, rZ) < TOL[dtype]
    assert rel(dV, rV) < TOL[dtype]
    assert rel(dW0, rW) < TOL[dtype]


def test_backward_single_chunk():
    # one chunk: no later chunk, so dVhat = 0 exactly and dZ = dO W_down0
    cfg = cfg_of("bf16", 1, 1, 256)
    x, dZ, dV, dW0 = run(cfg)
    rZ, rV, rW = oracle(x, cfg)
    assert not np.any(dV)
    assert rel(dZ, rZ) < TOL["bf16"] and rel(dW0, rW) < TOL["bf16"]


def test_backward_eta_zero():
    # eta = 0: the states never move and no gradient reaches Vhat; dZ = dO W_down0 for every chunk
    cfg = cfg_of("f32", 2, 3, 64, eta=0.0)
    x, dZ, dV, dW0 = run(cfg)
    assert not np.any(dV)
    ref = ti.to_f64(x["dO"]) @ ti.to_f64(x["W_down0"])
    assert rel(dZ, ref) < TOL["f32"]


def test_backward_empty():
    for B, n in ((0, 256), (2, 0)):
        cfg = ti.InplaceConfig("bwd", B, n, 264, 392, 128, 0.05, "dot", "f32", backward=True)
        x = ti.backward_inputs(cfg)
        g = {name: t.cuda() for name, t in x.items()}
        dW0 = torch.full((264, 392), float("nan"), device="cuda")
        cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], 128, 0.05, dW_down0=dW0)
        torch.cuda.synchronize()
        assert not torch.any(dW0)


def test_backward_rows_independent():
    # batch rows do not interact: row 1 alone gives row 1's dZ and dVhat bits, and dW_down0 adds the rows' parts
    cfg = cfg_of("bf16", 2, 4, 128)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    dZ, dV, dW0 = cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta)
    one = {name: (t[1:2].contiguous() if name != "W_down0" else t) for name, t in g.items()}
    dZ1, dV1, dW01 = cw.ttt_core_backward(one["Z"], one["Vhat"], one["W_down0"], one["dO"], cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    assert torch.equal(dZ[1:2], dZ1) and torch.equal(dV[1:2], dV1)
    assert rel(f64(dW0), oracle(x, cfg)[2]) < TOL["bf16"]


# packed documents: row 0 starts one every other chunk, row 1 at every chunk, row 2 holds one document; on the fused
# scan with two segments (k = 6: a segment starts inside a document, in both scan orders) and on the delta + scan path
@pytest.mark.parametrize("dtype,C,k", [("bf16", 128, 6), ("f32", 96, 4), ("bf16", 72, 4)])
def test_backward_packed_documents(dtype, C, k):
    cfg = cfg_of(dtype, 3, k, C)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    starts = np.zeros((3, k), dtype=np.uint8)
    starts[0, ::2] = 1
    starts[1, :] = 1
    dZ, dV, dW0 = cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta,
                                       doc_starts=torch.from_numpy(starts).cuda())
    torch.cuda.synchronize()
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    outs = [orc.chunk_core_backward(Z[b], V[b], W0, C, cfg.eta, dO[b], doc_starts=starts[b]) for b in range(3)]
    for b in range(3):
        assert rel(f64(dZ[b]), outs[b][0]) < TOL[dtype], b
        if b != 1:        # a document per chunk: no later chunk in any document, dV^ is exactly 0
            assert rel(f64(dV[b]), outs[b][1]) < TOL[dtype], b
    assert not torch.any(dV[1])
    assert rel(f64(dW0), sum(o[2] for o in outs)) < TOL[dtype]


# the states the forward chunk loop keeps are the ones the backward recomputes, bit for bit (same operands, same
# accumulation order), on the fused scan with segments, without, and on the delta + scan path
@pytest.mark.parametrize("dtype,C,k", [("bf16", 128, 4), ("f32", 96, 3), ("bf16", 72, 2)])
def test_backward_with_kept_states(dtype, C, k):
    cfg = cfg_of(dtype, 2, k, C)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    B, n, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    Ws = torch.full((B, k, d, f), float("nan"), dtype=g["Z"].dtype, device="cuda")
    O, Wf = cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, "dot", W_states=Ws)
    O0, Wf0 = cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, "dot")
    kept = cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, W_states=Ws)
    again = cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta)
    torch.cuda.synchronize()
    assert torch.equal(O, O0) and torch.equal(Wf, Wf0)
    assert all(torch.equal(a, b) for a, b in zip(kept, again))
    assert torch.equal(Ws[:, 0], g["W_down0"].expand(B, d, f))      # chunk 0 is applied with W_down0
    rZ, rV, rW = oracle(x, cfg)
    assert rel(f64(kept[0]), rZ) < TOL[dtype] and rel(f64(kept[1]), rV) < TOL[dtype]


def test_layer_keeps_states():
    # the whole layer hands out the states it applied; its outputs do not change
    cfg = ti.InplaceConfig("keep", 2, 1024, 264, 392, 256, 0.05, "dot", "bf16", seed=8)
    g = {name: t.cuda() for name, t in ti.inplace_inputs(cfg).items()}
    args = (g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"], cfg.chunk, cfg.eta)
    Ws = torch.full((2, 4, 264, 392), float("nan"), dtype=torch.bfloat16, device="cuda")
    O, Wf = cw.ttt_chunk_apply_update(*args, W_states=Ws)
    O0, Wf0 = cw.ttt_chunk_apply_update(*args)
    Zt = cw.ttt_produce_z(g["H"], g["W_gate"], g["W_up"], with_z=False)[1]
    O1 = cw.ttt_chunk_apply(Zt, Ws, cfg.chunk)          # the kept states reproduce the outputs
    torch.cuda.synchronize()
    assert torch.equal(O, O0) and torch.equal(Wf, Wf0) and torch.equal(O1, O)
    # the MSE scan keeps them too (one copy per chunk): chunk 0 saw W_down0, and they reproduce the outputs
    Om, Wm = cw.ttt_chunk_apply_update(*args[:-1], 0.5, "mse", W_states=Ws)
    Om0, Wm0 = cw.ttt_chunk_apply_update(*args[:-1], 0.5, "mse")
    O2 = cw.ttt_chunk_apply(Zt, Ws, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(Om, Om0) and torch.equal(Wm, Wm0)
    assert torch.equal(Ws[:, 0], g["W_down0"].expand(2, 264, 392))
    assert rel(f64(O2), f64(Om)) < 2e-3


def test_full_size_backward_sampled():
    """The 128K workload (131072 tokens, d 2560, d_ff 9728, chunk 4096).  The maps are separable: columns P of dZ
    and dW_down0 depend on columns P of Z and W_down0 only, and the last chunks' dVhat on those chunks alone (their
    suffixes), so the oracle runs on a column slice over the whole sequence and on the last two chunks."""
    cfg = ti.workload("inplace_bwd_bf16_128k")
    x, dZ, dV, dW0 = run(cfg)
    C = cfg.chunk
    rng = np.random.default_rng(5)
    P = np.sort(rng.choice(cfg.d_ff, 24, replace=False))
    Z = x["Z"][0]
    V = ti.to_f64(x["Vhat"][0])
    dO = ti.to_f64(x["dO"][0])
    W0 = ti.to_f64(x["W_down0"])
    rZ, _, rW = orc.chunk_core_backward(ti.to_f64(Z[:, P]), V, W0[:, P], C, cfg.eta, dO)
    assert rel(dZ[0][:, P], rZ) < TOL["bf16"]
    assert rel(dW0[:, P], rW) < TOL["bf16"]
    t0 = cfg.seq_len - 2 * C
    _, rV, _ = orc.chunk_core_backward(ti.to_f64(Z[t0:]), V[t0:], W0, C, cfg.eta, dO[t0:])
    assert rel(dV[0][t0:], rV) < TOL["bf16"]
    assert np.all(np.isfinite(dZ)) and np.all(np.isfinite(dV))


# ---------------------------------------------------------------- the whole layer

GRAD_NAMES = ("dH", "dX0", "dW_gate", "dW_up", "dW_down0", "dW_target", "dconv_w")


def layer_args(g):
    return (g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"])


def layer_case(dtype, B, n, C, K=4, d=264, f=392, eta=0.05, seed=41):
    cfg = ti.InplaceConfig("lbwd", B, n, d, f, C, eta, "dot", dtype, conv_k=K, seed=seed)
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(cfg.with_(seed=seed + 1))["dO"]
    return cfg, x, dO


@pytest.mark.parametrize("dtype,C,k,K", [("f32", 96, 3, 4), ("bf16", 128, 4, 4), ("bf16", 64, 3, 1), ("f32", 64, 4, 3)])
def test_layer_backward_matches_oracle(dtype, C, k, K):
    cfg, x, dO = layer_case(dtype, 2, k * C, C, K)
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), C, cfg.eta)
    torch.cuda.synchronize()
    ref = orc.layer_backward(*(ti.to_f64(x[name]) for name in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                               "conv_w")), C, cfg.eta, ti.to_f64(dO))
    for name, got, want in zip(GRAD_NAMES, grads, ref):
        assert rel(f64(got), want) < TOL[dtype], name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_backward_packed_documents(dtype):
    """Packed documents in the whole layer's backward: the convolution's gradient stops at document bounds and the
    chunk loop's suffixes at document ends; row 0 packs documents of 2, 3 and 1 chunks, row 1 of 1, 2 and 3."""
    cfg, x, dO = layer_case(dtype, 2, 6 * 128, 128, K=4)
    starts = np.array([[1, 0, 1, 0, 0, 1], [1, 1, 0, 1, 0, 0]], dtype=np.uint8)
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta,
                                  doc_starts=torch.from_numpy(starts).cuda())
    torch.cuda.synchronize()
    ref = orc.layer_backward(*(ti.to_f64(x[name]) for name in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                               "conv_w")), cfg.chunk, cfg.eta, ti.to_f64(dO),
                             doc_starts=starts)
    for name, got, want in zip(GRAD_NAMES, grads, ref):
        assert rel(f64(got), want) < TOL[dtype], name


def test_layer_backward_with_kept_states():
    # the layer's forward keeps its states; the backward given them agrees with the recomputing one
    cfg, x, dO = layer_case("bf16", 2, 512, 128)
    g = {name: t.cuda() for name, t in x.items()}
    Ws = torch.empty(2, 4, cfg.d_model, cfg.d_ff, dtype=torch.bfloat16, device="cuda")
    cw.ttt_chunk_apply_update(*layer_args(g), cfg.chunk, cfg.eta, W_states=Ws)
    kept = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta, W_states=Ws)
    again = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    for name, a, b in zip(GRAD_NAMES, kept, again):
        assert rel(f64(a), f64(b)) < 1e-2, name


def test_layer_backward_empty_and_unsupported():
    for B, n in ((0, 256), (2, 0)):
        cfg, x, dO = layer_case("f32", B, n, 128)
        g = {name: t.cuda() for name, t in x.items()}
        grads = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), 128, 0.05)
        torch.cuda.synchronize()
        assert all(not torch.any(t) for t in grads[2:])
    cfg, x, dO = layer_case("bf16", 1, 240, 80)          # chunk 80: not on the fused scan's 64-token steps
    g = {name: t.cuda() for name, t in x.items()}
    with pytest.raises(cw.TTTError) as e:
        cw.ttt_layer_backward(*layer_args(g), dO.cuda(), 80, 0.05)
    assert e.value.status == cw.TTT_ERR_UNSUPPORTED


def test_full_size_layer_backward_sampled():
    """The 128K layer's backward.  Rows P of dW_gate and dW_up and columns P of dW_down0 depend on the rows P of
    W_gate, W_up and the columns P of W_down0 alone (the chunk loop's states and suffixes are column-separable and
    the target does not depend on them), so the oracle's layer backward on those 16 d_ff columns gives them exactly;
    every other gradient must be finite."""
    cfg = ti.workload("inplace_bf16_128k")
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(ti.workload("inplace_bwd_bf16_128k"))["dO"]
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    got = [f64(t) for t in grads]
    del g, grads
    P = np.sort(np.random.default_rng(6).choice(cfg.d_ff, 16, replace=False))
    f = lambda name: ti.to_f64(x[name])
    ref = orc.layer_backward(f("H"), f("X0"), f("W_gate")[P], f("W_up")[P], f("W_down0")[:, P], f("W_target"),
                             f("conv_w"), cfg.chunk, cfg.eta, ti.to_f64(dO))
    assert rel(got[2][P], ref[2]) < TOL["bf16"]
    assert rel(got[3][P], ref[3]) < TOL["bf16"]
    assert rel(got[4][:, P], ref[4]) < TOL["bf16"]
    assert all(np.all(np.isfinite(t)) for t in got)


# ---------------------------------------------------------------- the MSE chunk loop

def mse_run(cfg):
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    dZ, dV, dW0 = cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    outs = [orc.mse_core_backward(Z[b], V[b], W0, cfg.chunk, cfg.eta, dO[b]) for b in range(cfg.batch)]
    ref = (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]), sum(o[2] for o in outs))
    return (f64(dZ), f64(dV), f64(dW0)), ref


@pytest.mark.parametrize("dtype,C,k", [("f32", 96, 3), ("bf16", 128, 4), ("bf16", 72, 3), ("f32", 40, 2)])
def test_mse_backward_matches_oracle(dtype, C, k):
    cfg = cfg_of(dtype, 2, k, C, eta=0.5)
    got, ref = mse_run(cfg)
    for name, a, b in zip(("dZ", "dVhat", "dW_down0"), got, ref):
        assert rel(a, b) < TOL[dtype], name


def test_mse_backward_single_chunk_and_eta_zero():
    got, ref = mse_run(cfg_of("bf16", 2, 1, 256, eta=0.5))      # one chunk: no later state, dVhat exactly 0
    assert not np.any(got[1])
    assert rel(got[0], ref[0]) < TOL["bf16"] and rel(got[2], ref[2]) < TOL["bf16"]
    got, ref = mse_run(cfg_of("f32", 2, 3, 64, eta=0.0))        # eta = 0: dZ = dO W_down0, dVhat = 0
    assert not np.any(got[1])
    assert rel(got[0], ref[0]) < TOL["f32"] and rel(got[2], ref[2]) < TOL["f32"]


def test_mse_backward_reduced_workload():
    """The MSE workload's row count and eta at a size the oracle's fp64 loop finishes quickly: 4 rows of 4096
    tokens, d 512, d_ff 2048, chunk 512 (8 chunks)."""
    cfg = ti.workload("mse_bf16_4x64k").with_(seq_len=4096, d_model=512, d_ff=2048, chunk=512, backward=True)
    got, ref = mse_run(cfg)
    for name, a, b in zip(("dZ", "dVhat", "dW_down0"), got, ref):
        assert rel(a, b) < TOL["bf16"], name


@pytest.mark.parametrize("dtype,C", [("f32", 96), ("bf16", 128)])
def test_mse_backward_with_kept_states(dtype, C):
    # the states the MSE forward keeps stand in for the backward's recomputed ones
    cfg = cfg_of(dtype, 2, 4, C, eta=0.5)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    B, d, f = 2, cfg.d_model, cfg.d_ff
    Ws = torch.full((B, 4, d, f), float("nan"), dtype=g["Z"].dtype, device="cuda")
    cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, "mse", W_states=Ws)
    kept = cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, W_states=Ws)
    again = cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta)
    torch.cuda.synchronize()
    for name, a, b in zip(("dZ", "dVhat", "dW_down0"), kept, again):
        assert rel(f64(a), f64(b)) < 1e-3, name
    _, ref = mse_run(cfg)
    for name, a, b in zip(("dZ", "dVhat", "dW_down0"), kept, ref):
        assert rel(f64(a), b) < TOL[dtype], name


@pytest.mark.parametrize("dtype,C", [("f32", 96), ("bf16", 128)])
def test_mse_backward_packed_documents(dtype, C):
    """Packed documents in the MSE loop's backward (recomputed states, and states kept by the forward call with the
    same document starts): row 0 starts a document every other chunk, row 1 at every chunk, row 2 holds one."""
    cfg = cfg_of(dtype, 3, 6, C, eta=0.5)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    starts = np.zeros((3, 6), dtype=np.uint8)
    starts[0, ::2] = 1
    starts[1, :] = 1
    dst = torch.from_numpy(starts).cuda()
    got = cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, doc_starts=dst)
    Ws = torch.empty(3, 6, cfg.d_model, cfg.d_ff, dtype=g["Z"].dtype, device="cuda")
    cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, "mse", W_states=Ws, doc_starts=dst)
    kept = cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, doc_starts=dst, W_states=Ws)
    torch.cuda.synchronize()
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    outs = [orc.mse_core_backward(Z[b], V[b], W0, C, cfg.eta, dO[b], doc_starts=starts[b]) for b in range(3)]
    ref = (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]), sum(o[2] for o in outs))
    for res in (got, kept):
        for name, a, b in zip(("dZ", "dVhat", "dW_down0"), res, ref):
            assert rel(f64(a), b) < TOL[dtype], name
    assert not torch.any(got[1][1])       # a document per chunk: no later state in any document


# ---------------------------------------------------------------- the whole MSE layer

def mse_layer_case(dtype, B, n, C, K=4, d=264, f=392, eta=0.5, seed=61):
    cfg = ti.InplaceConfig("mlbwd", B, n, d, f, C, eta, "mse", dtype, conv_k=K, seed=seed)
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(cfg.with_(seed=seed + 1))["dO"]
    return cfg, x, dO


def mse_layer_ref(cfg, x, dO, doc_starts=None):
    return orc.layer_backward(*(ti.to_f64(x[name]) for name in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                                "conv_w")), cfg.chunk, cfg.eta, ti.to_f64(dO),
                              doc_starts=doc_starts, mode="mse")


@pytest.mark.parametrize("dtype,C,k,K", [("f32", 96, 3, 4), ("bf16", 128, 4, 4), ("bf16", 64, 3, 1),
                                         ("f32", 64, 4, 3)])
def test_mse_layer_backward_matches_oracle(dtype, C, k, K):
    """Every gradient of the whole MSE-objective layer (ttt_layer_backward_mse) against the oracle, two rows sharing
    the weights, ragged 256-tiles in d and f."""
    cfg, x, dO = mse_layer_case(dtype, 2, k * C, C, K)
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), C, cfg.eta)
    torch.cuda.synchronize()
    for name, got, want in zip(GRAD_NAMES, grads, mse_layer_ref(cfg, x, dO)):
        assert rel(f64(got), want) < TOL[dtype], name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mse_layer_backward_packed_documents_and_kept_states(dtype):
    """Packed documents (row 0: documents of 2, 3 and 1 chunks; row 1: 1, 2 and 3) with the states recomputed and
    with the states the MSE forward layer kept under the same document starts."""
    cfg, x, dO = mse_layer_case(dtype, 2, 6 * 128, 128)
    starts = np.array([[1, 0, 1, 0, 0, 1], [1, 1, 0, 1, 0, 0]], dtype=np.uint8)
    dst = torch.from_numpy(starts).cuda()
    g = {name: t.cuda() for name, t in x.items()}
    got = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta, doc_starts=dst)
    Ws = torch.empty(2, 6, cfg.d_model, cfg.d_ff, dtype=g["H"].dtype, device="cuda")
    cw.ttt_chunk_apply_update(*layer_args(g), cfg.chunk, cfg.eta, "mse", W_states=Ws, doc_starts=dst)
    kept = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta, doc_starts=dst, W_states=Ws)
    torch.cuda.synchronize()
    ref = mse_layer_ref(cfg, x, dO, doc_starts=starts)
    for res in (got, kept):
        for name, a, want in zip(GRAD_NAMES, res, ref):
            assert rel(f64(a), want) < TOL[dtype], name


def test_mse_layer_backward_single_chunk_empty_and_unsupported():
    # one chunk: the targets reach no output, so dX0, dW_target and the taps' gradient are exactly zero
    cfg, x, dO = mse_layer_case("bf16", 2, 256, 256)
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    assert not torch.any(grads[1]) and not torch.any(grads[5]) and not torch.any(grads[6])
    ref = mse_layer_ref(cfg, x, dO)
    for i in (0, 2, 3, 4):
        assert rel(f64(grads[i]), ref[i]) < TOL["bf16"], GRAD_NAMES[i]
    for B, n in ((0, 256), (2, 0)):
        cfg, x, dO = mse_layer_case("f32", B, n, 128)
        g = {name: t.cuda() for name, t in x.items()}
        grads = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), 128, 0.5)
        torch.cuda.synchronize()
        assert all(not torch.any(t) for t in grads[2:])
    cfg, x, dO = mse_layer_case("bf16", 1, 240, 80)
    g = {name: t.cuda() for name, t in x.items()}
    with pytest.raises(cw.TTTError) as e:
        cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), 80, 0.5)
    assert e.value.status == cw.TTT_ERR_UNSUPPORTED


def test_mse_layer_backward_reduced_workload():
    """The MSE workload's rows, conv width and eta at a size the oracle finishes in seconds: 4 rows of 4096 tokens,
    d 512, d_ff 2048, chunk 512 (8 chunks)."""
    cfg = ti.workload("mse_bf16_4x64k").with_(seq_len=4096, d_model=512, d_ff=2048, chunk=512)
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(cfg.with_(seed=cfg.seed + 3, backward=True))["dO"]
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward_mse(*layer_args(g), dO.cuda(), cfg.chunk, cfg.eta)
    torch.cuda.synchronize()
    for name, got, want in zip(GRAD_NAMES, grads, mse_layer_ref(cfg, x, dO)):
        assert rel(f64(got), want) < TOL["bf16"], name


# ---------------------------------------------------------------- update masks and the forward conv

@pytest.mark.parametrize("mode,dtype,C,k", [("dot", "f32", 96, 4), ("dot", "bf16", 128, 4), ("dot", "bf16", 72, 3),
                                            ("mse", "f32", 96, 4), ("mse", "bf16", 128, 4)])
def test_core_backward_with_update_mask(mode, dtype, C, k):
    """The chunk loop's backward with an update mask (ttt_core_backward_ex): two rows with different masks, on the
    fused scan with segments, the delta + scan path (chunk 72) and the MSE recursion; masked chunks' dVhat rows
    exactly zero; the states the masked forward call keeps give the same results."""
    cfg = cfg_of(dtype, 2, k, C, eta=0.05 if mode == "dot" else 0.5, seed=33).with_(mode=mode)
    x = ti.backward_inputs(cfg)
    g = {name: t.cuda() for name, t in x.items()}
    mask = np.array([[1, 0, 1, 1][:k], [0, 1, 1, 0][:k]], dtype=np.uint8)
    um = torch.from_numpy(mask).cuda()
    fn = cw.ttt_core_backward if mode == "dot" else cw.ttt_core_backward_mse
    got = fn(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, update_mask=um)
    Ws = torch.empty(2, k, cfg.d_model, cfg.d_ff, dtype=g["Z"].dtype, device="cuda")
    cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, mode, W_states=Ws, update_mask=um)
    kept = fn(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, update_mask=um, W_states=Ws)
    torch.cuda.synchronize()
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    back = orc.chunk_core_backward if mode == "dot" else orc.mse_core_backward
    outs = [back(Z[b], V[b], W0, C, cfg.eta, dO[b], update_mask=mask[b]) for b in range(2)]
    ref = (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]), sum(o[2] for o in outs))
    for res in (got, kept):
        for name, a, b in zip(("dZ", "dVhat", "dW_down0"), res, ref):
            assert rel(f64(a), b) < TOL[dtype], name
    for b in range(2):
        for c in range(k):
            if not mask[b, c]:
                assert not torch.any(got[1][b, c * C:(c + 1) * C]), (b, c)


@pytest.mark.parametrize("mode", ["dot", "mse"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_backward_forward_conv_and_mask(mode, dtype):
    """The whole layer's backward (ttt_layer_backward_ex) with the forward-looking in-chunk convolution and an
    update mask, two rows with different masks, K = 4, ragged 264 x 392, four chunks."""
    C = 128
    cfg = ti.InplaceConfig("lbwdx", 2, 4 * C, 264, 392, C, 0.05 if mode == "dot" else 0.5, mode, dtype, seed=65)
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(cfg.with_(seed=66))["dO"]
    mask = np.array([[1, 0, 1, 1], [0, 1, 0, 1]], dtype=np.uint8)
    g = {name: t.cuda() for name, t in x.items()}
    grads = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), C, cfg.eta, mode=mode,
                                  update_mask=torch.from_numpy(mask).cuda(), conv_forward=True)
    torch.cuda.synchronize()
    ref = orc.layer_backward(*(ti.to_f64(x[name]) for name in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                               "conv_w")), C, cfg.eta, ti.to_f64(dO), mode=mode,
                             update_mask=mask, conv_forward=True)
    for name, got, want in zip(GRAD_NAMES, grads, ref):
        assert rel(f64(got), want) < TOL[dtype], name


# ---------------------------------------------------------------- resumed rows

@pytest.mark.parametrize("mode,dtype,C,k", [("dot", "f32", 96, 4), ("dot", "bf16", 128, 4), ("dot", "bf16", 72, 3),
                                            ("mse", "f32", 96, 4), ("mse", "bf16", 128, 4)])
@pytest.mark.parametrize("packed", [False, True])
def test_core_backward_resumed_rows(mode, dtype, C, k, packed):
    """The chunk loop's backward of resumed rows (ttt_core_backward_ex with W_init): dZ, dVhat, dW_down0 and
    dW_init against the oracle, on the fused scan with segments, the delta + scan path (chunk 72) and the MSE
    recursion.  Packed: row 0 continues into a second document at chunk 2, row 1 is flagged at chunk 0 (it starts
    from W_down0 and its dW_init is exactly zero).  The states the resumed forward call keeps give the same
    results."""
    cfg = cfg_of(dtype, 2, k, C, eta=0.05 if mode == "dot" else 0.5, seed=35).with_(mode=mode)
    x = ti.backward_inputs(cfg)
    r = ti.resume_inputs(cfg, seed=36)
    g = {name: t.cuda() for name, t in x.items()}
    Wi = r["W_init"].cuda()
    starts = np.zeros((2, k), dtype=np.uint8)
    if packed:
        starts[0, 2] = 1
        starts[1, 0] = 1
    ds = torch.from_numpy(starts).cuda() if packed else None
    fn = cw.ttt_core_backward if mode == "dot" else cw.ttt_core_backward_mse
    got = fn(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, doc_starts=ds, W_init=Wi)
    Ws = torch.empty(2, k, cfg.d_model, cfg.d_ff, dtype=g["Z"].dtype, device="cuda")
    cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], C, cfg.eta, mode, W_states=Ws, doc_starts=ds,
                             W_init=Wi)
    kept = fn(g["Z"], g["Vhat"], g["W_down0"], g["dO"], C, cfg.eta, doc_starts=ds, W_init=Wi, W_states=Ws)
    torch.cuda.synchronize()
    Z, V, W0, dO = (ti.to_f64(x[name]) for name in ("Z", "Vhat", "W_down0", "dO"))
    Wi64 = r["W_init"].double().numpy()
    outs = [orc.resumed_core_backward(Z[b], V[b], W0, Wi64[b], C, cfg.eta, dO[b], mode,
                                      doc_starts=starts[b] if packed else None) for b in range(2)]
    ref = (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]), sum(o[2] for o in outs),
           np.stack([o[3] for o in outs]))
    for res in (got, kept):
        for name, a, b in zip(("dZ", "dVhat", "dW_down0"), res, ref):
            assert rel(f64(a), b) < TOL[dtype], name
        for b in range(2):
            if packed and b == 1:
                assert not torch.any(res[3][1])
            else:
                assert rel(f64(res[3][b]), ref[3][b]) < TOL[dtype], ("dW_init", b)
    if not packed:                       # every row continues: nothing starts from W_down0
        assert not torch.any(got[2])


@pytest.mark.parametrize("mode", ["dot", "mse"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["both", "halo_only", "forward_conv"])
def test_layer_backward_resumed_rows(mode, dtype, case):
    """The whole layer's backward of resumed rows (ttt_layer_backward_ex with W_init and x0_halo, K = 4, ragged
    264 x 392, four chunks): three rows -- one continuing into a second document at chunk 2, one flagged at chunk 0
    (zero dW_init and dx0_halo), one continuing to its end -- every gradient against the oracle, dW_init and
    dx0_halo included.  halo_only: the first documents start from W_down0; forward_conv: the halo is never read
    (dx0_halo zero)."""
    C, K = 128, 4
    cfg = ti.InplaceConfig("lbwdr", 3, 4 * C, 264, 392, C, 0.05 if mode == "dot" else 0.5, mode, dtype, conv_k=K,
                           seed=67)
    x = ti.inplace_inputs(cfg)
    dO = ti.backward_inputs(cfg.with_(seed=68))["dO"]
    r = ti.resume_inputs(cfg, seed=69)
    starts = np.array([[0, 0, 1, 0], [1, 0, 0, 1], [0, 0, 0, 0]], dtype=np.uint8)
    g = {name: t.cuda() for name, t in x.items()}
    Wi = None if case == "halo_only" else r["W_init"].cuda()
    fwd = case == "forward_conv"
    res = cw.ttt_layer_backward(*layer_args(g), dO.cuda(), C, cfg.eta, mode=mode,
                                doc_starts=torch.from_numpy(starts).cuda(), conv_forward=fwd, W_init=Wi,
                                x0_halo=r["x0_halo"].cuda())
    torch.cuda.synchronize()
    assert len(res) == 9 and (res[7] is None) == (Wi is None)
    ref = orc.layer_backward(*(ti.to_f64(x[name]) for name in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                               "conv_w")), C, cfg.eta, ti.to_f64(dO),
                             doc_starts=starts, mode=mode, conv_forward=fwd,
                             W_init=None if Wi is None else r["W_init"].double().numpy(),
                             x0_halo=ti.to_f64(r["x0_halo"]))
    for name, got, want in zip(GRAD_NAMES, res[:7], ref[:7]):
        assert rel(f64(got), want) < TOL[dtype], name
    if Wi is not None:
        for b in (0, 2):
            assert rel(f64(res[7][b]), ref[7][b]) < TOL[dtype], ("dW_init", b)
        assert not torch.any(res[7][1])
    if fwd:
        assert not torch.any(res[8])
    else:
        for b in (0, 2):
            assert rel(f64(res[8][b]), ref[8][b]) < TOL[dtype], ("dx0_halo", b)
        assert not torch.any(res[8][1])
