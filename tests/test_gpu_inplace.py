"""GPU parity of the In-Place TTT layer against the float64 oracle.

Every call goes through the C ABI (ctypes binding).  Inputs come from the
seeded generators; the oracle sees the same (already rounded) values.
Tolerances: relative Frobenius <= 1e-4 for fp32 end to end, <= 2e-2 for bf16
storage with fp32 accumulation (each bf16 rounding of an intermediate costs
about 2^-9 relative; the layer rounds Z, V^, the applied state and O once
each, so the expected error is a few 1e-3).
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti
from oracle import inplace as orc

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
STEP_TOL = {"f32": 2e-5, "bf16": 1e-2}


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def dev(inputs):
    return {k: v.cuda() for k, v in inputs.items()}


def small_cfg(dtype, mode, B=1, n=1024, d=264, f=392, C=256, eta=0.05, K=4, seed=7):
    return ti.InplaceConfig("small", B, n, d, f, C, eta, mode, dtype, conv_k=K, seed=seed)


# ---------------------------------------------------------------- individual steps

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_produce_z(dtype):
    cfg = small_cfg(dtype, "dot", B=2, n=520, d=264, f=392)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    Z, Zt = cw.ttt_produce_z(g["H"], g["W_gate"], g["W_up"])
    torch.cuda.synchronize()
    ref = orc.gated_intermediate(ti.to_f64(x["H"]).reshape(-1, cfg.d_model), ti.to_f64(x["W_gate"]),
                                 ti.to_f64(x["W_up"])).reshape(2, 520, 392)
    assert rel(f64(Z), ref) < STEP_TOL[dtype]
    assert torch.equal(Zt, Z.transpose(1, 2).contiguous())      # the two layouts hold the same values
    _, Zt_only = cw.ttt_produce_z(g["H"], g["W_gate"], g["W_up"], with_z=False)
    torch.cuda.synchronize()
    assert torch.equal(Zt_only, Zt)


@pytest.mark.parametrize("dtype,K", [("f32", 4), ("bf16", 4), ("bf16", 1), ("bf16", 3), ("f32", 8)])
def test_produce_vhat(dtype, K):
    cfg = small_cfg(dtype, "dot", B=2, n=384, d=328, f=64, K=K)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    Vt = cw.ttt_produce_vhat(g["X0"], g["conv_w"], g["W_target"])
    Vt_s = cw.ttt_produce_vhat(g["X0"], g["conv_w"], g["W_target"], scale=0.25)
    torch.cuda.synchronize()
    ref = orc.target_values(ti.to_f64(x["X0"]), ti.to_f64(x["conv_w"]), ti.to_f64(x["W_target"]))
    assert rel(f64(Vt), ref.transpose(0, 2, 1)) < STEP_TOL[dtype]
    assert rel(f64(Vt_s), 0.25 * ref.transpose(0, 2, 1)) < STEP_TOL[dtype]


def _zv(dtype, B, n, d, f, seed):
    gen = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Z = (torch.randn(B, n, f, generator=gen) * 0.6).to(dt)
    V = torch.randn(B, n, d, generator=gen).to(dt)
    W0 = (torch.randn(d, f, generator=gen) / np.sqrt(f)).to(dt)
    return Z, V, W0


def _t(x):
    return x.transpose(1, 2).contiguous()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_delta_scan_apply_steps(dtype):
    B, n, d, f, C, eta = 2, 768, 264, 392, 192, 0.02
    Z, V, W0 = _zv(dtype, B, n, d, f, 11)
    Wg = W0.cuda()
    dW = cw.ttt_chunk_delta(_t(Z).cuda(), _t(V).cuda(), C)
    Wc, Wf = cw.ttt_chunk_scan(dW, Wg, eta, C, n)
    O = cw.ttt_chunk_apply(_t(Z).cuda(), Wc, C)
    torch.cuda.synchronize()
    Zn, Vn, W0n = f64(Z), f64(V), f64(W0)
    k = n // C
    for b in range(B):
        dref = np.stack([Vn[b, c * C:(c + 1) * C].T @ Zn[b, c * C:(c + 1) * C] for c in range(k)])
        assert rel(f64(dW[b]), dref) < 1e-5
        Oref, Wref = orc.chunk_prefix_form(Zn[b], Vn[b], W0n, C, eta)
        assert rel(f64(Wf[b]), Wref) < 1e-5
        assert rel(f64(Wf[b]) - W0n, Wref - W0n) < 1e-5
        pref = np.concatenate([np.zeros((1, d, f)), np.cumsum(dref, axis=0)[:-1]])
        assert rel(f64(Wc[b]), W0n + eta * pref) < STEP_TOL[dtype]
        assert rel(f64(O[b]), Oref) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_update_scan_matches_materialised(dtype):
    B, n, d, f, C, eta = 2, 1024, 264, 520, 256, 0.02
    Z, V, W0 = _zv(dtype, B, n, d, f, 12)
    dt = Z.dtype
    Vs = (V.double() * eta).to(dt)                # the eta-scaled target the fused update takes
    Zt, Wg = _t(Z).cuda(), W0.cuda()
    Wc1, Wf1 = cw.ttt_chunk_update_scan(Zt, _t(Vs).cuda(), Wg, C)
    Wc2, Wf2 = cw.ttt_chunk_scan(cw.ttt_chunk_delta(Zt, _t(V).cuda(), C), Wg, eta, C, n)
    torch.cuda.synchronize()
    Zn, Vsn, W0n = f64(Z), f64(Vs), f64(W0)
    for b in range(B):
        _, Wref = orc.chunk_prefix_form(Zn[b], Vsn[b], W0n, C, 1.0)
        assert rel(f64(Wf1[b]), Wref) < 1e-5
        assert rel(f64(Wf1[b]) - W0n, Wref - W0n) < 1e-5
    assert rel(f64(Wc1), f64(Wc2)) < STEP_TOL[dtype]
    assert rel(f64(Wf1), f64(Wf2)) < STEP_TOL[dtype]
    assert torch.equal(Wc1[:, 0], Wg.expand(B, d, f))      # chunk 0 is applied with W_down0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,n,d,f,C,segments", [
    (1, 2048, 1024, 4096, 256, 4),     # 64 state tiles: four sequence segments and the fix-up pass
    (2, 1024, 1024, 4096, 128, 4),     # two batch rows of 64 tiles: four segments each
    (1, 1024, 2560, 6656, 256, 2),     # 260 tiles: two chained segments (three rounds of tiles)
    (2, 512, 2560, 6656, 256, 2),      # two rows, one chunk per chained segment
])
def test_segmented_update_scan(dtype, B, n, d, f, C, segments):
    """The fused update-scan cut into sequence segments equals the materialised deltas + scan and the oracle's
    prefix form: with four segments the later segments' partial states receive the earlier totals in the fix-up
    pass, with two the second segment takes the first's end state inside the kernel."""
    shape = cw.InplaceShape(B, n, d, f, C, 1)
    k = n // C
    DF = d * f
    al = lambda x: (x + 255) // 256 * 256
    esz = 2 if dtype == "bf16" else 4
    want_ws = al(B * (k - k // segments) * DF * esz) + al(B * (segments - 1) * DF * 4)
    assert cw.ttt_update_scan_workspace_bytes(shape, torch.bfloat16 if dtype == "bf16" else torch.float32) == want_ws
    eta = 0.02
    Z, V, W0 = _zv(dtype, B, n, d, f, 31)
    dt = Z.dtype
    Vs = (V.double() * eta).to(dt)
    Zt, Wg = _t(Z).cuda(), W0.cuda()
    Wc1, Wf1 = cw.ttt_chunk_update_scan(Zt, _t(Vs).cuda(), Wg, C)
    Wc2, Wf2 = cw.ttt_chunk_scan(cw.ttt_chunk_delta(Zt, _t(V).cuda(), C), Wg, eta, C, n)
    torch.cuda.synchronize()
    assert rel(f64(Wc1), f64(Wc2)) < STEP_TOL[dtype]
    assert rel(f64(Wf1), f64(Wf2)) < STEP_TOL[dtype]
    Zn, Vsn, W0n = f64(Z), f64(Vs), f64(W0)
    for b in range(B):
        _, Wref = orc.chunk_prefix_form(Zn[b], Vsn[b], W0n, C, 1.0)
        assert rel(f64(Wf1[b]) - W0n, Wref - W0n) < 1e-5
        # every chunk's state, segment starts included
        Wcs = f64(Wc1[b])
        for c in range(k):
            _, Wc_ref = orc.chunk_prefix_form(Zn[b, : c * C], Vsn[b, : c * C], W0n, C, 1.0) if c else (None, W0n)
            assert rel(Wcs[c], Wc_ref) < STEP_TOL[dtype], (b, c)


def test_core_update_first_on_a_four_segment_shape():
    """A state of 64 tiles with 8 chunks, which the fused dot plan would scan as four sequence segments: in the
    update-then-apply order it runs one (the states after each step), against the oracle in that order."""
    B, n, d, f, C, eta = 1, 2048, 1024, 4096, 256, 0.02
    Z, V, W0 = _zv("bf16", B, n, d, f, 43)
    O, Wf = cw.ttt_core_apply_update(Z.cuda(), V.cuda(), W0.cuda(), C, eta, "dot", update_first=True)
    Oa, Wa = cw.ttt_core_apply_update(Z.cuda(), V.cuda(), W0.cuda(), C, eta, "dot")
    torch.cuda.synchronize()
    Oref, Wref = orc.chunk_apply_update(f64(Z[0]), f64(V[0]), f64(W0), C, eta, "dot", update_first=True)
    assert rel(f64(O[0]), Oref) < TOL["bf16"]
    assert rel(f64(Wf[0]), Wref) < TOL["bf16"] and rel(f64(Wa[0]), Wref) < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fallback", [False, True])
@pytest.mark.parametrize("update_first", [False, True])
def test_chained_segments_with_documents(dtype, fallback, update_first, monkeypatch):
    """Two chained segments (260 state tiles, 8 chunks, segment 1 from chunk 4) on the chunk loop given Z and V^
    (dot objective, fused plan), with documents starting further into segment 1 (row 0), at its first chunk (row
    1) and one chunk into it (row 2), and none (row 3), against the oracle run per document.  With the wait
    disabled (TTT_UPDATE_SCAN_WAIT_US=-1) every segment-1 tile keeps partial states and the fix-up kernel
    completes it: the same results up to rounding.  update_first: the scan writes the states after each chunk's step
    (the chained segment then also needs the first segment's end state when a document starts one chunk in)."""
    B, n, d, f, C, eta = 4, 2048, 2560, 6656, 256, 0.02
    k = n // C
    starts = np.zeros((B, k), dtype=np.uint8)
    starts[0, 6] = 1
    starts[1, 4] = 1
    starts[2, 5] = 1
    Z, V, W0 = _zv(dtype, B, n, d, f, 41)
    g = (Z.cuda(), V.cuda(), W0.cuda())
    if fallback:
        monkeypatch.setenv("TTT_UPDATE_SCAN_WAIT_US", "-1")
    O, Wf = cw.ttt_core_apply_update(*g, C, eta, "dot", doc_starts=torch.from_numpy(starts).cuda(),
                                     update_first=update_first)
    torch.cuda.synchronize()
    W0n = f64(W0)
    for b in range(B):
        bounds = [0] + [c for c in range(1, k) if starts[b, c]] + [k]
        for s0, e0 in zip(bounds[:-1], bounds[1:]):
            Oref, Wref = orc.chunk_apply_update(f64(Z[b, s0 * C:e0 * C]), f64(V[b, s0 * C:e0 * C]), W0n, C, eta,
                                                "dot", update_first=update_first)
            assert rel(f64(O[b, s0 * C:e0 * C]), Oref) < TOL[dtype], (b, s0)
        assert rel(f64(Wf[b]), Wref) < TOL[dtype] and rel(f64(Wf[b]) - W0n, Wref - W0n) < TOL[dtype], b
    if fallback:
        monkeypatch.delenv("TTT_UPDATE_SCAN_WAIT_US")
        O2, Wf2 = cw.ttt_core_apply_update(*g, C, eta, "dot", doc_starts=torch.from_numpy(starts).cuda(),
                                           update_first=update_first)
        torch.cuda.synchronize()
        assert rel(f64(O), f64(O2)) < STEP_TOL[dtype] and rel(f64(Wf), f64(Wf2)) < STEP_TOL[dtype]


# ---------------------------------------------------------------- whole layer

def run_layer(cfg, mode=None):
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], cfg.chunk, cfg.eta, mode or cfg.mode)
    torch.cuda.synchronize()
    return x, O, Wf


def oracle_layer(cfg, x):
    mode = "dot" if cfg.mode == "dot_scan" else cfg.mode       # two GPU plans of one objective
    return orc.inplace_layer(*(ti.to_f64(x[k]) for k in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                           "conv_w")), cfg.chunk, cfg.eta, mode)


def check_layer(cfg, x, O, Wf):
    Oref, Wref = oracle_layer(cfg, x)
    W0 = ti.to_f64(x["W_down0"])
    eO, eW, eD = rel(f64(O), Oref), rel(f64(Wf), Wref), rel(f64(Wf) - W0, Wref - W0)
    tol = TOL[cfg.dtype]
    assert eO < tol and eW < tol and eD < tol, (eO, eW, eD)
    return eO, eW, eD


def test_layer_fp32_2k_workload():
    """The fp32 end-to-end workload: batch 1, seq 2048, d 256, d_ff 512, chunk 256, eta 0.1."""
    cfg = ti.workload("inplace_f32_2k")
    x, O, Wf = run_layer(cfg)
    check_layer(cfg, x, O, Wf)


@pytest.mark.parametrize("mode", ["dot", "dot_scan"])
def test_layer_fp32_2k_both_dot_plans(mode):
    cfg = ti.workload("inplace_f32_2k")
    x, O, Wf = run_layer(cfg, mode)
    check_layer(cfg, x, O, Wf)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_ragged_multi_tile(dtype, mode):
    eta = 0.02 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=2, n=1536, d=264, f=392, C=384, eta=eta)
    x, O, Wf = run_layer(cfg)
    check_layer(cfg, x, O, Wf)


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_layer_chunk_synchronous_tile_order(mode):
    """d_model 2048 with chunk 4096: one chunk (for MSE, one batch row's chunk) is 8 x 16 = 128 output tiles,
    the size from which the applies hand every chunk to all XCDs at once; two batch rows, two chunks."""
    eta = 0.02 if mode == "dot" else 0.5
    cfg = small_cfg("bf16", mode, B=2, n=8192, d=2048, f=256, C=4096, eta=eta)
    x, O, Wf = run_layer(cfg)
    check_layer(cfg, x, O, Wf)


LAYER_W = ("H", "X0", "W_gate", "W_up", "W_down0", "W_target", "conv_w")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_update_mask(dtype, mode):
    """Strided updates (update_mask): flagged chunks update, the others are applied with the state they find,
    against the oracle with the same mask.  Row 0 updates on every other chunk (the first one masked), row 1 on
    none but the last, row 2 masks two chunks and also starts a document at chunk 3, row 3 updates everywhere.
    An all-ones mask gives the unmasked call's bits."""
    eta = 0.05 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=4, n=1536, d=264, f=392, C=256, eta=eta)
    k = cfg.seq_len // cfg.chunk
    mask = np.ones((4, k), dtype=np.uint8)
    mask[0, 0::2] = 0
    mask[1, :-1] = 0
    mask[2, [1, 4]] = 0
    starts = np.zeros((4, k), dtype=np.uint8)
    starts[2, 3] = 1
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    args = tuple(g[n] for n in LAYER_W)
    O, Wf = cw.ttt_chunk_apply_update(*args, cfg.chunk, cfg.eta, mode, update_mask=torch.from_numpy(mask).cuda(),
                                      doc_starts=torch.from_numpy(starts).cuda())
    O1, W1 = cw.ttt_chunk_apply_update(*args, cfg.chunk, cfg.eta, mode,
                                       update_mask=torch.ones(4, k, dtype=torch.uint8, device="cuda"))
    O0, W0g = cw.ttt_chunk_apply_update(*args, cfg.chunk, cfg.eta, mode)
    torch.cuda.synchronize()
    assert torch.equal(O1, O0) and torch.equal(W1, W0g)
    Oref, Wref = orc.inplace_layer(*(ti.to_f64(x[n]) for n in LAYER_W), cfg.chunk, cfg.eta,
                                   "dot" if mode == "dot_scan" else mode, update_mask=mask, doc_starts=starts)
    W0 = ti.to_f64(x["W_down0"])
    for b in range(4):
        assert rel(f64(O[b]), Oref[b]) < TOL[dtype], b
        assert rel(f64(Wf[b]), Wref[b]) < TOL[dtype] and rel(f64(Wf[b]) - W0, Wref[b] - W0) < TOL[dtype], b
    # row 1 updates only on its last chunk: every earlier chunk is applied with W_down0
    Z1 = orc.gated_intermediate(ti.to_f64(x["H"])[1, : (k - 1) * cfg.chunk], ti.to_f64(x["W_gate"]),
                                ti.to_f64(x["W_up"]))
    assert rel(f64(O[1, : (k - 1) * cfg.chunk]), Z1 @ W0.T) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_core_update_mask_is_a_zero_target(dtype):
    """The chunk loop given Z and V^ (dot objective): masking a chunk is, bit for bit, zeroing its targets."""
    cfg = small_cfg(dtype, "dot", B=2, n=1024, C=256)
    gz = torch.Generator().manual_seed(3)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Z = (torch.randn(2, 1024, 392, generator=gz) * 0.6).to(tdt).cuda()
    V = torch.randn(2, 1024, 264, generator=gz).to(tdt).cuda()
    W0 = (torch.randn(264, 392, generator=gz) * 0.05).to(tdt).cuda()
    mask = torch.tensor([[1, 0, 0, 1], [0, 1, 1, 1]], dtype=torch.uint8)
    Vz = V.clone()
    for b in range(2):
        for c in range(4):
            if not mask[b, c]:
                Vz[b, c * 256:(c + 1) * 256] = 0
    O, Wf = cw.ttt_core_apply_update(Z, V, W0, 256, 0.05, "dot", update_mask=mask.cuda())
    Oz, Wz = cw.ttt_core_apply_update(Z, Vz, W0, 256, 0.05, "dot")
    torch.cuda.synchronize()
    assert torch.equal(O, Oz) and torch.equal(Wf, Wz)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_packed_documents(dtype, mode):
    """Rows packing several documents (ttt_chunk_apply_update_ex): at every flagged chunk the state restarts
    from W_down0 and the convolution from zeros, against the oracle with the same document starts.  Row 0 packs
    documents of 2, 2 and 2 chunks, row 1 starts one at every chunk, row 2 holds a single document, row 3 two of
    3 chunks.  With two sequence segments of 3 chunks in the fused dot plan, row 0's second segment starts inside a
    document and resets in its middle, row 3's starts with a document."""
    eta = 0.05 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=4, n=1536, d=264, f=392, C=256, eta=eta)
    k = cfg.seq_len // cfg.chunk
    starts = np.zeros((4, k), dtype=np.uint8)
    starts[0, [0, 2, 4]] = 1
    starts[1, :] = 1
    starts[3, [0, 3]] = 1
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], cfg.chunk, cfg.eta, mode,
                                      doc_starts=torch.from_numpy(starts).cuda())
    torch.cuda.synchronize()
    Oref, Wref = orc.inplace_layer(*(ti.to_f64(x[n]) for n in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                                "conv_w")), cfg.chunk, cfg.eta,
                                   "dot" if mode == "dot_scan" else mode, doc_starts=starts)
    W0 = ti.to_f64(x["W_down0"])
    tol = TOL[dtype]
    for b in range(4):
        assert rel(f64(O[b]), Oref[b]) < tol, b
        assert rel(f64(Wf[b]), Wref[b]) < tol and rel(f64(Wf[b]) - W0, Wref[b] - W0) < tol, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_forward_conv(dtype, mode):
    """The forward-looking in-chunk convolution for the target (option conv_forward: tap j reads the token j
    ahead, zero past the chunk's end), against the oracle; row 1 also packs two documents, which the forward
    window (never leaving its chunk) does not see."""
    eta = 0.05 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=2, n=1536, d=264, f=392, C=256, eta=eta)
    k = cfg.seq_len // cfg.chunk
    starts = np.zeros((2, k), dtype=np.uint8)
    starts[1, [0, 3]] = 1
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], cfg.chunk, cfg.eta, mode,
                                      doc_starts=torch.from_numpy(starts).cuda(), conv_forward=True)
    torch.cuda.synchronize()
    Oref, Wref = orc.inplace_layer(*(ti.to_f64(x[n]) for n in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                                "conv_w")), cfg.chunk, cfg.eta,
                                   "dot" if mode == "dot_scan" else mode, doc_starts=starts, conv_forward=True)
    W0 = ti.to_f64(x["W_down0"])
    tol = TOL[dtype]
    for b in range(2):
        assert rel(f64(O[b]), Oref[b]) < tol, b
        assert rel(f64(Wf[b]), Wref[b]) < tol and rel(f64(Wf[b]) - W0, Wref[b] - W0) < tol, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_resumed_in_two_calls(dtype, mode):
    """A sequence processed in two calls, the second resuming each row from the first call's W_final (W_init)
    and its last K-1 rows of X0 (x0_halo), against the oracle's single call over the whole sequence.  The second
    call (4 chunks, so the fused dot plan runs sequence segments) flags a document start at its first chunk in
    row 1, which ignores both and matches a single call with a document starting there."""
    eta = 0.05 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=2, n=1536, d=264, f=392, C=256, eta=eta)
    C, K = cfg.chunk, cfg.conv_k
    s = 2 * C
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    w = (g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"])
    O1, W1 = cw.ttt_chunk_apply_update(g["H"][:, :s].contiguous(), g["X0"][:, :s].contiguous(), *w, C, cfg.eta, mode)
    starts = torch.zeros(2, (cfg.seq_len - s) // C, dtype=torch.uint8, device="cuda")
    starts[1, 0] = 1
    O2, W2 = cw.ttt_chunk_apply_update(g["H"][:, s:].contiguous(), g["X0"][:, s:].contiguous(), *w, C, cfg.eta,
                                       mode, W_init=W1, x0_halo=g["X0"][:, s - (K - 1): s].contiguous(),
                                       doc_starts=starts)
    torch.cuda.synchronize()
    full = np.zeros((2, cfg.seq_len // C), dtype=np.uint8)
    full[1, s // C] = 1
    Oref, Wref = orc.inplace_layer(*(ti.to_f64(x[n]) for n in ("H", "X0", "W_gate", "W_up", "W_down0", "W_target",
                                                                "conv_w")), C, cfg.eta,
                                   "dot" if mode == "dot_scan" else mode, doc_starts=full)
    O = torch.cat([O1, O2], dim=1)
    W0 = ti.to_f64(x["W_down0"])
    tol = TOL[dtype]
    for b in range(2):
        assert rel(f64(O[b]), Oref[b]) < tol, b
        assert rel(f64(W2[b]), Wref[b]) < tol and rel(f64(W2[b]) - W0, Wref[b] - W0) < tol, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_layer_update_first(dtype, mode):
    """The update-then-apply order (update_first): each chunk is applied with the state after its own step,
    against the oracle in that order, with every option it combines with.  Row 0 starts a document at chunk 0
    (so it ignores W_init and x0_halo), row 1 resumes, masks chunks 1 and 4 and starts a document at chunk 3, row 2
    resumes and masks chunk 0 (applied with W_init unchanged).  W_final is the apply-then-update call's, bit for
    bit (the steps are the same arithmetic in both orders)."""
    eta = 0.05 if mode != "mse" else 0.5
    cfg = small_cfg(dtype, mode, B=3, n=1536, d=264, f=392, C=256, eta=eta)
    k = cfg.seq_len // cfg.chunk
    starts = np.zeros((3, k), dtype=np.uint8)
    starts[0, 0] = 1
    starts[1, 3] = 1
    mask = np.ones((3, k), dtype=np.uint8)
    mask[1, [1, 4]] = 0
    mask[2, 0] = 0
    x = ti.inplace_inputs(cfg)
    r = ti.resume_inputs(cfg, seed=11)
    g = dev(x)
    args = tuple(g[n] for n in LAYER_W)
    opts = dict(doc_starts=torch.from_numpy(starts).cuda(), update_mask=torch.from_numpy(mask).cuda(),
                W_init=r["W_init"].cuda(), x0_halo=r["x0_halo"].cuda())
    O, Wf = cw.ttt_chunk_apply_update(*args, cfg.chunk, cfg.eta, mode, update_first=True, **opts)
    Oa, Wa = cw.ttt_chunk_apply_update(*args, cfg.chunk, cfg.eta, mode, **opts)
    torch.cuda.synchronize()
    assert torch.equal(Wf, Wa)
    Oref, Wref = orc.inplace_layer(*(ti.to_f64(x[n]) for n in LAYER_W), cfg.chunk, cfg.eta,
                                   "dot" if mode == "dot_scan" else mode, doc_starts=starts, update_mask=mask,
                                   W_init=ti.to_f64(r["W_init"]), x0_halo=ti.to_f64(r["x0_halo"]),
                                   update_first=True)
    W0 = ti.to_f64(x["W_down0"])
    for b in range(3):
        assert rel(f64(O[b]), Oref[b]) < TOL[dtype], b
        assert rel(f64(Wf[b]), Wref[b]) < TOL[dtype] and rel(f64(Wf[b]) - W0, Wref[b] - W0) < TOL[dtype], b
    # row 2's first chunk is masked: in both orders it is applied with W_init
    assert torch.equal(O[2, :cfg.chunk], Oa[2, :cfg.chunk])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_core_update_first(dtype, mode):
    """The chunk loop given Z and V^ in the update-then-apply order, against the oracle's sequential definition
    in that order, per row (ragged d and f, four chunks)."""
    eta = 0.05 if mode != "mse" else 0.5
    gz = torch.Generator().manual_seed(5)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Z = (torch.randn(2, 1024, 392, generator=gz) * 0.6).to(tdt)
    V = torch.randn(2, 1024, 264, generator=gz).to(tdt)
    W0 = (torch.randn(264, 392, generator=gz) * 0.05).to(tdt)
    O, Wf = cw.ttt_core_apply_update(Z.cuda(), V.cuda(), W0.cuda(), 256, eta, mode, update_first=True)
    torch.cuda.synchronize()
    for b in range(2):
        Oref, Wref = orc.chunk_apply_update(ti.to_f64(Z[b]), ti.to_f64(V[b]), ti.to_f64(W0), 256, eta,
                                            "dot" if mode == "dot_scan" else mode, update_first=True)
        assert rel(f64(O[b]), Oref) < TOL[dtype], b
        assert rel(f64(Wf[b]), Wref) < TOL[dtype], b


def test_layer_bf16_chunk_not_multiple_of_kstep():
    # chunk 40: the dot plan falls back to materialised deltas + scan
    cfg = small_cfg("bf16", "dot", B=1, n=400, d=128, f=256, C=40, eta=0.02)
    x, O, Wf = run_layer(cfg)
    check_layer(cfg, x, O, Wf)


def test_layer_mse_bf16_workload_shape_reduced():
    """The MSE workload's structure (batch 4, eta 1, Gaussian inits) at a reduced length."""
    cfg = ti.workload("mse_bf16_4x64k").with_(seq_len=4096, d_model=512, d_ff=2048, chunk=512)
    x, O, Wf = run_layer(cfg)
    check_layer(cfg, x, O, Wf)


def test_step_composition_equals_full_call():
    cfg = small_cfg("bf16", "dot", B=2, n=1024, C=256, eta=0.03)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], cfg.chunk, cfg.eta, "dot")
    Z, Zt = cw.ttt_produce_z(g["H"], g["W_gate"], g["W_up"])
    Vt = cw.ttt_produce_vhat(g["X0"], g["conv_w"], g["W_target"], scale=cfg.eta)
    Wc, Wf2 = cw.ttt_chunk_update_scan(Zt, Vt, g["W_down0"], cfg.chunk)
    O2 = cw.ttt_chunk_apply(Zt, Wc, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(Wf, Wf2)
    # the chunk loop alone, from Z and V^ in their natural layouts
    V = cw.ttt_produce_vhat(g["X0"], g["conv_w"], g["W_target"]).transpose(1, 2).contiguous()
    O3, Wf3 = cw.ttt_core_apply_update(Z, V, g["W_down0"], cfg.chunk, cfg.eta, "dot")
    torch.cuda.synchronize()
    assert rel(f64(O3), f64(O)) < STEP_TOL["bf16"] and rel(f64(Wf3), f64(Wf)) < STEP_TOL["bf16"]


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_eta_zero_is_plain_gated_mlp(mode):
    cfg = small_cfg("bf16", mode, n=768, eta=0.0)
    x, O, Wf = run_layer(cfg)
    W0 = ti.to_f64(x["W_down0"])
    assert np.array_equal(f64(Wf[0]), W0)
    ref = orc.gated_mlp(ti.to_f64(x["H"])[0], ti.to_f64(x["W_gate"]), ti.to_f64(x["W_up"]), W0)
    assert rel(f64(O[0]), ref) < TOL["bf16"]


@pytest.mark.parametrize("mode", ["dot", "dot_scan", "mse"])
def test_causality_future_rows_do_not_change_past_outputs(mode):
    cfg = small_cfg("bf16", mode, n=1024, C=256, eta=0.05 if mode != "mse" else 0.5)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    args = lambda gg: (gg["H"], gg["X0"], gg["W_gate"], gg["W_up"], gg["W_down0"], gg["W_target"], gg["conv_w"])
    O, _ = cw.ttt_chunk_apply_update(*args(g), cfg.chunk, cfg.eta, mode)
    c = 1
    g2 = dict(g)
    g2["X0"] = g["X0"].clone()
    g2["X0"][:, c * cfg.chunk:] = torch.randn_like(g2["X0"][:, c * cfg.chunk:], dtype=torch.float32).to(torch.bfloat16)
    g2["H"] = g["H"].clone()
    g2["H"][:, (c + 1) * cfg.chunk:] = 0
    O2, _ = cw.ttt_chunk_apply_update(*args(g2), cfg.chunk, cfg.eta, mode)
    torch.cuda.synchronize()
    r = (c + 1) * cfg.chunk
    assert torch.equal(O[:, :r], O2[:, :r])
    assert not torch.equal(O[:, r:], O2[:, r:])


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_batch_rows_equal_separate_runs_and_determinism(mode):
    cfg = small_cfg("bf16", mode, B=3, n=512, C=128, eta=0.05 if mode == "dot" else 0.5)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    w = (g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"])
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], *w, cfg.chunk, cfg.eta, mode)
    O_again, Wf_again = cw.ttt_chunk_apply_update(g["H"], g["X0"], *w, cfg.chunk, cfg.eta, mode)
    torch.cuda.synchronize()
    assert torch.equal(O, O_again) and torch.equal(Wf, Wf_again)
    for b in range(3):
        Ob, Wb = cw.ttt_chunk_apply_update(g["H"][b:b + 1].contiguous(), g["X0"][b:b + 1].contiguous(), *w,
                                           cfg.chunk, cfg.eta, mode)
        torch.cuda.synchronize()
        assert torch.equal(Ob[0], O[b]) and torch.equal(Wb[0], Wf[b])


@pytest.mark.parametrize("mode", ["dot", "mse"])
def test_empty_sequence_and_empty_batch(mode):
    cfg = small_cfg("bf16", mode, B=2, n=0, C=64)
    x = ti.inplace_inputs(cfg.with_(seq_len=0))
    g = dev(x)
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], 64, 0.1, mode)
    torch.cuda.synchronize()
    assert O.shape == (2, 0, cfg.d_model)
    assert torch.equal(Wf, g["W_down0"].float().expand(2, -1, -1))
    g0 = dev(ti.inplace_inputs(cfg.with_(batch=0, seq_len=128)))
    O, Wf = cw.ttt_chunk_apply_update(g0["H"], g0["X0"], g0["W_gate"], g0["W_up"], g0["W_down0"], g0["W_target"],
                                      g0["conv_w"], 64, 0.1, mode)
    assert O.shape[0] == 0 and Wf.shape[0] == 0


def test_core_entry_point_orthogonal_keys_reach_target():
    # chunk = d_ff, Z = sqrt(C) Q (Q orthogonal), V^ = Z W*^T, eta = 1, mse: one step lands on W*
    f, d = 256, 128
    rng = np.random.default_rng(5)
    Q, _ = np.linalg.qr(rng.standard_normal((f, f)))
    Z = np.sqrt(f) * Q
    Ws = rng.standard_normal((d, f)) * 0.1
    V = Z @ Ws.T
    W0 = rng.standard_normal((d, f)) * 0.1
    t = lambda a: torch.from_numpy(a).float().cuda()
    O, Wf = cw.ttt_core_apply_update(t(Z)[None].contiguous(), t(V)[None].contiguous(), t(W0), f, 1.0, "mse")
    torch.cuda.synchronize()
    assert rel(f64(Wf[0]), Ws) < 1e-4


# ---------------------------------------------------------------- full-size workloads, every element

class _FrobAcc:
    """Relative Frobenius error of a tensor compared piece by piece (rows of a batch, heads)."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, want):
        got = np.asarray(got, dtype=np.float64)
        want = np.asarray(want, dtype=np.float64)
        self.num += float(np.sum((got - want) ** 2))
        self.den += float(np.sum(want ** 2))

    def rel(self):
        return float(np.sqrt(self.num / self.den)) if self.den > 0 else float(np.sqrt(self.num))


def _full_size(name):
    """A workload at full size, called as the bench calls it (ttt_chunk_apply_update, its launch configuration),
    against the oracle's layer on every element of O, W_final and W_final - W_down0.  The oracle streams chunk by
    chunk and runs one batch row at a time, so host memory stays at a few GB (In-Place TTT review, Method §3: the
    parallel form reaches the sequential chunk loop's result)."""
    cfg = ti.workload(name)
    print(f"full-size case: {name} B={cfg.batch} n={cfg.seq_len} d={cfg.d_model} f={cfg.d_ff} C={cfg.chunk} "
          f"mode={cfg.mode}", flush=True)
    x = ti.inplace_inputs(cfg)
    g = dev(x)
    flags = cfg.doc_starts()
    docs = None if flags is None else torch.from_numpy(flags).cuda()
    O, Wf = cw.ttt_chunk_apply_update(g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"],
                                      g["conv_w"], cfg.chunk, cfg.eta, cfg.mode, doc_starts=docs,
                                      conv_forward=cfg.conv_forward)
    torch.cuda.synchronize()
    O, Wf = O.cpu(), Wf.cpu()
    del g
    torch.cuda.empty_cache()
    ws = {k: ti.to_f64(x[k]) for k in ("W_gate", "W_up", "W_down0", "W_target", "conv_w")}
    W0 = ws["W_down0"]
    eO, eW, edW = _FrobAcc(), _FrobAcc(), _FrobAcc()
    for b in range(cfg.batch):
        Oref, Wref = orc.inplace_layer(ti.to_f64(x["H"][b: b + 1]), ti.to_f64(x["X0"][b: b + 1]), ws["W_gate"],
                                       ws["W_up"], W0, ws["W_target"], ws["conv_w"], cfg.chunk, cfg.eta,
                                       "dot" if cfg.mode == "dot_scan" else cfg.mode,
                                       doc_starts=None if flags is None else flags[b: b + 1],
                                       conv_forward=cfg.conv_forward)
        eO.add(O[b].double().numpy(), Oref[0])
        Wg = Wf[b].double().numpy()
        eW.add(Wg, Wref[0])
        edW.add(Wg - W0, Wref[0] - W0)
        print(f"  row {b}: done", flush=True)
    errs = (eO.rel(), eW.rel(), edW.rel())
    print(f"  rel err O {errs[0]:.3e}  W_final {errs[1]:.3e}  W_final - W0 {errs[2]:.3e}", flush=True)
    assert max(errs) < TOL[cfg.dtype], errs
    return errs


@pytest.mark.slow
def test_full_size_32k():
    """32K tokens, d_model 2560, d_ff 9728, chunk 1024 (two sequence segments in the fused scan)."""
    _full_size("inplace_bf16_32k")


@pytest.mark.slow
def test_full_size_128k():
    """128K tokens, chunk 4096: the bench's workload.  The fused scan runs two chained sequence segments, so chunks
    17-31 are applied with states the second segment formed from the first's end state."""
    _full_size("inplace_bf16_128k")


@pytest.mark.slow
def test_full_size_mse():
    """The MSE workload, 4 x 64K tokens, d_model 2048, d_ff 8192, chunk 2048, eta 1: the whole 32-chunk scan of
    every row."""
    _full_size("mse_bf16_4x64k")


@pytest.mark.slow
def test_full_size_packed_documents():
    """The 128K row packing 8 documents of 4 chunks: every state restart, every convolution restart, and W_final
    holding the last document alone."""
    _full_size("inplace_bf16_128k_8docs")