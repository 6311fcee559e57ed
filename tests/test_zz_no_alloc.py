"""The allocation-free entry point ttt_chunk_apply_update_noalloc against the
call with a caller workspace (ttt_chunk_apply_update), through the C ABI.

Both run the same kernels with the same launch configuration, so their
outputs must be bit-identical; the first call is also held to the oracle's
bar.  Two calls in a row share the device's static scratch: the second, on a
smaller input, must not see anything the first left there.  The last call
must reject a shape whose scratch exceeds TTT_NOALLOC_SCRATCH_BYTES before
any device work (its outputs keep the values they had).
"""
import numpy as np
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti
from oracle import inplace as orc

pytestmark = pytest.mark.gpu

NAMES = ("H", "X0", "W_gate", "W_up", "W_down0", "W_target", "conv_w")


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _both(cfg):
    print(f"noalloc case: {cfg.name} dtype={cfg.dtype} mode={cfg.mode} B={cfg.batch} n={cfg.seq_len} "
          f"d={cfg.d_model} f={cfg.d_ff} C={cfg.chunk}", flush=True)
    x = ti.inplace_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    B, n, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    dt = g["H"].dtype
    # outputs filled with NaN, so that an element the call does not write shows
    O = torch.full((B, n, d), float("nan"), dtype=dt, device="cuda")
    Wf = torch.full((B, d, f), float("nan"), dtype=torch.float32, device="cuda")
    cw.ttt_chunk_apply_update_noalloc(*(g[k] for k in NAMES), cfg.chunk, cfg.eta, cfg.mode, O, Wf)
    Oref, Wref = cw.ttt_chunk_apply_update(*(g[k] for k in NAMES), cfg.chunk, cfg.eta, cfg.mode)
    torch.cuda.synchronize()
    return x, O, Wf, Oref, Wref


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    first = ti.workload("inplace_f32_2k")                      # 16.75 MiB of scratch
    x, O, Wf, Oref, Wref = _both(first)
    assert torch.equal(O, Oref) and torch.equal(Wf, Wref)
    Oo, Wo = orc.inplace_layer(*(ti.to_f64(x[k]) for k in NAMES), first.chunk, first.eta, first.mode)
    assert _rel(O.double().cpu().numpy(), Oo) < 1e-4
    assert _rel(Wf.double().cpu().numpy(), Wo) < 1e-4

    # a smaller input right after: half the sequence, the same state shape
    second = ti.InplaceConfig("noalloc_second", 1, 1024, 256, 512, 256, 0.1, "dot", "f32", seed=1011)
    x2, O2, Wf2, Oref2, Wref2 = _both(second)
    assert torch.equal(O2, Oref2) and torch.equal(Wf2, Wref2)
    Oo2, Wo2 = orc.inplace_layer(*(ti.to_f64(x2[k]) for k in NAMES), second.chunk, second.eta, second.mode)
    assert _rel(O2.double().cpu().numpy(), Oo2) < 1e-4
    assert _rel(Wf2.double().cpu().numpy(), Wo2) < 1e-4


@pytest.mark.parametrize("mode", ["mse", "dot_scan", "dot"])
def test_noalloc_other_plans_bf16(mode):
    # two rows, chunk 40 for the materialised scan (its deltas live in the scratch), ragged widths
    C = 40 if mode == "dot_scan" else 128
    cfg = ti.InplaceConfig(f"noalloc_{mode}", 2, 10 * C, 264, 392, C, 0.05 if mode != "mse" else 1.0, mode, "bf16",
                           seed=1012)
    x, O, Wf, Oref, Wref = _both(cfg)
    assert torch.equal(O, Oref) and torch.equal(Wf, Wref)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    cfg = ti.InplaceConfig("noalloc_big", 2, 4096, 512, 1024, 512, 0.01, "dot", "bf16", seed=1013)
    shape = cw.InplaceShape(2, 4096, 512, 1024, 512, 4)
    assert cw.ttt_inplace_workspace_bytes(shape, torch.bfloat16, "dot", True) > cw.TTT_NOALLOC_SCRATCH_BYTES
    x = ti.inplace_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    O = torch.zeros(2, 4096, 512, dtype=torch.bfloat16, device="cuda")
    Wf = torch.zeros(2, 512, 1024, dtype=torch.float32, device="cuda")
    with pytest.raises(cw.TTTError) as err:
        cw.ttt_chunk_apply_update_noalloc(*(g[k] for k in NAMES), cfg.chunk, cfg.eta, cfg.mode, O, Wf)
    assert err.value.status == cw.TTT_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert not O.any() and not Wf.any()
