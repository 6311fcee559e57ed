"""The seeded input generators: determinism, dtypes, shapes and the stated
distributions (variances, L2 normalisation) of the workloads."""
import numpy as np
import torch

import ttt_inputs as ti


def test_inplace_inputs_deterministic_and_shaped():
    cfg = ti.workload("inplace_f32_2k")
    a = ti.inplace_inputs(cfg)
    b = ti.inplace_inputs(cfg)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["H"].shape == (1, 2048, 256) and a["H"].dtype == torch.float32
    assert a["W_gate"].shape == (512, 256) and a["W_down0"].shape == (256, 512)
    assert a["W_target"].shape == (256, 256) and a["conv_w"].shape == (256, 4)
    # variances as stated: H ~ N(0,1), W_gate ~ N(0,1/d), W_down0 ~ N(0,1/f), conv ~ N(0,1/4)
    assert abs(a["H"].var().item() - 1.0) < 0.02
    assert abs(a["W_gate"].var().item() * 256 - 1.0) < 0.03
    assert abs(a["W_down0"].var().item() * 512 - 1.0) < 0.03
    assert abs(a["conv_w"].var().item() * 4 - 1.0) < 0.1


def test_bf16_inputs_are_rounded_once():
    cfg = ti.workload("inplace_bf16_32k").with_(seq_len=64, d_model=32, d_ff=48, chunk=16)
    a = ti.inplace_inputs(cfg)
    assert a["H"].dtype == torch.bfloat16
    x = ti.to_f64(a["H"])
    assert np.array_equal(ti.bf16_round(x), x)


def test_lact_inputs_are_unit_norm_per_token():
    cfg = ti.workload("lact_bf16_256k").with_(seq_len=32, chunk=8, dtype="f32")
    a = ti.lact_inputs(cfg)
    assert a["q"].shape == (1, 4, 32, 512)
    np.testing.assert_allclose(a["k"].norm(dim=-1).numpy(), 1.0, rtol=1e-5)
    assert a["W1"].shape == (4, 1024, 512) and a["W2"].shape == (4, 512, 1024)
    assert abs(a["W2"].var().item() * 1024 - 1.0) < 0.02


def test_workload_flop_counts():
    cfg = ti.workload("inplace_bf16_128k")
    d, f = 2560, 9728
    assert cfg.flops() == 131072 * (8 * d * f + 2 * d * d + 8 * d)
    lc = ti.workload("lact_bf16_256k")
    assert lc.flops() == 262144 * 4 * 20 * 512 * 1024
