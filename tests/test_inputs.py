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


def test_every_workload_states_its_flops():
    """Every workload's algorithmic flop count per token: the layer (8df + 2d^2 + 2Kd for In-Place, 20 dh m per head
    for LaCT before its variants), the chunk loop's backward (10df, 8df with kept states; 14df and 10df for MSE), and
    the whole layer's backward (26df + 6d^2, 24df + 6d^2 with kept states; 30df + 6d^2 and 26df + 6d^2 for
    MSE)."""
    for name, cfg in ti.WORKLOADS.items():
        assert cfg.flops() > 0, name
        if isinstance(cfg, ti.LactConfig):
            continue
        d, f, K, T = cfg.d_model, cfg.d_ff, cfg.conv_k, cfg.tokens
        if cfg.layer_backward and cfg.mode == "mse":
            want = (26 if cfg.kept_states else 30) * d * f + 6 * d * d
        elif cfg.layer_backward:
            want = (24 if cfg.kept_states else 26) * d * f + 6 * d * d
        elif cfg.backward and cfg.mode == "mse":
            want = (10 if cfg.kept_states else 14) * d * f
        elif cfg.backward:
            want = (8 if cfg.kept_states else 10) * d * f
        else:
            want = 8 * d * f + 2 * d * d + 2 * K * d
        assert cfg.flops() == float(T) * want, name


def test_backward_inputs_shapes_and_seed():
    cfg = ti.workload("inplace_bwd_bf16_128k").with_(seq_len=64, d_model=16, d_ff=24, chunk=16)
    x = ti.backward_inputs(cfg)
    assert [tuple(x[k].shape) for k in ("Z", "Vhat", "W_down0", "dO")] == [(1, 64, 24), (1, 64, 16), (16, 24), (1, 64, 16)]
    assert all(t.dtype == torch.bfloat16 for t in x.values())
    y = ti.backward_inputs(cfg)
    assert all(torch.equal(x[k], y[k]) for k in x)
