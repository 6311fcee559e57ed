"""Seeded synthetic inputs for the chunk-wise TTT fast-weight layer.

This module holds no arithmetic of the method: it only draws tensors.  Both
the oracle side (tests, CPU baseline) and the HIP side (tests, bench) take
their inputs from here, so that the two see bit-identical values.

Recipe (for every workload):
  * a ``torch.Generator`` on the CPU, seeded with ``seed``;
  * tensors are drawn in a fixed order with ``torch.randn`` in fp32, scaled
    by the stated standard deviation (the workloads give variances: N(0, x)
    means variance x, std sqrt(x));
  * for bf16 workloads the fp32 draw is rounded once to bf16 with
    round-to-nearest-even (torch's float->bfloat16 conversion);
  * the LaCT q, k, v are L2-normalised per token per head in fp32 *before*
    the bf16 rounding (input preparation, not part of the layer).

Draw order, In-Place layer: H, X0, W_gate, W_up, W_down0, W_target, conv_w.
Draw order, backward of the chunk loop: Z, Vhat, W_down0, dO (Z with the
variance of silu(a) b for independent standard normals a and b, about 0.356;
the target and the upstream gradient standard normal; W_down0 as above).
Draw order, LaCT layer: q, k, v, W1, W3, W2.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = [
    "InplaceConfig", "LactConfig", "WORKLOADS", "workload",
    "inplace_inputs", "backward_inputs", "lact_inputs", "to_f64", "bf16_round",
]


@dataclass(frozen=True)
class InplaceConfig:
    """Shape and hyper-parameters of one In-Place TTT layer call."""
    name: str
    batch: int
    seq_len: int
    d_model: int
    d_ff: int
    chunk: int
    eta: float
    mode: str            # "dot" (prefix-sum update) or "mse" (sequential scan)
    dtype: str           # "f32" or "bf16"
    conv_k: int = 4
    seed: int = 1000
    # variances of the Gaussian draws; None means "use the default"
    var_h: float = 1.0
    var_x0: float = 1.0
    var_gate: float | None = None    # default 1/d_model
    var_up: float | None = None      # default 1/d_model
    var_down: float | None = None    # default 1/d_ff
    var_target: float | None = None  # default 1/d_model
    var_conv: float = 0.25
    docs: int = 1        # documents packed into each row, of equal length in chunks
    conv_forward: bool = False   # forward-looking in-chunk convolution for the target
    pieces: int = 1      # the sequence processed in this many calls, each resuming the previous one
    backward: bool = False   # the workload is the backward of the dot chunk loop (inputs Z, Vhat, W_down0, dO)
    kept_states: bool = False   # backward: the forward call kept its per-chunk states (no recompute)
    layer_backward: bool = False   # the backward of the whole layer (inputs of the layer and dO)
    var_z: float = 0.356     # backward inputs: Z, the gated intermediate
    var_vhat: float = 1.0    # backward inputs: the target
    var_dout: float = 1.0    # backward inputs: the upstream gradient dLoss/dO

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def doc_starts(self):
        """Document-start flags [batch, n_chunks] (uint8: 1 where a document starts) for `docs` equal documents
        per row, or None for one document per row."""
        if self.docs <= 1:
            return None
        k = self.n_chunks
        if k % self.docs:
            raise ValueError(f"{k} chunks do not split into {self.docs} equal documents")
        flags = np.zeros((self.batch, k), dtype=np.uint8)
        flags[:, :: k // self.docs] = 1
        return flags

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk

    def flops(self) -> float:
        """Algorithmic flops of one layer call: producer 4df, target 2d^2 + 2Kd,
        update 2df, apply 2df per token.  Backward of the chunk loop: 10df per
        token (the states' scan, the suffixes' scan, dVhat, and dZ's two
        contractions, 2df each); 8df with the states kept by the forward call.
        Backward of the whole layer: that (or the MSE loop's, below), plus
        the producer's recompute and its backward (4df each), the gate and
        up weight gradients (4df), dH (4df), and V^, dW_target and dY (2d^2
        each)."""
        d, f, K = self.d_model, self.d_ff, self.conv_k
        if self.layer_backward and self.mode == "mse":
            return float(self.tokens) * ((26.0 if self.kept_states else 30.0) * d * f + 6.0 * d * d)
        if self.layer_backward:
            return float(self.tokens) * ((24.0 if self.kept_states else 26.0) * d * f + 6.0 * d * d)
        if self.backward and self.mode == "mse":
            # the forward scan again (4df, unless the states are kept), then per chunk two applies, dZ's two
            # contractions and the update
            return float(self.tokens) * (10.0 if self.kept_states else 14.0) * d * f
        if self.backward:
            return float(self.tokens) * (8.0 if self.kept_states else 10.0) * d * f
        return float(self.tokens) * (8.0 * d * f + 2.0 * d * d + 2.0 * K * d)

    def with_(self, **kw) -> "InplaceConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class LactConfig:
    """Shape and hyper-parameters of one LaCT SwiGLU fast-weight layer call."""
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    hidden: int
    chunk: int
    eta: float
    order: str = "update_then_apply"   # or "apply_then_update"
    dtype: str = "bf16"
    seed: int = 1004
    var_w1: float | None = None   # default 1/head_dim
    var_w3: float | None = None   # default 1/head_dim
    var_w2: float | None = None   # default 1/hidden
    update_every: int = 1         # only every update_every-th chunk takes the update step (1: all)
    loss: str = "mse"             # "mse" or "dot" (the dot-product loss -f(k)^T v)
    weight_norm: bool = False     # L2-normalise the weight rows after every update
    token_rates: bool = False     # draw per-token learning rates eta_tok ~ U(0, 1) (fp32)
    muon: bool = False            # the Muon update rule (Newton-Schulz orthogonalised gradients)
    backward: bool = False        # the layer's backward (inputs of the layer and dO)
    kept_states: bool = False     # the backward reads the states the forward call kept

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def update_mask(self):
        """Per-chunk update flags (list of 0/1) when only every update_every-th chunk updates, else None."""
        if self.update_every <= 1:
            return None
        return [1 if c % self.update_every == 0 else 0 for c in range(self.n_chunks)]

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk

    def flops(self) -> float:
        """Algorithmic flops: per token per head, key forward 6*dh*m and
        backward 8*dh*m (dH, G1, G2, G3) on the chunks that update, query apply
        6*dh*m on every chunk.  The layer's backward executes 66*dh*m per token
        and head: the states recomputed on the keys (14), the query apply's
        backward with its recompute (16: Aq, Uq, dHq, the three weight
        gradients, dq) and the update's (36: A, U, Y, dH again, ddA, ddU, dR,
        dHh, dk's four products, the three weight gradients); 52 with the
        states kept by the forward call."""
        if self.backward:
            per = 52.0 if self.kept_states else 66.0
            return float(self.tokens) * self.heads * per * self.head_dim * self.hidden
        mask = self.update_mask()
        upd = 1.0 if mask is None else sum(mask) / len(mask)
        key = 14.0 - (2.0 if self.loss == "dot" else 0.0)     # the dot loss needs no key output f(k)
        total = float(self.tokens) * self.heads * (6.0 + key * upd) * self.head_dim * self.hidden
        if self.muon:   # per updating chunk and head, 3 gradients x 5 steps of A = X X^T, A^2 and B X on [r, c]
            r, c = min(self.head_dim, self.hidden), max(self.head_dim, self.hidden)
            n_upd = self.n_chunks * upd
            total += self.batch * self.heads * n_upd * 3 * 5 * (2.0 * r * r * c + 2.0 * r ** 3 + 2.0 * r * r * c)
        return total

    def with_(self, **kw) -> "LactConfig":
        return replace(self, **kw)


# The five workloads (and the chunk-512 variant of the 128K one).
WORKLOADS = {
    "inplace_f32_2k": InplaceConfig("inplace_f32_2k", 1, 2048, 256, 512, 256, 0.1, "dot", "f32", seed=1000),
    "inplace_bf16_32k": InplaceConfig("inplace_bf16_32k", 1, 32768, 2560, 9728, 1024, 0.01, "dot", "bf16", seed=1001),
    "inplace_bf16_128k": InplaceConfig("inplace_bf16_128k", 1, 131072, 2560, 9728, 4096, 0.01, "dot", "bf16", seed=1002),
    "inplace_bf16_128k_c512": InplaceConfig("inplace_bf16_128k_c512", 1, 131072, 2560, 9728, 512, 0.01, "dot", "bf16", seed=1002),
    # the 128K layer with the forward-looking in-chunk convolution (next-token-style target)
    "inplace_bf16_128k_ntp": InplaceConfig("inplace_bf16_128k_ntp", 1, 131072, 2560, 9728, 4096, 0.01, "dot", "bf16",
                                           seed=1002, conv_forward=True),
    # the 128K layer processed as 4 calls of 32K tokens, each resuming the previous one's state and conv halo
    "inplace_bf16_128k_4pieces": InplaceConfig("inplace_bf16_128k_4pieces", 1, 131072, 2560, 9728, 4096, 0.01, "dot",
                                               "bf16", seed=1002, pieces=4),
    # the 128K row packing 8 documents of 16K tokens (4 chunks each)
    "inplace_bf16_128k_8docs": InplaceConfig("inplace_bf16_128k_8docs", 1, 131072, 2560, 9728, 4096, 0.01, "dot", "bf16",
                                             seed=1002, docs=8),
    # the backward of the 128K layer's dot chunk loop (gradients of Z, V^ and W_down0 from dLoss/dO)
    "inplace_bwd_bf16_128k": InplaceConfig("inplace_bwd_bf16_128k", 1, 131072, 2560, 9728, 4096, 0.01, "dot", "bf16",
                                           seed=1005, backward=True),
    # the same with the per-chunk states kept by the forward call (no recompute)
    "inplace_bwd_bf16_128k_kept": InplaceConfig("inplace_bwd_bf16_128k_kept", 1, 131072, 2560, 9728, 4096, 0.01, "dot",
                                                "bf16", seed=1005, backward=True, kept_states=True),
    # the backward of the whole 128K layer (gradients of every input and weight from dLoss/dO)
    "inplace_layer_bwd_bf16_128k": InplaceConfig("inplace_layer_bwd_bf16_128k", 1, 131072, 2560, 9728, 4096, 0.01, "dot",
                                                 "bf16", seed=1002, layer_backward=True),
    "inplace_layer_bwd_bf16_128k_kept": InplaceConfig("inplace_layer_bwd_bf16_128k_kept", 1, 131072, 2560, 9728, 4096,
                                                      0.01, "dot", "bf16", seed=1002, layer_backward=True,
                                                      kept_states=True),
    # the backward of the MSE chunk loop at the MSE workload's shape
    "mse_bwd_bf16_4x64k": InplaceConfig("mse_bwd_bf16_4x64k", 4, 65536, 2048, 8192, 2048, 1.0, "mse", "bf16", seed=1006,
                                        backward=True),
    "mse_bwd_bf16_4x64k_kept": InplaceConfig("mse_bwd_bf16_4x64k_kept", 4, 65536, 2048, 8192, 2048, 1.0, "mse", "bf16",
                                             seed=1006, backward=True, kept_states=True),
    "mse_bf16_4x64k": InplaceConfig("mse_bf16_4x64k", 4, 65536, 2048, 8192, 2048, 1.0, "mse", "bf16", seed=1003),
    # the backward of the whole MSE-objective layer at the MSE workload's shape (states recomputed, or kept)
    "mse_layer_bwd_bf16_4x64k": InplaceConfig("mse_layer_bwd_bf16_4x64k", 4, 65536, 2048, 8192, 2048, 1.0, "mse",
                                              "bf16", seed=1003, layer_backward=True),
    "mse_layer_bwd_bf16_4x64k_kept": InplaceConfig("mse_layer_bwd_bf16_4x64k_kept", 4, 65536, 2048, 8192, 2048, 1.0,
                                                   "mse", "bf16", seed=1003, layer_backward=True, kept_states=True),
    "lact_bf16_256k": LactConfig("lact_bf16_256k", 1, 4, 262144, 512, 1024, 4096, 1.0, seed=1004),
    # the LaCT review's own update: dot-product loss, per-token learning rates, L2 weight normalisation
    "lact_bf16_256k_paper": LactConfig("lact_bf16_256k_paper", 1, 4, 262144, 512, 1024, 4096, 1.0, seed=1004,
                                       loss="dot", weight_norm=True, token_rates=True),
    # the same with the Muon update rule (L2-Normalize(W - Muon(g)))
    "lact_bf16_256k_muon": LactConfig("lact_bf16_256k_muon", 1, 4, 262144, 512, 1024, 4096, 0.05, seed=1004,
                                      loss="dot", weight_norm=True, token_rates=True, muon=True),
    # the layer's backward (every input's gradient from dLoss/dO), squared error and plain GD
    "lact_bwd_bf16_256k": LactConfig("lact_bwd_bf16_256k", 1, 4, 262144, 512, 1024, 4096, 1.0, seed=1004,
                                     backward=True),
    # the same with the states kept by the forward call (no recompute in the backward)
    "lact_bwd_bf16_256k_kept": LactConfig("lact_bwd_bf16_256k_kept", 1, 4, 262144, 512, 1024, 4096, 1.0, seed=1004,
                                          backward=True, kept_states=True),
    # the same with the update on every other chunk only (a strided block-wise mask)
    "lact_bf16_256k_strided": LactConfig("lact_bf16_256k_strided", 1, 4, 262144, 512, 1024, 4096, 1.0, seed=1004,
                                         update_every=2),
}


def workload(name: str):
    return WORKLOADS[name]


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(gen: torch.Generator, shape, var: float, dtype: torch.dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    t.mul_(math.sqrt(var))
    return t.to(dtype)


def inplace_inputs(cfg: InplaceConfig, seed: int | None = None) -> dict:
    """Draw the In-Place TTT layer inputs on the CPU.

    Returns a dict of CPU torch tensors in the workload's dtype:
      H, X0 [B, n, d]; W_gate, W_up [f, d]; W_down0 [d, f];
      W_target [d, d] (indexed [d_in, d_out]); conv_w [d, K].
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed if seed is None else seed)
    dt = _torch_dtype(cfg.dtype)
    B, n, d, f, K = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.conv_k
    out = {}
    out["H"] = _draw(gen, (B, n, d), cfg.var_h, dt)
    out["X0"] = _draw(gen, (B, n, d), cfg.var_x0, dt)
    out["W_gate"] = _draw(gen, (f, d), cfg.var_gate if cfg.var_gate is not None else 1.0 / d, dt)
    out["W_up"] = _draw(gen, (f, d), cfg.var_up if cfg.var_up is not None else 1.0 / d, dt)
    out["W_down0"] = _draw(gen, (d, f), cfg.var_down if cfg.var_down is not None else 1.0 / f, dt)
    out["W_target"] = _draw(gen, (d, d), cfg.var_target if cfg.var_target is not None else 1.0 / d, dt)
    out["conv_w"] = _draw(gen, (d, K), cfg.var_conv, dt)
    return out


def backward_inputs(cfg: InplaceConfig, seed: int | None = None) -> dict:
    """Draw the inputs of the chunk loop's backward on the CPU: Z [B, n, f],
    Vhat [B, n, d], W_down0 [d, f], dO [B, n, d] (CPU torch tensors in the
    workload's dtype)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed if seed is None else seed)
    dt = _torch_dtype(cfg.dtype)
    B, n, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    out = {}
    out["Z"] = _draw(gen, (B, n, f), cfg.var_z, dt)
    out["Vhat"] = _draw(gen, (B, n, d), cfg.var_vhat, dt)
    out["W_down0"] = _draw(gen, (d, f), cfg.var_down if cfg.var_down is not None else 1.0 / f, dt)
    out["dO"] = _draw(gen, (B, n, d), cfg.var_dout, dt)
    return out


def resume_inputs(cfg: InplaceConfig, seed: int) -> dict:
    """Draw what a resumed row brings from an earlier call, on the CPU:
    W_init [B, d, f] fp32 (a state: W_down0's distribution, per row) and
    x0_halo [B, K-1, d] in the workload's dtype (X0's distribution)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    B, d, f, K = cfg.batch, cfg.d_model, cfg.d_ff, cfg.conv_k
    var_w = cfg.var_down if cfg.var_down is not None else 1.0 / f
    return {"W_init": _draw(gen, (B, d, f), var_w, torch.float32),
            "x0_halo": _draw(gen, (B, K - 1, d), cfg.var_x0, _torch_dtype(cfg.dtype))}


def lact_inputs(cfg: LactConfig, seed: int | None = None) -> dict:
    """Draw the LaCT layer inputs on the CPU.

    Returns q, k, v [B, H, n, dh] (L2-normalised over dh per token, then
    rounded), W1, W3 [H, m, dh], W2 [H, dh, m], and with token_rates the
    per-token learning rates eta_tok [B, H, n] (fp32, U(0, 1)), drawn last.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed if seed is None else seed)
    dt = _torch_dtype(cfg.dtype)
    B, Hh, n, dh, m = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.hidden
    out = {}
    for name in ("q", "k", "v"):
        t = torch.randn(B, Hh, n, dh, generator=gen, dtype=torch.float32)
        t = t / t.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        out[name] = t.to(dt)
    out["W1"] = _draw(gen, (Hh, m, dh), cfg.var_w1 if cfg.var_w1 is not None else 1.0 / dh, dt)
    out["W3"] = _draw(gen, (Hh, m, dh), cfg.var_w3 if cfg.var_w3 is not None else 1.0 / dh, dt)
    out["W2"] = _draw(gen, (Hh, dh, m), cfg.var_w2 if cfg.var_w2 is not None else 1.0 / m, dt)
    if cfg.token_rates:
        out["eta_tok"] = torch.rand(B, Hh, n, generator=gen, dtype=torch.float32)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor (bf16 or fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Goes through torch's float32 -> bfloat16 conversion; the float64 -> float32
    step is exact for the values this is used on (already-representable or
    test-constructed inputs)."""
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
