"""Throughput of the chunk-wise TTT fast-weight layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole layer call on one batch of synthetic input (the seeded
generators of ttt_inputs), inputs resident in HBM before the timed region:
  In-Place (dot):  produce Z, produce V^ (conv + projection), fused chunk
                   update + prefix scan, apply -- the four launches that
                   ttt_chunk_apply_update makes, called through the C ABI's
                   step entry points so that each kernel is bracketed by HIP
                   events on the launch stream;
  In-Place (mse):  ttt_chunk_apply_update (producers + in-order scan);
  LaCT:            ttt_lact_swiglu;
  backward:        ttt_core_backward (gradients of Z, V^ and W_down0 through
                   the dot chunk loop, given dLoss/dO).
Prints one JSON line.  The CPU baseline is the float64 oracle timed on a
bounded prefix of the same workload (whole chunks), on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-layer tokens/s (apply+update) at 32K/128K ctx; % of bf16 MFMA peak"
PEAK = {"bf16": 2500.0, "f32": 157.3}          # dense MFMA TFLOP/s, MI355X
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="inplace_bf16_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary figures (32K context; 128K with chunk 512)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference point for HBM byte counters)")
    return ap.parse_args()


def kernel_flops(cfg):
    """Algorithmic flops of each launch of the dot-mode step (per call)."""
    T, d, f, K = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.conv_k
    return {
        "produce_z": 4.0 * T * d * f,
        "produce_vhat": 2.0 * T * d * d + 2.0 * K * T * d,
        "update_scan": 2.0 * T * d * f,
        "apply": 2.0 * T * d * f,
    }


def kernel_bytes(cfg, esz=2):
    """Algorithmic HBM bytes of each launch: each operand read once, each result written once."""
    T, d, f, k, B = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.n_chunks, cfg.batch
    return {
        "produce_z": esz * (T * d + 2 * f * d + T * f),
        "produce_vhat": esz * (T * d + d * d + d * cfg.conv_k + T * d),
        "update_scan": esz * (T * f + T * d + d * f + B * k * d * f) + 4 * B * d * f,
        "apply": esz * (T * f + B * k * d * f + T * d),
    }


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none for this workload or the kernel sources changed since."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    h = hashlib.sha256()
    for f in ("common.hpp", "gemm.hpp", "inplace.hip"):
        with open(os.path.join(ROOT, "chunk_wise_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec["bytes_per_launch"].get("k_" + kernel)


def bench_inplace_dot(cfg, steps, warmup):
    import torch

    import chunk_wise_weight_amd as cw
    import ttt_inputs as ti

    x = ti.inplace_inputs(cfg)
    g = {k: v.cuda() for k, v in x.items()}
    B, n, d, f, C = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk
    k = n // C
    dt = g["H"].dtype
    Zt = torch.empty(B, f, n, dtype=dt, device="cuda")
    Vt = torch.empty(B, d, n, dtype=dt, device="cuda")
    Wc = torch.empty(B, k, d, f, dtype=dt, device="cuda")
    Wf = torch.empty(B, d, f, dtype=torch.float32, device="cuda")
    O = torch.empty(B, n, d, dtype=dt, device="cuda")
    shape = cw.InplaceShape(B, n, d, f, C, cfg.conv_k)
    vws = torch.empty(cw.ttt_vhat_workspace_bytes(shape, dt), dtype=torch.uint8, device="cuda")
    uws = torch.empty(max(1, cw.ttt_update_scan_workspace_bytes(shape, dt)), dtype=torch.uint8, device="cuda")
    names = ["produce_z", "produce_vhat", "update_scan", "apply"]

    def step(ev=None):
        if ev: ev[0].record()
        cw.ttt_produce_z(g["H"], g["W_gate"], g["W_up"], None, Zt, with_z=False)
        if ev: ev[1].record()
        cw.ttt_produce_vhat(g["X0"], g["conv_w"], g["W_target"], Vt, vws, scale=cfg.eta)
        if ev: ev[2].record()
        cw.ttt_chunk_update_scan(Zt, Vt, g["W_down0"], C, Wc, Wf, uws)
        if ev: ev[3].record()
        cw.ttt_chunk_apply(Zt, Wc, C, O)
        if ev: ev[4].record()

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {nm: sum(events[i][j].elapsed_time(events[i][j + 1]) for i in range(steps)) / steps
           for j, nm in enumerate(names)}
    del Zt, Vt, Wc, O, g
    return wall, per, Wf


def bench_generic(cfg, steps, warmup):
    """Whole-call timing (MSE In-Place, the dot layer's variants, the backward, or LaCT)."""
    import torch

    import chunk_wise_weight_amd as cw
    import ttt_inputs as ti

    if getattr(cfg, "layer_backward", False):
        x = ti.inplace_inputs(cfg)
        g = {k: v.cuda() for k, v in x.items()}
        dO = ti.backward_inputs(cfg.with_(seed=cfg.seed + 3))["dO"].cuda()
        B, n, d, f, K = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.conv_k
        dt = g["H"].dtype
        w = (g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"])
        Ws = None
        if cfg.kept_states:
            # the forward layer keeps its states (before the timed region, like the other inputs)
            Ws = torch.empty(B, n // cfg.chunk, d, f, dtype=dt, device="cuda")
            cw.ttt_chunk_apply_update(*w, cfg.chunk, cfg.eta, cfg.mode, W_states=Ws)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        grads = tuple(torch.empty(*shp, dtype=t, device="cuda") for shp, t in (
            ((B, n, d), dt), ((B, n, d), dt), ((f, d), torch.float32), ((f, d), torch.float32),
            ((d, f), torch.float32), ((d, d), torch.float32), ((d, K), torch.float32)))
        shape = cw.InplaceShape(B, n, d, f, cfg.chunk, K)
        nbytes = cw.ttt_layer_backward_workspace_bytes(shape, dt, cfg.kept_states, cfg.mode)
        ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
        call = lambda: cw.ttt_layer_backward(*w, dO, cfg.chunk, cfg.eta, W_states=Ws, grads=grads, workspace=ws,
                                             mode=cfg.mode)
    elif getattr(cfg, "backward", False) and not isinstance(cfg, ti.LactConfig):
        x = ti.backward_inputs(cfg)
        g = {k: v.cuda() for k, v in x.items()}
        B, n, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
        dt = g["Z"].dtype
        dZ = torch.empty(B, n, f, dtype=dt, device="cuda")
        dV = torch.empty(B, n, d, dtype=dt, device="cuda")
        dW0 = torch.empty(d, f, dtype=torch.float32, device="cuda")
        shape = cw.InplaceShape(B, n, d, f, cfg.chunk, 1)
        Ws = None
        if cfg.mode == "mse":
            if cfg.kept_states:
                # the forward MSE scan keeps its states (before the timed region, like the other inputs)
                Ws = torch.empty(B, n // cfg.chunk, d, f, dtype=dt, device="cuda")
                cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], cfg.chunk, cfg.eta, "mse", W_states=Ws)
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            nbytes = cw.ttt_core_backward_mse_workspace_bytes(shape, dt, cfg.kept_states)
            ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
            call = lambda: cw.ttt_core_backward_mse(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta, dZ,
                                                    dV, dW0, ws, W_states=Ws)
        elif cfg.kept_states:
            # the forward chunk loop keeps its states (before the timed region, like the other inputs)
            Ws = torch.empty(B, n // cfg.chunk, d, f, dtype=dt, device="cuda")
            cw.ttt_core_apply_update(g["Z"], g["Vhat"], g["W_down0"], cfg.chunk, cfg.eta, "dot", W_states=Ws)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        if cfg.mode != "mse":
            nbytes = cw.ttt_core_backward_workspace_bytes(shape, dt, cfg.kept_states)
            ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
            call = lambda: cw.ttt_core_backward(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta, dZ, dV,
                                                dW0, ws, W_states=Ws)
    elif isinstance(cfg, ti.LactConfig) and cfg.backward:
        x = ti.lact_inputs(cfg)
        g = {k: v.cuda() for k, v in x.items()}
        dO = lact_upstream(cfg, x).cuda()
        B, Hh, n, dh, m = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.hidden
        dt = g["q"].dtype
        grads = tuple(torch.empty(*shp, dtype=t, device="cuda") for shp, t in (
            ((B, Hh, n, dh), dt), ((B, Hh, n, dh), dt), ((B, Hh, n, dh), dt), ((Hh, m, dh), torch.float32),
            ((Hh, m, dh), torch.float32), ((Hh, dh, m), torch.float32)))
        Ws = None
        if cfg.kept_states:        # the forward call keeps its states (untimed); the backward reads them
            Ws = torch.empty(n // cfg.chunk + 1, B, Hh, 3, m * dh, dtype=dt, device="cuda")
            cw.ttt_lact_swiglu(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta, cfg.order,
                               W_states=Ws)
        nbytes = cw.ttt_lact_backward_workspace_bytes(cw.LactShape(B, Hh, n, dh, m, cfg.chunk), dt, Ws is not None)
        ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
        call = lambda: cw.ttt_lact_swiglu_backward(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO, cfg.chunk,
                                                   cfg.eta, cfg.order, grads=grads, workspace=ws, W_states=Ws)
    elif isinstance(cfg, ti.LactConfig):
        x = ti.lact_inputs(cfg)
        g = {k: v.cuda() for k, v in x.items()}
        side = cw.LactSideStream()      # the (batch, head) rows as two chains, on the current and a side stream
        call = lambda: cw.ttt_lact_swiglu(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta,
                                          cfg.order, update_mask=cfg.update_mask(), eta_tok=g.get("eta_tok"),
                                          loss=cfg.loss, weight_norm=cfg.weight_norm, muon=cfg.muon, side=side)
    else:
        x = ti.inplace_inputs(cfg)
        g = {k: v.cuda() for k, v in x.items()}
        flags = cfg.doc_starts()
        docs = None if flags is None else torch.from_numpy(flags).cuda()
        w = (g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"])
        if cfg.pieces > 1:
            # the sequence in equal pieces, each call resuming the previous one's state and conv halo
            L, K = cfg.seq_len // cfg.pieces, cfg.conv_k
            Hs = [g["H"][:, i * L:(i + 1) * L].contiguous() for i in range(cfg.pieces)]
            Xs = [g["X0"][:, i * L:(i + 1) * L].contiguous() for i in range(cfg.pieces)]
            halos = [None] + [g["X0"][:, i * L - (K - 1): i * L].contiguous() for i in range(1, cfg.pieces)]

            def call():
                Wf = None
                for i in range(cfg.pieces):
                    _, Wf = cw.ttt_chunk_apply_update(Hs[i], Xs[i], *w, cfg.chunk, cfg.eta, cfg.mode, W_init=Wf,
                                                      x0_halo=halos[i])
        else:
            call = lambda: cw.ttt_chunk_apply_update(g["H"], g["X0"], *w, cfg.chunk, cfg.eta, cfg.mode,
                                                     doc_starts=docs, conv_forward=cfg.conv_forward)
    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, {"layer": e0.elapsed_time(e1) / steps}


def lact_upstream(cfg, x):
    """The upstream gradient dLoss/dO of the LaCT backward: standard normal, seeded after the layer's inputs."""
    import torch
    gen = torch.Generator().manual_seed(cfg.seed + 7)
    return torch.randn(*x["q"].shape, generator=gen).to(x["q"].dtype)


def cpu_baseline(cfg, target_s):
    """The float64 oracle on whole leading chunks of the same workload."""
    import numpy as np
    import threadpoolctl

    import ttt_inputs as ti
    from oracle import inplace as orc
    from oracle import lact as olact

    # the host cores this process may run on, with the BLAS pool sized to match
    cores = len(os.sched_getaffinity(0))
    threadpoolctl.threadpool_limits(limits=cores)
    if isinstance(cfg, ti.LactConfig) and cfg.backward:
        x = ti.lact_inputs(cfg)
        dO = lact_upstream(cfg, x)
        run = lambda kc: olact.lact_backward(*(ti.to_f64(x[k][:, :1, : kc * cfg.chunk]) if k in "qkv"
                                               else ti.to_f64(x[k][:1]) for k in ("q", "k", "v", "W1", "W3", "W2")),
                                             cfg.chunk, cfg.eta, ti.to_f64(dO[:, :1, : kc * cfg.chunk]), cfg.order)
        per_tok_heads = 1
    elif isinstance(cfg, ti.LactConfig):
        x = ti.lact_inputs(cfg)
        umask = cfg.update_mask()
        run = lambda kc: olact.lact_layer(*(ti.to_f64(x[k][:, :1, : kc * cfg.chunk]) if k in "qkv"
                                            else ti.to_f64(x[k][:1]) for k in ("q", "k", "v", "W1", "W3", "W2")),
                                          cfg.chunk, cfg.eta, cfg.order,
                                          update_mask=None if umask is None else umask[:kc],
                                          eta_tok=(ti.to_f64(x["eta_tok"][:, :1, : kc * cfg.chunk])
                                                   if cfg.token_rates else None),
                                          loss=cfg.loss, weight_norm=cfg.weight_norm, use_muon=cfg.muon)
        per_tok_heads = 1
    elif cfg.layer_backward:
        x = ti.inplace_inputs(cfg)
        ws = {k: ti.to_f64(x[k]) for k in ("W_gate", "W_up", "W_down0", "W_target", "conv_w")}
        dO = ti.backward_inputs(cfg.with_(seed=cfg.seed + 3))["dO"]
        run = lambda kc: orc.layer_backward(ti.to_f64(x["H"][:1, : kc * cfg.chunk]),
                                            ti.to_f64(x["X0"][:1, : kc * cfg.chunk]), ws["W_gate"], ws["W_up"],
                                            ws["W_down0"], ws["W_target"], ws["conv_w"], cfg.chunk, cfg.eta,
                                            ti.to_f64(dO[:1, : kc * cfg.chunk]), mode=cfg.mode)
    elif cfg.backward:
        x = ti.backward_inputs(cfg)
        W0 = ti.to_f64(x["W_down0"])
        back = orc.mse_core_backward if cfg.mode == "mse" else orc.chunk_core_backward
        run = lambda kc: back(*(ti.to_f64(x[k][0, : kc * cfg.chunk]) for k in ("Z", "Vhat")), W0, cfg.chunk, cfg.eta,
                              ti.to_f64(x["dO"][0, : kc * cfg.chunk]))
    else:
        x = ti.inplace_inputs(cfg)
        ws = {k: ti.to_f64(x[k]) for k in ("W_gate", "W_up", "W_down0", "W_target", "conv_w")}
        flags = cfg.doc_starts()
        run = lambda kc: orc.inplace_layer(ti.to_f64(x["H"][:1, : kc * cfg.chunk]),
                                           ti.to_f64(x["X0"][:1, : kc * cfg.chunk]), ws["W_gate"], ws["W_up"],
                                           ws["W_down0"], ws["W_target"], ws["conv_w"], cfg.chunk, cfg.eta,
                                           "dot" if cfg.mode == "dot_scan" else cfg.mode,
                                           doc_starts=None if flags is None else flags[:1, :kc],
                                           conv_forward=cfg.conv_forward)
    t0 = time.perf_counter()
    run(1)
    t1 = time.perf_counter() - t0
    kc = int(max(1, min(cfg.n_chunks, target_s // max(t1, 1e-9))))
    if kc > 1:
        t0 = time.perf_counter()
        run(kc)
        t1 = time.perf_counter() - t0
    tokens = kc * cfg.chunk
    if isinstance(cfg, ti.LactConfig):
        sample = f"first {kc} chunk(s) of {cfg.chunk} tokens, batch row 0, head 0 of {cfg.heads}"
        value = tokens / t1 / cfg.heads          # whole-layer tokens/s (all heads)
    else:
        sample = f"first {kc} chunk(s) of {cfg.chunk} tokens of batch row 0 (of {cfg.n_chunks} x {cfg.batch})"
        value = tokens / t1
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "sample": sample,
            "seconds": t1}


def calibrate_copy(mib, steps):
    """A plain copy of known size: reads and writes mib MiB once per launch."""
    import torch

    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": steps}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, args.steps)
        return

    import ttt_inputs as ti

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = ti.workload(args.workload)
    dtype = cfg.dtype
    out = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded Gaussian inputs and random-init weights of the stated shapes)"}
    if isinstance(cfg, ti.LactConfig):
        out["config"] = {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.heads, "seq_len": cfg.seq_len,
                         "head_dim": cfg.head_dim, "hidden": cfg.hidden, "chunk": cfg.chunk, "eta": cfg.eta,
                         "order": cfg.order}
        if cfg.update_every > 1:
            out["config"]["update_every"] = cfg.update_every
        if cfg.loss != "mse" or cfg.weight_norm or cfg.token_rates or cfg.muon:
            out["config"].update({"loss": cfg.loss, "weight_norm": cfg.weight_norm, "token_rates": cfg.token_rates,
                                  "muon": cfg.muon})
        if cfg.backward:
            out["config"]["pass"] = "backward of the LaCT layer (dq, dk, dv and the initial weights' gradients)"
            out["config"]["states"] = "kept by the forward call" if cfg.kept_states else "recomputed"
            out["metric"] = "LaCT-layer backward tokens/s at 256K ctx; % of bf16 MFMA peak"
    else:
        out["config"] = {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq_len, "d_model": cfg.d_model,
                         "d_ff": cfg.d_ff, "chunk": cfg.chunk, "conv_k": cfg.conv_k, "eta": cfg.eta,
                         "mode": cfg.mode}
        if cfg.docs > 1:
            out["config"]["docs_per_row"] = cfg.docs
        if cfg.conv_forward:
            out["config"]["conv"] = "forward in-chunk"
        if cfg.pieces > 1:
            out["config"]["calls_per_sequence"] = cfg.pieces
        if cfg.backward:
            out["config"]["pass"] = "backward of the chunk loop (dZ, dVhat, dW_down0 from dLoss/dO)"
            out["config"]["states"] = "kept by the forward call" if cfg.kept_states else "recomputed"
            out["metric"] = ("TTT chunk-loop backward tokens/s at " + ("4x64K" if cfg.mode == "mse" else "128K") +
                             " ctx; % of bf16 MFMA peak")
        if cfg.layer_backward:
            out["config"]["pass"] = "backward of the whole layer (every input and weight gradient from dLoss/dO)"
            out["config"]["states"] = "kept by the forward call" if cfg.kept_states else "recomputed"
            out["metric"] = ("TTT-layer backward tokens/s at " + ("4x64K" if cfg.mode == "mse" else "128K") +
                             " ctx; % of bf16 MFMA peak")

    if (not isinstance(cfg, ti.LactConfig) and cfg.mode == "dot" and cfg.docs == 1 and not cfg.conv_forward and
            cfg.pieces == 1 and not cfg.backward and not cfg.layer_backward):
        wall, per, _ = bench_inplace_dot(cfg, args.steps, args.warmup)
        fl, by = kernel_flops(cfg), kernel_bytes(cfg, 2 if dtype == "bf16" else 4)
        kern = {}
        for nm, ms in per.items():
            tf = fl[nm] / (ms * 1e-3) / 1e12
            kern[nm] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK[dtype], 4),
                        "alg_GBs": round(by[nm] / (ms * 1e-3) / 1e9, 1)}
        out["kernels"] = kern
        dom = max(per, key=per.get)
        ach = fl[dom] / (per[dom] * 1e-3) / 1e12
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK[dtype],
                           "unit": "TFLOP/s", "frac": round(ach / PEAK[dtype], 4),
                           "traffic": measured_traffic(cfg.name, dom)}
    else:
        wall, per = bench_generic(cfg, args.steps, args.warmup)
        ms = per["layer"]
        ach = cfg.flops() / (ms * 1e-3) / 1e12
        out["roofline"] = {"kernel": "layer", "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK[dtype],
                           "unit": "TFLOP/s", "frac": round(ach / PEAK[dtype], 4), "traffic": None}
    ms_step = wall / args.steps * 1e3
    out["ms_per_step"] = round(ms_step, 4)
    out["value"] = round(cfg.tokens / (ms_step * 1e-3), 1)
    tf = cfg.flops() / (ms_step * 1e-3) / 1e12
    out["tflops"] = round(tf, 1)
    out["frac_bf16_mfma_peak"] = round(tf / PEAK["bf16"], 4)
    if args.workload == "inplace_bf16_128k" and not args.no_secondary:
        c2 = ti.workload("inplace_bf16_32k")
        w2, p2, _ = bench_inplace_dot(c2, max(5, args.steps // 2), args.warmup)
        ms2 = w2 / max(5, args.steps // 2) * 1e3
        out["secondary"] = {"workload": c2.name, "ms_per_step": round(ms2, 4),
                            "value": round(c2.tokens / (ms2 * 1e-3), 1),
                            "tflops": round(c2.flops() / (ms2 * 1e-3) / 1e12, 1),
                            "frac_bf16_mfma_peak": round(c2.flops() / (ms2 * 1e-3) / 1e12 / PEAK["bf16"], 4)}
        torch.cuda.empty_cache()
        # the same 128K layer with chunk 512: 256 per-chunk states instead of 32
        c3 = ti.workload("inplace_bf16_128k_c512")
        n3 = max(3, args.steps // 4)
        w3, p3, _ = bench_inplace_dot(c3, n3, min(args.warmup, 1))
        ms3 = w3 / n3 * 1e3
        out["small_chunk"] = {"workload": c3.name, "chunk": c3.chunk, "ms_per_step": round(ms3, 4),
                              "value": round(c3.tokens / (ms3 * 1e-3), 1),
                              "frac_bf16_mfma_peak": round(c3.flops() / (ms3 * 1e-3) / 1e12 / PEAK["bf16"], 4),
                              "kernels_ms": {k: round(v, 4) for k, v in p3.items()}}
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
