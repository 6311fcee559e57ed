"""The layer calls captured into HIP graphs (torch.cuda.CUDAGraph drives the capture).

The library enqueues kernels only -- no allocation, copy or memset (the chained update-scan clears its flags with a
kernel) -- and the LaCT call given a side stream adds an event fork and join with it, which a capture records as
parallel branches.  The backward entry points (the dot and MSE
chunk loops, the whole dot layer, the LaCT layer) are captured the same way.  Each graph is replayed three times with
the outputs clobbered, eager calls and synchronisations in between, and every replay must reproduce the eager
call's bits.
"""
import pytest
import torch

import chunk_wise_weight_amd as cw
import ttt_inputs as ti

pytestmark = pytest.mark.gpu


def _inplace(mode):
    if mode == "dot_chained":       # a 260-tile state: the fused scan runs two chained segments (flags zeroed per call)
        cfg = ti.InplaceConfig("graph", 1, 1024, 2560, 6656, 256, 0.02, "dot", "bf16", conv_k=4, seed=29)
    else:
        cfg = ti.InplaceConfig("graph", 2, 1024, 264, 392, 256, 0.05 if mode == "dot" else 0.5, mode, "bf16",
                               conv_k=4, seed=13)
    mode = cfg.mode
    g = {k: v.cuda() for k, v in ti.inplace_inputs(cfg).items()}
    args = (g["H"], g["X0"], g["W_gate"], g["W_up"], g["W_down0"], g["W_target"], g["conv_w"], cfg.chunk, cfg.eta,
            mode)
    return lambda: cw.ttt_chunk_apply_update(*args)


def _lact(two_chains):
    cfg = ti.LactConfig("graph", 1, 3, 512, 64, 128, 128, 0.7, "update_then_apply", "bf16", seed=17)
    g = {k: v.cuda() for k, v in ti.lact_inputs(cfg).items()}
    args = (g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], cfg.chunk, cfg.eta, cfg.order)
    side = cw.LactSideStream() if two_chains else None     # created before the capture
    return lambda: cw.ttt_lact_swiglu(*args, side=side)


def _lact_backward():
    cfg = ti.LactConfig("graph", 2, 2, 384, 64, 128, 128, 0.7, "update_then_apply", "bf16", seed=23)
    g = {k: v.cuda() for k, v in ti.lact_inputs(cfg).items()}
    dO = torch.randn(*g["q"].shape, generator=torch.Generator().manual_seed(24)).to(g["q"].dtype).cuda()
    return lambda: cw.ttt_lact_swiglu_backward(g["q"], g["k"], g["v"], g["W1"], g["W3"], g["W2"], dO, cfg.chunk,
                                               cfg.eta, cfg.order)


def _backward(kind):
    cfg = ti.InplaceConfig("graph", 2, 512, 264, 392, 128, 0.05 if kind != "mse_backward" else 0.5,
                           "mse" if kind == "mse_backward" else "dot", "bf16", seed=19, backward=True)
    g = {k: v.cuda() for k, v in ti.backward_inputs(cfg).items()}
    if kind == "layer_backward":
        x = {k: v.cuda() for k, v in ti.inplace_inputs(cfg.with_(backward=False)).items()}
        args = (x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down0"], x["W_target"], x["conv_w"], g["dO"])
        return lambda: cw.ttt_layer_backward(*args, cfg.chunk, cfg.eta)
    fn = cw.ttt_core_backward_mse if kind == "mse_backward" else cw.ttt_core_backward
    return lambda: fn(g["Z"], g["Vhat"], g["W_down0"], g["dO"], cfg.chunk, cfg.eta)


@pytest.mark.parametrize("kind", ["dot", "dot_chained", "mse", "lact", "lact_side", "backward", "mse_backward",
                                  "layer_backward", "lact_backward"])
def test_graph_replays_match_eager(kind):
    call = (_lact_backward() if kind == "lact_backward" else _lact(kind == "lact_side") if kind.startswith("lact")
            else _backward(kind) if "backward" in kind else _inplace(kind))
    eager = call()
    torch.cuda.synchronize()
    # warm-up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    for r in range(3):
        for t in out:
            t.fill_(float("nan"))
        again = call()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(again, eager)), r
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(out, eager)), r
