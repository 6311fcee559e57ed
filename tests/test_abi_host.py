"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ttt.h declares, sizes workspaces, and rejects bad
arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import chunk_wise_weight_amd as cw
from chunk_wise_weight_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = cw.lib()
    declared = _declared()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(declared) == sorted(cw.exported_symbols())


def test_status_strings():
    for st in range(8):
        assert cw.status_string(st).startswith("TTT_")
    assert cw.status_string(99) == "unknown status"


def _shape(B=1, n=2048, d=256, f=512, C=256, K=4):
    return cw.InplaceShape(B, n, d, f, C, K)


def _ws(shape, dtype=cw.TTT_BF16, mode=cw.TTT_MODE_DOT, prod=1):
    out = ctypes.c_size_t(0)
    st = cw.lib().ttt_inplace_workspace_bytes(ctypes.byref(shape), dtype, mode, prod, ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    B, n, d, f, C = 1, 2048, 256, 512, 256
    k = n // C
    al = lambda x: (x + 255) // 256 * 256
    core = lambda e, B=B: al(B * n * f * e) + al(B * n * d * e)          # Zt, Vt
    # producers: conv output and W_target^T (Z itself is only kept token-contiguous, as Zt)
    prod = lambda e: al(B * n * d * e) + al(d * d * e)
    # the fused dot plan of this 2-tile state runs 4 sequence segments: partial states of the last 6
    # chunks (dtype) and 3 fp32 segment totals
    seg = lambda e: al(B * (k - k // 4) * d * f * e) + al(B * 3 * d * f * 4)
    st, nb = _ws(_shape(), cw.TTT_F32, cw.TTT_MODE_DOT, 1)
    assert st == cw.TTT_OK
    assert nb == prod(4) + core(4) + al(B * k * d * f * 4) + seg(4)
    st, nb = _ws(_shape(), cw.TTT_BF16, cw.TTT_MODE_MSE, 1)
    assert st == cw.TTT_OK and nb == prod(2) + core(2) + al(C * d * 2) + al(d * f * 2)
    st, nb = _ws(_shape(), cw.TTT_BF16, cw.TTT_MODE_DOT_SCAN, 0)
    assert st == cw.TTT_OK and nb == core(2) + al(B * k * d * f * 2) + al(B * k * d * f * 4)
    st, nb = _ws(_shape(B=4), cw.TTT_BF16, cw.TTT_MODE_MSE, 0)
    assert st == cw.TTT_OK and nb == core(2, 4) + al(4 * C * d * 2) + al(4 * d * f * 2)
    st, nb = _ws(_shape(B=4), cw.TTT_F32, cw.TTT_MODE_MSE, 0)
    assert st == cw.TTT_OK and nb == core(4, 4) + al(4 * C * d * 4)
    # chunk not a multiple of the 64-element K step: dot falls back to the materialised scan
    n2 = 2000
    st, nb = _ws(_shape(n=n2, C=40), cw.TTT_BF16, cw.TTT_MODE_DOT, 0)
    assert st == cw.TTT_OK and nb == al(n2 * f * 2) + al(n2 * d * 2) + al(50 * d * f * 2) + al(50 * d * f * 4)
    out = ctypes.c_size_t(0)
    assert cw.lib().ttt_vhat_workspace_bytes(ctypes.byref(_shape()), cw.TTT_BF16, ctypes.byref(out)) == cw.TTT_OK
    assert out.value == al(n * d * 2) + al(d * d * 2)


def _update_scan_ws(shape, dtype=cw.TTT_BF16):
    out = ctypes.c_size_t(0)
    st = cw.lib().ttt_update_scan_workspace_bytes(ctypes.byref(shape), dtype, ctypes.byref(out))
    return st, out.value


def test_update_scan_segments_and_workspace():
    """The fused update-scan runs the sequence as S segments (S in 1, 2, 4 dividing the chunk count) when
    the model of its time -- rounds of 256 tiles times tokens per segment, with four segments plus the fix-up
    pass over the later segments' partial states, with two (chained) at least two rounds -- says so (S depends
    on the state's and the sequence's shape only, so rows do not depend on the batch they are in); its scratch
    holds the partial states of chunks past the first segment (bf16 here) and the S - 1 fp32 segment totals."""
    al = lambda x: (x + 255) // 256 * 256

    def expect(B, n, d, f, C):
        k = n // C
        tiles = -(-f // 256) * -(-d // 256)
        def cost(S):
            rounds = -(-tiles * S // 256)
            if S == 2:
                rounds = max(rounds, 2)
            return rounds * (k * C // S) * 28.1e-9 + ((k - k // S) * d * f * 4.0 / 5.5e12 if S > 2 else 0.0)
        S = 1
        for cand in (2, 4):
            if k % cand == 0 and cost(cand) < cost(S):
                S = cand
        return S, (0 if S == 1 else al(B * (k - k // S) * d * f * 2) + al(B * (S - 1) * d * f * 4))

    cases = [(1, 131072, 2560, 9728, 4096, 2), (1, 32768, 2560, 9728, 1024, 2), (1, 2048, 1024, 4096, 256, 4),
             (2, 1024, 1024, 4096, 128, 4), (1, 2048, 256, 512, 256, 4), (4, 65536, 2048, 8192, 2048, 1),
             (1, 131072, 2560, 9728, 512, 2),    # 256 short chunks: chained, no fix-up over 128 partial states
             (1, 4096, 2560, 9728, 4096, 1)]     # one chunk: nothing to split
    for B, n, d, f, C, S in cases:
        s_exp, ws = expect(B, n, d, f, C)
        assert s_exp == S, (B, n, d, f, C)
        st, nb = _update_scan_ws(cw.InplaceShape(B, n, d, f, C, 4))
        assert st == cw.TTT_OK and nb == ws, (B, n, d, f, C)
    # the layer's workspace carries the same regions in the fused dot plan
    s = cw.InplaceShape(1, 2048, 1024, 4096, 256, 4)
    st_seg, nb_seg = _ws(s, cw.TTT_BF16, cw.TTT_MODE_DOT, 0)
    B, n, d, f, k = 1, 2048, 1024, 4096, 8
    core = al(B * n * f * 2) + al(B * n * d * 2)
    assert st_seg == cw.TTT_OK and nb_seg == core + al(B * k * d * f * 2) + _update_scan_ws(s)[1]
    assert _update_scan_ws(cw.InplaceShape(1, 2048, 256, 512, 32, 4))[0] == cw.TTT_ERR_UNSUPPORTED
    assert cw.lib().ttt_update_scan_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, None) == cw.TTT_ERR_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(n=2000, C=256), cw.TTT_ERR_SHAPE),      # seq_len % chunk != 0
    (dict(C=0), cw.TTT_ERR_SHAPE),
    (dict(B=-1), cw.TTT_ERR_SHAPE),
    (dict(d=0), cw.TTT_ERR_SHAPE),
    (dict(K=0), cw.TTT_ERR_SHAPE),
    (dict(d=252), cw.TTT_ERR_UNSUPPORTED),        # d % 8
    (dict(f=500), cw.TTT_ERR_UNSUPPORTED),
    (dict(n=2044, C=4), cw.TTT_ERR_UNSUPPORTED),  # chunk % 8
    (dict(K=9), cw.TTT_ERR_UNSUPPORTED),
])
def test_shape_errors(kw, status):
    assert _ws(_shape(**kw))[0] == status


def test_dtype_and_mode_errors():
    assert _ws(_shape(), 7)[0] == cw.TTT_ERR_DTYPE
    assert _ws(_shape(), cw.TTT_BF16, 9)[0] == cw.TTT_ERR_ARG
    out = ctypes.c_size_t(0)
    assert cw.lib().ttt_inplace_workspace_bytes(None, cw.TTT_BF16, 0, 1, ctypes.byref(out)) == cw.TTT_ERR_ARG
    assert cw.lib().ttt_inplace_workspace_bytes(ctypes.byref(_shape()), cw.TTT_BF16, 0, 1, None) == cw.TTT_ERR_ARG


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)   # never dereferenced: every call below fails validation first


def test_call_rejects_null_and_misaligned_pointers_before_device_work():
    lib = cw.lib()
    s = _shape()
    st, nb = _ws(s, cw.TTT_BF16, cw.TTT_MODE_DOT, 1)
    p = [_fake() for _ in range(9)]
    # null H
    assert lib.ttt_chunk_apply_update(ctypes.byref(s), cw.TTT_BF16, 0, 0.1, None, *p[:8], _fake(), nb, None) == \
        cw.TTT_ERR_ARG
    # misaligned O
    args = [_fake() for _ in range(7)] + [ctypes.c_void_p(0x100004), _fake()]
    assert lib.ttt_chunk_apply_update(ctypes.byref(s), cw.TTT_BF16, 0, 0.1, *args, _fake(), nb, None) == \
        cw.TTT_ERR_ARG
    # workspace too small / missing
    args = [_fake() for _ in range(9)]
    assert lib.ttt_chunk_apply_update(ctypes.byref(s), cw.TTT_BF16, 0, 0.1, *args, _fake(), nb - 1, None) == \
        cw.TTT_ERR_WORKSPACE
    assert lib.ttt_chunk_apply_update(ctypes.byref(s), cw.TTT_BF16, 0, 0.1, *args, None, nb, None) == \
        cw.TTT_ERR_WORKSPACE
    # non-finite eta
    assert lib.ttt_chunk_apply_update(ctypes.byref(s), cw.TTT_BF16, 0, float("nan"), *args, _fake(), nb, None) == \
        cw.TTT_ERR_ARG
    # bad dtype on the core entry point
    assert lib.ttt_core_apply_update(ctypes.byref(s), 5, 0, 0.1, *[_fake() for _ in range(6)], nb, None) == \
        cw.TTT_ERR_DTYPE


def test_noalloc_entry_point_rejects_what_its_static_scratch_cannot_hold():
    lib = cw.lib()
    assert cw.TTT_NOALLOC_SCRATCH_BYTES == 64 << 20
    args = [_fake() for _ in range(9)]
    # the fp32 layer of 2048 tokens (d 256, d_ff 512, chunk 256) needs 16.75 MiB: it fits, so it passes validation
    # (not called here: it would run); 2 x 4096 bf16 tokens at d 512, d_ff 1024, chunk 512 need 72.5 MiB
    st, nb = _ws(_shape(), cw.TTT_F32, cw.TTT_MODE_DOT, 1)
    assert st == cw.TTT_OK and nb <= cw.TTT_NOALLOC_SCRATCH_BYTES
    big = _shape(B=2, n=4096, d=512, f=1024, C=512)
    st, nb = _ws(big, cw.TTT_BF16, cw.TTT_MODE_DOT, 1)
    assert st == cw.TTT_OK and nb > cw.TTT_NOALLOC_SCRATCH_BYTES
    assert lib.ttt_chunk_apply_update_noalloc(ctypes.byref(big), cw.TTT_BF16, cw.TTT_MODE_DOT, 0.01, *args,
                                              None) == cw.TTT_ERR_SCRATCH_LIMIT
    assert "TTT_NOALLOC_SCRATCH_BYTES" in cw.status_string(cw.TTT_ERR_SCRATCH_LIMIT)
    # argument errors come first, as for the call with a workspace
    assert lib.ttt_chunk_apply_update_noalloc(ctypes.byref(big), cw.TTT_BF16, cw.TTT_MODE_DOT, 0.01, None,
                                              *args[1:], None) == cw.TTT_ERR_ARG
    assert lib.ttt_chunk_apply_update_noalloc(ctypes.byref(_shape(n=2000)), cw.TTT_BF16, 0, 0.01, *args,
                                              None) == cw.TTT_ERR_SHAPE


def test_step_entry_points_validate():
    lib = cw.lib()
    s = _shape()
    assert lib.ttt_produce_z(ctypes.byref(s), cw.TTT_BF16, None, _fake(), _fake(), _fake(), _fake(), None) == \
        cw.TTT_ERR_ARG
    assert lib.ttt_produce_z(ctypes.byref(s), cw.TTT_BF16, _fake(), _fake(), _fake(), _fake(), None, None) == \
        cw.TTT_ERR_ARG                                                      # Zt is required
    assert lib.ttt_produce_vhat(ctypes.byref(_shape(K=9)), cw.TTT_BF16, 1.0, *[_fake()] * 5, 1 << 30, None) == \
        cw.TTT_ERR_UNSUPPORTED
    assert lib.ttt_produce_vhat(ctypes.byref(s), cw.TTT_BF16, 1.0, *[_fake()] * 5, 16, None) == \
        cw.TTT_ERR_WORKSPACE
    assert lib.ttt_chunk_delta(ctypes.byref(_shape(n=100)), cw.TTT_BF16, *[_fake()] * 3, None) == cw.TTT_ERR_SHAPE
    assert lib.ttt_chunk_scan(ctypes.byref(s), cw.TTT_BF16, float("inf"), *[_fake()] * 4, None) == cw.TTT_ERR_ARG
    # the fused update-scan needs chunk boundaries on 64-token steps in bf16
    assert lib.ttt_chunk_update_scan(ctypes.byref(_shape(n=2048, C=32)), cw.TTT_BF16, *[_fake()] * 6, 0, None) == \
        cw.TTT_ERR_UNSUPPORTED
    # a segmented shape needs its scratch
    seg = cw.InplaceShape(1, 2048, 1024, 4096, 256, 4)
    assert lib.ttt_chunk_update_scan(ctypes.byref(seg), cw.TTT_BF16, *[_fake()] * 5, None, 0, None) == \
        cw.TTT_ERR_WORKSPACE
    assert lib.ttt_chunk_apply(ctypes.byref(s), cw.TTT_BF16, _fake(), None, _fake(), None) == cw.TTT_ERR_ARG


def test_backward_workspace_and_validation():
    """ttt_core_backward's workspace: eta V^ (row-major), the recomputed states (unless the caller keeps them) and
    the suffix states (dtype), the rows' fp32 totals, a zero start state, and the scans' own scratch: segment
    partials for the fused scan (which reads Z, V^ and dO as they are); token-contiguous copies of Z, of V^, of
    Z and dO in reverse chunk order, and fp32 per-chunk deltas for the delta + scan path."""
    lib = cw.lib()
    al = lambda x: (x + 255) // 256 * 256
    out = ctypes.c_size_t(0)

    def ws(B, n, d, f, C, dtype=cw.TTT_BF16, saved=0):
        st = lib.ttt_core_backward_workspace_bytes(ctypes.byref(cw.InplaceShape(B, n, d, f, C, 1)), dtype, saved,
                                                   ctypes.byref(out))
        return st, out.value

    B, n, d, f, C = 2, 2048, 256, 512, 256      # fused, four segments (as the forward plan of this shape)
    k, e = n // C, 2
    states = al(B * k * d * f * e)
    base = al(B * n * d * e) + states + al(B * d * f * 4) + al(d * f * e) + al(B * k)    # + reversed doc starts
    seg = al(B * (k - k // 4) * d * f * e) + al(B * 3 * d * f * 4)
    assert ws(B, n, d, f, C) == (cw.TTT_OK, base + states + seg)
    assert ws(B, n, d, f, C, saved=1) == (cw.TTT_OK, base + seg)
    # chunk 40: not on the 64-token step of the fused scan, so per-chunk fp32 deltas
    n2, C2 = 2000, 40
    k2 = n2 // C2
    base2 = al(B * n2 * d * e) + 2 * (al(B * n2 * d * e) + al(B * n2 * f * e)) + 2 * al(B * k2 * d * f * e) + \
        al(B * d * f * 4) + al(d * f * e)
    assert ws(B, n2, d, f, C2) == (cw.TTT_OK, base2 + al(B * k2 * d * f * 4) + al(B * k2))
    assert ws(0, n, d, f, C) == (cw.TTT_OK, 0) and ws(B, 0, d, f, C) == (cw.TTT_OK, 0)
    assert ws(B, 2000, d, f, C)[0] == cw.TTT_ERR_SHAPE
    assert lib.ttt_core_backward_workspace_bytes(ctypes.byref(cw.InplaceShape(B, n, d, f, C, 1)), cw.TTT_BF16, 0,
                                                 None) == cw.TTT_ERR_ARG
    s = cw.InplaceShape(B, n, d, f, C, 1)
    nb = ws(B, n, d, f, C)[1]
    ins = [_fake() for _ in range(4)]    # Z, Vhat, W_down0, dO
    outs = [_fake() for _ in range(2)]   # dZ, dVhat

    def call(eta, ins, Ws, outs, dW, w, nbytes, dtype=cw.TTT_BF16):
        return lib.ttt_core_backward(ctypes.byref(s), dtype, eta, *ins, Ws, None, *outs, dW, w, nbytes, None)

    assert call(0.1, ins, None, outs, _fake(), _fake(), nb - 1) == cw.TTT_ERR_WORKSPACE
    assert call(0.1, ins, None, outs, _fake(), None, nb) == cw.TTT_ERR_WORKSPACE
    # kept states shrink the workspace by one set of states
    assert call(0.1, ins, _fake(), outs, _fake(), _fake(), nb - states - 1) == cw.TTT_ERR_WORKSPACE
    assert call(float("nan"), ins, None, outs, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, None, outs, None, _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, [None] + ins[1:], None, outs, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins[:3] + [ctypes.c_void_p(0x100008)], None, outs, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, ctypes.c_void_p(0x100008), outs, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, None, outs, _fake(), _fake(), nb, dtype=7) == cw.TTT_ERR_DTYPE


def test_layer_backward_validation():
    """ttt_layer_backward validates before any device work: the fused scan's token step, pointers, eta, workspace."""
    lib = cw.lib()
    out = ctypes.c_size_t(0)
    s = cw.InplaceShape(1, 2048, 256, 512, 256, 4)
    assert lib.ttt_layer_backward_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, 0, ctypes.byref(out)) == cw.TTT_OK
    nb = out.value
    kept = ctypes.c_size_t(0)
    assert lib.ttt_layer_backward_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, 1, ctypes.byref(kept)) == cw.TTT_OK
    assert kept.value < nb            # kept states: no recomputed states in the workspace
    odd = cw.InplaceShape(1, 2000, 256, 512, 40, 4)     # chunk 40: off the fused scan's 64-token steps
    assert lib.ttt_layer_backward_workspace_bytes(ctypes.byref(odd), cw.TTT_BF16, 0,
                                                  ctypes.byref(out)) == cw.TTT_ERR_UNSUPPORTED
    ins = [_fake() for _ in range(8)]     # H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO
    outs = [_fake() for _ in range(7)]    # dH, dX0, dW_gate, dW_up, dW_down0, dW_target, dconv_w

    def call(eta, ins, outs, w, nbytes, shape=s):
        return lib.ttt_layer_backward(ctypes.byref(shape), cw.TTT_BF16, eta, *ins, None, None, *outs, w, nbytes, None)

    assert call(0.1, ins, outs, _fake(), nb - 1) == cw.TTT_ERR_WORKSPACE
    assert call(0.1, ins, outs, None, nb) == cw.TTT_ERR_WORKSPACE
    assert call(float("inf"), ins, outs, _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins[:6] + [None] + ins[7:], outs, _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, outs[:6] + [ctypes.c_void_p(0x100004)], _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, outs, _fake(), 1 << 40, shape=odd) == cw.TTT_ERR_UNSUPPORTED


@pytest.mark.parametrize("mode", [0, 1])
def test_backward_resume_validation(mode):
    """Resumed rows in ttt_backward_options: each gradient goes with its input (W_init with dW_init; in the whole
    layer x0_halo with dx0_halo), both 16-byte aligned, checked before any device work."""
    lib = cw.lib()
    s = cw.InplaceShape(2, 1024, 256, 512, 256, 4)
    m = cw.TTT_MODE_MSE if mode else cw.TTT_MODE_DOT
    bad = ctypes.c_void_p(0x100004)

    def opts(Wi=None, halo=None, dWi=None, dhalo=None):
        return cw.BackwardOptions(None, None, None, 0, Wi, halo, dWi, dhalo)

    def core(o):
        return lib.ttt_core_backward_ex(ctypes.byref(s), cw.TTT_BF16, m, 0.1, *[_fake() for _ in range(4)],
                                        ctypes.byref(o), _fake(), _fake(), _fake(), _fake(), 1 << 40, None)

    def layer(o):
        return lib.ttt_layer_backward_ex(ctypes.byref(s), cw.TTT_BF16, m, 0.1, *[_fake() for _ in range(8)],
                                         ctypes.byref(o), *[_fake() for _ in range(7)], _fake(), 1 << 40, None)

    for call in (core, layer):
        assert call(opts(Wi=_fake())) == cw.TTT_ERR_ARG              # no dW_init
        assert call(opts(dWi=_fake())) == cw.TTT_ERR_ARG             # a gradient without its input
        assert call(opts(Wi=bad, dWi=_fake())) == cw.TTT_ERR_ARG
        assert call(opts(Wi=_fake(), dWi=bad)) == cw.TTT_ERR_ARG
    assert layer(opts(halo=_fake())) == cw.TTT_ERR_ARG
    assert layer(opts(dhalo=_fake())) == cw.TTT_ERR_ARG
    assert layer(opts(halo=_fake(), dhalo=bad)) == cw.TTT_ERR_ARG


def test_mse_backward_validation():
    """ttt_core_backward_mse: workspace sizes with and without kept states, and validation before device work."""
    lib = cw.lib()
    al = lambda x: (x + 255) // 256 * 256
    B, n, d, f, C = 2, 1024, 256, 512, 256
    k, e = n // C, 2
    s = cw.InplaceShape(B, n, d, f, C, 1)

    def ws(saved):
        out = ctypes.c_size_t(0)
        assert lib.ttt_core_backward_mse_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, saved,
                                                         ctypes.byref(out)) == cw.TTT_OK
        return out.value

    # V^ and dO token-contiguous, the state gradient (fp32 + bf16 copy), two chunk residual buffers; the recomputing
    # call adds the chunk-major states, the forward state and its bf16 copy
    # (packed rows add each document's gradient into dW_down0 directly: no per-row sums)
    common = 2 * al(B * n * d * e) + al(B * d * f * 4) + al(B * d * f * e) + 2 * al(B * d * C * e)
    assert ws(1) == common
    assert ws(0) == common + al(k * B * d * f * e) + al(B * d * f * 4) + al(B * d * f * e)
    ins = [_fake() for _ in range(4)]      # Z, Vhat, W_down0, dO
    outs = [_fake() for _ in range(2)]     # dZ, dVhat

    def call(eta, ins, Ws, dW, w, nbytes):
        return lib.ttt_core_backward_mse(ctypes.byref(s), cw.TTT_BF16, eta, *ins, Ws, None, *outs, dW, w, nbytes,
                                         None)

    nb = ws(0)
    assert call(0.1, ins, None, _fake(), _fake(), nb - 1) == cw.TTT_ERR_WORKSPACE
    assert call(0.1, ins, _fake(), _fake(), _fake(), ws(1) - 1) == cw.TTT_ERR_WORKSPACE
    assert call(float("nan"), ins, None, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, None, None, _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, [ctypes.c_void_p(0x100002)] + ins[1:], None, _fake(), _fake(), nb) == cw.TTT_ERR_ARG
    assert call(0.1, ins, ctypes.c_void_p(0x100004), _fake(), _fake(), nb) == cw.TTT_ERR_ARG


def test_forward_rejects_misaligned_kept_states():
    lib = cw.lib()
    s = cw.InplaceShape(1, 2048, 256, 512, 256, 4)
    out = ctypes.c_size_t(0)
    assert lib.ttt_inplace_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, cw.TTT_MODE_MSE, 0,
                                           ctypes.byref(out)) == cw.TTT_OK
    args = [_fake() for _ in range(3)]    # Z, Vhat, W_down0
    opts = cw.LayerOptions(None, 0, None, None, ctypes.c_void_p(0x100004))
    assert lib.ttt_core_apply_update_ex(ctypes.byref(s), cw.TTT_BF16, cw.TTT_MODE_DOT, 0.1, *args, ctypes.byref(opts),
                                        _fake(), _fake(), _fake(), 1 << 40, None) == cw.TTT_ERR_ARG


def test_update_first_validation():
    # the update-then-apply order: 0/1 only, and not with kept states
    lib = cw.lib()
    s = cw.InplaceShape(1, 2048, 256, 512, 256, 4)
    out = ctypes.c_size_t(0)
    assert lib.ttt_inplace_workspace_bytes(ctypes.byref(s), cw.TTT_BF16, cw.TTT_MODE_DOT_SCAN, 0,
                                           ctypes.byref(out)) == cw.TTT_OK
    args = [_fake() for _ in range(3)]    # Z, Vhat, W_down0

    def call(mode, opts):
        return lib.ttt_core_apply_update_ex(ctypes.byref(s), cw.TTT_BF16, mode, 0.1, *args, ctypes.byref(opts),
                                            _fake(), _fake(), _fake(), 1 << 40, None)

    assert call(cw.TTT_MODE_MSE, cw.LayerOptions(None, 0, None, None, None, None, 2)) == cw.TTT_ERR_ARG
    assert call(cw.TTT_MODE_DOT, cw.LayerOptions(None, 0, None, None, None, None, -1)) == cw.TTT_ERR_ARG
    for mode in (cw.TTT_MODE_DOT, cw.TTT_MODE_DOT_SCAN, cw.TTT_MODE_MSE):
        assert call(mode, cw.LayerOptions(None, 0, None, None, _fake(), None, 1)) == cw.TTT_ERR_UNSUPPORTED
    lw = [_fake() for _ in range(7)]      # H, X0, W_gate, W_up, W_down0, W_target, conv_w
    opts = cw.LayerOptions(None, 0, None, None, None, None, 3)
    assert lib.ttt_chunk_apply_update_ex(ctypes.byref(s), cw.TTT_BF16, cw.TTT_MODE_DOT, 0.1, *lw, ctypes.byref(opts),
                                         _fake(), _fake(), _fake(), 1 << 40, None) == cw.TTT_ERR_ARG


def test_lact_validation():
    lib = cw.lib()
    out = ctypes.c_size_t(0)
    good = cw.LactShape(1, 4, 8192, 512, 1024, 4096)
    assert lib.ttt_lact_workspace_bytes(ctypes.byref(good), cw.TTT_BF16, ctypes.byref(out)) == cw.TTT_OK
    bad = cw.LactShape(1, 4, 8000, 512, 1024, 4096)
    assert lib.ttt_lact_workspace_bytes(ctypes.byref(bad), cw.TTT_BF16, ctypes.byref(out)) == cw.TTT_ERR_SHAPE
    args = [_fake() for _ in range(10)]
    assert lib.ttt_lact_swiglu(ctypes.byref(good), cw.TTT_BF16, 7, 1.0, *args, _fake(), out.value, None) == \
        cw.TTT_ERR_ARG
    # a side stream needs both of its events
    for fork, join in ((None, _fake()), (_fake(), None), (None, None)):
        opts = cw.LactOptions(0, None, None, 0, 0, 0, _fake(), fork, join)
        assert lib.ttt_lact_swiglu_ex(ctypes.byref(good), cw.TTT_BF16, 1.0, *args[:6], ctypes.byref(opts),
                                      *args[6:], _fake(), out.value, None) == cw.TTT_ERR_ARG


def test_lact_backward_validation():
    lib = cw.lib()
    out = ctypes.c_size_t(0)
    good = cw.LactShape(1, 4, 8192, 512, 1024, 4096)
    assert lib.ttt_lact_backward_workspace_bytes(ctypes.byref(good), cw.TTT_BF16, ctypes.byref(out)) == cw.TTT_OK
    fwd = ctypes.c_size_t(0)
    assert lib.ttt_lact_workspace_bytes(ctypes.byref(good), cw.TTT_BF16, ctypes.byref(fwd)) == cw.TTT_OK
    # the forward's workspace, three kept states of 3 m dh per row, and the gradients and intermediates beside
    assert out.value > fwd.value + 3 * 4 * 3 * 512 * 1024 * 2
    bad = cw.LactShape(1, 4, 8000, 512, 1024, 4096)
    assert lib.ttt_lact_backward_workspace_bytes(ctypes.byref(bad), cw.TTT_BF16, ctypes.byref(out)) == \
        cw.TTT_ERR_SHAPE
    args = [_fake() for _ in range(13)]
    nb = ctypes.c_size_t(0)
    lib.ttt_lact_backward_workspace_bytes(ctypes.byref(good), cw.TTT_BF16, ctypes.byref(nb))
    call = lambda order, eta, a, ws, nbytes: lib.ttt_lact_swiglu_backward(ctypes.byref(good), cw.TTT_BF16, order, eta,
                                                                          *a, ws, nbytes, None)
    assert call(5, 1.0, args, _fake(), nb.value) == cw.TTT_ERR_ARG                 # unknown order
    assert call(0, float("inf"), args, _fake(), nb.value) == cw.TTT_ERR_ARG        # non-finite eta
    assert call(0, 1.0, [None] + args[1:], _fake(), nb.value) == cw.TTT_ERR_ARG   # null q
    assert call(0, 1.0, args, _fake(), nb.value - 1) == cw.TTT_ERR_WORKSPACE
    assert call(0, 1.0, args, None, nb.value) == cw.TTT_ERR_WORKSPACE
    # the options form: NULL options, invalid flags, and the update variants that have no backward
    ex = lambda o: lib.ttt_lact_swiglu_backward_ex(ctypes.byref(good), cw.TTT_BF16, 1.0, *args[:7],
                                                   None if o is None else ctypes.byref(o), *args[7:], _fake(),
                                                   nb.value, None)
    assert ex(None) == cw.TTT_ERR_ARG
    assert ex(cw.LactOptions(0, None, None, 2, 0, 0, None, None, None)) == cw.TTT_ERR_ARG
    assert ex(cw.LactOptions(0, None, None, 1, 0, 0, None, None, None)) == cw.TTT_ERR_UNSUPPORTED   # dot loss
    assert ex(cw.LactOptions(0, None, _fake(), 0, 0, 0, None, None, None)) == cw.TTT_ERR_UNSUPPORTED
    assert ex(cw.LactOptions(0, None, None, 0, 1, 0, None, None, None)) == cw.TTT_ERR_UNSUPPORTED
    assert ex(cw.LactOptions(0, None, None, 0, 0, 1, None, None, None)) == cw.TTT_ERR_UNSUPPORTED
    assert ex(cw.LactOptions(7, None, None, 0, 0, 0, None, None, None)) == cw.TTT_ERR_ARG           # order
    assert ex(cw.LactOptions(0, None, None, 0, 0, 0, None, None, None, ctypes.c_void_p(0x100004))) == cw.TTT_ERR_ARG
    # kept states: the forward's workspace and the state slots drop out of the backward's
    kept = ctypes.c_size_t(0)
    assert lib.ttt_lact_backward_workspace_bytes_ex(ctypes.byref(good), cw.TTT_BF16, 1,
                                                    ctypes.byref(kept)) == cw.TTT_OK
    k, BH, md = 8192 // 4096, 4, 512 * 1024
    assert kept.value <= nb.value - fwd.value - (k + 1) * BH * 3 * md * 2
    assert lib.ttt_lact_backward_workspace_bytes_ex(ctypes.byref(good), cw.TTT_BF16, 0,
                                                    ctypes.byref(kept)) == cw.TTT_OK and kept.value == nb.value
    assert lib.ttt_lact_backward_workspace_bytes_ex(ctypes.byref(good), cw.TTT_BF16, 2,
                                                    ctypes.byref(kept)) == cw.TTT_ERR_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    H = torch.zeros(1, 16, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        cw.ttt_produce_z(H, torch.zeros(8, 8), torch.zeros(8, 8))
