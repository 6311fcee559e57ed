"""ctypes marshalling for libttt.so.  No arithmetic of the layer happens here:
the functions check that the tensors they are given match the shape they
declare (the C ABI sees only raw pointers), allocate outputs and workspace
with torch on the tensors' device, and pass pointers and the current stream."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libttt.so")

(TTT_OK, TTT_ERR_ARG, TTT_ERR_SHAPE, TTT_ERR_DTYPE, TTT_ERR_WORKSPACE, TTT_ERR_DEVICE, TTT_ERR_UNSUPPORTED,
 TTT_ERR_SCRATCH_LIMIT) = range(8)
TTT_NOALLOC_SCRATCH_BYTES = 64 << 20     # the static scratch of ttt_chunk_apply_update_noalloc
TTT_F32, TTT_BF16 = 0, 1
TTT_MODE_DOT, TTT_MODE_MSE, TTT_MODE_DOT_SCAN = 0, 1, 2
TTT_UPDATE_THEN_APPLY, TTT_APPLY_THEN_UPDATE = 0, 1

_MODES = {"dot": TTT_MODE_DOT, "mse": TTT_MODE_MSE, "dot_scan": TTT_MODE_DOT_SCAN}
_ORDERS = {"update_then_apply": TTT_UPDATE_THEN_APPLY, "apply_then_update": TTT_APPLY_THEN_UPDATE}
_DTYPES = {torch.float32: TTT_F32, torch.bfloat16: TTT_BF16}


class InplaceShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("batch", "seq_len", "d_model", "d_ff", "chunk", "conv_k")]


class LayerOptions(ctypes.Structure):
    _fields_ = [("doc_starts", ctypes.c_void_p), ("conv_forward", ctypes.c_int), ("W_init", ctypes.c_void_p),
                ("x0_halo", ctypes.c_void_p), ("W_states", ctypes.c_void_p), ("update_mask", ctypes.c_void_p),
                ("update_first", ctypes.c_int)]


class LactOptions(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int), ("update_mask", ctypes.c_void_p), ("eta_tok", ctypes.c_void_p),
                ("loss", ctypes.c_int), ("weight_norm", ctypes.c_int), ("muon", ctypes.c_int),
                ("side_stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p), ("join_event", ctypes.c_void_p),
                ("W_states", ctypes.c_void_p)]


class LactSideStream:
    """A side stream and the fork / join events that let ttt_lact_swiglu run its (batch, head) rows as two chains
    (the caller owns all three; the library creates none).  Create it outside graph capture and keep it alive while
    calls that use it may run; calls that may be enqueued concurrently need one each."""

    def __init__(self, device=None):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.device = dev
        self.stream = torch.cuda.Stream(device=dev)
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        # torch creates an event's handle at its first record
        self.fork.record(self.stream)
        self.join.record(self.stream)
        self.stream.synchronize()

    def handles(self):
        return (ctypes.c_void_p(self.stream.cuda_stream), ctypes.c_void_p(self.fork.cuda_event),
                ctypes.c_void_p(self.join.cuda_event))


class BackwardOptions(ctypes.Structure):
    _fields_ = [("W_states", ctypes.c_void_p), ("doc_starts", ctypes.c_void_p), ("update_mask", ctypes.c_void_p),
                ("conv_forward", ctypes.c_int), ("W_init", ctypes.c_void_p), ("x0_halo", ctypes.c_void_p),
                ("dW_init", ctypes.c_void_p), ("dx0_halo", ctypes.c_void_p)]


class LactShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("batch", "heads", "seq_len", "head_dim", "hidden", "chunk")]


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_SIGNATURES = {
    "ttt_status_string": (ctypes.c_char_p, [_I]),
    "ttt_inplace_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _I, ctypes.POINTER(_S)]),
    "ttt_chunk_apply_update": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _S, _P]),
    "ttt_chunk_apply_update_ex": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.POINTER(LayerOptions), _P, _P, _P, _S, _P]),
    "ttt_chunk_apply_update_noalloc": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F] + [_P] * 10),
    "ttt_core_apply_update": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F, _P, _P, _P, _P, _P, _P, _S, _P]),
    "ttt_core_apply_update_ex": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F, _P, _P, _P,
                                      ctypes.POINTER(LayerOptions), _P, _P, _P, _S, _P]),
    "ttt_core_backward_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, _I, ctypes.POINTER(_S)]),
    "ttt_core_backward_mse_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, _I, ctypes.POINTER(_S)]),
    "ttt_core_backward_mse": (_I, [ctypes.POINTER(InplaceShape), _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _S, _P]),
    "ttt_layer_backward_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, _I, ctypes.POINTER(_S)]),
    "ttt_layer_backward": (_I, [ctypes.POINTER(InplaceShape), _I, _F] + [_P] * 18 + [_S, _P]),
    "ttt_layer_backward_mse_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, _I, ctypes.POINTER(_S)]),
    "ttt_layer_backward_ex": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F] + [_P] * 8 +
                              [ctypes.POINTER(BackwardOptions)] + [_P] * 7 + [_P, _S, _P]),
    "ttt_core_backward_ex": (_I, [ctypes.POINTER(InplaceShape), _I, _I, _F, _P, _P, _P, _P,
                                  ctypes.POINTER(BackwardOptions), _P, _P, _P, _P, _S, _P]),
    "ttt_layer_backward_mse": (_I, [ctypes.POINTER(InplaceShape), _I, _F] + [_P] * 18 + [_S, _P]),
    "ttt_core_backward": (_I, [ctypes.POINTER(InplaceShape), _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                               _P]),
    "ttt_produce_z": (_I, [ctypes.POINTER(InplaceShape), _I, _P, _P, _P, _P, _P, _P]),
    "ttt_vhat_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, ctypes.POINTER(_S)]),
    "ttt_produce_vhat": (_I, [ctypes.POINTER(InplaceShape), _I, _F, _P, _P, _P, _P, _P, _S, _P]),
    "ttt_chunk_delta": (_I, [ctypes.POINTER(InplaceShape), _I, _P, _P, _P, _P]),
    "ttt_chunk_scan": (_I, [ctypes.POINTER(InplaceShape), _I, _F, _P, _P, _P, _P, _P]),
    "ttt_update_scan_workspace_bytes": (_I, [ctypes.POINTER(InplaceShape), _I, ctypes.POINTER(_S)]),
    "ttt_chunk_update_scan": (_I, [ctypes.POINTER(InplaceShape), _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "ttt_chunk_apply": (_I, [ctypes.POINTER(InplaceShape), _I, _P, _P, _P, _P]),
    "ttt_lact_workspace_bytes": (_I, [ctypes.POINTER(LactShape), _I, ctypes.POINTER(_S)]),
    "ttt_lact_swiglu": (_I, [ctypes.POINTER(LactShape), _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _S, _P]),
    "ttt_lact_swiglu_ex": (_I, [ctypes.POINTER(LactShape), _I, _F, _P, _P, _P, _P, _P, _P,
                                ctypes.POINTER(LactOptions), _P, _P, _P, _P, _P, _S, _P]),
    "ttt_lact_backward_workspace_bytes": (_I, [ctypes.POINTER(LactShape), _I, ctypes.POINTER(_S)]),
    "ttt_lact_backward_workspace_bytes_ex": (_I, [ctypes.POINTER(LactShape), _I, _I, ctypes.POINTER(_S)]),
    "ttt_lact_swiglu_backward": (_I, [ctypes.POINTER(LactShape), _I, _I, _F] + [_P] * 13 + [_P, _S, _P]),
    "ttt_lact_swiglu_backward_ex": (_I, [ctypes.POINTER(LactShape), _I, _F] + [_P] * 7 +
                                    [ctypes.POINTER(LactOptions)] + [_P] * 6 + [_P, _S, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libttt.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with `python -m chunk_wise_weight_amd.build`")
        handle = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def status_string(status: int) -> str:
    return lib().ttt_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != TTT_OK:
        raise TTTError(status, what)


def _dt(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"dtype must be float32 or bfloat16, got {dtype}")
    return _DTYPES[dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _vp(t):
    """A tensor's address, or None for a missing or empty tensor."""
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the layer runs only in the HIP library)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mode(mode) -> int:
    if isinstance(mode, str):
        return _MODES[mode]
    return int(mode)


def _inplace_shape(B, n, d, f, chunk, K) -> InplaceShape:
    return InplaceShape(int(B), int(n), int(d), int(f), int(chunk), int(K))


def _flags(t, name, shape, dev):
    """A per-chunk flag tensor (bool or uint8, device) as uint8, or None."""
    if t is None:
        return None
    if t.dtype == torch.bool:
        t = t.to(torch.uint8)
    _need(t, name, shape, torch.uint8, dev)
    return t


def ttt_inplace_workspace_bytes(shape: InplaceShape, dtype: torch.dtype, mode="dot", with_producers=True) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ttt_inplace_workspace_bytes(ctypes.byref(shape), _dt(dtype), _mode(mode), int(bool(with_producers)),
                                             ctypes.byref(out)), "ttt_inplace_workspace_bytes")
    return out.value


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.device.type != "cuda" or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def ttt_chunk_apply_update(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk: int, eta: float, mode="dot",
                           O=None, W_final=None, workspace=None, doc_starts=None, conv_forward=False, W_init=None,
                           x0_halo=None, W_states=None, update_mask=None, update_first=False):
    """The whole In-Place layer.  Returns (O [B, n, d], W_final [B, d, f] fp32).

    Options (ttt_chunk_apply_update_ex): doc_starts, a uint8 (or bool) device tensor [B, seq_len // chunk] whose
    nonzero entries mark the chunks that start a new document in their row; conv_forward, the forward-looking
    in-chunk convolution for the target; W_init [B, d, f] fp32 and x0_halo [B, K-1, d] to resume rows from an
    earlier call (its W_final and its last K-1 rows of X0); W_states [B, seq_len // chunk, d, f] (dtype) to keep
    the per-chunk states of the dot objective for ttt_core_backward; update_mask, a uint8 (or bool) device tensor
    [B, seq_len // chunk] whose zero entries mark chunks that are applied without updating the state;
    update_first, each chunk's step taken before its apply (every mode; not with W_states)."""
    B, n, d = H.shape
    f = W_gate.shape[0]
    K = conv_w.shape[1]
    dt, dev = H.dtype, H.device
    for name, t, shp in (("H", H, (B, n, d)), ("X0", X0, (B, n, d)), ("W_gate", W_gate, (f, d)),
                         ("W_up", W_up, (f, d)), ("W_down0", W_down0, (d, f)), ("W_target", W_target, (d, d)),
                         ("conv_w", conv_w, (d, K))):
        _need(t, name, shp, dt, dev)
    shape = _inplace_shape(B, n, d, f, chunk, K)
    O = torch.empty(B, n, d, dtype=dt, device=dev) if O is None else O
    W_final = torch.empty(B, d, f, dtype=torch.float32, device=dev) if W_final is None else W_final
    _need(O, "O", (B, n, d), dt, dev)
    _need(W_final, "W_final", (B, d, f), torch.float32, dev)
    nbytes = ttt_inplace_workspace_bytes(shape, dt, mode, True)
    ws = _workspace(nbytes, dev, workspace)
    if W_init is not None:
        _need(W_init, "W_init", (B, d, f), torch.float32, dev)
    if x0_halo is not None:
        _need(x0_halo, "x0_halo", (B, K - 1, d), dt, dev)
    if W_states is not None:
        _need(W_states, "W_states", (B, n // chunk, d, f), dt, dev)
    update_mask = _flags(update_mask, "update_mask", (B, n // chunk if chunk > 0 else 0), dev)
    if doc_starts is None and not conv_forward and W_init is None and x0_halo is None and W_states is None and \
            update_mask is None and not update_first:
        _check(lib().ttt_chunk_apply_update(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(H),
                                            _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(W_target),
                                            _ptr(conv_w), _ptr(O), _ptr(W_final), _ptr(ws), nbytes, _stream(dev)),
               "ttt_chunk_apply_update")
        return O, W_final
    if doc_starts is not None:
        if doc_starts.dtype == torch.bool:
            doc_starts = doc_starts.to(torch.uint8)
        _need(doc_starts, "doc_starts", (B, n // chunk if chunk > 0 else 0), torch.uint8, dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None
    opts = LayerOptions(ptr(doc_starts), 1 if conv_forward else 0, ptr(W_init), ptr(x0_halo), ptr(W_states),
                        ptr(update_mask), 1 if update_first else 0)
    _check(lib().ttt_chunk_apply_update_ex(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(H),
                                           _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(W_target),
                                           _ptr(conv_w), ctypes.byref(opts), _ptr(O), _ptr(W_final), _ptr(ws),
                                           nbytes, _stream(dev)),
           "ttt_chunk_apply_update_ex")
    return O, W_final


def ttt_chunk_apply_update_noalloc(H, X0, W_gate, W_up, W_down0, W_target, conv_w, chunk: int, eta: float, mode,
                                   O, W_final):
    """The whole In-Place layer into the caller's O [B, n, d] and W_final [B, d, f] (fp32), with its scratch taken
    from the library's static device buffer (TTT_NOALLOC_SCRATCH_BYTES): nothing is allocated here or in the
    library.  Raises TTTError with TTT_ERR_SCRATCH_LIMIT for shapes whose scratch does not fit.  Returns (O,
    W_final)."""
    B, n, d = H.shape
    f = W_gate.shape[0]
    K = conv_w.shape[1]
    dt, dev = H.dtype, H.device
    for name, t, shp in (("H", H, (B, n, d)), ("X0", X0, (B, n, d)), ("W_gate", W_gate, (f, d)),
                         ("W_up", W_up, (f, d)), ("W_down0", W_down0, (d, f)), ("W_target", W_target, (d, d)),
                         ("conv_w", conv_w, (d, K)), ("O", O, (B, n, d))):
        _need(t, name, shp, dt, dev)
    _need(W_final, "W_final", (B, d, f), torch.float32, dev)
    shape = _inplace_shape(B, n, d, f, chunk, K)
    _check(lib().ttt_chunk_apply_update_noalloc(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(H),
                                                _ptr(X0), _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(W_target),
                                                _ptr(conv_w), _ptr(O), _ptr(W_final), _stream(dev)),
           "ttt_chunk_apply_update_noalloc")
    return O, W_final


def ttt_core_apply_update(Z, Vhat, W_down0, chunk: int, eta: float, mode="dot", O=None, W_final=None,
                          workspace=None, W_states=None, update_mask=None, doc_starts=None, W_init=None,
                          update_first=False):
    """The chunk loop given Z [B, n, f] and Vhat [B, n, d].  Returns (O, W_final).  W_states [B, n // chunk, d, f]
    (dtype), if given, receives the per-chunk states; update_mask and doc_starts [B, n // chunk], W_init
    [B, d, f] fp32 and update_first as for the layer (all through ttt_core_apply_update_ex)."""
    B, n, f = Z.shape
    d = Vhat.shape[2]
    dt, dev = Z.dtype, Z.device
    _need(Z, "Z", (B, n, f), dt, dev)
    _need(Vhat, "Vhat", (B, n, d), dt, dev)
    _need(W_down0, "W_down0", (d, f), dt, dev)
    shape = _inplace_shape(B, n, d, f, chunk, 1)
    O = torch.empty(B, n, d, dtype=dt, device=dev) if O is None else O
    W_final = torch.empty(B, d, f, dtype=torch.float32, device=dev) if W_final is None else W_final
    _need(O, "O", (B, n, d), dt, dev)
    _need(W_final, "W_final", (B, d, f), torch.float32, dev)
    nbytes = ttt_inplace_workspace_bytes(shape, dt, mode, False)
    ws = _workspace(nbytes, dev, workspace)
    update_mask = _flags(update_mask, "update_mask", (B, n // chunk if chunk > 0 else 0), dev)
    doc_starts = _flags(doc_starts, "doc_starts", (B, n // chunk if chunk > 0 else 0), dev)
    if W_states is not None or update_mask is not None or doc_starts is not None or W_init is not None or \
            update_first:
        if W_states is not None:
            _need(W_states, "W_states", (B, n // chunk, d, f), dt, dev)
        if W_init is not None:
            _need(W_init, "W_init", (B, d, f), torch.float32, dev)
        opts = LayerOptions(_vp(doc_starts), 0, _vp(W_init), None, _vp(W_states), _vp(update_mask),
                            1 if update_first else 0)
        _check(lib().ttt_core_apply_update_ex(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(Z),
                                              _ptr(Vhat), _ptr(W_down0), ctypes.byref(opts), _ptr(O), _ptr(W_final),
                                              _ptr(ws), nbytes, _stream(dev)),
               "ttt_core_apply_update_ex")
        return O, W_final
    _check(lib().ttt_core_apply_update(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(Z), _ptr(Vhat),
                                       _ptr(W_down0), _ptr(O), _ptr(W_final), _ptr(ws), nbytes, _stream(dev)),
           "ttt_core_apply_update")
    return O, W_final


def ttt_core_backward_workspace_bytes(shape: InplaceShape, dtype: torch.dtype, saved_states=False) -> int:
    n = ctypes.c_size_t()
    _check(lib().ttt_core_backward_workspace_bytes(ctypes.byref(shape), _dt(dtype), int(bool(saved_states)),
                                                   ctypes.byref(n)),
           "ttt_core_backward_workspace_bytes")
    return n.value


def _core_backward(mode, Z, Vhat, W_down0, dO, chunk, eta, dZ, dVhat, dW_down0, workspace, W_states, doc_starts,
                   update_mask, W_init):
    B, n, f = Z.shape
    d = Vhat.shape[2]
    dt, dev = Z.dtype, Z.device
    _need(Z, "Z", (B, n, f), dt, dev)
    _need(Vhat, "Vhat", (B, n, d), dt, dev)
    _need(W_down0, "W_down0", (d, f), dt, dev)
    _need(dO, "dO", (B, n, d), dt, dev)
    shape = _inplace_shape(B, n, d, f, chunk, 1)
    dZ = torch.empty(B, n, f, dtype=dt, device=dev) if dZ is None else dZ
    dVhat = torch.empty(B, n, d, dtype=dt, device=dev) if dVhat is None else dVhat
    dW_down0 = torch.empty(d, f, dtype=torch.float32, device=dev) if dW_down0 is None else dW_down0
    _need(dZ, "dZ", (B, n, f), dt, dev)
    _need(dVhat, "dVhat", (B, n, d), dt, dev)
    _need(dW_down0, "dW_down0", (d, f), torch.float32, dev)
    k = n // chunk if chunk > 0 else 0
    if W_states is not None:
        _need(W_states, "W_states", (B, k, d, f), dt, dev)
    dW_init = None
    if W_init is not None:
        _need(W_init, "W_init", (B, d, f), torch.float32, dev)
        dW_init = torch.empty(B, d, f, dtype=torch.float32, device=dev)
    nbytes = (ttt_core_backward_mse_workspace_bytes if mode == "mse" else ttt_core_backward_workspace_bytes)(
        shape, dt, W_states is not None)
    ws = _workspace(nbytes, dev, workspace)
    sp = _vp(W_states)
    doc_starts = _flags(doc_starts, "doc_starts", (B, k), dev)
    dp = _vp(doc_starts)
    if update_mask is not None or W_init is not None:
        um = _flags(update_mask, "update_mask", (B, k), dev)
        opts = BackwardOptions(sp, dp, _vp(um), 0, _vp(W_init), None, _vp(dW_init), None)
        _check(lib().ttt_core_backward_ex(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(Z), _ptr(Vhat),
                                          _ptr(W_down0), _ptr(dO), ctypes.byref(opts), _ptr(dZ), _ptr(dVhat),
                                          _ptr(dW_down0), _ptr(ws), nbytes, _stream(dev)), "ttt_core_backward_ex")
    else:
        name = "ttt_core_backward_mse" if mode == "mse" else "ttt_core_backward"
        _check(getattr(lib(), name)(ctypes.byref(shape), _dt(dt), float(eta), _ptr(Z), _ptr(Vhat), _ptr(W_down0),
                                    _ptr(dO), sp, dp, _ptr(dZ), _ptr(dVhat), _ptr(dW_down0), _ptr(ws), nbytes,
                                    _stream(dev)), name)
    return (dZ, dVhat, dW_down0) if W_init is None else (dZ, dVhat, dW_down0, dW_init)


def ttt_core_backward(Z, Vhat, W_down0, dO, chunk: int, eta: float, dZ=None, dVhat=None, dW_down0=None,
                      workspace=None, W_states=None, doc_starts=None, update_mask=None, W_init=None):
    """Gradients through the dot chunk loop given dO = dLoss/dO [B, n, d], with the per-chunk states W_states
    [B, n // chunk, d, f] kept by the forward call, or recomputed (None); doc_starts [B, n // chunk] packs documents,
    update_mask [B, n // chunk] masks updates and W_init [B, d, f] fp32 resumes rows as for the forward layer (the
    last two through ttt_core_backward_ex).  Returns (dZ [B, n, f], dVhat [B, n, d], dW_down0 [d, f] fp32), and
    dW_init [B, d, f] fp32 after them when W_init is given."""
    return _core_backward("dot", Z, Vhat, W_down0, dO, chunk, eta, dZ, dVhat, dW_down0, workspace, W_states,
                          doc_starts, update_mask, W_init)


def ttt_core_backward_mse_workspace_bytes(shape: InplaceShape, dtype: torch.dtype, saved_states=False) -> int:
    n = ctypes.c_size_t()
    _check(lib().ttt_core_backward_mse_workspace_bytes(ctypes.byref(shape), _dt(dtype), int(bool(saved_states)),
                                                       ctypes.byref(n)),
           "ttt_core_backward_mse_workspace_bytes")
    return n.value


def ttt_core_backward_mse(Z, Vhat, W_down0, dO, chunk: int, eta: float, dZ=None, dVhat=None, dW_down0=None,
                          workspace=None, W_states=None, doc_starts=None, update_mask=None, W_init=None):
    """ttt_core_backward for the MSE chunk loop (same arguments and results)."""
    return _core_backward("mse", Z, Vhat, W_down0, dO, chunk, eta, dZ, dVhat, dW_down0, workspace, W_states,
                          doc_starts, update_mask, W_init)


def ttt_layer_backward_workspace_bytes(shape: InplaceShape, dtype: torch.dtype, saved_states=False,
                                       mode="dot") -> int:
    n = ctypes.c_size_t()
    name = "ttt_layer_backward_mse_workspace_bytes" if mode == "mse" else "ttt_layer_backward_workspace_bytes"
    _check(getattr(lib(), name)(ctypes.byref(shape), _dt(dtype), int(bool(saved_states)), ctypes.byref(n)), name)
    return n.value


def ttt_layer_backward_mse_workspace_bytes(shape: InplaceShape, dtype: torch.dtype, saved_states=False) -> int:
    return ttt_layer_backward_workspace_bytes(shape, dtype, saved_states, "mse")


def ttt_layer_backward_mse(H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, chunk: int, eta: float,
                           W_states=None, grads=None, workspace=None, doc_starts=None, update_mask=None,
                           conv_forward=False):
    """ttt_layer_backward for the MSE objective (see there)."""
    return ttt_layer_backward(H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, chunk, eta, W_states, grads,
                              workspace, doc_starts, mode="mse", update_mask=update_mask, conv_forward=conv_forward)


def ttt_layer_backward(H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, chunk: int, eta: float, W_states=None,
                       grads=None, workspace=None, doc_starts=None, mode="dot", update_mask=None, conv_forward=False,
                       W_init=None, x0_halo=None):
    """Gradients of the layer (objective `mode`, "dot" or "mse") with respect to every input, given
    dO = dLoss/dO [B, n, d], with the per-chunk states W_states kept by the forward call or recomputed (None), and
    doc_starts [B, n // chunk], update_mask [B, n // chunk], conv_forward and the resumed rows' W_init [B, d, f]
    fp32 and x0_halo [B, K-1, d] as the forward layer took them (all but the first through ttt_layer_backward_ex).
    Returns (dH, dX0, dW_gate, dW_up, dW_down0, dW_target, dconv_w): activations in the inputs' dtype, weight
    gradients fp32 summed over the batch rows; with W_init or x0_halo given, dW_init [B, d, f] fp32 and dx0_halo
    [B, K-1, d] follow (None for the one not given)."""
    if mode not in ("dot", "mse"):
        raise ValueError(f"mode must be 'dot' or 'mse', got {mode!r}")
    B, n, d = H.shape
    f = W_gate.shape[0]
    K = conv_w.shape[1]
    dt, dev = H.dtype, H.device
    for name, t, shp in (("H", H, (B, n, d)), ("X0", X0, (B, n, d)), ("W_gate", W_gate, (f, d)),
                         ("W_up", W_up, (f, d)), ("W_down0", W_down0, (d, f)), ("W_target", W_target, (d, d)),
                         ("conv_w", conv_w, (d, K)), ("dO", dO, (B, n, d))):
        _need(t, name, shp, dt, dev)
    shapes = (((B, n, d), dt), ((B, n, d), dt), ((f, d), torch.float32), ((f, d), torch.float32),
              ((d, f), torch.float32), ((d, d), torch.float32), ((d, K), torch.float32))
    if grads is None:
        grads = tuple(torch.empty(*shp, dtype=t, device=dev) for shp, t in shapes)
    for g, (shp, t) in zip(grads, shapes):
        _need(g, "gradient", shp, t, dev)
    if W_states is not None:
        _need(W_states, "W_states", (B, n // chunk, d, f), dt, dev)
    resumed = W_init is not None or x0_halo is not None
    dW_init = dx0_halo = None
    if W_init is not None:
        _need(W_init, "W_init", (B, d, f), torch.float32, dev)
        dW_init = torch.empty(B, d, f, dtype=torch.float32, device=dev)
    if x0_halo is not None:
        _need(x0_halo, "x0_halo", (B, K - 1, d), dt, dev)
        dx0_halo = torch.empty(B, K - 1, d, dtype=dt, device=dev)
    shape = _inplace_shape(B, n, d, f, chunk, K)
    nbytes = ttt_layer_backward_workspace_bytes(shape, dt, W_states is not None, mode)
    ws = _workspace(nbytes, dev, workspace)
    sp = _vp(W_states)
    doc_starts = _flags(doc_starts, "doc_starts", (B, n // chunk if chunk > 0 else 0), dev)
    dp = _vp(doc_starts)
    if update_mask is not None or conv_forward or resumed:
        um = _flags(update_mask, "update_mask", (B, n // chunk if chunk > 0 else 0), dev)
        halo_ok = x0_halo is not None and K > 1
        opts = BackwardOptions(sp, dp, _vp(um), 1 if conv_forward else 0, _vp(W_init),
                               _vp(x0_halo) if halo_ok else None, _vp(dW_init), _vp(dx0_halo) if halo_ok else None)
        _check(lib().ttt_layer_backward_ex(ctypes.byref(shape), _dt(dt), _mode(mode), float(eta), _ptr(H), _ptr(X0),
                                           _ptr(W_gate), _ptr(W_up), _ptr(W_down0), _ptr(W_target), _ptr(conv_w),
                                           _ptr(dO), ctypes.byref(opts), *[_ptr(g) for g in grads], _ptr(ws),
                                           nbytes, _stream(dev)), "ttt_layer_backward_ex")
        return tuple(grads) + (dW_init, dx0_halo) if resumed else grads
    name = "ttt_layer_backward_mse" if mode == "mse" else "ttt_layer_backward"
    _check(getattr(lib(), name)(ctypes.byref(shape), _dt(dt), float(eta), _ptr(H), _ptr(X0), _ptr(W_gate),
                                _ptr(W_up), _ptr(W_down0), _ptr(W_target), _ptr(conv_w), _ptr(dO), sp, dp,
                                *[_ptr(g) for g in grads], _ptr(ws), nbytes, _stream(dev)), name)
    return grads


def ttt_produce_z(H, W_gate, W_up, Z=None, Zt=None, with_z=True):
    """Z = silu(H W_gate^T) * (H W_up^T).  Returns (Z [B, n, f] or None, Zt [B, f, n])."""
    B, n, d = H.shape
    f = W_gate.shape[0]
    dt, dev = H.dtype, H.device
    _need(H, "H", (B, n, d), dt, dev)
    _need(W_gate, "W_gate", (f, d), dt, dev)
    _need(W_up, "W_up", (f, d), dt, dev)
    if with_z:
        Z = torch.empty(B, n, f, dtype=dt, device=dev) if Z is None else Z
        _need(Z, "Z", (B, n, f), dt, dev)
    Zt = torch.empty(B, f, n, dtype=dt, device=dev) if Zt is None else Zt
    _need(Zt, "Zt", (B, f, n), dt, dev)
    shape = _inplace_shape(B, n, d, f, max(n, 8), 1)
    _check(lib().ttt_produce_z(ctypes.byref(shape), _dt(dt), _ptr(H), _ptr(W_gate), _ptr(W_up),
                               _ptr(Z) if with_z else None, _ptr(Zt), _stream(dev)), "ttt_produce_z")
    return (Z if with_z else None), Zt


def ttt_vhat_workspace_bytes(shape: InplaceShape, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ttt_vhat_workspace_bytes(ctypes.byref(shape), _dt(dtype), ctypes.byref(out)),
           "ttt_vhat_workspace_bytes")
    return out.value


def ttt_produce_vhat(X0, conv_w, W_target, Vt=None, workspace=None, scale: float = 1.0):
    """Vt [B, d, n] = scale * (CausalDepthwiseConv1D(X0) W_target)^T."""
    B, n, d = X0.shape
    K = conv_w.shape[1]
    dt, dev = X0.dtype, X0.device
    _need(X0, "X0", (B, n, d), dt, dev)
    _need(conv_w, "conv_w", (d, K), dt, dev)
    _need(W_target, "W_target", (d, d), dt, dev)
    Vt = torch.empty(B, d, n, dtype=dt, device=dev) if Vt is None else Vt
    _need(Vt, "Vt", (B, d, n), dt, dev)
    shape = _inplace_shape(B, n, d, 8, max(n, 8), K)
    nbytes = ttt_vhat_workspace_bytes(shape, dt)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().ttt_produce_vhat(ctypes.byref(shape), _dt(dt), float(scale), _ptr(X0), _ptr(conv_w), _ptr(W_target),
                                  _ptr(Vt), _ptr(ws), nbytes, _stream(dev)), "ttt_produce_vhat")
    return Vt


def ttt_chunk_delta(Zt, Vt, chunk: int, dW=None):
    """dW [B, k, d, f] fp32, dW[b, c] = Vhat_c^T Z_c, from Zt [B, f, n] and Vt [B, d, n]."""
    B, f, n = Zt.shape
    d = Vt.shape[1]
    dt, dev = Zt.dtype, Zt.device
    _need(Zt, "Zt", (B, f, n), dt, dev)
    _need(Vt, "Vt", (B, d, n), dt, dev)
    k = n // chunk if chunk > 0 else 0
    dW = torch.empty(B, k, d, f, dtype=torch.float32, device=dev) if dW is None else dW
    _need(dW, "dW", (B, k, d, f), torch.float32, dev)
    shape = _inplace_shape(B, n, d, f, chunk, 1)
    _check(lib().ttt_chunk_delta(ctypes.byref(shape), _dt(dt), _ptr(Zt), _ptr(Vt), _ptr(dW), _stream(dev)),
           "ttt_chunk_delta")
    return dW


def ttt_chunk_scan(dW, W_down0, eta: float, chunk: int, seq_len: int, Wc=None, W_final=None):
    """Exclusive prefix over chunks.  Returns (Wc [B, k, d, f] dtype, W_final [B, d, f] fp32)."""
    B, k, d, f = dW.shape
    dt, dev = W_down0.dtype, W_down0.device
    _need(dW, "dW", (B, k, d, f), torch.float32, dev)
    _need(W_down0, "W_down0", (d, f), dt, dev)
    Wc = torch.empty(B, k, d, f, dtype=dt, device=dev) if Wc is None else Wc
    W_final = torch.empty(B, d, f, dtype=torch.float32, device=dev) if W_final is None else W_final
    _need(Wc, "Wc", (B, k, d, f), dt, dev)
    _need(W_final, "W_final", (B, d, f), torch.float32, dev)
    if seq_len != k * chunk:
        raise ValueError("seq_len must equal k * chunk")
    shape = _inplace_shape(B, seq_len, d, f, chunk, 1)
    _check(lib().ttt_chunk_scan(ctypes.byref(shape), _dt(dt), float(eta), _ptr(W_down0), _ptr(dW), _ptr(Wc),
                                _ptr(W_final), _stream(dev)), "ttt_chunk_scan")
    return Wc, W_final


def ttt_update_scan_workspace_bytes(shape: InplaceShape, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ttt_update_scan_workspace_bytes(ctypes.byref(shape), _dt(dtype), ctypes.byref(out)),
           "ttt_update_scan_workspace_bytes")
    return out.value


def ttt_chunk_update_scan(Zt, Vt, W_down0, chunk: int, Wc=None, W_final=None, workspace=None):
    """Fused deltas + prefix from Zt [B, f, n] and the eta-scaled target Vt [B, d, n] (ttt_produce_vhat with
    scale = eta).  Returns (Wc [B, k, d, f] dtype, W_final fp32)."""
    B, f, n = Zt.shape
    d = Vt.shape[1]
    dt, dev = Zt.dtype, Zt.device
    _need(Zt, "Zt", (B, f, n), dt, dev)
    _need(Vt, "Vt", (B, d, n), dt, dev)
    _need(W_down0, "W_down0", (d, f), dt, dev)
    k = n // chunk if chunk > 0 else 0
    Wc = torch.empty(B, k, d, f, dtype=dt, device=dev) if Wc is None else Wc
    W_final = torch.empty(B, d, f, dtype=torch.float32, device=dev) if W_final is None else W_final
    _need(Wc, "Wc", (B, k, d, f), dt, dev)
    _need(W_final, "W_final", (B, d, f), torch.float32, dev)
    shape = _inplace_shape(B, n, d, f, chunk, 1)
    need = ttt_update_scan_workspace_bytes(shape, dt) if B * n > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ttt_chunk_update_scan(ctypes.byref(shape), _dt(dt), _ptr(W_down0), _ptr(Zt), _ptr(Vt), _ptr(Wc),
                                       _ptr(W_final), _ptr(workspace), wsb, _stream(dev)), "ttt_chunk_update_scan")
    return Wc, W_final


def ttt_chunk_apply(Zt, Wc, chunk: int, O=None):
    """O [B, n, d], O_c = Z_c Wc[b, c]^T, with Z given as its token-contiguous copy Zt [B, f, n]."""
    B, f, n = Zt.shape
    k, d = Wc.shape[1], Wc.shape[2]
    dt, dev = Zt.dtype, Zt.device
    _need(Zt, "Zt", (B, f, n), dt, dev)
    _need(Wc, "Wc", (B, k, d, f), dt, dev)
    if k * chunk != n:
        raise ValueError("Wc must hold one state per chunk")
    O = torch.empty(B, n, d, dtype=dt, device=dev) if O is None else O
    _need(O, "O", (B, n, d), dt, dev)
    shape = _inplace_shape(B, n, d, f, chunk, 1)
    _check(lib().ttt_chunk_apply(ctypes.byref(shape), _dt(dt), _ptr(Zt), _ptr(Wc), _ptr(O), _stream(dev)),
           "ttt_chunk_apply")
    return O


def ttt_lact_workspace_bytes(shape: LactShape, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ttt_lact_workspace_bytes(ctypes.byref(shape), _dt(dtype), ctypes.byref(out)),
           "ttt_lact_workspace_bytes")
    return out.value


def _host_flags(update_mask, n, chunk):
    """A per-chunk host flag sequence as a ctypes uint8 array (kept alive by the caller), or None."""
    if update_mask is None:
        return None
    flags = [1 if bool(x) else 0 for x in (update_mask.tolist() if hasattr(update_mask, "tolist") else update_mask)]
    if chunk <= 0 or len(flags) != n // chunk:
        raise ValueError(f"update_mask needs {n // chunk if chunk > 0 else 0} entries, got {len(flags)}")
    return (ctypes.c_ubyte * max(1, len(flags)))(*flags)


def ttt_lact_swiglu(q, k, v, W1, W3, W2, chunk: int, eta: float, order="update_then_apply", O=None, finals=None,
                    workspace=None, update_mask=None, eta_tok=None, loss="mse", weight_norm=False, muon=False,
                    side=None, W_states=None):
    """LaCT SwiGLU layer.  Returns (O [B, H, n, dh], W1_f, W3_f [B, H, m, dh], W2_f [B, H, dh, m]).

    Options (ttt_lact_swiglu_ex): update_mask, a host sequence of n // chunk flags (only the flagged chunks
    take the update step, every chunk is applied); eta_tok, per-token learning rates [B, H, n] fp32 on the
    device; loss, "mse" or "dot"; weight_norm, L2-normalise the weight rows after every update; muon, step
    along Muon(g) (Newton-Schulz orthogonalised gradients); side, a LactSideStream on the tensors' device to run
    half of the (batch, head) rows on (None: one chain on the current stream); W_states, a [n // chunk + 1, B, H, 3,
    m * dh] tensor of the layer's dtype that receives every chunk's state for ttt_lact_swiglu_backward."""
    B, Hh, n, dh = q.shape
    m = W1.shape[1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, Hh, n, dh)), ("k", k, (B, Hh, n, dh)), ("v", v, (B, Hh, n, dh)),
                         ("W1", W1, (Hh, m, dh)), ("W3", W3, (Hh, m, dh)), ("W2", W2, (Hh, dh, m))):
        _need(t, name, shp, dt, dev)
    O = torch.empty(B, Hh, n, dh, dtype=dt, device=dev) if O is None else O
    _need(O, "O", (B, Hh, n, dh), dt, dev)
    if finals is None:
        finals = (torch.empty(B, Hh, m, dh, dtype=torch.float32, device=dev),
                  torch.empty(B, Hh, m, dh, dtype=torch.float32, device=dev),
                  torch.empty(B, Hh, dh, m, dtype=torch.float32, device=dev))
    W1f, W3f, W2f = finals
    _need(W1f, "W1_f", (B, Hh, m, dh), torch.float32, dev)
    _need(W3f, "W3_f", (B, Hh, m, dh), torch.float32, dev)
    _need(W2f, "W2_f", (B, Hh, dh, m), torch.float32, dev)
    shape = LactShape(B, Hh, n, dh, m, int(chunk))
    nbytes = ttt_lact_workspace_bytes(shape, dt)
    ws = _workspace(nbytes, dev, workspace)
    ordc = _ORDERS[order] if isinstance(order, str) else int(order)
    if side is not None and side.device != dev:
        raise ValueError(f"the side stream is on {side.device}, the tensors on {dev}")
    if W_states is not None:
        _need(W_states, "W_states", (n // chunk + 1, B, Hh, 3, m * dh), dt, dev)
    if (update_mask is None and eta_tok is None and loss == "mse" and not weight_norm and not muon and side is None
            and W_states is None):
        _check(lib().ttt_lact_swiglu(ctypes.byref(shape), _dt(dt), ordc, float(eta), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(W1), _ptr(W3), _ptr(W2), _ptr(O), _ptr(W1f), _ptr(W3f), _ptr(W2f),
                                     _ptr(ws), nbytes, _stream(dev)), "ttt_lact_swiglu")
        return O, W1f, W3f, W2f
    mask = _host_flags(update_mask, n, chunk)
    if eta_tok is not None:
        _need(eta_tok, "eta_tok", (B, Hh, n), torch.float32, dev)
    if loss not in ("mse", "dot"):
        raise ValueError(f"loss must be 'mse' or 'dot', got {loss!r}")
    opts = LactOptions(ordc, ctypes.cast(mask, ctypes.c_void_p) if mask is not None else None,
                       ctypes.c_void_p(eta_tok.data_ptr()) if eta_tok is not None and eta_tok.numel() else None,
                       1 if loss == "dot" else 0, 1 if weight_norm else 0, 1 if muon else 0,
                       *(side.handles() if side is not None else (None, None, None)), _vp(W_states))
    _check(lib().ttt_lact_swiglu_ex(ctypes.byref(shape), _dt(dt), float(eta), _ptr(q), _ptr(k), _ptr(v), _ptr(W1),
                                    _ptr(W3), _ptr(W2), ctypes.byref(opts), _ptr(O), _ptr(W1f), _ptr(W3f),
                                    _ptr(W2f), _ptr(ws), nbytes, _stream(dev)),
           "ttt_lact_swiglu_ex")
    return O, W1f, W3f, W2f


def ttt_lact_backward_workspace_bytes(shape: LactShape, dtype: torch.dtype, saved_states=False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().ttt_lact_backward_workspace_bytes_ex(ctypes.byref(shape), _dt(dtype), int(bool(saved_states)),
                                                      ctypes.byref(out)), "ttt_lact_backward_workspace_bytes_ex")
    return out.value


def ttt_lact_swiglu_backward(q, k, v, W1, W3, W2, dO, chunk: int, eta: float, order="update_then_apply",
                             grads=None, workspace=None, update_mask=None, W_states=None):
    """Backward of the LaCT layer (squared error, plain GD) given dO = dLoss/dO [B, H, n, dh]; update_mask, a host
    sequence of n // chunk flags as the forward layer took it, and W_states, the states the forward call kept
    (both through ttt_lact_swiglu_backward_ex).  Returns (dq, dk, dv [B, H, n, dh] in the inputs' dtype, dW1, dW3
    [H, m, dh], dW2 [H, dh, m] fp32, summed over the batch rows)."""
    B, Hh, n, dh = q.shape
    m = W1.shape[1]
    dt, dev = q.dtype, q.device
    for name, t, shp in (("q", q, (B, Hh, n, dh)), ("k", k, (B, Hh, n, dh)), ("v", v, (B, Hh, n, dh)),
                         ("W1", W1, (Hh, m, dh)), ("W3", W3, (Hh, m, dh)), ("W2", W2, (Hh, dh, m)),
                         ("dO", dO, (B, Hh, n, dh))):
        _need(t, name, shp, dt, dev)
    shapes = (((B, Hh, n, dh), dt),) * 3 + (((Hh, m, dh), torch.float32), ((Hh, m, dh), torch.float32),
                                            ((Hh, dh, m), torch.float32))
    if grads is None:
        grads = tuple(torch.empty(*shp, dtype=t, device=dev) for shp, t in shapes)
    for gt, (shp, t) in zip(grads, shapes):
        _need(gt, "gradient", shp, t, dev)
    shape = LactShape(B, Hh, n, dh, m, int(chunk))
    if W_states is not None:
        _need(W_states, "W_states", (n // chunk + 1, B, Hh, 3, m * dh), dt, dev)
    nbytes = ttt_lact_backward_workspace_bytes(shape, dt, W_states is not None)
    ws = _workspace(nbytes, dev, workspace)
    ordc = _ORDERS[order] if isinstance(order, str) else int(order)
    if update_mask is not None or W_states is not None:
        mask = _host_flags(update_mask, n, chunk)
        opts = LactOptions(ordc, ctypes.cast(mask, ctypes.c_void_p) if mask is not None else None, None, 0, 0, 0,
                           None, None, None, _vp(W_states))
        _check(lib().ttt_lact_swiglu_backward_ex(ctypes.byref(shape), _dt(dt), float(eta), _ptr(q), _ptr(k),
                                                 _ptr(v), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(dO), ctypes.byref(opts),
                                                 *[_ptr(g) for g in grads], _ptr(ws), nbytes, _stream(dev)),
               "ttt_lact_swiglu_backward_ex")
        return grads
    _check(lib().ttt_lact_swiglu_backward(ctypes.byref(shape), _dt(dt), ordc, float(eta), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(W1), _ptr(W3), _ptr(W2), _ptr(dO), *[_ptr(g) for g in grads],
                                          _ptr(ws), nbytes, _stream(dev)), "ttt_lact_swiglu_backward")
    return grads
