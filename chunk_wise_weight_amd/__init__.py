"""chunk_wise_weight_amd -- chunk-wise TTT fast-weight layer on MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/ttt.h`` (libttt.so, built
in-tree by ``chunk_wise_weight_amd.build``).  PyTorch is used only to hold
device memory and to name the current stream: every step of the layer runs
in the library's HIP kernels.  There is no CPU fallback; if the library is
missing or no GPU is present the calls raise.

Functions keep the C names:
  ttt_chunk_apply_update, ttt_chunk_apply_update_noalloc, ttt_core_apply_update(_ex), ttt_core_backward,
  ttt_core_backward_mse, ttt_layer_backward, ttt_layer_backward_mse, ttt_produce_z,
  ttt_produce_vhat, ttt_chunk_delta, ttt_chunk_scan, ttt_chunk_update_scan,
  ttt_chunk_apply, ttt_lact_swiglu, ttt_lact_swiglu_backward (and its _ex form), plus the workspace queries.
"""
from ._lib import (  # noqa: F401
    TTT_OK, TTT_ERR_ARG, TTT_ERR_SHAPE, TTT_ERR_DTYPE, TTT_ERR_WORKSPACE, TTT_ERR_DEVICE,
    TTT_ERR_UNSUPPORTED, TTT_ERR_SCRATCH_LIMIT, TTT_NOALLOC_SCRATCH_BYTES, TTT_F32, TTT_BF16, TTT_MODE_DOT,
    TTT_MODE_MSE, TTT_MODE_DOT_SCAN,
    TTT_UPDATE_THEN_APPLY, TTT_APPLY_THEN_UPDATE, TTTError, InplaceShape, LactShape, LayerOptions, LactOptions,
    LactSideStream, BackwardOptions,
    lib, lib_path, exported_symbols, status_string,
    ttt_inplace_workspace_bytes, ttt_lact_workspace_bytes, ttt_vhat_workspace_bytes, ttt_update_scan_workspace_bytes,
    ttt_core_backward_workspace_bytes, ttt_core_backward, ttt_layer_backward_workspace_bytes, ttt_layer_backward,
    ttt_layer_backward_mse_workspace_bytes, ttt_layer_backward_mse,
    ttt_core_backward_mse_workspace_bytes, ttt_core_backward_mse,
    ttt_chunk_apply_update, ttt_chunk_apply_update_noalloc, ttt_core_apply_update, ttt_produce_z, ttt_produce_vhat,
    ttt_chunk_delta, ttt_chunk_scan, ttt_chunk_update_scan, ttt_chunk_apply, ttt_lact_swiglu,
    ttt_lact_backward_workspace_bytes, ttt_lact_swiglu_backward,
)
