"""libtwell for MI355X: the ReLU-gated FFN that skips exact-zero gate
activations through TwELL (tile-wise ELLPACK).

The package is a thin ctypes binding over lib/libtwell.so (C ABI declared in
include/twell.h); all computation happens in the library's HIP kernels.
Build the library with ``python -m activation_sparse_feedforward_gate_amd.build``.
"""
from ._lib import (  # noqa: F401
    C_TILE, R_TILE, TWELL_BF16, TWELL_EHIP, TWELL_EINVAL, TWELL_EUNSUPPORTED, TWELL_EWORKSPACE,
    TWELL_F32, TWELL_OK, TwellError, TwellMat, alloc_twell_mat, c_twell_ffn_shape, c_twell_mat,
    ffn_shape, header_functions, lib, twell_ffn_bwd_hybrid, twell_ffn_bwd_hybrid_l1, twell_ffn_bwd_workspace,
    twell_ffn_dense_fwd,
    twell_ffn_dense_fwd_workspace, twell_ffn_dense_bwd, twell_ffn_dense_bwd_workspace,
    twell_ffn_fwd, twell_ffn_fwd_ex, twell_ffn_fwd_workspace, twell_gate_pack, twell_last_error, twell_mat_bytes, twell_pack,
    twell_sparse_down, twell_sparse_up, twell_status_string, twell_unpack,
    twell_relu_ffn_fwd, twell_relu_ffn_fwd_workspace, twell_relu_ffn_dense_fwd, twell_relu_ffn_dense_fwd_workspace,
    TwellCMat, alloc_twell_cmat, c_twell_cmat, twell_cmat_bytes, twell_compact, twell_expand,
    twell_ffn_bwd_compact_workspace, twell_ffn_bwd_hybrid_compact, twell_ffn_fwd_noalloc, NOALLOC_SCRATCH_BYTES,
    twell_ffn_fwd_bounded_workspace, twell_ffn_fwd_bounded,
    twell_ffn_fwd_compact_workspace, twell_ffn_fwd_compact,
    twell_relu_ffn_fwd_bounded_workspace, twell_relu_ffn_fwd_bounded,
)
