"""Python binding of libfa355 (exact tiled attention for MI355X / gfx950).

Argument marshalling only: every step of the attention computation runs in
the library's HIP kernels.  Tensors are PyTorch tensors on a ROCm device;
PyTorch supplies the device memory and the stream.  If the compiled library
is missing, importing the ABI raises: there is no fallback path.

Names mirror the C entry points of ``include/fa355.h``:

    fa_fwd(q, k, v, causal, scale, o=None, lse=None, stream=None) -> (o, lse)
    fa_bwd(q, k, v, o, lse, dout, causal, scale, ...) -> (dq, dk, dv)
    fa_bwd_noalloc(q, k, v, o, lse, dout, causal, scale, ...) -> (dq, dk, dv)
    fa_bwd_prepare(o, dout) -> delta
    fa_bwd_dkdv(q, k, v, lse, dout, delta, causal, scale) -> (dk, dv)
    fa_bwd_dq(q, k, v, lse, dout, delta, causal, scale) -> dq
    fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype) -> int
    fa_fwd_splitkv(q, k, v, causal, scale, num_splits=0, ...) -> (o, lse)
    fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits) -> int
    fa_fwd_splitkv_default_splits(B, H_q, H_kv, N_q, N_kv, d) -> int
    fa_fwd_dropout(q, k, v, causal, scale, dropout_p, seed, offset=0) -> (o, lse)
    fa_bwd_dropout(q, k, v, o, lse, dout, causal, scale, dropout_p, seed, offset=0) -> (dq, dk, dv)
    fa_fwd_blocksparse(q, k, v, block_mask, causal, scale) -> (o, lse)
    fa_bwd_blocksparse(q, k, v, o, lse, dout, block_mask, causal, scale) -> (dq, dk, dv)
    fa_fwd_varlen(q, k, v, seqlens, causal, scale) -> (o, lse)
    fa_bwd_varlen(q, k, v, o, lse, dout, seqlens, causal, scale) -> (dq, dk, dv)
    fa_fp8_quantize(x, signs=None, ...) -> (codes, scales)
    fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal, scale, out_dtype="bf16") -> (o, lse)
    fa_status_string(code) -> str
    fa_version() -> int
"""
from ._abi import (FA_DTYPE, FP8_BLOCK_ROWS, NOALLOC_SCRATCH_BYTES, FaError, fa_bwd,
                   fa_bwd_dkdv, fa_bwd_dq, fa_bwd_noalloc,
                   fa_bwd_blocksparse, fa_bwd_dropout, fa_bwd_prepare, fa_bwd_workspace_size,
                   fa_bwd_varlen, fa_fp8_quantize, fa_fwd, fa_fwd_blocksparse, fa_fwd_dropout,
                   fa_fwd_fp8, fa_fwd_varlen,
                   fa_fwd_splitkv, fa_fwd_splitkv_default_splits,
                   fa_fwd_splitkv_workspace_size, fa_status_string, fa_version, lib_path,
                   load_library)

__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "fa_bwd_prepare", "fa_bwd_dkdv", "fa_bwd_dq",
           "fa_bwd_workspace_size", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
           "fa_fwd_splitkv_default_splits", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_blocksparse", "fa_bwd_blocksparse", "fa_fwd_varlen", "fa_bwd_varlen", "fa_fp8_quantize", "fa_fwd_fp8", "FP8_BLOCK_ROWS",
           "fa_status_string", "fa_version", "FaError", "FA_DTYPE",
           "load_library", "lib_path"]
