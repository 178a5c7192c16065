"""ctypes declarations for libfa355 and torch-tensor marshalling."""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa355.so"

# fa_dtype values (include/fa355.h)
FA_DTYPE = {"fp32": 0, "fp16": 1, "bf16": 2}

STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED", 3: "FA_ERR_HIP",
          4: "FA_ERR_TOO_LARGE"}

# fixed scratch of fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES in include/fa355.h)
NOALLOC_SCRATCH_BYTES = 16 << 20

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


class FaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({fa_status_string(code)})")


def lib_path() -> str:
    return os.environ.get("FA355_LIB", os.path.join(PKG, _LIB_NAME))


def load_library() -> ctypes.CDLL:
    """Load the compiled library; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m exact_attention_99_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                               i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_noalloc.restype = i
        lib.fa_bwd_prepare.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
        lib.fa_bwd_prepare.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_dq.restype = i
        lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i, i]
        lib.fa_bwd_workspace_size.restype = sz
        lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, i, vp]
        lib.fa_fwd_splitkv.restype = i
        lib.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i]
        lib.fa_fwd_splitkv_workspace_size.restype = sz
        lib.fa_fwd_splitkv_default_splits.argtypes = [i, i, i, i, i, i]
        lib.fa_fwd_splitkv_default_splits.restype = i
        u64 = ctypes.c_ulonglong
        lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, u64, u64, i, vp]
        lib.fa_fwd_dropout.restype = i
        lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       i, i, i, i, i, i, f, f, u64, u64, i, vp]
        lib.fa_bwd_dropout.restype = i
        lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_blocksparse.restype = i
        lib.fa_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i,
                                           i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_blocksparse.restype = i
        lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_varlen.restype = i
        lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                      i, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_varlen.restype = i
        lib.fa_fp8_quantize.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
        lib.fa_fp8_quantize.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_status_string.argtypes = [i]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = i
        _lib = lib
        return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def fa_version() -> int:
    return int(load_library().fa_version())


def fa_bwd_workspace_size(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H_q, H_kv, N, d, FA_DTYPE[dtype]))


def _dtype_name(t) -> str:
    import torch
    m = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _shape(q, k, v) -> Tuple[int, int, int, int, int]:
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return B, Hq, k.shape[1], N, d


def _check_same(ref, *ts):
    if ref.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in ts:
        if t.device != ref.device:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _expect(t, shape, dtype, name: str):
    """Shape and dtype of a tensor handed to the library (the layouts of
    include/fa355.h); a mismatch raises instead of reaching a kernel."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")


def _check_qkv_dtype(q, k, v):
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")


def _check_fwd_out(q, o, lse, B, Hq, N):
    import torch
    _expect(o, q.shape, q.dtype, "o")
    _expect(lse, (B, Hq, N), torch.float32, "lse")


def _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N):
    """Forward results and gradient buffers of the backward entry points."""
    import torch
    if o is not None:
        _expect(o, q.shape, q.dtype, "o")
    _expect(lse, (B, Hq, N), torch.float32, "lse")
    _expect(dout, q.shape, q.dtype, "dout")
    if dq is not None:
        _expect(dq, q.shape, q.dtype, "dq")
    if dk is not None:
        _expect(dk, k.shape, q.dtype, "dk")
    if dv is not None:
        _expect(dv, k.shape, q.dtype, "dv")


def _stream(ref, stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream(ref.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fa_fwd(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None):
    """O = softmax(scale * q k^T [causal]) v and the row logsumexp; returns (o, lse)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_fwd_out(q, o, lse, B, Hq, N)
    _check_same(q, k, v, o, lse)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, Hq, Hkv, N, d, int(bool(causal)), float(scale), FA_DTYPE[dt],
                    _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd")
    return o, lse


def fa_fwd_splitkv_workspace_size(B: int, H_q: int, N_q: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits))


def fa_fwd_splitkv_default_splits(B: int, H_q: int, H_kv: int, N_q: int, N_kv: int, d: int) -> int:
    return int(load_library().fa_fwd_splitkv_default_splits(B, H_q, H_kv, N_q, N_kv, d))


def fa_fwd_splitkv(q, k, v, causal: bool, scale: float, num_splits: int = 0, o=None, lse=None,
                   workspace=None, stream=None):
    """Split-KV forward for q [B, H_q, N_q, d] against k, v [B, H_kv, N_kv, d];
    num_splits = 0 takes fa_fwd_splitkv_default_splits().  Returns (o, lse)."""
    import torch
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Nkv = k.shape[1], k.shape[2]
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if num_splits == 0:
        num_splits = int(lib.fa_fwd_splitkv_default_splits(B, Hq, Hkv, Nq, Nkv, d))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_fwd_out(q, o, lse, B, Hq, Nq)
    need = int(lib.fa_fwd_splitkv_workspace_size(B, Hq, Nq, d, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_same(q, k, v, o, lse, workspace)
    st = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            B, Hq, Hkv, Nq, Nkv, d, int(bool(causal)), float(scale), int(num_splits),
                            FA_DTYPE[dt], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd_splitkv")
    return o, lse


def fa_bwd(q, k, v, o, lse, dout, causal: bool, scale: float, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """Gradients of sum(dout * o) for q, k, v; returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N)
    need = int(lib.fa_bwd_workspace_size(B, Hq, Hkv, N, d, FA_DTYPE[dt]))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_same(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                    B, Hq, Hkv, N, d, int(bool(causal)), float(scale), FA_DTYPE[dt],
                    _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, dout, causal: bool, scale: float, dq=None, dk=None, dv=None,
                   stream=None):
    """fa_bwd without a workspace: the library's fixed per-device scratch holds
    the row terms (at most NOALLOC_SCRATCH_BYTES / 4 rows of B * H_q * N), so
    the entry point itself allocates nothing.  Returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N)
    _check_same(q, k, v, o, lse, dout, dq, dk, dv)
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            B, Hq, Hkv, N, d, int(bool(causal)), float(scale), FA_DTYPE[dt],
                            _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_bwd_prepare(o, dout, delta=None, stream=None):
    """delta_i = sum_k dout_ik o_ik (float32 [B, H_q, N]); returns delta."""
    import torch
    lib = load_library()
    if o.dim() != 4:
        raise ValueError("o must be 4-D [B, H_q, N, d]")
    B, Hq, N, d = o.shape
    _dtype_name(o)
    _expect(dout, o.shape, o.dtype, "dout")
    if delta is None:
        delta = torch.empty((B, Hq, N), dtype=torch.float32, device=o.device)
    _expect(delta, (B, Hq, N), torch.float32, "delta")
    _check_same(o, dout, delta)
    st = lib.fa_bwd_prepare(o.data_ptr(), dout.data_ptr(), delta.data_ptr(), B, Hq, N, d,
                            FA_DTYPE[_dtype_name(o)], _stream(o, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_prepare")
    return delta


def fa_bwd_dkdv(q, k, v, lse, dout, delta, causal: bool, scale: float, dk=None, dv=None,
                stream=None):
    """dk, dv from the forward's lse and the prepared delta; returns (dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, None, lse, dout, None, dk, dv, B, Hq, N)
    _expect(delta, (B, Hq, N), torch.float32, "delta")
    _check_same(q, k, v, lse, dout, delta, dk, dv)
    st = lib.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                         delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d,
                         int(bool(causal)), float(scale), FA_DTYPE[_dtype_name(q)],
                         _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_dkdv")
    return dk, dv


def fa_bwd_dq(q, k, v, lse, dout, delta, causal: bool, scale: float, dq=None, stream=None):
    """dq from the forward's lse and the prepared delta; returns dq."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    _check_bwd_args(q, k, None, lse, dout, dq, None, None, B, Hq, N)
    _expect(delta, (B, Hq, N), torch.float32, "delta")
    _check_same(q, k, v, lse, dout, delta, dq)
    st = lib.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                       delta.data_ptr(), dq.data_ptr(), B, Hq, Hkv, N, d, int(bool(causal)),
                       float(scale), FA_DTYPE[_dtype_name(q)], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_dq")
    return dq


FP8_BLOCK_ROWS = 64


def fa_fp8_quantize(x, signs=None, codes=None, scales=None, stream=None):
    """Block-quantize x [B, H, N, d] (bf16 / fp16) to e4m3 codes (uint8, same
    shape) and float32 scales [B, H, ceil(N / 64)]; ``signs`` (d float32 +-1
    values) applies the rotation first.  Returns (codes, scales)."""
    import torch
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be 4-D [B, H, N, d]")
    B, H, N, d = x.shape
    dt = _dtype_name(x)
    nblk = (N + FP8_BLOCK_ROWS - 1) // FP8_BLOCK_ROWS
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
    if codes.dtype != torch.uint8 or tuple(codes.shape) != tuple(x.shape):
        raise ValueError("codes must be uint8 with the shape of x")
    if scales.dtype != torch.float32 or tuple(scales.shape) != (B, H, nblk):
        raise ValueError(f"scales must be float32 [{B}, {H}, {nblk}]")
    tensors = [x, codes, scales]
    if signs is not None:
        if signs.dtype != torch.float32 or tuple(signs.shape) != (d,):
            raise ValueError(f"signs must be float32 [{d}]")
        tensors.append(signs)
    _check_same(*tensors)
    st = lib.fa_fp8_quantize(x.data_ptr(), signs.data_ptr() if signs is not None else None,
                             codes.data_ptr(), scales.data_ptr(), B, H, N, d, FA_DTYPE[dt],
                             _stream(x, stream))
    if st != 0:
        raise FaError(st, "fa_fp8_quantize")
    return codes, scales


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, causal: bool, scale: float,
               out_dtype: str = "bf16", o=None, lse=None, stream=None):
    """Attention of block-quantized inputs (e4m3 codes q, k, v and their
    block scales); returns (o, lse) with o in ``out_dtype``."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    for t in (q, k, v):
        if t.dtype != torch.uint8:
            raise TypeError("q, k, v must be uint8 e4m3 codes")
    nblk = (N + FP8_BLOCK_ROWS - 1) // FP8_BLOCK_ROWS
    for t, h in ((q_scale, Hq), (k_scale, Hkv), (v_scale, Hkv)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, h, nblk):
            raise ValueError(f"block scales must be float32 [B, H, {nblk}]")
    if out_dtype not in ("bf16", "fp16"):
        raise ValueError("out_dtype must be bf16 or fp16")
    if o is None:
        o = torch.empty(q.shape, dtype=_OUT_DTYPES()[out_dtype], device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _expect(o, q.shape, _OUT_DTYPES()[out_dtype], "o")
    _expect(lse, (B, Hq, N), torch.float32, "lse")
    _check_same(q, k, v, q_scale, k_scale, v_scale, o, lse)
    st = lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(),
                        k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, int(bool(causal)), float(scale), FA_DTYPE[out_dtype],
                        _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def _OUT_DTYPES():
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}


def fa_fwd_dropout(q, k, v, causal: bool, scale: float, dropout_p: float, seed: int, offset: int = 0,
                   o=None, lse=None, stream=None):
    """Forward with attention dropout (mask drawn from Philox4x64-10 keyed by
    seed and offset); returns (o, lse)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_fwd_out(q, o, lse, B, Hq, N)
    _check_same(q, k, v, o, lse)
    st = lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, N, d, int(bool(causal)), float(scale), float(dropout_p),
                            int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), FA_DTYPE[dt],
                            _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd_dropout")
    return o, lse


def fa_bwd_dropout(q, k, v, o, lse, dout, causal: bool, scale: float, dropout_p: float, seed: int,
                   offset: int = 0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd_dropout with the same dropout_p, seed and offset;
    returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N)
    need = int(lib.fa_bwd_workspace_size(B, Hq, Hkv, N, d, FA_DTYPE[dt]))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_same(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    st = lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            B, Hq, Hkv, N, d, int(bool(causal)), float(scale), float(dropout_p),
                            int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), FA_DTYPE[dt],
                            _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_dropout")
    return dq, dk, dv


SPARSE_BLOCK = 128


def _check_block_mask(block_mask, H_q, N):
    import torch
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if block_mask.dtype not in (torch.uint8, torch.bool) or block_mask.dim() != 3 or \
            tuple(block_mask.shape[1:]) != (nb, nb) or block_mask.shape[0] not in (1, H_q):
        raise ValueError(f"block_mask must be uint8/bool [1 or {H_q}, {nb}, {nb}]")
    return block_mask.shape[0]


def fa_fwd_blocksparse(q, k, v, block_mask, causal: bool, scale: float, o=None, lse=None, stream=None):
    """Attention restricted to the 128 x 128 blocks block_mask allows
    ([1 or H_q, nb, nb], nonzero = visible); returns (o, lse)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    mh = _check_block_mask(block_mask, Hq, N)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_fwd_out(q, o, lse, B, Hq, N)
    _check_same(q, k, v, o, lse, block_mask)
    st = lib.fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                block_mask.data_ptr(), mh, B, Hq, Hkv, N, d, int(bool(causal)),
                                float(scale), FA_DTYPE[dt], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd_blocksparse")
    return o, lse


def fa_bwd_blocksparse(q, k, v, o, lse, dout, block_mask, causal: bool, scale: float, dq=None,
                       dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd_blocksparse with the same mask; returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    mh = _check_block_mask(block_mask, Hq, N)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N)
    need = int(lib.fa_bwd_workspace_size(B, Hq, Hkv, N, d, FA_DTYPE[dt]))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_same(q, k, v, o, lse, dout, dq, dk, dv, workspace, block_mask)
    st = lib.fa_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                block_mask.data_ptr(), mh, B, Hq, Hkv, N, d, int(bool(causal)),
                                float(scale), FA_DTYPE[dt], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_blocksparse")
    return dq, dk, dv


def _check_seqlens(seqlens, B):
    import torch
    if seqlens.dtype != torch.int32 or tuple(seqlens.shape) != (B,):
        raise ValueError(f"seqlens must be int32 [{B}]")


def fa_fwd_varlen(q, k, v, seqlens, causal: bool, scale: float, o=None, lse=None, stream=None):
    """Attention of a padded batch whose element b holds seqlens[b] tokens
    (int32 [B] on the device); returns (o, lse), zero / -inf on padding."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_qkv_dtype(q, k, v)
    _check_seqlens(seqlens, B)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_fwd_out(q, o, lse, B, Hq, N)
    _check_same(q, k, v, o, lse, seqlens)
    st = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           seqlens.data_ptr(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                           FA_DTYPE[dt], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen")
    return o, lse


def fa_bwd_varlen(q, k, v, o, lse, dout, seqlens, causal: bool, scale: float, dq=None, dk=None,
                  dv=None, workspace=None, stream=None):
    """Backward of fa_fwd_varlen with the same lengths; returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k, v)
    dt = _dtype_name(q)
    _check_seqlens(seqlens, B)
    _check_qkv_dtype(q, k, v)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_bwd_args(q, k, o, lse, dout, dq, dk, dv, B, Hq, N)
    need = int(lib.fa_bwd_workspace_size(B, Hq, Hkv, N, d, FA_DTYPE[dt]))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_same(q, k, v, o, lse, dout, dq, dk, dv, workspace, seqlens)
    st = lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           seqlens.data_ptr(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                           FA_DTYPE[dt], _stream(q, stream))
    if st != 0:
        raise FaError(st, "fa_bwd_varlen")
    return dq, dk, dv
