"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from exact_attention_99_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

INVALID, UNSUPPORTED = 1, 2
FP32, FP16, BF16 = 0, 1, 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _abi.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_blocksparse", "fa_bwd_dkdv", "fa_bwd_dq",
                                    "fa_bwd_dropout", "fa_bwd_noalloc", "fa_bwd_prepare",
                                    "fa_bwd_varlen",
                                    "fa_bwd_workspace_size", "fa_fp8_quantize", "fa_fwd",
                                    "fa_fwd_blocksparse", "fa_fwd_dropout", "fa_fwd_fp8",
                                    "fa_fwd_splitkv", "fa_fwd_splitkv_default_splits",
                                    "fa_fwd_splitkv_workspace_size", "fa_fwd_varlen",
                                    "fa_status_string", "fa_version"]


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    raw = ctypes.CDLL(_abi.lib_path())
    for name in declared_functions():
        getattr(raw, name)


def test_shipped_library_has_no_clock_probe(lib):
    """The per-wave clock records exist only in measurement builds
    (FA355_CLOCK_PROBE=1); the package's own library compiles them away."""
    if os.environ.get("FA355_LIB"):
        pytest.skip("an alternative library is selected")
    for name in ("fa355_clock_fwd_read", "fa355_clock_bwd_read"):
        assert not hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert _abi.fa_version() == 100
    for code in range(5):
        s = _abi.fa_status_string(code)
        assert s.startswith(_abi.STATUS[code])
    assert _abi.fa_status_string(99) == "unknown fa_status"


def test_workspace_size_is_linear_in_N(lib):
    def ws(N):
        return _abi.fa_bwd_workspace_size(2, 8, 2, N, 128, "bf16")
    rows = 2 * 8 * 4096
    assert ws(4096) == rows * 4
    assert ws(8192) == 2 * ws(4096)
    assert _abi.fa_bwd_workspace_size(1, 1, 1, 1, 64, "fp32") == 256
    # invalid sizes give 0
    assert _abi.fa_bwd_workspace_size(1, 3, 2, 16, 64, "bf16") == 0
    assert _abi.fa_bwd_workspace_size(1, 1, 1, 0, 64, "bf16") == 0
    assert _abi.fa_bwd_workspace_size(1, 1, 1, 16, 96, "bf16") == 0


# Fake device addresses: argument checks run before any device access, and
# every call below is rejected by them.
A = 1 << 20          # 16-byte aligned
MIS = A + 8          # misaligned


def fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=1, N=16, d=64, causal=0, scale=0.125,
        dtype=BF16):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, None)


def bwd(lib, ws_bytes=1 << 30, d=64, N=16, causal=0, scale=0.125, dtype=BF16, B=1, Hq=2, Hkv=1,
        ptrs=None):
    p = ptrs or [A] * 10
    return lib.fa_bwd(*p[:9], p[9], ws_bytes, B, Hq, Hkv, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, INVALID), ({"k": None}, INVALID), ({"v": None}, INVALID),
    ({"o": None}, INVALID), ({"lse": None}, INVALID),
    ({"q": MIS}, INVALID), ({"o": MIS}, INVALID), ({"lse": MIS}, INVALID),
    ({"B": 0}, INVALID), ({"Hq": 0}, INVALID), ({"Hkv": 0}, INVALID), ({"N": 0}, INVALID),
    ({"N": -5}, INVALID), ({"Hq": 3, "Hkv": 2}, INVALID), ({"causal": 2}, INVALID),
    ({"scale": float("nan")}, INVALID), ({"scale": float("inf")}, INVALID),
    ({"scale": 0.0}, INVALID), ({"scale": -0.1}, INVALID),
    ({"dtype": 7}, INVALID), ({"d": 96}, UNSUPPORTED), ({"d": 256}, UNSUPPORTED),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_bwd_rejects(lib):
    assert bwd(lib, ptrs=[A] * 9 + [None]) == INVALID
    for i in range(10):
        p = [A] * 10
        p[i] = None
        assert bwd(lib, ptrs=p) == INVALID
        p[i] = MIS
        assert bwd(lib, ptrs=p) == INVALID
    need = _abi.fa_bwd_workspace_size(1, 2, 1, 16, 64, "bf16")
    assert bwd(lib, ws_bytes=need - 1) == INVALID
    assert bwd(lib, d=80) == UNSUPPORTED
    assert bwd(lib, causal=-1) == INVALID
    assert bwd(lib, scale=float("nan")) == INVALID
    assert bwd(lib, Hq=4, Hkv=3) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("FA355_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _abi.load_library()


def test_phase_entry_points_reject(lib):
    assert lib.fa_bwd_prepare(None, A, A, 1, 2, 16, 64, BF16, None) == INVALID
    assert lib.fa_bwd_prepare(A, A, MIS, 1, 2, 16, 64, BF16, None) == INVALID
    assert lib.fa_bwd_prepare(A, A, A, 1, 2, 16, 80, BF16, None) == UNSUPPORTED
    assert lib.fa_bwd_prepare(A, A, A, 0, 2, 16, 64, BF16, None) == INVALID
    args = [A] * 8
    for i in range(8):
        p = list(args)
        p[i] = None
        assert lib.fa_bwd_dkdv(*p, 1, 2, 1, 16, 64, 0, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_dkdv(*args, 1, 3, 2, 16, 64, 0, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_dkdv(*args, 1, 2, 1, 16, 64, 0, -1.0, BF16, None) == INVALID
    assert lib.fa_bwd_dkdv(*args, 1, 2, 1, 16, 32, 0, 0.1, BF16, None) == UNSUPPORTED
    for i in range(7):
        p = [A] * 7
        p[i] = MIS
        assert lib.fa_bwd_dq(*p, 1, 2, 1, 16, 64, 1, 0.1, FP16, None) == INVALID
    assert lib.fa_bwd_dq(*([A] * 7), 1, 2, 1, 16, 64, 3, 0.1, FP16, None) == INVALID
    assert lib.fa_bwd_dq(*([A] * 7), 1, 2, 1, 16, 64, 1, 0.1, 9, None) == INVALID


def split(lib, ptrs=None, ws_bytes=1 << 30, B=1, Hq=4, Hkv=1, Nq=1, Nkv=1000, d=128, causal=1,
          scale=0.088, splits=8, dtype=BF16):
    p = ptrs or [A] * 6
    return lib.fa_fwd_splitkv(*p[:5], p[5], ws_bytes, B, Hq, Hkv, Nq, Nkv, d, causal, scale, splits,
                              dtype, None)


def test_splitkv_rejects(lib):
    for i in range(6):
        p = [A] * 6
        p[i] = None
        assert split(lib, ptrs=p) == INVALID
        p[i] = MIS
        assert split(lib, ptrs=p) == INVALID
    need = _abi.fa_fwd_splitkv_workspace_size(1, 4, 1, 128, 8)
    assert split(lib, ws_bytes=need - 1) == INVALID
    assert split(lib, Nq=1001, Nkv=1000) == INVALID          # causal needs N_q <= N_kv
    assert split(lib, Nq=0) == INVALID and split(lib, Nkv=0) == INVALID
    assert split(lib, Hq=3, Hkv=2) == INVALID
    assert split(lib, splits=0) == INVALID and split(lib, splits=1025) == INVALID
    assert split(lib, causal=2) == INVALID
    assert split(lib, scale=0.0) == INVALID and split(lib, scale=float("nan")) == INVALID
    assert split(lib, dtype=7) == INVALID
    assert split(lib, d=96) == UNSUPPORTED
    assert split(lib, dtype=FP32) == UNSUPPORTED


def test_splitkv_sizes(lib):
    # partial outputs (splits x rows x d floats) then partial logsumexps, each
    # rounded up to 256 bytes
    rows = 2 * 8 * 3
    assert _abi.fa_fwd_splitkv_workspace_size(2, 8, 3, 64, 5) == (
        (5 * rows * 64 * 4 + 255) // 256 * 256 + (5 * rows * 4 + 255) // 256 * 256)
    assert _abi.fa_fwd_splitkv_workspace_size(1, 1, 1, 64, 0) == 0
    assert _abi.fa_fwd_splitkv_workspace_size(1, 1, 1, 80, 1) == 0
    # the suggested split count fills the device but keeps chunks of >= 4 tiles
    assert 1 <= _abi.fa_fwd_splitkv_default_splits(1, 32, 8, 1, 65536, 128) <= 512
    assert _abi.fa_fwd_splitkv_default_splits(1, 1, 1, 1, 64, 128) == 1
    assert _abi.fa_fwd_splitkv_default_splits(1, 3, 2, 1, 64, 128) == 0


def test_fp8_entry_points_reject(lib):
    # fa_fp8_quantize(x, signs, codes, scales, B, H, N, d, dtype, stream)
    assert lib.fa_fp8_quantize(None, None, A, A, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, None, None, A, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, None, A, None, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(MIS, None, A, A, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, MIS, A, A, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, None, A, A + 2, 1, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, None, A, A, 0, 2, 100, 128, BF16, None) == INVALID
    assert lib.fa_fp8_quantize(A, None, A, A, 1, 2, 100, 96, BF16, None) == UNSUPPORTED
    assert lib.fa_fp8_quantize(A, None, A, A, 1, 2, 100, 128, FP32, None) == UNSUPPORTED
    assert lib.fa_fp8_quantize(A, None, A, A, 1, 2, 100, 128, 5, None) == INVALID
    # fa_fwd_fp8(q, k, v, sq, sk, sv, o, lse, B, Hq, Hkv, N, d, causal, scale, out_dtype, stream)
    for i in range(8):
        p = [A] * 8
        p[i] = None
        assert lib.fa_fwd_fp8(*p, 1, 4, 2, 100, 128, 1, 0.1, BF16, None) == INVALID
    for i in (0, 1, 2, 6, 7):
        p = [A] * 8
        p[i] = MIS
        assert lib.fa_fwd_fp8(*p, 1, 4, 2, 100, 128, 1, 0.1, BF16, None) == INVALID
    p = [A] * 8
    p[4] = A + 2
    assert lib.fa_fwd_fp8(*p, 1, 4, 2, 100, 128, 1, 0.1, BF16, None) == INVALID
    q = [A] * 8
    assert lib.fa_fwd_fp8(*q, 1, 4, 3, 100, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_fwd_fp8(*q, 1, 4, 2, 100, 128, 2, 0.1, BF16, None) == INVALID
    assert lib.fa_fwd_fp8(*q, 1, 4, 2, 100, 128, 1, 0.0, BF16, None) == INVALID
    assert lib.fa_fwd_fp8(*q, 1, 4, 2, 100, 32, 1, 0.1, BF16, None) == UNSUPPORTED
    assert lib.fa_fwd_fp8(*q, 1, 4, 2, 100, 128, 1, 0.1, FP32, None) == UNSUPPORTED


def test_dropout_entry_points_reject(lib):
    # fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, p, seed, offset, dtype, stream)
    ok = [A] * 5
    for i in range(5):
        p = [A] * 5
        p[i] = None
        assert lib.fa_fwd_dropout(*p, 1, 2, 1, 64, 128, 1, 0.1, 0.1, 1, 2, BF16, None) == INVALID
        p[i] = MIS
        assert lib.fa_fwd_dropout(*p, 1, 2, 1, 64, 128, 1, 0.1, 0.1, 1, 2, BF16, None) == INVALID
    for bad_p in (-0.1, 1.0, 0.999, float("nan")):
        assert lib.fa_fwd_dropout(*ok, 1, 2, 1, 64, 128, 1, 0.1, bad_p, 1, 2, BF16, None) == INVALID
    assert lib.fa_fwd_dropout(*ok, 1, 2, 1, 64, 96, 1, 0.1, 0.1, 1, 2, BF16, None) == UNSUPPORTED
    assert lib.fa_fwd_dropout(*ok, 1, 2, 1, 64, 128, 1, 0.1, 0.1, 1, 2, FP32, None) == UNSUPPORTED
    assert lib.fa_fwd_dropout(*ok, 1, 3, 2, 64, 128, 1, 0.1, 0.1, 1, 2, BF16, None) == INVALID
    # fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, N, d, causal,
    #                scale, p, seed, offset, dtype, stream)
    for i in range(10):
        p = [A] * 10
        p[i] = None
        assert lib.fa_bwd_dropout(*p, 1 << 20, 1, 2, 1, 64, 128, 0, 0.1, 0.1, 1, 2, BF16, None) == INVALID
    need = _abi.fa_bwd_workspace_size(1, 2, 1, 64, 128, "bf16")
    assert lib.fa_bwd_dropout(*([A] * 10), need - 1, 1, 2, 1, 64, 128, 0, 0.1, 0.1, 1, 2, BF16, None) == INVALID
    assert lib.fa_bwd_dropout(*([A] * 10), need, 1, 2, 1, 64, 128, 0, 0.1, 1.5, 1, 2, BF16, None) == INVALID
    assert lib.fa_bwd_dropout(*([A] * 10), need, 1, 2, 1, 64, 128, 0, 0.1, 0.1, 1, 2, FP32, None) == UNSUPPORTED


def test_blocksparse_entry_points_reject(lib):
    # fa_fwd_blocksparse(q, k, v, o, lse, mask, mask_heads, B, Hq, Hkv, N, d, causal, scale, dtype, stream)
    for i in range(6):
        p = [A] * 6
        p[i] = None
        assert lib.fa_fwd_blocksparse(*p, 1, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    for i in range(5):
        p = [A] * 6
        p[i] = MIS
        assert lib.fa_fwd_blocksparse(*p, 1, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    ok = [A] * 5 + [A + 3]     # the mask needs no alignment
    assert lib.fa_fwd_blocksparse(*ok, 2, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID   # mask_heads
    assert lib.fa_fwd_blocksparse(*ok, 1, 1, 4, 2, 300, 96, 1, 0.1, BF16, None) == UNSUPPORTED
    assert lib.fa_fwd_blocksparse(*ok, 1, 1, 4, 2, 300, 128, 1, 0.1, FP32, None) == UNSUPPORTED
    assert lib.fa_fwd_blocksparse(*ok, 1, 1, 4, 2, 300, 128, 3, 0.1, BF16, None) == INVALID
    # fa_bwd_blocksparse(10 pointers, ws_bytes, mask, mask_heads, B, Hq, Hkv, N, d, causal, scale, dtype, stream)
    need = _abi.fa_bwd_workspace_size(1, 4, 2, 300, 128, "bf16")
    for i in range(10):
        p = [A] * 10
        p[i] = None
        assert lib.fa_bwd_blocksparse(*p, need, A, 1, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_blocksparse(*([A] * 10), need, None, 1, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_blocksparse(*([A] * 10), need - 1, A, 1, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_blocksparse(*([A] * 10), need, A, 3, 1, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_blocksparse(*([A] * 10), need, A, 4, 1, 4, 2, 300, 128, 1, 0.1, FP32, None) == UNSUPPORTED


def test_varlen_entry_points_reject(lib):
    # fa_fwd_varlen(q, k, v, o, lse, seqlens, B, Hq, Hkv, N, d, causal, scale, dtype, stream)
    for i in range(6):
        p = [A] * 6
        p[i] = None
        assert lib.fa_fwd_varlen(*p, 2, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    p = [A] * 5 + [A + 2]       # seqlens must be 4-byte aligned
    assert lib.fa_fwd_varlen(*p, 2, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    ok = [A] * 6
    assert lib.fa_fwd_varlen(*ok, 2, 4, 2, 300, 96, 1, 0.1, BF16, None) == UNSUPPORTED
    assert lib.fa_fwd_varlen(*ok, 2, 4, 2, 300, 128, 1, 0.1, FP32, None) == UNSUPPORTED
    assert lib.fa_fwd_varlen(*ok, 2, 4, 3, 300, 128, 1, 0.1, BF16, None) == INVALID
    need = _abi.fa_bwd_workspace_size(2, 4, 2, 300, 128, "bf16")
    for i in range(10):
        p = [A] * 10
        p[i] = None
        assert lib.fa_bwd_varlen(*p, need, A, 2, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_varlen(*([A] * 10), need, None, 2, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_varlen(*([A] * 10), need - 1, A, 2, 4, 2, 300, 128, 1, 0.1, BF16, None) == INVALID
    assert lib.fa_bwd_varlen(*([A] * 10), need, A, 2, 4, 2, 300, 128, 1, 0.1, FP32, None) == UNSUPPORTED


def test_binding_checks_buffers_before_the_call(lib):
    """The binding checks the shape and dtype of every tensor it hands over
    (the layouts of include/fa355.h) and that they live on a GPU, so a
    mis-sized output raises instead of reaching a kernel."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 64, 64
    q = torch.zeros(B, Hq, N, d, dtype=torch.bfloat16)
    k = torch.zeros(B, Hkv, N, d, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    lse = torch.zeros(B, Hq, N)
    with pytest.raises(ValueError, match="o must be"):
        _abi.fa_fwd(q, k, v, True, 0.1, o=torch.zeros(B, Hq, N - 1, d, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must be"):
        _abi.fa_fwd(q, k, v, True, 0.1, lse=torch.zeros(B, Hq, N, dtype=torch.float64))
    with pytest.raises(ValueError, match="GPU"):
        _abi.fa_fwd(q, k, v, True, 0.1)
    with pytest.raises(ValueError, match="dout must be"):
        _abi.fa_bwd(q, k, v, q, lse, q.to(torch.float16), True, 0.1)
    with pytest.raises(ValueError, match="dk must be"):
        _abi.fa_bwd(q, k, v, q, lse, q, True, 0.1, dk=torch.zeros_like(q))
    with pytest.raises(ValueError, match="lse must be"):
        _abi.fa_bwd_dq(q, k, v, lse[:, :2], q, lse, True, 0.1)
    with pytest.raises(ValueError, match="delta must be"):
        _abi.fa_bwd_dkdv(q, k, v, lse, q, lse[..., :8], True, 0.1)
    with pytest.raises(ValueError, match="dout must be"):
        _abi.fa_bwd_prepare(q, k)
    with pytest.raises(TypeError, match="share a dtype"):
        _abi.fa_bwd(q, k.float(), v, q, lse, q, True, 0.1)


def test_noalloc_rejects(lib):
    """fa_bwd_noalloc takes fa_bwd's checks, and problems whose row terms do
    not fit the fixed scratch (more than FA_NOALLOC_SCRATCH_BYTES / 4 rows of
    B * H_q * N) get FA_ERR_TOO_LARGE before anything is enqueued."""
    TOO_LARGE = 4

    def call(ptrs=None, B=1, Hq=2, Hkv=1, N=16, d=64, causal=0, scale=0.125, dtype=BF16):
        p = ptrs or [A] * 9
        return lib.fa_bwd_noalloc(*p, B, Hq, Hkv, N, d, causal, scale, dtype, None)

    for i in range(9):
        p = [A] * 9
        p[i] = None
        assert call(ptrs=p) == INVALID
        p[i] = MIS
        assert call(ptrs=p) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(causal=3) == INVALID
    assert call(Hq=3, Hkv=2) == INVALID
    rows_max = _abi.NOALLOC_SCRATCH_BYTES // 4
    assert call(B=1, Hq=32, Hkv=8, N=rows_max // 32 + 1) == TOO_LARGE
    assert call(B=4, Hq=32, Hkv=32, N=65536) == TOO_LARGE
    assert _abi.fa_status_string(TOO_LARGE).startswith("FA_ERR_TOO_LARGE")
