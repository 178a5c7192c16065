"""The FP8 quantization oracle against facts outside itself (CPU only):
torch's float8_e4m3fn casts, scipy's Hadamard matrix, closed forms."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import types

import oracle.fp8 as fp8_real


def _torch_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_decode_every_code_matches_torch(fp8):
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[finite], ref[finite])
    assert fp8.e4m3_decode(np.array([0x7E]))[0] == 448.0       # largest finite value
    assert fp8.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9   # smallest subnormal
    assert fp8.e4m3_decode(np.array([0x38]))[0] == 1.0


def check_encode_round_trip_and_ties_match_torch(fp8):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)
    # every midpoint between neighbouring codes (ties to even) and random values
    pos = fp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(3)
    rand = rng.uniform(-448, 448, 20000) * rng.choice([1, 1e-2, 1e-4], 20000)
    for x in (mids, -mids, rand, np.array([0.0, -0.0, 2.0 ** -10, -2.0 ** -10])):
        x32 = np.asarray(x, dtype=np.float32)
        assert np.array_equal(fp8.e4m3_encode(x32), _torch_codes(x32))
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))


def check_rotation_is_the_scaled_hadamard_product(fp8, d):
    import scipy.linalg
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, 5, d)).astype(np.float32)
    s = rng.choice([-1.0, 1.0], d).astype(np.float32)
    y = fp8.wht_fp32(x, s)
    ref = (x.astype(np.float64) * s) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()
    # an orthogonal map: scores of rotated queries and keys are the scores
    q = rng.standard_normal((7, d))
    k = rng.standard_normal((9, d))
    H = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.allclose((q * s) @ H @ ((k * s) @ H).T, q @ k.T, atol=1e-10)
    # two-point closed form: [a, b] -> [a + b, a - b] / sqrt(2)
    y2 = fp8.wht_fp32(np.array([[3.0, 1.0]], np.float32), np.array([1.0, 1.0], np.float32))
    assert np.allclose(y2, [[4 / np.sqrt(2), 2 / np.sqrt(2)]], rtol=1e-6)


def check_block_quantization_closed_forms(fp8):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 100, 64)).astype(np.float32) * 3
    codes, scales = fp8.quantize_blocks(x, 32)
    assert scales.shape == (2, 3, 4)
    for b in range(2):
        for h in range(3):
            for i in range(4):
                blk = x[b, h, 32 * i:32 * (i + 1)]
                amax = np.abs(blk).max()
                assert scales[b, h, i] == np.float32(amax / np.float32(448))
                # the largest element lands on +-448
                j = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                assert codes[b, h, 32 * i + j[0], j[1]] & 0x7F == 0x7E
    deq = fp8.dequantize_blocks(codes, scales, 32)
    # round to nearest: relative error at most 2^-4 for normal values
    big = np.abs(x) > 2.0 ** -6 * scales.repeat(32, axis=2)[:, :, :100, None]
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-7)
    # an all-zero block gets scale 1 and zero codes
    z, zs = fp8.quantize_blocks(np.zeros((1, 1, 8, 64), np.float32), 8)
    assert zs[0, 0, 0] == 1.0 and not z.any()
    # so does a block whose 448 / amax overflows float32 (amax = 2^-122 <
    # 448 / FLT_MAX ~ 2^-119.2), while one just above that limit (2^-119)
    # keeps its scale and puts its largest element on 448
    t = np.zeros((1, 1, 16, 64), np.float32)
    t[0, 0, 3, 5] = -(2.0 ** -122)
    t[0, 0, 8, 9] = 2.0 ** -119
    tc, ts = fp8.quantize_blocks(t, 8)
    assert ts[0, 0, 0] == 1.0 and not tc[0, 0, :8].any()
    assert ts[0, 0, 1] == np.float32(2.0 ** -119) / np.float32(448) and tc[0, 0, 8, 9] == 0x7E


def check_exactly_representable_inputs_give_exact_attention(fp8):
    """When every block already holds e4m3 values times a power of two with
    its largest magnitude at 448 times that power, quantization is exact and
    the FP8 oracle equals the plain attention oracle."""
    import oracle
    rng = np.random.default_rng(8)
    B, H, N, d, br = 1, 2, 96, 64, 32
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)

    def draw(shift):
        codes = rng.choice(finite, size=(B, H, N, d)).astype(np.uint8)
        codes[:, :, ::br, 0] = 0x7E                      # +448 in every block
        return fp8.e4m3_decode(codes) * 2.0 ** shift

    Q, K, V = draw(-9), draw(-8), draw(-3)
    for causal in (False, True):
        O8, L8 = fp8.attention_fp8(Q, K, V, 0.125, causal, block_rows=br)
        O, L = oracle.attention_forward(Q, K, V, 0.125, causal)
        assert np.array_equal(O8, O) and np.array_equal(L8, L)


def check_rotation_lowers_the_error_on_outlier_inputs(fp8):
    """The point of block scales and the rotation: on inputs with rare large
    entries, per-block scales beat one scale per head, and rotating Q and K
    (with the same signs) lowers the error again; on plain N(0, 1) inputs all
    variants stay within the e4m3 rounding level."""
    import math
    import oracle
    import workloads
    B, H, N, d = 1, 2, 512, 128
    sc = 1 / math.sqrt(d)
    s = workloads.make_signs(d, 12).numpy()
    q, k, v = (workloads.to_f64(x) for x in workloads.make_outlier_inputs(B, H, H, N, d, "bf16", 11))
    O, _ = oracle.attention_forward(q, k, v, sc, False)

    def rmse(**kw):
        return float(np.sqrt(np.mean((fp8.attention_fp8(q, k, v, sc, False, **kw)[0] - O) ** 2)))

    e_head, e_block, e_rot = rmse(block_rows=N), rmse(block_rows=64), rmse(block_rows=64, signs=s)
    assert e_block < 0.9 * e_head and e_rot < 0.85 * e_block, (e_head, e_block, e_rot)
    # a rotation applied to K only (a plausible slip) destroys the scores
    qc, qs = fp8.quantize_blocks(q, 64)
    kc, ks = fp8.quantize_blocks(k, 64, s)
    vc, vs = fp8.quantize_blocks(v, 64)
    Obad, _ = oracle.attention_forward(fp8.dequantize_blocks(qc, qs, 64), fp8.dequantize_blocks(kc, ks, 64),
                                       fp8.dequantize_blocks(vc, vs, 64), sc, False)
    assert np.sqrt(np.mean((Obad - O) ** 2)) > 10 * e_rot
    # plain inputs: the relative RMS error stays at the level of the rounding
    # of three operands to 3 mantissa bits (below 2^-3)
    q, k, v = (workloads.to_f64(x) for x in workloads.make_inputs(B, H, H, N, d, "bf16", 13)[:3])
    O, _ = oracle.attention_forward(q, k, v, sc, False)
    O8, _ = fp8.attention_fp8(q, k, v, sc, False, signs=s)
    assert np.sqrt(np.mean((O8 - O) ** 2)) < 2.0 ** -3 * np.sqrt(np.mean(O ** 2))


# ------------------------------------------------------------- the pins --

def test_decode_every_code_matches_torch():
    check_decode_every_code_matches_torch(fp8_real)


def test_encode_round_trip_and_ties_match_torch():
    check_encode_round_trip_and_ties_match_torch(fp8_real)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_the_scaled_hadamard_product(d):
    check_rotation_is_the_scaled_hadamard_product(fp8_real, d)


def test_block_quantization_closed_forms():
    check_block_quantization_closed_forms(fp8_real)


def test_exactly_representable_inputs_give_exact_attention():
    check_exactly_representable_inputs_give_exact_attention(fp8_real)


def test_rotation_lowers_the_error_on_outlier_inputs():
    check_rotation_lowers_the_error_on_outlier_inputs(fp8_real)


# ------------------------------------------------------- planted mistakes --

MUTATIONS = [
    ("exponent bias off by one", "np.exp2(e - 7.0)", "np.exp2(e - 6.0)"),
    ("subnormal step wrong", "sub = m * 2.0 ** -9", "sub = m * 2.0 ** -10"),
    ("ties rounded away from zero", "((dhi == dlo) & (hi % 2 == 0))", "(dhi == dlo)"),
    ("sign of negative zero dropped", "np.where(np.signbit(x), code | 0x80, code)",
     "np.where(x < 0, code | 0x80, code)"),
    ("butterfly difference reversed", "y[..., 1, :] = a - b", "y[..., 1, :] = b - a"),
    ("rotation not normalised", "return y * np.float32(1.0 / np.sqrt(d))", "return y"),
    ("scale inverted", "amax / np.float32(E4M3_MAX)", "np.float32(E4M3_MAX) / amax"),
    ("block rows misaligned", "blk = y[:, :, i * block_rows:(i + 1) * block_rows]",
     "blk = y[:, :, i * block_rows:(i + 1) * block_rows + 1]"),
    ("V rotated too", "vc, vs = quantize_blocks(V, block_rows)", "vc, vs = quantize_blocks(V, block_rows, signs)"),
    ("K left unrotated", "kc, ks = quantize_blocks(K, block_rows, signs)", "kc, ks = quantize_blocks(K, block_rows)"),
]


def _mutant(old, new):
    with open(fp8_real.__file__) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<fp8 mutant>", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    checks = [
        lambda: check_decode_every_code_matches_torch(mod),
        lambda: check_encode_round_trip_and_ties_match_torch(mod),
        lambda: check_rotation_is_the_scaled_hadamard_product(mod, 64),
        lambda: check_block_quantization_closed_forms(mod),
        lambda: check_exactly_representable_inputs_give_exact_attention(mod),
        lambda: check_rotation_lowers_the_error_on_outlier_inputs(mod),
    ]
    for chk in checks:
        try:
            with np.errstate(all="ignore"):
                chk()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _caught(_mutant(old, new)), f"no pin catches: {name}"


def test_unmutated_module_passes_every_check():
    assert not _caught(_mutant("", ""))
