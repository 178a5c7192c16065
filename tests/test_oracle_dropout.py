"""The dropout oracle against facts outside itself (CPU only): numpy's Philox
bit generator, a pure-Python brute force with its own scalar generator, the
plain attention oracle at p = 0, keep statistics and finite differences."""
from __future__ import annotations

import types

import numpy as np
import pytest

import oracle
import oracle.dropout as drop_real

MASK64 = (1 << 64) - 1


def _scalar_philox(ctr, key):
    """Philox4x64-10 on Python integers (the 128-bit products are exact)."""
    M0, M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
    W0, W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    for _ in range(10):
        p0, p1 = M0 * c0, M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & MASK64)
        k0, k1 = (k0 + W0) & MASK64, (k1 + W1) & MASK64
    return c0, c1, c2, c3


def _brute_byte(bh, i, j, seed, offset):
    words = _scalar_philox((j // 32, i, bh, 0), (seed, offset))
    t = j % 32
    return (words[t // 8] >> (8 * (t % 8))) & 0xFF


def _brute_forward(Q, K, V, scale, causal, p, seed, offset):
    B, Hq, N, d = Q.shape
    G = Hq // K.shape[1]
    t = int(np.floor((1 - p) * 256 + 0.5))
    O = np.zeros((B, Hq, N, d))
    for b in range(B):
        for h in range(Hq):
            for i in range(N):
                js = [j for j in range(N) if not causal or j <= i]
                s = [scale * sum(Q[b, h, i, c] * K[b, h // G, j, c] for c in range(d)) for j in js]
                m = max(s)
                e = [np.exp(x - m) for x in s]
                z = sum(e)
                for jj, j in enumerate(js):
                    if _brute_byte(b * Hq + h, i, j, seed, offset) < t:
                        O[b, h, i] += (e[jj] / z) * (256.0 / t) * V[b, h // G, j]
    return O


# ------------------------------------------------------------ check functions

def check_philox_matches_numpy(mod):
    rng = np.random.default_rng(1)
    for _ in range(20):
        ctr = [int(x) for x in rng.integers(0, 2 ** 64 - 1, 4, dtype=np.uint64)]
        key = [int(x) for x in rng.integers(0, 2 ** 64 - 1, 2, dtype=np.uint64)]
        out = mod.philox4x64([np.uint64(c) for c in ctr], key)
        full = sum(c << (64 * i) for i, c in enumerate(ctr))
        # numpy advances its counter before each block
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=(full - 1) % (1 << 256))
        assert [int(x) for x in out] == [int(x) for x in bg.random_raw(4)]


def check_bytes_match_scalar_definition(mod):
    rows = np.array([0, 1, 7, 300])
    by = mod.random_bytes(5, rows, 70, 1234, 99)
    for a, i in enumerate(rows):
        for j in (0, 1, 7, 8, 31, 32, 33, 63, 64, 69):
            assert by[a, j] == _brute_byte(5, int(i), j, 1234, 99), (i, j)


def check_brute_force(mod):
    rng = np.random.default_rng(2)
    for causal in (False, True):
        for (B, Hq, Hkv, N, d, p) in ((1, 2, 1, 37, 4, 0.3), (2, 1, 1, 9, 3, 0.1)):
            Q, K, V = (rng.standard_normal((B, h, N, d)) for h in (Hq, Hkv, Hkv))
            O, lse = mod.attention_forward_dropout(Q, K, V, 0.5, causal, p, 77, 5)
            assert np.allclose(O, _brute_forward(Q, K, V, 0.5, causal, p, 77, 5), atol=1e-12)
            _, lse0 = oracle.attention_forward(Q, K, V, 0.5, causal)
            assert np.allclose(lse, lse0, atol=1e-12)


def check_no_dropout_is_plain_attention(mod):
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((1, 2, 50, 8)) for _ in range(3))
    for causal in (False, True):
        O, lse = mod.attention_forward_dropout(Q, K, V, 0.3, causal, 0.0, 1, 2)
        O0, lse0 = oracle.attention_forward(Q, K, V, 0.3, causal)
        assert np.array_equal(O, O0) and np.array_equal(lse, lse0)
    assert mod.keep_threshold(0.0) == 256 and mod.keep_threshold(0.1) == 230
    with pytest.raises(ValueError):
        mod.keep_threshold(0.999)


def check_keep_statistics(mod):
    for p in (0.1, 0.5):
        Z = mod.keep_mask(1, 2, 256, 512, p, 42, 0)
        t = mod.keep_threshold(p)
        n = Z.size
        q = t / 256
        assert abs(Z.mean() - q) < 5 * np.sqrt(q * (1 - q) / n)
    # different offsets give different masks
    assert (mod.keep_mask(1, 1, 64, 64, 0.5, 42, 0) != mod.keep_mask(1, 1, 64, 64, 0.5, 42, 1)).mean() > 0.3


def check_finite_differences(mod):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, N, d = 1, 2, 1, 12, 4
    Q, K, V = (rng.standard_normal((B, h, N, d)) for h in (Hq, Hkv, Hkv))
    dO = rng.standard_normal((B, Hq, N, d))
    for causal in (False, True):
        _, _, dQ, dK, dV = mod.attention_backward_dropout(Q, K, V, dO, 0.4, causal, 0.25, 9, 3)

        def f(Q_, K_, V_):
            return float((mod.attention_forward_dropout(Q_, K_, V_, 0.4, causal, 0.25, 9, 3)[0] * dO).sum())

        eps = 1e-6
        for X, G_ in ((Q, dQ), (K, dK), (V, dV)):
            for idx in [(0, 0, 3, 1), (0, 0, 11, 2), (0, X.shape[1] - 1, 0, 0), (0, X.shape[1] - 1, 7, 3)]:
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += eps
                Xm[idx] -= eps
                args_p = [Xp if Y is X else Y for Y in (Q, K, V)]
                args_m = [Xm if Y is X else Y for Y in (Q, K, V)]
                num = (f(*args_p) - f(*args_m)) / (2 * eps)
                assert abs(num - G_[idx]) < 1e-6 * max(1.0, abs(num)), (causal, idx, num, G_[idx])


CHECKS = [check_philox_matches_numpy, check_bytes_match_scalar_definition, check_brute_force,
          check_no_dropout_is_plain_attention, check_keep_statistics, check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check(drop_real)


# ------------------------------------------------------- planted mistakes --

MUTATIONS = [
    ("carry of the middle products dropped", "+ (mid >> _S32)", ""),
    ("key not advanced", "k0 = k0 + np.uint64(PHILOX_W[0])", "k0 = k0"),
    ("multiplier outputs swapped", "c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]",
     "c = [hi0 ^ c[1] ^ k0, lo1, hi1 ^ c[3] ^ k1, lo0]"),
    ("row and key block swapped in the counter", "c0 = np.broadcast_to(blk[None, :], (len(rows), nblk))\n"
     "    c1 = np.broadcast_to(rows[:, None], (len(rows), nblk))",
     "c1 = np.broadcast_to(blk[None, :], (len(rows), nblk))\n"
     "    c0 = np.broadcast_to(rows[:, None], (len(rows), nblk))"),
    ("big-endian bytes", 'words.astype("<u8")', 'words.astype(">u8")'),
    ("threshold inclusive", "Z = random_bytes(b * Hq + h, rows, N, seed, offset) < t",
     "Z = random_bytes(b * Hq + h, rows, N, seed, offset) <= t"),
    ("scale 1 / (1 - p)", "return 256.0 / keep_threshold(p)", "return 1.0 / (1.0 - p)"),
    ("mask left out of dP", "dP = (dor @ Vh.T) * Zs", "dP = (dor @ Vh.T)"),
    ("D from the undropped output", "D = (dor * Or).sum(axis=1, keepdims=True)",
     "D = (dor * (P @ Vh)).sum(axis=1, keepdims=True)"),
    ("dV from the undropped probabilities", "dV[b, hk] += Pd.T @ dor", "dV[b, hk] += P.T @ dor"),
]


def _mutant(old, new):
    with open(drop_real.__file__) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle.dropout_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<dropout mutant>", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    for chk in CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _caught(_mutant(old, new)), f"no pin catches: {name}"


def test_unmutated_module_passes_every_check():
    assert not _caught(_mutant("", ""))
