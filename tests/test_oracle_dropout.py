"""Pins of the oracle's dropout extension.

alphabetamath.cc, "Exact tiled attention and memory-aware differentiation"
(Algorithm, reverse procedure; Remark on rounding) fixes only the requirement:
the base method has no dropout, and an extension must replay the same realized
mask in its reverse pass.  The oracle's reading: inverted dropout on the
normalized weights with a mask drawn from the 32-bit xxHash function (XXH32)
keyed on (seed, head, row, 4-key group).  These tests check it against things
other than itself: the xxhash library's XXH32, the undropped oracle (no weight
dropped), central finite differences of the dropped function (the mask held
fixed), a brute-force loop, and the keep rate.  CPU only.
"""
import itertools
import math

import numpy as np
import pytest
import xxhash

MASKS = [("none", 0), ("causal", 0), ("window", 3)]


def lib_xxh32(words, seed):
    return xxhash.xxh32_intdigest(np.asarray(words, dtype="<u4").tobytes(), seed=seed & 0xFFFFFFFF)


def lib_keep(seed, thr, bh, i, j):
    """The mask definition evaluated with the library's XXH32."""
    row_key = lib_xxh32([seed >> 32, bh, i], seed)
    u = lib_xxh32([j >> 2], row_key)
    return ((u >> (8 * (j & 3))) & 0xFF) >= thr


def test_xxh32_matches_library(oracle_mod):
    rng = np.random.default_rng(0)
    for _ in range(300):
        nw = int(rng.integers(0, 4))
        words = [int(x) for x in rng.integers(0, 2**32, nw, dtype=np.uint64)]
        seed = int(rng.integers(0, 2**32))
        assert oracle_mod.xxh32_words(words, seed) == lib_xxh32(words, seed)


def test_keep_matches_library_definition(oracle_mod):
    rng = np.random.default_rng(1)
    for _ in range(2000):
        seed = int(rng.integers(0, 2**63))
        thr = int(rng.integers(0, 256))
        bh, i, j = (int(x) for x in rng.integers(0, 5000, 3))
        assert oracle_mod.dropout_keep(seed, thr, bh, i, j) == lib_keep(seed, thr, bh, i, j)


@pytest.mark.parametrize("thr", [1, 26, 128, 230])
def test_keep_rate(oracle_mod, thr):
    """The kept fraction over a 256 x 256 block is 1 - thr / 256 within 5 sigma."""
    n = 256 * 256
    kept = sum(oracle_mod.dropout_keep(99, thr, 3, i, j) for i in range(256) for j in range(256))
    p = 1 - thr / 256
    assert abs(kept / n - p) < 5 * math.sqrt(p * (1 - p) / n)


def _inputs(seed, nh, n, d, dv):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((nh, n, d)) * 0.8, rng.standard_normal((nh, n, d)) * 0.8,
            rng.standard_normal((nh, n, dv)), rng.standard_normal((nh, n, dv)))


@pytest.mark.parametrize("mask,win", MASKS)
def test_nothing_dropped_equals_base(oracle_mod, mask, win):
    """thr = 0 keeps every weight with factor 1: the undropped oracle exactly."""
    q, k, v, g = _inputs(2, 2, 11, 3, 4)
    y, lse = oracle_mod.fwd_drop(q, k, v, 0.7, mask, win, seed=5, thr=0)
    y0, _, _, l0 = oracle_mod.fwd(q, k, v, 0.7, mask, win)
    np.testing.assert_array_equal(y, y0)
    np.testing.assert_array_equal(lse, l0)
    got = oracle_mod.bwd_drop(q, k, v, g, 0.7, mask, win, seed=5, thr=0)
    ref = oracle_mod.bwd(q, k, v, g, 0.7, mask, win)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("mask,win", MASKS)
def test_forward_brute_force(oracle_mod, mask, win):
    """Scalar loops: unshifted exponentials, the library's mask, LSE undropped."""
    q, k, v, _ = _inputs(3, 2, 9, 3, 2)
    seed, thr, c = 1234567890123, 77, 0.9
    y, lse = oracle_mod.fwd_drop(q, k, v, c, mask, win, seed=seed, thr=thr)
    for h, i in itertools.product(range(2), range(9)):
        js = [j for j in range(9) if mask == "none" or (j <= i and (mask == "causal" or j > i - win))]
        w = {j: math.exp(c * float(q[h, i] @ k[h, j])) for j in js}
        tot = sum(w.values())
        ref = sum(w[j] / tot * (256 / (256 - thr) if lib_keep(seed, thr, h, i, j) else 0.0) * v[h, j]
                  for j in js)
        np.testing.assert_allclose(y[h, i], ref, rtol=0, atol=1e-12)
        assert abs(lse[h, i] - math.log(tot)) < 1e-12


@pytest.mark.parametrize("mask,win", MASKS)
def test_backward_finite_differences(oracle_mod, mask, win):
    """The VJP of sum(G * Y) with the mask held fixed (the replayed realized mask)
    against central differences of the fp64 forward."""
    nh, n, d, dv = 1, 10, 3, 2
    q, k, v, g = _inputs(4, nh, n, d, dv)
    seed, thr, c = 42, 90, 0.8
    dq, dk, dvv, _, _, _ = oracle_mod.bwd_drop(q, k, v, g, c, mask, win, seed=seed, thr=thr)

    def phi(q_, k_, v_):
        y, _ = oracle_mod.fwd_drop(q_, k_, v_, c, mask, win, seed=seed, thr=thr)
        return float(np.sum(g * y))

    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (phi(**{a + "_": b for a, b in args_p.items()})
                        - phi(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-8, err_msg=name)


def test_mask_depends_on_every_key_part(oracle_mod):
    """Seed, head, row and key each change the realized mask."""
    base = [oracle_mod.dropout_keep(7, 128, 1, 2, j) for j in range(64)]
    for kw in ({"seed": 8}, {"bh": 2}, {"i": 3}):
        args = {"seed": 7, "bh": 1, "i": 2}
        args.update(kw)
        other = [oracle_mod.dropout_keep(args["seed"], 128, args["bh"], args["i"], j)
                 for j in range(64)]
        assert other != base, kw
    hi = [oracle_mod.dropout_keep(7 + (1 << 40), 128, 1, 2, j) for j in range(64)]
    assert hi != base  # the high seed word is part of the row key


def test_head_offset_selects_the_head(oracle_mod):
    """bh0 + h is the mask's head: the second of two heads equals that head alone at bh0 = 1."""
    q, k, v, g = _inputs(6, 2, 12, 3, 3)
    y2, l2 = oracle_mod.fwd_drop(q, k, v, 0.5, "causal", seed=9, thr=100)
    y1, l1 = oracle_mod.fwd_drop(q[1:], k[1:], v[1:], 0.5, "causal", seed=9, thr=100, bh0=1)
    np.testing.assert_array_equal(y2[1:], y1)
    b2 = oracle_mod.bwd_drop(q, k, v, g, 0.5, "causal", seed=9, thr=100)
    b1 = oracle_mod.bwd_drop(q[1:], k[1:], v[1:], g[1:], 0.5, "causal", seed=9, thr=100, bh0=1)
    for a, b in zip(b2, b1):
        np.testing.assert_array_equal(a[1:], b)
