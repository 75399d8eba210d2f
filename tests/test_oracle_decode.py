"""Pins of the oracle's decode-shaped forward (new rows against a key/value cache).

The rows are the last nq positions of a sequence whose nk keys and values are all
cached (the KV-cache setting of the Principia page "Bellek Duvarinin Fizigi",
section on the KV cache and long context); H query heads share Hkv key/value
heads.  Each test checks the oracle against something other than itself: an
independent brute-force loop, the (already pinned) full forward on the whole
sequence, the key/value-head sharing written out as repetition, a closed form,
and the merge identity of alphabetamath.cc's Definition "Stable summary of an
attention key block" over a split of the cache.  CPU only.
"""
import itertools
import math

import numpy as np
import pytest

CASES = [
    # B, H, Hkv, nq, nk, d, mask, window
    (1, 1, 1, 1, 5, 4, "none", 0),
    (2, 4, 2, 3, 7, 3, "causal", 0),
    (1, 6, 3, 2, 9, 5, "window", 3),
    (2, 4, 1, 4, 4, 2, "causal", 0),
    (1, 8, 2, 1, 6, 4, "window", 1),
    (1, 2, 2, 5, 11, 3, "window", 20),
]


def _inputs(seed, B, H, Hkv, nq, nk, d, dv=None, scale=0.7):
    rng = np.random.default_rng(seed)
    dv = dv or d
    q = rng.standard_normal((B, H, nq, d)) * scale
    k = rng.standard_normal((B, Hkv, nk, d)) * scale
    v = rng.standard_normal((B, Hkv, nk, dv))
    return q, k, v


def _allowed(mask, window, p, j):
    if mask == "none":
        return True
    if mask == "causal":
        return j <= p
    return p - window + 1 <= j <= p


@pytest.mark.parametrize("case", CASES)
def test_decode_brute_force(oracle_mod, case):
    """Scalar loops with unshifted exponentials (safe at these sizes)."""
    B, H, Hkv, nq, nk, d, mask, window = case
    q, k, v = _inputs(11, B, H, Hkv, nq, nk, d, dv=d + 1)
    c = 0.9
    y, lse = oracle_mod.decode(q, k, v, c, mask, window)
    G = H // Hkv
    for b, h, i in itertools.product(range(B), range(H), range(nq)):
        p = nk - nq + i
        hk = h // G
        wsum, acc = 0.0, [0.0] * (d + 1)
        for j in range(nk):
            if not _allowed(mask, window, p, j):
                continue
            s = c * sum(q[b, h, i, r] * k[b, hk, j, r] for r in range(d))
            w = math.exp(s)
            wsum += w
            for a in range(d + 1):
                acc[a] += w * v[b, hk, j, a]
        for a in range(d + 1):
            assert abs(y[b, h, i, a] - acc[a] / wsum) < 1e-12
        assert abs(lse[b, h, i] - math.log(wsum)) < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_decode_is_suffix_of_full_forward(oracle_mod, case):
    """The nq new rows are the last rows of the full forward over all nk positions."""
    B, H, Hkv, nq, nk, d, mask, window = case
    q, k, v = _inputs(12, B, H, Hkv, nq, nk, d)
    G = H // Hkv
    y, lse = oracle_mod.decode(q, k, v, 0.6, mask, window)
    rng = np.random.default_rng(5)
    for b, h in itertools.product(range(B), range(H)):
        qfull = rng.standard_normal((nk, d))
        qfull[nk - nq:] = q[b, h]
        yf, _, _, lf = oracle_mod.fwd(qfull, k[b, h // G], v[b, h // G], 0.6, mask, window)
        np.testing.assert_allclose(y[b, h], yf[nk - nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b, h], lf[nk - nq:], rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", [c for c in CASES if c[1] != c[2]])
def test_decode_shared_heads_equal_repetition(oracle_mod, case):
    """Query head h reads key/value head h // (H / Hkv): same as repeating each
    key/value head H / Hkv times and giving every query head its own."""
    B, H, Hkv, nq, nk, d, mask, window = case
    q, k, v = _inputs(13, B, H, Hkv, nq, nk, d)
    G = H // Hkv
    y, lse = oracle_mod.decode(q, k, v, 1.1, mask, window)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    y2, lse2 = oracle_mod.decode(q, kr, vr, 1.1, mask, window)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("case", CASES)
def test_decode_zero_scale_closed_form(oracle_mod, case):
    """c = 0: every allowed key has weight 1, so Y is the mean of the allowed V
    rows and LSE = ln |A_i|."""
    B, H, Hkv, nq, nk, d, mask, window = case
    q, k, v = _inputs(14, B, H, Hkv, nq, nk, d)
    G = H // Hkv
    y, lse = oracle_mod.decode(q, k, v, 0.0, mask, window)
    for b, h, i in itertools.product(range(B), range(H), range(nq)):
        p = nk - nq + i
        js = [j for j in range(nk) if _allowed(mask, window, p, j)]
        np.testing.assert_allclose(y[b, h, i], v[b, h // G, js].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[b, h, i] - math.log(len(js))) < 1e-14


@pytest.mark.parametrize("split", [[3], [1, 1, 4], [2, 5], [6]])
def test_decode_split_cache_merge(oracle_mod, split):
    """Summaries of consecutive key ranges of the cache, merged left to right,
    give the row exactly: z / l = Y and m + ln l = LSE (the split-KV identity)."""
    nq, nk, d = 2, 9, 4
    q, k, v = _inputs(15, 1, 1, 1, nq, nk, d)
    c = 0.8
    y, lse = oracle_mod.decode(q, k, v, c, "causal")
    bounds = np.cumsum([0] + split + [nk])
    bounds = [int(x) for x in bounds if x <= nk]
    if bounds[-1] != nk:
        bounds.append(nk)
    for i in range(nq):
        p = nk - nq + i
        state = None
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            js = [j for j in range(lo, hi) if j <= p]
            if not js:
                continue
            s = np.array([c * float(q[0, 0, i] @ k[0, 0, j]) for j in js])
            part = oracle_mod.summary(s, v[0, 0, js])
            state = part if state is None else oracle_mod.merge(state, part)
        m, l, z = state
        np.testing.assert_allclose(z / l, y[0, 0, i], rtol=0, atol=1e-13)
        assert abs(m + math.log(l) - lse[0, 0, i]) < 1e-13


def test_decode_rejects_bad_shapes(oracle_mod):
    q, k, v = _inputs(16, 1, 3, 2, 2, 4, 2)
    with pytest.raises(RuntimeError):
        oracle_mod.decode(q, k, v, 1.0)  # 3 query heads do not split over 2
    q, k, v = _inputs(16, 1, 2, 2, 5, 4, 2)
    with pytest.raises(RuntimeError):
        oracle_mod.decode(q, k, v, 1.0)  # more new rows than cached keys
