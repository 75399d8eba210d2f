"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's formulas: each compares it with a value
printed on a page, a closed form, an invariant, finite differences, or an
independent brute-force evaluation.  They run on the CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

from conftest import GOLDEN

MASKS = [("none", 0), ("causal", 0), ("window", 1), ("window", 3), ("window", 5)]


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Worked examples of "The Arithmetic of Intelligence", ch. 12, "Streaming softmax"
# ---------------------------------------------------------------------------
with open(os.path.join(GOLDEN, "streaming_softmax_examples.json")) as f:
    EXAMPLES = json.load(f)


@pytest.mark.parametrize("ex", EXAMPLES["examples"])
def test_worked_example_streaming(oracle_mod, ex):
    tol = EXAMPLES["printed_tolerance"]
    b1, b2 = ex["blocks"]
    s1 = oracle_mod.summary(b1, np.zeros((len(b1), 1)))
    assert s1[0] == ex["after_first_block"]["m"]
    assert abs(s1[1] - ex["after_first_block"]["l"]) < tol
    s2 = oracle_mod.summary(b2, np.zeros((len(b2), 1)))
    m, l, _ = oracle_mod.merge(s1, s2)
    assert m == ex["final"]["m"]
    assert abs(l - ex["final"]["l"]) < tol
    # the two printed addends of the update
    assert abs(s1[1] * math.exp(s1[0] - m) - ex["rescaled_old"]) < tol
    assert abs(s2[1] * math.exp(s2[0] - m) - ex["new_block"]) < tol
    # exact closed form: sum of e^{s - max} over every score
    allv = b1 + b2
    exact = sum(math.exp(s - max(allv)) for s in allv)
    assert abs(l - exact) < 1e-12
    for term, s in zip(ex["one_shot_terms"], allv):
        assert abs(math.exp(s - max(allv)) - term) < tol


@pytest.mark.parametrize("ex", EXAMPLES["examples"])
def test_worked_example_one_shot_dense(oracle_mod, ex):
    """The dense oracle reproduces the one-shot normaliser: d = 1, q = 1, k_j = s_j, c = 1."""
    tol = EXAMPLES["printed_tolerance"]
    s = np.array(ex["blocks"][0] + ex["blocks"][1], dtype=np.float64)
    n = len(s)
    q = np.ones((n, 1))
    k = s.reshape(n, 1)
    v = np.eye(n)
    y, m, l, lse = oracle_mod.fwd(q, k, v, 1.0, "none")
    assert np.all(m == ex["final"]["m"])
    assert np.all(np.abs(l - ex["one_shot"]) < tol)
    exact = np.exp(s - s.max()).sum()
    assert np.allclose(l, exact, rtol=0, atol=1e-12)
    assert np.allclose(lse, s.max() + math.log(exact), rtol=0, atol=1e-12)
    # rows of P (here Y, since V = I) are the normalised exponentials
    assert np.allclose(y[0], np.exp(s - s.max()) / exact, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Definition "Stable summary of an attention key block": the merge identity
# ---------------------------------------------------------------------------
def test_merge_identity_random_partitions(oracle_mod):
    rng = np.random.default_rng(0)
    for trial in range(50):
        k = int(rng.integers(2, 40))
        dv = int(rng.integers(1, 6))
        s = _rand(rng, k, scale=3.0)
        vr = _rand(rng, k, dv)
        perm = rng.permutation(k)
        cut = int(rng.integers(1, k))
        S, T = perm[:cut], perm[cut:]
        whole = oracle_mod.summary(s, vr)
        a = oracle_mod.summary(s[S], vr[S])
        b = oracle_mod.summary(s[T], vr[T])
        for merged in (oracle_mod.merge(a, b), oracle_mod.merge(b, a)):
            assert merged[0] == whole[0]
            assert abs(merged[1] - whole[1]) <= 1e-12 * whole[1]
            assert np.allclose(merged[2], whole[2], rtol=1e-12, atol=1e-12)


def test_merge_associative(oracle_mod):
    rng = np.random.default_rng(1)
    for trial in range(30):
        parts = [oracle_mod.summary(_rand(rng, 5, scale=4.0), _rand(rng, 5, 3)) for _ in range(3)]
        left = oracle_mod.merge(oracle_mod.merge(parts[0], parts[1]), parts[2])
        right = oracle_mod.merge(parts[0], oracle_mod.merge(parts[1], parts[2]))
        assert left[0] == right[0]
        assert abs(left[1] - right[1]) <= 1e-12 * left[1]
        assert np.allclose(left[2], right[2], rtol=1e-12, atol=1e-12)


def test_summary_single_score(oracle_mod):
    m, l, z = oracle_mod.summary([1.5], [[2.0, -3.0]])
    assert (m, l) == (1.5, 1.0)
    assert np.array_equal(z, [2.0, -3.0])


# ---------------------------------------------------------------------------
# Theorem "Tiled attention ... are exact": tiled forward == dense rows, any b
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mask,window", MASKS)
def test_tiled_equals_dense_any_block(oracle_mod, mask, window):
    rng = np.random.default_rng(2)
    nh, n, d, dv = 3, 37, 5, 4
    q, k, v = _rand(rng, nh, n, d), _rand(rng, nh, n, d), _rand(rng, nh, n, dv)
    c = 0.7
    y, m, l, _ = oracle_mod.fwd(q, k, v, c, mask, window)
    for b in (1, 2, 7, 16, 37, 64):
        yt, mt, lt = oracle_mod.fwd_tiled(q, k, v, c, mask, window, block=b)
        assert np.array_equal(mt, m)
        assert np.allclose(lt, l, rtol=1e-12, atol=0)
        assert np.allclose(yt, y, rtol=1e-11, atol=1e-12)


def test_broken_rescale_control(oracle_mod):
    """Night School, "Forget one step": without shrinking the running total the
    answer is wrong unless the largest score arrives in the first tile."""
    rng = np.random.default_rng(3)
    n, d, dv, b = 32, 4, 3, 8
    q = np.ones((1, n, d))
    v = _rand(rng, 1, n, dv)
    # scores rise along the keys: the row max sits in the last tile
    k_late = np.repeat(np.linspace(-2, 2, n).reshape(1, n, 1), d, axis=2)
    y, _, _, _ = oracle_mod.fwd(q, k_late, v, 1.0, "none")
    yb, _, _ = oracle_mod.fwd_tiled(q, k_late, v, 1.0, "none", block=b, broken=True)
    yg, _, _ = oracle_mod.fwd_tiled(q, k_late, v, 1.0, "none", block=b, broken=False)
    assert np.allclose(yg, y, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(yb - y)) > 1e-2
    # scores fall along the keys: the max is in the first tile, so the broken
    # update coincides with the correct one
    k_early = k_late[:, ::-1, :].copy()
    y2, _, _, _ = oracle_mod.fwd(q, k_early, v, 1.0, "none")
    yb2, _, _ = oracle_mod.fwd_tiled(q, k_early, v, 1.0, "none", block=b, broken=True)
    assert np.allclose(yb2, y2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and invariants of the dense forward
# ---------------------------------------------------------------------------
def _allowed(mask, window, i, j):
    if mask == "none":
        return True
    if mask == "causal":
        return j <= i
    return i - window + 1 <= j <= i


@pytest.mark.parametrize("mask,window", MASKS)
def test_zero_scale_is_mean(oracle_mod, mask, window):
    rng = np.random.default_rng(4)
    n, d, dv = 11, 3, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv)
    y, m, l, lse = oracle_mod.fwd(q, k, v, 0.0, mask, window)
    for i in range(n):
        js = [j for j in range(n) if _allowed(mask, window, i, j)]
        assert np.allclose(y[i], v[js].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(len(js))) < 1e-14
        assert m[i] == 0.0


def test_causal_row_zero_and_window_one(oracle_mod):
    rng = np.random.default_rng(5)
    n, d, dv = 9, 4, 2
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv)
    c = 0.9
    y, m, l, lse = oracle_mod.fwd(q, k, v, c, "causal")
    assert np.array_equal(y[0], v[0])
    assert abs(lse[0] - c * float(q[0] @ k[0])) < 1e-14
    # window of one key: each row sees only itself
    y1, _, l1, lse1 = oracle_mod.fwd(q, k, v, c, "window", 1)
    assert np.array_equal(y1, v)
    assert np.array_equal(l1, np.ones(n))
    assert np.allclose(lse1, c * np.einsum("id,id->i", q, k), rtol=0, atol=1e-14)


def test_window_at_least_n_equals_causal(oracle_mod):
    rng = np.random.default_rng(6)
    n, d, dv = 13, 3, 3
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv)
    yc, _, _, lc = oracle_mod.fwd(q, k, v, 0.5, "causal")
    for w in (n, n + 5):
        yw, _, _, lw = oracle_mod.fwd(q, k, v, 0.5, "window", w)
        assert np.array_equal(yw, yc)
        assert np.array_equal(lw, lc)


@pytest.mark.parametrize("mask,window", MASKS)
def test_key_shift_invariance(oracle_mod, mask, window):
    """Adding 1 u^T to K shifts row i's scores by c q_i.u: Y unchanged, LSE_i += c q_i.u."""
    rng = np.random.default_rng(7)
    n, d, dv, c = 10, 4, 3, 0.6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv)
    u = _rand(rng, d)
    y, _, _, lse = oracle_mod.fwd(q, k, v, c, mask, window)
    y2, _, _, lse2 = oracle_mod.fwd(q, k + u, v, c, mask, window)
    assert np.allclose(y2, y, rtol=0, atol=1e-12)
    assert np.allclose(lse2 - lse, c * q @ u, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", MASKS)
def test_rows_are_distributions_on_allowed_keys(oracle_mod, mask, window):
    """With V = I the output rows are the probabilities: they sum to 1, are
    positive exactly on A_i and zero elsewhere."""
    rng = np.random.default_rng(8)
    n, d = 12, 3
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    y, _, _, _ = oracle_mod.fwd(q, k, np.eye(n), 1.3, mask, window)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    for i in range(n):
        for j in range(n):
            if _allowed(mask, window, i, j):
                assert y[i, j] > 0
            else:
                assert y[i, j] == 0.0


def test_constant_value_column(oracle_mod):
    rng = np.random.default_rng(9)
    n, d = 15, 4
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    v = np.concatenate([np.full((n, 1), 2.5), _rand(rng, n, 2)], axis=1)
    y, _, _, _ = oracle_mod.fwd(q, k, v, 1.1, "causal")
    assert np.allclose(y[:, 0], 2.5, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mask,window", MASKS)
def test_brute_force_unshifted(oracle_mod, mask, window):
    """Independent scalar evaluation (unshifted exponentials, plain Python loops)."""
    rng = np.random.default_rng(10)
    n, d, dv, c = 7, 3, 2, 0.8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv)
    y, _, _, lse = oracle_mod.fwd(q, k, v, c, mask, window)
    for i in range(n):
        num = [0.0] * dv
        den = 0.0
        for j in range(n):
            if not _allowed(mask, window, i, j):
                continue
            e = math.exp(c * sum(q[i, r] * k[j, r] for r in range(d)))
            den += e
            for a in range(dv):
                num[a] += e * v[j, a]
        assert np.allclose(y[i], [x / den for x in num], rtol=1e-12, atol=1e-13)
        assert abs(lse[i] - math.log(den)) < 1e-12


def test_row_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(11)
    nh, n, d, dv = 2, 20, 4, 3
    q, k, v = _rand(rng, nh, n, d), _rand(rng, nh, n, d), _rand(rng, nh, n, dv)
    y, m, l, lse = oracle_mod.fwd(q, k, v, 0.5, "window", 6)
    rows = [19, 0, 5, 6, 7]
    ys, ms, ls, lses = oracle_mod.fwd(q, k, v, 0.5, "window", 6, rows=rows)
    assert np.array_equal(ys, y[:, rows])
    assert np.array_equal(lses, lse[:, rows])


def test_large_scores_do_not_overflow(oracle_mod):
    """Max shift: scores far beyond exp's double range still give finite rows."""
    n, d = 6, 1
    q = np.ones((n, d))
    k = np.array([[800.0], [799.0], [-800.0], [790.0], [801.0], [0.0]])
    v = np.arange(n, dtype=np.float64).reshape(n, 1)
    y, m, l, lse = oracle_mod.fwd(q, k, v, 1.0, "none")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(lse))
    e = np.exp(k[:, 0] - 801.0)
    assert np.allclose(y[:, 0], (e * v[:, 0]).sum() / e.sum(), rtol=1e-14)
    assert np.allclose(lse, 801.0 + math.log(e.sum()), rtol=0, atol=1e-12)


def test_fp16_overflow_facts():
    """Night School, "Why keep the largest": the fp16 limits behind the overflow workload."""
    with open(os.path.join(GOLDEN, "fp16_overflow_facts.json")) as f:
        facts = json.load(f)
    fmax = facts["fp16_max"]
    assert float(np.finfo(np.float16).max) == fmax
    assert round(math.log(facts["fits"]["exp_printed"]), 2) == facts["fits"]["score"]
    assert facts["fits"]["exp_printed"] < fmax
    assert math.exp(facts["would_overflow_score"]) > fmax
    assert math.exp(facts["held_out_max_score"]) > fmax


def test_invalid_arguments(oracle_mod):
    q = np.zeros((2, 2))
    with pytest.raises(RuntimeError):
        oracle_mod.fwd(q, q, q, 1.0, "window", 0)
    with pytest.raises(RuntimeError):
        oracle_mod.fwd(q, q, q, 1.0, "none", rows=[2])


# ---------------------------------------------------------------------------
# Reverse procedure: finite differences and gradient invariants
# ---------------------------------------------------------------------------
def _phi(oracle_mod, q, k, v, g, c, mask, window):
    y, _, _, _ = oracle_mod.fwd(q, k, v, c, mask, window)
    return float((g * y).sum())


@pytest.mark.parametrize("mask,window", MASKS)
@pytest.mark.parametrize("d,dv", [(1, 1), (2, 3), (3, 2), (8, 8)])
def test_vjp_finite_differences(oracle_mod, mask, window, d, dv):
    rng = np.random.default_rng(100 + d * 10 + dv)
    n, c = 6 if d == 8 else 9, 0.75
    q, k, v, g = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv), _rand(rng, n, dv)
    dq, dk, dvv, y, delta, lse = oracle_mod.bwd(q, k, v, g, c, mask, window)
    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _phi(oracle_mod, args["q"], args["k"], args["v"], g, c, mask, window)
            args[name] = xm
            fm = _phi(oracle_mod, args["q"], args["k"], args["v"], g, c, mask, window)
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), name


def test_vjp_finite_differences_n16(oracle_mod):
    rng = np.random.default_rng(200)
    n, d, dv, c = 16, 2, 2, 1.0
    q, k, v, g = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv), _rand(rng, n, dv)
    dq, dk, dvv, _, _, _ = oracle_mod.bwd(q, k, v, g, c, "causal")
    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        for idx in list(np.ndindex(x.shape))[::3]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _phi(oracle_mod, args["q"], args["k"], args["v"], g, c, "causal", 0)
            args[name] = xm
            fm = _phi(oracle_mod, args["q"], args["k"], args["v"], g, c, "causal", 0)
            assert abs(grad[idx] - (fp - fm) / (2 * h)) < 1e-7


@pytest.mark.parametrize("mask,window", MASKS)
def test_vjp_invariants(oracle_mod, mask, window):
    rng = np.random.default_rng(12)
    nh, n, d, dv, c = 2, 24, 5, 3, 0.9
    q, k, v, g = (_rand(rng, nh, n, d), _rand(rng, nh, n, d), _rand(rng, nh, n, dv),
                  _rand(rng, nh, n, dv))
    dq, dk, dvv, y, delta, lse = oracle_mod.bwd(q, k, v, g, c, mask, window)
    # score-gradient rows sum to zero, so the key gradients sum to zero
    assert np.allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
    # each probability row sums to one, so the value gradients sum to sum_i G_i
    assert np.allclose(dvv.sum(axis=1), g.sum(axis=1), rtol=0, atol=1e-12)
    # s_ij = c q_i.k_j is bilinear: <Q, dQ> = <K, dK> = sum_ij gamma_ij s_ij
    assert np.allclose(np.einsum("hnd,hnd->h", q, dq), np.einsum("hnd,hnd->h", k, dk),
                       rtol=1e-10, atol=1e-12)
    # the forward outputs returned alongside agree with the dense forward
    y2, _, _, lse2 = oracle_mod.fwd(q, k, v, c, mask, window)
    assert np.array_equal(y, y2)
    assert np.allclose(lse, lse2, rtol=0, atol=0)
    assert np.allclose(delta, (g * y).sum(axis=-1), rtol=1e-14, atol=1e-14)


def test_vjp_value_gradient_zero_scale(oracle_mod):
    """c = 0: p_ij = 1/|A_i|, so dV_j = sum_{i: j in A_i} G_i / |A_i| and dQ = dK = 0."""
    rng = np.random.default_rng(13)
    n, d, dv = 8, 2, 2
    q, k, v, g = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, dv), _rand(rng, n, dv)
    dq, dk, dvv, _, _, _ = oracle_mod.bwd(q, k, v, g, 0.0, "causal")
    assert np.array_equal(dq, np.zeros_like(dq)) and np.array_equal(dk, np.zeros_like(dk))
    for j in range(n):
        exp_dv = sum(g[i] / (i + 1) for i in range(j, n))
        assert np.allclose(dvv[j], exp_dv, rtol=0, atol=1e-14)
