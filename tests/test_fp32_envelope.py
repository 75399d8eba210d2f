"""The float32 tolerance reading, pinned on the CPU.

The parity bar for float32 inputs is a max-abs error of 1e-5 for unit-variance
scores (c = 1/sqrt(d) on N(0, 1) rows), scaled to 1e-5 * c * sqrt(d) for larger
scores and to 1e-5 * max(1, max |exact|) for gradients.  The reason is that
float32 rounding of a score s_ij = c q_i . k_j is proportional to its size, and
the weights e^{s - m} carry that absolute score error as a relative one.

These tests evaluate the dense definition (and its VJP) in plain float32 --
products added in index order, one rounding per operation, no blocking -- on
the very inputs of the float32 GPU parity tests, and compare with the fp64
oracle: a faithful float32 evaluation exceeds a flat 1e-5 as soon as the scores
are large, and stays inside the scaled bounds.  The GPU kernels accumulate in
float32 as well, so the scaled bounds are float32's own envelope, not a bound
fitted to the kernels.
"""
import numpy as np
import pytest

from exact_io_aware_tiled_amd.inputs import Workload, make_inputs
from helpers import TOL_F32, TOL_GRAD_F32

F = np.float32


def seqdot(a, b):
    """a [n, k] . b[m, k]^T in float32, the k products added in index order."""
    acc = np.zeros((a.shape[0], b.shape[0]), F)
    for r in range(a.shape[1]):
        acc = (acc + (a[:, r:r + 1] * b[None, :, r]).astype(F)).astype(F)
    return acc


def allowed(n, mask):
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    return np.ones((n, n), bool) if mask == "none" else j <= i


def f32_forward(q, k, v, c, mask):
    """Row softmax attention of one head evaluated in float32."""
    q, k, v = (x.astype(F) for x in (q, k, v))
    n = q.shape[0]
    s = np.where(allowed(n, mask), (F(c) * seqdot(q, k)).astype(F), F(-np.inf))
    m = s.max(1, keepdims=True)
    p = np.exp(s - m).astype(F)
    l = np.zeros((n, 1), F)
    for j in range(n):
        l = (l + p[:, j:j + 1]).astype(F)
    o = (seqdot(p, v.T.copy()) / l).astype(F)
    return o, (m[:, 0] + np.log(l[:, 0])).astype(F), p / l


def f32_vjp(q, k, v, do, c, mask):
    """dQ, dK, dV of sum(dO * O) for one head, evaluated in float32."""
    q, k, v, do = (x.astype(F) for x in (q, k, v, do))
    o, _, p = f32_forward(q, k, v, c, mask)
    p = p.astype(F)
    delta = np.zeros((q.shape[0], 1), F)
    for a in range(do.shape[1]):
        delta = (delta + (do[:, a:a + 1] * o[:, a:a + 1]).astype(F)).astype(F)
    ds = (p * (seqdot(do, v) - delta)).astype(F)
    dq = (F(c) * seqdot(ds, k.T.copy())).astype(F)
    dk = (F(c) * seqdot(ds.T.copy(), q.T.copy())).astype(F)
    dv = seqdot(p.T.copy(), do.T.copy())
    return dq, dk, dv


def fwd_errors(oracle_mod, c, seed=17):
    """Max errors of the float32 evaluation on the inputs of the float32 forward
    scale test (1 x 2 x 150 x 64, causal)."""
    w = Workload("scale", 1, 2, 150, 64, 64, "f32", "causal", scale=c, seed=seed)
    inp = make_inputs(w)
    q, k, v = (inp[x].double().numpy() for x in ("q", "k", "v"))
    y, _, _, lref = oracle_mod.fwd(q, k, v, c, "causal")
    eo = el = 0.0
    for h in range(2):
        o32, l32, _ = f32_forward(q[0, h], k[0, h], v[0, h], c, "causal")
        eo = max(eo, float(np.abs(o32 - y[0, h]).max()))
        el = max(el, float(np.abs(l32 - lref[0, h]).max()))
    return eo, el


def test_unit_variance_scores_meet_flat_bound(oracle_mod):
    eo, el = fwd_errors(oracle_mod, 1.0 / 8.0)
    assert eo <= TOL_F32 and el <= TOL_F32, (eo, el)


def test_large_scores_exceed_flat_bound_within_scaled(oracle_mod):
    """c = 1 at d = 64: scores eight times unit variance.  The float32
    evaluation's O error is above 1e-5 (a flat bound would reject it) and
    below 1e-5 * c * sqrt(d)."""
    c = 1.0
    eo, el = fwd_errors(oracle_mod, c)
    scaled = TOL_F32 * c * 64 ** 0.5
    assert eo > TOL_F32, eo
    assert eo <= scaled and el <= scaled, (eo, el, scaled)
    # the scaled bound is of the size of the error, not far above it
    assert eo >= 0.1 * scaled


def test_negative_scale_within_scaled(oracle_mod):
    eo, el = fwd_errors(oracle_mod, -0.3)
    scaled = TOL_F32 * max(1.0, 0.3 * 64 ** 0.5)
    assert eo <= scaled and el <= scaled, (eo, el, scaled)


@pytest.mark.parametrize("case", ["scale-0.4", "unit"])
def test_gradient_envelope(oracle_mod, case):
    """The float32 backward scale test's inputs (c = -0.4, 1 x 2 x 150 x 64,
    causal): the float32 VJP's error exceeds a flat 1e-5 where the gradients
    are large, and stays below 1e-5 * max(1, max |exact|) per slice.  On a
    unit-variance case (c = 1/8) it stays below the flat 1e-5 as well."""
    if case == "unit":
        w = Workload("u", 1, 2, 150, 64, 64, "f32", "causal", seed=43)
    else:
        w = Workload("scale", 1, 2, 150, 64, 64, "f32", "causal", scale=-0.4, seed=43)
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].double().numpy() for x in ("q", "k", "v", "do"))
    refs = oracle_mod.bwd(q, k, v, do, w.c, "causal")[:3]
    worst_flat = 0.0
    for h in range(2):
        got = f32_vjp(q[0, h], k[0, h], v[0, h], do[0, h], w.c, "causal")
        for g, ref in zip(got, refs):
            err = float(np.abs(g - ref[0, h]).max())
            bound = TOL_GRAD_F32 * max(1.0, float(np.abs(ref[0, h]).max()))
            assert err <= bound, (err, bound)
            worst_flat = max(worst_flat, err)
    if case == "unit":
        assert worst_flat <= TOL_GRAD_F32
    else:
        assert worst_flat > TOL_GRAD_F32
