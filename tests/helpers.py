"""Shared test utilities: tolerances, row sampling, and GPU-vs-oracle comparison.

Tolerances (the bar each GPU result must meet against the fp64 oracle):
  float32 inputs             : max |err| <= 1e-5 on O and LSE for unit-variance
                               scores (c = 1/sqrt(d) on N(0,1) inputs).  fp32
                               rounding of a score is proportional to its size, so
                               for larger scores the bound is 1e-5 * c * sqrt(d).
                               Gradients: max |err| <= 1e-5 * max(1, max |oracle|).
  bf16 / fp16 inputs, fp32 acc: max |err| <= 2e-2 on O, <= 1e-3 on LSE,
                               and dQ, dK, dV within 5e-2 normwise-relative error
                               (max |err| / max(max |oracle|, 1e-3) over each
                               (b, h) slice; the floor only matters where the exact
                               gradient is identically zero, e.g. n = 1).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-5
TOL_O_16 = 2e-2
TOL_LSE_16 = 1e-3
TOL_GRAD_16 = 5e-2
# float32 gradients: an absolute bound scaled by the slice's largest value
TOL_GRAD_F32 = 1e-5


def announce(msg: str):
    """Name the case on stderr before a GPU step, flushed, so a crash names it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of fp16/bf16/fp32 values to float64 on the CPU."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_rows(n: int, count: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must if 0 <= r < n)
    if count >= n:
        return np.arange(n)
    while len(rows) < count:
        rows.add(int(rng.integers(0, n)))
    return np.array(sorted(rows), dtype=np.int64)


GRAD_FLOOR = 1e-3


def fwd_tolerances(dtype: torch.dtype, score_scale: float = 1.0):
    """score_scale: c * sqrt(d) * (input std)^2, the std of the scores (1 for the workloads)."""
    if dtype == torch.float32:
        t = TOL_F32 * max(1.0, abs(score_scale))
        return t, t
    return TOL_O_16, TOL_LSE_16


def check_fwd(o_gpu, lse_gpu, y_ref, lse_ref, dtype, what="", score_scale: float = 1.0):
    """o_gpu/lse_gpu: numpy float64 of the GPU outputs at the compared rows."""
    tol_o, tol_l = fwd_tolerances(dtype, score_scale)
    err_o = float(np.max(np.abs(o_gpu - y_ref))) if o_gpu.size else 0.0
    err_l = float(np.max(np.abs(lse_gpu - lse_ref))) if lse_gpu.size else 0.0
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), f"{what}: non-finite"
    assert err_o <= tol_o, f"{what}: O max abs err {err_o:.3g} > {tol_o}"
    assert err_l <= tol_l, f"{what}: LSE max abs err {err_l:.3g} > {tol_l}"
    return err_o, err_l


def check_grad(g_gpu, g_ref, dtype, what="", unit_scores: bool = False):
    """Per (b, h) slice: max |err| / max |ref| (16-bit) or max |err| (fp32).

    float32: 1e-5 * max(1, max |ref|) in general, the flat 1e-5 when
    `unit_scores` (c = 1/sqrt(d) on N(0, 1) rows, the scores of the workloads);
    tests/test_fp32_envelope.py shows a plain float32 evaluation needs the
    scaled form once the scores or gradients are large."""
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite gradient"
    g_gpu = g_gpu.reshape(-1, *g_gpu.shape[-2:])
    g_ref = g_ref.reshape(-1, *g_ref.shape[-2:])
    worst = 0.0
    for s in range(g_gpu.shape[0]):
        err = float(np.max(np.abs(g_gpu[s] - g_ref[s])))
        ref = max(float(np.max(np.abs(g_ref[s]))), GRAD_FLOOR)
        if dtype == torch.float32:
            bound = TOL_GRAD_F32 if unit_scores else TOL_GRAD_F32 * max(1.0, ref)
            assert err <= bound, f"{what}[{s}]: max abs err {err:.3g} > {bound:.3g}"
            worst = max(worst, err / max(1.0, ref))
        else:
            rel = err / ref
            assert rel <= TOL_GRAD_16, f"{what}[{s}]: normwise rel err {rel:.3g} > {TOL_GRAD_16}"
            worst = max(worst, rel)
    return worst


# FP8 scores.  The gfx950 block-scaled FP8 MFMA adds the products of each group
# of 8 consecutive contraction indices (an aligned octet of d) aligned to the
# group's largest product, keeping 13 bits below that product's leading bit
# and dropping the rest (measured on the GPU with one-hot operands: 1 + 2^-13
# is kept, 1 + 2^-14 and 448^2 + 1 are not, in one octet; across octets and
# half-waves the sum is float32).  So a score's error is below
#     delta_ij = |c| * 7 * 2^-13 * sum_octets max_{r in octet} |Qd_ir Kd_jr|
# (the largest product of an octet is exact), and with every score of row i
# off by at most delta_i = max_j delta_ij, LSE moves by at most delta_i and the
# weights by a factor within e^{+-2 delta_i}, so O by at most
# (e^{2 delta_i} - 1) max |V|.  The FP8 forward is held to the 16-bit bar plus
# these amounts.
FP8_GROUP = 8
FP8_KEEP_BITS = 13


def fp8_score_slack(qd: np.ndarray, kd: np.ndarray, c: float, chunk: int = 64) -> np.ndarray:
    """delta_i for dequantized rows qd [nq, d] against keys kd [nk, d]."""
    nq, d = qd.shape
    aq, ak = np.abs(qd), np.abs(kd)
    out = np.zeros(nq)
    for i0 in range(0, nq, chunk):
        p = aq[i0:i0 + chunk, None, :] * ak[None, :, :]
        g = p.reshape(p.shape[0], p.shape[1], d // FP8_GROUP, FP8_GROUP).max(-1).sum(-1)
        out[i0:i0 + chunk] = g.max(-1)
    return abs(c) * (FP8_GROUP - 1) * 2.0 ** -FP8_KEEP_BITS * out


def check_fwd_fp8(o_gpu, lse_gpu, y_ref, lse_ref, dtype, slack, vmax, what=""):
    """check_fwd for FP8 scores; slack [rows] from fp8_score_slack, vmax = max |V|."""
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), f"{what}: non-finite"
    tol_o, tol_l = fwd_tolerances(dtype)
    err_o = np.max(np.abs(o_gpu - y_ref), axis=-1) if o_gpu.size else np.zeros(0)
    err_l = np.abs(lse_gpu - lse_ref)
    bound_o = tol_o + np.expm1(2 * slack) * vmax
    bound_l = tol_l + slack
    assert np.all(err_o <= bound_o), \
        f"{what}: O err {np.max(err_o):.3g} > bound {bound_o[np.argmax(err_o - bound_o)]:.3g}"
    assert np.all(err_l <= bound_l), \
        f"{what}: LSE err {np.max(err_l):.3g} > bound {bound_l[np.argmax(err_l - bound_l)]:.3g}"
    return float(np.max(err_o, initial=0.0)), float(np.max(err_l, initial=0.0))
