"""Pins of the oracle's block-scaled FP8 quantizer.

webturing.com.tr Principia, "Bellek Duvarinin Fizigi", section on
FlashAttention-3, names FP8 scores with block scaling and incoherent processing
(random sign multipliers) and fixes nothing more.  The oracle's reading: rows
rotated as H (s * x), H the unnormalized Sylvester Walsh-Hadamard matrix, then
OCP-microscaling blocks of 32 values with a power-of-two scale 2^e (e the least
with max |x| <= 448 2^e) and e4m3 codes.  These tests pin it to things other
than itself: torch's float8_e4m3fn type (decode of every code, round to
nearest even on encode), scipy's Hadamard matrix, brute force over the scale
exponent, exact round trips, the identity H H^T = d I on scores, and the
purpose the page states for the rotation (less precision loss when a few
channels dominate).  CPU only.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

F8 = torch.float8_e4m3fn


def torch_encode(x32: np.ndarray) -> np.ndarray:
    """torch's float32 -> e4m3fn conversion (round to nearest even), as bytes."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(F8).view(
        torch.uint8).numpy()


def test_decode_every_code_matches_torch(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(F8).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9  # largest, smallest subnormal


def test_encode_matches_torch_including_ties(oracle_mod):
    """Random values over the whole range (subnormals included), every exact
    midpoint between neighbouring codes (ties go to the even code), the codes'
    own values, and signed zeros."""
    rng = np.random.default_rng(0)
    vals = [np.float32(x) for x in
            rng.choice([-1, 1], 3000) * np.exp2(rng.uniform(-12, math.log2(448), 3000))]
    pos = sorted({oracle_mod.e4m3_decode(c) for c in range(0x7F)})
    vals += [np.float32(v) for v in pos] + [np.float32(-v) for v in pos]
    vals += [np.float32((a + b) / 2) for a, b in zip(pos, pos[1:])]
    vals += [np.float32(-(a + b) / 2) for a, b in zip(pos, pos[1:])]
    vals += [np.float32(0.0), np.float32(-0.0)]
    x = np.array(vals, dtype=np.float32)
    got = np.array([oracle_mod.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, torch_encode(x))


@pytest.mark.parametrize("n", [1, 2, 32, 64, 128])
def test_fwht_is_the_sylvester_hadamard_product(oracle_mod, n):
    """Integer inputs make every float32 sum exact: H x with scipy's H, exactly;
    real inputs agree within the rounding of log2(n) stages."""
    rng = np.random.default_rng(n)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    xi = rng.integers(-1000, 1000, n).astype(np.float32)
    np.testing.assert_array_equal(oracle_mod.fwht_f32(xi), H @ xi.astype(np.float64))
    xr = rng.standard_normal(n).astype(np.float32)
    ref = H @ xr.astype(np.float64)
    bound = 2.0 ** -23 * max(1, math.log2(n)) * np.abs(H) @ np.abs(xr.astype(np.float64))
    assert np.all(np.abs(oracle_mod.fwht_f32(xr) - ref) <= bound + 1e-30)


def _exp_of(byte):
    return int(byte) - 127


@pytest.mark.parametrize("rotate", [False, True])
def test_scale_is_the_least_that_fits(oracle_mod, rotate):
    """Brute force on each block: amax <= 448 2^e and amax > 448 2^(e-1); a zero
    block has e = 0; tiny blocks stop at e = -127."""
    rng = np.random.default_rng(3)
    d = 64
    x = rng.standard_normal((40, d)) * np.exp2(rng.uniform(-20, 20, (40, 1)))
    x[0] = 0.0
    x[1, :32] = 0.0
    x[2] = 1e-38 * rng.standard_normal(d)
    x = x.astype(np.float32)
    signs = np.where(rng.random(d) < 0.5, -1, 1) if rotate else None
    _, scales = oracle_mod.mx_quant(x, signs)
    xr = x.astype(np.float64)
    if rotate:
        xr = (scipy.linalg.hadamard(d) @ (signs * xr).T).T
    for r in range(x.shape[0]):
        for b in range(d // 32):
            amax = np.max(np.abs(xr[r, 32 * b:32 * b + 32]))
            e = _exp_of(scales[r, b])
            if amax == 0:
                assert e == 0
                continue
            rel = 1 + 1e-6 if rotate else 1  # the float32 transform vs fp64 at the edge
            assert amax <= 448 * 2.0 ** e * rel
            assert e == -127 or amax > 448 * 2.0 ** (e - 1) / rel


def test_codes_are_torch_nearest_after_scaling(oracle_mod):
    """Without rotation each code is torch's e4m3 of x / 2^e; with rotation and
    integer inputs (an exact transform) each code is torch's e4m3 of
    H (s * x) / 2^e.  Ragged last block (d = 80) included."""
    rng = np.random.default_rng(4)
    for d, rotate in ((80, False), (64, False), (128, True), (64, True)):
        if rotate:
            x = rng.integers(-50, 50, (16, d)).astype(np.float32)
            signs = np.where(rng.random(d) < 0.5, -1, 1)
            xr = (scipy.linalg.hadamard(d) @ (signs * x.astype(np.float64)).T).T
        else:
            x = (rng.standard_normal((16, d)) * np.exp2(rng.uniform(-8, 8, (16, 1)))).astype(
                np.float32)
            signs, xr = None, x.astype(np.float64)
        codes, scales = oracle_mod.mx_quant(x, signs)
        nb = (d + 31) // 32
        assert scales.shape == (16, nb)
        e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)[:, :d]
        np.testing.assert_array_equal(codes, torch_encode(xr * np.exp2(-e.astype(np.float64))))


def test_exact_values_round_trip(oracle_mod):
    """Rows built from e4m3 values times 2^e, each block holding +-448 2^e, come
    back exactly; dequantize agrees with torch's decode times the scale."""
    rng = np.random.default_rng(5)
    vals = np.array([oracle_mod.e4m3_decode(c) for c in range(0x7F)])
    x = rng.choice(vals, (8, 96)) * rng.choice([-1, 1], (8, 96))
    ex = rng.integers(-20, 20, (8, 3))
    x[:, ::32] = 448.0
    x = x * np.exp2(np.repeat(ex, 32, axis=1))
    codes, scales = oracle_mod.mx_quant(x)
    np.testing.assert_array_equal(scales.astype(np.int64) - 127, ex)
    back = oracle_mod.mx_dequant(codes, scales)
    np.testing.assert_array_equal(back, x)
    tdec = torch.from_numpy(codes).view(F8).to(torch.float64).numpy()
    np.testing.assert_array_equal(back, tdec * np.exp2(np.repeat(ex, 32, axis=1)))


def _err_bound(xr, codes, scales, deq):
    """Per value: |x^ - x'| <= 2^-4 |x'| (normal codes) or 2^-10 2^e (subnormal)."""
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)[..., :xr.shape[-1]]
    return np.maximum(2.0 ** -4 * np.abs(xr), 2.0 ** -10 * np.exp2(e.astype(np.float64)))


def test_rotated_scores_are_d_times_the_scores(oracle_mod):
    """Q and K rotated with the same signs: dequantized Q^ K^T is d Q K^T up to
    the per-value rounding bound carried through the dot products."""
    rng = np.random.default_rng(6)
    d = 128
    q = rng.standard_normal((20, d)).astype(np.float32)
    k = rng.standard_normal((30, d)).astype(np.float32)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    qr, kr = (H @ (signs * q.astype(np.float64)).T).T, (H @ (signs * k.astype(np.float64)).T).T
    np.testing.assert_allclose(qr @ kr.T, d * (q.astype(np.float64) @ k.astype(np.float64).T),
                               rtol=0, atol=1e-9)
    cq, sq = oracle_mod.mx_quant(q, signs)
    ck, sk = oracle_mod.mx_quant(k, signs)
    qh, kh = oracle_mod.mx_dequant(cq, sq), oracle_mod.mx_dequant(ck, sk)
    dq, dk = _err_bound(qr, cq, sq, qh), _err_bound(kr, ck, sk, kh)
    assert np.all(np.abs(qh - qr) <= dq * (1 + 1e-6)) and np.all(np.abs(kh - kr) <= dk * (1 + 1e-6))
    bound = dq @ np.abs(kr).T + np.abs(qr) @ dk.T + dq @ dk.T
    err = np.abs(qh @ kh.T - d * (q.astype(np.float64) @ k.astype(np.float64).T))
    assert np.all(err <= bound * (1 + 1e-5) + 1e-3)


def test_incoherent_processing_reduces_score_error(oracle_mod):
    """The stated purpose of the random signs: with a few dominant channels the
    rotation spreads them over all d values and the FP8 score error drops
    (here by well over 2x); with i.i.d. channels it changes little."""
    rng = np.random.default_rng(7)
    d = 64

    def rms_err(q, k, signs):
        exact = q.astype(np.float64) @ k.astype(np.float64).T
        qh = oracle_mod.mx_dequant(*oracle_mod.mx_quant(q, signs))
        kh = oracle_mod.mx_dequant(*oracle_mod.mx_quant(k, signs))
        f = d if signs is not None else 1
        return np.sqrt(np.mean((qh @ kh.T / f - exact) ** 2)) / np.sqrt(np.mean(exact ** 2))

    signs = np.where(rng.random(d) < 0.5, -1, 1)
    q = rng.standard_normal((64, d)).astype(np.float32)
    k = rng.standard_normal((64, d)).astype(np.float32)
    iid_plain, iid_rot = rms_err(q, k, None), rms_err(q, k, signs)
    assert 0.5 < iid_rot / iid_plain < 2.0
    q[:, 3] *= 40.0
    k[:, 3] *= 40.0
    q[:, 17] *= 25.0
    k[:, 17] *= 25.0
    out_plain, out_rot = rms_err(q, k, None), rms_err(q, k, signs)
    assert out_rot < out_plain / 2.5, (out_plain, out_rot)


def test_rejects_bad_shapes(oracle_mod):
    with pytest.raises(RuntimeError):
        oracle_mod.mx_quant(np.zeros((2, 48)), np.ones(48))  # rotation needs a power of two
    with pytest.raises(ValueError):
        oracle_mod.mx_quant(np.zeros((2, 64)), np.ones(32))
