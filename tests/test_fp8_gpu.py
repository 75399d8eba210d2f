"""FP8-score forward parity: the HIP quantizer and forward (through the C ABI)
against the oracle's block-scaled FP8 quantizer and its fp64 attention.

The codes and scale bytes are integers the two sides decide in the same float32
arithmetic, so they are compared bit for bit.  The forward is attention of the
dequantized rows: its expected values are the oracle's forward on the oracle's
dequantized codes, and the GPU forward is fed those same codes (uploaded), so
the forward test does not lean on the GPU quantizer; an end-to-end case chains
the two GPU calls.  Tolerances are the 16-bit bar (weights and values are
16-bit) plus the effect of the FP8 matrix cores' summation, bounded per row
from the dequantized inputs (helpers.fp8_score_slack).
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_tiled_amd import attn_fwd_fp8, attn_fwd_fp8_pv, attn_quant_fp8, attn_quant_fp8_v
from exact_io_aware_tiled_amd.inputs import (FP8_SIGNS_SEED, WORKLOADS, Workload, make_inputs,
                                             make_signs)
from helpers import announce, check_fwd_fp8, fp8_score_slack, sample_rows, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def quant_rows(rng, rows, d, dt):
    """Rows with a spread of magnitudes: zero rows, a zero block, tiny and huge rows."""
    x = rng.standard_normal((rows, d)) * np.exp2(rng.uniform(-12, 12, (rows, 1)))
    x[0] = 0.0
    x[1, :32] = 0.0
    x[2] *= 1e-30 if dt == "f32" else 1.0
    x[3, 5] = 3e4 if dt != "f16" else 6e4
    return torch.from_numpy(x).to(DT[dt])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rotate", [False, True])
def test_quant_codes_exact(dt, d, rotate):
    """1000 rows (a ragged last workgroup): codes and scales equal the oracle's."""
    rng = np.random.default_rng(d + 3 * rotate)
    x = quant_rows(rng, 1000, d, dt)
    signs = make_signs(d, 11) if rotate else None
    announce(f"attn_quant_fp8 {dt} d={d} rotate={rotate}")
    codes, scales = attn_quant_fp8(x.to(DEV), None if signs is None else signs.to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quant(to64(x), None if signs is None else signs.numpy())
    assert np.array_equal(scales.cpu().numpy(), rs)
    bad = np.nonzero(codes.cpu().numpy() != rc)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]}, {bad[1][0]}"


def test_quant_one_row_and_shapes():
    """A single row, and a [B, H, n, d] tensor (rows are the flattened leading dims)."""
    x = torch.randn(1, 64, dtype=torch.bfloat16)
    signs = make_signs(64, 12)
    announce("attn_quant_fp8 one row")
    c, s = attn_quant_fp8(x.to(DEV), signs.to(DEV))
    x4 = torch.randn(2, 3, 37, 128, dtype=torch.float16)
    c4, s4 = attn_quant_fp8(x4.to(DEV), signs=None)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quant(to64(x), signs.numpy())
    assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)
    rc4, rs4 = oracle.mx_quant(to64(x4))
    assert c4.shape == (2, 3, 37, 128) and s4.shape == (2, 3, 37, 4)
    assert np.array_equal(c4.cpu().numpy(), rc4) and np.array_equal(s4.cpu().numpy(), rs4)


def oracle_inputs(inp, d, rotate, seed=FP8_SIGNS_SEED):
    """The oracle's codes and scales of Q and K, and their dequantized values."""
    signs = make_signs(d, seed).numpy() if rotate else None
    cq, sq = oracle.mx_quant(to64(inp["q"]), signs)
    ck, sk = oracle.mx_quant(to64(inp["k"]), signs)
    return (cq, sq, ck, sk), oracle.mx_dequant(cq, sq), oracle.mx_dequant(ck, sk)


def check(o, lse, y, lref, qd, kd, v, c, dtype, what):
    """Compare a [.., n, dv] GPU forward with the oracle, head by head."""
    o64, l64 = to64(o), to64(lse)
    qd = qd.reshape(-1, *qd.shape[-2:])
    kd = kd.reshape(-1, *kd.shape[-2:])
    v64 = to64(v).reshape(-1, *v.shape[-2:])
    y = y.reshape(v64.shape[0], -1, v64.shape[-1])
    lref = lref.reshape(v64.shape[0], -1)
    o64 = o64.reshape(y.shape)
    l64 = l64.reshape(lref.shape)
    for hh in range(qd.shape[0]):
        slack = fp8_score_slack(qd[hh], kd[hh], c)
        check_fwd_fp8(o64[hh], l64[hh], y[hh], lref[hh], dtype, slack,
                      float(np.abs(v64[hh]).max(initial=0.0)), f"{what} head {hh}")


def run_fwd(codes, v, c_eff, mask, win):
    cq, sq, ck, sk = (torch.from_numpy(a).to(DEV) for a in codes)
    o, lse = attn_fwd_fp8(cq, sq, ck, sk, v.to(DEV), c_eff, mask, win)
    torch.cuda.synchronize()
    return o, lse


SMALL = [(dt, d, mask, win, rot) for dt in ("f16", "bf16") for d in (64, 128)
         for mask, win in (("none", 0), ("causal", 0), ("window", 50)) for rot in (False, True)]


@pytest.mark.parametrize("dt,d,mask,win,rot", SMALL)
def test_fwd_fp8_small(dt, d, mask, win, rot):
    """n = 200 (several tiles, ragged tail), 3 heads."""
    w = Workload("fp8", 1, 3, 200, d, d, dt, mask, window=win, seed=41)
    inp = make_inputs(w)
    codes, qd, kd = oracle_inputs(inp, d, rot)
    c_eff = w.c / d if rot else w.c
    announce(f"attn_fwd_fp8 {w} rotate={rot}")
    o, lse = run_fwd(codes, inp["v"], c_eff, mask, win)
    y, _, _, lref = oracle.fwd(qd, kd, to64(inp["v"]), c_eff, mask, win)
    check(o, lse, y, lref, qd, kd, inp["v"], c_eff, DT[dt], w.name)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
def test_fwd_fp8_scales(scale):
    """c = 0 (mean of the allowed values), c < 0 (codes negated, zero kept) and c > 0."""
    w = Workload("fp8s", 1, 2, 150, 64, 64, "bf16", "causal", seed=42)
    inp = make_inputs(w)
    codes, qd, kd = oracle_inputs(inp, 64, True)
    announce(f"attn_fwd_fp8 scale={scale}")
    o, lse = run_fwd(codes, inp["v"], scale, "causal", 0)
    y, _, _, lref = oracle.fwd(qd, kd, to64(inp["v"]), scale, "causal")
    check(o, lse, y, lref, qd, kd, inp["v"], scale, torch.bfloat16, "scale")


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 129])
def test_fwd_fp8_edges(n):
    """Tiny and ragged sequence lengths around the 64-key tile."""
    for mask in ("none", "causal"):
        w = Workload("fp8e", 1, 2, n, 128, 128, "f16", mask, seed=43)
        inp = make_inputs(w)
        codes, qd, kd = oracle_inputs(inp, 128, True)
        announce(f"attn_fwd_fp8 n={n} {mask}")
        o, lse = run_fwd(codes, inp["v"], w.c / 128, mask, 0)
        y, _, _, lref = oracle.fwd(qd, kd, to64(inp["v"]), w.c / 128, mask)
        check(o, lse, y, lref, qd, kd, inp["v"], w.c / 128, torch.float16, f"n={n}")


def test_fwd_fp8_empty():
    z = torch.empty(1, 2, 0, 64, dtype=torch.uint8, device=DEV)
    zs = torch.empty(1, 2, 0, 2, dtype=torch.uint8, device=DEV)
    v = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = attn_fwd_fp8(z, zs, z, zs, v, 0.1, "causal")
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)


def test_end_to_end_gpu_quantizer():
    """GPU quantizer then GPU forward == oracle quantizer then oracle forward."""
    w = Workload("fp8e2e", 2, 2, 300, 64, 64, "bf16", "window", window=77, seed=44)
    inp = make_inputs(w)
    signs = make_signs(64, FP8_SIGNS_SEED)
    announce("attn_fwd_fp8 end to end")
    q8, qs = attn_quant_fp8(inp["q"].to(DEV), signs.to(DEV))
    k8, ks = attn_quant_fp8(inp["k"].to(DEV), signs.to(DEV))
    o, lse = attn_fwd_fp8(q8, qs, k8, ks, inp["v"].to(DEV), w.c / 64, "window", 77)
    torch.cuda.synchronize()
    _, qd, kd = oracle_inputs(inp, 64, True)
    y, _, _, lref = oracle.fwd(qd, kd, to64(inp["v"]), w.c / 64, "window", 77)
    check(o, lse, y, lref, qd, kd, inp["v"], w.c / 64, torch.bfloat16, "e2e")


@pytest.mark.parametrize("name", ["page_d64", "page_d128"])
def test_fwd_fp8_full_size(name):
    """The page shape (32 heads, n = 4096, causal, bf16) with rotated FP8 scores:
    the GPU quantizer's codes are checked whole against the oracle for two heads,
    and sampled rows of every head against the oracle's forward."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    d = w.d
    signs = make_signs(d, FP8_SIGNS_SEED)
    announce(f"attn_fwd_fp8 full size {w}")
    q8, qs = attn_quant_fp8(inp["q"].to(DEV), signs.to(DEV))
    k8, ks = attn_quant_fp8(inp["k"].to(DEV), signs.to(DEV))
    o, lse = attn_fwd_fp8(q8, qs, k8, ks, inp["v"].to(DEV), w.c / d, "causal")
    torch.cuda.synchronize()
    for h in (0, 31):
        rc, rs = oracle.mx_quant(to64(inp["k"][0, h]), signs.numpy())
        assert np.array_equal(k8[0, h].cpu().numpy(), rc) and np.array_equal(ks[0, h].cpu().numpy(), rs)
    rows = sample_rows(w.n, 48, 7, must=(0, 1, 63, 64, 4095))
    q8c, qsc, k8c, ksc = (t.cpu().numpy() for t in (q8, qs, k8, ks))
    for h in range(0, 32, 5):
        qd = oracle.mx_dequant(q8c[0, h], qsc[0, h])
        kd = oracle.mx_dequant(k8c[0, h], ksc[0, h])
        y, _, _, lref = oracle.fwd(qd, kd, to64(inp["v"][0, h]), w.c / d, "causal", rows=rows)
        slack = fp8_score_slack(qd[rows], kd, w.c / d)
        check_fwd_fp8(to64(o[0, h, rows]), to64(lse[0, h, rows]), y, lref, torch.bfloat16, slack,
                      float(np.abs(to64(inp["v"][0, h])).max()), f"h={h}")


def test_rotation_lowers_error_against_exact_attention():
    """The point of the incoherent processing, on the GPU path: with a few
    dominant channels in Q and K, the output's error against exact (unquantized)
    attention is lower with the rotation than without."""
    w = Workload("fp8out", 1, 4, 512, 64, 64, "bf16", "none", seed=45)
    inp = make_inputs(w)
    g = torch.Generator("cpu").manual_seed(46)
    boost = torch.ones(64)
    boost[torch.randint(0, 64, (3,), generator=g)] = 12.0
    q = (inp["q"].float() * boost).to(torch.bfloat16)
    k = (inp["k"].float() * boost).to(torch.bfloat16)
    c = 0.25 / 8
    exact, _, _, _ = oracle.fwd(to64(q), to64(k), to64(inp["v"]), c, "none")
    errs = {}
    for rot in (False, True):
        signs = make_signs(64, FP8_SIGNS_SEED).to(DEV) if rot else None
        announce(f"attn_fwd_fp8 outliers rotate={rot}")
        q8, qs = attn_quant_fp8(q.to(DEV), signs)
        k8, ks = attn_quant_fp8(k.to(DEV), signs)
        o, _ = attn_fwd_fp8(q8, qs, k8, ks, inp["v"].to(DEV), c / 64 if rot else c, "none")
        torch.cuda.synchronize()
        errs[rot] = float(np.sqrt(np.mean((to64(o) - exact) ** 2)))
    assert errs[True] < errs[False], errs


# ---------------------------------------------------------------------------
# FP8 weights and values (attn_quant_fp8_v, attn_fwd_fp8_pv)
# ---------------------------------------------------------------------------

def v_tile_layout(cv, sv, n):
    """The oracle's codes cv [dv][n] and scales sv [dv][ceil(n / 32)] of one head's
    V^T, arranged as the tile-major layout the C ABI documents: codes [nt][dv][64]
    with key 64 t + 32 b + 8 g + 4 h + i at byte 32 b + 16 h + 4 g + i, scales
    [nt][dv][2]; keys past n are code 0, blocks past n scale byte 127."""
    dv = cv.shape[0]
    nt = (n + 63) // 64
    pos = np.arange(64)
    b, q = pos // 32, pos % 32
    key_in_tile = 32 * b + 8 * ((q % 16) // 4) + 4 * (q // 16) + q % 4
    codes = np.zeros((nt, dv, 64), dtype=np.uint8)
    for t in range(nt):
        keys = 64 * t + key_in_tile
        ok = keys < n
        codes[t][:, ok] = cv[:, keys[ok]]
    scales = np.full((nt, dv, 2), 127, dtype=np.uint8)
    nb = sv.shape[1]
    for t in range(nt):
        for bb in range(2):
            if 2 * t + bb < nb:
                scales[t, :, bb] = sv[:, 2 * t + bb]
    return codes, scales


def oracle_v(v64):
    """Per head: the oracle's block-scaled codes of V along the keys, their tile
    layout, and the dequantized V.  v64 [nh, n, dv] float64."""
    out_c, out_s, vd = [], [], []
    n = v64.shape[1]
    for hh in range(v64.shape[0]):
        cv, sv = oracle.mx_quant(v64[hh].T)
        c, s = v_tile_layout(cv, sv, n)
        out_c.append(c)
        out_s.append(s)
        vd.append(oracle.mx_dequant(cv, sv).T)
    return np.stack(out_c), np.stack(out_s), np.stack(vd)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("n", [1, 65, 200, 256])
def test_quant_v_codes_exact(dt, dv, n):
    rng = np.random.default_rng(n + dv)
    v = rng.standard_normal((2, 3, n, dv)) * np.exp2(rng.uniform(-8, 8, (2, 3, 1, dv)))
    v[0, 0, :, 5] = 0.0  # a zero column
    vt = torch.from_numpy(v).to(DT[dt])
    announce(f"attn_quant_fp8_v {dt} dv={dv} n={n}")
    codes, scales = attn_quant_fp8_v(vt.to(DEV))
    torch.cuda.synchronize()
    rc, rs, _ = oracle_v(to64(vt).reshape(6, n, dv))
    nt = (n + 63) // 64
    assert codes.shape == (2, 3, nt, dv, 64) and scales.shape == (2, 3, nt, dv, 2)
    assert np.array_equal(scales.cpu().numpy().reshape(rs.shape), rs)
    assert np.array_equal(codes.cpu().numpy().reshape(rc.shape), rc)


def pv_bound(qd, kd, vd, c, mask, win, lref):
    """Per element, the effect of rounding the weights to e4m3 on O (rows of
    one head): 2^-4 sum_j w_ij |V_jc| + 2^-10 e^(m_i - LSE_i) sum_{j in A_i} |V_jc|,
    m_i the row's largest score.  The kernel's weights are 2^(x - m'), m' <= m_i,
    rounded with error <= 2^-4 p + 2^-10; its normaliser is the unrounded sum,
    at least e^(LSE_i - m_i)."""
    n = qd.shape[0]
    s = c * (qd @ kd.T)
    i, j = np.arange(n)[:, None], np.arange(kd.shape[0])[None, :]
    allowed = np.ones(s.shape, dtype=bool)
    if mask != "none":
        allowed &= j <= i
    if mask == "window":
        allowed &= j > i - win
    m = np.where(allowed, s, -np.inf).max(axis=1)
    wabs, _, _, _ = oracle.fwd(qd[None], kd[None], np.abs(vd)[None], c, mask, win)
    vabs = allowed.astype(np.float64) @ np.abs(vd)
    return 2.0 ** -4 * wabs[0] + 2.0 ** -10 * np.exp(m - lref)[:, None] * vabs


def check_pv(o, lse, y, lref, qd, kd, vd, c, mask, win, dtype, what):
    o64, l64 = to64(o).reshape(y.shape), to64(lse).reshape(lref.shape)
    nh = qd.shape[0]
    for hh in range(nh):
        slack = fp8_score_slack(qd[hh], kd[hh], c)
        pvb = pv_bound(qd[hh], kd[hh], vd[hh], c, mask, win, lref[hh])
        vmax = float(np.abs(vd[hh]).max(initial=0.0))
        err = np.abs(o64[hh] - y[hh])
        bound = 2e-2 + np.expm1(2 * slack)[:, None] * vmax + pvb
        assert np.all(err <= bound), f"{what} head {hh}: O err {err.max():.3g}, worst margin " \
            f"{(err - bound).max():.3g}"
        assert np.all(np.abs(l64[hh] - lref[hh]) <= 1e-3 + slack), f"{what} head {hh}: LSE"
        # the bound is a worst case (every rounding in one direction): the mean
        # error sits well inside it
        assert err.mean() <= 0.25 * bound.mean(), f"{what} head {hh}: mean error {err.mean():.3g}"


PV_SMALL = [(dt, d, mask, win) for dt in ("f16", "bf16") for d in (64, 128)
            for mask, win in (("none", 0), ("causal", 0), ("window", 50))]


@pytest.mark.parametrize("dt,d,mask,win", PV_SMALL)
def test_fwd_fp8_pv_small(dt, d, mask, win):
    """n = 200, 3 heads, rotated Q and K: the oracle's codes of Q, K and V uploaded,
    O against the oracle's attention of the dequantized rows."""
    w = Workload("fp8pv", 1, 3, 200, d, d, dt, mask, window=win, seed=47)
    inp = make_inputs(w)
    codes, qd, kd = oracle_inputs(inp, d, True)
    vc, vs, vd = oracle_v(to64(inp["v"]).reshape(3, 200, d))
    c_eff = w.c / d
    cq, sq, ck, sk = (torch.from_numpy(a).to(DEV) for a in codes)
    announce(f"attn_fwd_fp8_pv {w}")
    o, lse = attn_fwd_fp8_pv(cq, sq, ck, sk, torch.from_numpy(vc.reshape(1, 3, *vc.shape[1:])).to(DEV),
                             torch.from_numpy(vs.reshape(1, 3, *vs.shape[1:])).to(DEV), c_eff, mask,
                             win, dtype=DT[dt])
    torch.cuda.synchronize()
    qd3, kd3 = qd.reshape(3, 200, d), kd.reshape(3, 200, d)
    y, _, _, lref = oracle.fwd(qd3, kd3, vd, c_eff, mask, win)
    check_pv(o, lse, y, lref, qd3, kd3, vd, c_eff, mask, win, DT[dt], w.name)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 129])
def test_fwd_fp8_pv_edges(n):
    w = Workload("fp8pve", 1, 2, n, 64, 64, "bf16", "causal", seed=48)
    inp = make_inputs(w)
    codes, qd, kd = oracle_inputs(inp, 64, True)
    vc, vs, vd = oracle_v(to64(inp["v"]).reshape(2, n, 64))
    cq, sq, ck, sk = (torch.from_numpy(a).to(DEV) for a in codes)
    announce(f"attn_fwd_fp8_pv n={n}")
    o, lse = attn_fwd_fp8_pv(cq, sq, ck, sk, torch.from_numpy(vc[None]).to(DEV),
                             torch.from_numpy(vs[None]).to(DEV), w.c / 64, "causal")
    torch.cuda.synchronize()
    qd2, kd2 = qd.reshape(2, n, 64), kd.reshape(2, n, 64)
    y, _, _, lref = oracle.fwd(qd2, kd2, vd, w.c / 64, "causal")
    check_pv(o, lse, y, lref, qd2, kd2, vd, w.c / 64, "causal", 0, torch.bfloat16, f"n={n}")


@pytest.mark.parametrize("name", ["page_d64", "page_d128"])
def test_fwd_fp8_pv_full_size(name):
    """GPU quantizers then the FP8-value forward at the page shape; V's codes of
    two heads checked whole, sampled rows of every fifth head against the oracle."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    d = w.d
    signs = make_signs(d, FP8_SIGNS_SEED)
    announce(f"attn_fwd_fp8_pv full size {w}")
    q8, qs = attn_quant_fp8(inp["q"].to(DEV), signs.to(DEV))
    k8, ks = attn_quant_fp8(inp["k"].to(DEV), signs.to(DEV))
    v8, vs = attn_quant_fp8_v(inp["v"].to(DEV))
    o, lse = attn_fwd_fp8_pv(q8, qs, k8, ks, v8, vs, w.c / d, "causal")
    torch.cuda.synchronize()
    q8c, qsc, k8c, ksc = (t.cpu().numpy() for t in (q8, qs, k8, ks))
    v8c, vsc = v8.cpu().numpy(), vs.cpu().numpy()
    rows = sample_rows(w.n, 40, 9, must=(0, 1, 63, 64, 4095))
    for h in range(0, 32, 5):
        rc, rs, vd = oracle_v(to64(inp["v"][0, h:h + 1]))
        if h in (0, 30):
            assert np.array_equal(v8c[0, h], rc[0]) and np.array_equal(vsc[0, h], rs[0])
        qd = oracle.mx_dequant(q8c[0, h], qsc[0, h])
        kd = oracle.mx_dequant(k8c[0, h], ksc[0, h])
        y, _, _, lref = oracle.fwd(qd, kd, vd[0], w.c / d, "causal", rows=rows)
        slack = fp8_score_slack(qd[rows], kd, w.c / d)
        pvb = pv_bound(qd, kd, vd[0], w.c / d, "causal", 0,
                       oracle.fwd(qd, kd, vd[0], w.c / d, "causal")[3])[rows]
        err = np.abs(to64(o[0, h, rows]) - y)
        bound = 2e-2 + np.expm1(2 * slack)[:, None] * float(np.abs(vd).max()) + pvb
        assert np.all(err <= bound), f"h={h}: O err {err.max():.3g}"
        assert np.all(np.abs(to64(lse[0, h, rows]) - lref) <= 1e-3 + slack), f"h={h}: LSE"
        assert err.mean() <= 0.25 * bound.mean()
