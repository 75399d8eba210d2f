"""Dropout parity: the HIP forward and reverse with dropout (through the C ABI)
against the oracle's dropout extension.

The realized mask is checked exactly: with c = 0 every allowed weight is
1 / |A_i|, and with V the identity (n <= d) output column j of row i is
D_ij / |A_i|, nonzero exactly where the kernel kept the weight; the kept set is
compared bit for bit with the oracle's mask.  Outputs and gradients are then
compared with the oracle's dropout forward and VJP at the usual tolerances
(the same realized mask replayed in the reverse, as the Algorithm requires).
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_tiled_amd import attn_bwd, attn_fwd
from exact_io_aware_tiled_amd.inputs import WORKLOADS, Workload, make_inputs
from helpers import announce, check_fwd, check_grad, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def thr_of(p):
    return min(255, int(round(p * 256)))


def keep_scale(p):
    """256 / (256 - thr): kept weights are scaled by it, so O and every rounding
    error in O are too; O is compared after dividing it out (the 16-bit O bound
    is for outputs of order one)."""
    return 256.0 / (256 - thr_of(p))


def allowed(mask, win, i, j):
    if mask == "none":
        return True
    return j <= i and (mask == "causal" or j > i - win)


@pytest.mark.parametrize("dt,d", [("bf16", 64), ("f16", 128), ("f32", 64), ("bf16", 16)])
@pytest.mark.parametrize("mask,win", [("none", 0), ("causal", 0), ("window", 9)])
def test_realized_mask_exact(dt, d, mask, win):
    n, H, p, seed = d, 3, 0.3, 0xDEADBEEF12345
    g = torch.Generator("cpu").manual_seed(31)
    q = torch.randn(1, H, n, d, generator=g).to(DT[dt])
    k = torch.randn(1, H, n, d, generator=g).to(DT[dt])
    v = torch.eye(n, d).expand(1, H, n, d).contiguous().to(DT[dt])
    announce(f"dropout mask {dt} d={d} {mask}")
    o, _ = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 0.0, mask, win, p_drop=p, seed=seed)
    kept = (to64(o) != 0)[0]
    thr = thr_of(p)
    for h in range(H):
        for i in range(n):
            for j in range(n):
                want = allowed(mask, win, i, j) and oracle.dropout_keep(seed, thr, h, i, j)
                assert kept[h, i, j] == want, (h, i, j)


SMALL = [(dt, d, mask, win) for dt in ("f32", "f16", "bf16") for d in (16, 64, 128)
         for mask, win in (("none", 0), ("causal", 0), ("window", 50))]


@pytest.mark.parametrize("dt,d,mask,win", SMALL)
def test_dropout_fwd_bwd_small(dt, d, mask, win):
    """n = 200 (several tiles, ragged tail), drop probability 0.1."""
    w = Workload("drop", 1, 3, 200, d, d, dt, mask, window=win, seed=32)
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    p, seed = 0.1, 2024
    announce(f"dropout fwd+bwd {w}")
    o, lse = attn_fwd(q, k, v, w.c, mask, win, p_drop=p, seed=seed)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, w.c, mask, win, p_drop=p, seed=seed)
    torch.cuda.synchronize()
    ref = oracle.bwd_drop(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), to64(inp["do"]), w.c,
                          mask, win, seed=seed, thr=thr_of(p))
    rdq, rdk, rdv, ry, _, rlse = ref
    ks = keep_scale(p)
    check_fwd(to64(o) / ks, to64(lse), ry / ks, rlse, DT[dt], w.name, w.c * d ** 0.5)
    check_grad(to64(dq), rdq, DT[dt], "dq")
    check_grad(to64(dk), rdk, DT[dt], "dk")
    check_grad(to64(dv), rdv, DT[dt], "dv")


@pytest.mark.parametrize("p", [0.02, 0.5, 0.9])
def test_dropout_probabilities(p):
    w = Workload("drop_p", 2, 2, 160, 64, 64, "bf16", "causal", seed=33)
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    announce(f"dropout p={p}")
    o, lse = attn_fwd(q, k, v, w.c, "causal", p_drop=p, seed=5)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, w.c, "causal", p_drop=p, seed=5)
    torch.cuda.synchronize()
    flat = lambda t: to64(t).reshape(-1, w.n, t.shape[-1])  # noqa: E731
    ref = oracle.bwd_drop(flat(inp["q"]), flat(inp["k"]), flat(inp["v"]), flat(inp["do"]), w.c,
                          "causal", seed=5, thr=thr_of(p))
    ks = keep_scale(p)
    check_fwd(flat(o) / ks, to64(lse).reshape(-1, w.n), ref[3] / ks, ref[5], torch.bfloat16, "o")
    for got, r, nm in ((dq, ref[0], "dq"), (dk, ref[1], "dk"), (dv, ref[2], "dv")):
        check_grad(flat(got), r, torch.bfloat16, nm)


def test_zero_probability_is_the_base_path():
    w = Workload("drop0", 1, 2, 300, 64, 64, "f16", "causal", seed=34)
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    announce("dropout p=0")
    from exact_io_aware_tiled_amd import attn as A
    lib = A.load_library()
    o0, l0 = attn_fwd(q, k, v, w.c, "causal")
    o1 = torch.empty_like(o0)
    l1 = torch.empty_like(l0)
    assert lib.attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                                l1.data_ptr(), 1, 2, 300, 64, 64, 1, w.c, 1, 0, 0.0, 9,
                                None) == 0
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_dropout_stages_and_determinism():
    w = Workload("drop_st", 1, 2, 260, 128, 128, "bf16", "window", window=70, seed=35)
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    announce("dropout stages")
    o, lse = attn_fwd(q, k, v, w.c, "window", 70, p_drop=0.25, seed=77)
    full = attn_bwd(q, k, v, o, lse, do, w.c, "window", 70, p_drop=0.25, seed=77)
    ws = torch.empty(w.H * w.n * 4, dtype=torch.uint8, device=DEV)
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    for st in (0, 1, 2):
        attn_bwd(q, k, v, o, lse, do, w.c, "window", 70, dq=outs[0], dk=outs[1], dv=outs[2],
                 workspace=ws, stage=st, p_drop=0.25, seed=77)
    again = attn_bwd(q, k, v, o, lse, do, w.c, "window", 70, p_drop=0.25, seed=77)
    torch.cuda.synchronize()
    for a, b, c in zip(full, outs, again):
        assert torch.equal(a, b) and torch.equal(a, c)
    o2, _ = attn_fwd(q, k, v, w.c, "window", 70, p_drop=0.25, seed=78)
    assert not torch.equal(o, o2)  # another seed, another mask


def test_dropout_full_size_page_heads():
    """The page shape (32 heads, n = 4096, d = 64, bf16, causal) with p = 0.1:
    heads 0 and 31 (the mask depends on the head index) against the oracle."""
    w = WORKLOADS["page_d64"]
    inp = make_inputs(w, with_grad=True)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    announce(f"dropout full size {w}")
    o, lse = attn_fwd(q, k, v, w.c, "causal", p_drop=0.1, seed=123)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, w.c, "causal", p_drop=0.1, seed=123)
    torch.cuda.synchronize()
    for h in (0, 31):
        ref = oracle.bwd_drop(to64(inp["q"][0, h:h + 1]), to64(inp["k"][0, h:h + 1]),
                              to64(inp["v"][0, h:h + 1]), to64(inp["do"][0, h:h + 1]), w.c,
                              "causal", seed=123, thr=thr_of(0.1), bh0=h)
        ks = keep_scale(0.1)
        check_fwd(to64(o[0, h:h + 1]) / ks, to64(lse[0, h:h + 1]), ref[3] / ks, ref[5],
                  torch.bfloat16, "o")
        check_grad(to64(dq[0, h:h + 1]), ref[0], torch.bfloat16, f"dq h={h}")
        check_grad(to64(dk[0, h:h + 1]), ref[1], torch.bfloat16, f"dk h={h}")
        check_grad(to64(dv[0, h:h + 1]), ref[2], torch.bfloat16, f"dv h={h}")
