"""Decode-shaped forward parity: the split-cache HIP kernels (through the C ABI)
against the fp64 oracle's decode rows.

Every row is compared, also at the full decode workloads (a decode call has only
B * H * nq rows).  The cases cover both 16-bit types and head dims, every mask,
shared key/value heads, the largest row count per key/value head (32), ragged
cache lengths around the 32-key tile, a single key, rows as long as the cache,
many cache ranges per head (the merge of many range summaries) and one range.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_tiled_amd import attn_decode
from exact_io_aware_tiled_amd.inputs import DECODE_WORKLOADS, DecodeWorkload, make_decode_inputs
from helpers import announce, check_fwd, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def run(w: DecodeWorkload):
    inp = make_decode_inputs(w)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    announce(f"attn_decode {w}")
    o, lse = attn_decode(q, k, v, scale=w.c, mask=w.mask, window=w.window)
    torch.cuda.synchronize()
    return inp, o, lse


def compare(w: DecodeWorkload, inp, o, lse):
    y, lref = oracle.decode(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), w.c, w.mask,
                            w.window)
    score_std = w.c * w.d ** 0.5
    return check_fwd(to64(o), to64(lse), y, lref, DT[w.dtype], w.name, score_std)


SMALL = [
    (dt, d, mask, win)
    for dt in ("f16", "bf16")
    for d in (64, 128)
    for mask, win in (("none", 0), ("causal", 0), ("window", 37))
]


@pytest.mark.parametrize("dt,d,mask,win", SMALL)
def test_decode_small(dt, d, mask, win):
    """Shared heads (4 query heads per key/value head), 3 new rows, ragged cache."""
    w = DecodeWorkload("small", 2, 8, 2, 3, 200, d, d, dt, mask, window=win, seed=21)
    compare(w, *run(w))


@pytest.mark.parametrize("nk", [1, 2, 31, 32, 33, 95, 1000, 4097])
def test_decode_ragged_cache(nk):
    for mask in ("none", "causal"):
        w = DecodeWorkload("ragged", 1, 4, 4, 1, nk, 128, 128, "bf16", mask, seed=22)
        compare(w, *run(w))


@pytest.mark.parametrize("H,Hkv,nq", [(32, 1, 1), (8, 2, 8), (4, 4, 8), (2, 1, 16)])
def test_decode_rows_per_group(H, Hkv, nq):
    """Up to 32 rows per key/value head (the single 32-row block of the kernel)."""
    for mask in ("causal", "window"):
        w = DecodeWorkload("rows", 1, H, Hkv, nq, 300, 64, 64, "f16", mask, window=20, seed=23)
        compare(w, *run(w))


def test_decode_rows_as_long_as_cache():
    """nq == nk: the rows are the whole sequence (a causal prefill of 16 rows)."""
    for mask, win in (("causal", 0), ("window", 5), ("none", 0)):
        w = DecodeWorkload("full", 1, 2, 2, 16, 16, 64, 64, "bf16", mask, window=win, seed=24)
        compare(w, *run(w))


def test_decode_window_of_one():
    """Each new row sees only its own key."""
    w = DecodeWorkload("w1", 1, 4, 2, 4, 64, 64, 64, "bf16", "window", window=1, seed=25)
    inp, o, lse = run(w)
    compare(w, inp, o, lse)


@pytest.mark.parametrize("nk", [20000, 65536])
def test_decode_many_ranges(nk):
    """One key/value head: the cache is split into one range per 32-key tile
    (up to 2048 ranges) and their summaries are merged."""
    w = DecodeWorkload("ranges", 1, 4, 1, 2, nk, 128, 128, "bf16", "causal", seed=26)
    compare(w, *run(w))


def test_decode_one_range_per_head():
    """Many key/value heads: one range per head (no merge across ranges)."""
    w = DecodeWorkload("one", 4, 1024, 512, 1, 40, 64, 64, "f16", seed=27)
    compare(w, *run(w))


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.37])
def test_decode_scales(scale):
    """c = 0 (mean of the allowed values), c < 0 and an arbitrary c > 0."""
    w = DecodeWorkload("scale", 1, 4, 2, 2, 300, 64, 64, "bf16", "causal", scale=scale, seed=28)
    compare(w, *run(w))


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    """The decode workloads at full size, every row against the oracle."""
    w = DECODE_WORKLOADS[name]
    compare(w, *run(w))


def test_decode_deterministic():
    w = DECODE_WORKLOADS["decode_gqa"].replace(nk=3000)
    _, o1, l1 = run(w)
    _, o2, l2 = run(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_stages_equal_one_call():
    """attn_decode_stage 0 then 1 (the benchmark's timed steps) == attn_decode."""
    w = DECODE_WORKLOADS["decode_verify"].replace(B=2, nk=1500)
    inp, o, lse = run(w)
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    o2, l2 = attn_decode(q, k, v, w.c, w.mask, w.window, workspace=ws, stage=0)
    o2, l2 = attn_decode(q, k, v, w.c, w.mask, w.window, out=o2, lse=l2, workspace=ws, stage=1)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
