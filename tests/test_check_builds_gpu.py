"""Race and tile-shape checks on the GPU, through the check builds of the
library (exact_io_aware_tiled_amd/build.py, CHECK_BUILDS).

Poison build: every direct HBM -> LDS tile load first fills its destination
with NaN.  A kernel that read a tile before its loads had landed and been
published by a barrier would return non-finite or different values; a
correctly synchronized one returns bitwise the results of the product build.

Timing build: the forward also records per-workgroup wall-clock stamps and
hardware positions (wg_timeline.py reads them); its outputs must be bitwise the
product's, and the stamps must be complete and ordered.

Tile-shape build: other keys-per-tile and rows-per-tile.  The exactness theorem
(alphabetamath.cc, Theorem "Tiled attention and its recomputed reverse pass are
exact") makes the result independent of the block size; in floating point
the two builds may differ by rounding only, so they are compared with the
parity tolerances, and the other build is compared with the oracle as well.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_tiled_amd import attn as A
from exact_io_aware_tiled_amd.inputs import (DECODE_WORKLOADS, WORKLOADS, Workload,
                                             make_decode_inputs, make_inputs)
from helpers import (TOL_GRAD_16, TOL_LSE_16, TOL_O_16, announce, check_fwd, check_grad,
                     to64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fwd_bwd(lib, w: Workload, inp):
    """O, LSE, dQ, dK, dV through the C ABI of `lib`."""
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "do"))
    B, H, n, d = q.shape
    o = torch.empty_like(v)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = max(lib.attn_bwd_workspace_bytes(B, H, n), 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    sh = A._stream_handle(None)
    code, mcode = A.DTYPE_CODES[q.dtype], A.MASK_CODES[w.mask]
    announce(f"check build fwd+bwd {w}")
    assert lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                        H, n, d, d, code, float(w.c), mcode, w.window, sh) == 0
    assert lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                        ws_bytes, B, H, n, d, d, code, float(w.c), mcode, w.window, sh) == 0
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def decode(lib, w, inp):
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    o = torch.empty(w.B, w.H, w.nq, w.dv, dtype=q.dtype, device=DEV)
    lse = torch.empty(w.B, w.H, w.nq, dtype=torch.float32, device=DEV)
    ws_bytes = max(lib.attn_decode_workspace_bytes(w.B, w.H, w.Hkv, w.nq, w.nk, w.dv), 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    announce(f"check build decode {w}")
    assert lib.attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           ws.data_ptr(), ws_bytes, w.B, w.H, w.Hkv, w.nq, w.nk, w.d, w.dv,
                           A.DTYPE_CODES[q.dtype], float(w.c), A.MASK_CODES[w.mask], w.window,
                           A._stream_handle(None)) == 0
    torch.cuda.synchronize()
    return o, lse


CASES = [
    WORKLOADS["page_d64"].replace(backward=True),
    WORKLOADS["page_d128"].replace(H=8, backward=True),
    Workload("small", 1, 3, 200, 64, 64, "bf16", "window", window=50, seed=71),
    Workload("small", 2, 2, 333, 128, 128, "f16", "causal", seed=73),
    Workload("small", 1, 2, 130, 64, 64, "bf16", "none", seed=79),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-{w.d}-{w.mask}-{w.n}")
def test_poison_build_bitwise(w):
    inp = make_inputs(w, with_grad=True)
    ref = fwd_bwd(A.load_library(), w, inp)
    got = fwd_bwd(A.load_check_library("poison"), w, inp)
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), name


@pytest.mark.parametrize("name", ["decode_7b", "decode_verify"])
def test_poison_build_decode_bitwise(name):
    w = DECODE_WORKLOADS[name].replace(B=4)
    inp = make_decode_inputs(w)
    ref = decode(A.load_library(), w, inp)
    got = decode(A.load_check_library("poison"), w, inp)
    for a, b in zip(got, ref):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


def close(a, b, what):
    a, b = to64(a), to64(b)
    if what == "O":
        assert np.max(np.abs(a - b)) <= TOL_O_16, what
    elif what == "LSE":
        assert np.max(np.abs(a - b)) <= TOL_LSE_16, what
    else:
        a = a.reshape(-1, *a.shape[-2:])
        b = b.reshape(-1, *b.shape[-2:])
        for s in range(a.shape[0]):
            ref = max(float(np.max(np.abs(b[s]))), 1e-3)
            assert float(np.max(np.abs(a[s] - b[s]))) / ref <= TOL_GRAD_16, (what, s)


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.name}-{w.d}-{w.mask}-{w.n}")
def test_other_tile_shapes_agree(w):
    inp = make_inputs(w, with_grad=True)
    ref = fwd_bwd(A.load_library(), w, inp)
    got = fwd_bwd(A.load_check_library("alt"), w, inp)
    differ = False
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(a).all(), name
        close(a, b, name)
        differ = differ or not torch.equal(a, b)
    assert differ, "the tile-shape build computed bitwise the same values: shapes not changed?"
    if w.n <= 400:
        # the other build against the oracle, every row
        q, k, v, do = (to64(inp[x]) for x in ("q", "k", "v", "do"))
        y, _, _, lref = oracle.fwd(q, k, v, w.c, w.mask, w.window)
        check_fwd(to64(got[0]), to64(got[1]), y, lref, got[0].dtype, "alt tiles")
        gq, gk, gv, _, _, _ = oracle.bwd(q, k, v, do, w.c, w.mask, w.window)
        for g, r, nm in zip(got[2:], (gq, gk, gv), ("dQ", "dK", "dV")):
            check_grad(to64(g), r, g.dtype, f"alt tiles {nm}")


@pytest.mark.parametrize("w", [WORKLOADS["page_d64"].replace(H=8),
                               Workload("small", 2, 3, 333, 128, 128, "bf16", "causal", seed=83),
                               Workload("small", 1, 2, 300, 64, 64, "f16", "window", window=70,
                                        seed=89)],
                         ids=lambda w: f"{w.name}-{w.d}-{w.mask}-{w.n}")
def test_timing_build(w):
    inp = make_inputs(w, with_grad=True)
    ref = fwd_bwd(A.load_library(), w, inp)
    lib = A.load_check_library("timing")
    fns = (lib.eiat_wg_times, lib.eiat_wg_times_dq, lib.eiat_wg_times_dkdv)
    for fn in fns:
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
        fn.restype = ctypes.c_int
    got = fwd_bwd(lib, w, inp)
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), name
    # forward and dQ: 128 query rows per workgroup; dK/dV: 128 keys
    grid = w.B * w.H * ((w.n + 127) // 128)
    for fn in fns:
        buf = np.zeros(6 * grid, np.uint64)
        khz = ctypes.c_int(0)
        assert fn(buf.ctypes.data, buf.nbytes, ctypes.byref(khz)) == 0
        assert khz.value > 0
        r = buf.reshape(grid, 6).astype(np.int64)
        assert (r[:, 0] > 0).all(), "a workgroup left no stamp"
        assert (r[:, 0] <= r[:, 1]).all() and (r[:, 1] <= r[:, 2]).all()
        span_us = (r[:, 2].max() - r[:, 0].min()) * 1e3 / khz.value
        assert 0 < span_us < 1e6
        assert (r[:, 5] >= r[:, 4]).all()  # shader clock counter, start to end


def test_wg_timeline_summary():
    """The workgroup-timeline summary runs end to end on a small workload."""
    from exact_io_aware_tiled_amd import wg_timeline

    lib = A.load_check_library("timing")
    for fn in (lib.eiat_wg_times, lib.eiat_wg_times_dq, lib.eiat_wg_times_dkdv):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
        fn.restype = ctypes.c_int
    for spec in ("smoke", "smoke:dq", "smoke:dkdv"):
        announce(f"wg_timeline {spec}")
        out = wg_timeline.timeline(lib, spec, warm_s=0.05)
        for key in ("span", "slot use", "prologue", "steady rate", "clock"):
            assert key in out, out
