"""attn_bwd_noalloc (the backward with the per-row delta in the library's own
per-GPU scratch instead of a workspace) against attn_bwd through the C ABI:
bitwise the same gradients, on two calls in a row, the second smaller, so the
second call runs on the scratch the first one left behind."""
import ctypes

import pytest
import torch

from exact_io_aware_tiled_amd import attn as A
from exact_io_aware_tiled_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, n, d, dtype, mask, window): a larger call, then a smaller one
    (1, 4, 1000, 64, "bf16", "causal", 0),
    (2, 1, 300, 128, "f16", "window", 77),
]


def run_pair(lib, B, H, n, d, dt, mask, window):
    w = WORKLOADS["page_d64"].replace(B=B, H=H, n=n, d=d, dv=d, dtype=dt, mask=mask,
                                      window=window)
    dev = torch.device("cuda:0")
    inp = make_inputs(w, with_grad=True, seed=4242 + n, device=dev)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    o, lse = A.attn_fwd(q, k, v, scale=w.c, mask=mask, window=window)
    sh = A._stream_handle(None)
    code, mcode = A.DTYPE_CODES[q.dtype], A.MASK_CODES[mask]
    ref = [torch.empty_like(t) for t in (q, k, v)]
    ws_bytes = max(lib.attn_bwd_workspace_bytes(B, H, n), 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    assert lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                        lse.data_ptr(), ref[0].data_ptr(), ref[1].data_ptr(), ref[2].data_ptr(),
                        ws.data_ptr(), ws_bytes, B, H, n, d, d, code, float(w.c), mcode, window,
                        sh) == 0
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    s = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                             lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(),
                             got[2].data_ptr(), B, H, n, d, d, code, float(w.c), mcode, window, sh)
    assert s == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_noalloc_matches_attn_bwd_twice():
    lib = A.load_library()
    for case in CASES:
        print("noalloc case", case, flush=True)
        run_pair(lib, *case)


def test_noalloc_python_binding():
    w = WORKLOADS["smoke"].replace(n=130)
    dev = torch.device("cuda:0")
    inp = make_inputs(w, with_grad=True, device=dev)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    o, lse = A.attn_fwd(q, k, v, scale=w.c, mask=w.mask)
    ref = A.attn_bwd(q, k, v, o, lse, do, scale=w.c, mask=w.mask)
    got = A.attn_bwd_noalloc(q, k, v, o, lse, do, *(torch.empty_like(t) for t in (q, k, v)),
                             scale=w.c, mask=w.mask)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
