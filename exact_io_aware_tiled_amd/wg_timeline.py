"""Workgroup timeline of one kernel launch, from the timing check build.

    python -m exact_io_aware_tiled_amd.wg_timeline page_d64 page_d128 long_causal
    python -m exact_io_aware_tiled_amd.wg_timeline page_d64:dq page_d64:dkdv

libeiat_attn_timing.so (build.py, CHECK_BUILDS) is the product build with
per-workgroup wall-clock stamps in the forward, dQ and dK/dV kernels: start,
end of the prologue (forward: Q loaded, the first key/value tiles in LDS, the
first score block formed; dQ: the first key/value tile in LDS; dK/dV: the key
tile's K and V and the first query tile in place) and end, plus the CU and XCD
each workgroup ran on.  A workload name alone times the forward; ":dq" and
":dkdv" time that backward kernel (after one forward and, for dK/dV, one dQ
launch that forms delta).  For each, the kernel runs back to back for half a
second (so that the clock has settled under load) and one further launch is
summarised:

  span          first start to last end
  slots         most workgroups resident at once
  slot use      sum of workgroup durations / (span x slots): the share of the
                span the resident slots were busy (1 - tail and refill gaps)
  prologue      start -> first score block, per workgroup
  fit           workgroup duration = a + b x (keys it visits; for dK/dV the
                query rows it visits): a is the fixed cost per workgroup
                (prologue, diagonal, epilogue), b the steady-state time per key
                (row); the steady rate is the algorithmic FLOP rate of all
                slots streaming at b
  clock         shader clock cycles / wall time over each workgroup: the
                engine clock under the full load of the launch
  spread        per-XCD median workgroup time and the CUs' last-end times

Every input is the seeded synthetic workload of inputs.py; nothing is timed
but the one kernel.
"""
from __future__ import annotations

import ctypes
import sys
import time

import numpy as np
import torch

from exact_io_aware_tiled_amd import attn as A
from exact_io_aware_tiled_amd.inputs import DTYPES, WORKLOADS, make_inputs

BM = 128    # query rows per forward or dQ workgroup
BNK = 128   # keys per dK/dV workgroup
WORDS = 6   # stamps per workgroup (WgStamps in attn_device.h, EIAT_WG_TIMING)
# Algorithmic FLOP per (query row, allowed key) pair and head dimension: the
# forward's two products, dQ's three (S, dP, dQ), dK/dV's four (S, dP, dV, dK).
FLOP_PER_PAIR_D = {"fwd": 4.0, "dq": 6.0, "dkdv": 8.0}


def visible_keys(n: int, mask: str, window: int, qt: np.ndarray) -> np.ndarray:
    """Keys any row of query tile qt may see (the workgroup's key range)."""
    q0 = qt * BM
    end = np.minimum(n, q0 + BM) if mask != "none" else np.full_like(qt, n)
    beg = np.maximum(0, q0 - window + 1) if mask == "window" else np.zeros_like(qt)
    return end - beg


def visible_rows(n: int, mask: str, window: int, kt: np.ndarray) -> np.ndarray:
    """Query rows any key of key tile kt may be seen by (a dK/dV workgroup's range)."""
    k0 = kt * BNK
    beg = k0 if mask != "none" else np.zeros_like(kt)
    end = np.minimum(n, k0 + BNK - 1 + window) if mask == "window" else np.full_like(kt, n)
    return end - beg


def timeline(lib, spec: str, warm_s: float = 0.5) -> str:
    name, _, kernel = spec.partition(":")
    kernel = kernel or "fwd"
    if kernel not in FLOP_PER_PAIR_D:
        raise ValueError(f"{spec}: kernel must be fwd, dq or dkdv")
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = make_inputs(w, with_grad=kernel != "fwd", device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, n, d = q.shape
    dt = DTYPES[w.dtype]
    o = torch.empty(B, H, n, d, dtype=dt, device=dev)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    bh = B * H
    ntiles = (n + (BNK if kernel == "dkdv" else BM) - 1) // (BNK if kernel == "dkdv" else BM)
    grid = ntiles * bh
    if grid > 65536:
        raise ValueError(f"{spec}: {grid} workgroups, more than the 65536 the build records")
    sh = A._stream_handle(None)
    args = (B, H, n, d, d, A.DTYPE_CODES[dt], float(w.c), A.MASK_CODES[w.mask], w.window, sh)

    def check(s):
        if s:
            raise A.AttnError(s, lib.attn_last_error().decode())

    def fwd():
        check(lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           *args))

    if kernel == "fwd":
        run, times = fwd, lib.eiat_wg_times
    else:
        do = inp["do"]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = max(lib.attn_bwd_workspace_bytes(B, H, n), 16)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def stage(st):
            check(lib.attn_bwd_stage(st, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), ws.data_ptr(), ws_bytes, *args))

        fwd()
        stage(2)                                          # dQ, which also forms delta
        run = (lambda: stage(2)) if kernel == "dq" else (lambda: stage(1))
        times = lib.eiat_wg_times_dq if kernel == "dq" else lib.eiat_wg_times_dkdv

    # Back-to-back launches for warm_s seconds first: the engine clock settles
    # under sustained load (the first launches after idle run at another
    # clock), then the recorded launch.
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            run()
        torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    buf = np.zeros(WORDS * grid, np.uint64)
    khz = ctypes.c_int(0)
    e = times(buf.ctypes.data, buf.nbytes, ctypes.byref(khz))
    if e:
        raise RuntimeError(f"{spec}: copying the stamps failed, hip error {e}")
    r = buf.reshape(grid, WORDS).astype(np.int64)
    us = 1e3 / khz.value                                  # microseconds per tick
    t0 = (r[:, 0] - r[:, 0].min()) * us
    t1 = (r[:, 1] - r[:, 0].min()) * us
    t2 = (r[:, 2] - r[:, 0].min()) * us
    hw, xcc = r[:, 3] & 0xFFFFFFFF, (r[:, 3] >> 32) & 0xF
    cu = xcc * 1024 + ((hw >> 13) & 7) * 64 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
    bid = np.arange(grid)
    if kernel == "dkdv":
        keys = visible_rows(n, w.mask, w.window, bid // bh)   # key tiles, heaviest first
    else:
        qt = bid // bh
        if w.mask != "none":
            qt = ntiles - 1 - qt                          # heaviest query tiles first
        keys = visible_keys(n, w.mask, w.window, qt)
    dur = t2 - t0
    span = t2.max()
    mhz = (r[:, 5] - r[:, 4]) / np.maximum(dur, 1e-9)     # shader clock cycles per microsecond
    xmhz = [np.median(mhz[xcc == x]) for x in range(int(xcc.max()) + 1)]
    events = np.concatenate([np.stack([t0, np.ones(grid)], 1), np.stack([t2, -np.ones(grid)], 1)])
    events = events[np.lexsort((events[:, 1], events[:, 0]))]
    slots = int(np.cumsum(events[:, 1]).max())
    use = dur.sum() / (span * slots)
    A_ = np.stack([np.ones(grid), keys], 1)
    (a, b), *_ = np.linalg.lstsq(A_, dur, rcond=None)
    per_pair = FLOP_PER_PAIR_D[kernel] * d
    flop_per_key = per_pair * (BNK if kernel == "dkdv" else BM)  # one key (row) for all the tile's rows (keys)
    steady = slots * flop_per_key / (b * 1e-6) / 1e12
    pairs = {"none": n * n, "causal": n * (n + 1) // 2}.get(w.mask)
    if pairs is None:
        W = min(w.window, n)
        pairs = W * (W + 1) // 2 + (n - W) * W
    rate = per_pair * pairs * bh / (span * 1e-6) / 1e12
    last = {}
    for c_, e_ in zip(cu.tolist(), t2.tolist()):
        last[c_] = max(last.get(c_, 0.0), e_)
    le = np.array(sorted(last.values()))
    per_xcd = [np.median(dur[xcc == x]) for x in range(int(xcc.max()) + 1)]
    unit = "rows" if kernel == "dkdv" else "keys"
    what = {"fwd": "forward", "dq": "dQ", "dkdv": "dK/dV"}[kernel]
    lines = [
        f"== {spec}: {what}, B={B} H={H} n={n} d={d} {w.dtype} {w.mask}; {grid} workgroups on "
        f"{len(last)} CUs",
        f"   span {span:8.1f} us   rate {rate:7.1f} TFLOP/s   slots {slots}   slot use {use:.3f}",
        f"   prologue  median {np.median(t1 - t0):5.2f} us  (p10 {np.percentile(t1 - t0, 10):.2f}, "
        f"p90 {np.percentile(t1 - t0, 90):.2f})",
        f"   fit       duration = {a:6.2f} us + {b * 1024:7.3f} us per 1024 {unit}   steady rate "
        f"{steady:7.1f} TFLOP/s",
        f"   clock     {np.median(mhz):6.0f} MHz median over workgroups (per-XCD medians "
        f"{min(xmhz):.0f} .. {max(xmhz):.0f})",
        f"   spread    per-XCD median duration {min(per_xcd):.1f} .. {max(per_xcd):.1f} us; CU last "
        f"end {le[0]:.1f} (min) {np.median(le):.1f} (median) {le[-1]:.1f} (max) us",
    ]
    return "\n".join(lines)


def main(argv):
    names = argv or ["page_d64", "page_d128", "long_causal"]
    lib = A.load_check_library("timing")
    for fn in (lib.eiat_wg_times, lib.eiat_wg_times_dq, lib.eiat_wg_times_dkdv):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
        fn.restype = ctypes.c_int
    dev = torch.cuda.get_device_properties(0)
    print(f"# workgroup timelines (timing check build), {dev.name}", flush=True)
    for name in names:
        print(timeline(lib, name), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
