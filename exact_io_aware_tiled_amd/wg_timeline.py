"""Workgroup timeline of one forward launch, from the timing check build.

    python -m exact_io_aware_tiled_amd.wg_timeline page_d64 page_d128 long_causal

libeiat_attn_timing.so (build.py, CHECK_BUILDS) is the product forward with
per-workgroup wall-clock stamps: start, end of the prologue (Q loaded, the
first key/value tiles in LDS, the first score block formed) and end, plus the
CU and XCD each workgroup ran on.  For each workload this runs the forward
for half a second (so that the clock has settled under load) and summarises
one further launch:

  span          first start to last end
  slots         most workgroups resident at once
  slot use      sum of workgroup durations / (span x slots): the share of the
                span the resident slots were busy (1 - tail and refill gaps)
  prologue      start -> first score block, per workgroup
  fit           workgroup duration = a + b x (keys it visits): a is the fixed
                cost per workgroup (prologue, diagonal, epilogue), b the
                steady-state time per key; the steady rate is the algorithmic
                FLOP rate of all slots streaming keys at b
  clock         shader clock cycles / wall time over each workgroup: the
                engine clock under the full load of the launch
  spread        per-XCD median workgroup time and the CUs' last-end times

Every input is the seeded synthetic workload of inputs.py; nothing is timed
but the forward.
"""
from __future__ import annotations

import ctypes
import sys
import time

import numpy as np
import torch

from exact_io_aware_tiled_amd import attn as A
from exact_io_aware_tiled_amd.inputs import DTYPES, WORKLOADS, make_inputs

BM = 128    # query rows per forward workgroup
WORDS = 6   # stamps per workgroup (attn_fwd.hip, EIAT_WG_TIMING)


def visible_keys(n: int, mask: str, window: int, qt: np.ndarray) -> np.ndarray:
    """Keys any row of query tile qt may see (the workgroup's key range)."""
    q0 = qt * BM
    end = np.minimum(n, q0 + BM) if mask != "none" else np.full_like(qt, n)
    beg = np.maximum(0, q0 - window + 1) if mask == "window" else np.zeros_like(qt)
    return end - beg


def timeline(lib, name: str, warm_s: float = 0.5) -> str:
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = make_inputs(w, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, n, d = q.shape
    dt = DTYPES[w.dtype]
    o = torch.empty(B, H, n, d, dtype=dt, device=dev)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    nqt = (n + BM - 1) // BM
    bh = B * H
    grid = nqt * bh
    if grid > 65536:
        raise ValueError(f"{name}: {grid} workgroups, more than the 65536 the build records")
    sh = A._stream_handle(None)

    def run():
        s = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                         H, n, d, d, A.DTYPE_CODES[dt], float(w.c), A.MASK_CODES[w.mask],
                         w.window, sh)
        if s:
            raise A.AttnError(s, lib.attn_last_error().decode())

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
    e = lib.eiat_wg_times(buf.ctypes.data, buf.nbytes, ctypes.byref(khz))
    if e:
        raise RuntimeError(f"eiat_wg_times: hip error {e}")
    r = buf.reshape(grid, WORDS).astype(np.int64)
    us = 1e3 / khz.value                                  # microseconds per tick
    t0 = (r[:, 0] - r[:, 0].min()) * us
    t1 = (r[:, 1] - r[:, 0].min()) * us
    t2 = (r[:, 2] - r[:, 0].min()) * us
    hw, xcc = r[:, 3] & 0xFFFFFFFF, (r[:, 3] >> 32) & 0xF
    cu = xcc * 1024 + ((hw >> 13) & 7) * 64 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
    bid = np.arange(grid)
    qt = bid // bh
    if w.mask != "none":
        qt = nqt - 1 - qt                                 # heaviest query tiles first
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
    flop_per_key = 4.0 * d * BM                           # S and P V for the workgroup's rows
    steady = slots * flop_per_key / (b * 1e-6) / 1e12
    pairs = {"none": n * n, "causal": n * (n + 1) // 2}.get(w.mask)
    if pairs is None:
        W = min(w.window, n)
        pairs = W * (W + 1) // 2 + (n - W) * W
    rate = 4.0 * d * pairs * bh / (span * 1e-6) / 1e12
    last = {}
    for c_, e_ in zip(cu.tolist(), t2.tolist()):
        last[c_] = max(last.get(c_, 0.0), e_)
    le = np.array(sorted(last.values()))
    per_xcd = [np.median(dur[xcc == x]) for x in range(int(xcc.max()) + 1)]
    lines = [
        f"== {name}: B={B} H={H} n={n} d={d} {w.dtype} {w.mask}; {grid} workgroups on "
        f"{len(last)} CUs",
        f"   span {span:8.1f} us   rate {rate:7.1f} TFLOP/s   slots {slots}   slot use {use:.3f}",
        f"   prologue  median {np.median(t1 - t0):5.2f} us  (p10 {np.percentile(t1 - t0, 10):.2f}, "
        f"p90 {np.percentile(t1 - t0, 90):.2f})",
        f"   fit       duration = {a:6.2f} us + {b * 1024:7.3f} us per 1024 keys   steady rate "
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
    lib.eiat_wg_times.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
    lib.eiat_wg_times.restype = ctypes.c_int
    dev = torch.cuda.get_device_properties(0)
    print(f"# workgroup timelines of the forward (timing check build), {dev.name}", flush=True)
    for name in names:
        print(timeline(lib, name), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
