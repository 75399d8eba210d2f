#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM: the forward (attn_fwd: O and LSE) followed by the
two kernels of the backward in attn_bwd's order (dQ, which also forms the
per-row delta, then dK/dV; called through attn_bwd_stage so each kernel can be
timed on its own).  Default workload: batch 1, 32 heads,
n = 4096, d = v = 64, bf16, causal, c = 1/8.

Timing: --settle-s seconds (default 0.3) of untimed back-to-back steps, so
that the engine clock has settled under sustained load, then --warmup untimed
steps, then --steps timed steps (the line's `settle` records the first phase).

Prints ONE JSON line on stdout.  `value` is whole-step algorithmic TFLOP/s with
the FLOP convention: forward 4 d per allowed (query, key) pair (two products
of 2 d), backward 2.5 x forward.  `roofline` is for the kernel with the largest
share of the step time, from HIP events recorded around every launch in the
timed region, against the MI355X dense bf16/fp16 MFMA peak.  `cpu_baseline`
times the fp64 CPU oracle (the test reference, never tuned) on whole heads of
the same workload within a bounded time budget.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd/bwd attention TFLOP/s, n=4096 d=64 bf16 causal; % of MFMA peak"
# MI355X published dense peaks (TFLOP/s): bf16 / fp16 MFMA, fp32 MFMA, fp8 MFMA
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "fp8": 5033.2}
# The FP8-score forward runs half its work (S = Q K^T) on the fp8 peak and half
# (P V) on the 16-bit peak: its ceiling is the harmonic combination.
PEAK_FP8_FWD = 1.0 / (0.5 / PEAK_TFLOPS["fp8"] + 0.5 / PEAK_TFLOPS["bf16"])
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["attn_device.h", "attn_internal.h", "attn_bwd_common.h", "attn_fwd.hip",
                  "attn_bwd.hip", "attn_bwd_dq.hip", "attn_decode.hip", "attn_fp8.hip"]
DECODE_METRIC = ("decode attention GB/s: algorithmic HBM bytes (Q, K, V read once, O and LSE "
                 "written once) per second")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def allowed_pairs(n: int, mask: str, window: int) -> int:
    """Number of allowed (query, key) pairs of one head."""
    if mask == "none":
        return n * n
    if mask == "causal":
        return n * (n + 1) // 2
    w = min(window, n)
    return w * (w + 1) // 2 + (n - w) * w


def convention_pairs(n: int, mask: str, window: int) -> float:
    """Pairs used by the headline FLOP convention: n^2 / 2 for causal, as quoted."""
    if mask == "causal":
        return n * n / 2.0
    return float(allowed_pairs(n, mask, window))


def sources_digest() -> str:
    """Hash of the kernel sources with comments removed, of the compile flags
    (common and per source) and of the target architecture: a change to the
    code or to how it is compiled invalidates the committed counter summaries,
    a change to a comment does not."""
    from exact_io_aware_tiled_amd import build as _build
    h = hashlib.sha256()
    h.update(repr(sorted(_build.PER_SOURCE_FLAGS.items())).encode())
    h.update(repr([f for f in _build.CFLAGS if not f.startswith("-I")]).encode())
    h.update(_build.ARCH.encode())
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_io_aware_tiled_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def _counter_entry(kernel: str, workload) -> dict | None:
    """The committed rocprofv3 counter summary of `kernel` on this exact
    workload, if it was taken on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("sources_sha") != sources_digest():
        return None
    return data.get("workloads", {}).get(repr(workload), {}).get("kernels", {}).get(kernel)


def load_traffic(kernel: str, workload) -> float | None:
    """Counter-derived HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated)."""
    entry = _counter_entry(kernel, workload)
    return entry.get("bytes_per_launch") if entry else None


def load_activity(kernel: str, workload) -> dict | None:
    """MFMA busy share, LDS bank-conflict stall share and VALU/MFMA instruction
    ratio of `kernel` from the committed rocprofv3 pass."""
    entry = _counter_entry(kernel, workload)
    act = entry.get("activity") if entry else None
    return {"kernel": kernel, **act, "source": "profiles/attn_activity_counters.txt"} if act else None


def device_info(torch, kernel: str | None = None, workload=None) -> dict:
    """The GPU the run sees: compute units and peak engine clock reported by the
    HIP runtime, the dense 16-bit MFMA peak they imply (CUs x 4096 FLOP/clk x
    clock), and, when the committed counter summary of `kernel` on this
    workload is current, the engine clock observed under that kernel (its
    GRBM_GUI_ACTIVE cycles over its traced duration) with the peak at that clock.
    The roofline fraction itself stays against the published peak."""
    import ctypes

    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "max_sclk_mhz": None}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, dev) == 0:  # hipDeviceAttributeClockRate (kHz)
            info["max_sclk_mhz"] = round(val.value / 1000.0, 1)
    except OSError:
        pass
    if info["max_sclk_mhz"]:
        info["mfma16_peak_at_max_sclk_tflops"] = round(
            info["cus"] * 4096 * info["max_sclk_mhz"] * 1e6 / 1e12, 1)
    entry = _counter_entry(kernel, workload) if kernel else None
    act = entry.get("activity") if entry else None
    if act and act.get("sclk_mhz"):
        info["observed_sclk_mhz"] = act["sclk_mhz"]
        info["mfma16_peak_at_observed_sclk_tflops"] = round(
            info["cus"] * 4096 * act["sclk_mhz"] * 1e6 / 1e12, 1)
        info["observed_sclk_source"] = "profiles/attn_activity_counters.txt"
    return info


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle (fwd + VJP) on whole heads of the workload until budget_s."""
    import oracle
    from exact_io_aware_tiled_amd.inputs import make_inputs

    inp = make_inputs(w, with_grad=True)
    flat = {x: inp[x].reshape(-1, w.n, inp[x].shape[-1]) for x in ("q", "k", "v", "do")}
    f64 = lambda t: t.double().numpy()  # noqa: E731
    per_head = 4.0 * w.d * convention_pairs(w.n, w.mask, w.window) * 3.5  # fwd + 2.5 x fwd
    heads, t_total = 0, 0.0
    for h in range(flat["q"].shape[0]):
        args = [f64(flat[x][h]) for x in ("q", "k", "v", "do")]
        t0 = time.perf_counter()
        oracle.bwd(*args, w.c, w.mask, w.window)  # dense forward + analytic VJP
        t_total += time.perf_counter() - t0
        heads += 1
        if t_total >= budget_s:
            break
    total_heads = flat["q"].shape[0]
    return {
        "value": per_head * heads / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"fp64 dense oracle, forward + VJP, {heads} of {total_heads} heads of the "
                   f"same workload (n={w.n}, d={w.d}, {w.mask}); {t_total:.2f} s; "
                   f"full-workload time at this rate {t_total * total_heads / heads:.1f} s"),
    }


def fp8_cpu_baseline(w, budget_s: float, signs, values: bool = False):
    """The oracle's FP8 path on whole heads: quantize Q and K (rotation and
    block scales; with `values` also V along the keys), dequantize, fp64
    forward with c / d."""
    import torch

    import oracle
    from exact_io_aware_tiled_amd.inputs import make_inputs

    inp = make_inputs(w)
    flat = {k_: t.reshape(-1, w.n, t.shape[-1]).to(torch.float64).numpy() for k_, t in inp.items()}
    sg = signs.cpu().numpy()
    per_head = 4.0 * w.d * convention_pairs(w.n, w.mask, w.window)
    heads, t_total = 0, 0.0
    for hh in range(flat["q"].shape[0]):
        t0 = time.perf_counter()
        qd = oracle.mx_dequant(*oracle.mx_quant(flat["q"][hh], sg))
        kd = oracle.mx_dequant(*oracle.mx_quant(flat["k"][hh], sg))
        vv = flat["v"][hh]
        if values:
            vv = oracle.mx_dequant(*oracle.mx_quant(vv.T)).T
        oracle.fwd(qd[None], kd[None], vv[None], w.c / w.d, w.mask, w.window)
        t_total += time.perf_counter() - t0
        heads += 1
        if t_total >= budget_s:
            break
    total_heads = flat["q"].shape[0]
    return {
        "value": per_head * heads / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"oracle FP8 quantizer{' (Q, K, V)' if values else ' (Q, K)'} + fp64 dense "
                   f"forward, {heads} of {total_heads} heads "
                   f"of the same workload (n={w.n}, d={w.d}, {w.mask}); {t_total:.2f} s"),
    }


def bench_fp8(args, w):
    """Forward with FP8 scores: a step quantizes Q and K from the 16-bit inputs
    (rotation with one random sign vector, E8M0 block scales) and runs the FP8
    forward; every kernel is timed on its own."""
    import torch

    from exact_io_aware_tiled_amd import attn
    from exact_io_aware_tiled_amd.inputs import DTYPES, FP8_SIGNS_SEED, make_inputs, make_signs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = attn.load_library()
    inp = make_inputs(w, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, n, d, dv = w.B, w.H, w.n, w.d, w.dv
    dt = DTYPES[w.dtype]
    signs = make_signs(d, FP8_SIGNS_SEED).to(dev)
    q8 = torch.empty(B, H, n, d, dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    qs = torch.empty(B, H, n, d // 32, dtype=torch.uint8, device=dev)
    ks = torch.empty_like(qs)
    o = torch.empty(B, H, n, dv, dtype=dt, device=dev)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    pv8 = bool(args.fp8_values)
    nt = (n + 63) // 64
    v8 = torch.empty(B, H, nt, dv, 64, dtype=torch.uint8, device=dev)
    vs = torch.empty(B, H, nt, dv, 2, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = attn._stream_handle(stream)
    dcode, mcode = attn.DTYPE_CODES[dt], attn.MASK_CODES[w.mask]
    rows = B * H * n

    def chk(s):
        if s:
            raise attn.AttnError(s, lib.attn_last_error().decode())

    def quant(x, codes, scales):
        chk(lib.attn_quant_fp8(x.data_ptr(), signs.data_ptr(), codes.data_ptr(),
                               scales.data_ptr(), rows, d, dcode, sh))

    def fwd8():
        if pv8:
            chk(lib.attn_fwd_fp8_pv(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                                    v8.data_ptr(), vs.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                                    H, n, d, dv, dcode, float(w.c) / d, mcode, w.window, sh))
        else:
            chk(lib.attn_fwd_fp8(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                                 v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, n, d, dv, dcode,
                                 float(w.c) / d, mcode, w.window, sh))

    def quant_v():
        chk(lib.attn_quant_fp8_v(v.data_ptr(), v8.data_ptr(), vs.data_ptr(), B * H, n, dv, dcode,
                                 sh))

    kernels = [("quant_q", lambda: quant(q, q8, qs)), ("quant_k", lambda: quant(k, k8, ks))]
    if pv8:
        kernels.append(("quant_v", quant_v))
    fwd_name = "attn_fwd_fp8_pv" if pv8 else "attn_fwd_fp8"
    kernels.append((fwd_name, fwd8))
    log(f"bench: fp8 workload {w}")
    K = args.steps
    ms_per_step, kern_ms = time_kernels(torch, kernels, args.warmup, K, stream, args.settle_s)
    log("bench: kernel ms " + json.dumps({k_: round(v_, 4) for k_, v_ in kern_ms.items()}))

    bh = B * H
    pairs = allowed_pairs(n, w.mask, w.window) * bh
    conv_fwd = 4.0 * d * convention_pairs(n, w.mask, w.window) * bh
    value = conv_fwd / (ms_per_step * 1e-3) / 1e12
    e = 2 if dt != torch.float32 else 4
    qbytes = float(rows * d * (e + 1) + rows * (d // 32) + d)  # read x, signs; write codes, scales
    vbytes = float(rows * dv * e + B * H * nt * dv * (64 + 2))  # read V; write the tile layout
    work = {"quant_q": ("hbm", qbytes), "quant_k": ("hbm", qbytes), "quant_v": ("hbm", vbytes),
            fwd_name: ("mfma", 4.0 * d * pairs)}
    per_kernel = {}
    for name, ms in kern_ms.items():
        b_, amt = work[name]
        rate = amt / (ms * 1e-3) / (1e12 if b_ == "mfma" else 1e9)
        per_kernel[name] = {"ms": round(ms, 4), "bound": b_,
                            ("tflops" if b_ == "mfma" else "gbs"): round(rate, 2)}
    dom = fwd_name
    achieved = work[dom][1] / (kern_ms[dom] * 1e-3) / 1e12
    peak = PEAK_TFLOPS["fp8"] if pv8 else PEAK_FP8_FWD  # both products on FP8, or S only
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
            "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": load_traffic(dom, w)}
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)
    cpu = fp8_cpu_baseline(w, args.cpu_budget, signs, pv8) if args.cpu_budget > 0 else None
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": dict(SETTLE),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"fp8-e4m3 scores, weights and values (E8M0 block scales), {w.dtype} O" if pv8
                  else f"fp8-e4m3 scores (E8M0 block scales), {w.dtype} P and V"),
        "data": "synthetic (seeded N(0,1) Q, K, V; seeded random signs)",
        "config": {"workload": (f"{w.name}: B={B} H={H} n={n} d=v={d} {w.dtype} {w.mask}, forward "
                                + ("with FP8 scores, weights and values: quantize Q, K and V + FP8 "
                                   "forward" if pv8 else
                                   "with FP8 scores: quantize Q and K + FP8 forward")),
                   "global_batch": B, "seq_len": n, "heads": H, "head_dim": d,
                   "mask": w.mask, "parallelism": "none (1 GPU)"},
        "fwd_tflops": round(conv_fwd / (kern_ms[dom] * 1e-3) / 1e12, 2),
        "kernels": per_kernel,
        "roofline": roof,
        "counters": load_activity(dom, w),
        "device": device_info(torch, dom, w),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_calibration(torch, dev, mib: int):
    """One plain device copy of `mib` MiB, the reference the HBM counters are scaled by."""
    nbytes = mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy calibration {nbytes} bytes read, {nbytes} bytes written")


SETTLE = {"seconds": 0.0, "steps": 0}


def time_kernels(torch, kernels, warmup: int, steps: int, stream, settle_s: float = 0.0):
    """Run `steps` timed steps (each: every kernel once, in order) after
    `warmup` untimed ones; per-kernel mean ms from HIP events on `stream`,
    and the wall-clock ms per step.

    Before the warmup steps, steps run back to back for `settle_s` seconds
    (untimed; recorded in SETTLE).  The engine clock takes tens of
    milliseconds of sustained load to settle: on MI355X the page step ran
    at 351 us right after start, 385-408 us 10-16 ms in, and 337 us from
    about 30 ms on.  A few warmup steps of a sub-millisecond step end inside
    that transient, so without the settle phase the timed steps measure the
    power management's ramp rather than the kernels' sustained rate."""
    def step(evs=None):
        for i, (_, fn) in enumerate(kernels):
            if evs is not None:
                evs[i].record(stream)
            fn()
        if evs is not None:
            evs[len(kernels)].record(stream)

    n_settle = 0
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        n_settle += 4
        torch.cuda.synchronize()
    SETTLE.update(seconds=settle_s, steps=n_settle)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
              for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(events[s_])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    kern_ms = {name: sum(events[s_][i].elapsed_time(events[s_][i + 1]) for s_ in range(steps)) / steps
               for i, (name, _) in enumerate(kernels)}
    return ms_per_step, kern_ms


def decode_cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle's decode rows on whole key/value-head groups of batch
    entry 0 until budget_s; rate in the metric's unit (algorithmic bytes / s)."""
    import oracle
    from exact_io_aware_tiled_amd.inputs import make_decode_inputs

    inp = make_decode_inputs(w)
    G = w.H // w.Hkv
    e = 2
    f64 = lambda t: t.double().numpy()  # noqa: E731
    groups, t_total, nbytes = 0, 0.0, 0.0
    for g in range(w.Hkv):
        q = f64(inp["q"][:1, g * G:(g + 1) * G])
        k = f64(inp["k"][:1, g:g + 1])
        v = f64(inp["v"][:1, g:g + 1])
        t0 = time.perf_counter()
        oracle.decode(q, k, v, w.c, w.mask, w.window)
        t_total += time.perf_counter() - t0
        groups += 1
        nbytes += (G * w.nq * (w.d + w.dv) + w.nk * (w.d + w.dv)) * e + G * w.nq * 4
        if t_total >= budget_s:
            break
    return {
        "value": nbytes / t_total / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"fp64 dense oracle decode rows, {groups} of {w.B * w.Hkv} key/value-head "
                   f"groups (batch entry 0) of the same workload; {t_total:.2f} s"),
    }


def bench_decode(args, w):
    import torch

    from exact_io_aware_tiled_amd import attn
    from exact_io_aware_tiled_amd.inputs import make_decode_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_decode_inputs(w, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.empty(w.B, w.H, w.nq, w.dv, dtype=q.dtype, device=dev)
    lse = torch.empty(w.B, w.H, w.nq, dtype=torch.float32, device=dev)
    ws = torch.empty(max(attn.attn_decode_workspace_bytes(w.B, w.H, w.Hkv, w.nq, w.nk, w.dv), 16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def stage(s_):
        return lambda: attn.attn_decode(q, k, v, w.c, w.mask, w.window, out=o, lse=lse,
                                        workspace=ws, stream=stream, stage=s_)

    log(f"bench: decode workload {w}")
    kernels = [("decode_split", stage(0)), ("decode_merge", stage(1))]
    ms_per_step, kern_ms = time_kernels(torch, kernels, args.warmup, args.steps, stream, args.settle_s)
    log("bench: kernel ms " + json.dumps({k_: round(v_, 4) for k_, v_ in kern_ms.items()}))

    e = q.element_size()
    q_b = w.B * w.H * w.nq * w.d * e
    kv_b = w.B * w.Hkv * w.nk * (w.d + w.dv) * e
    out_b = w.B * w.H * w.nq * w.dv * e + w.B * w.H * w.nq * 4
    work = {"decode_split": q_b + kv_b, "decode_merge": out_b}
    value = (q_b + kv_b + out_b) / (ms_per_step * 1e-3) / 1e9
    per_kernel = {name: {"ms": round(ms, 4), "bound": "hbm",
                         "gbs": round(work[name] / (ms * 1e-3) / 1e9, 1)}
                  for name, ms in kern_ms.items()}
    dom = max(kern_ms, key=kern_ms.get)
    achieved = work[dom] / (kern_ms[dom] * 1e-3) / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(dom, w)}
    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)
    cpu = decode_cpu_baseline(w, args.cpu_budget) if args.cpu_budget > 0 else None
    line = {
        "metric": DECODE_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": dict(SETTLE),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V)",
        "config": {"workload": (f"{w.name}: B={w.B} H={w.H} Hkv={w.Hkv} nq={w.nq} nk={w.nk} "
                                f"d=v={w.d} {w.dtype} {w.mask}"),
                   "global_batch": w.B, "seq_len": w.nk, "heads": w.H, "kv_heads": w.Hkv,
                   "new_rows": w.nq, "head_dim": w.d, "mask": w.mask,
                   "parallelism": "none (1 GPU)"},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "kernels": per_kernel,
        "roofline": roof,
        "counters": load_activity(dom, w),
        "device": device_info(torch, dom, w),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed back-to-back steps before the warmup steps, so that "
                         "the engine clock has settled under load (0 disables)")
    ap.add_argument("--workload", default="page_d64")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward alone")
    ap.add_argument("--p-drop", type=float, default=0.0,
                    help="dropout probability on the weights (attn_fwd_dropout / attn_bwd_dropout)")
    ap.add_argument("--seed", type=int, default=1, help="dropout mask seed")
    ap.add_argument("--fp8", action="store_true",
                    help="forward with FP8 scores (attn_quant_fp8 on Q and K, then attn_fwd_fp8)")
    ap.add_argument("--fp8-values", action="store_true",
                    help="with --fp8: FP8 weights and values too (attn_quant_fp8_v on V, then "
                         "attn_fwd_fp8_pv)")
    ap.add_argument("--set", action="append", default=[], metavar="KEY=VALUE",
                    help="override a workload field, e.g. --set n=16384 --set mask=none")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py: --gpus {args.gpus} (WORLD_SIZE {world}) requested, but this benchmark runs "
            "on exactly one GPU: the attention path has no multi-GPU code. Run with --gpus 1.")
        sys.exit(2)

    import torch

    from exact_io_aware_tiled_amd import attn
    from exact_io_aware_tiled_amd.inputs import DECODE_WORKLOADS, DTYPES, WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload in DECODE_WORKLOADS:
        w = DECODE_WORKLOADS[args.workload]
        for kv in args.set:
            key, val = kv.split("=", 1)
            cur = getattr(w, key)
            w = w.replace(**{key: type(cur)(val) if cur is not None else float(val)})
        bench_decode(args, w)
        return
    w = WORKLOADS[args.workload]
    for kv in args.set:
        key, val = kv.split("=", 1)
        cur = getattr(w, key)
        w = w.replace(**{key: type(cur)(val) if cur is not None else float(val)})
    if args.fp8:
        bench_fp8(args, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = attn.load_library()

    inp = make_inputs(w, with_grad=True, device=dev)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    B, H, n, d, dv = w.B, w.H, w.n, w.d, w.dv
    dt = DTYPES[w.dtype]
    o = torch.empty(B, H, n, dv, dtype=dt, device=dev)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = max(attn.attn_bwd_workspace_bytes(B, H, n), 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = attn._stream_handle(stream)
    dcode, mcode = attn.DTYPE_CODES[dt], attn.MASK_CODES[w.mask]
    c = float(w.c)

    pdrop, seed = float(args.p_drop), int(args.seed)

    def fwd():
        fa = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, n, d, dv,
              dcode, c, mcode, w.window)
        s = lib.attn_fwd_dropout(*fa, pdrop, seed, sh) if pdrop else lib.attn_fwd(*fa, sh)
        if s:
            raise attn.AttnError(s, lib.attn_last_error().decode())

    def bwd_stage(stage):
        ba = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dvv.data_ptr(), ws.data_ptr(),
              ws_bytes, B, H, n, d, dv, dcode, c, mcode, w.window)
        if pdrop:
            s = lib.attn_bwd_dropout_stage(stage, *ba, pdrop, seed, sh)
        else:
            s = lib.attn_bwd_stage(stage, *ba, sh)
        if s:
            raise attn.AttnError(s, lib.attn_last_error().decode())

    kernels = [("attn_fwd", fwd)]
    if not args.fwd_only:
        kernels += [("bwd_dq", lambda: bwd_stage(2)), ("bwd_dkdv", lambda: bwd_stage(1))]

    log(f"bench: workload {w}")
    K = args.steps
    ms_per_step, kern_ms = time_kernels(torch, kernels, args.warmup, K, stream, args.settle_s)
    log("bench: kernel ms " + json.dumps({k_: round(v_, 4) for k_, v_ in kern_ms.items()}))

    bh = B * H
    pairs = allowed_pairs(n, w.mask, w.window) * bh
    conv_fwd = 4.0 * d * convention_pairs(n, w.mask, w.window) * bh
    conv_bwd = 2.5 * conv_fwd
    step_flops = conv_fwd + (0.0 if args.fwd_only else conv_bwd)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # algorithmic work per launch of each kernel
    work = {
        "attn_fwd": ("mfma", 4.0 * d * pairs),      # S and P V
        "bwd_dkdv": ("mfma", 8.0 * d * pairs),      # S, dP, dV, dK
        "bwd_dq": ("mfma", 6.0 * d * pairs),        # S, dP, dQ (and delta, O . dO per row)
    }
    dom = max(kern_ms, key=kern_ms.get)
    bound, amount = work[dom]
    if bound == "mfma":
        achieved = amount / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = amount / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = None if pdrop else load_traffic(dom, w)  # counters were taken without dropout

    per_kernel = {}
    for name, ms in kern_ms.items():
        b_, amt = work[name]
        rate = amt / (ms * 1e-3) / (1e12 if b_ == "mfma" else 1e9)
        per_kernel[name] = {"ms": round(ms, 4), "bound": b_,
                            ("tflops" if b_ == "mfma" else "gbs"): round(rate, 2)}

    if args.copy_calibration:
        copy_calibration(torch, dev, args.copy_calibration)

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(w, args.cpu_budget)

    fwd_ms = kern_ms["attn_fwd"]
    bwd_ms = sum(v_ for k_, v_ in kern_ms.items() if k_ != "attn_fwd")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": dict(SETTLE),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V, dO)",
        "config": {"workload": f"{w.name}: B={B} H={H} n={n} d=v={d} {w.dtype} {w.mask}"
                               + ("" if args.fwd_only else ", forward + backward")
                               + (f", dropout p={pdrop}" if pdrop else ""),
                   "global_batch": B, "seq_len": n, "heads": H, "head_dim": d,
                   "mask": w.mask, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_tflops": round(conv_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": None if args.fwd_only else round(conv_bwd / (bwd_ms * 1e-3) / 1e12, 2),
        "kernels": per_kernel,
        "roofline": roof,
        "counters": None if pdrop else load_activity(dom, w),
        "device": device_info(torch, dom, w),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
