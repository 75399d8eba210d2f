"""Seeded synthetic workloads (shapes, value distributions, masks).

This module only draws random numbers and describes shapes; it holds none of the
attention arithmetic.  Both the HIP path's callers and the oracle's tests take
their inputs from here, so the two sides see the very same rounded values.

Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws float32 tensors in
the order Q, K, V, dO; each draw is then rounded once to the workload dtype.
The oracle reads those rounded values widened to float64 (an exact widening).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: layout [B, H, n, d] for Q, K and [B, H, n, dv] for V, O."""

    name: str
    B: int
    H: int
    n: int
    d: int
    dv: int
    dtype: str
    mask: str  # "none" | "causal" | "window"
    window: int = 0  # allowed keys per row including the diagonal (mask == "window")
    scale: Optional[float] = None  # default 1/sqrt(d)
    qk_mult: float = 1.0  # Q and K are drawn as qk_mult * N(0, 1)
    v_dist: str = "normal"  # "normal": N(0,1); "uniform": U(-1, 1)
    backward: bool = False
    seed: int = 1000

    @property
    def c(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the tests and the benchmark use (seed = 1000 + index).
WORKLOADS = {
    # 1: smoke, fp32, finishes in the oracle in well under a second
    "smoke": Workload("smoke", 1, 4, 256, 64, 64, "f32", "causal", seed=1001),
    # 2: the page workload; forward and backward are timed on it
    "page_d64": Workload("page_d64", 1, 32, 4096, 64, 64, "bf16", "causal", seed=1002),
    # 2b: same shape at d = v = 16, no mask (the Night School traffic comparison)
    "page_d16": Workload("page_d16", 1, 32, 4096, 16, 16, "bf16", "none", seed=1002),
    # 2c: the page shape at d = v = 128 (second forward throughput point)
    "page_d128": Workload("page_d128", 1, 32, 4096, 128, 128, "bf16", "causal", seed=1002),
    # 3: fp16 overflow stress: scores exceed 20 so e^s overflows fp16 without the shift
    "overflow": Workload("overflow", 2, 16, 4096, 128, 128, "f16", "none", qk_mult=2.0,
                         v_dist="uniform", seed=1003),
    # 4: long context, causal and a 4096-key sliding window
    "long_causal": Workload("long_causal", 1, 8, 65536, 128, 128, "bf16", "causal", seed=1004),
    "long_window": Workload("long_window", 1, 8, 65536, 128, 128, "bf16", "window", window=4096,
                            seed=1004),
    # 5: training step: forward saving LSE, then backward
    "train": Workload("train", 4, 16, 8192, 128, 128, "bf16", "causal", backward=True,
                      seed=1005),
}


def make_inputs(w: Workload, seed: Optional[int] = None, with_grad: bool = False,
                device="cpu") -> dict:
    """Draw Q, K, V (and dO) for workload ``w``; returns tensors in ``w.dtype``."""
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    dt = DTYPES[w.dtype]
    qshape = (w.B, w.H, w.n, w.d)
    vshape = (w.B, w.H, w.n, w.dv)
    q = torch.randn(qshape, generator=g, dtype=torch.float32)
    k = torch.randn(qshape, generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        q.mul_(w.qk_mult)
        k.mul_(w.qk_mult)
    if w.v_dist == "uniform":
        v = torch.rand(vshape, generator=g, dtype=torch.float32).mul_(2.0).sub_(1.0)
    else:
        v = torch.randn(vshape, generator=g, dtype=torch.float32)
    out = {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt)}
    if with_grad or w.backward:
        out["do"] = torch.randn(vshape, generator=g, dtype=torch.float32).to(dt)
    if device != "cpu":
        out = {key: t.to(device) for key, t in out.items()}
    return out


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of ``w`` (same dtype, mask and distributions) for fast checks."""
    return w.replace(**kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """nq new rows per query head against a cache of nk keys and values.

    Q: [B, H, nq, d]; K: [B, Hkv, nk, d]; V: [B, Hkv, nk, dv]; H a multiple of Hkv.
    The rows are the last nq of nk positions.
    """

    name: str
    B: int
    H: int
    Hkv: int
    nq: int
    nk: int
    d: int
    dv: int
    dtype: str
    mask: str = "none"
    window: int = 0
    scale: Optional[float] = None  # default 1/sqrt(d)
    seed: int = 2000

    @property
    def c(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# Decode shapes.  decode_7b is the Principia page's own KV-cache example (a
# 7B-class model: 32 heads of 128, fp16, 4096 cached tokens per session), one
# layer for a batch of 16 sessions; the others vary the head sharing, the
# context length and the number of new rows (a few drafted positions checked
# in one pass).
DECODE_WORKLOADS = {
    "decode_7b": DecodeWorkload("decode_7b", 16, 32, 32, 1, 4096, 128, 128, "f16", seed=2001),
    "decode_gqa": DecodeWorkload("decode_gqa", 16, 32, 8, 1, 16384, 128, 128, "bf16", seed=2002),
    "decode_long": DecodeWorkload("decode_long", 1, 32, 8, 1, 65536, 128, 128, "bf16", seed=2003),
    "decode_verify": DecodeWorkload("decode_verify", 16, 32, 32, 4, 4096, 128, 128, "f16",
                                    "causal", seed=2004),
}


def make_decode_inputs(w: DecodeWorkload, seed: Optional[int] = None, device="cpu") -> dict:
    """Draw Q, K, V for a decode workload (CPU generator, float32 N(0, 1) in the
    order Q, K, V, each rounded once to ``w.dtype``)."""
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    dt = DTYPES[w.dtype]
    q = torch.randn((w.B, w.H, w.nq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.nk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.nk, w.dv), generator=g, dtype=torch.float32)
    out = {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt)}
    if device != "cpu":
        out = {key: t.to(device) for key, t in out.items()}
    return out



def make_signs(d: int, seed: int) -> torch.Tensor:
    """The random sign vector of the FP8 path's incoherent processing: d values
    of +-1 (int8), each sign drawn with probability 1/2 by a CPU generator."""
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    bits = torch.randint(0, 2, (d,), generator=g, dtype=torch.int64)
    return (1 - 2 * bits).to(torch.int8)


# Signs seed for the FP8 workloads (one vector per run, shared by Q and K).
FP8_SIGNS_SEED = 3001
