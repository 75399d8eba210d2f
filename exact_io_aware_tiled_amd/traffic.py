"""HBM byte models for one attention head (measurement support, no compute).

Night School "Fused attention" (sections "The lab: the cannery" and "One trip")
counts the global-memory requests of its own fp32 WebGPU kernels at n = 4096:
a fused kernel whose query tile holds 8 KiB (Br = 2048 / d rows of fp32) reads
Q once, re-reads K and V once per query tile, and writes O; the plain
three-pass form additionally moves the n x n score table four times (write S,
read S and write P, read P).  These models reproduce the printed counts and
give the compulsory bytes of the fused kernel built here for comparison with
measured traffic.
"""
from __future__ import annotations


def page_fused_bytes(n: int, d: int, elem: int = 4) -> int:
    """Request bytes of the page's fused kernel: Q + O once, K + V once per query tile."""
    br = 2048 // d
    tiles = n // br
    return elem * (2 * n * d + 2 * tiles * n * d)


def page_plain_bytes(n: int, d: int, elem: int = 4) -> int:
    """The fused count plus the score table crossing HBM four times."""
    return page_fused_bytes(n, d, elem) + elem * 4 * n * n


def compulsory_bytes(n: int, d: int, dv: int, elem: int) -> int:
    """Q, K, V read once, O written once, LSE (fp32) written once: the algorithmic minimum."""
    return elem * (2 * n * d + 2 * n * dv) + 4 * n


def request_bytes(n: int, d: int, dv: int, elem: int, block_m: int) -> int:
    """Requests of this library's forward with query tiles of block_m rows and no
    causal skip: Q and O once, K and V once per query tile, plus LSE."""
    tiles = -(-n // block_m)
    return elem * (n * d + n * dv + tiles * n * (d + dv)) + 4 * n
