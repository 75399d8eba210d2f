"""The byte model reproduces the Night School page's printed traffic counts."""
import json
import os

from conftest import GOLDEN
from exact_io_aware_tiled_amd import traffic


def test_page_counts_exact():
    with open(os.path.join(GOLDEN, "night_school_traffic.json")) as f:
        g = json.load(f)
    n = g["n"]
    for d, counts in g["bytes"].items():
        assert traffic.page_fused_bytes(n, int(d)) == counts["fused"]
        assert traffic.page_plain_bytes(n, int(d)) == counts["plain"]
    for d, mib in g["mebibytes"].items():
        assert round(traffic.page_fused_bytes(n, int(d)) / 2**20, 1) == mib["fused"]
        assert round(traffic.page_plain_bytes(n, int(d)) / 2**20, 1) == mib["plain"]
    # one head's fp32 score table
    assert 4 * n * n / 2**20 == g["scores_one_head_fp32_mebibytes"]


def test_compulsory_bytes():
    # 32 heads of the d = 16 bf16 page workload: Q, K, V, O (2 B) + LSE (4 B)
    assert 32 * traffic.compulsory_bytes(4096, 16, 16, 2) == 32 * (2 * 4 * 4096 * 16 + 4 * 4096)
    assert traffic.request_bytes(4096, 64, 64, 2, 128) >= traffic.compulsory_bytes(4096, 64, 64, 2)
