"""The key and row ranges the workgroup timeline fits durations against (CPU)."""
import numpy as np

from exact_io_aware_tiled_amd.wg_timeline import BM, BNK, visible_keys, visible_rows


def test_visible_keys_match_the_masks():
    n, W = 1000, 300
    qt = np.arange((n + BM - 1) // BM)
    # brute force: the keys any row of the tile may see, per mask
    for mask in ("none", "causal", "window"):
        got = visible_keys(n, mask, W, qt)
        for t in qt:
            rows = range(t * BM, min(n, (t + 1) * BM))
            keys = set()
            for i in rows:
                lo = max(0, i - W + 1) if mask == "window" else 0
                hi = n - 1 if mask == "none" else i
                keys.update(range(lo, hi + 1))
            assert got[t] == max(keys) - min(keys) + 1, (mask, t)


def test_visible_rows_match_the_masks():
    n, W = 1000, 300
    kt = np.arange((n + BNK - 1) // BNK)
    # brute force: the query rows that see any key of the tile, per mask
    for mask in ("none", "causal", "window"):
        got = visible_rows(n, mask, W, kt)
        for t in kt:
            rows = set()
            for j in range(t * BNK, min(n, (t + 1) * BNK)):
                lo = 0 if mask == "none" else j
                hi = n - 1 if mask != "window" else min(n - 1, j + W - 1)
                rows.update(range(lo, hi + 1))
            assert got[t] == max(rows) - min(rows) + 1, (mask, t)
