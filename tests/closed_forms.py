"""Hand-derived closed forms for the workloads' layout rules (test helpers).

count(name, q) is |A(q)|, the number of keys query q may attend to, derived
from each workload's rule on paper -- independent of the oracle's interval
code and of the C++ planner.
"""
import numpy as np


def count(name, q, N, bitmap_row_nnz=None):
    """Vectorised |A(q)| for an int64 array of queries q."""
    q = np.asarray(q, dtype=np.int64)
    if name.startswith("window16k"):          # causal window of 512 keys
        return np.minimum(q + 1, 512)
    if name.startswith("gqa256k"):            # causal window 4096 + 8 global keys
        return np.minimum(q + 1, 4096) + np.clip(q - 4095, 0, 8)
    if name.startswith("dense256k"):
        return q + 1
    if name.startswith("winglobal128k"):      # blocks: i - j < 64 or j < 4, causal
        i = q // 128
        row = np.minimum(i + 1, 64) + np.clip(i - 63, 0, 4)
        return 128 * (row - 1) + q % 128 + 1
    if name.startswith("tiny_f32"):           # 64-blocks: |i-j| <= 2 or i == 0 or j == 0
        nb = N // 64
        i = q // 64
        win = np.minimum(i + 2, nb - 1) - np.maximum(i - 2, 0) + 1
        blocks = np.where(i == 0, nb, win + (i > 2))
        return 64 * blocks
    if name.startswith("random32k"):          # bitmap, non-causal: whole blocks
        return 128 * bitmap_row_nnz[q // 128]
    raise KeyError(name)
