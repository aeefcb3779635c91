"""Work accounting for blockwise ring attention: visible (query, key) pairs and
the algorithmic FLOPs / bytes derived from them.

Counted work is what the definition needs, on visible pairs only:
  forward      4*D per pair   (S = Q K^T and P V, two multiply-adds per element)
  backward    10*D per pair   (S, dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K)
  dK/dV kernel 8*D per pair   (its own products: S, dP, dV, dK)
  dQ kernel    6*D per pair   (its own products: S, dP, dQ)
Tile padding, skipped-but-read work and the two backward kernels' shared
recomputation of S and dP are not counted in the 14*D whole-step figure.
"""
import numpy as np


def visible_pairs_per_head(q_first, q_len, kv_len, causal, segment_ids=None):
    """Visible pairs of one head, summed over the batch rows of segment_ids (or one row).

    Queries sit at global positions q_first .. q_first + q_len - 1.
    """
    if q_len <= 0 or kv_len <= 0:
        return 0
    if segment_ids is None:
        if not causal:
            return q_len * kv_len
        lo, hi = q_first + 1, q_first + q_len          # sum of (p + 1) over the query positions
        return (lo + hi) * q_len // 2
    total = 0
    seg = np.asarray(segment_ids)
    for row in seg:
        row = row.astype(np.int64)
        qpos = np.arange(q_first, q_first + q_len)
        if causal:
            # 1 + the number of earlier keys with the same id: rank inside the id's run
            order = np.argsort(row, kind="stable")
            sorted_ids = row[order]
            starts = np.zeros(len(row), dtype=np.int64)
            bounds = np.flatnonzero(np.diff(sorted_ids)) + 1
            starts[bounds] = bounds
            starts = np.maximum.accumulate(starts)
            rank = np.empty(len(row), dtype=np.int64)
            rank[order] = np.arange(len(row)) - starts
            total += int((rank[qpos] + 1).sum())
        else:
            inv = np.unique(row, return_inverse=True)[1]
            total += int(np.bincount(inv)[inv][qpos].sum())
    return total


def flops(pairs, head_dim, heads, batch_rows=1):
    """Dict of algorithmic FLOPs for `pairs` visible pairs per head (already summed over batch)."""
    n = pairs * heads * batch_rows
    return {"fwd": 4 * head_dim * n, "bwd": 10 * head_dim * n, "dkdv": 8 * head_dim * n,
            "dq": 6 * head_dim * n, "fwd_bwd": 14 * head_dim * n}


# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # fp32 vector
PEAK_HBM_GBS = 8000.0
