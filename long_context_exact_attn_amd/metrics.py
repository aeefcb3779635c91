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

    Queries sit at global positions q_first .. q_first + q_len - 1.  causal is False / 0 (no
    mask), True (token level) or a causal block size c: a query at p sees keys below
    min((p // c + 1) * c, kv_len).
    """
    if q_len <= 0 or kv_len <= 0:
        return 0
    c = 0 if causal is None or causal is False else (1 if causal is True else int(causal))
    qpos = np.arange(q_first, q_first + q_len, dtype=np.int64)
    lim = np.minimum((qpos // c + 1) * c, kv_len) if c else np.full(q_len, kv_len, dtype=np.int64)
    if segment_ids is None:
        return int(lim.sum())
    total = 0
    for row in np.asarray(segment_ids):
        row = row.astype(np.int64)
        # keys of the query's segment below its limit: sort (id, position) pairs and count
        comb = np.sort((row - row.min()) * (kv_len + 1) + np.arange(kv_len, dtype=np.int64))
        base = (row[qpos] - row.min()) * (kv_len + 1)
        total += int((np.searchsorted(comb, base + lim) - np.searchsorted(comb, base)).sum())
    return total


def flops(pairs, head_dim, heads, batch_rows=1):
    """Dict of algorithmic FLOPs for `pairs` visible pairs per head (already summed over batch)."""
    n = pairs * heads * batch_rows
    return {"fwd": 4 * head_dim * n, "bwd": 10 * head_dim * n, "dkdv": 8 * head_dim * n,
            "dq": 6 * head_dim * n, "fwd_bwd": 14 * head_dim * n}


def executed_pairs_per_head(q_first, q_len, kv_len, causal, tile_q, tile_k):
    """(query, key) pairs inside the tile_q x tile_k tiles a kernel computes for one head and batch
    row: a tile is computed in full (masked and padding pairs included) when the causal mask leaves
    any of its pairs visible.  Dense masks only (no segment ids); token-level causal or none."""
    if q_len <= 0 or kv_len <= 0:
        return 0
    if causal is not True and causal not in (1, False, 0, None):
        return None
    n_kt = -(-kv_len // tile_k)
    total = 0
    for r0 in range(0, q_len, tile_q):
        if causal in (False, 0, None):
            kt = n_kt
        else:
            last = q_first + min(r0 + tile_q, q_len) - 1   # the tile's last existing query
            kt = min(n_kt, last // tile_k + 1)
        total += tile_q * tile_k * kt
    return total


# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # dense fp32, matrix unit and vector unit alike
PEAK_HBM_GBS = 8000.0
