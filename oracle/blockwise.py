"""The ring-attention procedure itself, step by step, in float64 -- test infrastructure only.

This is the method as the pages describe it, not the plain definition:

* Each device keeps its query block; key/value blocks travel round a ring
  of ``n`` devices until every query block has met every K/V block
  ("手把手拆解RingAttention", section 1, and section 2 for the neighbour
  exchange).  On one host this is a loop over ring steps: at step ``s`` the
  device holding query block ``r`` works on K/V block ``(r - s) mod n``.
* Inside a device the work is blockwise, in chunks of ``query_chunk_size``
  queries by ``key_chunk_size`` keys ("RingAttention核心功能全解析",
  section "分块注意力计算").
* The pages state that the full attention map is kept but do not write out
  how partial results of different K/V blocks are combined.  The reading
  taken is the online-softmax merge: per query row keep a running maximum
  m, a running sum of exponentials l and an unnormalised output acc; a new
  chunk of scores s rescales the old state by exp(m_old - m_new) and adds
  exp(s - m_new) (and its product with V).  At the end out = acc / l and
  lse = m + log l.  Exactness of this merge is a theorem (exp(a-m)exp(m-m')
  = exp(a-m')), which the tests check numerically against ``attention``.

The optional ``order`` argument replaces the ring order by any permutation of
the K/V blocks, so the tests can check that the result does not depend on it.
"""
import math

import numpy as np

from .attention import causal_block


def ring_forward(q, k, v, *, n_ring, ring_rank, q_chunk, k_chunk, causal, scale=None,
                 bias=None, segment_ids=None, order=None):
    """Blockwise ring attention forward in float64.

    q: [B, Lq, H, D]; k, v: [B, Lk, H, D] with Lk = n_ring * Lb.
    ring_rank = r: q is ring block r (Lq == Lb).  ring_rank < 0: q holds all
    n_ring blocks (Lq == Lk) and each query block r follows its own ring order.
    order: optional callable (r, n) -> sequence of K/V block indices.
    Returns (out [B, Lq, H, D], lse [B, H, Lq]).
    """
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    if Lk % n_ring:
        raise ValueError("ring not closed: kv_len is not n_ring * block length")
    Lb = Lk // n_ring
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    cb = causal_block(causal)   # causal block size (0: no causal mask), as in the plain definition
    if ring_rank is None or ring_rank < 0:
        if Lq != Lk:
            raise ValueError("all-ranks mode needs Lq == Lk")
        q_blocks = [(r, r * Lb) for r in range(n_ring)]          # (rank, first local row)
    else:
        if Lq != Lb:
            raise ValueError("per-rank mode needs Lq == block length")
        q_blocks = [(ring_rank, 0)]
    if order is None:
        order = lambda r, n: [(r - s) % n for s in range(n)]    # noqa: E731

    out = np.zeros((B, Lq, H, D), dtype=np.float64)
    lse = np.full((B, H, Lq), -np.inf, dtype=np.float64)
    for b in range(B):
        seg = None if segment_ids is None else np.asarray(segment_ids[b], dtype=np.int64)
        for h in range(H):
            kb_all = np.asarray(k[b, :, h, :], dtype=np.float64)
            vb_all = np.asarray(v[b, :, h, :], dtype=np.float64)
            for r, row0 in q_blocks:
                for c0 in range(0, Lb, q_chunk):
                    c1 = min(Lb, c0 + q_chunk)
                    qc = np.asarray(q[b, row0 + c0:row0 + c1, h, :], dtype=np.float64)
                    pos = r * Lb + np.arange(c0, c1)                  # global query positions
                    m = np.full(len(pos), -np.inf)
                    l_ = np.zeros(len(pos))
                    acc = np.zeros((len(pos), D))
                    for j in order(r, n_ring):                        # K/V block arriving at this step
                        for k0 in range(0, Lb, k_chunk):
                            kpos = j * Lb + np.arange(k0, min(Lb, k0 + k_chunk))
                            s = scale * (qc @ kb_all[kpos].T)
                            if bias is not None:
                                s = s + np.asarray(bias, dtype=np.float64)[h, kpos % bias.shape[1]][None, :]
                            vis = np.ones(s.shape, dtype=bool)
                            if cb:
                                vis &= (kpos // cb)[None, :] <= (pos // cb)[:, None]
                            if seg is not None:
                                vis &= seg[kpos][None, :] == seg[pos][:, None]
                            s = np.where(vis, s, -np.inf)
                            m_new = np.maximum(m, s.max(axis=1))
                            # subtrahend 0 while a row has seen no visible key
                            base = np.where(np.isfinite(m_new), m_new, 0.0)
                            alpha = np.exp(np.where(np.isfinite(m), m, -np.inf) - base)
                            p = np.exp(s - base[:, None])
                            l_ = alpha * l_ + p.sum(axis=1)
                            acc = alpha[:, None] * acc + p @ vb_all[kpos]
                            m = m_new
                    ok = l_ > 0
                    out[b, row0 + c0:row0 + c1, h, :] = np.where(ok[:, None], acc / np.where(ok, l_, 1.0)[:, None], 0.0)
                    with np.errstate(divide="ignore"):
                        lse[b, h, row0 + c0:row0 + c1] = np.where(ok, m + np.log(np.where(ok, l_, 1.0)), -np.inf)
    return out, lse
