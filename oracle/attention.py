"""Plain float64 definition of (ring) attention -- test infrastructure only.

Tensor layout follows the sharding spec shown on "RingAttention核心功能全解析"
(section "计算与通信重叠"): ``[batch, sequence, heads, head_dim]``.  Every
function upcasts its inputs to float64 per (batch, head) slice; callers pass
the values the GPU sees (already rounded to the working dtype), so the only
differences left are the GPU's own rounding.

Definition (exact full attention; "手把手拆解RingAttention" section 1 says
the ring keeps the whole attention map, so the result must equal plain
attention over all keys):

    visible(i, j) = (not causal or j // c <= p_i // c) and (seg is None or seg[j] == seg[p_i])
    s_ij  = scale * <q_i, k_j> + bias[h, j mod bias_len]
    lse_i = log sum_{visible j} exp(s_ij)
    P_ij  = exp(s_ij - lse_i) if visible else 0
    out_i = sum_j P_ij v_j

``p_i`` is the global sequence position of local query ``i``: on ring rank
``r`` of a ring of ``n`` blocks of ``Lb`` tokens it is ``r*Lb + i``.  The
causal mask compares *global* positions.  Its granularity is the page's
``causal_block_size`` c (section "分块注意力计算" of the wmrh.cn page, where
c = 1 turns on causal attention): the page gives no other value a meaning,
and the reading taken is that positions fall into consecutive blocks of c
tokens and a key is visible when its block does not come after the query's
block.  c = 1 is token-level causal attention (j <= p_i).  ``causal`` below is
False / 0 (no mask), True (c = 1) or the integer c.  A row with no visible
key has out = 0 and lse = -inf.

Backward (recompute policy ``nothing_saveable``, section "快速上手"), given dO:

    Delta_i = <dO_i, out_i>
    dP_ij   = <dO_i, v_j>
    dS_ij   = P_ij (dP_ij - Delta_i)
    dQ_i    = scale * sum_j dS_ij k_j
    dK_j    = scale * sum_i dS_ij q_i
    dV_j    = sum_i P_ij dO_i
"""
import math

import numpy as np

# rows per chunk so that one [rows, Lk] float64 score block stays near 256 MiB
_BLOCK_BYTES = 256 << 20


def query_positions(q_len, kv_len, n_ring, ring_rank):
    """Global positions of the local queries.

    ``ring_rank < 0``: the queries are the whole sequence (q_len == kv_len).
    ``ring_rank = r``: the queries are ring block r, of length kv_len / n_ring.
    """
    if ring_rank is None or ring_rank < 0:
        if q_len != kv_len:
            raise ValueError("all-ranks mode needs q_len == kv_len")
        return np.arange(q_len, dtype=np.int64)
    if kv_len % n_ring:
        raise ValueError("kv_len must be n_ring * block length")
    block = kv_len // n_ring
    if q_len != block or not 0 <= ring_rank < n_ring:
        raise ValueError("per-rank mode needs q_len == block length and 0 <= rank < n_ring")
    return ring_rank * block + np.arange(q_len, dtype=np.int64)


def causal_block(causal):
    """The causal block size c of a ``causal`` argument: 0 for none, 1 for True."""
    if causal is None or causal is False:
        return 0
    if causal is True:
        return 1
    c = int(causal)
    if c < 0:
        raise ValueError("causal block size must be >= 0")
    return c


def _visible(q_pos, kv_len, causal, seg_row):
    """Boolean [nq, kv_len]: which keys each query may attend to."""
    j = np.arange(kv_len, dtype=np.int64)
    vis = np.ones((len(q_pos), kv_len), dtype=bool)
    c = causal_block(causal)
    if c:
        vis &= (j // c)[None, :] <= (q_pos // c)[:, None]
    if seg_row is not None:
        seg_row = np.asarray(seg_row)
        vis &= seg_row[None, :] == seg_row[q_pos][:, None]
    return vis


def _bias_row(bias, h, kv_len):
    if bias is None:
        return None
    bias = np.asarray(bias, dtype=np.float64)
    return bias[h, np.arange(kv_len) % bias.shape[1]]


def _scores(qb, kb, scale, bias_row, vis):
    s = scale * (qb @ kb.T)
    if bias_row is not None:
        s = s + bias_row[None, :]
    return np.where(vis, s, -np.inf)


def _softmax_rows(s):
    """Return (P, lse) for masked scores s (masked entries are -inf)."""
    m = s.max(axis=1, initial=-np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) == 0 for masked entries
    z = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    p = e / np.where(z > 0, z, 1.0)[:, None]
    return p, lse


def _chunks(nq, kv_len):
    rows = max(1, min(nq, _BLOCK_BYTES // max(1, 8 * kv_len)))
    for i0 in range(0, nq, rows):
        yield i0, min(nq, i0 + rows)


def _default_scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def forward(q, k, v, *, q_pos, causal, scale=None, bias=None, segment_ids=None):
    """Exact attention forward in float64.

    q: [B, nq, H, D]; k, v: [B, Lk, H, D]; q_pos: [nq] global positions;
    bias: [H, bias_len] or None; segment_ids: [B, Lk] or None.
    Returns (out [B, nq, H, D] float64, lse [B, H, nq] float64, natural log).
    """
    B, nq, H, D = q.shape
    Lk = k.shape[1]
    scale = _default_scale(scale, D)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    out = np.zeros((B, nq, H, D), dtype=np.float64)
    lse = np.full((B, H, nq), -np.inf, dtype=np.float64)
    for b in range(B):
        seg_row = None if segment_ids is None else np.asarray(segment_ids[b])
        for h in range(H):
            kb = np.asarray(k[b, :, h, :], dtype=np.float64)
            vb = np.asarray(v[b, :, h, :], dtype=np.float64)
            brow = _bias_row(bias, h, Lk)
            for i0, i1 in _chunks(nq, Lk):
                qb = np.asarray(q[b, i0:i1, h, :], dtype=np.float64)
                vis = _visible(q_pos[i0:i1], Lk, causal, seg_row)
                p, l_ = _softmax_rows(_scores(qb, kb, scale, brow, vis))
                out[b, i0:i1, h, :] = p @ vb
                lse[b, h, i0:i1] = l_
    return out, lse


def probabilities(q, k, *, q_pos, causal, scale=None, bias=None, segment_ids=None, b=0, h=0):
    """The attention matrix P [nq, Lk] of one (batch, head); for small cases."""
    D = q.shape[-1]
    Lk = k.shape[1]
    scale = _default_scale(scale, D)
    seg_row = None if segment_ids is None else np.asarray(segment_ids[b])
    vis = _visible(np.asarray(q_pos, dtype=np.int64), Lk, causal, seg_row)
    s = _scores(np.asarray(q[b, :, h, :], dtype=np.float64), np.asarray(k[b, :, h, :], dtype=np.float64),
                scale, _bias_row(bias, h, Lk), vis)
    return _softmax_rows(s)[0]


def backward(q, k, v, dout, *, q_pos, causal, scale=None, bias=None, segment_ids=None):
    """Gradients of sum(dout * out) w.r.t. q, k, v, in float64.

    P is recomputed from the inputs (the recompute policy), exactly as the
    forward defines it.  When q holds only some of the queries (sampled rows),
    dk and dv are those rows' contributions.
    Returns (dq [B,nq,H,D], dk [B,Lk,H,D], dv [B,Lk,H,D], delta [B,H,nq]).
    """
    B, nq, H, D = q.shape
    Lk = k.shape[1]
    scale = _default_scale(scale, D)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    dq = np.zeros((B, nq, H, D), dtype=np.float64)
    dk = np.zeros((B, Lk, H, D), dtype=np.float64)
    dv = np.zeros((B, Lk, H, D), dtype=np.float64)
    delta = np.zeros((B, H, nq), dtype=np.float64)
    for b in range(B):
        seg_row = None if segment_ids is None else np.asarray(segment_ids[b])
        for h in range(H):
            kb = np.asarray(k[b, :, h, :], dtype=np.float64)
            vb = np.asarray(v[b, :, h, :], dtype=np.float64)
            brow = _bias_row(bias, h, Lk)
            for i0, i1 in _chunks(nq, Lk):
                qb = np.asarray(q[b, i0:i1, h, :], dtype=np.float64)
                dob = np.asarray(dout[b, i0:i1, h, :], dtype=np.float64)
                vis = _visible(q_pos[i0:i1], Lk, causal, seg_row)
                p, _ = _softmax_rows(_scores(qb, kb, scale, brow, vis))
                ob = p @ vb
                dl = np.sum(dob * ob, axis=1)
                dp = dob @ vb.T
                ds = p * (dp - dl[:, None])
                dq[b, i0:i1, h, :] = scale * (ds @ kb)
                dk[b, :, h, :] += scale * (ds.T @ qb)
                dv[b, :, h, :] += p.T @ dob
                delta[b, h, i0:i1] = dl
    return dq, dk, dv, delta


def bias_grad(q, k, v, dout, *, q_pos, causal, scale=None, bias, segment_ids=None):
    """Gradient of sum(dout * out) w.r.t. the additive bias [H, bias_len], in float64.

    Key j adds bias[h, j mod bias_len] to every query's score, so the bias entry t collects
    dS_ij = dL/ds_ij over all batch rows, queries i and keys j with j mod bias_len = t (the bias
    is not scaled).  P is recomputed as in ``backward``.  Returns dbias [H, bias_len].
    """
    B, nq, H, D = q.shape
    Lk = k.shape[1]
    scale = _default_scale(scale, D)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    bias = np.asarray(bias, dtype=np.float64)
    nb = bias.shape[1]
    dbias = np.zeros((H, nb), dtype=np.float64)
    for b in range(B):
        seg_row = None if segment_ids is None else np.asarray(segment_ids[b])
        for h in range(H):
            kb = np.asarray(k[b, :, h, :], dtype=np.float64)
            vb = np.asarray(v[b, :, h, :], dtype=np.float64)
            brow = _bias_row(bias, h, Lk)
            for i0, i1 in _chunks(nq, Lk):
                qb = np.asarray(q[b, i0:i1, h, :], dtype=np.float64)
                dob = np.asarray(dout[b, i0:i1, h, :], dtype=np.float64)
                vis = _visible(q_pos[i0:i1], Lk, causal, seg_row)
                p, _ = _softmax_rows(_scores(qb, kb, scale, brow, vis))
                dl = np.sum(dob * (p @ vb), axis=1)
                ds = p * (dob @ vb.T - dl[:, None])
                np.add.at(dbias[h], np.arange(Lk) % nb, ds.sum(axis=0))
    return dbias


def visible_pairs(q_pos, kv_len, causal, segment_ids=None):
    """Number of visible (query, key) pairs per head, summed over the batch.

    segment_ids: [B, Lk] or None (then the count is for one batch row).
    Closed forms are used where they exist; with segments, the count is the
    sum over queries of the keys that share the query's segment (and precede
    it when causal).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    c = causal_block(causal)
    if segment_ids is None:
        if c:
            # keys up to the end of the query's causal block
            return int(np.sum(np.minimum((q_pos // c + 1) * c, kv_len)))
        return int(len(q_pos) * kv_len)
    total = 0
    for row in np.asarray(segment_ids):
        row = np.asarray(row, dtype=np.int64)
        if c > 1:
            # per query: keys of its segment that end no later than its causal block
            lim = np.minimum((q_pos // c + 1) * c, kv_len)
            total += int(sum(int(np.count_nonzero(row[:lim_i] == row[p])) for p, lim_i in zip(q_pos, lim)))
        elif c:
            # count j <= p with row[j] == row[p]: rank of p among equal ids
            order = np.argsort(row, kind="stable")
            rank = np.empty(kv_len, dtype=np.int64)
            ids_sorted = row[order]
            start = np.searchsorted(ids_sorted, ids_sorted, side="left")
            rank[order] = np.arange(kv_len) - start + 1
            total += int(rank[q_pos].sum())
        else:
            _, inv, counts = np.unique(row, return_inverse=True, return_counts=True)
            total += int(counts[inv][q_pos].sum())
    return total
