"""Pins for the CPU oracle (no GPU).

The oracle is trusted only because these checks tie it to things other than
itself: hand-derived worked examples, numbers the pages print, closed forms,
an independent library routine (torch's scaled_dot_product_attention, float64,
on the CPU), finite differences for the gradients, mathematical invariants,
and the method's own blockwise ring procedure.  ``test_planted_mistakes``
checks that plausible mistakes planted in a copy of the oracle are caught.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261202)


def _rand_case(B=2, L=12, H=2, D=5, n_ring=3, ring_rank=-1, bias_len=0, seg=False, seed=0):
    rng = np.random.default_rng(seed)
    Lb = L // n_ring
    Lq = L if ring_rank < 0 else Lb
    q = rng.standard_normal((B, Lq, H, D))
    k = rng.standard_normal((B, L, H, D))
    v = rng.standard_normal((B, L, H, D))
    bias = rng.standard_normal((H, bias_len)) if bias_len else None
    segs = rng.integers(0, 3, size=(B, L)) if seg else None
    pos = A.query_positions(Lq, L, n_ring, ring_rank)
    return q, k, v, bias, segs, pos


# ---------------------------------------------------------------- worked examples
def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", [c for c in _load("worked_examples.json") if not c.startswith("_")])
def test_worked_examples(case):
    ex = _load("worked_examples.json")[case]
    q = np.array(ex["q"])[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    bias = np.array(ex["bias"])[None, :] if "bias" in ex else None
    seg = np.array(ex["segment_ids"])[None, :] if "segment_ids" in ex else None
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(q.shape[1]), causal=ex["causal"],
                              scale=ex["scale"], bias=bias, segment_ids=seg)
    np.testing.assert_allclose(out[0, :, 0, :], np.array(ex["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(ex["lse"]), rtol=0, atol=1e-12)
    if q.shape[1] != k.shape[1]:
        return
    # the method's blockwise procedure reaches the same numbers
    ob, lb = oracle.ring_forward(q, k, v, n_ring=1, ring_rank=-1, q_chunk=1, k_chunk=1,
                                 causal=ex["causal"], scale=ex["scale"], bias=bias, segment_ids=seg)
    np.testing.assert_allclose(ob[0, :, 0, :], np.array(ex["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lb[0, 0], np.array(ex["lse"]), rtol=0, atol=1e-12)


def test_pages_numbers():
    g = _load("pages_numbers.json")
    for key in ("ring_block_1m_over_8", "ring_block_100k_over_8"):
        e = g[key]
        r = e["n_ring"] - 1
        pos = A.query_positions(e["block_len"], e["kv_len"], e["n_ring"], r)
        assert len(pos) == e["block_len"] and pos[0] == r * e["block_len"] and pos[-1] == e["kv_len"] - 1
    e = g["score_matrix_100k_fp32"]
    # the non-causal, unmasked pair count is the N x N matrix the page sizes at 4 bytes a score
    pairs = A.visible_pairs(np.arange(e["n"]), e["n"], causal=False)
    assert pairs * e["bytes_per_score"] == e["bytes"]


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, pos, causal, scale, bias, seg, b, h):
    """Pure-Python loops with math.exp / math.fsum, one (batch, head)."""
    Lq, D = q.shape[1], q.shape[3]
    Lk = k.shape[1]
    outs, lses = [], []
    for i in range(Lq):
        logits = {}
        c = 1 if causal is True else int(causal)   # causal block size (0: no mask)
        for j in range(Lk):
            if c and j // c > pos[i] // c:   # the key's block comes after the query's
                continue
            if seg is not None and seg[b][j] != seg[b][pos[i]]:
                continue
            s = scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D))
            if bias is not None:
                s += float(bias[h][j % len(bias[h])])
            logits[j] = s
        if not logits:
            outs.append([0.0] * D)
            lses.append(-math.inf)
            continue
        m = max(logits.values())
        z = math.fsum(math.exp(s - m) for s in logits.values())
        outs.append([math.fsum(math.exp(s - m) / z * float(v[b, j, h, d]) for j, s in logits.items())
                     for d in range(D)])
        lses.append(m + math.log(z))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("ring_rank", [-1, 0, 2])
@pytest.mark.parametrize("causal", [False, True, 3, 8])
@pytest.mark.parametrize("bias_len,seg", [(0, False), (5, False), (0, True), (4, True)])
def test_brute_force(ring_rank, causal, bias_len, seg):
    q, k, v, bias, segs, pos = _rand_case(ring_rank=ring_rank, bias_len=bias_len, seg=seg,
                                           seed=hash((ring_rank, causal, bias_len, seg)) % 1000)
    scale = 0.37
    out, lse = oracle.forward(q, k, v, q_pos=pos, causal=causal, scale=scale, bias=bias, segment_ids=segs)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            o_ref, l_ref = _brute(q, k, v, pos, causal, scale, bias, segs, b, h)
            np.testing.assert_allclose(out[b, :, h, :], o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], l_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- library special case
def _sdpa(q, k, v, pos, causal, scale, bias, seg):
    """torch SDPA (float64, CPU) with the mask and bias as one additive matrix, plus autograd."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), requires_grad=True) for x in (q, k, v))
    add = torch.zeros((B, H, Lq, Lk), dtype=torch.float64)
    j = torch.arange(Lk)
    p = torch.as_tensor(pos)
    if bias is not None:
        add += torch.as_tensor(bias)[:, j % bias.shape[1]][None, :, None, :]
    if causal:
        add = add.masked_fill((j[None, :] > p[:, None])[None, None], float("-inf"))
    if seg is not None:
        st = torch.as_tensor(seg)
        add = add.masked_fill((st[:, None, :] != st[:, p][:, :, None])[:, None], float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    return out, (tq, tk, tv)


@pytest.mark.parametrize("ring_rank", [-1, 1])
@pytest.mark.parametrize("causal,bias_len,seg", [(False, 0, False), (True, 0, False), (True, 3, True),
                                                 (False, 7, True)])
def test_against_torch_sdpa(ring_rank, causal, bias_len, seg):
    q, k, v, bias, segs, pos = _rand_case(B=2, L=24, H=3, D=8, n_ring=4, ring_rank=ring_rank,
                                           bias_len=bias_len, seg=seg, seed=11)
    if segs is not None:        # keep every query's own key visible so that no SDPA row is empty
        segs = np.sort(segs, axis=1)
    scale = 0.29
    out, lse = oracle.forward(q, k, v, q_pos=pos, causal=causal, scale=scale, bias=bias, segment_ids=segs)
    t_out, leaves = _sdpa(q, k, v, pos, causal, scale, bias, segs)
    np.testing.assert_allclose(out, t_out.detach().numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
    dout = np.random.default_rng(3).standard_normal(out.shape)
    t_out.backward(torch.tensor(dout.transpose(0, 2, 1, 3).copy()))
    dq, dk, dv, _ = oracle.backward(q, k, v, dout, q_pos=pos, causal=causal, scale=scale, bias=bias,
                                    segment_ids=segs)
    for mine, leaf in zip((dq, dk, dv), leaves):
        np.testing.assert_allclose(mine, leaf.grad.numpy().transpose(0, 2, 1, 3), rtol=0, atol=1e-11)


# ---------------------------------------------------------------- closed forms
def test_closed_form_zero_keys():
    B, L, H, D, n = 1, 16, 2, 4, 4
    v = RNG.standard_normal((B, L, H, D))
    q = RNG.standard_normal((B, L, H, D))
    k = np.zeros((B, L, H, D))
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(L), causal=False)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=1, keepdims=True), out.shape), atol=1e-13)
    np.testing.assert_allclose(lse, np.log(L), atol=1e-13)
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True)
    cum = np.cumsum(v, axis=1) / np.arange(1, L + 1)[None, :, None, None]
    np.testing.assert_allclose(out, cum, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, L + 1)), lse.shape), atol=1e-13)
    # one ring rank: global positions r*Lb + i
    r, Lb = 2, L // n
    pos = A.query_positions(Lb, L, n, r)
    out, lse = oracle.forward(q[:, :Lb], k, v, q_pos=pos, causal=True)
    np.testing.assert_allclose(out, cum[:, r * Lb:(r + 1) * Lb], atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(pos + 1), atol=1e-13)


def test_closed_form_own_segment_and_first_row():
    B, L, H, D = 2, 10, 2, 3
    q, k, v = (RNG.standard_normal((B, L, H, D)) for _ in range(3))
    bias = RNG.standard_normal((H, 4))
    scale = 0.7
    seg = np.tile(np.arange(L), (B, 1))          # every token its own document
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(L), causal=False, scale=scale, bias=bias, segment_ids=seg)
    np.testing.assert_allclose(out, v, atol=1e-14)
    s_ii = scale * np.einsum("blhd,blhd->bhl", q, k) + bias[:, np.arange(L) % 4][None]
    np.testing.assert_allclose(lse, s_ii, atol=1e-13)
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True, scale=scale, bias=bias)
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], s_ii[:, :, 0], atol=1e-13)


def test_closed_form_constant_values_and_bias_shift():
    B, L, H, D = 1, 9, 2, 4
    q, k = RNG.standard_normal((B, L, H, D)), RNG.standard_normal((B, L, H, D))
    row = RNG.standard_normal(D)
    v = np.broadcast_to(row, (B, L, H, D)).copy()
    out, _ = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), atol=1e-13)
    v = RNG.standard_normal((B, L, H, D))
    bias = RNG.standard_normal((H, 3))
    o1, l1 = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True, bias=bias)
    o2, l2 = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True, bias=bias + 2.5)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + 2.5, atol=1e-13)


def test_two_keys_is_logistic():
    # softmax over two logits is the logistic function of their difference
    q, k, v = (RNG.standard_normal((1, 2, 1, 3)) for _ in range(3))
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(2), causal=False, scale=1.0)
    for i in range(2):
        s0, s1 = q[0, i, 0] @ k[0, 0, 0], q[0, i, 0] @ k[0, 1, 0]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(out[0, i, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.logaddexp(s0, s1), atol=1e-14)


def test_empty_rows_and_empty_inputs():
    B, L, H, D = 1, 6, 1, 2
    q, k, v = (RNG.standard_normal((B, L, H, D)) for _ in range(3))
    # no keys at all: every row is empty (out 0, lse -inf)
    out, lse = oracle.forward(q, k[:, :0], v[:, :0], q_pos=np.zeros(L, dtype=np.int64), causal=False)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    out, lse = oracle.forward(q[:, :0], k, v, q_pos=np.arange(0), causal=True)
    assert out.shape == (B, 0, H, D) and lse.shape == (B, H, 0)
    dq, dk, dv, _ = oracle.backward(q, k[:, :0], v[:, :0], q, q_pos=np.zeros(L, dtype=np.int64), causal=False)
    assert np.all(dq == 0) and dk.shape == (B, 0, H, D)
    # a row whose own segment holds no visible key: query at position 1 with ids (0, 1) and a
    # causal mask sees key 1 only; position 0's id 7 appears nowhere else before it
    seg = np.array([[7, 3, 3, 3, 3, 3]])
    out, lse = oracle.forward(q, k, v, q_pos=np.arange(L), causal=True, segment_ids=seg)
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=1e-14)
    p = A.probabilities(q[:, :2], k, q_pos=np.array([0, 1]), causal=True, segment_ids=np.array([[7, 3, 3, 3, 3, 3]]))
    assert p[0, 0] == 1.0 and p[1, 0] == 0.0 and p[1, 1] == 1.0


def test_scale_default_and_invariance():
    q, k, v, _, _, pos = _rand_case(D=16, seed=5)
    o1, l1 = oracle.forward(q, k, v, q_pos=pos, causal=True)             # default 1/sqrt(16)
    o2, l2 = oracle.forward(q * 4.0, k, v, q_pos=pos, causal=True, scale=1.0 / 16)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_key_permutation_equivariance():
    # without causal masking, the order of the keys does not matter
    q, k, v, _, segs, pos = _rand_case(L=12, seg=True, seed=8)
    bias = RNG.standard_normal((2, 12))
    perm = RNG.permutation(12)
    o1, l1 = oracle.forward(q, k, v, q_pos=pos, causal=False, bias=bias)
    o2, l2 = oracle.forward(q, k[:, perm], v[:, perm], q_pos=pos, causal=False, bias=bias[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


# ---------------------------------------------------------------- probabilities
def test_rows_sum_to_one_and_masks_zero():
    q, k, v, bias, segs, pos = _rand_case(L=15, n_ring=3, bias_len=4, seg=True, seed=9)
    for causal in (False, True):
        p = A.probabilities(q, k, q_pos=pos, causal=causal, bias=bias, segment_ids=segs, b=1, h=1)
        j = np.arange(15)
        vis = segs[1][None, :] == segs[1][pos][:, None]
        if causal:
            vis &= j[None, :] <= pos[:, None]
            assert np.all(p[j[None, :] > pos[:, None]] == 0.0)
        assert np.all(p[~vis] == 0.0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)


# ---------------------------------------------------------------- gradients
def _loss(q, k, v, dout, pos, causal, scale, bias, segs):
    out, _ = oracle.forward(q, k, v, q_pos=pos, causal=causal, scale=scale, bias=bias, segment_ids=segs)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("ring_rank,causal,bias_len,seg", [(-1, True, 0, False), (-1, False, 3, True),
                                                            (1, True, 2, True)])
def test_finite_differences(ring_rank, causal, bias_len, seg):
    q, k, v, bias, segs, pos = _rand_case(B=1, L=8, H=1, D=3, n_ring=2, ring_rank=ring_rank,
                                           bias_len=bias_len, seg=seg, seed=21)
    dout = np.random.default_rng(22).standard_normal(q.shape)
    scale = 0.8
    dq, dk, dv, _ = oracle.backward(q, k, v, dout, q_pos=pos, causal=causal, scale=scale, bias=bias,
                                    segment_ids=segs)
    eps = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        args = [q, k, v]
        num = np.zeros_like(grad)
        it = np.nditer(args[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            num[idx] = (_loss(*xp, dout, pos, causal, scale, bias, segs)
                        - _loss(*xm, dout, pos, causal, scale, bias, segs)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7)


def test_gradient_invariants():
    q, k, v, bias, segs, pos = _rand_case(B=2, L=16, H=2, D=6, n_ring=4, bias_len=5, seg=True, seed=31)
    dout = RNG.standard_normal(q.shape)
    scale = 0.45
    dq, dk, dv, delta = oracle.backward(q, k, v, dout, q_pos=pos, causal=True, scale=scale, bias=bias,
                                        segment_ids=segs)
    # each row of dS sums to zero, so the key gradients sum to zero per (batch, head)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # each row of P sums to one, so the value gradients sum to the output gradients
    np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=1), atol=1e-12)
    # <dQ, Q> and <dK, K> both equal scale * sum_ij dS_ij s_ij: a transposed operand breaks this
    np.testing.assert_allclose(np.einsum("blhd,blhd->bh", dq, q), np.einsum("blhd,blhd->bh", dk, k), atol=1e-12)
    out, _ = oracle.forward(q, k, v, q_pos=pos, causal=True, scale=scale, bias=bias, segment_ids=segs)
    np.testing.assert_allclose(delta, np.einsum("blhd,blhd->bhl", dout, out), atol=1e-13)


# ---------------------------------------------------------------- the method's procedure
@pytest.mark.parametrize("q_chunk,k_chunk", [(1, 1), (3, 5), (4, 4), (6, 6), (2, 6)])
@pytest.mark.parametrize("ring_rank", [-1, 0, 3])
def test_blockwise_ring_equals_definition(q_chunk, k_chunk, ring_rank):
    q, k, v, bias, segs, pos = _rand_case(B=1, L=24, H=2, D=4, n_ring=4, ring_rank=ring_rank,
                                           bias_len=5, seg=True, seed=41)
    for causal in (False, True):
        ref_o, ref_l = oracle.forward(q, k, v, q_pos=pos, causal=causal, bias=bias, segment_ids=segs)
        o, l_ = oracle.ring_forward(q, k, v, n_ring=4, ring_rank=ring_rank, q_chunk=q_chunk, k_chunk=k_chunk,
                                    causal=causal, bias=bias, segment_ids=segs)
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(l_, ref_l, atol=1e-12)


def test_blockwise_ring_order_invariance():
    q, k, v, bias, segs, pos = _rand_case(B=1, L=30, H=1, D=4, n_ring=5, bias_len=3, seed=43)
    ref_o, ref_l = oracle.forward(q, k, v, q_pos=pos, causal=True, bias=bias)
    rng = np.random.default_rng(44)
    for _ in range(4):
        perms = {r: list(rng.permutation(5)) for r in range(5)}
        o, l_ = oracle.ring_forward(q, k, v, n_ring=5, ring_rank=-1, q_chunk=4, k_chunk=2, causal=True,
                                    bias=bias, order=lambda r, n: perms[r])
        np.testing.assert_allclose(o, ref_o, atol=1e-12)
        np.testing.assert_allclose(l_, ref_l, atol=1e-12)


def test_visible_pairs_counts():
    L = 40
    assert A.visible_pairs(np.arange(L), L, causal=True) == L * (L + 1) // 2
    assert A.visible_pairs(np.arange(10, 20), L, causal=True) == sum(range(11, 21))
    seg = np.array([[0] * 7 + [1] * 20 + [2] * 13])
    assert A.visible_pairs(np.arange(L), L, causal=True, segment_ids=seg) == 28 + 210 + 91
    assert A.visible_pairs(np.arange(L), L, causal=False, segment_ids=seg) == 49 + 400 + 169
    # brute force on a random non-monotone pattern
    seg = np.random.default_rng(5).integers(0, 4, size=(2, L))
    for causal in (False, True):
        brute = sum(int(((seg[b] == seg[b][i]) & ((np.arange(L) <= i) | (not causal))).sum())
                    for b in range(2) for i in range(L))
        assert A.visible_pairs(np.arange(L), L, causal=causal, segment_ids=seg) == brute


def test_visible_pairs_counts_causal_blocks():
    L = 40
    # blocks of 8: a query sees every key up to the end of its block
    assert A.visible_pairs(np.arange(L), L, causal=8) == sum(8 * (i // 8 + 1) for i in range(L))
    assert A.visible_pairs(np.arange(L), L, causal=1) == L * (L + 1) // 2
    assert A.visible_pairs(np.arange(L), L, causal=L) == L * L
    # blocks that do not divide the length: the last one is cut at L
    assert A.visible_pairs(np.arange(L), L, causal=16) == 16 * 16 + 16 * 32 + 8 * 40
    seg = np.random.default_rng(6).integers(0, 3, size=(2, L))
    for c in (2, 5, 16):
        brute = sum(int(((seg[b] == seg[b][i]) & (np.arange(L) // c <= i // c)).sum()) for b in range(2)
                    for i in range(L))
        assert A.visible_pairs(np.arange(L), L, causal=c, segment_ids=seg) == brute


def test_causal_block_one_is_token_causal():
    q, k, v, bias, segs, pos = _rand_case(ring_rank=1, bias_len=5, seg=True, seed=21)
    a = oracle.forward(q, k, v, q_pos=pos, causal=True, bias=bias, segment_ids=segs)
    b = oracle.forward(q, k, v, q_pos=pos, causal=1, bias=bias, segment_ids=segs)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_ring_forward_causal_blocks():
    # the method's own procedure with a causal block size gives the plain definition's result
    q, k, v, bias, segs, pos = _rand_case(ring_rank=-1, bias_len=7, seg=True, seed=22)
    n = 4
    for c in (2, 4):
        o, l_ = oracle.ring_forward(q, k, v, n_ring=n, ring_rank=-1, q_chunk=2, k_chunk=4, causal=c, bias=bias,
                                    segment_ids=segs)
        ro, rl = oracle.forward(q, k, v, q_pos=pos, causal=c, bias=bias, segment_ids=segs)
        np.testing.assert_allclose(o, ro, atol=1e-12)
        np.testing.assert_allclose(l_, rl, atol=1e-12)


# ---------------------------------------------------------------- bias gradient
@pytest.mark.parametrize("causal,seg,bias_len", [(False, False, 7), (True, True, 5), (3, False, 24), (True, False, 50)])
def test_bias_grad_against_torch_autograd(causal, seg, bias_len):
    # library special case: SDPA with the bias gathered by key position as a leaf tensor
    q, k, v, bias, segs, pos = _rand_case(B=2, L=24, H=3, D=8, n_ring=4, ring_rank=-1, bias_len=bias_len, seg=seg,
                                           seed=31)
    if segs is not None:
        segs = np.sort(segs, axis=1)
    scale = 0.41
    B, L, H, D = q.shape
    tb = torch.tensor(bias, requires_grad=True)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy()) for x in (q, k, v))
    j, p = torch.arange(L), torch.as_tensor(pos)
    add = tb[:, j % bias_len][None, :, None, :].expand(B, H, L, L)
    c = oracle.causal_block(causal)
    mask = torch.zeros((B, H, L, L), dtype=torch.bool)
    if c:
        mask |= ((j // c)[None, :] > (p // c)[:, None])[None, None]
    if segs is not None:
        st = torch.as_tensor(segs)
        mask |= (st[:, None, :] != st[:, p][:, :, None])[:, None]
    add = add.masked_fill(mask, float("-inf"))
    t_out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    dout = np.random.default_rng(32).standard_normal(q.shape)
    t_out.backward(torch.tensor(dout.transpose(0, 2, 1, 3).copy()))
    mine = oracle.bias_grad(q, k, v, dout, q_pos=pos, causal=causal, scale=scale, bias=bias, segment_ids=segs)
    np.testing.assert_allclose(mine, tb.grad.numpy(), rtol=0, atol=1e-11)


def test_bias_grad_sums_to_zero_and_matches_finite_differences():
    q, k, v, bias, segs, pos = _rand_case(B=1, L=12, H=2, D=4, n_ring=3, ring_rank=1, bias_len=5, seg=True, seed=33)
    dout = np.random.default_rng(34).standard_normal(q.shape)
    g = oracle.bias_grad(q, k, v, dout, q_pos=pos, causal=True, bias=bias, segment_ids=segs)
    # every row of P sums to 1, so the scores' gradient sums to 0 over each row's keys
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-13)
    eps = 1e-6
    for h, t in ((0, 0), (1, 3), (1, 4)):
        bp, bm = bias.copy(), bias.copy()
        bp[h, t] += eps
        bm[h, t] -= eps
        fp = np.sum(dout * oracle.forward(q, k, v, q_pos=pos, causal=True, bias=bp, segment_ids=segs)[0])
        fm = np.sum(dout * oracle.forward(q, k, v, q_pos=pos, causal=True, bias=bm, segment_ids=segs)[0])
        assert abs((fp - fm) / (2 * eps) - g[h, t]) < 1e-7
