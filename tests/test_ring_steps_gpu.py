"""GPU parity of the per-ring-step entry points: a chain of ra_blockwise_attn_fwd_step calls,
one per K/V block in ring order, then ra_blockwise_attn_fwd_finalize, must give the oracle's
attention of the device's query block over the whole sequence; ra_attn_merge of two partial
results over disjoint key blocks must give the same ("手把手拆解RingAttention", sections 1-2:
a device keeps its query block while K/V blocks pass it, one per step)."""
import numpy as np
import pytest
import torch

import long_context_exact_attn_amd as ra
from long_context_exact_attn_amd import workloads as W
import _parity as P

pytestmark = pytest.mark.gpu


def _block(x, j, lb):
    return x[:, j * lb:(j + 1) * lb].contiguous()


def _chain(w, t, blocks, state=None, init=None):
    lb, r = w.block_len, w.ring_rank
    for s, j in enumerate(blocks):
        state = ra.blockwise_attn_fwd_step(t["q"], _block(t["k"], j, lb), _block(t["v"], j, lb), t["bias"],
                                           t["segment_ids"], q_pos0=r * lb, kv_pos0=j * lb, causal=w.causal,
                                           state=state, init=init if s == 0 else False)
    return state


def _ring_order(w):
    n, r = w.n_ring, w.ring_rank
    return [(r - s) % n for s in range(n)]


def _oracle(w, t):
    d = P.oracle_inputs(t)
    return P.oracle_forward(w, d, w.q_positions())


CASES = [
    ("causal-ring4-r3", dict(kv_len=2048, n_ring=4, ring_rank=3)),
    ("causal-ring4-r0", dict(kv_len=2048, n_ring=4, ring_rank=0)),
    ("noncausal-ring3-r1", dict(kv_len=1536, n_ring=3, ring_rank=1, causal=False)),
    ("ragged-250", dict(kv_len=1000, n_ring=4, ring_rank=2)),
    ("bias-seg", dict(kv_len=2048, n_ring=4, ring_rank=2, bias_len=300, segments="docs", doc_len=(20, 400))),
    ("seg-noncausal", dict(kv_len=1536, n_ring=3, ring_rank=2, causal=False, segments="docs", doc_len=(5, 120))),
    ("d128-batch2", dict(head_dim=128, batch=2, heads=3, kv_len=1024, n_ring=2, ring_rank=1, bias_len=77)),
    ("heads5-ring8", dict(heads=5, kv_len=2048, n_ring=8, ring_rank=5)),
    ("causal-block-64-r2", dict(kv_len=2048, n_ring=4, ring_rank=2, causal=64, segments="docs", doc_len=(40, 300))),
    ("causal-block-100-r1", dict(kv_len=1200, n_ring=3, ring_rank=1, causal=100, bias_len=30)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_step_chain_matches_oracle_and_fused(gpu, name, kw):
    w = W.small(name, **kw)
    t = P.make(w, gpu)
    out, lse = ra.blockwise_attn_fwd_finalize(_chain(w, t, _ring_order(w)))
    fo, fl = P.gpu_forward(w, t)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(w, t)
    P.assert_close(f"{name} steps vs oracle", P.np64(out), ref_o, "bf16", strict=False)
    P.assert_lse(lse.cpu().numpy().astype(np.float64), ref_l, "bf16")
    # the same tiles in the same order as the fused kernel: only the summation order of l differs
    P.assert_close(f"{name} steps vs fused", P.np64(out), P.np64(fo), "bf16", strict=False)
    assert float((lse - fl).abs().max()) < 1e-5


def test_future_blocks_leave_the_state_unchanged(gpu):
    # causal: a K/V block wholly after the query block is masked out; folding it in is a no-op
    w = W.small("future", kv_len=2048, n_ring=4, ring_rank=1, bias_len=64, segments="docs", doc_len=(30, 300))
    t = P.make(w, gpu)
    state = _chain(w, t, [1, 0])
    snap = tuple(x.clone() for x in state)
    _chain(w, t, [2, 3], state=state, init=False)
    torch.cuda.synchronize()
    for a, b in zip(state, snap):
        assert torch.equal(a, b)


def test_init_ignores_what_the_state_holds(gpu):
    w = W.small("init", kv_len=1024, n_ring=2, ring_rank=1)
    t = P.make(w, gpu)
    B, Lq, H, D = t["q"].shape
    junk = (torch.full((B, Lq, H, D), float("nan"), device=gpu), torch.full((B, H, Lq), 3e38, device=gpu),
            torch.full((B, H, Lq), -7.0, device=gpu))
    a = ra.blockwise_attn_fwd_finalize(_chain(w, t, _ring_order(w), state=junk, init=True))
    b = ra.blockwise_attn_fwd_finalize(_chain(w, t, _ring_order(w)))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_step_order_changes_only_rounding(gpu):
    w = W.small("order", kv_len=2048, n_ring=8, ring_rank=4, causal=False, heads=3)
    t = P.make(w, gpu)
    a = ra.blockwise_attn_fwd_finalize(_chain(w, t, _ring_order(w)))
    b = ra.blockwise_attn_fwd_finalize(_chain(w, t, [3, 7, 0, 5, 1, 6, 2, 4]))
    torch.cuda.synchronize()
    P.assert_close("order", P.np64(b[0]), P.np64(a[0]), "bf16")
    assert float((a[1] - b[1]).abs().max()) < 1e-4


@pytest.mark.parametrize("name,kw,split", [
    ("causal-r3", dict(kv_len=2048, n_ring=4, ring_rank=3), 2),
    ("seg-r2", dict(kv_len=2048, n_ring=4, ring_rank=2, segments="docs", doc_len=(10, 200), bias_len=50), 1),
    ("noncausal-d128", dict(head_dim=128, kv_len=1536, n_ring=3, ring_rank=0, causal=False, heads=3), 1),
])
def test_merge_of_partial_results(gpu, name, kw, split):
    # two devices each fold in a disjoint set of K/V blocks; merging their normalised partial
    # results (out, lse) must give attention over the union
    w = W.small(name, **kw)
    t = P.make(w, gpu)
    order = _ring_order(w)
    oa, la = ra.blockwise_attn_fwd_finalize(_chain(w, t, order[:split]))
    ob, lb = ra.blockwise_attn_fwd_finalize(_chain(w, t, order[split:]))
    ra.attn_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle(w, t)
    P.assert_close(f"{name} merged", P.np64(oa), ref_o, "bf16", strict=False)
    P.assert_lse(la.cpu().numpy().astype(np.float64), ref_l, "bf16")


def test_merge_with_empty_sides(gpu):
    # rows whose partial result saw no visible key carry lse = -inf and out = 0: merging such a
    # side changes nothing, and two empty sides stay empty
    w = W.small("empty", kv_len=1024, n_ring=2, ring_rank=0)
    t = P.make(w, gpu)
    o, l_ = ra.blockwise_attn_fwd_finalize(_chain(w, t, [0]))
    eo, el = ra.blockwise_attn_fwd_finalize(_chain(w, t, [1]))   # causal: block 1 is all future
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(el)) and torch.all(eo == 0)
    mo, ml = o.clone(), l_.clone()
    ra.attn_merge(mo, ml, eo, el)
    assert torch.equal(mo, o) and torch.equal(ml, l_)
    eo2, el2 = eo.clone(), el.clone()
    ra.attn_merge(eo2, el2, eo, el)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(el2)) and torch.all(eo2 == 0)


def test_step_errors(gpu):
    w = W.small("err", kv_len=1024, n_ring=2, ring_rank=1)
    t = P.make(w, gpu)
    k = _block(t["k"], 0, w.block_len)
    with pytest.raises(ra.RAError, match="equal query and key blocks"):
        ra.blockwise_attn_fwd_step(t["q"], k[:, :100].contiguous(), k[:, :100].contiguous(), q_pos0=512,
                                   kv_pos0=0, causal=True)
    seg = torch.zeros(1, 600, dtype=torch.int32, device=gpu)
    with pytest.raises(ra.RAError, match="do not cover"):
        ra.blockwise_attn_fwd_step(t["q"], k, k, None, seg, q_pos0=512, kv_pos0=0, causal=True)
    qf = t["q"].float()
    with pytest.raises(ra.RAError, match="RA_BF16"):
        ra.blockwise_attn_fwd_step(qf, qf, qf, q_pos0=0, kv_pos0=0, causal=True)


# ------------------------------------------------------------------ backward ring steps
def _ring_backward(w, t, out, lse, skip_future=True, with_dbias=False):
    """All ranks of a ring on one GPU, one ra_blockwise_attn_bwd_step per (rank, step): dQ sums
    stay with each rank's queries, dK / dV sums (and, with_dbias, the per-key sums of dS) travel with
    their block.  with_dbias also returns dbias, the blocks' shares added in block order."""
    n, lb = w.n_ring, w.block_len
    delta = ra.blockwise_attn_bwd_preprocess(out, t["dout"])
    dq_acc = [None] * n
    dkv_acc = [None] * n
    kb_sums = [None] * n
    if with_dbias:
        for j in range(n):
            kb_sums[j] = torch.full((w.batch, w.heads, lb), float("nan"), device=t["q"].device)
    for r in range(n):
        rows = slice(r * lb, (r + 1) * lb)
        q_r, g_r = t["q"][:, rows].contiguous(), t["dout"][:, rows].contiguous()
        lse_r, dl_r = lse[:, :, rows].contiguous(), delta[:, :, rows].contiguous()
        for s in range(n):
            j = (r - s) % n
            if skip_future and w.causal and j > r:
                continue
            kb, vb = _block(t["k"], j, lb), _block(t["v"], j, lb)
            dk_a, dv_a = dkv_acc[j] if dkv_acc[j] is not None else (None, None)
            first_visit = dkv_acc[j] is None
            dq_acc[r], dk_a, dv_a = ra.blockwise_attn_bwd_step(
                q_r, kb, vb, lse_r, dl_r, g_r, t["bias"], t["segment_ids"], q_pos0=r * lb, kv_pos0=j * lb,
                causal=w.causal, dq_acc=dq_acc[r], dk_acc=dk_a, dv_acc=dv_a, dbias_acc=kb_sums[j],
                init_dkv=first_visit)
            dkv_acc[j] = (dk_a, dv_a)
    grads = [ra.blockwise_attn_bwd_finalize(dq_acc[i], *dkv_acc[i]) for i in range(n)]
    dq = torch.cat([g[0] for g in grads], dim=1)
    dk = torch.cat([g[1] for g in grads], dim=1)
    dv = torch.cat([g[2] for g in grads], dim=1)
    if not with_dbias:
        return dq, dk, dv
    dbias = torch.full_like(t["bias"], float("nan"))
    for j in range(n):
        ra.blockwise_attn_bwd_dbias_reduce(kb_sums[j], j * lb, dbias, accumulate=j > 0)
    return dq, dk, dv, dbias


BWD_CASES = [
    ("causal-ring4", dict(kv_len=2048, n_ring=4)),
    ("noncausal-bias-seg", dict(kv_len=1536, n_ring=3, causal=False, bias_len=100, segments="docs", doc_len=(20, 400))),
    ("ragged-250", dict(kv_len=1000, n_ring=4, segments="scattered")),
    ("d128-batch2", dict(head_dim=128, batch=2, heads=3, kv_len=1024, n_ring=2, bias_len=64)),
    ("causal-block-32", dict(kv_len=1024, n_ring=4, causal=32, segments="docs", doc_len=(20, 200))),
    ("causal-block-100", dict(kv_len=1200, n_ring=3, causal=100)),
]


@pytest.mark.parametrize("name,kw", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_step_ring_matches_oracle_and_fused(gpu, name, kw):
    w = W.small(name, backward=True, **kw)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = _ring_backward(w, t, out, lse)
    fq, fk, fv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    d = P.oracle_inputs(t)
    import oracle
    rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                                       bias=d["bias"], segment_ids=d["segment_ids"])
    for gname, g, f, r in (("dq", dq, fq, rdq), ("dk", dk, fk, rdk), ("dv", dv, fv, rdv)):
        P.assert_close(f"{name} {gname} steps vs oracle", P.np64(g), r, "bf16", strict=False)
        P.assert_close(f"{name} {gname} steps vs fused", P.np64(g), P.np64(f), "bf16", strict=False)


DBIAS_STEP_CASES = [
    ("bias-causal", dict(kv_len=2048, n_ring=4, bias_len=300)),
    ("bias-seg-noncausal", dict(kv_len=1536, n_ring=3, causal=False, bias_len=64, segments="docs", doc_len=(20, 400))),
    ("bias-longer-than-block", dict(kv_len=1024, n_ring=4, bias_len=700, segments="scattered")),
    ("bias-d128-batch2-blocks", dict(head_dim=128, batch=2, heads=3, kv_len=1200, n_ring=3, bias_len=100, causal=40)),
]


@pytest.mark.parametrize("name,kw", DBIAS_STEP_CASES, ids=[c[0] for c in DBIAS_STEP_CASES])
def test_bwd_step_ring_bias_gradient(gpu, name, kw):
    # the per-key sums of dS travel with their K/V block; each block's share is reduced into dbias with the
    # block's global key positions (bias entry (kv_pos0 + j) mod bias_len)
    w = W.small(name, backward=True, **kw)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv, db = _ring_backward(w, t, out, lse, with_dbias=True)
    kwr = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    fdb = ra.blockwise_attn_bwd_dbias(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"],
                                      **kwr)[3]
    torch.cuda.synchronize()
    d = P.oracle_inputs(t)
    import oracle
    ref = oracle.bias_grad(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                           bias=d["bias"], segment_ids=d["segment_ids"])
    got = db.double().cpu().numpy()
    P.assert_close_sums(f"{name} dbias steps vs oracle", got, ref)
    P.assert_close_sums(f"{name} dbias steps vs fused", got, fdb.double().cpu().numpy())


def test_bwd_step_future_block_is_a_no_op(gpu):
    w = W.small("bwd-future", backward=True, kv_len=2048, n_ring=4, bias_len=64, segments="docs", doc_len=(30, 300))
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    a = _ring_backward(w, t, out, lse, skip_future=True)
    b = _ring_backward(w, t, out, lse, skip_future=False)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_step_errors(gpu):
    w = W.small("bwd-err", kv_len=1024, n_ring=2, ring_rank=1, backward=True)
    t = P.make(w, gpu)
    k = _block(t["k"], 0, w.block_len)
    lse = torch.zeros(1, 2, 512, device=gpu)
    with pytest.raises(ra.RAError, match="equal query and key blocks"):
        ra.blockwise_attn_bwd_step(t["q"], k[:, :256].contiguous(), k[:, :256].contiguous(), lse, lse, t["dout"],
                                   q_pos0=512, kv_pos0=0, causal=True)
    qf = t["q"].float()
    with pytest.raises(ra.RAError, match="RA_BF16"):
        ra.blockwise_attn_bwd_step(qf, qf, qf, lse, lse, qf, q_pos0=0, kv_pos0=0, causal=True)


# ------------------------------------------------------------------ seeded random sweep of the ring steps
STEP_SEED = 20261204
N_STEP_CASES = 16
STEP_MAX_PAIRS = 1 << 23   # batch * heads * kv_len^2 per case (all ranks of the ring), so the oracle stays in seconds


def step_sweep_cases(seed=STEP_SEED, n=N_STEP_CASES):
    """Seeded random shapes for the ring-step entry points (bfloat16, as the steps are): every rank
    of a ring on one GPU, blocks of any length (ragged included), head_dim 64 or 128, no causal mask,
    token-level or block-level causality, a bias of any length, segment ids sorted or scattered; plus
    the rank whose forward step chain is checked.  Pure host logic."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        i = len(cases)
        head_dim = int(rng.choice([64, 128]))
        batch = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 4))
        n_ring = int(rng.choice([2, 3, 4, 8]))
        if rng.random() < 0.4:
            lb = int(rng.integers(1, 1024 // n_ring + 1))
        else:
            lb = int(rng.choice([64, 128, 200, 256]))
        lb = max(1, min(lb, 2048 // n_ring))
        kv_len = n_ring * lb
        if batch * heads * kv_len * kv_len > STEP_MAX_PAIRS:
            continue
        divs = [d for d in range(2, lb + 1) if lb % d == 0]
        u = rng.random()
        causal = False if u < 0.25 else (True if (u < 0.7 or not divs) else int(rng.choice(divs)))
        bias_len = 0 if rng.random() < 0.4 else int(rng.integers(1, 2 * kv_len + 2))
        segments = str(rng.choice(["none", "docs", "scattered"]))
        lo = int(rng.integers(1, max(2, kv_len // 4) + 1))
        doc_len = (lo, int(rng.integers(lo, max(lo, kv_len // 2) + 1)))
        rank = int(rng.integers(0, n_ring))
        w = W.small(f"steps{i:02d}", batch=batch, heads=heads, head_dim=head_dim, kv_len=kv_len, n_ring=n_ring,
                    causal=causal, bias_len=bias_len, segments=segments, doc_len=doc_len, backward=True,
                    seed=int(rng.integers(0, 2**31)))
        cases.append((w, rank))
    return cases


STEP_CASES = step_sweep_cases()

# batch * heads a multiple of 8: the step kernels then run one (batch, head) per XCD at a time (the
# random shapes above have at most 6 pairs)
STEP_ORDER_CASES = [
    (W.small("steps-order-b2h4", batch=2, heads=4, kv_len=1024, n_ring=4, backward=True, seed=21), 2),
    (W.small("steps-order-b1h8-d128-bias", batch=1, heads=8, head_dim=128, kv_len=768, n_ring=3, bias_len=200,
             backward=True, seed=22), 1),
    (W.small("steps-order-b1h16-blocks", batch=1, heads=16, kv_len=512, n_ring=4, causal=32, backward=True,
             seed=23), 3),
]


def test_step_order_cases_are_valid():
    for w, r in STEP_ORDER_CASES:
        assert w.batch * w.heads % 8 == 0 and 0 <= r < w.n_ring
        assert w.batch * w.heads * w.kv_len * w.kv_len <= STEP_MAX_PAIRS


@pytest.mark.parametrize("case", STEP_CASES + STEP_ORDER_CASES, ids=[c[0].name for c in STEP_CASES + STEP_ORDER_CASES])
def test_step_sweep(gpu, case):
    w, r = case
    print("case", w, "rank", r, flush=True)
    t = P.make(w, gpu)
    lb = w.block_len
    rows = slice(r * lb, (r + 1) * lb)
    # forward: rank r's query block folds in every K/V block in ring order, then finalizes
    wr = W.replace(w, ring_rank=r)
    tr = dict(t, q=t["q"][:, rows].contiguous())
    out_r, lse_r = ra.blockwise_attn_fwd_finalize(_chain(wr, tr, _ring_order(wr)))
    # backward: every rank, dQ sums staying with the queries, dK / dV (and with a bias the per-key sums
    # of dS) travelling with their block
    out, lse = P.gpu_forward(w, t)
    res = _ring_backward(w, t, out, lse, with_dbias=t["bias"] is not None)
    torch.cuda.synchronize()
    d = P.oracle_inputs(t)
    import oracle
    ref_o, ref_l = P.oracle_forward(w, d, w.q_positions())
    P.assert_close(f"{w.name} rank {r} steps", P.np64(out_r), ref_o[:, rows], "bf16", strict=False)
    P.assert_lse(lse_r.cpu().numpy().astype(np.float64), ref_l[:, :, rows], "bf16")
    rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                                       bias=d["bias"], segment_ids=d["segment_ids"])
    for gname, g, ref in zip(("dq", "dk", "dv"), res[:3], (rdq, rdk, rdv)):
        P.assert_close(f"{w.name} {gname} steps", P.np64(g), ref, "bf16", strict=False)
    if t["bias"] is not None:
        ref_db = oracle.bias_grad(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                                  bias=d["bias"], segment_ids=d["segment_ids"])
        P.assert_close_sums(f"{w.name} dbias steps", res[3].double().cpu().numpy(), ref_db)
