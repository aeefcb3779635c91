"""GPU parity: the HIP path (through the C-ABI) against the float64 CPU oracle
on the same seeded inputs, plus properties that must hold at any size."""
import numpy as np
import pytest
import torch

import long_context_exact_attn_amd as ra
from long_context_exact_attn_amd import workloads as W
import _parity as P

pytestmark = pytest.mark.gpu


def _check_forward(w, dev, rows=None, heads=None, strict=True):
    t = P.make(w, dev)
    out, lse = P.gpu_forward(w, t)
    torch.cuda.synchronize()
    qpos = w.q_positions()
    sel = slice(None) if rows is None else rows
    d = P.oracle_inputs(t, heads=heads, rows=rows)
    ref_o, ref_l = P.oracle_forward(w, d, qpos[sel])
    hs = slice(None) if heads is None else heads
    got_o = P.np64(out[:, :, hs][:, sel])
    got_l = lse[:, hs].detach().cpu().numpy().astype(np.float64)[:, :, sel]
    P.assert_close(f"{w.name} out", got_o, ref_o, w.dtype, strict=strict)
    P.assert_lse(got_l, ref_l, w.dtype)
    return t, out, lse


# ------------------------------------------------------------------ the configured workloads
def test_tiny_f32_full(gpu):
    w = W.WORKLOADS["tiny-f32-1k"]
    t, out, lse = _check_forward(w, gpu)
    # all segment ids 0 means no masking: identical to passing no segment ids at all
    out2, lse2 = ra.blockwise_attn_fwd(t["q"], t["k"], t["v"], None, None, n_ring=w.n_ring, q_chunk=w.q_chunk,
                                       k_chunk=w.k_chunk, causal=w.causal)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_causal_32k_full(gpu):
    # every row of every head against the oracle (row blocks in threads)
    w = W.WORKLOADS["causal-32k"]
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    torch.cuda.synchronize()
    ref_o, ref_l = P.oracle_forward_rows(P.oracle_inputs(t), w.q_positions(), w.causal)
    P.assert_close(f"{w.name} out", P.np64(out), ref_o, w.dtype)
    P.assert_lse(lse.cpu().numpy().astype(np.float64), ref_l, w.dtype)


def test_share_1m_rank7_sampled_rows(gpu):
    w = W.WORKLOADS["share-1m-r7"]
    _check_forward(w, gpu, rows=P.sample_rows(w, 96, seed=2), heads=slice(0, 16, 5))


def test_share_1m_rank7_backward_sampled(gpu):
    # the full backward at the 1M-token share, in the launch configuration bench.py times:
    # dQ on sampled rows of two heads against the oracle (which forms lse and Delta itself),
    # dK / dV through properties that hold at any size
    w = W.replace(W.WORKLOADS["share-1m-r7"], backward=True)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    rows = P.sample_rows(w, 32, seed=4)
    import oracle
    for h in (0, 11):
        d = P.oracle_inputs(t, heads=slice(h, h + 1), rows=rows)
        rdq, _, _, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions()[rows], causal=True)
        P.assert_close(f"{w.name} dq[h={h}]", P.np64(dq[:, rows, h:h + 1]), rdq, "bf16")
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i on every head (the keys see only this rank's queries)
    sdk = dk.float().sum(dim=1)
    sdv, sdo = dv.float().sum(dim=1), t["dout"].float().sum(dim=1)
    scale_k = dk.float().abs().sum(dim=1)
    assert torch.all(sdk.abs() <= 2e-2 * scale_k + 1e-3), float((sdk.abs() / scale_k).max())
    assert torch.allclose(sdv, sdo, rtol=2e-2, atol=2e-1), float((sdv - sdo).abs().max())


def test_packed_docs_64k_sampled_rows(gpu):
    w = W.WORKLOADS["packed-docs-64k"]
    _check_forward(w, gpu, rows=P.sample_rows(w, 192, seed=3), heads=slice(0, 32, 7))


def test_train_32k_full_backward_four_heads(gpu):
    # dQ, dK, dV of heads 0, 5, 10 and 15 element by element; invariants on every head
    w = W.WORKLOADS["train-32k"]
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    for h in (0, 5, 10, 15):
        d = P.oracle_inputs(t, heads=slice(h, h + 1))
        rdq, rdk, rdv = P.oracle_backward_rows(d, w.q_positions(), w.causal)
        for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            P.assert_close(f"{w.name} {name}[h={h}]", P.np64(g[:, :, h:h + 1]), r, "bf16", strict=False)
    # invariants on every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    sdk = dk.float().sum(dim=1)
    sdv, sdo = dv.float().sum(dim=1), t["dout"].float().sum(dim=1)
    scale_k = dk.float().abs().sum(dim=1)
    assert torch.all(sdk.abs() <= 2e-2 * scale_k + 1e-3), float((sdk.abs() / scale_k).max())
    assert torch.allclose(sdv, sdo, rtol=2e-2, atol=2e-1), float((sdv - sdo).abs().max())


def test_share_1m_keys_full_head_gradients(gpu):
    # One rank's launch whose K/V spans all 1,048,576 keys: ring rank 255 of 256 blocks of 4096
    # tokens, 16 heads, causal.  Head 9's dQ (all 4096 rows) and dK, dV (all 1,048,576 keys, so
    # every ring block's first and last key, and the top blocks whose byte offsets pass 2^31) are
    # compared element by element with the oracle, which forms P, lse and Delta itself.
    w = W.replace(W.WORKLOADS["share-1m-r7"], name="share-1m-keys-r255", n_ring=256, ring_rank=255,
                  backward=True)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    h = 9
    d = P.oracle_inputs(t, heads=slice(h, h + 1))
    rdq, rdk, rdv = P.oracle_backward_rows(d, w.q_positions(), w.causal)
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        P.assert_close(f"{w.name} {name}[h={h}]", P.np64(g[:, :, h:h + 1]), r, "bf16")
    # the last ring block's keys: the causal diagonal, partly visible
    lb = w.block_len
    P.assert_close(f"{w.name} dk[h={h}] last block", P.np64(dk[:, -lb:, h:h + 1]), rdk[:, -lb:], "bf16")


def test_packed_docs_64k_backward(gpu):
    # The packed-document workload's backward in the launch bench-style runs use: dQ on sampled rows
    # of three heads; and, for the two shortest documents of each batch row in two heads, dQ of all
    # their rows and dK, dV of all their keys (a key is seen only by its own document's queries, so
    # the oracle over that document's rows gives the whole gradient of its keys).
    w = W.replace(W.WORKLOADS["packed-docs-64k"], backward=True)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    import oracle
    rows = P.sample_rows(w, 64, seed=6)
    heads = (0, 17, 31)
    for h in heads:
        d = P.oracle_inputs(t, heads=slice(h, h + 1), rows=rows)
        rdq, _, _, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions()[rows],
                                       causal=w.causal, bias=d["bias"], segment_ids=d["segment_ids"])
        P.assert_close(f"{w.name} dq[h={h}] sampled", P.np64(dq[:, rows, h:h + 1]), rdq, "bf16", strict=False)
    seg = t["segment_ids"].cpu().numpy()
    for b in range(w.batch):
        ids, starts, counts = np.unique(seg[b], return_index=True, return_counts=True)
        for doc in ids[np.argsort(counts, kind="stable")[:2]]:
            sel = np.nonzero(seg[b] == doc)[0]
            lo, hi = int(sel[0]), int(sel[-1]) + 1
            for h in (5, 26):
                tb = {k_: (None if v_ is None else v_[b:b + 1]) for k_, v_ in t.items() if k_ != "bias"}
                tb["bias"] = t["bias"]
                d = P.oracle_inputs(tb, heads=slice(h, h + 1), rows=np.arange(lo, hi))
                rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=np.arange(lo, hi),
                                                   causal=w.causal, bias=d["bias"], segment_ids=d["segment_ids"])
                tag = f"{w.name} b={b} doc={doc} [{lo},{hi}) h={h}"
                P.assert_close(f"{tag} dq", P.np64(dq[b:b + 1, lo:hi, h:h + 1]), rdq, "bf16", strict=False)
                P.assert_close(f"{tag} dk", P.np64(dk[b:b + 1, lo:hi, h:h + 1]), rdk[:, lo:hi], "bf16",
                               strict=False)
                P.assert_close(f"{tag} dv", P.np64(dv[b:b + 1, lo:hi, h:h + 1]), rdv[:, lo:hi], "bf16",
                               strict=False)
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i on every (batch, head)
    sdk = dk.float().sum(dim=1)
    sdv, sdo = dv.float().sum(dim=1), t["dout"].float().sum(dim=1)
    scale_k = dk.float().abs().sum(dim=1)
    assert torch.all(sdk.abs() <= 2e-2 * scale_k + 1e-3), float((sdk.abs() / scale_k).max())
    assert torch.allclose(sdv, sdo, rtol=2e-2, atol=2e-1), float((sdv - sdo).abs().max())


# ------------------------------------------------------------------ small full-tensor sweep
SWEEP = [
    # (name, kwargs)
    ("causal-ring4", dict(kv_len=1024, n_ring=4)),
    ("noncausal-ring2", dict(kv_len=512, n_ring=2, causal=False)),
    ("rank0", dict(kv_len=2048, n_ring=4, ring_rank=0)),
    ("rank3", dict(kv_len=2048, n_ring=4, ring_rank=3)),
    ("rank2-noncausal", dict(kv_len=1536, n_ring=3, ring_rank=2, causal=False)),
    ("ragged-100", dict(kv_len=400, n_ring=4)),
    ("ragged-250-rank1", dict(kv_len=1000, n_ring=4, ring_rank=1)),
    ("ragged-1-token-blocks", dict(kv_len=7, n_ring=7)),
    ("bias", dict(kv_len=1024, n_ring=2, bias_len=300)),
    ("segments", dict(kv_len=1024, n_ring=4, segments="docs", doc_len=(20, 200))),
    ("bias-seg-noncausal", dict(kv_len=768, n_ring=3, causal=False, bias_len=64, segments="docs", doc_len=(5, 90))),
    ("d128", dict(head_dim=128, kv_len=1024, n_ring=4, heads=3)),
    ("d128-all", dict(head_dim=128, kv_len=960, n_ring=3, batch=2, bias_len=100, segments="docs", doc_len=(30, 300),
                      ring_rank=2)),
    ("batch3-heads5", dict(batch=3, heads=5, kv_len=640, n_ring=5)),
    ("n_ring1", dict(kv_len=1000, n_ring=1)),
    ("f32-causal-seg", dict(dtype="f32", kv_len=600, n_ring=3, segments="docs", doc_len=(10, 150), bias_len=33)),
    # several 64-tile windows of segment ids per ring block, long and short documents
    ("docs-long", dict(kv_len=12288, n_ring=3, ring_rank=2, segments="docs", doc_len=(50, 3000), heads=2)),
    ("docs-long-d128", dict(head_dim=128, kv_len=9216, n_ring=2, segments="docs", doc_len=(20, 5000), heads=2,
                            bias_len=512)),
    # causal block sizes c > 1 (a key is visible when its block of c tokens does not come after the
    # query's): c below, equal to and above the 64-token tile, a ragged block, with masks and bias
    ("causal-block-64", dict(kv_len=1024, n_ring=4, causal=64)),
    ("causal-block-16-ragged", dict(kv_len=1000, n_ring=4, causal=50)),
    ("causal-block-128-rank2", dict(kv_len=2048, n_ring=4, ring_rank=2, causal=128, segments="docs", doc_len=(30, 500),
                                    bias_len=100)),
    ("causal-block-whole-ring-block", dict(kv_len=1024, n_ring=4, causal=256)),
    ("causal-block-d128", dict(head_dim=128, kv_len=1536, n_ring=3, causal=256, heads=3)),
    ("causal-block-f32", dict(dtype="f32", kv_len=512, n_ring=2, causal=32, bias_len=9)),
    # unsorted ids, int32 extremes included: tile skipping must stay exact for any ids
    ("ids-scattered", dict(kv_len=6144, n_ring=3, segments="scattered", heads=2)),
    ("ids-scattered-noncausal", dict(kv_len=2048, n_ring=2, causal=False, segments="scattered", bias_len=77)),
    ("f32-d128-rank1", dict(dtype="f32", head_dim=128, kv_len=512, n_ring=4, ring_rank=1)),
]


@pytest.mark.parametrize("name,kw", SWEEP, ids=[s[0] for s in SWEEP])
def test_small_forward(gpu, name, kw):
    w = W.small(name, **kw)
    _check_forward(w, gpu, strict=False)


@pytest.mark.parametrize("name,kw", [s for s in SWEEP if s[0] not in ("ragged-1-token-blocks",)],
                         ids=[s[0] for s in SWEEP if s[0] not in ("ragged-1-token-blocks",)])
def test_small_backward(gpu, name, kw):
    w = W.small(name, backward=True, **kw)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    d = P.oracle_inputs(t)
    import oracle
    rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                                       bias=d["bias"], segment_ids=d["segment_ids"])
    tol = "f32" if w.dtype == "f32" else "bf16"
    if tol == "f32":
        # float32 gradients accumulate over many keys; allow 1e-4 relative to the gradient's scale
        for name_, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            err = np.max(np.abs(P.np64(g) - r))
            print(f"{name_}: max_abs={err:.3e}", flush=True)
            assert err <= 1e-4 * max(1.0, np.max(np.abs(r)))
    else:
        for name_, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            P.assert_close(name_, P.np64(g), r, "bf16", strict=False)


# ------------------------------------------------------------------ properties
def test_chunk_sizes_do_not_change_results(gpu):
    w = W.small("chunks", kv_len=2048, n_ring=2, bias_len=128, segments="docs", doc_len=(50, 400))
    t = P.make(w, gpu)
    ref = P.gpu_forward(w, t, q_chunk=1024, k_chunk=1024)
    for qc, kc in ((1, 1), (64, 512), (256, 8), (1024, 16)):
        o, l_ = P.gpu_forward(w, t, q_chunk=qc, k_chunk=kc)
        assert torch.equal(o, ref[0]) and torch.equal(l_, ref[1]), (qc, kc)


def test_ring_order_changes_only_rounding(gpu):
    base = W.small("ring", kv_len=4096, n_ring=1, heads=4)
    t = P.make(base, gpu)
    o1, l1 = P.gpu_forward(base, t)
    for n in (2, 4, 8, 16):
        o, l_ = P.gpu_forward(base, t, n_ring=n, q_chunk=4096 // n, k_chunk=4096 // n)
        P.assert_close(f"n_ring={n} vs 1", P.np64(o), P.np64(o1), "bf16")
        assert float((l_ - l1).abs().max()) < 1e-4


def test_masked_keys_do_not_leak(gpu):
    # causal: rewriting every key/value after position p leaves rows <= p bitwise unchanged
    w = W.small("leak", kv_len=2048, n_ring=4, heads=2, segments="docs", doc_len=(40, 300), bias_len=512)
    t = P.make(w, gpu)
    o1, l1 = P.gpu_forward(w, t)
    p = 1234
    t2 = dict(t)
    t2["k"] = t["k"].clone()
    t2["v"] = t["v"].clone()
    t2["k"][:, p + 1:] = torch.randn_like(t["k"][:, p + 1:].float()).to(t["k"].dtype) * 3
    t2["v"][:, p + 1:] = torch.randn_like(t["v"][:, p + 1:].float()).to(t["v"].dtype) * 3
    o2, l2 = P.gpu_forward(w, t2)
    assert torch.equal(o1[:, :p + 1], o2[:, :p + 1]) and torch.equal(l1[:, :, :p + 1], l2[:, :, :p + 1])
    assert not torch.equal(o1[:, p + 1:], o2[:, p + 1:])


def test_forward_is_deterministic(gpu):
    w = W.small("det", kv_len=4096, n_ring=8, heads=4, bias_len=100)
    t = P.make(w, gpu)
    o1, l1 = P.gpu_forward(w, t)
    for _ in range(3):
        o, l_ = P.gpu_forward(w, t)
        assert torch.equal(o, o1) and torch.equal(l_, l1)


def test_empty_inputs(gpu):
    q = torch.empty(0, 256, 2, 64, dtype=torch.bfloat16, device=gpu)
    out, lse = ra.blockwise_attn_fwd(q, q, q, n_ring=1, q_chunk=256, k_chunk=256, causal=True)
    assert out.shape == q.shape and lse.shape == (0, 2, 256)
    q = torch.empty(1, 0, 2, 64, dtype=torch.bfloat16, device=gpu)
    out, lse = ra.blockwise_attn_fwd(q, q, q, n_ring=4, q_chunk=1, k_chunk=1, causal=True)
    assert out.shape == q.shape
    # no pair is visible: the bias gradient is cleared, whatever its buffer held
    bias = torch.ones(2, 40, dtype=torch.float32, device=gpu)
    dbias = torch.full_like(bias, 7.0)
    ra.blockwise_attn_bwd_dbias(q, q, q, out, lse, q, bias, n_ring=4, q_chunk=1, k_chunk=1, causal=True, dbias=dbias)
    torch.cuda.synchronize()
    assert not dbias.any()


def test_errors_surface_as_exceptions(gpu):
    q = torch.zeros(1, 1000, 2, 64, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(ra.RAError, match="ring does not close"):
        ra.blockwise_attn_fwd(q, q, q, n_ring=3, q_chunk=1, k_chunk=1, causal=True)
    q96 = torch.zeros(1, 64, 2, 96, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(ra.RAError, match="head_dim"):
        ra.blockwise_attn_fwd(q96, q96, q96, n_ring=1, q_chunk=64, k_chunk=64, causal=True)


# ------------------------------------------------------------------ bias gradient
DBIAS = [
    ("bias-causal", dict(kv_len=1024, n_ring=4, bias_len=300)),
    ("bias-f32", dict(dtype="f32", kv_len=768, n_ring=3, bias_len=50, segments="docs", doc_len=(10, 200))),
    ("bias-f32-rank1-blocks", dict(dtype="f32", head_dim=128, kv_len=512, n_ring=4, ring_rank=1, bias_len=600,
                                   causal=16)),
    ("bias-seg-noncausal", dict(kv_len=768, n_ring=3, causal=False, bias_len=64, segments="docs", doc_len=(5, 90))),
    ("bias-rank2-longer-than-keys", dict(kv_len=2048, n_ring=4, ring_rank=2, bias_len=3000)),
    ("bias-d128-batch2-blocks", dict(head_dim=128, batch=2, heads=3, kv_len=960, n_ring=3, bias_len=100, causal=40,
                                     segments="scattered")),
]


@pytest.mark.parametrize("name,kw", DBIAS, ids=[c[0] for c in DBIAS])
def test_bias_gradient(gpu, name, kw):
    w = W.small(name, backward=True, **kw)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    kwr = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    dq, dk, dv, db = ra.blockwise_attn_bwd_dbias(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"],
                                                 t["segment_ids"], **kwr)
    fq, fk, fv = P.gpu_backward(w, t, out, lse)
    db2 = ra.blockwise_attn_bwd_dbias(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"],
                                      **kwr)[3]
    torch.cuda.synchronize()
    # the other gradients are those of the plain backward, bit for bit; dbias is deterministic
    assert torch.equal(dq, fq) and torch.equal(dk, fk) and torch.equal(dv, fv)
    assert torch.equal(db, db2)
    d = P.oracle_inputs(t)
    import oracle
    ref = oracle.bias_grad(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                           bias=d["bias"], segment_ids=d["segment_ids"])
    got = db.double().cpu().numpy()
    P.assert_close_sums(f"{name} dbias", got, ref)
    if w.dtype == "f32":
        # float32 throughout: the sums match to float32 rounding
        assert np.abs(got - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())
    assert abs(float(got.sum())) <= 1e-2 * np.abs(got).sum() + 1e-3   # scores' gradient sums to zero per row
