"""Seeded random sweep of small shapes: forward and backward of the HIP path against the oracle
on full tensors.  One fixed seed draws 40 cases over batch, heads, head_dim, ring size and rank,
block length (ragged included), query / key chunk sizes, causal block size, bias length and
segment ids.  Chunk sizes and the ring's blocking change nothing but rounding, because the method
keeps the whole attention map ("手把手拆解RingAttention", section 1; the chunk sizes are the
query_chunk_size / key_chunk_size of "RingAttention核心功能全解析", section "分块注意力计算")."""
import numpy as np
import pytest
import torch

from long_context_exact_attn_amd import workloads as W
import _parity as P

SEED = 20261203
N_CASES = 40
MAX_PAIRS = 1 << 24   # batch * heads * q_len * kv_len per case, so the oracle stays in seconds


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def sweep_cases(seed=SEED, n=N_CASES):
    """The sweep's workloads, drawn from one seeded generator (pure host logic)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        i = len(cases)
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        head_dim = int(rng.choice([64, 128]))
        batch = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 5))
        n_ring = int(rng.choice([1, 2, 4, 8]))
        lb = int(rng.integers(1, 4096 // n_ring + 1)) if rng.random() < 0.3 else int(rng.choice([64, 128, 192, 256, 320, 512]))
        lb = max(1, min(lb, 4096 // n_ring))
        kv_len = n_ring * lb
        ring_rank = -1 if rng.random() < 0.5 else int(rng.integers(0, n_ring))
        q_len = kv_len if ring_rank < 0 else lb
        if batch * heads * q_len * kv_len > MAX_PAIRS:
            continue
        divs = _divisors(lb)
        q_chunk, k_chunk = int(rng.choice(divs)), int(rng.choice(divs))
        u = rng.random()
        if u < 0.25:
            causal = False
        elif u < 0.75:
            causal = True
        else:
            big = [d for d in divs if d > 1]
            causal = int(rng.choice(big)) if big else True
        bias_len = 0 if rng.random() < 0.5 else int(rng.integers(1, 2 * kv_len + 2))
        segments = str(rng.choice(["none", "none", "docs", "scattered"]))
        lo = int(rng.integers(1, max(2, kv_len // 4) + 1))
        doc_len = (lo, int(rng.integers(lo, max(lo, kv_len // 2) + 1)))
        cases.append(W.small(f"sweep{i:02d}", batch=batch, heads=heads, head_dim=head_dim, kv_len=kv_len,
                             n_ring=n_ring, ring_rank=ring_rank, dtype=dtype, causal=causal, bias_len=bias_len,
                             segments=segments, doc_len=doc_len, backward=True, q_chunk=q_chunk, k_chunk=k_chunk,
                             seed=int(rng.integers(0, 2**31))))
    return cases


CASES = sweep_cases()


def test_sweep_cases_are_valid():
    # host logic only: every drawn case satisfies the C ABI's blocking rules
    assert len(CASES) == N_CASES
    for w in CASES:
        lb = w.block_len
        assert w.kv_len == w.n_ring * lb and lb % w.q_chunk == 0 and lb % w.k_chunk == 0
        assert w.causal in (False, True) or lb % int(w.causal) == 0
        assert w.batch * w.heads * w.q_len * w.kv_len <= MAX_PAIRS
    # the draw is reproducible
    assert [c.name for c in sweep_cases()] == [c.name for c in CASES]
    assert sweep_cases()[7] == CASES[7]


# Workgroup order: with batch * heads a multiple of 8, every kernel of a single rank's share (and the forward
# of the whole ring) runs the (batch, head) pairs one after the other on each XCD; otherwise pairs vary
# fastest.  Full tensors of both orders, over several tiles per pair.
ORDER_CASES = [
    W.small("order-b2h4-rank1", batch=2, heads=4, kv_len=1024, n_ring=4, ring_rank=1, backward=True, seed=11),
    W.small("order-b1h16-rank3", batch=1, heads=16, kv_len=1024, n_ring=4, ring_rank=3, backward=True, seed=12),
    W.small("order-b1h24-ring", batch=1, heads=24, kv_len=512, n_ring=2, ring_rank=-1, backward=True, seed=13),
    W.small("order-b2h8-d128-rank0-bias", batch=2, heads=8, head_dim=128, kv_len=512, n_ring=2, ring_rank=0,
            bias_len=96, backward=True, seed=14),
    W.small("order-b1h12-rank2", batch=1, heads=12, kv_len=1024, n_ring=4, ring_rank=2, backward=True, seed=15),
]


def test_order_cases_are_valid():
    for w in ORDER_CASES:
        assert w.batch * w.heads * w.q_len * w.kv_len <= MAX_PAIRS
    assert {w.batch * w.heads % 8 == 0 for w in ORDER_CASES} == {True, False}


@pytest.mark.gpu
@pytest.mark.parametrize("w", ORDER_CASES, ids=[c.name for c in ORDER_CASES])
def test_workgroup_order(gpu, w):
    _check(gpu, w)


@pytest.mark.gpu
@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_sweep(gpu, w):
    _check(gpu, w)


def _check(gpu, w):
    print(w, flush=True)
    t = P.make(w, gpu)
    out, lse = P.gpu_forward(w, t)
    dq, dk, dv = P.gpu_backward(w, t, out, lse)
    torch.cuda.synchronize()
    d = P.oracle_inputs(t)
    import oracle
    ref_o, ref_l = P.oracle_forward(w, d, w.q_positions())
    rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(), causal=w.causal,
                                       bias=d["bias"], segment_ids=d["segment_ids"])
    if w.dtype == "f32":
        P.assert_close("out", P.np64(out), ref_o, "f32")
        P.assert_lse(lse.cpu().numpy().astype(np.float64), ref_l, "f32")
        # float32 gradients sum over many keys: 1e-4 relative to the gradient's scale
        for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            err = float(np.max(np.abs(P.np64(g) - r))) if r.size else 0.0
            print(f"{name}: max_abs={err:.3e}", flush=True)
            assert err <= 1e-4 * max(1.0, float(np.max(np.abs(r))) if r.size else 1.0)
    else:
        P.assert_close("out", P.np64(out), ref_o, "bf16", strict=False)
        P.assert_lse(lse.cpu().numpy().astype(np.float64), ref_l, "bf16")
        for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            P.assert_close(name, P.np64(g), r, "bf16", strict=False)
