"""The allocation-free backward (ra_blockwise_attn_bwd_noalloc, Delta in the library's static device
scratch) against the ordinary backward (ra_blockwise_attn_bwd, Delta in a caller workspace) and the
oracle: two calls in a row on one GPU, the second with a smaller input, so the second reuses what
the first left in the scratch array.  The same call captured in a HIP graph (torch.cuda.CUDAGraph) must
reproduce the eager gradients bit for bit on every replay, with eager work between replays that leaves
other values in the scratch array and overwrites the outputs."""
import numpy as np
import pytest
import torch

import long_context_exact_attn_amd as ra
from long_context_exact_attn_amd import workloads as W
import _parity as P

pytestmark = pytest.mark.gpu


def _run(w, dev):
    t = P.make(w, dev)
    out, lse = P.gpu_forward(w, t)
    kw = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    dq0, dk0, dv0 = ra.blockwise_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"],
                                          **kw)
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ra.blockwise_attn_bwd_noalloc(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"], **kw,
                                  dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return t, (dq0, dk0, dv0), (dq, dk, dv)


def test_noalloc_matches_workspace_backward_twice(gpu):
    big = W.small("noalloc-big", batch=2, heads=3, kv_len=4096, n_ring=4, bias_len=300, segments="docs",
                  doc_len=(100, 900), backward=True, seed=11)
    small = W.small("noalloc-small", batch=1, heads=2, kv_len=1000, n_ring=4, ring_rank=2, backward=True, seed=12)
    for w in (big, small):
        print("case", w.name, flush=True)
        t, ref, got = _run(w, gpu)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), f"{w.name} {name} differs from the workspace backward"
        d = P.oracle_inputs(t)
        import oracle
        rdq, rdk, rdv, _ = oracle.backward(d["q"], d["k"], d["v"], d["dout"], q_pos=w.q_positions(),
                                           causal=w.causal, bias=d["bias"], segment_ids=d["segment_ids"])
        for name, g, r in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
            P.assert_close(f"{w.name} {name}", P.np64(g), r, "bf16", strict=False)


def test_noalloc_rejects_sizes_over_its_scratch(gpu):
    lib = ra.load_library()
    cap_rows = lib.ra_blockwise_attn_bwd_noalloc_max_workspace() // 4
    assert cap_rows == 4194304
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device=gpu)
    # a shape one block past the limit is refused before anything is launched (pointers never read)
    from long_context_exact_attn_amd import api
    import ctypes
    s = api.Shape(1, 65, 64, -1, 65536, 65536, 0, 0.0, api.RA_BF16)
    rc = lib.ra_blockwise_attn_bwd_noalloc(*([None] * 5), 1, 1, 1, 1, *([None] * 6), ctypes.byref(s), None)
    assert rc == -4 and b"4,194,304" in lib.ra_noalloc_last_error()
    del q


def test_noalloc_backward_replays_in_a_graph(gpu):
    w = W.small("noalloc-graph", batch=1, heads=2, kv_len=2048, n_ring=2, bias_len=64, segments="docs",
                doc_len=(100, 700), backward=True, seed=13)
    other = W.small("noalloc-graph-other", batch=2, heads=3, kv_len=1536, n_ring=3, backward=True, seed=14)
    t, u = P.make(w, gpu), P.make(other, gpu)
    out, lse = P.gpu_forward(w, t)
    out_u, lse_u = P.gpu_forward(other, u)
    kw = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    kw_u = dict(n_ring=other.n_ring, q_chunk=other.q_chunk, k_chunk=other.k_chunk, causal=other.causal,
                ring_rank=other.ring_rank)
    args = (t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"])
    args_u = (u["q"], u["k"], u["v"], out_u, lse_u, u["dout"], u["bias"], u["segment_ids"])
    grads = [torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])]
    grads_u = [torch.empty_like(u["q"]), torch.empty_like(u["k"]), torch.empty_like(u["v"])]

    # eager call first (it also looks up the scratch array's device address, outside any capture)
    ra.blockwise_attn_bwd_noalloc(*args, **kw, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    ref = [g.clone() for g in grads]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ra.blockwise_attn_bwd_noalloc(*args, **kw, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()

    for i in range(4):
        print("replay", i, flush=True)
        for g in grads:
            g.fill_(float("nan"))
        # another shape through the same scratch array, eagerly
        ra.blockwise_attn_bwd_noalloc(*args_u, **kw_u, dq=grads_u[0], dk=grads_u[1], dv=grads_u[2])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            assert torch.equal(g, r), f"replay {i}: {name} differs from the eager call"
