"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding, run the oracle on the same (rounded) inputs, and compare."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import long_context_exact_attn_amd as ra
import oracle
from long_context_exact_attn_amd import workloads as W

# tolerances: float32 path max abs 1e-4 on outputs; bfloat16 path max abs 2e-2 and
# relative RMS 1e-2 on outputs and gradients; lse (float32 in both) max abs 1e-3 / 1e-5
TOL = {"f32": dict(max_abs=1e-4, rel_rms=None, lse=1e-5), "bf16": dict(max_abs=2e-2, rel_rms=1e-2, lse=1e-3)}


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_forward(w, t, **over):
    kw = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    kw.update(over)
    return ra.blockwise_attn_fwd(t["q"], t["k"], t["v"], t["bias"], t["segment_ids"], **kw)


def gpu_backward(w, t, out, lse, **over):
    kw = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    kw.update(over)
    return ra.blockwise_attn_bwd(t["q"], t["k"], t["v"], out, lse, t["dout"], t["bias"], t["segment_ids"], **kw)


def oracle_inputs(t, heads=None, rows=None):
    """float64 numpy copies of the inputs, optionally for some heads / query rows."""
    hs = slice(None) if heads is None else heads
    q = t["q"][:, :, hs]
    if rows is not None:
        q = q[:, rows]
    d = dict(q=np64(q), k=np64(t["k"][:, :, hs]), v=np64(t["v"][:, :, hs]),
             bias=None if t["bias"] is None else np64(t["bias"][hs]),
             segment_ids=None if t["segment_ids"] is None else t["segment_ids"].cpu().numpy())
    if t.get("dout") is not None:
        g = t["dout"][:, :, hs]
        d["dout"] = np64(g if rows is None else g[:, rows])
    return d


def oracle_forward(w, d, q_pos):
    return oracle.forward(d["q"], d["k"], d["v"], q_pos=q_pos, causal=w.causal, bias=d["bias"],
                          segment_ids=d["segment_ids"])


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


# Rounding a float to bfloat16 (round to nearest even, 8 significant bits) moves it by at most half
# a unit in the last place, i.e. by at most 2^-8 |x|.  Outputs and gradients are rounded to
# bfloat16 once, so where |ref| is large that rounding alone can exceed the absolute bound.
HALF_ULP_BF16 = 2.0 ** -8


def assert_close(name, got, ref, dtype, strict=True):
    """strict: max |got - ref| <= the absolute bound.  Otherwise (small synthetic cases and
    gradients whose values can exceed 4, where bfloat16's own spacing exceeds the bound):
    elementwise |got - ref| <= bound + 2^-8 |ref|, the bound plus the half ulp that rounding
    the result to bfloat16 may cost.  The relative RMS bound applies in both cases."""
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs, rel = errors(got, ref)
    msg = f"{name}: max_abs={max_abs:.3e} rel_rms={rel:.3e} max|ref|={np.abs(ref).max() if ref.size else 0:.3g}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    if strict or dtype == "f32":
        assert max_abs <= tol["max_abs"], msg
    else:
        excess = np.abs(got - ref) - (tol["max_abs"] + HALF_ULP_BF16 * np.abs(ref))
        assert excess.size == 0 or excess.max() <= 0, msg + f" (worst excess {excess.max():.3e})"
    if tol["rel_rms"] is not None:
        assert rel <= tol["rel_rms"], msg


def assert_close_sums(name, got, ref):
    """Gradients that are sums over many products (the bias gradient, the feed-forward's weight
    gradients): the bfloat16 path's bounds (max abs 2e-2, relative RMS 1e-2) applied to the gradient
    normalised by its own scale, i.e.
    max |got - ref| <= 2e-2 max|ref| + 1e-3 and relative RMS <= 1e-2.  (Their size grows with the
    number of summed terms, so a fixed absolute bound would say nothing at large sizes.)"""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs, rel = errors(got, ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    msg = f"{name}: max_abs={max_abs:.3e} rel_rms={rel:.3e} max|ref|={scale:.3g}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), name + ": non-finite values"
    assert max_abs <= 2e-2 * scale + 1e-3, msg
    assert rel <= 1e-2, msg


def assert_lse(got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same_inf = np.isneginf(got) == np.isneginf(ref)
    assert np.all(same_inf), "lse: rows with no visible key differ"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    print(f"lse: max_abs={err:.3e}", flush=True)
    assert err <= TOL[dtype]["lse"], f"lse max_abs {err}"


def sample_rows(w, n, seed=0):
    """A fixed sample of local query rows: n seeded rows plus the first and last row of every ring block
    the queries span."""
    rng = np.random.default_rng(seed)
    Lq, Lb = w.q_len, w.block_len
    rows = set(rng.choice(Lq, size=min(n, Lq), replace=False).tolist())
    for start in range(0, Lq, Lb):
        rows.update((start, start + Lb - 1))
    return np.array(sorted(rows), dtype=np.int64)


def make(w, device):
    return W.make(w, device=device)


# ------------------------------------------------------------------ the oracle over row blocks
def workers():
    """Threads for the oracle: the host's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _split(n, parts):
    step = max(1, -(-n // parts))
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def _pool_map(fn, items, nthreads):
    """fn over items in threads, each with a one-thread BLAS (numpy releases the GIL in its
    loops, so the row blocks run in parallel)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(nthreads) as ex:
            return list(ex.map(fn, items))


def oracle_forward_rows(d, q_pos, causal, nthreads=None):
    """oracle.forward over blocks of query rows in threads; same result as one call."""
    import oracle
    nthreads = nthreads or workers()
    nq = d["q"].shape[1]

    def one(r):
        i0, i1 = r
        return oracle.forward(d["q"][:, i0:i1], d["k"], d["v"], q_pos=q_pos[i0:i1], causal=causal, bias=d["bias"],
                              segment_ids=d["segment_ids"])
    parts = _pool_map(one, _split(nq, 4 * nthreads), nthreads)
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=2)


def oracle_backward_rows(d, q_pos, causal, nthreads=None):
    """oracle.backward over blocks of query rows in threads: dq by rows, and dk / dv as the sum of
    every block's contributions (the oracle returns a row subset's contributions)."""
    import oracle
    nthreads = nthreads or workers()
    nq = d["q"].shape[1]

    def one(r):
        i0, i1 = r
        return oracle.backward(d["q"][:, i0:i1], d["k"], d["v"], d["dout"][:, i0:i1], q_pos=q_pos[i0:i1],
                               causal=causal, bias=d["bias"], segment_ids=d["segment_ids"])
    parts = _pool_map(one, _split(nq, nthreads), nthreads)
    dq = np.concatenate([p[0] for p in parts], axis=1)
    dk = parts[0][1]
    dv = parts[0][2]
    for p in parts[1:]:
        dk += p[1]
        dv += p[2]
    return dq, dk, dv
