"""GPU parity of the blockwise feed-forward (SwiGLU, chunk by chunk over tokens) against the
float64 oracle, through the C-ABI binding."""
import numpy as np
import pytest
import torch

import long_context_exact_attn_amd as ra
import oracle
import _parity as P

pytestmark = pytest.mark.gpu


def _inputs(T, d, f, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    w1 = (torch.randn((f, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    w3 = (torch.randn((f, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn((d, f), generator=g, device=dev) / f ** 0.5).to(torch.bfloat16)
    dout = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    return x, w1, w3, w2, dout


def _close(name, got, ref):
    # bfloat16 operands, float32 accumulation: relative RMS <= 1e-2, max error <= 2e-2 of the scale
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"{name}: max_abs={err.max():.3e} rel_rms={rel:.3e} max|ref|={np.abs(ref).max():.3g}", flush=True)
    assert np.all(np.isfinite(got))
    assert rel <= 1e-2 and err.max() <= 2e-2 * np.abs(ref).max() + 1e-3, name


CASES = [
    ("ragged-chunks", 3000, 256, 704, 1024),
    ("one-chunk", 512, 128, 352, 4096),
    ("chunk-1-token", 5, 64, 96, 1),
    ("wide", 1536, 512, 1408, 512),
    # d_ff 200: one wave's 32 hidden units straddle the end; d_model 136: a ragged K step; 777 = 2 x 300 + 177
    ("ragged-hidden", 777, 136, 200, 300),
]


@pytest.mark.parametrize("name,T,d,f,chunk", CASES, ids=[c[0] for c in CASES])
def test_ffn_matches_oracle(gpu, name, T, d, f, chunk):
    x, w1, w3, w2, dout = _inputs(T, d, f, seed=T + d, dev=gpu)
    out = ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=chunk)
    dx, dw1, dw3, dw2 = ra.blockwise_ffn_bwd(x, w1, w3, w2, dout, chunk=chunk)
    torch.cuda.synchronize()
    a = [P.np64(t) for t in (x, w1, w3, w2, dout)]
    _close(f"{name} out", P.np64(out), oracle.ffn_forward(*a[:4]))
    for gname, g, r in zip(("dx", "dw1", "dw3", "dw2"), (dx, dw1, dw3, dw2), oracle.ffn_backward(*a)):
        _close(f"{name} {gname}", P.np64(g), r)


def test_ffn_chunking_changes_only_rounding(gpu):
    x, w1, w3, w2, dout = _inputs(2048, 256, 704, seed=5, dev=gpu)
    o1 = ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=2048)
    g1 = ra.blockwise_ffn_bwd(x, w1, w3, w2, dout, chunk=2048)
    for chunk in (7, 333, 1024):
        o = ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=chunk)
        g = ra.blockwise_ffn_bwd(x, w1, w3, w2, dout, chunk=chunk)
        torch.cuda.synchronize()
        _close(f"chunk {chunk} out", P.np64(o), P.np64(o1))
        for a, b in zip(g, g1):
            _close(f"chunk {chunk} grad", P.np64(a), P.np64(b))


def test_ffn_empty_and_errors(gpu):
    x, w1, w3, w2, dout = _inputs(0, 64, 96, seed=1, dev=gpu)
    assert ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=16).shape == (0, 64)
    # no token contributes: the weight gradients are cleared, whatever the buffers held
    dws = [torch.full(w.shape, 7.0, dtype=torch.float32, device=gpu) for w in (w1, w3, w2)]
    dx, dw1, dw3, dw2 = ra.blockwise_ffn_bwd(x, w1, w3, w2, dout, chunk=16, dw1=dws[0], dw3=dws[1], dw2=dws[2])
    torch.cuda.synchronize()
    assert dx.shape == (0, 64) and not dw1.any() and not dw3.any() and not dw2.any()
    x, w1, w3, w2, dout = _inputs(8, 64, 96, seed=2, dev=gpu)
    with pytest.raises(ra.RAError, match="chunk"):
        ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=0)
