"""Host-side checks of the Python binding (no GPU): it refuses CPU tensors and
bad layouts before calling into the library."""
import numpy as np
import pytest
import torch

import long_context_exact_attn_amd as ra


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ra.blockwise_attn_fwd(q, q, q, n_ring=1, q_chunk=64, k_chunk=64, causal=True)


def test_missing_library_raises(monkeypatch, tmp_path):
    from long_context_exact_attn_amd import api
    monkeypatch.setattr(api, "_LIB", None)
    monkeypatch.setenv("RA_ATTN_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(api.RAError):
        api.load_library()


def test_pair_accounting_matches_the_oracle_count():
    # bench.py's work accounting (product side) against the oracle's own count, causal block sizes
    # and segment ids included
    import oracle
    from long_context_exact_attn_amd import metrics as M
    L = 96
    rng = np.random.default_rng(3)
    seg = np.sort(rng.integers(-3, 4, size=(2, L)), axis=1)
    seg[1] = rng.permutation(seg[1])
    for causal in (False, True, 1, 7, 32, 200):
        for q_first, q_len in ((0, L), (32, 32)):
            qpos = np.arange(q_first, q_first + q_len)
            assert M.visible_pairs_per_head(q_first, q_len, L, causal) == oracle.visible_pairs(qpos, L, causal)
            assert (M.visible_pairs_per_head(q_first, q_len, L, causal, seg)
                    == oracle.visible_pairs(qpos, L, causal, segment_ids=seg))


# ------------------------------------------------------------------ buffer checks of the binding
# The C ABI receives raw pointers and cannot size them, so the binding checks every buffer's shape and
# dtype before the call; these run on the CPU (shape checks come before the device check) and would
# reach no kernel on a GPU either.
def _qkv(B=1, L=128, H=2, D=64, dt=torch.bfloat16):
    return (torch.zeros(B, L, H, D, dtype=dt), torch.zeros(B, L, H, D, dtype=dt), torch.zeros(B, L, H, D, dtype=dt))


KW = dict(n_ring=1, q_chunk=128, k_chunk=128, causal=True)


@pytest.mark.parametrize("name,bad", [
    ("out", dict(out=torch.zeros(1, 128, 2, 32, dtype=torch.bfloat16))),
    ("out", dict(out=torch.zeros(1, 128, 2, 64, dtype=torch.float32))),
    ("lse", dict(lse=torch.zeros(1, 2, 128, dtype=torch.bfloat16))),
    ("lse", dict(lse=torch.zeros(1, 128, 2, dtype=torch.float32))),
])
def test_forward_rejects_mismatched_outputs(name, bad):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match=name):
        ra.blockwise_attn_fwd(q, k, v, **KW, **bad)


def test_backward_rejects_mismatched_buffers():
    q, k, v = _qkv()
    out, dout = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(1, 2, 128, dtype=torch.float32)
    cases = [
        ("dout", dict(dout=torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16))),
        ("lse", dict(lse=torch.zeros(1, 2, 128, dtype=torch.bfloat16))),
        ("dq", dict(dq=torch.zeros(1, 128, 2, 64, dtype=torch.float32))),
        ("dk", dict(dk=torch.zeros(1, 256, 2, 64, dtype=torch.bfloat16))),
        ("dv", dict(dv=torch.zeros(1, 128, 1, 64, dtype=torch.bfloat16))),
        ("workspace", dict(workspace=torch.zeros(1024, dtype=torch.float32))),
    ]
    for name, bad in cases:
        args = dict(out=out, lse=lse, dout=dout)
        args.update({k_: v_ for k_, v_ in bad.items() if k_ in args})
        extra = {k_: v_ for k_, v_ in bad.items() if k_ not in args}
        with pytest.raises(ValueError, match=name):
            ra.blockwise_attn_bwd(q, k, v, args["out"], args["lse"], args["dout"], **KW, **extra)
    bias = torch.zeros(2, 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="dbias"):
        ra.blockwise_attn_bwd_dbias(q, k, v, out, lse, dout, bias, **KW, dbias=torch.zeros(2, 8, dtype=torch.float32))
    delta = torch.zeros(1, 2, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="delta"):
        ra.blockwise_attn_bwd_dkdv(q, k, v, lse, torch.zeros(1, 2, 64), dout, **KW)
    with pytest.raises(ValueError, match="dq"):
        ra.blockwise_attn_bwd_dq(q, k, v, lse, delta, dout, **KW, dq=torch.zeros(1, 128, 2, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="delta"):
        ra.blockwise_attn_bwd_preprocess(out, dout, delta=torch.zeros(1, 128, 2))


def test_ring_step_rejects_mismatched_state():
    q, k, v = _qkv()
    f32 = dict(dtype=torch.float32)
    good = (torch.zeros(1, 128, 2, 64, **f32), torch.zeros(1, 2, 128, **f32), torch.zeros(1, 2, 128, **f32))
    for i, bad in ((0, torch.zeros(1, 128, 2, 64, dtype=torch.bfloat16)), (1, torch.zeros(1, 2, 64, **f32)),
                   (2, torch.zeros(2, 2, 128, **f32))):
        state = list(good)
        state[i] = bad
        with pytest.raises(ValueError, match="^[oml] must be"):
            ra.blockwise_attn_fwd_step(q, k, v, q_pos0=0, kv_pos0=0, causal=True, state=tuple(state))
    lse = delta = torch.zeros(1, 2, 128, **f32)
    with pytest.raises(ValueError, match="dk_acc"):
        ra.blockwise_attn_bwd_step(q, k, v, lse, delta, q.clone(), q_pos0=0, kv_pos0=0, causal=True,
                                   dk_acc=torch.zeros(1, 64, 2, 64, **f32))
    with pytest.raises(ValueError, match="lse_b"):
        ra.attn_merge(q.clone(), lse.clone(), q.clone(), torch.zeros(1, 2, 127, **f32))
    with pytest.raises(ValueError, match="out"):
        ra.blockwise_attn_fwd_finalize(good, out=torch.zeros(1, 128, 2, 64, **f32))


def test_mixed_devices_are_rejected_on_cpu_tensors():
    # CPU tensors with correct shapes reach the device check, which refuses them
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        ra.blockwise_attn_fwd(q, k, v, **KW)
