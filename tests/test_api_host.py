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
