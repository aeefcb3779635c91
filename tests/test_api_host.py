"""Host-side checks of the Python binding (no GPU): it refuses CPU tensors and
bad layouts before calling into the library."""
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
