"""Host-side checks of the seeded input generators (no GPU)."""
import numpy as np
import torch

from long_context_exact_attn_amd import workloads as W


def test_doc_segments_recipe():
    ids = W.doc_segment_ids(2, 65536, 512, 16384, seed=1003)
    assert ids.shape == (2, 65536) and ids.dtype == np.int32
    for row in ids:
        assert row[0] == 0 and np.all(np.diff(row) >= 0) and np.all(np.diff(row) <= 1)
        lengths = np.bincount(row)
        assert np.all(lengths[:-1] >= 512) and np.all(lengths[:-1] <= 16384)   # last document is cut to fit
        assert 1 <= lengths[-1] <= 16384


def test_make_is_seeded_and_rounded():
    w = W.small(kv_len=256, n_ring=4, ring_rank=1, bias_len=32, segments="docs", backward=True)
    a, b = W.make(w), W.make(w)
    for key in ("q", "k", "v", "bias", "segment_ids", "dout"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].shape == (1, 64, 2, 64) and a["k"].shape == (1, 256, 2, 64)
    assert a["q"].dtype == torch.bfloat16 and a["bias"].dtype == torch.float32
    assert a["segment_ids"].dtype == torch.int32
    c = W.make(w, seed=w.seed + 1)
    assert not torch.equal(a["q"], c["q"])
    assert abs(float(a["k"].float().std()) - 0.5) < 0.05


def test_named_workloads_shapes():
    w = W.WORKLOADS["share-1m-r7"]
    assert (w.q_len, w.kv_len, w.block_len) == (131072, 1048576, 131072)
    assert w.q_positions()[0] == 7 * 131072
    w = W.WORKLOADS["packed-docs-64k"]
    assert (w.batch, w.heads, w.head_dim, w.block_len, w.bias_len) == (2, 32, 128, 4096, 4096)
    t = W.make(W.WORKLOADS["tiny-f32-1k"])
    assert t["q"].dtype == torch.float32 and torch.all(t["segment_ids"] == 0)


def test_scattered_segments_recipe():
    ids = W.scattered_segment_ids(2, 5000, seed=3)
    assert ids.dtype == np.int32 and ids.shape == (2, 5000)
    assert np.array_equal(ids, W.scattered_segment_ids(2, 5000, seed=3))
    vals = set(np.unique(ids).tolist())
    assert vals <= {-2**31, -5, 3, 7, 2**31 - 1} and {-2**31, 2**31 - 1} <= vals
    # unsorted: ids go down as well as up along the sequence
    d = np.diff(ids[0].astype(np.int64))
    assert (d > 0).any() and (d < 0).any()
