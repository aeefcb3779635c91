"""Seeded synthetic inputs for blockwise ring attention.

This module holds no attention arithmetic: it only draws random tensors of
the shapes, dtypes and value distributions of the workloads, rounds them
once to the working dtype, and builds packed-document segment ids.  Both the
GPU path and the CPU oracle read the tensors it returns.

Layout is [batch, sequence, heads, head_dim] for q/k/v/dout, [heads,
bias_len] float32 for the additive bias and [batch, kv_len] int32 for the
segment ids (global key positions).

Workloads (sizes as the pages' long-context setting suggests: 1M tokens over
8 devices is 128K per device, "手把手拆解RingAttention" section 2; ring block
4096 from the tuning table in section 5; chunks of 512 and d_model 1024 /
16 heads from "RingAttention核心功能全解析" and "Ring Attention技术解析"):
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    kv_len: int
    n_ring: int
    ring_rank: int = -1          # -1: queries are the whole sequence; r: queries are ring block r
    q_chunk: int = 512
    k_chunk: int = 512
    dtype: str = "bf16"          # "bf16" or "f32"
    causal: bool = True
    std: float = 0.5             # q, k, v ~ N(0, 1) * std
    bias_len: int = 0            # 0: no bias; else bias ~ N(0,1) of shape [heads, bias_len]
    segments: str = "none"       # "none", "zeros" (all ids 0), "docs" (packed documents) or
                                 # "scattered" (unsorted runs of a few ids, extremes included)
    doc_len: tuple = (512, 16384)
    backward: bool = False       # also draw dout ~ N(0, 1)
    seed: int = 0

    @property
    def block_len(self):
        return self.kv_len // self.n_ring

    @property
    def q_len(self):
        return self.kv_len if self.ring_rank < 0 else self.block_len

    def q_positions(self):
        first = 0 if self.ring_rank < 0 else self.ring_rank * self.block_len
        return np.arange(first, first + self.q_len, dtype=np.int64)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-f32-1k", batch=1, heads=1, head_dim=64, kv_len=1024, n_ring=4, q_chunk=128,
                 k_chunk=128, dtype="f32", causal=False, std=1.0, segments="zeros", seed=1000),
        Workload("causal-32k", batch=1, heads=16, head_dim=64, kv_len=32768, n_ring=8, seed=1001),
        Workload("share-1m-r7", batch=1, heads=16, head_dim=64, kv_len=1048576, n_ring=8, ring_rank=7,
                 seed=1002),
        Workload("packed-docs-64k", batch=2, heads=32, head_dim=128, kv_len=65536, n_ring=16,
                 bias_len=4096, segments="docs", seed=1003),
        Workload("train-32k", batch=1, heads=16, head_dim=64, kv_len=32768, n_ring=8, backward=True,
                 seed=1004),
    ]
}


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def doc_segment_ids(batch, kv_len, lo, hi, seed):
    """Packed documents: lengths ~ U{lo..hi} drawn in order per batch row, the
    last one cut to fit; ids 0, 1, 2, ... in order.  int32 [batch, kv_len]."""
    rng = np.random.default_rng(seed)
    ids = np.empty((batch, kv_len), dtype=np.int32)
    for b in range(batch):
        pos, doc = 0, 0
        while pos < kv_len:
            n = int(rng.integers(lo, hi, endpoint=True))
            ids[b, pos:pos + n] = doc
            pos += n
            doc += 1
    return ids


def scattered_segment_ids(batch, kv_len, seed, max_run=200):
    """Unsorted ids: runs of 1..max_run positions, each run's id drawn from a small set that
    includes the int32 extremes.  int32 [batch, kv_len]."""
    rng = np.random.default_rng(seed)
    alphabet = np.array([-2**31, -5, 3, 7, 2**31 - 1], dtype=np.int64)
    ids = np.empty((batch, kv_len), dtype=np.int32)
    for b in range(batch):
        pos = 0
        while pos < kv_len:
            n = int(rng.integers(1, max_run, endpoint=True))
            ids[b, pos:pos + n] = alphabet[rng.integers(len(alphabet))]
            pos += n
    return ids


def _normal(shape, gen, device, std, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make(w: Workload, device="cpu", seed: Optional[int] = None):
    """Draw the inputs of workload ``w`` on ``device``; returns a dict of tensors.

    Keys: q, k, v (working dtype), bias (float32 or None), segment_ids (int32
    or None), dout (working dtype, when w.backward).  Values are drawn in
    float32 with a generator seeded from ``seed`` (default ``w.seed``) and
    rounded once to the working dtype.
    """
    seed = w.seed if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = torch_dtype(w.dtype)
    B, H, D = w.batch, w.heads, w.head_dim
    t = {
        "q": _normal((B, w.q_len, H, D), gen, dev, w.std, dt),
        "k": _normal((B, w.kv_len, H, D), gen, dev, w.std, dt),
        "v": _normal((B, w.kv_len, H, D), gen, dev, w.std, dt),
        "bias": None,
        "segment_ids": None,
        "dout": None,
    }
    if w.bias_len:
        t["bias"] = _normal((H, w.bias_len), gen, dev, 1.0, torch.float32)
    if w.segments == "zeros":
        t["segment_ids"] = torch.zeros((B, w.kv_len), dtype=torch.int32, device=dev)
    elif w.segments == "docs":
        t["segment_ids"] = torch.from_numpy(doc_segment_ids(B, w.kv_len, *w.doc_len, seed)).to(dev)
    elif w.segments == "scattered":
        t["segment_ids"] = torch.from_numpy(scattered_segment_ids(B, w.kv_len, seed)).to(dev)
    if w.backward:
        t["dout"] = _normal((B, w.q_len, H, D), gen, dev, 1.0, dt)
    return t


def small(name="small", *, batch=1, heads=2, head_dim=64, kv_len=512, n_ring=2, ring_rank=-1,
          dtype="bf16", causal=True, bias_len=0, segments="none", doc_len=(16, 96), std=0.5,
          backward=False, q_chunk=None, k_chunk=None, seed=7):
    """A small workload for parity tests (sizes the oracle finishes in seconds)."""
    lb = kv_len // n_ring
    return Workload(name, batch=batch, heads=heads, head_dim=head_dim, kv_len=kv_len, n_ring=n_ring,
                    ring_rank=ring_rank, q_chunk=q_chunk or lb, k_chunk=k_chunk or lb, dtype=dtype,
                    causal=causal, std=std, bias_len=bias_len, segments=segments, doc_len=doc_len,
                    backward=backward, seed=seed)


__all__ = ["Workload", "WORKLOADS", "make", "small", "doc_segment_ids", "scattered_segment_ids", "torch_dtype", "replace", "field"]
