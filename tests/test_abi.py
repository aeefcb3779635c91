"""The C-ABI library on the host (no GPU): it loads, exports every symbol the
header declares, and rejects bad arguments before anything is launched.

Every rejected call below also leaves at least one required output pointer
NULL, so that a validation bug could never reach a kernel launch with the
fake (non-dereferenceable) input pointers these tests use.  The call-based
tests are skipped where a GPU is visible; they belong to the CPU suite.
"""
import ctypes
import os
import re

import pytest

from long_context_exact_attn_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra_attn.h")

FAKE = ctypes.c_void_p(0x7f0000010000)   # aligned, never dereferenced: every call below fails validation


def _lib():
    try:
        return api.load_library()
    except api.RAError as e:
        pytest.fail(f"library not built: {e}")


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert "ra_blockwise_attn_fwd" in names and "ra_blockwise_attn_bwd" in names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ra_abi_version() == 2


def test_shape_struct_layout():
    assert ctypes.sizeof(api.Shape) == 48
    assert api.Shape.q_len.offset == 16 and api.Shape.scale.offset == 40 and api.Shape.dtype.offset == 44


def test_workspace_size():
    lib = _lib()
    s = api.Shape(2, 3, 64, -1, 1000, 1000, 0, 0.0, api.RA_BF16)
    for n_ring in (1, 4, 1000):
        assert lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(s), n_ring) == (2 * 3 * 1000 * 4 + 255) // 256 * 256
    assert lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(s), 0) == 0
    assert lib.ra_blockwise_attn_bwd_workspace_size(None, 1) == 0
    s = api.Shape(0, 3, 64, -1, 0, 0, 0, 0.0, api.RA_BF16)
    assert lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(s), 1) == 0


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


needs_cpu = pytest.mark.skipif(_gpu_visible(), reason="validation calls with fake pointers run on the CPU suite only")


def _fwd(lib, shape, n_ring=4, q_chunk=64, k_chunk=64, causal=1, out=None, lse=None, bias=None, seg=None,
         q=FAKE, k=FAKE, v=FAKE):
    return lib.ra_blockwise_attn_fwd(q, k, v, bias, seg, n_ring, q_chunk, k_chunk, causal, out, lse,
                                     ctypes.byref(shape) if shape is not None else None, None)


@needs_cpu
@pytest.mark.parametrize("case,expect", [
    ("ring_not_closed", -2), ("rank_out_of_range", -1), ("q_len_vs_rank", -2), ("all_ranks_q_len", -2),
    ("head_dim", -3), ("dtype", -3), ("negative", -2), ("causal", -1), ("causal_negative", -1), ("chunk_zero", -1),
    ("chunk_not_dividing", -1), ("n_ring_zero", -1), ("bias_len", -1), ("null_out", -1), ("null_lse", -1),
    ("null_q", -1), ("misaligned_k", -1), ("null_shape", -1),
])
def test_forward_validation(case, expect):
    lib = _lib()
    S = lambda **kw: api.Shape(**{**dict(batch=1, heads=2, head_dim=64, ring_rank=-1, q_len=1024, kv_len=1024,  # noqa
                                         bias_len=0, scale=0.0, dtype=api.RA_BF16), **kw})
    kw = {}
    shape = S()
    if case == "ring_not_closed":
        kw["n_ring"] = 3
    elif case == "rank_out_of_range":
        shape = S(ring_rank=4, q_len=256)
    elif case == "q_len_vs_rank":
        shape = S(ring_rank=1, q_len=1024)
    elif case == "all_ranks_q_len":
        shape = S(q_len=512)
    elif case == "head_dim":
        shape = S(head_dim=96)
    elif case == "dtype":
        shape = S(dtype=7)
    elif case == "negative":
        shape = S(batch=-1)
    elif case == "causal":
        kw["causal"] = 3   # a causal block size that does not divide the ring block of 256
    elif case == "causal_negative":
        kw["causal"] = -1
    elif case == "chunk_zero":
        kw["q_chunk"] = 0
    elif case == "chunk_not_dividing":
        kw["k_chunk"] = 100
    elif case == "n_ring_zero":
        kw["n_ring"] = 0
    elif case == "bias_len":
        kw["bias"] = FAKE
    elif case == "null_lse":
        kw["out"] = FAKE
    elif case == "null_q":
        kw["q"] = None
    elif case == "misaligned_k":
        kw["k"] = ctypes.c_void_p(0x7f0000010008)
    elif case == "null_shape":
        shape = None
    rc = _fwd(lib, shape, **kw)
    assert rc == expect, (case, rc, lib.ra_last_error())
    assert lib.ra_last_error()


@needs_cpu
def test_backward_validation():
    lib = _lib()
    s = api.Shape(1, 2, 64, -1, 1024, 1024, 0, 0.0, api.RA_BF16)
    # workspace missing: every tensor pointer is given, dv is NULL so the call cannot launch regardless
    rc = lib.ra_blockwise_attn_bwd(FAKE, FAKE, FAKE, None, None, 4, 256, 256, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None, None, 0, ctypes.byref(s), None)
    assert rc == -1 and "dv" in lib.ra_last_error().decode()
    rc = lib.ra_blockwise_attn_bwd_dkdv(FAKE, FAKE, FAKE, None, None, 5, 256, 256, 1, FAKE, FAKE, FAKE, FAKE, None,
                                        ctypes.byref(s), None)
    assert rc == -2
    rc = lib.ra_blockwise_attn_bwd_dq(FAKE, FAKE, FAKE, None, None, 4, 256, 256, 1, FAKE, None, FAKE, FAKE,
                                      ctypes.byref(s), None)
    assert rc == -1 and "delta" in lib.ra_last_error().decode()
    s2 = api.Shape(1, 2, 48, -1, 1024, 1024, 0, 0.0, api.RA_BF16)
    rc = lib.ra_blockwise_attn_bwd_preprocess(FAKE, FAKE, None, ctypes.byref(s2), None)
    assert rc == -3


@needs_cpu
def test_empty_problem_is_a_no_op():
    lib = _lib()
    s = api.Shape(0, 2, 64, -1, 1024, 1024, 0, 0.0, api.RA_BF16)   # batch 0: nothing to do, NULLs allowed
    assert _fwd(lib, s, q=None, k=None, v=None) == 0
    assert lib.ra_last_error() == b""


@needs_cpu
def test_ring_step_validation():
    lib = _lib()
    S = lambda **kw: api.Shape(**{**dict(batch=1, heads=2, head_dim=64, ring_rank=-1, q_len=512, kv_len=512,  # noqa
                                         bias_len=0, scale=0.0, dtype=api.RA_BF16), **kw})

    def step(shape, seg=None, seg_len=0, q_pos0=512, kv_pos0=0, init=1, o=None, m=FAKE, l_=FAKE, causal=1):
        return lib.ra_blockwise_attn_fwd_step(FAKE, FAKE, FAKE, None, seg, seg_len, q_pos0, kv_pos0, causal, o, m,
                                              l_, init, ctypes.byref(shape), None)

    # o_state stays NULL in every call: none can reach a launch
    assert step(S(kv_len=256)) == -2 and b"equal query and key" in lib.ra_last_error()
    assert step(S(dtype=api.RA_F32)) == -3
    assert step(S(head_dim=80)) == -3
    assert step(S(), q_pos0=-1) == -1
    assert step(S(), init=2) == -1
    assert step(S(), causal=3) == -1
    assert step(S(), seg=FAKE, seg_len=1000) == -2 and b"do not cover" in lib.ra_last_error()
    assert step(S()) == -1 and b"o_state" in lib.ra_last_error()
    assert step(S(batch=0), m=None, l_=None) == 0   # nothing to do

    s = S()
    rc = lib.ra_blockwise_attn_fwd_finalize(FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(s), None)
    assert rc == -1 and b"lse" in lib.ra_last_error()
    rc = lib.ra_blockwise_attn_fwd_finalize(FAKE, FAKE, FAKE, None, FAKE, ctypes.byref(S(head_dim=32)), None)
    assert rc == -3
    rc = lib.ra_attn_merge(FAKE, FAKE, FAKE, None, ctypes.byref(s), None)
    assert rc == -1 and b"lse_b" in lib.ra_last_error()
    rc = lib.ra_attn_merge(None, FAKE, FAKE, FAKE, ctypes.byref(S(batch=-2)), None)
    assert rc == -2


@needs_cpu
def test_positions_must_fit_32_bits():
    lib = _lib()
    s = api.Shape(1, 2, 64, -1, 1 << 30, 1 << 30, 0, 0.0, api.RA_BF16)
    assert _fwd(lib, s, n_ring=1, q_chunk=1 << 30, k_chunk=1 << 30) == -2
    assert b"2^30" in lib.ra_last_error()
    s = api.Shape(1, 2, 64, -1, 512, 512, 0, 0.0, api.RA_BF16)
    rc = lib.ra_blockwise_attn_fwd_step(FAKE, FAKE, FAKE, None, None, 0, (1 << 30) - 100, 0, 1, None, FAKE, FAKE, 1,
                                        ctypes.byref(s), None)
    assert rc == -2 and b"2^30" in lib.ra_last_error()
    s = api.Shape(1, 2, 64, -1, 512, 512, 1 << 30, 0.0, api.RA_BF16)
    assert _fwd(lib, s, n_ring=1, q_chunk=512, k_chunk=512, bias=FAKE) == -1


@needs_cpu
def test_bwd_step_validation():
    lib = _lib()
    S = lambda **kw: api.Shape(**{**dict(batch=1, heads=2, head_dim=64, ring_rank=-1, q_len=512, kv_len=512,  # noqa
                                         bias_len=0, scale=0.0, dtype=api.RA_BF16), **kw})

    def step(shape, seg=None, seg_len=0, q_pos0=512, kv_pos0=0, i_dq=1, i_dkv=1, dv=None, delta=FAKE, dbias=None,
             bias=None):
        return lib.ra_blockwise_attn_bwd_step(FAKE, FAKE, FAKE, bias, seg, seg_len, q_pos0, kv_pos0, 1, FAKE, delta,
                                              FAKE, FAKE, FAKE, dv, dbias, i_dq, i_dkv, ctypes.byref(shape), None)

    # dv_acc stays NULL in every call: none can reach a launch
    assert step(S(kv_len=256)) == -2 and b"equal query and key" in lib.ra_last_error()
    assert step(S(dtype=api.RA_F32)) == -3
    assert step(S(), kv_pos0=-1) == -1
    assert step(S(), q_pos0=(1 << 30) - 10) == -2
    assert step(S(), i_dkv=3) == -1
    assert step(S(), seg=FAKE, seg_len=600) == -2 and b"do not cover" in lib.ra_last_error()
    assert step(S(), delta=None) == -1 and b"delta" in lib.ra_last_error()
    assert step(S()) == -1 and b"dv_acc" in lib.ra_last_error()
    assert step(S(batch=0)) == 0
    # per-key dS sums for the bias gradient need a bias
    assert step(S(), dv=FAKE, dbias=FAKE) == -1 and b"dbias_acc needs a bias" in lib.ra_last_error()

    # the block's share of dbias: argument checks (dbias stays NULL: nothing is launched)
    def red(shape, kv_pos0=0, acc=1, dbias=None):
        return lib.ra_blockwise_attn_bwd_dbias_reduce(FAKE, kv_pos0, dbias, acc, ctypes.byref(shape), None)
    assert red(S(bias_len=0)) == -1 and b"bias_len" in lib.ra_last_error()
    assert red(S(bias_len=7), kv_pos0=-1) == -1
    assert red(S(bias_len=7), acc=2) == -1
    assert red(S(bias_len=7)) == -1 and b"dbias" in lib.ra_last_error()

    s = S()
    rc = lib.ra_blockwise_attn_bwd_finalize(FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(s), None)
    assert rc == -1 and b"dv" in lib.ra_last_error()
    rc = lib.ra_blockwise_attn_bwd_finalize(FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(S(head_dim=72)), None)
    assert rc == -3


@needs_cpu
def test_dbias_validation():
    lib = _lib()
    s = api.Shape(1, 2, 64, -1, 1024, 1024, 100, 0.0, api.RA_BF16)
    need = lib.ra_blockwise_attn_bwd_dbias_workspace_size(ctypes.byref(s))
    assert need == lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(s), 1) + 1 * 2 * 1024 * 4

    def call(shape, bias=FAKE, dbias=FAKE, ws=None, ws_bytes=0, dv=None):
        return lib.ra_blockwise_attn_bwd_dbias(FAKE, FAKE, FAKE, bias, None, 4, 256, 256, 1, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, dv, dbias, ws, ws_bytes, ctypes.byref(shape), None)

    # dv stays NULL in every call: none can reach a launch
    assert call(s, dbias=None) == -1 and b"dbias" in lib.ra_last_error()
    assert call(s, bias=None) == -1
    assert call(api.Shape(1, 2, 64, -1, 1024, 1024, 100, 0.0, api.RA_F32), dv=None) == -1   # dv checked first
    assert call(s, dv=FAKE) == -4 and b"workspace" in lib.ra_last_error()
    assert call(s, dv=FAKE, ws=FAKE, ws_bytes=need - 4) == -4
    # float32 is supported: with dv NULL the float32 call is refused for dv, not for its dtype
    f32 = api.Shape(1, 2, 64, -1, 1024, 1024, 100, 0.0, api.RA_F32)
    assert call(f32, ws=FAKE, ws_bytes=need) == -1 and b"dv" in lib.ra_last_error()


@needs_cpu
def test_ffn_validation():
    lib = _lib()
    # the forward holds the chunk's activation h (bfloat16); the backward also dh and the gradients of g, u
    assert lib.ra_blockwise_ffn_workspace_size(1000, 256, 704, 512, 0) >= 512 * 704 * 2
    assert lib.ra_blockwise_ffn_workspace_size(1000, 256, 704, 512, 1) >= 512 * 704 * (2 + 2 + 4)
    assert lib.ra_blockwise_ffn_workspace_size(1000, 256, 704, 512, 1) > lib.ra_blockwise_ffn_workspace_size(
        1000, 256, 704, 512, 0)

    def fwd(T=64, d=64, f=96, chunk=16, out=None, ws=None, ws_bytes=0):
        return lib.ra_blockwise_ffn_fwd(FAKE, FAKE, FAKE, FAKE, out, T, d, f, chunk, ws, ws_bytes, None)

    assert fwd(d=66) == -2
    assert fwd(d=68) == -2 and b"multiples of 8" in lib.ra_last_error()
    assert fwd(f=0) == -2
    assert fwd(chunk=0) == -1
    assert fwd(T=-1) == -2
    assert fwd() == -1 and b"out" in lib.ra_last_error()
    assert fwd(out=FAKE) == -4 and b"workspace" in lib.ra_last_error()
    assert fwd(T=0) == 0   # nothing to do, nothing launched
    rc = lib.ra_blockwise_ffn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 64, 96, 16, None, 0, None)
    assert rc == -1 and b"dw2" in lib.ra_last_error()


def test_noalloc_rejects_sizes_over_its_scratch_on_the_host():
    # the allocation-free backward refuses a problem whose Delta exceeds its static scratch before it
    # touches a device (all pointers NULL: nothing could be launched)
    if _gpu_visible():
        pytest.skip("host-only check")
    lib = _lib()
    assert lib.ra_blockwise_attn_bwd_noalloc_max_workspace() == 16 << 20
    s = api.Shape(1, 65, 64, -1, 65536, 65536, 0, 0.0, api.RA_BF16)
    rc = lib.ra_blockwise_attn_bwd_noalloc(*([None] * 5), 1, 1, 1, 1, *([None] * 6), ctypes.byref(s), None)
    assert rc == api.RA_ERR_WORKSPACE if hasattr(api, "RA_ERR_WORKSPACE") else rc == -4
    assert b"4,194,304" in lib.ra_noalloc_last_error()
    assert lib.ra_blockwise_attn_bwd_noalloc(*([None] * 5), 1, 1, 1, 1, *([None] * 6), None, None) == -1
