"""ctypes binding of libra_attn.so -- argument marshalling only.

Each function checks the torch tensors it is given (device, dtype, shape,
contiguity), allocates outputs the caller did not supply, and passes raw
device pointers and the current HIP stream to the C entry point of the same
name (include/ra_attn.h).  All arithmetic happens in the HIP kernels; there
is no CPU path, and a missing library raises RAError.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

RA_F32, RA_BF16 = 0, 1
_DTYPES = {torch.float32: RA_F32, torch.bfloat16: RA_BF16}


class RAError(RuntimeError):
    """A libra_attn call failed; the message carries the library's description."""

    def __init__(self, code, message):
        super().__init__(f"libra_attn error {code}: {message}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ring_rank", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("bias_len", ctypes.c_int64), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


def library_path():
    return os.environ.get("RA_ATTN_LIB", os.path.join(_HERE, "libra_attn.so"))


def load_library():
    """Load libra_attn.so once; raise RAError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RAError(-100, f"{path} is missing: build it with long_context_exact_attn_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH = ctypes.POINTER(Shape)
    sig = {
        "ra_blockwise_attn_fwd": [P, P, P, P, P, I32, I64, I64, I32, P, P, SH, P],
        "ra_blockwise_attn_bwd": [P, P, P, P, P, I32, I64, I64, I32, P, P, P, P, P, P, P, SZ, SH, P],
        "ra_blockwise_attn_bwd_preprocess": [P, P, P, SH, P],
        "ra_blockwise_attn_bwd_dkdv": [P, P, P, P, P, I32, I64, I64, I32, P, P, P, P, P, SH, P],
        "ra_blockwise_attn_bwd_dq": [P, P, P, P, P, I32, I64, I64, I32, P, P, P, P, SH, P],
        "ra_blockwise_attn_fwd_step": [P, P, P, P, P, I64, I64, I64, I32, P, P, P, I32, SH, P],
        "ra_blockwise_attn_fwd_finalize": [P, P, P, P, P, SH, P],
        "ra_attn_merge": [P, P, P, P, SH, P],
        "ra_blockwise_attn_bwd_step": [P, P, P, P, P, I64, I64, I64, I32, P, P, P, P, P, P, P, I32, I32, SH, P],
        "ra_blockwise_attn_bwd_dbias_reduce": [P, I64, P, I32, SH, P],
        "ra_blockwise_attn_bwd_finalize": [P, P, P, P, P, P, SH, P],
        "ra_blockwise_attn_bwd_dbias": [P, P, P, P, P, I32, I64, I64, I32, P, P, P, P, P, P, P, P, SZ, SH, P],
        "ra_blockwise_ffn_fwd": [P, P, P, P, P, I64, I32, I32, I64, P, SZ, P],
        "ra_blockwise_attn_bwd_noalloc": [P, P, P, P, P, I32, I64, I64, I32, P, P, P, P, P, P, SH, P],
        "ra_blockwise_ffn_bwd": [P, P, P, P, P, P, P, P, P, I64, I32, I32, I64, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ra_blockwise_attn_bwd_workspace_size.argtypes = [SH, I32]
    lib.ra_blockwise_attn_bwd_workspace_size.restype = SZ
    lib.ra_blockwise_attn_bwd_dbias_workspace_size.argtypes = [SH]
    lib.ra_blockwise_attn_bwd_dbias_workspace_size.restype = SZ
    lib.ra_blockwise_ffn_workspace_size.argtypes = [I64, I32, I32, I64, I32]
    lib.ra_blockwise_ffn_workspace_size.restype = SZ
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_noalloc_last_error.argtypes = []
    lib.ra_noalloc_last_error.restype = ctypes.c_char_p
    lib.ra_blockwise_attn_bwd_noalloc_max_workspace.argtypes = []
    lib.ra_blockwise_attn_bwd_noalloc_max_workspace.restype = SZ
    lib.ra_abi_version.argtypes = []
    lib.ra_abi_version.restype = ctypes.c_int32
    if lib.ra_abi_version() != 2:
        raise RAError(-101, "unexpected libra_attn ABI version")
    _LIB = lib
    return lib


def _causal(causal):
    """The C ABI's causal argument: 0 (False / None), 1 (True) or a causal block size c >= 1."""
    if causal is None or causal is False:
        return 0
    if causal is True:
        return 1
    return int(causal)


def _check(rc):
    if rc != 0:
        raise RAError(rc, _LIB.ra_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def make_shape(q, k, *, ring_rank=-1, scale=None, bias=None):
    B, Lq, H, D = q.shape
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return Shape(B, H, D, ring_rank, Lq, k.shape[1], 0 if bias is None else bias.shape[-1],
                 0.0 if scale is None else float(scale), _DTYPES[q.dtype])


def _expect(name, t, shape, dtype):
    """t must have exactly this shape and dtype (checked before anything reaches the library, which
    receives raw pointers and cannot size them)."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)} (got {t.dtype} {tuple(t.shape)})")


def _devices(*named):
    """Every given tensor is a contiguous GPU tensor on the first one's device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, not on {dev} with the other tensors")


def _rows(q):
    """[B, H, Lq] of float32 per-row statistics (lse, delta, m, l) for q [B, Lq, H, D]."""
    return (q.shape[0], q.shape[2], q.shape[1])


def _tensors(q, k, v, bias, segment_ids, extra=(), devices=True):
    """Shapes and dtypes of q, k, v, bias and segment_ids of an attention call; with devices, also
    that they and the named extra tensors (whose shapes and dtypes the caller checks with _expect)
    are contiguous GPU tensors on one device."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"q and k must be [batch, seq, heads, head_dim] (got {tuple(q.shape)}, {tuple(k.shape)})")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype or v.shape != k.shape:
        raise ValueError("k and v must match each other and q's dtype")
    if k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    if bias is not None and (bias.dtype != torch.float32 or bias.dim() != 2 or bias.shape[0] != q.shape[2]):
        raise ValueError("bias must be a float32 tensor of shape [heads, bias_len]")
    if segment_ids is not None and (segment_ids.dtype != torch.int32 or tuple(segment_ids.shape) !=
                                    (k.shape[0], k.shape[1])):
        raise ValueError("segment_ids must be an int32 tensor of shape [batch, kv_len]")
    if devices:
        _devices(("q", q), ("k", k), ("v", v), ("bias", bias), ("segment_ids", segment_ids), *extra)


def _step_segments(segment_ids, q):
    if segment_ids is not None and (segment_ids.dtype != torch.int32 or segment_ids.dim() != 2
                                    or segment_ids.shape[0] != q.shape[0]):
        raise ValueError("segment_ids must be an int32 tensor of shape [batch, seq_len]")


def _workspace(name, t):
    if t is not None and t.dtype != torch.uint8:
        raise ValueError(f"{name} must be a uint8 (byte) tensor")
    return t


def blockwise_attn_fwd(q, k, v, bias=None, segment_ids=None, *, n_ring, q_chunk, k_chunk, causal,
                       ring_rank=-1, scale=None, out=None, lse=None):
    """out, lse = ra_blockwise_attn_fwd(...) on the current stream of q's device."""
    lib = load_library()
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(_rows(q), dtype=torch.float32, device=q.device)
    _expect("out", out, q.shape, q.dtype)
    _expect("lse", lse, _rows(q), torch.float32)
    _tensors(q, k, v, bias, segment_ids, extra=(("out", out), ("lse", lse)))
    _check(lib.ra_blockwise_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                     int(q_chunk), int(k_chunk), _causal(causal), _ptr(out), _ptr(lse),
                                     ctypes.byref(shape), _stream(q.device)))
    return out, lse


def bwd_workspace_size(q, k, *, n_ring=1, ring_rank=-1):
    lib = load_library()
    shape = make_shape(q, k, ring_rank=ring_rank)
    return int(lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(shape), int(n_ring)))


def _check_grads(q, k, out, lse, dout, dq, dk, dv):
    _expect("out", out, q.shape, q.dtype)
    _expect("dout", dout, q.shape, q.dtype)
    _expect("lse", lse, _rows(q), torch.float32)
    _expect("dq", dq, q.shape, q.dtype)
    _expect("dk", dk, k.shape, k.dtype)
    _expect("dv", dv, k.shape, k.dtype)


def blockwise_attn_bwd(q, k, v, out, lse, dout, bias=None, segment_ids=None, *, n_ring, q_chunk, k_chunk,
                       causal, ring_rank=-1, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """dq, dk, dv = ra_blockwise_attn_bwd(...) on the current stream of q's device."""
    lib = load_library()
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_grads(q, k, out, lse, dout, dq, dk, dv)
    need = int(lib.ra_blockwise_attn_bwd_workspace_size(ctypes.byref(shape), int(n_ring)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace("workspace", workspace)
    _tensors(q, k, v, bias, segment_ids, extra=(("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                                                ("dv", dv), ("workspace", workspace)))
    _check(lib.ra_blockwise_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                     int(q_chunk), int(k_chunk), _causal(causal), _ptr(out), _ptr(lse),
                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), ctypes.byref(shape),
                                     _stream(q.device)))
    return dq, dk, dv


def blockwise_attn_bwd_noalloc(q, k, v, out, lse, dout, bias=None, segment_ids=None, *, n_ring, q_chunk, k_chunk,
                               causal, ring_rank=-1, scale=None, dq=None, dk=None, dv=None):
    """dq, dk, dv = ra_blockwise_attn_bwd_noalloc(...): the backward with Delta in the library's static
    device scratch (no workspace).  Outputs the caller does not pass are allocated here, by torch; pass
    dq, dk and dv to allocate nothing."""
    lib = load_library()
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_grads(q, k, out, lse, dout, dq, dk, dv)
    _tensors(q, k, v, bias, segment_ids, extra=(("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                                                ("dv", dv)))
    rc = lib.ra_blockwise_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                           int(q_chunk), int(k_chunk), _causal(causal), _ptr(out), _ptr(lse),
                                           _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.byref(shape),
                                           _stream(q.device))
    if rc != 0:
        own = lib.ra_noalloc_last_error().decode()
        raise RAError(rc, own or lib.ra_last_error().decode())
    return dq, dk, dv


def blockwise_attn_bwd_dbias(q, k, v, out, lse, dout, bias, segment_ids=None, *, n_ring, q_chunk, k_chunk, causal,
                             ring_rank=-1, scale=None, dq=None, dk=None, dv=None, dbias=None, workspace=None):
    """dq, dk, dv, dbias = ra_blockwise_attn_bwd_dbias(...): the backward plus the bias gradient
    (float32 [heads, bias_len])."""
    lib = load_library()
    if bias is None:
        raise ValueError("the bias gradient needs a bias")
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dbias = torch.empty_like(bias) if dbias is None else dbias
    _check_grads(q, k, out, lse, dout, dq, dk, dv)
    _expect("dbias", dbias, bias.shape, torch.float32)
    need = int(lib.ra_blockwise_attn_bwd_dbias_workspace_size(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace("workspace", workspace)
    _tensors(q, k, v, bias, segment_ids, extra=(("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                                                ("dv", dv), ("dbias", dbias), ("workspace", workspace)))
    _check(lib.ra_blockwise_attn_bwd_dbias(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                           int(q_chunk), int(k_chunk), _causal(causal), _ptr(out), _ptr(lse),
                                           _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), ctypes.byref(shape),
                                           _stream(q.device)))
    return dq, dk, dv, dbias


def blockwise_attn_bwd_preprocess(out, dout, *, delta=None):
    """delta = ra_blockwise_attn_bwd_preprocess(out, dout): float32 [B, H, Lq]."""
    lib = load_library()
    _tensors(out, out, out, None, None, devices=False)
    _expect("dout", dout, out.shape, out.dtype)
    B, Lq, H, D = out.shape
    shape = Shape(B, H, D, -1, Lq, Lq, 0, 0.0, _DTYPES[out.dtype])
    if delta is None:
        delta = torch.empty((B, H, Lq), dtype=torch.float32, device=out.device)
    _expect("delta", delta, (B, H, Lq), torch.float32)
    _devices(("out", out), ("dout", dout), ("delta", delta))
    _check(lib.ra_blockwise_attn_bwd_preprocess(_ptr(out), _ptr(dout), _ptr(delta), ctypes.byref(shape),
                                                _stream(out.device)))
    return delta


def _check_rowstats(q, lse, delta, dout):
    _expect("lse", lse, _rows(q), torch.float32)
    _expect("delta", delta, _rows(q), torch.float32)
    _expect("dout", dout, q.shape, q.dtype)


def blockwise_attn_bwd_dkdv(q, k, v, lse, delta, dout, bias=None, segment_ids=None, *, n_ring, q_chunk,
                            k_chunk, causal, ring_rank=-1, scale=None, dk=None, dv=None):
    lib = load_library()
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_rowstats(q, lse, delta, dout)
    _expect("dk", dk, k.shape, k.dtype)
    _expect("dv", dv, k.shape, k.dtype)
    _tensors(q, k, v, bias, segment_ids, extra=(("lse", lse), ("delta", delta), ("dout", dout), ("dk", dk),
                                                ("dv", dv)))
    _check(lib.ra_blockwise_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                          int(q_chunk), int(k_chunk), _causal(causal), _ptr(lse), _ptr(delta),
                                          _ptr(dout), _ptr(dk), _ptr(dv), ctypes.byref(shape), _stream(q.device)))
    return dk, dv


def blockwise_attn_bwd_dq(q, k, v, lse, delta, dout, bias=None, segment_ids=None, *, n_ring, q_chunk, k_chunk,
                          causal, ring_rank=-1, scale=None, dq=None):
    lib = load_library()
    _tensors(q, k, v, bias, segment_ids, devices=False)
    shape = make_shape(q, k, ring_rank=ring_rank, scale=scale, bias=bias)
    dq = torch.empty_like(q) if dq is None else dq
    _check_rowstats(q, lse, delta, dout)
    _expect("dq", dq, q.shape, q.dtype)
    _tensors(q, k, v, bias, segment_ids, extra=(("lse", lse), ("delta", delta), ("dout", dout), ("dq", dq)))
    _check(lib.ra_blockwise_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(n_ring),
                                        int(q_chunk), int(k_chunk), _causal(causal), _ptr(lse), _ptr(delta),
                                        _ptr(dout), _ptr(dq), ctypes.byref(shape), _stream(q.device)))
    return dq


def blockwise_attn_fwd_step(q, k, v, bias=None, segment_ids=None, *, q_pos0, kv_pos0, causal, state=None,
                            init=None, scale=None):
    """One ring step (ra_blockwise_attn_fwd_step): fold the K/V block held (keys at global positions
    kv_pos0 + j) into the running state of the queries q (global positions q_pos0 + i).

    state is (o, m, l) from the previous step, updated in place; None allocates a new one.  init
    (default: state is None) makes the step ignore what the state holds and start afresh.
    segment_ids, when given, is int32 [batch, seg_len] on global positions.  Returns the state."""
    lib = load_library()
    _step_segments(segment_ids, q)
    _tensors(q, k, v, bias, None, devices=False)
    B, Lq, H, D = q.shape
    init = state is None if init is None else bool(init)
    if state is None:
        state = (torch.empty((B, Lq, H, D), dtype=torch.float32, device=q.device),
                 torch.empty((B, H, Lq), dtype=torch.float32, device=q.device),
                 torch.empty((B, H, Lq), dtype=torch.float32, device=q.device))
    o, m, l_ = state
    _expect("o", o, q.shape, torch.float32)
    _expect("m", m, _rows(q), torch.float32)
    _expect("l", l_, _rows(q), torch.float32)
    _tensors(q, k, v, bias, None, extra=(("segment_ids", segment_ids), ("o", o), ("m", m), ("l", l_)))
    shape = make_shape(q, k, ring_rank=0, scale=scale, bias=bias)
    seg_len = 0 if segment_ids is None else segment_ids.shape[1]
    _check(lib.ra_blockwise_attn_fwd_step(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(seg_len),
                                          int(q_pos0), int(kv_pos0), _causal(causal), _ptr(o), _ptr(m), _ptr(l_),
                                          int(init), ctypes.byref(shape), _stream(q.device)))
    return state


def blockwise_attn_fwd_finalize(state, *, dtype=torch.bfloat16, out=None, lse=None):
    """out, lse = ra_blockwise_attn_fwd_finalize(state) after the last ring step."""
    lib = load_library()
    o, m, l_ = state
    B, Lq, H, D = o.shape
    out = torch.empty((B, Lq, H, D), dtype=dtype, device=o.device) if out is None else out
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=o.device) if lse is None else lse
    if dtype not in _DTYPES or o.dtype != torch.float32:
        raise ValueError("the state's o must be float32 and dtype bfloat16 or float32")
    _expect("m", m, (B, H, Lq), torch.float32)
    _expect("l", l_, (B, H, Lq), torch.float32)
    _expect("out", out, (B, Lq, H, D), dtype)
    _expect("lse", lse, (B, H, Lq), torch.float32)
    _tensors(o, o, o, None, None, extra=(("m", m), ("l", l_), ("out", out), ("lse", lse)))
    shape = Shape(B, H, D, -1, Lq, Lq, 0, 0.0, _DTYPES[dtype])
    _check(lib.ra_blockwise_attn_fwd_finalize(_ptr(o), _ptr(m), _ptr(l_), _ptr(out), _ptr(lse), ctypes.byref(shape),
                                              _stream(o.device)))
    return out, lse


def attn_merge(out_a, lse_a, out_b, lse_b):
    """ra_attn_merge: fold (out_b, lse_b) into (out_a, lse_a) in place; returns out_a, lse_a."""
    lib = load_library()
    _expect("out_b", out_b, out_a.shape, out_a.dtype)
    _expect("lse_a", lse_a, _rows(out_a), torch.float32)
    _expect("lse_b", lse_b, _rows(out_a), torch.float32)
    _tensors(out_a, out_a, out_a, None, None, extra=(("lse_a", lse_a), ("out_b", out_b), ("lse_b", lse_b)))
    B, Lq, H, D = out_a.shape
    shape = Shape(B, H, D, -1, Lq, Lq, 0, 0.0, _DTYPES[out_a.dtype])
    _check(lib.ra_attn_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), ctypes.byref(shape),
                             _stream(out_a.device)))
    return out_a, lse_a


def blockwise_attn_bwd_step(q, k, v, lse, delta, dout, bias=None, segment_ids=None, *, q_pos0, kv_pos0, causal,
                            dq_acc=None, dk_acc=None, dv_acc=None, dbias_acc=None, init_dq=None, init_dkv=None,
                            scale=None):
    """One backward ring step (ra_blockwise_attn_bwd_step): add this K/V block's contributions to
    the float32 sums dq_acc (of the queries q) and dk_acc, dv_acc (of the block), and with a given
    dbias_acc (float32 [batch, heads, block length]) the block's per-key sums of dS.  A sum passed as
    None is allocated and started at zero; init_dq / init_dkv (default: the sum was None) start a
    given one at zero.  Returns (dq_acc, dk_acc, dv_acc)."""
    lib = load_library()
    _step_segments(segment_ids, q)
    _tensors(q, k, v, bias, None, devices=False)
    _check_rowstats(q, lse, delta, dout)
    f32 = dict(dtype=torch.float32, device=q.device)
    i_dq = dq_acc is None if init_dq is None else bool(init_dq)
    i_dkv = (dk_acc is None or dv_acc is None) if init_dkv is None else bool(init_dkv)
    dq_acc = torch.empty(q.shape, **f32) if dq_acc is None else dq_acc
    dk_acc = torch.empty(k.shape, **f32) if dk_acc is None else dk_acc
    dv_acc = torch.empty(v.shape, **f32) if dv_acc is None else dv_acc
    _expect("dq_acc", dq_acc, q.shape, torch.float32)
    _expect("dk_acc", dk_acc, k.shape, torch.float32)
    _expect("dv_acc", dv_acc, k.shape, torch.float32)
    if dbias_acc is not None:
        if bias is None:
            raise ValueError("dbias_acc needs a bias")
        _expect("dbias_acc", dbias_acc, (k.shape[0], k.shape[2], k.shape[1]), torch.float32)
    _tensors(q, k, v, bias, None, extra=(("lse", lse), ("delta", delta), ("dout", dout), ("segment_ids", segment_ids),
                                         ("dq_acc", dq_acc), ("dk_acc", dk_acc), ("dv_acc", dv_acc),
                                         ("dbias_acc", dbias_acc)))
    shape = make_shape(q, k, ring_rank=0, scale=scale, bias=bias)
    seg_len = 0 if segment_ids is None else segment_ids.shape[1]
    _check(lib.ra_blockwise_attn_bwd_step(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(segment_ids), int(seg_len),
                                          int(q_pos0), int(kv_pos0), _causal(causal), _ptr(lse), _ptr(delta),
                                          _ptr(dout), _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _ptr(dbias_acc),
                                          int(i_dq), int(i_dkv), ctypes.byref(shape), _stream(q.device)))
    return dq_acc, dk_acc, dv_acc


def blockwise_attn_bwd_dbias_reduce(key_sums, kv_pos0, dbias, *, accumulate=True):
    """ra_blockwise_attn_bwd_dbias_reduce: add (or write) one K/V block's share of the bias gradient,
    from the per-key sums key_sums [batch, heads, block length] it carried round the ring (keys at
    global positions kv_pos0 + j), into dbias [heads, bias_len].  Returns dbias."""
    lib = load_library()
    if key_sums.dim() != 3 or dbias.dim() != 2 or dbias.shape[0] != key_sums.shape[1]:
        raise ValueError("key_sums [batch, heads, block length] and dbias [heads, bias_len] expected")
    _expect("key_sums", key_sums, key_sums.shape, torch.float32)
    _expect("dbias", dbias, dbias.shape, torch.float32)
    _devices(("key_sums", key_sums), ("dbias", dbias))
    B, H, Lk = key_sums.shape
    shape = Shape(B, H, 64, -1, Lk, Lk, dbias.shape[1], 0.0, RA_F32)
    _check(lib.ra_blockwise_attn_bwd_dbias_reduce(_ptr(key_sums), int(kv_pos0), _ptr(dbias), int(bool(accumulate)),
                                                  ctypes.byref(shape), _stream(dbias.device)))
    return dbias


def blockwise_attn_bwd_finalize(dq_acc, dk_acc, dv_acc, *, dtype=torch.bfloat16, scale=None, dq=None, dk=None,
                                dv=None):
    """dq, dk, dv = ra_blockwise_attn_bwd_finalize(...) from the ring-step sums."""
    lib = load_library()
    B, Lq, H, D = dq_acc.shape
    Lk = dk_acc.shape[1]
    dq = torch.empty(dq_acc.shape, dtype=dtype, device=dq_acc.device) if dq is None else dq
    dk = torch.empty(dk_acc.shape, dtype=dtype, device=dq_acc.device) if dk is None else dk
    dv = torch.empty(dv_acc.shape, dtype=dtype, device=dq_acc.device) if dv is None else dv
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    _expect("dq_acc", dq_acc, dq_acc.shape, torch.float32)
    _expect("dk_acc", dk_acc, (B, Lk, H, D), torch.float32)
    _expect("dv_acc", dv_acc, (B, Lk, H, D), torch.float32)
    _expect("dq", dq, (B, Lq, H, D), dtype)
    _expect("dk", dk, (B, Lk, H, D), dtype)
    _expect("dv", dv, (B, Lk, H, D), dtype)
    _tensors(dq_acc, dq_acc, dq_acc, None, None,
             extra=(("dk_acc", dk_acc), ("dv_acc", dv_acc), ("dq", dq), ("dk", dk), ("dv", dv)))
    shape = Shape(B, H, D, -1, Lq, Lk, 0, 0.0 if scale is None else float(scale), _DTYPES[dtype])
    _check(lib.ra_blockwise_attn_bwd_finalize(_ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _ptr(dq), _ptr(dk), _ptr(dv),
                                              ctypes.byref(shape), _stream(dq_acc.device)))
    return dq, dk, dv


def _ffn_args(x, w1, w3, w2):
    if x.dim() != 2 or w1.dim() != 2 or w1.shape != w3.shape or w2.shape != (w1.shape[1], w1.shape[0]) \
            or x.shape[1] != w1.shape[1]:
        raise ValueError("x [tokens, d_model], w1 and w3 [d_ff, d_model], w2 [d_model, d_ff] expected")
    for name, t in (("x", x), ("w1", w1), ("w3", w3), ("w2", w2)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    _devices(("x", x), ("w1", w1), ("w3", w3), ("w2", w2))
    return x.shape[0], x.shape[1], w1.shape[0]


def _ffn_workspace(lib, device, tokens, d, f, chunk, backward, workspace):
    need = int(lib.ra_blockwise_ffn_workspace_size(int(tokens), int(d), int(f), int(chunk), int(backward)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)   # torch aligns to 256 bytes
    _workspace("workspace", workspace)
    _devices(("workspace", workspace),)
    if workspace.device != device:
        raise ValueError("workspace must be on the inputs' device")
    return workspace


def blockwise_ffn_fwd(x, w1, w3, w2, *, chunk, out=None, workspace=None):
    """out = ra_blockwise_ffn_fwd(...): SwiGLU feed-forward of every token, chunk tokens at a time."""
    lib = load_library()
    T, d, f = _ffn_args(x, w1, w3, w2)
    out = torch.empty_like(x) if out is None else out
    _expect("out", out, x.shape, x.dtype)
    _devices(("x", x), ("out", out))
    workspace = _ffn_workspace(lib, x.device, T, d, f, chunk, False, workspace)
    _check(lib.ra_blockwise_ffn_fwd(_ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out), int(T), int(d), int(f),
                                    int(chunk), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(x.device)))
    return out


def blockwise_ffn_bwd(x, w1, w3, w2, dout, *, chunk, dx=None, dw1=None, dw3=None, dw2=None, workspace=None):
    """dx, dw1, dw3, dw2 = ra_blockwise_ffn_bwd(...): dx bfloat16, weight gradients float32."""
    lib = load_library()
    T, d, f = _ffn_args(x, w1, w3, w2)
    _expect("dout", dout, x.shape, x.dtype)
    dx = torch.empty_like(x) if dx is None else dx
    f32 = dict(dtype=torch.float32, device=x.device)
    dw1 = torch.empty(w1.shape, **f32) if dw1 is None else dw1
    dw3 = torch.empty(w3.shape, **f32) if dw3 is None else dw3
    dw2 = torch.empty(w2.shape, **f32) if dw2 is None else dw2
    _expect("dx", dx, x.shape, x.dtype)
    _expect("dw1", dw1, w1.shape, torch.float32)
    _expect("dw3", dw3, w3.shape, torch.float32)
    _expect("dw2", dw2, w2.shape, torch.float32)
    _devices(("x", x), ("dout", dout), ("dx", dx), ("dw1", dw1), ("dw3", dw3), ("dw2", dw2))
    workspace = _ffn_workspace(lib, x.device, T, d, f, chunk, True, workspace)
    _check(lib.ra_blockwise_ffn_bwd(_ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(dout), _ptr(dx), _ptr(dw1),
                                    _ptr(dw3), _ptr(dw2), int(T), int(d), int(f), int(chunk), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(x.device)))
    return dx, dw1, dw3, dw2

