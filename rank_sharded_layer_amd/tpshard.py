"""Thin Python binding of libtpshard (argument marshalling only).

Every function has the name of the C entry point it calls and does three
things: checks that the tensors it is given are contiguous, on the GPU and of
matching shapes and dtypes (the C library receives raw pointers and cannot
check buffer extents); allocates outputs/workspace with torch when the caller
does not pass them; and calls the C function on torch's current stream.  All
arithmetic happens in the library's HIP kernels.  There is no fallback: if
the library is not built, or the GPU is missing, the call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_F32, TP_BF16 = 0, 1
TP_ORDER_RING = 0
TP_ORDER_RANK = 1
TP_MAX_RANKS = 64
STATUS_NAMES = {0: "TP_OK", 1: "TP_EINVAL", 2: "TP_ESHAPE", 3: "TP_EDTYPE", 4: "TP_EALIGN",
                5: "TP_EHIP", 6: "TP_EWORKSPACE"}


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class RingStep(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int), ("step", ctypes.c_int), ("src", ctypes.c_int),
                ("dst", ctypes.c_int), ("chunk", ctypes.c_int), ("offset", ctypes.c_int64),
                ("len", ctypes.c_int64)]


_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)
_szp = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "tp_abi_version": (ctypes.c_int, []),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_shard_weights": (_int, [_vp, _i64, _i64, _int, _int, _int, _int, _vp, _vp]),
    "tp_shard_gate_up": (_int, [_vp, _vp, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "tp_kv_heads_for_rank": (_int, [_i64, _int, _int, _i64p, _i64p]),
    "tp_shard_qkv": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "tp_load_staging_bytes": (_int, [_i64, _i64, _int, _int, _szp]),
    "tp_load_shard": (_int, [_vp, _int, _i64, _i64, _int, _int, _int, _vp, _int, _vp, _sz, _vp]),
    "tp_load_gate_up": (_int, [_vp, _int, _int, _i64, _i64, _int, _int, _vp, _int, _vp, _sz, _vp]),
    "tp_load_qkv": (_int, [_vp, _int, _int, _i64, _i64, _i64, _i64, _int, _int, _vp, _int, _vp, _sz, _vp]),
    "tp_gate_up_workspace_bytes": (_int, [_i64, _i64, _i64, _int, _szp]),
    "tp_gate_up_act_rank": (_int, [_vp, _i64, _i64, _vp, _i64, _int, _vp, _vp, _sz, _vp]),
    "tp_linear_workspace_bytes": (_int, [_i64, _i64, _i64, _int, _szp]),
    "tp_linear_rank_forward": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _int, _vp, _int, _vp, _sz, _vp]),
    "tp_mlp_workspace_bytes": (_int, [_i64, _i64, _i64, _int, _szp]),
    "tp_mlp_rank_forward": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _int, _vp, _int, _vp, _sz, _vp]),
    "tp_mlp_rank_forward_noalloc": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _int, _vp, _int, _vp]),
    "tp_partial_reduce": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _vp, _int, _int, _vp]),
    "tp_ring_schedule": (_int, [_int, _i64, ctypes.POINTER(RingStep), _int, ctypes.POINTER(_int)]),
    "tp_sp_rows": (_int, [_i64, _int, _int, _i64p, _i64p]),
    "tp_attention_workspace_bytes": (_int, [_i64, _int, _int, _int, _int, _int, _szp]),
    "tp_attention_rank": (_int, [_vp, _i64, _int, _int, _int, _int, _int, _vp, _vp, _sz, _vp]),
    "tp_logits_gather_argmax": (_int, [ctypes.POINTER(_vp), _int, _i64, _i64, _int, _vp, _vp, _vp]),
    "tp_rs_add_rmsnorm": (_int, [ctypes.POINTER(_vp), _int, _int, _i64, _i64, _int, _vp, _vp, ctypes.c_float,
                                 _vp, _vp, _vp]),
    "tp_vocab_range": (_int, [_i64, _int, _int, _i64p, _i64p]),
    "tp_vocab_embed_rank": (_int, [_vp, _i64, _vp, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "tp_lm_head_rank": (_int, [_vp, _i64, _i64, _vp, _i64, _int, _vp, _int, _vp, _sz, _vp]),
}

_lib = None


def lib():
    """Load libtpshard.so (after torch, so that it binds torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_names():
    return list(_SIGS)


def _check(status: int):
    if status != 0:
        raise TPError(status, lib().tp_last_error().decode())


def _dt(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return TP_BF16
    if dtype == torch.float32:
        return TP_F32
    raise TPError(3, f"unsupported dtype {dtype}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream):
    """The torch stream object for a caller's `stream` (None: the current one)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _empty(shape, dtype, device, stream):
    """torch.empty allocated on the stream the kernels will run on.  torch's
    caching allocator ties a block to the stream current at allocation time
    and reuses it for later allocations on that stream once freed; a block
    made on another stream could be handed out again while this call's
    kernels still use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    s = _torch_stream(stream)
    if s == torch.cuda.current_stream():
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(s):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device, workspace, stream=None):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = _empty(nbytes, torch.uint8, device, stream)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise TPError(6, f"workspace of {nbytes} bytes needed")
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


# ---- library ---------------------------------------------------------------

def tp_abi_version() -> int:
    return lib().tp_abi_version()


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


# ---- shard selection -------------------------------------------------------

def tp_shard_weights(full, dim, tp_rank, tp_size, out=None, stream=None):
    rows, cols = full.shape
    shape = (rows // max(tp_size, 1), cols) if dim == 0 else (rows, cols // max(tp_size, 1))
    if out is None:
        out = _empty(shape, full.dtype, full.device, stream)
    p_full = _dev(full, "full")
    p_out = _dev(out, "out", full.dtype, shape)
    _check(lib().tp_shard_weights(p_full, rows, cols, _dt(full.dtype), dim, tp_rank, tp_size,
                                  p_out, _stream(stream)))
    return out


def tp_shard_gate_up(gate, up, tp_rank, tp_size, out=None, stream=None):
    f, h = gate.shape
    shape = (2 * (f // max(tp_size, 1)), h)
    if out is None:
        out = _empty(shape, gate.dtype, gate.device, stream)
    pg = _dev(gate, "gate")
    pu = _dev(up, "up", gate.dtype, gate.shape)
    po = _dev(out, "out", gate.dtype, shape)
    _check(lib().tp_shard_gate_up(pg, pu, f, h, _dt(gate.dtype), tp_rank, tp_size, po,
                                  _stream(stream)))
    return out


# ---- checkpoint-style loaders ------------------------------------------------

def _host(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.is_cuda:
        raise ValueError(f"{name} must be a host (CPU) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return ctypes.c_void_p(t.data_ptr())


def tp_load_staging_bytes(rows, cols, src_dtype, dst_dtype) -> int:
    b = ctypes.c_size_t()
    _check(lib().tp_load_staging_bytes(rows, cols, _dt(src_dtype), _dt(dst_dtype), ctypes.byref(b)))
    return b.value


def _staging(rows, cols, src_dtype, out, staging, stream):
    return _workspace(tp_load_staging_bytes(rows, cols, src_dtype, out.dtype), out.device, staging, stream)


def tp_load_shard(src, dim, tp_rank, tp_size, dtype=torch.bfloat16, out=None, staging=None, stream=None):
    rows, cols = src.shape
    shape = (rows // max(tp_size, 1), cols) if dim == 0 else (rows, cols // max(tp_size, 1))
    if out is None:
        out = _empty(shape, dtype, "cuda", stream)
    ps = _host(src, "src")
    po = _dev(out, "out", None, shape)
    pw, nw = _staging(shape[0], shape[1], src.dtype, out, staging, stream)
    _check(lib().tp_load_shard(ps, _dt(src.dtype), rows, cols, dim, tp_rank, tp_size, po, _dt(out.dtype), pw, nw,
                               _stream(stream)))
    return out


def tp_load_gate_up(src, shard_id, tp_rank, tp_size, out, staging=None, stream=None):
    f, h = src.shape
    ps = _host(src, "src")
    po = _dev(out, "out", None, (2 * (f // max(tp_size, 1)), h))
    pw, nw = _staging(f // max(tp_size, 1), h, src.dtype, out, staging, stream)
    _check(lib().tp_load_gate_up(ps, _dt(src.dtype), shard_id, f, h, tp_rank, tp_size, po, _dt(out.dtype), pw, nw,
                                 _stream(stream)))
    return out


def tp_load_qkv(src, shard_id, n_q, n_kv, head_dim, tp_rank, tp_size, out, staging=None, stream=None):
    h = src.shape[1]
    _, kvc = tp_kv_heads_for_rank(n_kv, tp_rank, tp_size)
    nq_r = n_q // max(tp_size, 1)
    ps = _host(src, "src")
    po = _dev(out, "out", None, ((nq_r + 2 * kvc) * head_dim, h))
    rows = (nq_r if shard_id == 0 else kvc) * head_dim
    pw, nw = _staging(rows, h, src.dtype, out, staging, stream)
    _check(lib().tp_load_qkv(ps, _dt(src.dtype), shard_id, n_q, n_kv, head_dim, h, tp_rank, tp_size, po,
                             _dt(out.dtype), pw, nw, _stream(stream)))
    return out


def tp_kv_heads_for_rank(n_kv, tp_rank, tp_size):
    first, count = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tp_kv_heads_for_rank(n_kv, tp_rank, tp_size, ctypes.byref(first), ctypes.byref(count)))
    return first.value, count.value


def tp_shard_qkv(wq, wk, wv, n_q, n_kv, head_dim, tp_rank, tp_size, out=None, stream=None):
    h = wq.shape[1]
    if tuple(wq.shape) != (n_q * head_dim, h):
        raise ValueError("wq must be [n_q*head_dim, h]")
    _, kvc = tp_kv_heads_for_rank(n_kv, tp_rank, tp_size)
    shape = ((n_q // tp_size + 2 * kvc) * head_dim, h)
    if out is None:
        out = _empty(shape, wq.dtype, wq.device, stream)
    pq = _dev(wq, "wq")
    pk = _dev(wk, "wk", wq.dtype, (n_kv * head_dim, h))
    pv = _dev(wv, "wv", wq.dtype, (n_kv * head_dim, h))
    po = _dev(out, "out", wq.dtype, shape)
    _check(lib().tp_shard_qkv(pq, pk, pv, n_q, n_kv, head_dim, h, _dt(wq.dtype), tp_rank, tp_size,
                              po, _stream(stream)))
    return out


# ---- GEMMs -----------------------------------------------------------------

def tp_gate_up_workspace_bytes(n, h, f_local, dtype) -> int:
    b = ctypes.c_size_t()
    _check(lib().tp_gate_up_workspace_bytes(n, h, f_local, _dt(dtype), ctypes.byref(b)))
    return b.value


def tp_gate_up_act_rank(x, w_gate_up, act=None, workspace=None, stream=None):
    n, h = x.shape
    f_local = w_gate_up.shape[0] // 2
    px = _dev(x, "x")
    pw = _dev(w_gate_up, "w_gate_up", x.dtype, (2 * f_local, h))
    if act is None:
        act = _empty((n, f_local), x.dtype, x.device, stream)
    pa = _dev(act, "act", x.dtype, (n, f_local))
    pws, nws = _workspace(tp_gate_up_workspace_bytes(n, h, f_local, x.dtype), x.device, workspace, stream)
    _check(lib().tp_gate_up_act_rank(px, n, h, pw, f_local, _dt(x.dtype), pa, pws, nws,
                                     _stream(stream)))
    return act


def tp_linear_workspace_bytes(n, k, m, dtype) -> int:
    b = ctypes.c_size_t()
    _check(lib().tp_linear_workspace_bytes(n, k, m, _dt(dtype), ctypes.byref(b)))
    return b.value


def tp_linear_rank_forward(x, w, bias=None, out_dtype=None, y=None, workspace=None, stream=None):
    n, k = x.shape
    m = w.shape[0]
    out_dtype = out_dtype or x.dtype
    px = _dev(x, "x")
    pw = _dev(w, "w", x.dtype, (m, k))
    pb = _dev(bias, "bias", x.dtype, (m,)) if bias is not None else None
    if y is None:
        y = _empty((n, m), out_dtype, x.device, stream)
    py = _dev(y, "y", out_dtype, (n, m))
    pws, nws = _workspace(tp_linear_workspace_bytes(n, k, m, x.dtype), x.device, workspace, stream)
    _check(lib().tp_linear_rank_forward(px, n, k, pw, m, pb, _dt(x.dtype), py, _dt(out_dtype),
                                        pws, nws, _stream(stream)))
    return y


def tp_mlp_workspace_bytes(n, h, f_local, dtype) -> int:
    b = ctypes.c_size_t()
    _check(lib().tp_mlp_workspace_bytes(n, h, f_local, _dt(dtype), ctypes.byref(b)))
    return b.value


def tp_mlp_rank_forward(x, w_gate_up, w_down, out_dtype=None, partial=None, workspace=None,
                        stream=None):
    n, h = x.shape
    f_local = w_gate_up.shape[0] // 2
    out_dtype = out_dtype or x.dtype
    px = _dev(x, "x")
    pgu = _dev(w_gate_up, "w_gate_up", x.dtype, (2 * f_local, h))
    pd = _dev(w_down, "w_down", x.dtype, (h, f_local))
    if partial is None:
        partial = _empty((n, h), out_dtype, x.device, stream)
    pp = _dev(partial, "partial", out_dtype, (n, h))
    need = tp_mlp_workspace_bytes(n, h, f_local, x.dtype)
    if workspace is None:
        workspace = _empty(need, torch.uint8, x.device, stream)
    pws = _dev(workspace, "workspace")
    nws = workspace.numel() * workspace.element_size()
    _check(lib().tp_mlp_rank_forward(px, n, h, pgu, pd, f_local, _dt(x.dtype), pp, _dt(out_dtype),
                                     pws, nws, _stream(stream)))
    return partial


# ---- reduce ------------------------------------------------------------------

def tp_partial_reduce(partials, out=None, out_dtype=None, order=TP_ORDER_RING, stream=None):
    t = len(partials)
    if t < 1:
        raise TPError(1, "no partials")
    p0 = partials[0]
    out_dtype = out_dtype or p0.dtype
    ptrs = (ctypes.c_void_p * t)(*[_dev(p, f"partials[{i}]", p0.dtype, p0.shape).value
                                   for i, p in enumerate(partials)])
    if out is None:
        out = _empty(p0.shape, out_dtype, p0.device, stream)
    po = _dev(out, "out", out_dtype, p0.shape)
    _check(lib().tp_partial_reduce(ptrs, t, p0.numel(), _dt(p0.dtype), po, _dt(out_dtype), order,
                                   _stream(stream)))
    return out


def tp_ring_schedule(t, K):
    n = max(2 * t * (t - 1), 1)
    arr = (RingStep * n)()
    got = ctypes.c_int()
    _check(lib().tp_ring_schedule(t, K, arr, n, ctypes.byref(got)))
    return [dict(phase=s.phase, step=s.step, src=s.src, dst=s.dst, chunk=s.chunk, offset=s.offset,
                 len=s.len) for s in arr[:got.value]]


def tp_attention_workspace_bytes(n, nq, nkv, head_dim=128, causal=True) -> int:
    b = ctypes.c_size_t()
    _check(lib().tp_attention_workspace_bytes(n, nq, nkv, head_dim, _dt(torch.bfloat16), 1 if causal else 0,
                                              ctypes.byref(b)))
    return b.value


def tp_attention_rank(qkv, nq, nkv, head_dim=128, causal=True, out=None, workspace=None, stream=None):
    """softmax(q k^T / sqrt(d)) v for the rank's nq query heads over its nkv KV
    heads, from the packed QKV projection output [n, (nq + 2 nkv) d]."""
    n = qkv.shape[0]
    pq = _dev(qkv, "qkv", torch.bfloat16, (n, (nq + 2 * nkv) * head_dim))
    if out is None:
        out = _empty((n, nq * head_dim), torch.bfloat16, qkv.device, stream)
    po = _dev(out, "out", torch.bfloat16, (n, nq * head_dim))
    ws, wsb = _workspace(tp_attention_workspace_bytes(n, nq, nkv, head_dim, causal), qkv.device, workspace, stream)
    _check(lib().tp_attention_rank(pq, n, nq, nkv, head_dim, _dt(torch.bfloat16), 1 if causal else 0, po, ws, wsb,
                                   _stream(stream)))
    return out


def tp_logits_gather_argmax(shards, vocab, full=None, argmax=None, want_full=True, stream=None):
    """Concatenation of the t fp32 logits shards [n, end_r - start_r] along the
    vocabulary ([n, vocab]) and each row's first argmax (int64).  Returns
    (full or None, argmax)."""
    t = len(shards)
    if t < 1:
        raise TPError(1, "no shards")
    n = shards[0].shape[0]
    dev = shards[0].device
    ptrs = []
    for r, sh in enumerate(shards):
        s, e = tp_vocab_range(vocab, r, t)
        ptrs.append(_dev(sh, f"shards[{r}]", torch.float32, (n, e - s)).value if e > s else None)
    arr = (ctypes.c_void_p * t)(*ptrs)
    if want_full and full is None:
        full = _empty((n, vocab), torch.float32, dev, stream)
    pf = _dev(full, "full", torch.float32, (n, vocab)) if full is not None else None
    if argmax is None:
        argmax = _empty((n,), torch.int64, dev, stream)
    pa = _dev(argmax, "argmax", torch.int64, (n,))
    _check(lib().tp_logits_gather_argmax(arr, t, n, vocab, _dt(torch.float32), pf, pa, _stream(stream)))
    return full, argmax


# ---- sequence-parallel epilogue -------------------------------------------------

def tp_sp_rows(n, tp_rank, tp_size):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tp_sp_rows(n, tp_rank, tp_size, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def tp_rs_add_rmsnorm(partials, tp_rank, residual, weight, eps, residual_out=None, out=None, stream=None):
    """Rank tp_rank's rows after the ring reduce-scatter of `partials` ([n, h]
    each), plus `residual` (the rank's rows), RMSNorm with `weight`.  Returns
    (residual_out, out); residual_out may be `residual` (in place)."""
    t = len(partials)
    if t < 1:
        raise TPError(1, "no partials")
    p0 = partials[0]
    n, h = p0.shape
    lo, hi = tp_sp_rows(n, tp_rank, t)
    ptrs = (ctypes.c_void_p * t)(*[_dev(p, f"partials[{i}]", p0.dtype, p0.shape).value
                                   for i, p in enumerate(partials)])
    rows = (hi - lo, h)
    pr = _dev(residual, "residual", p0.dtype, rows)
    pw = _dev(weight, "weight", p0.dtype, (h,))
    if residual_out is None:
        residual_out = _empty(rows, p0.dtype, p0.device, stream)
    if out is None:
        out = _empty(rows, p0.dtype, p0.device, stream)
    pro = _dev(residual_out, "residual_out", p0.dtype, rows)
    po = _dev(out, "out", p0.dtype, rows)
    _check(lib().tp_rs_add_rmsnorm(ptrs, t, tp_rank, n, h, _dt(p0.dtype), pr, pw, float(eps), pro, po,
                                   _stream(stream)))
    return residual_out, out


# ---- vocab parallel -----------------------------------------------------------

def tp_vocab_range(vocab, tp_rank, tp_size):
    s, e = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tp_vocab_range(vocab, tp_rank, tp_size, ctypes.byref(s), ctypes.byref(e)))
    return s.value, e.value


def tp_vocab_embed_rank(ids, table_shard, vocab, tp_rank, tp_size, out=None, stream=None):
    n = ids.numel()
    h = table_shard.shape[1]
    s, e = tp_vocab_range(vocab, tp_rank, tp_size)
    pi = _dev(ids, "ids", torch.int64)
    pt = _dev(table_shard, "table_shard", None, (e - s, h))
    if out is None:
        out = _empty((n, h), table_shard.dtype, ids.device, stream)
    po = _dev(out, "out", table_shard.dtype, (n, h))
    _check(lib().tp_vocab_embed_rank(pi, n, pt, vocab, h, tp_rank, tp_size, _dt(table_shard.dtype),
                                     po, _stream(stream)))
    return out


def tp_lm_head_rank(x, table_shard, out_dtype=torch.float32, logits=None, workspace=None, stream=None):
    n, h = x.shape
    v_local = table_shard.shape[0]
    px = _dev(x, "x")
    pt = _dev(table_shard, "table_shard", x.dtype, (v_local, h))
    if logits is None:
        logits = _empty((n, v_local), out_dtype, x.device, stream)
    pl = _dev(logits, "logits", out_dtype, (n, v_local))
    pws, nws = _workspace(tp_linear_workspace_bytes(n, h, v_local, x.dtype), x.device, workspace, stream)
    _check(lib().tp_lm_head_rank(px, n, h, pt, v_local, _dt(x.dtype), pl, _dt(out_dtype), pws, nws,
                                 _stream(stream)))
    return logits
