"""fp64 CPU oracle for one tensor-parallel rank's share of a Transformer layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The GPU library never imports it and
shares no code with it; the oracle takes numpy arrays and returns numpy
arrays.  The arithmetic lives in tp_oracle.c (plain loops, fp64); this file
only marshals arguments.

Every function cites the passage of the pages it follows in tp_oracle.c.
Parity status: every function here is pinned by tests/test_oracle_pins.py
(worked examples the pages print, closed forms, library routines the pages
themselves call, brute force and invariants).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


class RingStep(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int), ("step", ctypes.c_int),
                ("src", ctypes.c_int), ("dst", ctypes.c_int),
                ("chunk", ctypes.c_int), ("offset", ctypes.c_int64),
                ("len", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_silu": (ctypes.c_double, [ctypes.c_double]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_bf16_array": (None, [_f32p, _i64, _u16p]),
        "orc_bf16_to_f64_array": (None, [_u16p, _i64, _f64p]),
        "orc_linear": (None, [_f64p, _i64, _i64, _f64p, _i64, _f64p, _f64p]),
        "orc_mlp": (None, [_f64p, _i64, _i64, _f64p, _f64p, _i64, _f64p, _f64p]),
        "orc_mlp_rank": (None, [_f64p, _i64, _i64, _f64p, _f64p, _i64, _f64p,
                                _int, _int, _f64p]),
        "orc_silu_mul": (None, [_f64p, _f64p, _i64, _f64p]),
        "orc_narrow": (_int, [_vp, _i64, _i64, _int, _int, _i64, _i64, _vp]),
        "orc_shard": (_int, [_vp, _i64, _i64, _int, _int, _int, _int, _vp]),
        "orc_shard_gate_up": (_int, [_vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
        "orc_kv_heads_for_rank": (_int, [_i64, _int, _int, _i64p, _i64p]),
        "orc_shard_qkv": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                 _int, _int, _vp]),
        "orc_vocab_range": (_int, [_i64, _int, _int, _i64p, _i64p]),
        "orc_embed_full": (None, [_i64p, _i64, _vp, _i64, _i64, _int, _vp]),
        "orc_embed_rank": (_int, [_i64p, _i64, _vp, _i64, _i64, _int, _int, _int, _vp]),
        "orc_lm_head_rank": (_int, [_f64p, _i64, _i64, _f64p, _i64, _int, _int, _f64p]),
        "orc_chunk_bounds": (None, [_i64, _int, _int, _i64p, _i64p]),
        "orc_ring_schedule": (_int, [_int, _i64, ctypes.POINTER(RingStep), _int]),
        "orc_ring_allreduce_f32": (_int, [ctypes.POINTER(_f32p), _int, _i64, _i64,
                                          _i64, _f32p]),
        "orc_reduce_sum_f64": (None, [ctypes.POINTER(_f64p), _int, _i64, _f64p]),
        "orc_ring_traffic": (_int, [_int, _i64, _i64p, _i64p, ctypes.POINTER(ctypes.c_int)]),
        "orc_sp_rows": (None, [_i64, _int, _int, _i64p, _i64p]),
        "orc_reduce_rank_f32": (None, [ctypes.POINTER(_f32p), _int, _i64, _f32p]),
        "orc_attention_rank": (_int, [_f64p, _i64, _int, _int, _int, _int, _i64p, _i64, _f64p]),
        "orc_logits_gather_argmax": (_int, [ctypes.POINTER(_f64p), _int, _i64, _i64, _f64p, _i64p]),
        "orc_load_shard": (_int, [_vp, _int, _i64, _i64, _int, _int, _int, _vp, _int]),
        "orc_load_gate_up": (_int, [_vp, _int, _vp, _int, _int, _i64, _i64, _int, _int]),
        "orc_load_qkv": (_int, [_vp, _int, _vp, _int, _int, _i64, _i64, _i64, _i64, _int, _int]),
        "orc_rs_add_rmsnorm": (_int, [ctypes.POINTER(_f32p), _int, _int, _i64, _i64, _f32p, _f64p,
                                      ctypes.c_double, _int, _f32p, _f64p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a, t):
    return a.ctypes.data_as(t)


# --- scalar / conversion --------------------------------------------------

def silu(z: float) -> float:
    return _load().orc_silu(float(z))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(_p(a, _f32p), a.size, _p(out, _u16p))
    return out


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_bf16_to_f64_array(_p(b, _u16p), b.size, _p(out, _f64p))
    return out


# --- linear / MLP ---------------------------------------------------------

def linear(x, w, bias=None) -> np.ndarray:
    """y = x . w^T (+ bias), weights stored [out, in]."""
    x, w = _f64(x), _f64(w)
    n, k = x.shape
    m, k2 = w.shape
    assert k == k2
    y = np.empty((n, m), dtype=np.float64)
    b = _f64(bias) if bias is not None else None
    _load().orc_linear(_p(x, _f64p), n, k, _p(w, _f64p), m,
                       _p(b, _f64p) if b is not None else None, _p(y, _f64p))
    return y


def mlp(x, gate, up, down) -> np.ndarray:
    """Unsharded SwiGLU MLP: (SiLU(x gate^T) * (x up^T)) down^T."""
    x, gate, up, down = _f64(x), _f64(gate), _f64(up), _f64(down)
    n, h = x.shape
    f = gate.shape[0]
    assert gate.shape == (f, h) and up.shape == (f, h) and down.shape == (h, f)
    y = np.empty((n, h), dtype=np.float64)
    _load().orc_mlp(_p(x, _f64p), n, h, _p(gate, _f64p), _p(up, _f64p), f,
                    _p(down, _f64p), _p(y, _f64p))
    return y


def mlp_rank(x, gate, up, down, tp_rank, tp_size) -> np.ndarray:
    """Rank tp_rank's full-shape [n, h] partial, from the FULL weights."""
    x, gate, up, down = _f64(x), _f64(gate), _f64(up), _f64(down)
    n, h = x.shape
    f = gate.shape[0]
    assert f % tp_size == 0
    y = np.empty((n, h), dtype=np.float64)
    _load().orc_mlp_rank(_p(x, _f64p), n, h, _p(gate, _f64p), _p(up, _f64p), f,
                         _p(down, _f64p), tp_rank, tp_size, _p(y, _f64p))
    return y


def silu_mul(g, u) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    assert g.shape == u.shape
    out = np.empty(g.shape, dtype=np.float64)
    _load().orc_silu_mul(_p(g, _f64p), _p(u, _f64p), g.size, _p(out, _f64p))
    return out


# --- shard selection (bit-exact, any element type) -------------------------

def _es(a):
    return a.dtype.itemsize


def narrow(full, dim, start, length) -> np.ndarray:
    full = np.ascontiguousarray(full)
    rows, cols = full.shape
    shape = (length, cols) if dim == 0 else (rows, length)
    out = np.empty(shape, dtype=full.dtype)
    _check(_load().orc_narrow(full.ctypes.data, rows, cols, _es(full), dim, start,
                              length, out.ctypes.data), "narrow")
    return out


def shard(full, dim, tp_rank, tp_size) -> np.ndarray:
    full = np.ascontiguousarray(full)
    rows, cols = full.shape
    s = rows if dim == 0 else cols
    if s % tp_size:
        raise OracleError("shard: size not divisible by tp_size")
    shape = (rows // tp_size, cols) if dim == 0 else (rows, cols // tp_size)
    out = np.empty(shape, dtype=full.dtype)
    _check(_load().orc_shard(full.ctypes.data, rows, cols, _es(full), dim, tp_rank,
                             tp_size, out.ctypes.data), "shard")
    return out


def shard_gate_up(gate, up, tp_rank, tp_size) -> np.ndarray:
    gate, up = np.ascontiguousarray(gate), np.ascontiguousarray(up)
    assert gate.shape == up.shape and gate.dtype == up.dtype
    f, h = gate.shape
    out = np.empty((2 * (f // tp_size), h), dtype=gate.dtype)
    _check(_load().orc_shard_gate_up(gate.ctypes.data, up.ctypes.data, f, h, _es(gate),
                                     tp_rank, tp_size, out.ctypes.data), "shard_gate_up")
    return out


def kv_heads_for_rank(n_kv, tp_rank, tp_size):
    first, count = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().orc_kv_heads_for_rank(n_kv, tp_rank, tp_size, ctypes.byref(first),
                                         ctypes.byref(count)), "kv_heads_for_rank")
    return first.value, count.value


def shard_qkv(wq, wk, wv, n_q, n_kv, head_dim, tp_rank, tp_size) -> np.ndarray:
    wq, wk, wv = (np.ascontiguousarray(a) for a in (wq, wk, wv))
    h = wq.shape[1]
    _, kvc = kv_heads_for_rank(n_kv, tp_rank, tp_size)
    rows = (n_q // tp_size + 2 * kvc) * head_dim
    out = np.empty((rows, h), dtype=wq.dtype)
    _check(_load().orc_shard_qkv(wq.ctypes.data, wk.ctypes.data, wv.ctypes.data, n_q,
                                 n_kv, head_dim, h, _es(wq), tp_rank, tp_size,
                                 out.ctypes.data), "shard_qkv")
    return out


# --- checkpoint-style loaders ----------------------------------------------
# [NANO22] §3-§5 weight_loader applied to a full checkpoint tensor, in the
# order of [MINISGL] §8 (weight loading and sharding): select the rank's
# shard, convert the dtype, copy it into the local parameter (tp_oracle.c:
# orc_load_shard, orc_load_gate_up, orc_load_qkv).  Tensors are float32
# arrays or bfloat16 as uint16 bit arrays.

def _ldt(a):
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise OracleError("loader: float32 or bf16 bits (uint16) expected")


def load_shard(src, dim, tp_rank, tp_size, to_bf16) -> np.ndarray:
    """Column (dim 0, [NANO22] §3) or row (dim 1, §4) parallel loader: the
    rank's narrow(dim, r S/t, S/t) of the full tensor, then converted."""
    src = np.ascontiguousarray(src)
    rows, cols = src.shape
    s = rows if dim == 0 else cols
    if s % tp_size:
        raise OracleError("load_shard: size not divisible by tp_size")
    shape = (rows // tp_size, cols) if dim == 0 else (rows, cols // tp_size)
    out = np.empty(shape, dtype=np.uint16 if to_bf16 else np.float32)
    _check(_load().orc_load_shard(src.ctypes.data, _ldt(src), rows, cols, dim, tp_rank, tp_size,
                                  out.ctypes.data, _ldt(out)), "load_shard")
    return out


def load_gate_up(table, src, shard_id, tp_rank, tp_size) -> None:
    """[NANO22] §5 merged column-parallel loader, in place on the rank's
    [2 f/t, h] table: the projection's segment (first cut) receives
    src.chunk(t, 0)[tp_rank] (second cut), converted to the table's dtype."""
    src = np.ascontiguousarray(src)
    f, h = src.shape
    if f % tp_size:
        raise OracleError("load_gate_up: f not divisible by tp_size")
    if not table.flags["C_CONTIGUOUS"] or table.shape != (2 * (f // tp_size), h):
        raise OracleError("load_gate_up: table must be a contiguous [2 f/t, h] array")
    _check(_load().orc_load_gate_up(table.ctypes.data, _ldt(table), src.ctypes.data, _ldt(src), shard_id, f, h,
                                    tp_rank, tp_size), "load_gate_up")


def load_qkv(table, src, shard_id, n_q, n_kv, head_dim, tp_rank, tp_size) -> None:
    """[NANO22] §5 QKV loader, in place on the rank's table: segments q
    (n_q/t heads), k and v (the rank's KV heads each) in that order, with the
    KV replication of kv_heads_for_rank ([GUIDE62] §2.2)."""
    src = np.ascontiguousarray(src)
    if n_q % tp_size:
        raise OracleError("load_qkv: n_q not divisible by tp_size")
    if shard_id not in (0, 1, 2):
        raise OracleError("load_qkv: shard_id must be 0 (q), 1 (k) or 2 (v)")
    h = src.shape[1]
    _, kvc = kv_heads_for_rank(n_kv, tp_rank, tp_size)
    rows = (n_q // tp_size + 2 * kvc) * head_dim
    if not table.flags["C_CONTIGUOUS"] or table.shape != (rows, h):
        raise OracleError("load_qkv: table must be a contiguous [(n_q/t + 2 kvc) hd, h] array")
    if src.shape[0] != (n_q if shard_id == 0 else n_kv) * head_dim:
        raise OracleError("load_qkv: src has the wrong number of rows")
    _check(_load().orc_load_qkv(table.ctypes.data, _ldt(table), src.ctypes.data, _ldt(src), shard_id, n_q, n_kv,
                                head_dim, h, tp_rank, tp_size), "load_qkv")


# --- vocab parallel ----------------------------------------------------------

def vocab_range(vocab, tp_rank, tp_size):
    s, e = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().orc_vocab_range(vocab, tp_rank, tp_size, ctypes.byref(s),
                                   ctypes.byref(e)), "vocab_range")
    return s.value, e.value


def embed_full(ids, table) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    table = np.ascontiguousarray(table)
    V, h = table.shape
    out = np.empty((ids.size, h), dtype=table.dtype)
    _load().orc_embed_full(_p(ids, _i64p), ids.size, table.ctypes.data, V, h,
                           _es(table), out.ctypes.data)
    return out


def embed_rank(ids, table_shard, vocab, tp_rank, tp_size) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    table_shard = np.ascontiguousarray(table_shard)
    h = table_shard.shape[1]
    s, e = vocab_range(vocab, tp_rank, tp_size)
    if table_shard.shape[0] != e - s:
        raise OracleError("embed_rank: shard rows != end - start")
    out = np.empty((ids.size, h), dtype=table_shard.dtype)
    _check(_load().orc_embed_rank(_p(ids, _i64p), ids.size, table_shard.ctypes.data,
                                  vocab, h, _es(table_shard), tp_rank, tp_size,
                                  out.ctypes.data), "embed_rank")
    return out


def lm_head_rank(x, table_full, tp_rank, tp_size) -> np.ndarray:
    x, table_full = _f64(x), _f64(table_full)
    n, h = x.shape
    V = table_full.shape[0]
    s, e = vocab_range(V, tp_rank, tp_size)
    out = np.empty((n, e - s), dtype=np.float64)
    _check(_load().orc_lm_head_rank(_p(x, _f64p), n, h, _p(table_full, _f64p), V,
                                     tp_rank, tp_size, _p(out, _f64p)), "lm_head_rank")
    return out


# --- ring all-reduce -----------------------------------------------------------

def chunk_bounds(K, t, c):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _load().orc_chunk_bounds(K, t, c, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def ring_schedule(t, K):
    n = 2 * t * (t - 1)
    arr = (RingStep * max(n, 1))()
    got = _load().orc_ring_schedule(t, K, arr, max(n, 1))
    if got < 0:
        raise OracleError("ring_schedule: buffer too small")
    return [dict(phase=s.phase, step=s.step, src=s.src, dst=s.dst, chunk=s.chunk,
                 offset=s.offset, len=s.len) for s in arr[:got]]


def ring_traffic(t, K):
    sent = (ctypes.c_int64 * t)()
    recv = (ctypes.c_int64 * t)()
    rounds = ctypes.c_int()
    _check(_load().orc_ring_traffic(t, K, sent, recv, ctypes.byref(rounds)), "ring_traffic")
    return list(sent), list(recv), rounds.value


def ring_allreduce_f32(parts, lo=0, hi=None) -> np.ndarray:
    """Simulate the ring all-reduce on t fp32 rank buffers over window [lo, hi)."""
    parts = [np.ascontiguousarray(p, dtype=np.float32).reshape(-1) for p in parts]
    t = len(parts)
    K = parts[0].size
    assert all(p.size == K for p in parts)
    if hi is None:
        hi = K
    arr = (_f32p * t)(*[_p(p, _f32p) for p in parts])
    out = np.empty(hi - lo, dtype=np.float32)
    _check(_load().orc_ring_allreduce_f32(arr, t, K, lo, hi, _p(out, _f32p)),
           "ring_allreduce_f32")
    return out


def reduce_sum_f64(parts) -> np.ndarray:
    parts = [_f64(p).reshape(-1) for p in parts]
    t = len(parts)
    K = parts[0].size
    arr = (_f64p * t)(*[_p(p, _f64p) for p in parts])
    out = np.empty(K, dtype=np.float64)
    _load().orc_reduce_sum_f64(arr, t, K, _p(out, _f64p))
    return out


# --- sequence-parallel epilogue (reduce-scatter + residual add + RMSNorm) -------

def sp_rows(n, t, c):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _load().orc_sp_rows(n, t, c, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def rs_add_rmsnorm(parts, rank, residual, weight, eps, round_bf16):
    """Rank `rank`'s rows after the ring reduce-scatter of the t fp32 partials
    [n, h], plus the residual, then RMSNorm.  residual: the owned chunk's rows
    (fp32 values); returns (residual_out fp32 values, out fp64)."""
    parts = [np.ascontiguousarray(p, dtype=np.float32) for p in parts]
    t = len(parts)
    n, h = parts[0].shape
    lo, hi = sp_rows(n, t, (rank + 1) % t)
    res = np.ascontiguousarray(residual, dtype=np.float32).reshape(hi - lo, h)
    w = _f64(weight).reshape(h)
    arr = (_f32p * t)(*[_p(p, _f32p) for p in parts])
    res_out = np.empty((hi - lo, h), dtype=np.float32)
    out = np.empty((hi - lo, h), dtype=np.float64)
    _check(_load().orc_rs_add_rmsnorm(arr, t, rank, n, h, _p(res, _f32p), _p(w, _f64p), float(eps),
                                      1 if round_bf16 else 0, _p(res_out, _f32p), _p(out, _f64p)),
           "rs_add_rmsnorm")
    return res_out, out


# --- one-shot (rank-order) reduce; vocab logits gather + greedy argmax -----------

def reduce_rank_f32(parts) -> np.ndarray:
    """((0 + P_0) + P_1) + ... in fp32, the one-shot all-reduce's order."""
    parts = [np.ascontiguousarray(p, dtype=np.float32).reshape(-1) for p in parts]
    t = len(parts)
    K = parts[0].size
    arr = (_f32p * t)(*[_p(p, _f32p) for p in parts])
    out = np.empty(K, dtype=np.float32)
    _load().orc_reduce_rank_f32(arr, t, K, _p(out, _f32p))
    return out


def logits_gather_argmax(shards, vocab):
    """Concatenation of the t logits shards [n, end_r - start_r] along the
    vocabulary (fp64) and the first index of each row's maximum."""
    shards = [_f64(s) for s in shards]
    t = len(shards)
    n = shards[0].shape[0]
    arr = (_f64p * t)(*[_p(s, _f64p) for s in shards])
    full = np.empty((n, vocab), dtype=np.float64)
    am = np.empty(n, dtype=np.int64)
    _check(_load().orc_logits_gather_argmax(arr, t, n, vocab, _p(full, _f64p), _p(am, _i64p)),
           "logits_gather_argmax")
    return full, am


# --- head-parallel attention core -------------------------------------------------

def attention_rank(qkv, nq, nkv, head_dim, causal, rows=None) -> np.ndarray:
    """softmax(q k^T / sqrt(d) [causal mask]) v for the rank's nq query heads
    over its nkv KV heads (GQA), from the packed QKV projection output
    [n, (nq + 2 nkv) d]; rows: query rows to compute (default all)."""
    qkv = _f64(qkv)
    n = qkv.shape[0]
    assert qkv.shape[1] == (nq + 2 * nkv) * head_dim
    rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, nq * head_dim), dtype=np.float64)
    _check(_load().orc_attention_rank(_p(qkv, _f64p), n, nq, nkv, head_dim, 1 if causal else 0,
                                      _p(rows, _i64p), rows.size, _p(out, _f64p)), "attention_rank")
    return out
