"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, its host-only entry points agree with the oracle, and every
argument error is reported with a status and message before any launch.

No compute call reaches the GPU here.  The error-path cases pass dummy
(non-null, never dereferenced) pointers, so they run only where no GPU is
present: a validation slip must not turn into a launch with a bogus address.
"""
import ctypes
import os
import re

import pytest
import torch

import oracle
from rank_sharded_layer_amd import tpshard as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="dummy-pointer error paths run on a GPU-less host only")


def header_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"TP_API\s+[\w\s\*]*?\b(tp_\w+)\s*\(", src)))


def test_library_loads_and_exports_every_header_symbol():
    L = T.lib()
    syms = header_symbols()
    assert len(syms) >= 17
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(T.exported_names()) == syms
    assert T.tp_abi_version() == 1


def test_status_strings():
    L = T.lib()
    for k, v in T.STATUS_NAMES.items():
        assert L.tp_status_string(k).decode() == v


@pytest.mark.parametrize("V,t", [(151936, 2), (10, 2), (11, 4), (10, 8), (7, 3), (1, 1), (5, 64)])
def test_vocab_range_matches_oracle(V, t):
    for r in range(t):
        assert T.tp_vocab_range(V, r, t) == oracle.vocab_range(V, r, t)


@pytest.mark.parametrize("n_kv,t", [(8, 1), (8, 2), (8, 4), (8, 8), (8, 16), (2, 4), (2, 8), (1, 64)])
def test_kv_heads_match_oracle(n_kv, t):
    for r in range(t):
        assert T.tp_kv_heads_for_rank(n_kv, r, t) == oracle.kv_heads_for_rank(n_kv, r, t)


@pytest.mark.parametrize("t,K", [(1, 10), (2, 32768), (3, 1000), (4, 524288), (5, 7), (8, 67108864),
                                 (16, 67108864), (64, 1 << 20)])
def test_ring_schedule_matches_oracle(t, K):
    assert T.tp_ring_schedule(t, K) == oracle.ring_schedule(t, K)


def test_workspace_queries():
    # large-M shapes whose tiles fill whole rounds need no workspace
    # (8192 x 8192 in 256 x 256 tiles at one workgroup per CU: 1024 = 4 x 256)
    assert T.tp_linear_workspace_bytes(8192, 3584, 8192, torch.bfloat16) == 0
    # 8192 x 3584 (448 tiles of 256 x 256, under two rounds): 128 x 192 tiles,
    # 64 x 19 = 1216 = 4 x 256 + 192, whole K per tile, no workspace
    assert T.tp_linear_workspace_bytes(8192, 8192, 3584, torch.bfloat16) == 0
    # gated 8192 -> 1792 (gated products never take 128 x 192 tiles): 128 x 128
    # tiles of 64 act columns at two per CU, 64 x 28 = 1792 = 3 x 512 + 256, the
    # last 256 tiles cut into two K pieces of 4096 (fp32 128 x 128 partials)
    assert T.tp_gate_up_workspace_bytes(8192, 8192, 1792, torch.bfloat16) == 256 * 2 * 128 * 128 * 4
    # 896 gated tiles = 3 rounds + 128: the last 128 tiles are cut into two
    # K pieces each, whose fp32 256 x 256 partial tiles need a workspace
    assert T.tp_gate_up_workspace_bytes(8192, 8192, 3584, torch.bfloat16) == 128 * 2 * 256 * 256 * 4
    # long K, few columns (the QKV projection at TP=16): 256 x 192 tiles, K
    # split in two, two fp32 [M, N] partials
    assert T.tp_linear_workspace_bytes(8192, 8192, 768, torch.bfloat16) == 2 * 8192 * 768 * 4
    # decode shapes (register-streaming kernel): one fp32 [64 x 16] partial
    # tile per K slice of at most 1024 and 16-row weight block
    assert T.tp_gate_up_workspace_bytes(64, 8192, 7168, torch.bfloat16) == 8 * (14336 // 16) * 4096
    assert T.tp_linear_workspace_bytes(64, 7168, 8192, torch.bfloat16) == 7 * (8192 // 16) * 4096
    assert T.tp_linear_workspace_bytes(1, 4104, 2744, torch.bfloat16) == 5 * 172 * 4096
    assert T.tp_gate_up_workspace_bytes(64, 8192, 4096, torch.bfloat16) == 8 * (8192 // 16) * 4096
    # few output tiles: split-K partial sums
    assert T.tp_gate_up_workspace_bytes(64, 8192, 64, torch.bfloat16) > 0
    # few output tiles and a long K: split-K partial sums need a workspace
    assert T.tp_gate_up_workspace_bytes(80, 2048, 128, torch.bfloat16) > 0
    assert T.tp_linear_workspace_bytes(64, 7167, 8192, torch.bfloat16) > 0
    mlp = T.tp_mlp_workspace_bytes(80, 2048, 128, torch.bfloat16)
    act = 80 * 128 * 2
    assert mlp >= act + T.tp_gate_up_workspace_bytes(80, 2048, 128, torch.bfloat16)
    assert mlp >= act + T.tp_linear_workspace_bytes(80, 128, 2048, torch.bfloat16)
    assert T.tp_mlp_workspace_bytes(16, 1024, 1536, torch.float32) >= 16 * 1536 * 4


def _status(fn, *args):
    return fn(*args), T.lib().tp_last_error().decode()


DUMMY = ctypes.c_void_p(0x1000)
NULL = None


@no_gpu
def test_shard_errors():
    L = T.lib()
    st, msg = _status(L.tp_shard_weights, NULL, 4, 4, 1, 0, 0, 2, DUMMY, NULL)
    assert st == 1 and "null" in msg
    st, msg = _status(L.tp_shard_weights, DUMMY, 5, 4, 1, 0, 0, 2, DUMMY, NULL)
    assert st == 2 and "divisible" in msg
    st, msg = _status(L.tp_shard_weights, DUMMY, 4, 5, 1, 1, 0, 2, DUMMY, NULL)
    assert st == 2
    st, _ = _status(L.tp_shard_weights, DUMMY, 4, 4, 1, 2, 0, 2, DUMMY, NULL)
    assert st == 1                    # dim not 0/1
    st, _ = _status(L.tp_shard_weights, DUMMY, 4, 4, 1, 0, 2, 2, DUMMY, NULL)
    assert st == 1                    # rank >= size
    st, _ = _status(L.tp_shard_weights, DUMMY, 4, 4, 1, 0, -1, 2, DUMMY, NULL)
    assert st == 1
    st, _ = _status(L.tp_shard_weights, DUMMY, 4, 4, 1, 0, 0, 65, DUMMY, NULL)
    assert st == 1                    # t > 64
    st, _ = _status(L.tp_shard_weights, DUMMY, 4, 4, 7, 0, 0, 2, DUMMY, NULL)
    assert st == 3                    # dtype
    st, _ = _status(L.tp_shard_gate_up, DUMMY, DUMMY, 6, 4, 1, 0, 4, DUMMY, NULL)
    assert st == 2
    st, _ = _status(L.tp_shard_qkv, DUMMY, DUMMY, DUMMY, 6, 2, 4, 8, 1, 0, 4, DUMMY, NULL)
    assert st == 2                    # n_q 6 not divisible by 4
    st, _ = _status(L.tp_shard_qkv, DUMMY, DUMMY, DUMMY, 12, 8, 4, 8, 1, 0, 3, DUMMY, NULL)
    assert st == 2                    # 8 kv heads over 3 ranks
    st, _ = _status(L.tp_shard_qkv, DUMMY, DUMMY, DUMMY, 12, 4, 4, 8, 1, 0, 6, DUMMY, NULL)
    assert st == 2                    # 6 ranks, 4 kv heads: neither divides


@no_gpu
def test_gemm_errors():
    L = T.lib()
    st, _ = _status(L.tp_linear_rank_forward, NULL, 4, 4, DUMMY, 4, NULL, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 1
    st, _ = _status(L.tp_linear_rank_forward, DUMMY, 0, 4, DUMMY, 4, NULL, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 1                    # n = 0
    st, _ = _status(L.tp_linear_rank_forward, DUMMY, 4, 4, DUMMY, 4, NULL, 0, DUMMY, 1, NULL, 0, NULL)
    assert st == 3                    # f32 -> bf16 unsupported
    st, msg = _status(L.tp_linear_rank_forward, DUMMY, 64, 7167, DUMMY, 8192, NULL, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 6 and "workspace" in msg   # split-K shape without workspace
    st, _ = _status(L.tp_gate_up_act_rank, DUMMY, 80, 2048, DUMMY, 128, 1, DUMMY, NULL, 0, NULL)
    assert st == 6
    st, _ = _status(L.tp_mlp_rank_forward, DUMMY, 4, 8, DUMMY, DUMMY, 6, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 6
    st, msg = _status(L.tp_mlp_rank_forward, DUMMY, 4, 8, DUMMY, DUMMY, 6, 1, DUMMY, 1,
                      ctypes.c_void_p(0x1001), 1 << 20, NULL)
    assert st == 4 and "aligned" in msg   # TP_EALIGN: workspace not 256-byte aligned
    st, msg = _status(L.tp_linear_rank_forward, DUMMY, 64, 7167, DUMMY, 8192, NULL, 1, DUMMY, 1,
                      ctypes.c_void_p(0x1008), 1 << 30, NULL)
    assert st == 4 and "16-byte" in msg   # split-K workspace not 16-byte aligned
    st, _ = _status(L.tp_lm_head_rank, DUMMY, 4, 8, NULL, 16, 1, DUMMY, 0, NULL, 0, NULL)
    assert st == 1


@no_gpu
def test_gemm_32bit_offset_guard():
    """The bf16 kernels address a tile's operand rows with 32-bit byte
    offsets: K beyond 2^22, or a fused gate_up table whose up rows lie 2 GiB
    or more past its gate rows, is rejected with TP_ESHAPE before any launch
    (the fp32 kernels index with 64 bits and take these shapes)."""
    L = T.lib()
    sz = ctypes.c_size_t()
    big_k = 1 << 22
    st, msg = _status(L.tp_linear_rank_forward, DUMMY, 4, big_k, DUMMY, 16, NULL, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 2 and "reduction size" in msg
    assert L.tp_linear_workspace_bytes(4, big_k, 16, 1, ctypes.byref(sz)) == 2
    assert L.tp_linear_workspace_bytes(4, big_k - 8, 16, 1, ctypes.byref(sz)) == 0
    assert L.tp_linear_workspace_bytes(4, big_k, 16, 0, ctypes.byref(sz)) == 0      # fp32: no limit
    st, _ = _status(L.tp_lm_head_rank, DUMMY, 4, big_k, DUMMY, 16, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 2
    # gated: (f_local + 256) * h * 2 must stay under 2^31
    h = 8192
    f_ok = (1 << 31) // (2 * h) - 257
    f_bad = f_ok + 1
    assert L.tp_gate_up_workspace_bytes(64, h, f_ok, 1, ctypes.byref(sz)) == 0
    assert L.tp_gate_up_workspace_bytes(64, h, f_bad, 1, ctypes.byref(sz)) == 2
    st, msg = _status(L.tp_gate_up_act_rank, DUMMY, 64, h, DUMMY, f_bad, 1, DUMMY, NULL, 0, NULL)
    assert st == 2 and "gate_up" in msg
    st, _ = _status(L.tp_mlp_rank_forward, DUMMY, 64, h, DUMMY, DUMMY, f_bad, 1, DUMMY, 1, NULL, 0, NULL)
    assert st == 2
    assert L.tp_mlp_workspace_bytes(64, h, f_bad, 1, ctypes.byref(sz)) == 2
    # a 405B-shaped MLP (h 16384, f 53248) fits even unsharded: its up rows
    # start 1.74 GB after its gate rows
    assert L.tp_mlp_workspace_bytes(64, 16384, 53248, 1, ctypes.byref(sz)) == 0
    assert L.tp_mlp_workspace_bytes(64, 16384, 65536, 1, ctypes.byref(sz)) == 2


@no_gpu
def test_attention_alignment_errors():
    """Every alignment rejection returns TP_EALIGN: qkv / out and the
    workspace of the attention core must be 16-byte aligned."""
    L = T.lib()
    sz = ctypes.c_size_t()
    assert L.tp_attention_workspace_bytes(8192, 4, 1, 128, 1, 1, ctypes.byref(sz)) == 0 and sz.value > 0
    ws = ctypes.c_void_p(0x40000000)
    st, msg = _status(L.tp_attention_rank, ctypes.c_void_p(0x1008), 8192, 4, 1, 128, 1, 1, ctypes.c_void_p(1 << 36),
                      ws, sz.value, NULL)
    assert st == 4 and "aligned" in msg
    st, msg = _status(L.tp_attention_rank, ctypes.c_void_p(1 << 34), 8192, 4, 1, 128, 1, 1, ctypes.c_void_p(1 << 36),
                      ctypes.c_void_p(0x40000004), sz.value, NULL)
    assert st == 4 and "workspace" in msg
    st, _ = _status(L.tp_attention_rank, ctypes.c_void_p(1 << 34), 8192, 4, 1, 128, 1, 1, ctypes.c_void_p(1 << 36),
                    ws, sz.value - 16, NULL)
    assert st == 6


@no_gpu
def test_reduce_and_vocab_errors():
    L = T.lib()
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    st, _ = _status(L.tp_partial_reduce, arr, 0, 8, 1, DUMMY, 1, 0, NULL)
    assert st == 1                    # t = 0
    st, _ = _status(L.tp_partial_reduce, arr, 65, 8, 1, DUMMY, 1, 0, NULL)
    assert st == 1                    # t > 64
    arr2 = (ctypes.c_void_p * 2)(0x1000, None)
    st, msg = _status(L.tp_partial_reduce, arr2, 2, 8, 1, DUMMY, 1, 0, NULL)
    assert st == 1 and "partials[1]" in msg
    st, _ = _status(L.tp_partial_reduce, arr, 2, 8, 0, DUMMY, 1, 0, NULL)
    assert st == 3
    st, _ = _status(L.tp_partial_reduce, arr, 2, 8, 1, DUMMY, 1, 5, NULL)
    assert st == 1                    # unknown order
    st, _ = _status(L.tp_vocab_embed_rank, NULL, 4, DUMMY, 10, 4, 0, 2, 1, DUMMY, NULL)
    assert st == 1
    st, _ = _status(L.tp_vocab_embed_rank, DUMMY, 4, NULL, 10, 4, 0, 2, 1, DUMMY, NULL)
    assert st == 1                    # null table for a non-empty shard
    st, _ = _status(L.tp_vocab_embed_rank, DUMMY, 4, DUMMY, 10, 4, 3, 2, 1, DUMMY, NULL)
    assert st == 1
    first, count = ctypes.c_int64(), ctypes.c_int64()
    assert L.tp_kv_heads_for_rank(0, 0, 1, ctypes.byref(first), ctypes.byref(count)) == 1
    steps = (T.RingStep * 2)()
    n = ctypes.c_int()
    assert L.tp_ring_schedule(3, 9, steps, 2, ctypes.byref(n)) == 2   # room for 2 < 12
    assert T.tp_last_error() != ""
    # success clears the message
    assert L.tp_ring_schedule(1, 9, steps, 2, ctypes.byref(n)) == 0
    assert T.tp_last_error() == ""


def test_binding_rejects_host_tensors():
    with pytest.raises(ValueError):
        T.tp_partial_reduce([torch.zeros(8), torch.zeros(8)])
    with pytest.raises(ValueError):
        T.tp_shard_weights(torch.zeros(4, 4), 0, 0, 2)


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("n", [0, 5, 13, 8192])
def test_sp_rows_match_oracle_ring_owner(t, n):
    """The rows a rank holds after the reduce-scatter: the chunk the oracle's
    ring schedule completes on that rank, cut as whole token rows."""
    sched = oracle.ring_schedule(t, n)
    owner = {s["dst"]: s["chunk"] for s in sched if s["phase"] == 0 and s["step"] == t - 2}
    for r in range(t):
        c = owner.get(r, 0)            # t = 1: the single rank holds chunk 0
        assert T.tp_sp_rows(n, r, t) == oracle.sp_rows(n, t, c)


@no_gpu
def test_rs_add_rmsnorm_errors():
    L = T.lib()
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    ok_args = dict(t=2, rank=0, n=8, h=16, dt=1, res=DUMMY, w=DUMMY, eps=1e-5, ro=ctypes.c_void_p(0x3000),
                   out=ctypes.c_void_p(0x4000))

    def call(**kw):
        a = dict(ok_args, **kw)
        return _status(L.tp_rs_add_rmsnorm, kw.get("arr", arr), a["t"], a["rank"], a["n"], a["h"], a["dt"], a["res"],
                       a["w"], a["eps"], a["ro"], a["out"], NULL)

    assert call(t=0)[0] == 1
    assert call(rank=2)[0] == 1                      # rank outside [0, t)
    assert call(h=0)[0] == 1
    assert call(dt=7)[0] == 3
    assert call(eps=-1.0)[0] == 1
    assert call(eps=float("nan"))[0] == 1
    assert call(w=NULL)[0] == 1
    st, msg = call(out=ctypes.c_void_p(0x3000))
    assert st == 1 and "alias" in msg                # out is residual_out
    st, msg = call(ro=ctypes.c_void_p(0x2000))
    assert st == 1 and "partials[1]" in msg          # residual_out is a partial
    st, msg = call(arr=(ctypes.c_void_p * 2)(0x1000, None))
    assert st == 1 and "partials[1]" in msg
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    assert L.tp_sp_rows(8, 3, 2, ctypes.byref(lo), ctypes.byref(hi)) == 1


@no_gpu
def test_load_errors():
    L = T.lib()
    sz = ctypes.c_size_t()
    assert L.tp_load_staging_bytes(4, 6, 0, 1, ctypes.byref(sz)) == 0 and sz.value == 256   # 4*6 fp32, 256-aligned
    assert L.tp_load_staging_bytes(4, 6, 1, 1, ctypes.byref(sz)) == 0 and sz.value == 0     # same dtype: none
    st, _ = _status(L.tp_load_staging_bytes, 4, 6, 9, 1, ctypes.byref(sz))
    assert st == 3
    # tp_load_shard(src, src_dt, rows, cols, dim, rank, t, dst, dst_dt, staging, bytes, stream)
    st, msg = _status(L.tp_load_shard, NULL, 0, 4, 4, 0, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 1 and "null" in msg
    st, _ = _status(L.tp_load_shard, DUMMY, 0, 4, 4, 2, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 1                    # dim
    st, msg = _status(L.tp_load_shard, DUMMY, 0, 5, 4, 0, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 2 and "divisible" in msg
    st, _ = _status(L.tp_load_shard, DUMMY, 5, 4, 4, 0, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 3                    # source dtype
    st, _ = _status(L.tp_load_shard, DUMMY, 0, 4, 4, 0, 3, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 1                    # rank
    st, msg = _status(L.tp_load_shard, DUMMY, 0, 64, 64, 0, 0, 2, DUMMY, 1, DUMMY, 1024, NULL)
    assert st == 6 and "staging" in msg   # 32 x 64 fp32 = 8 KiB needed
    st, msg = _status(L.tp_load_shard, DUMMY, 0, 64, 64, 0, 0, 2, DUMMY, 1, NULL, 0, NULL)
    assert st == 6
    st, msg = _status(L.tp_load_shard, DUMMY, 0, 64, 64, 0, 0, 2, DUMMY, 1, ctypes.c_void_p(0x1008), 1 << 20, NULL)
    assert st == 4 and "aligned" in msg
    # tp_load_gate_up(src, src_dt, shard_id, f, h, rank, t, dst, dst_dt, staging, bytes, stream)
    st, _ = _status(L.tp_load_gate_up, DUMMY, 0, 2, 8, 4, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 1                    # shard id
    st, _ = _status(L.tp_load_gate_up, DUMMY, 0, 0, 6, 4, 0, 4, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 2                    # 6 rows over 4 ranks
    # tp_load_qkv(src, src_dt, shard_id, n_q, n_kv, hd, h, rank, t, dst, dst_dt, staging, bytes, stream)
    st, _ = _status(L.tp_load_qkv, DUMMY, 0, 3, 8, 2, 4, 8, 0, 2, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 1                    # shard id
    st, _ = _status(L.tp_load_qkv, DUMMY, 0, 1, 12, 8, 4, 8, 0, 3, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 2                    # 8 kv heads over 3 ranks
    st, _ = _status(L.tp_load_qkv, DUMMY, 0, 0, 6, 2, 4, 8, 0, 4, DUMMY, 1, DUMMY, 4096, NULL)
    assert st == 2                    # n_q 6 over 4 ranks


def test_last_error_is_per_thread():
    """tp_last_error() keeps each host thread's own message: a failure on one
    thread neither overwrites nor clears another thread's, and a successful
    host-only call clears only the caller's."""
    import threading
    L = T.lib()
    assert L.tp_vocab_range(10, 5, 2, ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_int64())) != 0
    mine = L.tp_last_error().decode()
    assert mine
    seen = {}

    def other():
        seen["before"] = L.tp_last_error().decode()
        st = L.tp_kv_heads_for_rank(3, 0, 2, ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_int64()))
        seen["status"] = st
        seen["after"] = L.tp_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["before"] == ""
    assert seen["status"] != 0 and seen["after"] and seen["after"] != mine
    assert L.tp_last_error().decode() == mine
    assert L.tp_vocab_range(10, 1, 2, ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_int64())) == 0
    assert L.tp_last_error().decode() == ""
