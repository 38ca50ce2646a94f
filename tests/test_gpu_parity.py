"""GPU parity: the HIP library against the fp64 oracle on small and ragged
shapes (several tiles plus ragged tails, edge ids, degenerate cases).

Bar: bit-exact for shard selection, embedding masking/indexing and the ring
reduce (against the oracle's fp32 ring simulation, rounded once); relative
Frobenius error <= 1e-5 (fp32) / 1e-2 (bf16 inputs, fp32 accumulation)
against the fp64 oracle for everything with products.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from rank_sharded_layer_amd import tpshard as T
from tests.helpers import TOL, bits, relf, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

DTYPES = [torch.float32, torch.bfloat16]


def rnd(shape, std, seed, dtype):
    return synth.normal(shape, std, seed, dtype).to(DEV)


# --------------------------------------------------------------------------
# shard selection (a1): bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,cols,t", [(8, 12, 2), (12, 8, 3), (64, 96, 4), (16, 40, 8),
                                         (6, 6, 1), (24, 3, 3), (5, 7, 1)])
@pytest.mark.parametrize("dim", [0, 1])
def test_shard_weights_bit_exact(dtype, rows, cols, t, dim):
    if (rows if dim == 0 else cols) % t:
        pytest.skip("not divisible")
    full = rnd((rows, cols), 1.0, 1000 + rows * cols + t, dtype)
    ref_full = bits(full)
    for r in range(t):
        got = T.tp_shard_weights(full, dim, r, t)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), oracle.shard(ref_full, dim, r, t))


def test_shard_column_worked_example_on_gpu():
    full = torch.arange(4.0).reshape(4, 1).repeat(1, 3).to(DEV)
    assert T.tp_shard_weights(full, 0, 0, 2)[:, 0].tolist() == [0.0, 1.0]
    assert T.tp_shard_weights(full, 0, 1, 2)[:, 0].tolist() == [2.0, 3.0]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("f,h,t", [(8, 3, 2), (12, 16, 3), (64, 40, 4), (24, 8, 8)])
def test_shard_gate_up_bit_exact(dtype, f, h, t):
    gate = rnd((f, h), 1.0, 11 + f, dtype)
    up = rnd((f, h), 1.0, 12 + f, dtype)
    for r in range(t):
        got = T.tp_shard_gate_up(gate, up, r, t)
        assert np.array_equal(bits(got), oracle.shard_gate_up(bits(gate), bits(up), r, t))


@pytest.mark.parametrize("n_q,n_kv,hd,h,t", [(4, 2, 2, 3, 2), (8, 2, 4, 16, 4), (8, 2, 4, 16, 8),
                                             (64, 8, 8, 16, 16), (16, 8, 4, 8, 2)])
def test_shard_qkv_bit_exact(n_q, n_kv, hd, h, t):
    wq = rnd((n_q * hd, h), 1.0, 21, torch.bfloat16)
    wk = rnd((n_kv * hd, h), 1.0, 22, torch.bfloat16)
    wv = rnd((n_kv * hd, h), 1.0, 23, torch.bfloat16)
    for r in range(t):
        got = T.tp_shard_qkv(wq, wk, wv, n_q, n_kv, hd, r, t)
        ref = oracle.shard_qkv(bits(wq), bits(wk), bits(wv), n_q, n_kv, hd, r, t)
        assert np.array_equal(bits(got), ref)


# --------------------------------------------------------------------------
# ring-order reduce (a5): bit-exact against the oracle's ring simulation
# --------------------------------------------------------------------------

def oracle_reduce_bits(parts, out_dtype):
    f32 = [to_f64(p).astype(np.float32) for p in parts]   # exact: bf16/fp32 -> fp32
    s = oracle.ring_allreduce_f32(f32)
    if out_dtype == torch.bfloat16:
        return oracle.f32_to_bf16_bits(s)
    return s.view(np.uint32)


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32)])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("K", [1, 7, 64, 8 * 1000 + 5, 65536 * 3 + 11])
def test_partial_reduce_ring_order_bit_exact(in_dt, out_dt, t, K):
    parts = [rnd((K,), 1.0, 500 + 31 * r + K, in_dt) for r in range(t)]
    got = T.tp_partial_reduce(parts, out_dtype=out_dt)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), oracle_reduce_bits(parts, out_dt))


@pytest.mark.parametrize("t", [2, 4, 8, 16])
def test_partial_reduce_many_workgroups_per_chunk(t):
    """Chunks spanning many workgroups, with a remainder after the unrolled
    passes and unaligned chunk bounds (K odd)."""
    K = 1_000_003
    parts = [rnd((K,), 1.0, 1300 + 17 * r + t, torch.bfloat16) for r in range(t)]
    got = T.tp_partial_reduce(parts)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), oracle_reduce_bits(parts, torch.bfloat16))


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32])
def test_partial_reduce_unaligned_buffers(in_dt):
    t, K = 3, 4099
    bufs = [rnd((K + 1,), 1.0, 900 + r, in_dt) for r in range(t)]
    parts = [b[1:] for b in bufs]          # contiguous views, misaligned by one element
    out_buf = torch.empty(K + 1, dtype=in_dt, device=DEV)
    got = T.tp_partial_reduce(parts, out=out_buf[1:])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), oracle_reduce_bits(parts, in_dt))


def test_partial_reduce_order_pin_on_gpu():
    """(P_i + P_{i+1}) + P_{i+2} for element i of chunk i: 1 + 2^-24 ties."""
    e = 2.0 ** -24
    P0 = torch.tensor([e, 1.0, e], device=DEV)
    P1 = torch.tensor([1.0, e, e], device=DEV)
    P2 = torch.tensor([e, e, 1.0], device=DEV)
    out = T.tp_partial_reduce([P0, P1, P2])
    assert out.tolist() == [1.0, 1.0 + 2.0 ** -23, 1.0]


def test_partial_reduce_is_deterministic():
    parts = [rnd((1 << 20,), 1.0, 77 + r, torch.bfloat16) for r in range(8)]
    a = bits(T.tp_partial_reduce(parts))
    b = bits(T.tp_partial_reduce(parts))
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# vocab-parallel embedding (a6): bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("V", [10, 11])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("h", [4, 3, 64])
def test_vocab_embed_edges_bit_exact(dtype, V, t, h):
    table = rnd((V, h), 0.02, 300 + V * h, dtype)
    ids_set = {-1, 0, V - 1, V, V + 7, -(1 << 40)}
    for r in range(t):
        s, e = T.tp_vocab_range(V, r, t)
        ids_set |= {s - 1, s, e - 1, e}
    ids = torch.tensor(sorted(ids_set), dtype=torch.int64, device=DEV)
    outs = []
    for r in range(t):
        s, e = T.tp_vocab_range(V, r, t)
        shard = table[s:e].contiguous()
        got = T.tp_vocab_embed_rank(ids, shard, V, r, t)
        ref = oracle.embed_rank(ids.cpu().numpy(), bits(shard).reshape(e - s, h), V, r, t)
        assert np.array_equal(bits(got), ref)
        outs.append(got)
    total = T.tp_partial_reduce(outs)
    full = oracle.embed_full(ids.cpu().numpy(), bits(table))
    full64 = oracle.bf16_bits_to_f64(full) if dtype == torch.bfloat16 else full.view(np.float32).astype(np.float64)
    # values equal (a -0.0 table entry would come back as +0.0 from the sum)
    assert np.array_equal(to_f64(total), full64)


def test_vocab_embed_demo_from_pages():
    """vLLM source analysis 13 §2.4.1 demo: vocab 10, ids [[1,6],[3,8]], 2 ranks."""
    V, h = 10, 4
    table = rnd((V, h), 1.0, 42, torch.float32)
    ids = torch.tensor([1, 6, 3, 8], dtype=torch.int64, device=DEV)
    o0 = T.tp_vocab_embed_rank(ids, table[:5].contiguous(), V, 0, 2)
    o1 = T.tp_vocab_embed_rank(ids, table[5:].contiguous(), V, 1, 2)
    assert (o0.abs().sum(1) > 0).tolist() == [True, False, True, False]
    assert (o1.abs().sum(1) > 0).tolist() == [False, True, False, True]
    assert torch.equal(T.tp_partial_reduce([o0, o1]), table[ids])


# --------------------------------------------------------------------------
# GEMMs (a2-a4, a7, a8)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_row_parallel_worked_example_exact(dtype):
    """Nano-vLLM walkthrough 22 §4: partials [[13,31]] (rank 0, with bias) and
    [[7,15]]; their sum [[20,46]].  Small integers are exact in bf16/fp32."""
    W = torch.tensor([[1.0, 2, 3, 4], [5.0, 6, 7, 8]], dtype=dtype, device=DEV)
    b = torch.tensor([10.0, 20.0], dtype=dtype, device=DEV)
    x = torch.tensor([[1.0, 1, 1, 1]], dtype=dtype, device=DEV)
    parts = []
    for r in range(2):
        w = T.tp_shard_weights(W, 1, r, 2)
        xr = T.tp_shard_weights(x, 1, r, 2)
        parts.append(T.tp_linear_rank_forward(xr, w, bias=b if r == 0 else None, out_dtype=torch.float32
                                              if dtype == torch.bfloat16 else dtype))
    assert parts[0].tolist() == [[13.0, 31.0]]
    assert parts[1].tolist() == [[7.0, 15.0]]
    assert T.tp_partial_reduce(parts).tolist() == [[20.0, 46.0]]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k,m", [(1, 8, 12), (3, 16, 7), (5, 24, 300), (37, 1000, 129),
                                   (130, 64, 256), (64, 3, 5), (200, 520, 72), (257, 128, 390)])
def test_linear_matches_oracle(dtype, n, k, m):
    x = rnd((n, k), 1.0, 40 + n, dtype)
    w = rnd((m, k), 0.02, 41 + m, dtype)
    b = rnd((m,), 0.02, 42 + m, dtype)
    for bias in (None, b):
        for out_dt in ([torch.float32] if dtype == torch.float32 else [torch.bfloat16, torch.float32]):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            ref = oracle.linear(to_f64(x), to_f64(w), to_f64(bias) if bias is not None else None)
            assert relf(to_f64(y), ref) <= TOL[dtype], (n, k, m, out_dt)


@pytest.mark.parametrize("dtype", DTYPES)
def test_linear_one_hot_rows_gather_exactly(dtype):
    n, k, m = 40, 96, 200
    idx = torch.arange(n, device=DEV) * 7 % k
    x = torch.zeros((n, k), dtype=dtype, device=DEV)
    x[torch.arange(n, device=DEV), idx] = 1.0
    w = rnd((m, k), 0.02, 55, dtype)
    y = T.tp_linear_rank_forward(x, w, out_dtype=dtype)
    assert torch.equal(y, w.t()[idx].contiguous())


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,h,f_local", [(1, 8, 6), (3, 16, 12), (5, 64, 96), (70, 128, 200),
                                         (130, 1024, 96), (16, 1024, 1536), (64, 64, 33)])
def test_gate_up_act_matches_oracle(dtype, n, h, f_local):
    x = rnd((n, h), 1.0, 60 + n, dtype)
    wgu = rnd((2 * f_local, h), 0.1, 61 + f_local, dtype)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg = to_f64(x)
    W = to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:f_local]), oracle.linear(xg, W[f_local:]))
    assert relf(to_f64(act), ref) <= TOL[dtype]


def test_gate_up_zero_gate_gives_exact_zero():
    n, h, fl = 33, 64, 40
    x = rnd((n, h), 1.0, 70, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.1, 71, torch.bfloat16)
    wgu[:fl] = 0
    act = T.tp_gate_up_act_rank(x, wgu)
    assert torch.all(act == 0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("t", [1, 2, 3, 4])
@pytest.mark.parametrize("n,h,f", [(1, 8, 12), (3, 16, 24), (5, 8, 24), (5, 16, 12)])
def test_mlp_brute_force_tiny(dtype, t, n, h, f):
    """Brute force on tiny shapes: each rank's partial against the oracle's
    rank partial, and the ring-order sum of the partials against the
    unsharded fp64 MLP."""
    if f % t:
        pytest.skip("f not divisible by t")
    x = rnd((n, h), 1.0, 80 + n * h, dtype)
    gate = rnd((f, h), 0.3, 81, dtype)
    up = rnd((f, h), 0.3, 82, dtype)
    down = rnd((h, f), 0.3, 83, dtype)
    parts = []
    for r in range(t):
        wgu = T.tp_shard_gate_up(gate, up, r, t)
        wd = T.tp_shard_weights(down, 1, r, t)
        parts.append(T.tp_mlp_rank_forward(x, wgu, wd))
        ref_r = oracle.mlp_rank(to_f64(x), to_f64(gate), to_f64(up), to_f64(down), r, t)
        assert relf(to_f64(parts[-1]), ref_r) <= TOL[dtype]
    y = T.tp_partial_reduce(parts)
    ref = oracle.mlp(to_f64(x), to_f64(gate), to_f64(up), to_f64(down))
    assert relf(to_f64(y), ref) <= TOL[dtype]


def test_mlp_t1_is_unsharded_and_reduce_is_copy():
    n, h, f = 9, 32, 48
    x = rnd((n, h), 1.0, 90, torch.bfloat16)
    gate, up = rnd((f, h), 0.2, 91, torch.bfloat16), rnd((f, h), 0.2, 92, torch.bfloat16)
    down = rnd((h, f), 0.2, 93, torch.bfloat16)
    wgu = T.tp_shard_gate_up(gate, up, 0, 1)
    assert torch.equal(wgu, torch.cat([gate, up]))
    p = T.tp_mlp_rank_forward(x, wgu, T.tp_shard_weights(down, 1, 0, 1))
    assert torch.equal(T.tp_partial_reduce([p]), p)


def test_wrong_dim_shard_fails_parity():
    """Sharding gate/up along the wrong dim (a row split of the first GEMM)
    and applying SiLU before the reduce must NOT match the unsharded MLP."""
    n, h, f, t = 8, 64, 64, 2
    x = rnd((n, h), 1.0, 95, torch.float32)
    gate, up = rnd((f, h), 0.3, 96, torch.float32), rnd((f, h), 0.3, 97, torch.float32)
    down = rnd((h, f), 0.3, 98, torch.float32)
    parts = []
    for r in range(t):
        xr = T.tp_shard_weights(x, 1, r, t)
        wgu = torch.cat([T.tp_shard_weights(gate, 1, r, t), T.tp_shard_weights(up, 1, r, t)])
        act = T.tp_gate_up_act_rank(xr, wgu)
        parts.append(T.tp_linear_rank_forward(act, down))
    y = T.tp_partial_reduce(parts)
    ref = oracle.mlp(to_f64(x), to_f64(gate), to_f64(up), to_f64(down))
    assert relf(to_f64(y), ref) > 0.05


@pytest.mark.parametrize("t", [1, 2, 3])
def test_lm_head_concat_matches_oracle(t):
    V, h, n = 1000, 64, 37
    table = rnd((V, h), 0.02, 120, torch.bfloat16)
    x = rnd((n, h), 1.0, 121, torch.bfloat16)
    cat = []
    for r in range(t):
        s, e = T.tp_vocab_range(V, r, t)
        cat.append(T.tp_lm_head_rank(x, table[s:e].contiguous()))
    got = torch.cat(cat, dim=1)
    ref = np.concatenate([oracle.lm_head_rank(to_f64(x), to_f64(table), r, t) for r in range(t)], axis=1)
    assert relf(to_f64(got), ref) <= TOL[torch.bfloat16]


def test_split_k_path_matches_oracle():
    """Few output tiles with a long K take the split-K path (fp32 partials in
    the workspace, reduced in split order); same bar as the direct path."""
    n, h, fl = 80, 2048, 256
    assert T.tp_gate_up_workspace_bytes(n, h, fl, torch.bfloat16) > 0
    x = rnd((n, h), 1.0, 130, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.02, 131, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    assert relf(to_f64(act), ref) <= 1e-2
    wd = rnd((h, fl), 0.02, 132, torch.bfloat16)
    assert T.tp_linear_workspace_bytes(n, fl, h, torch.bfloat16) >= 0
    p = T.tp_mlp_rank_forward(x, wgu, wd)
    Wg, Wu = W[:fl], W[fl:]
    ref_p = oracle.linear(oracle.silu_mul(oracle.linear(xg, Wg), oracle.linear(xg, Wu)), to_f64(wd))
    assert relf(to_f64(p), ref_p) <= 1e-2


@pytest.mark.parametrize("n", [1, 7, 33, 64])
@pytest.mark.parametrize("k,m", [(64, 32), (200, 100), (1024, 96), (1000, 64), (4096, 160)])
@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float32])
def test_decode_linear_matches_oracle(n, k, m, out_dt):
    """Token counts <= 64 (the decode path; split-K where the shape has few
    output tiles)."""
    x = rnd((n, k), 1.0, 140 + n, torch.bfloat16)
    w = rnd((m, k), 0.05, 141 + m, torch.bfloat16)
    b = rnd((m,), 0.05, 142, torch.bfloat16)
    for bias in (None, b):
        y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
        ref = oracle.linear(to_f64(x), to_f64(w), to_f64(bias) if bias is not None else None)
        assert relf(to_f64(y), ref) <= 1e-2


@pytest.mark.parametrize("n", [1, 5, 64])
@pytest.mark.parametrize("h,fl", [(64, 32), (1000, 48), (2048, 96), (8192, 64)])
def test_decode_gate_up_matches_oracle(n, h, fl):
    x = rnd((n, h), 1.0, 150 + n, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.05, 151 + fl, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    assert relf(to_f64(act), ref) <= 1e-2


def test_decode_is_deterministic():
    x = rnd((64, 4096), 1.0, 160, torch.bfloat16)
    w = rnd((256, 4096), 0.05, 161, torch.bfloat16)
    a = bits(T.tp_linear_rank_forward(x, w))
    b = bits(T.tp_linear_rank_forward(x, w))
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# balanced last round: the tiles of a partial last round are cut along K,
# their fp32 pieces added in piece order by a fix-up pass
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,m", [(1024, 2600, 11342), (4900, 2600, 8100)])
def test_tail_split_linear_matches_oracle(n, k, m):
    """Tile counts one full round of resident workgroups plus a part round
    (8 x 89 tiles of 128 at 2 per CU: 512 + 200; 20 x 32 tiles of 256 at
    one per CU: 512 + 128); the part round's tiles are cut in two K pieces,
    the last of them ending inside a 64-wide K tile."""
    assert T.tp_linear_workspace_bytes(n, k, m, torch.bfloat16) > 0
    x = rnd((n, k), 1.0, 170, torch.bfloat16)
    w = rnd((m, k), 0.02, 171, torch.bfloat16)
    b = rnd((m,), 0.02, 172, torch.bfloat16)
    rows = sorted(set(synth.sample_rows(n, 16, 173) + list(range(n - 8, n))))
    for bias in (None, b):
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            ref = oracle.linear(to_f64(x[rows]), to_f64(w), to_f64(bias) if bias is not None else None)
            got = to_f64(y[rows])
            assert relf(got, ref) <= 1e-2, (bias is None, out_dt)
            # the last tile columns (cut tiles), on their own
            assert relf(got[:, -300:], ref[:, -300:]) <= 1e-2


@pytest.mark.parametrize("n,h,fl", [(4900, 2600, 4000), (4096, 3200, 4696)])
def test_tail_split_gate_up_matches_oracle(n, h, fl):
    """Gated 256 x 128-act-column tiles: 20 x 32 = 512 + 128 (two K pieces
    per cut tile) and 16 x 37 = 512 + 80 (three pieces), ragged last tile
    row and column."""
    assert T.tp_gate_up_workspace_bytes(n, h, fl, torch.bfloat16) > 0
    x = rnd((n, h), 1.0, 180, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.02, 181, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    rows = sorted(set(synth.sample_rows(n, 12, 182) + list(range(n - 8, n))))
    xg, W = to_f64(x[rows]), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    got = to_f64(act[rows])
    assert relf(got, ref) <= 1e-2
    assert relf(got[:, -300:], ref[:, -300:]) <= 1e-2
    again = T.tp_gate_up_act_rank(x, wgu)
    assert torch.equal(act, again)          # fixed piece order: deterministic


@pytest.mark.parametrize("n,k,m", [(8100, 1024, 760), (8192, 2048, 768), (8192, 640, 1536)])
def test_mid_tiles_linear_matches_oracle(n, k, m):
    """128 x 192 paired-stage tiles, chosen when 256 x 256 tiles would be
    too few and 128 x 192 ones fill at least three quarters of the CUs:
    (8100, 760) leaves ragged last tiles in both dimensions (64 x 4 tiles),
    (8192, 1536) gives 64 x 8 = 512 tiles (two rounds).  Bias and both
    output types; the fp32 store goes element-wise here."""
    x = rnd((n, k), 1.0, 270, torch.bfloat16)
    w = rnd((m, k), 0.05, 271, torch.bfloat16)
    b = rnd((m,), 0.05, 272, torch.bfloat16)
    rows = synth.sample_rows(n, 10, 273)
    for bias in (None, b):
        ref = oracle.linear(to_f64(x)[rows], to_f64(w), to_f64(bias) if bias is not None else None)
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            assert relf(to_f64(y)[rows], ref) <= 1e-2, (bias is None, out_dt)
            assert relf(to_f64(y[-1:]), oracle.linear(to_f64(x)[-1:], to_f64(w),
                                                      to_f64(bias) if bias is not None else None)) <= 1e-2


@pytest.mark.parametrize("n,k,m", [(8100, 4096, 760), (8192, 8192, 768), (6000, 4224, 900)])
def test_w192_split_tiles_linear_matches_oracle(n, k, m):
    """256 x 192 paired-stage tiles with K split in two and the split finish
    pass, chosen for long K when the two halves fill one round: (8100, 760)
    leaves ragged last tiles in both dimensions (32 x 4 tiles x 2 halves),
    (8192, 768) is the QKV projection at TP=16, (6000, 900) gives 24 x 5 x 2
    = 240 units with K halves of 2112.  Bias and both output types."""
    x = rnd((n, k), 1.0, 280, torch.bfloat16)
    w = rnd((m, k), 0.05, 281, torch.bfloat16)
    b = rnd((m,), 0.05, 282, torch.bfloat16)
    rows = synth.sample_rows(n, 8, 283)
    assert T.tp_linear_workspace_bytes(n, k, m, torch.bfloat16) == 2 * n * m * 4
    for bias in (None, b):
        ref = oracle.linear(to_f64(x)[rows], to_f64(w), to_f64(bias) if bias is not None else None)
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            assert relf(to_f64(y)[rows], ref) <= 1e-2, (bias is None, out_dt)
            assert relf(to_f64(y[-1:]), oracle.linear(to_f64(x)[-1:], to_f64(w),
                                                      to_f64(bias) if bias is not None else None)) <= 1e-2


@pytest.mark.parametrize("n,k,m", [(4100, 1024, 7800), (8192, 3584, 8192)])
def test_paired_stage_tiles_linear_matches_oracle(n, k, m):
    """256 x 256 tiles with K a multiple of 64 (paired K = 64 LDS stages):
    17 x 31 = 527 tiles with a ragged last tile row and column, and the 70B
    down shape (1024 tiles).  Plain and biased bf16 stores and the staged
    fp32 store, every 256-column tile of the sampled rows checked."""
    x = rnd((n, k), 1.0, 190 + n, torch.bfloat16)
    w = rnd((m, k), 0.02, 191 + m, torch.bfloat16)
    b = rnd((m,), 0.02, 192, torch.bfloat16)
    rows = sorted(set(synth.sample_rows(n, 10, 193) + list(range(n - 4, n)) + [255, 256, 4095 % n]))
    for bias in (None, b):
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            ref = oracle.linear(to_f64(x[rows]), to_f64(w), to_f64(bias) if bias is not None else None)
            got = to_f64(y[rows])
            assert relf(got, ref) <= 1e-2, (bias is None, out_dt)
            assert relf(got[:, -300:], ref[:, -300:]) <= 1e-2
            # every 256-column tile of the sampled rows, on its own
            for c0 in range(0, m, 256):
                assert relf(got[:, c0:c0 + 256], ref[:, c0:c0 + 256]) <= 1e-2, (c0, bias is None, out_dt)
    y1 = T.tp_linear_rank_forward(x, w)
    assert torch.equal(y1, T.tp_linear_rank_forward(x, w))


def test_paired_stage_tiles_gate_up_matches_oracle():
    """Gated paired-stage tiles: 17 x 31 = 527 tiles of 256 x 128 act
    columns, ragged last tile row and column."""
    n, h, fl = 4100, 1024, 3900
    x = rnd((n, h), 1.0, 195, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.02, 196, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    rows = sorted(set(synth.sample_rows(n, 10, 197) + list(range(n - 4, n)) + [255, 256]))
    xg, W = to_f64(x[rows]), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    got = to_f64(act[rows])
    assert relf(got, ref) <= 1e-2
    for c0 in range(0, fl, 128):
        assert relf(got[:, c0:c0 + 128], ref[:, c0:c0 + 128]) <= 1e-2, c0
    assert torch.equal(act, T.tp_gate_up_act_rank(x, wgu))


def test_tail_split_not_used_for_short_k_or_one_round():
    # 594 tiles of 256 but K = 1024: pieces would be too short
    assert T.tp_linear_workspace_bytes(512, 1024, 75968, torch.bfloat16) == 0
    # 256 tiles of 128 x 192 at one workgroup per CU (K = 2048, too short to
    # split in two): a single round, no workspace
    assert T.tp_linear_workspace_bytes(8192, 2048, 768, torch.bfloat16) == 0


# --------------------------------------------------------------------------
# weight-streaming decode kernel (M <= 64 tokens, at least 512 work units of
# one 128-row tile x 128-wide K chunk): per-tile partials added in K order
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 33, 64])
@pytest.mark.parametrize("k,m", [(2056, 4000), (4096, 4096)])
def test_stream_decode_linear_matches_oracle(n, k, m):
    """k = 2056 ends inside a 128-wide K chunk; m = 4000 leaves a ragged
    last tile (32 x 17 = 544 and 32 x 32 = 1024 units)."""
    x = rnd((n, k), 1.0, 190 + n, torch.bfloat16)
    w = rnd((m, k), 0.05, 191, torch.bfloat16)
    b = rnd((m,), 0.05, 192, torch.bfloat16)
    assert T.tp_linear_workspace_bytes(n, k, m, torch.bfloat16) > 0
    for bias in (None, b):
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            ref = oracle.linear(to_f64(x), to_f64(w), to_f64(bias) if bias is not None else None)
            assert relf(to_f64(y), ref) <= 1e-2, (bias is None, out_dt)


@pytest.mark.parametrize("n", [1, 64])
@pytest.mark.parametrize("h,fl", [(4000, 1100), (4096, 2048)])
def test_stream_decode_gate_up_matches_oracle(n, h, fl):
    """Gated tiles of 64 act columns: 18 x 32 = 576 and 32 x 32 = 1024 units;
    h = 4000 ends inside a K chunk, fl = 1100 leaves a ragged last tile."""
    x = rnd((n, h), 1.0, 200 + n, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.05, 201, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    assert relf(to_f64(act), ref) <= 1e-2
    assert torch.equal(act, T.tp_gate_up_act_rank(x, wgu))     # fixed order: deterministic



# --------------------------------------------------------------------------
# register-streaming decode kernel (M <= 64 tokens, K >= 1024, at least two
# 16-row weight blocks per workgroup): one fp32 partial tile [64][16] per
# K slice of at most 1024 and 16-row block, added in slice order
# --------------------------------------------------------------------------

def rs_ws(k, rows):
    return -(-k // 1024) * -(-rows // 16) * 4096


@pytest.mark.parametrize("n", [1, 33, 64])
@pytest.mark.parametrize("k,m", [(4104, 2744), (6144, 4000), (7168, 4104)])
def test_rs_decode_linear_matches_oracle(n, k, m):
    """k = 4104: 3 slices of 8 x 192 with a ragged end; m = 2744 and 4104
    end inside a 16-row block; k = 7168 is the 70B down shard's K at TP=4
    (4 slices of 8 x 224).  Outputs under 6144 columns: too few 32-column
    workgroups for the whole-K kernel."""
    assert T.tp_linear_workspace_bytes(n, k, m, torch.bfloat16) == rs_ws(k, m)
    x = rnd((n, k), 1.0, 230 + n, torch.bfloat16)
    w = rnd((m, k), 0.05, 231, torch.bfloat16)
    b = rnd((m,), 0.05, 232, torch.bfloat16)
    for bias in (None, b):
        ref = oracle.linear(to_f64(x), to_f64(w), to_f64(bias) if bias is not None else None)
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            assert relf(to_f64(y), ref) <= 1e-2, (bias is None, out_dt)
            assert relf(to_f64(y[:, -20:]), ref[:, -20:]) <= 1e-2


@pytest.mark.parametrize("n", [1, 64])
@pytest.mark.parametrize("h,fl", [(4104, 1372), (4104, 1375), (8192, 4096)])
def test_rs_decode_gate_up_matches_oracle(n, h, fl):
    """fl = 1375: act columns not a multiple of 4 (element-wise finish) and
    up rows that start inside a 16-row block."""
    assert T.tp_gate_up_workspace_bytes(n, h, fl, torch.bfloat16) == rs_ws(h, 2 * fl)
    x = rnd((n, h), 1.0, 240 + n, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.05, 241, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    assert relf(to_f64(act), ref) <= 1e-2
    assert relf(to_f64(act[:, -20:]), ref[:, -20:]) <= 1e-2
    assert torch.equal(act, T.tp_gate_up_act_rank(x, wgu))     # fixed order: deterministic


@pytest.mark.parametrize("n", [1, 33, 64])
@pytest.mark.parametrize("k,m", [(2048, 8200), (7168, 8192), (4104, 6150), (1032, 6200)])
def test_rs_decode_wide_linear_matches_oracle(n, k, m):
    """Wide outputs: (7168, 8192) is the 70B down shard at TP=4 (7 slices of
    4 x 256); m = 8200, 6150 and 6200 end inside a 16-row block; k = 4104
    and 1032 cut the slices and the waves' K ranges raggedly (at k = 1032
    the second slice holds 8 columns)."""
    assert T.tp_linear_workspace_bytes(n, k, m, torch.bfloat16) == rs_ws(k, m)
    x = rnd((n, k), 1.0, 250 + n, torch.bfloat16)
    w = rnd((m, k), 0.05, 251, torch.bfloat16)
    b = rnd((m,), 0.05, 252, torch.bfloat16)
    for bias in (None, b):
        ref = oracle.linear(to_f64(x), to_f64(w), to_f64(bias) if bias is not None else None)
        for out_dt in (torch.bfloat16, torch.float32):
            y = T.tp_linear_rank_forward(x, w, bias=bias, out_dtype=out_dt)
            assert relf(to_f64(y), ref) <= 1e-2, (bias is None, out_dt)
            assert relf(to_f64(y[:, -40:]), ref[:, -40:]) <= 1e-2


@pytest.mark.parametrize("n", [1, 64])
@pytest.mark.parametrize("h,fl", [(4104, 6150), (1032, 6200), (8192, 6144)])
def test_rs_decode_wide_gate_up_matches_oracle(n, h, fl):
    """Wide gated outputs; fl = 6150 ends inside a 16-row block, so the up
    rows start inside one."""
    assert T.tp_gate_up_workspace_bytes(n, h, fl, torch.bfloat16) == rs_ws(h, 2 * fl)
    x = rnd((n, h), 1.0, 260 + n, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.05, 261, torch.bfloat16)
    act = T.tp_gate_up_act_rank(x, wgu)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:]))
    assert relf(to_f64(act), ref) <= 1e-2
    assert relf(to_f64(act[:, -40:]), ref[:, -40:]) <= 1e-2
    assert torch.equal(act, T.tp_gate_up_act_rank(x, wgu))     # fixed order: deterministic


@pytest.mark.parametrize("n", [1, 64])
@pytest.mark.parametrize("h,fl", [(4000, 2040), (4096, 2048)])
@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float32])
def test_streamed_decode_mlp_matches_oracle(n, h, fl, out_dt):
    """Decode-sized MLP share whose two products both take the weight-
    streaming kernel (at least 512 units each) through one workspace;
    h = 4000 and fl = 2040 end inside K chunks and leave ragged last tiles."""
    x = rnd((n, h), 1.0, 210 + n, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.05, 211, torch.bfloat16)
    wd = rnd((h, fl), 0.05, 212, torch.bfloat16)
    p = T.tp_mlp_rank_forward(x, wgu, wd, out_dtype=out_dt)
    xg, W = to_f64(x), to_f64(wgu)
    ref = oracle.linear(oracle.silu_mul(oracle.linear(xg, W[:fl]), oracle.linear(xg, W[fl:])), to_f64(wd))
    assert relf(to_f64(p), ref) <= 1e-2
    assert torch.equal(p, T.tp_mlp_rank_forward(x, wgu, wd, out_dtype=out_dt))   # deterministic



# --------------------------------------------------------------------------
# sequence-parallel epilogue: ring reduce-scatter + residual add + RMSNorm.
# residual_out bit-exact against the oracle's fp32 ring simulation (one
# rounding); out within one unit in the last place of the storage type of
# the fp64 RMSNorm of the stored residual (bf16: 2^-7 relative; fp32: the
# fp32 mean-square and scaling, 1e-5 relative).
# --------------------------------------------------------------------------

SP_ULP = {torch.bfloat16: 2.0 ** -7, torch.float32: 1e-5}


def sp_check(parts, rank, residual, weight, eps, ro, out):
    dt = parts[0].dtype
    P = [to_f64(p).astype(np.float32) for p in parts]          # exact widening
    R = to_f64(residual).astype(np.float32)
    exp_ro, exp_out = oracle.rs_add_rmsnorm(P, rank, R, to_f64(weight), float(np.float32(eps)),
                                            dt == torch.bfloat16)
    if dt == torch.bfloat16:
        assert np.array_equal(bits(ro), oracle.f32_to_bf16_bits(exp_ro))
    else:
        assert np.array_equal(bits(ro), exp_ro.view(np.uint32))
    g = to_f64(out)
    assert g.shape == exp_out.shape
    assert np.all(np.abs(g - exp_out) <= SP_ULP[dt] * np.abs(exp_out) + 1e-30)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("t,n,h", [(1, 5, 64), (2, 7, 1024), (3, 13, 1000), (4, 64, 8192), (8, 37, 12288),
                                   (16, 50, 256), (5, 3, 512)])
def test_rs_add_rmsnorm_matches_oracle(dt, t, n, h):
    """h = 1000 (bf16) is not a whole number of 16-byte vectors (element-wise
    path); h = 12288 keeps only 8192 per row in registers and reads the rest
    back; n = 3 < t = 5 leaves two ranks without rows."""
    parts = [rnd((n, h), 1.0, 600 + 13 * r + h, dt) for r in range(t)]
    weight = rnd((h,), 0.5, 601, dt) + 1.0
    eps = 1e-5
    for rank in range(t):
        lo, hi = T.tp_sp_rows(n, rank, t)
        residual = rnd((hi - lo, h), 1.0, 602 + rank, dt)
        ro, out = T.tp_rs_add_rmsnorm(parts, rank, residual, weight, eps)
        torch.cuda.synchronize()
        sp_check(parts, rank, residual, weight, eps, ro, out)


def test_rs_add_rmsnorm_in_place_and_deterministic():
    t, n, h = 4, 40, 4096
    dt = torch.bfloat16
    parts = [rnd((n, h), 1.0, 610 + r, dt) for r in range(t)]
    weight = rnd((h,), 0.5, 611, dt) + 1.0
    rank = 2
    lo, hi = T.tp_sp_rows(n, rank, t)
    residual = rnd((hi - lo, h), 1.0, 612, dt)
    ro_a, out_a = T.tp_rs_add_rmsnorm(parts, rank, residual, weight, 1e-6)
    buf = residual.clone()
    ro_b, out_b = T.tp_rs_add_rmsnorm(parts, rank, buf, weight, 1e-6, residual_out=buf)
    torch.cuda.synchronize()
    assert ro_b.data_ptr() == buf.data_ptr()
    assert torch.equal(ro_a, buf) and torch.equal(out_a, out_b)
    sp_check(parts, rank, residual, weight, 1e-6, ro_a, out_a)


def test_rs_add_rmsnorm_unaligned_buffers():
    t, n, h = 3, 9, 256
    dt = torch.bfloat16
    bufs = [rnd((n * h + 1,), 1.0, 620 + r, dt) for r in range(t)]
    parts = [b[1:].view(n, h) for b in bufs]                   # misaligned by one element
    weight = rnd((h,), 0.5, 621, dt) + 1.0
    rank = 1
    lo, hi = T.tp_sp_rows(n, rank, t)
    residual = rnd((hi - lo, h), 1.0, 622, dt)
    ro, out = T.tp_rs_add_rmsnorm(parts, rank, residual, weight, 1e-5)
    torch.cuda.synchronize()
    sp_check(parts, rank, residual, weight, 1e-5, ro, out)


def test_rs_add_rmsnorm_order_and_rounding_pins_on_gpu():
    """The oracle's tie pins, on the GPU: ring order (2^-24 + 2^-24 + 1) and
    the single rounding of the residual add (1 + 2^-8 + 2^-16 -> 1 + 2^-7)."""
    e = 2.0 ** -24
    n = t = 3
    P = [torch.zeros(n, 4, device=DEV) for _ in range(t)]
    for c in range(n):
        P[c][c] = e
        P[(c + 1) % t][c] = e
        P[(c + 2) % t][c] = 1.0
    w = torch.ones(4, device=DEV)
    for r in range(t):
        ro, _ = T.tp_rs_add_rmsnorm(P, r, torch.zeros(1, 4, device=DEV), w, 1e-5)
        assert ro.tolist() == [[1.0 + 2.0 ** -23] * 4]
    P = [torch.zeros(2, 8, device=DEV, dtype=torch.bfloat16) for _ in range(2)]
    for c in range(2):
        P[c][c] = 1.0
        P[(c + 1) % 2][c] = 2.0 ** -8
    wb = torch.ones(8, device=DEV, dtype=torch.bfloat16)
    for r in range(2):
        res = torch.full((1, 8), 2.0 ** -16, device=DEV, dtype=torch.bfloat16)
        ro, _ = T.tp_rs_add_rmsnorm(P, r, res, wb, 1e-5)
        assert ro.float().tolist() == [[1.0 + 2.0 ** -7] * 8]


# --------------------------------------------------------------------------
# one-shot (rank-order) reduce: bit-exact against the oracle's zero-started
# fp32 rank-order sum, rounded once
# --------------------------------------------------------------------------

def oracle_rank_bits(parts, out_dtype):
    f32 = [to_f64(p).astype(np.float32) for p in parts]
    s = oracle.reduce_rank_f32(f32)
    return oracle.f32_to_bf16_bits(s) if out_dtype == torch.bfloat16 else s.view(np.uint32)


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32)])
@pytest.mark.parametrize("t", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("K", [1, 7, 8 * 1000 + 5, 1_000_003])
def test_partial_reduce_rank_order_bit_exact(in_dt, out_dt, t, K):
    parts = [rnd((K,), 1.0, 700 + 31 * r + K % 97, in_dt) for r in range(t)]
    got = T.tp_partial_reduce(parts, out_dtype=out_dt, order=T.TP_ORDER_RANK)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), oracle_rank_bits(parts, out_dt))


def test_partial_reduce_rank_order_pins_on_gpu():
    e = 2.0 ** -24
    P0 = torch.tensor([e, 1.0, e], device=DEV)
    P1 = torch.tensor([1.0, e, e], device=DEV)
    P2 = torch.tensor([e, e, 1.0], device=DEV)
    assert T.tp_partial_reduce([P0, P1, P2], order=T.TP_ORDER_RANK).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -23]
    assert T.tp_partial_reduce([P0, P1, P2]).tolist() == [1.0, 1.0 + 2.0 ** -23, 1.0]
    nz = [torch.full((4099,), -0.0, device=DEV) for _ in range(4)]
    r = T.tp_partial_reduce(nz, order=T.TP_ORDER_RANK)
    assert not torch.signbit(r).any()                    # 0 + (-0) = +0
    assert torch.signbit(T.tp_partial_reduce(nz)).all()  # the ring has no zero start


def test_partial_reduce_rank_order_unaligned():
    t, K = 3, 4099
    bufs = [rnd((K + 1,), 1.0, 720 + r, torch.bfloat16) for r in range(t)]
    parts = [b[1:] for b in bufs]
    got = T.tp_partial_reduce(parts, order=T.TP_ORDER_RANK)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), oracle_rank_bits(parts, torch.bfloat16))


# --------------------------------------------------------------------------
# vocab logits gather + greedy argmax: full logits bit-exact (a copy), argmax
# exact against the oracle's first-maximum rule
# --------------------------------------------------------------------------

def gather_check(shards, vocab, full, am):
    exp_full, exp_am = oracle.logits_gather_argmax([to_f64(s) for s in shards], vocab)
    if full is not None:
        assert np.array_equal(bits(full), exp_full.astype(np.float32).view(np.uint32))
    assert am.cpu().tolist() == exp_am.tolist()


@pytest.mark.parametrize("V,t,n", [(10, 3, 5), (11, 4, 3), (7, 8, 2), (4096, 4, 9), (151936, 2, 17), (1000, 3, 4)])
def test_logits_gather_argmax_matches_oracle(V, t, n):
    """Ragged shard widths (10 = 4 + 4 + 2; 11 = 3 + 3 + 3 + 2; 7 over 8
    ranks leaves the last empty; 1000 = 334 + 334 + 332 takes the element-wise
    path); values drawn from a few levels so that ties are common."""
    shards = []
    for r in range(t):
        s, e = T.tp_vocab_range(V, r, t)
        g = torch.Generator(device="cpu").manual_seed(800 + r + V)
        shards.append(torch.randint(-3, 4, (n, e - s), generator=g).float().to(DEV) if e > s
                      else torch.empty((n, 0), device=DEV))
    full, am = T.tp_logits_gather_argmax(shards, V)
    torch.cuda.synchronize()
    gather_check(shards, V, full, am)
    _, am2 = T.tp_logits_gather_argmax(shards, V, want_full=False)
    assert torch.equal(am, am2)


def test_logits_gather_argmax_nan_and_signed_zero():
    V, t, n = 12, 3, 3
    rows = torch.tensor([[0.0, -0.0, 0.0, -1.0, 0.0, 0.0, -0.0, 0.0, -5.0, 0.0, 0.0, 0.0],
                         [1.0, 2.0, 3.0, float("nan"), 9.0, float("nan"), 1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                         [-3.0] * 11 + [-2.0]], device=DEV)
    shards = [rows[:, 4 * r:4 * r + 4].contiguous() for r in range(t)]
    full, am = T.tp_logits_gather_argmax(shards, V)
    torch.cuda.synchronize()
    assert am.tolist() == torch.argmax(rows.cpu(), dim=1).tolist() == [0, 3, 11]
    gather_check(shards, V, full, am)


# --------------------------------------------------------------------------
# head-parallel attention core: rel-Frobenius <= 1e-2 per head against the
# fp64 oracle (bf16 inputs, fp32 softmax, bf16 probabilities and output)
# --------------------------------------------------------------------------

def attn_check(qkv, nq, nkv, causal, out, rows=None):
    ref = oracle.attention_rank(to_f64(qkv), nq, nkv, 128, causal, rows=rows)
    got = to_f64(out) if rows is None else to_f64(out[rows])
    for h in range(nq):
        e = relf(got[:, h * 128:(h + 1) * 128], ref[:, h * 128:(h + 1) * 128])
        assert e <= 1e-2, (h, e)


@pytest.mark.parametrize("n,nq,nkv,causal", [(1, 4, 1, True), (31, 4, 1, True), (33, 4, 1, False), (64, 4, 2, True),
                                             (100, 8, 2, True), (129, 4, 4, False), (200, 12, 2, True),
                                             (257, 4, 1, False)])
def test_attention_rank_matches_oracle(n, nq, nkv, causal):
    """Partial query tiles and key blocks, GQA groups of 4 (one wave per
    head), MHA (three idle waves), groups of 6 (a second head quad)."""
    qkv = rnd((n, (nq + 2 * nkv) * 128), 1.0, 900 + n + nq, torch.bfloat16)
    out = T.tp_attention_rank(qkv, nq, nkv, causal=causal)
    torch.cuda.synchronize()
    attn_check(qkv, nq, nkv, causal, out)
    assert torch.equal(out, T.tp_attention_rank(qkv, nq, nkv, causal=causal))     # deterministic


def test_attention_rank_peaked_and_flat_scores():
    """Large logits (scores of several hundred: the running max must carry
    the scale) and identical keys (uniform weights)."""
    n, nq, nkv = 96, 4, 1
    qkv = rnd((n, (nq + 2 * nkv) * 128), 1.0, 950, torch.bfloat16)
    big = qkv.clone()
    big[:, :nq * 128] *= 8.0
    big[:, nq * 128:(nq + 1) * 128] *= 8.0
    out = T.tp_attention_rank(big, nq, nkv, causal=True)
    torch.cuda.synchronize()
    attn_check(big, nq, nkv, True, out)
    flat = qkv.clone()
    flat[:, nq * 128:(nq + 1) * 128] = flat[0, nq * 128:(nq + 1) * 128]
    out = T.tp_attention_rank(flat, nq, nkv, causal=False)
    torch.cuda.synchronize()
    attn_check(flat, nq, nkv, False, out)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_rank_split_key_chunks(causal):
    """n = 4100: 129 query tiles in 65 (light, heavy) pairs, each pair's key
    blocks cut into chunks of about 16 that a second kernel merges; sampled
    rows around tile edges and the pair of the middle tile."""
    n, nq, nkv = 4100, 8, 2
    assert T.tp_attention_workspace_bytes(n, nq, nkv, causal=causal) > 0
    qkv = rnd((n, (nq + 2 * nkv) * 128), 1.0, 960 + causal, torch.bfloat16)
    out = T.tp_attention_rank(qkv, nq, nkv, causal=causal)
    torch.cuda.synchronize()
    rows = [0, 31, 2047, 2048, 2049, 2079, 2080, 4064, 4095, 4096, 4099]
    attn_check(qkv, nq, nkv, causal, out, rows=rows)
    assert torch.equal(out, T.tp_attention_rank(qkv, nq, nkv, causal=causal))


@pytest.mark.parametrize("n,nq,nkv,causal", [(2600, 16, 2, True), (2600, 16, 2, False), (3000, 2, 2, True)])
def test_attention_rank_split_with_head_quads_and_idle_waves(n, nq, nkv, causal):
    """Split tiles (partials and the combine) with two KV groups of 8 heads
    (two head quads per group: partial slots over groups and quads), and MHA
    (one head per group: three idle waves per query half).  Rows on both
    sides of the 32-query halves and the 64-query tiles."""
    assert T.tp_attention_workspace_bytes(n, nq, nkv, causal=causal) > 0
    qkv = rnd((n, (nq + 2 * nkv) * 128), 1.0, 970 + n + nq + causal, torch.bfloat16)
    out = T.tp_attention_rank(qkv, nq, nkv, causal=causal)
    torch.cuda.synchronize()
    rows = [0, 1, 31, 32, 63, 64, 95, 96, 1023, 1024, 1300, 1301, n // 2, n - 33, n - 32, n - 1]
    attn_check(qkv, nq, nkv, causal, out, rows=rows)
    assert torch.equal(out, T.tp_attention_rank(qkv, nq, nkv, causal=causal))


def test_attention_workspace_is_zero_for_short_sequences():
    """Short sequences: every workgroup takes whole query tiles (a light and
    a heavy one), so nothing is merged and no workspace is needed."""
    assert T.tp_attention_workspace_bytes(512, 4, 1, causal=True) == 0
    assert T.tp_attention_workspace_bytes(256, 4, 1, causal=False) == 0
    assert T.tp_attention_workspace_bytes(8192, 4, 1, causal=True) > 0
    assert T.tp_attention_workspace_bytes(4100, 8, 2, causal=False) > 0

# --------------------------------------------------------------------------
# checkpoint-style loaders: host checkpoint tensor -> the rank's device
# table, bit-exact against the oracle's loaders
# --------------------------------------------------------------------------

def host_np(t):
    """numpy view of a host tensor in the oracle's convention (bf16 as bits)."""
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


def host_tensor(shape, seed, dtype, pinned=False):
    a = synth.normal(shape, 1.0, seed, torch.float32)
    a[0, :4] = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130])   # ties, subnormal
    a = a.to(dtype)
    return a.pin_memory() if pinned else a


@pytest.mark.parametrize("src_dt,dst_dt", [(torch.float32, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                           (torch.bfloat16, torch.float32), (torch.float32, torch.float32)])
@pytest.mark.parametrize("rows,cols,t", [(96, 160, 4), (48, 150, 2), (64, 64, 1), (40, 24, 8)])
@pytest.mark.parametrize("dim", [0, 1])
def test_load_shard_matches_oracle(src_dt, dst_dt, rows, cols, t, dim):
    """Column and row cuts, with and without conversion; 150 columns (and 75
    after a row cut) take the element-wise conversion."""
    if (rows if dim == 0 else cols) % t:
        pytest.skip("not divisible")
    src = host_tensor((rows, cols), 1300 + rows + cols + t, src_dt)
    for r in range(t):
        out = T.tp_load_shard(src, dim, r, t, dtype=dst_dt)
        torch.cuda.synchronize()
        ref = oracle.load_shard(host_np(src), dim, r, t, dst_dt == torch.bfloat16)
        assert np.array_equal(bits(out), ref.view(np.uint16 if dst_dt == torch.bfloat16 else np.uint32))


def test_load_shard_from_pinned_memory_and_caller_staging():
    src = host_tensor((64, 256), 1400, torch.float32, pinned=True)
    staging = torch.empty(T.tp_load_staging_bytes(16, 256, torch.float32, torch.bfloat16), dtype=torch.uint8,
                          device=DEV)
    out = torch.full((16, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    T.tp_load_shard(src, 0, 3, 4, out=out, staging=staging)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.load_shard(host_np(src), 0, 3, 4, True))


@pytest.mark.parametrize("n_q,n_kv,t", [(8, 2, 2), (8, 2, 8), (16, 4, 4), (4, 4, 2)])
def test_load_qkv_and_gate_up_tables(n_q, n_kv, t):
    """One projection per call into the rank's merged table (other rows
    untouched until their call), fp32 checkpoint -> bf16 table; equal to the
    oracle's loaders and to tp_shard_qkv / tp_shard_gate_up of the converted
    full tensors (GQA replication when t > n_kv)."""
    hd, h, f = 16, 72, 24 * t
    wq = host_tensor((n_q * hd, h), 1500 + t, torch.float32)
    wk = host_tensor((n_kv * hd, h), 1501 + t, torch.float32)
    wv = host_tensor((n_kv * hd, h), 1502 + t, torch.float32)
    gate = host_tensor((f, h), 1503 + t, torch.float32)
    up = host_tensor((f, h), 1504 + t, torch.float32)
    dev = [a.to(DEV).to(torch.bfloat16) for a in (wq, wk, wv, gate, up)]
    for r in range(t):
        _, kvc = T.tp_kv_heads_for_rank(n_kv, r, t)
        table = torch.full(((n_q // t + 2 * kvc) * hd, h), float("nan"), dtype=torch.bfloat16, device=DEV)
        ref = np.full(table.shape, 0x7FC0, dtype=np.uint16)
        for sid in (1, 2, 0):
            T.tp_load_qkv((wq, wk, wv)[sid], sid, n_q, n_kv, hd, r, t, out=table)
            oracle.load_qkv(ref, host_np((wq, wk, wv)[sid]), sid, n_q, n_kv, hd, r, t)
        torch.cuda.synchronize()
        assert np.array_equal(bits(table), ref)
        assert torch.equal(table.view(torch.int16),
                           T.tp_shard_qkv(dev[0], dev[1], dev[2], n_q, n_kv, hd, r, t).view(torch.int16))
        gu = torch.full((2 * f // t, h), float("nan"), dtype=torch.bfloat16, device=DEV)
        T.tp_load_gate_up(up, 1, r, t, out=gu)
        T.tp_load_gate_up(gate, 0, r, t, out=gu)
        torch.cuda.synchronize()
        assert torch.equal(gu.view(torch.int16), T.tp_shard_gate_up(dev[3], dev[4], r, t).view(torch.int16))


# --------------------------------------------------------------------------
# binding: buffers it allocates live on the caller's stream
# --------------------------------------------------------------------------

def test_mlp_on_side_stream_while_current_stream_reuses_memory():
    """tp_mlp_rank_forward queued on a side stream behind a delay, with the
    binding allocating (and dropping) the workspace; meanwhile the current
    stream keeps allocating blocks of the workspace's size and filling them
    with NaN.  Were the workspace allocated on the current stream, torch's
    caching allocator would hand its block to those fills while the side
    stream's kernels still read the activation and split-K partials from
    it.  The result must equal the oracle's and the same call made on the
    current stream."""
    n, h, fl = 64, 4096, 2048
    x = rnd((n, h), 1.0, 300, torch.bfloat16)
    wgu = rnd((2 * fl, h), 0.02, 301, torch.bfloat16)
    wd = rnd((h, fl), 0.02, 302, torch.bfloat16)
    ref_same = T.tp_mlp_rank_forward(x, wgu, wd)
    need = T.tp_mlp_workspace_bytes(n, h, fl, torch.bfloat16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        with torch.cuda.stream(side):
            torch.cuda._sleep(2_000_000)              # the MLP starts after the fills below begin
            out = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
        T.tp_mlp_rank_forward(x, wgu, wd, partial=out, stream=side)
        for _ in range(64):                           # the current stream's traffic meanwhile
            junk = torch.empty(need, dtype=torch.uint8, device=DEV)
            junk.fill_(0xFF)                          # bf16/fp32 NaN patterns
            torch.cuda._sleep(20_000)
            del junk
        outs.append(out)
    torch.cuda.synchronize()
    ref = oracle.mlp_rank(to_f64(x), to_f64(wgu[:fl]), to_f64(wgu[fl:]), to_f64(wd), 0, 1)
    for out in outs:
        assert torch.equal(out, ref_same)
        assert relf(to_f64(out), ref) <= TOL[torch.bfloat16]
