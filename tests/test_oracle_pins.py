"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself.  The pins are: the pages'
printed worked examples (tests/golden/, each file names its passage), closed
forms, the library routines the pages' own code calls (torch.nn.functional
linear/silu/embedding, computed in float64), exactly representable integer
cases, brute force on tiny shapes, and invariants the pages state (the row-
parallel partials sum to the unsharded result, vocab shards sum to the full
lookup, the ring moves 2(t-1)K/t elements per rank).  Each pin is chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, SiLU on the wrong operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def relf(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# bf16 rounding: pinned to torch's own float32 -> bfloat16 conversion (RNE)
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e-39),   # subnormals
        np.clip(rng.standard_normal(20000) * 1e38, -3.4e38, 3.4e38).astype(np.float32),
    ])
    # exact ties: low half == 0x8000 with both parities of the kept bit
    ties = (np.arange(0, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                        3.4028235e38, 1.0, -1.0, 1e-45], dtype=np.float32)
    vals = np.concatenate([vals, ties, special]).astype(np.float32)
    got = oracle.f32_to_bf16_bits(vals)
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_nan_stays_nan_and_widening_exact():
    bits = oracle.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert (int(bits[0]) & 0x7f80) == 0x7f80 and (int(bits[0]) & 0x7f) != 0
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = oracle.bf16_bits_to_f64(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(w[finite], ref[finite])
    assert np.array_equal(np.isnan(w), np.isnan(ref))


# --------------------------------------------------------------------------
# SiLU: closed forms
# --------------------------------------------------------------------------

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # SiLU(z) - SiLU(-z) = z  (z*s(z) + z*s(-z)... rearranged: s(z) + s(-z) = 1)
    for z in [0.3, 1.7, 5.0, 12.0]:
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, rel=1e-14)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300


def test_silu_mul_matches_torch_silu_of_gate_times_up():
    """Tensor parallelism: implemented from scratch, "Implementation", class
    TPMLP: the local activation is F.silu(gate(x)) * up(x), SiLU applied to
    the gate product only.  Pinned to torch's F.silu in float64 on inputs
    where gate and up differ in sign and scale, so that SiLU taken of the up
    product, a dropped factor or a swapped pair fails."""
    rng = np.random.default_rng(11)
    g = rng.standard_normal((7, 33)) * 3.0
    u = rng.standard_normal((7, 33)) * 0.5 + 0.25
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    got = oracle.silu_mul(g, u)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-15)
    # the swapped-operand form SiLU(u) * g and a plain product are far off
    swapped = (F.silu(torch.from_numpy(u)) * torch.from_numpy(g)).numpy()
    assert relf(got, swapped) > 0.5
    assert relf(got, g * u) > 0.1
    # closed forms element by element: a zero gate gives 0, SiLU(32) * u is
    # 32 u up to e^-32, and a negative gate of large size gives (-0) * u
    z = oracle.silu_mul(np.array([0.0, 32.0, -50.0]), np.array([5.0, 3.0, 2.0]))
    assert z[0] == 0.0
    assert z[1] == pytest.approx(96.0, rel=1e-13)
    assert abs(z[2]) < 1e-19


# --------------------------------------------------------------------------
# Linear layers: the pages' printed worked examples (bit-exact integers)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.uint16])
def test_narrow_is_torch_narrow(dtype):
    """The pages' loaders cut a shard with narrow(dim, start, length) and copy
    it (Nano-vLLM walkthrough no. 22, §3 and §4): the oracle's narrow equals
    torch.narrow on either dimension, and a cut along the other dimension
    (a transposed reading) does not."""
    rng = np.random.default_rng(7)
    full = (rng.integers(0, 60000, size=(12, 10)) if dtype == np.uint16
            else rng.standard_normal((12, 10))).astype(dtype)
    tf = torch.from_numpy(full.astype(np.int64) if dtype == np.uint16 else full)
    for dim, start, length in [(0, 0, 12), (0, 3, 4), (0, 11, 1), (1, 0, 10), (1, 2, 5), (1, 9, 1)]:
        got = oracle.narrow(full, dim, start, length)
        ref = tf.narrow(dim, start, length).numpy().astype(dtype)
        assert got.dtype == full.dtype and np.array_equal(got, ref), (dim, start, length)
    wrong = tf.narrow(1, 3, 4).numpy().astype(dtype)
    assert not np.array_equal(oracle.narrow(full, 0, 3, 4)[:, :4], wrong[:4, :])


def test_column_parallel_worked_example():
    g = gold("nano22_column_parallel.json")
    full = np.repeat(np.array(g["full_row_labels"], dtype=np.float32)[:, None],
                     g["in_features"], axis=1)
    t = g["tp_size"]
    for r in range(t):
        w = oracle.shard(full, g["tp_dim"], r, t)
        assert list(w.shape) == g["rank_weight_shape"]
        assert w[:, 0].tolist() == g["rank_rows"][str(r)]
        x = np.random.default_rng(r).standard_normal(g["input_shape"])
        y = oracle.linear(x, w)
        assert list(y.shape) == g["rank_output_shape"]


def test_row_parallel_worked_example_with_rank0_bias():
    g = gold("nano22_row_parallel.json")
    W = np.array(g["weight"])
    b = np.array(g["bias"])
    x = np.array(g["x"])
    t = g["tp_size"]
    parts = []
    for r in range(t):
        w = oracle.shard(W, 1, r, t)
        assert list(w.shape) == g["rank_weight_shape"]
        assert w.tolist() == g["rank_cols"][str(r)]
        xr = oracle.shard(x, 1, r, t)
        parts.append(oracle.linear(xr, w, b if r == 0 else None))
    assert parts[0].tolist() == g["partial_rank0_with_bias"]
    assert parts[1].tolist() == g["partial_rank1_no_bias"]
    s = oracle.reduce_sum_f64(parts).reshape(1, -1)
    assert s.tolist() == g["all_reduce_sum"]
    assert oracle.linear(x, W, b).tolist() == g["single_card"]
    # the fp32 ring simulation gives the same exact integers
    ring = oracle.ring_allreduce_f32([p.astype(np.float32) for p in parts])
    assert ring.tolist() == g["all_reduce_sum"][0]


def test_linear_matches_torch_functional_linear():
    rng = np.random.default_rng(7)
    for (n, k, m) in [(1, 1, 1), (3, 5, 7), (9, 16, 4), (2, 33, 17)]:
        x = rng.standard_normal((n, k))
        w = rng.standard_normal((m, k))
        b = rng.standard_normal(m)
        y = oracle.linear(x, w, b)
        ref = F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
        # a transposed weight must not pass (non-square shapes chosen above)
        if m == k and n > 1:
            assert not np.allclose(oracle.linear(x, w.T.copy()), F.linear(
                torch.from_numpy(x), torch.from_numpy(w)).numpy())


# --------------------------------------------------------------------------
# MLP
# --------------------------------------------------------------------------

def _torch_mlp(x, gate, up, down):
    """The pages' own formulation: down(silu(gate(x)) * up(x)) with F.linear/F.silu."""
    X, G, U, D = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, gate, up, down))
    return F.linear(F.silu(F.linear(X, G)) * F.linear(X, U), D).numpy()


@pytest.mark.parametrize("n,h,f", [(1, 8, 12), (3, 16, 24), (5, 8, 12), (4, 32, 48)])
def test_mlp_matches_torch_functional(n, h, f):
    rng = np.random.default_rng(n * 100 + h)
    x = rng.standard_normal((n, h))
    gate = rng.standard_normal((f, h)) * 0.3
    up = rng.standard_normal((f, h)) * 0.3
    down = rng.standard_normal((h, f)) * 0.3
    y = oracle.mlp(x, gate, up, down)
    assert np.allclose(y, _torch_mlp(x, gate, up, down), rtol=1e-12, atol=1e-13)
    # SiLU on the wrong operand (up instead of gate) must fail
    wrong = _torch_mlp(x, up, gate, down)
    assert relf(y, wrong) > 1e-3


def test_mlp_zero_gate_gives_exact_zero_and_tiny_closed_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 8))
    up = rng.standard_normal((12, 8))
    down = rng.standard_normal((8, 12))
    y = oracle.mlp(x, np.zeros((12, 8)), up, down)
    assert np.all(y == 0.0)
    # h = f = 1: y = silu(x g) * (x u) * d
    y1 = oracle.mlp(np.array([[1.0]]), np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]))
    assert y1[0, 0] == pytest.approx(6.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


@pytest.mark.parametrize("t", [1, 2, 3, 4])
@pytest.mark.parametrize("n,h,f", [(1, 8, 12), (3, 16, 24), (5, 8, 24)])
def test_row_parallel_partials_sum_to_unsharded(t, n, h, f):
    """AIInfraGuide 6.2 §1: Y = sum_i act(X A_i) B_i."""
    rng = np.random.default_rng(t * 1000 + n * 10 + h)
    x = rng.standard_normal((n, h))
    gate = rng.standard_normal((f, h)) * 0.5
    up = rng.standard_normal((f, h)) * 0.5
    down = rng.standard_normal((h, f)) * 0.5
    full = _torch_mlp(x, gate, up, down)
    parts = [oracle.mlp_rank(x, gate, up, down, r, t) for r in range(t)]
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-12)
    if t == 1:
        assert np.array_equal(parts[0], oracle.mlp(x, gate, up, down))
    # each partial is the MLP restricted to the rank's slice, checked with
    # torch on explicitly sliced weights
    fl = f // t
    for r in range(t):
        sl = slice(r * fl, (r + 1) * fl)
        ref = _torch_mlp(x, gate[sl], up[sl], down[:, sl])
        assert np.allclose(parts[r], ref, rtol=1e-12, atol=1e-13)


def test_nonlinearity_before_reduce_is_wrong():
    """vLLM source analysis 13, §2.2.2 demo: with the first matrix split along
    its input dim the partial products must be summed BEFORE the nonlinearity;
    applying it per rank and summing afterwards gives a different result."""
    rng = np.random.default_rng(42)
    n, h, f, t = 4, 16, 24, 2
    x = rng.standard_normal((n, h))
    gate = rng.standard_normal((f, h))
    up = rng.standard_normal((f, h))
    ok = oracle.silu_mul(oracle.linear(x, gate), oracle.linear(x, up))
    wrong = 0
    for r in range(t):
        xr, gr, ur = oracle.shard(x, 1, r, t), oracle.shard(gate, 1, r, t), oracle.shard(up, 1, r, t)
        wrong = wrong + oracle.silu_mul(oracle.linear(xr, gr), oracle.linear(xr, ur))
    assert relf(wrong, ok) > 0.05
    # while summing the pre-activation partials first is right
    g = sum(oracle.linear(oracle.shard(x, 1, r, t), oracle.shard(gate, 1, r, t)) for r in range(t))
    u = sum(oracle.linear(oracle.shard(x, 1, r, t), oracle.shard(up, 1, r, t)) for r in range(t))
    assert np.allclose(oracle.silu_mul(g, u), ok, rtol=1e-12, atol=1e-12)


def test_wrong_dim_gate_up_shard_fails_invariant():
    """Sharding gate/up along the input dim (instead of the output dim) breaks
    the sum of partials."""
    rng = np.random.default_rng(5)
    n, h, f, t = 3, 16, 16, 2
    x = rng.standard_normal((n, h))
    gate = rng.standard_normal((f, h))
    up = rng.standard_normal((f, h))
    down = rng.standard_normal((h, f))
    full = oracle.mlp(x, gate, up, down)
    fl = f // t
    parts = []
    for r in range(t):
        xr = oracle.shard(x, 1, r, t)
        g = oracle.linear(xr, oracle.shard(gate, 1, r, t))
        u = oracle.linear(xr, oracle.shard(up, 1, r, t))
        parts.append(oracle.linear(oracle.silu_mul(g, u), down))
    assert relf(sum(parts), full) > 0.05


# --------------------------------------------------------------------------
# Merged tables and GQA replication
# --------------------------------------------------------------------------

def _by_head(num_heads, base, head_size, hidden):
    rows = [[float(base + hh)] * hidden for hh in range(num_heads) for _ in range(head_size)]
    return np.array(rows, dtype=np.float32)


def test_merged_qkv_and_gate_up_worked_example():
    g = gold("nano22_merged_double_cut.json")
    q = g["qkv"]
    wq = _by_head(q["num_q_heads"], q["q_base"], q["head_size"], q["hidden"])
    wk = _by_head(q["num_kv_heads"], q["k_base"], q["head_size"], q["hidden"])
    wv = _by_head(q["num_kv_heads"], q["v_base"], q["head_size"], q["hidden"])
    t = q["tp_size"]
    for r in range(t):
        m = oracle.shard_qkv(wq, wk, wv, q["num_q_heads"], q["num_kv_heads"], q["head_size"], r, t)
        c = m[:, 0].tolist()
        exp = q[f"rank{r}"]
        nq = len(exp["q"])
        nk = len(exp["k"])
        assert c[:nq] == exp["q"]
        assert c[nq:nq + nk] == exp["k"]
        assert c[nq + nk:] == exp["v"]
    gu = g["gate_up"]
    gate = np.full((gu["intermediate"], gu["hidden"]), gu["gate_fill"], dtype=np.float32)
    up = np.full((gu["intermediate"], gu["hidden"]), gu["up_fill"], dtype=np.float32)
    m0 = oracle.shard_gate_up(gate, up, 0, gu["tp_size"])
    half = gu["intermediate"] // gu["tp_size"]
    assert m0[:half, 0].tolist() == gu["rank0"]["gate_segment"]
    assert m0[half:2 * half, 0].tolist() == gu["rank0"]["up_segment"]


def test_gate_up_double_cut_is_not_a_cut_of_the_concatenation():
    f, h, t = 8, 3, 4
    gate = np.arange(f, dtype=np.float32)[:, None].repeat(h, 1)
    up = 100 + np.arange(f, dtype=np.float32)[:, None].repeat(h, 1)
    for r in range(t):
        m = oracle.shard_gate_up(gate, up, r, t)
        fl = f // t
        assert m[:fl, 0].tolist() == list(range(r * fl, (r + 1) * fl))
        assert m[fl:, 0].tolist() == [100 + v for v in range(r * fl, (r + 1) * fl)]


def test_kv_head_counts_from_pages():
    g = gold("kv_head_counts.json")
    for c in g["cases"]:
        t = c["tp"]
        heads = []
        for r in range(t):
            first, count = oracle.kv_heads_for_rank(c["n_kv"], r, t)
            assert count == c["kv_per_rank"]
            heads.extend(range(first, first + count))
        # every KV head stored exactly `replicas` times
        for hh in range(c["n_kv"]):
            assert heads.count(hh) == c["replicas"]
        assert c["n_q"] // t == c["q_per_rank"]
        if "f" in c:
            assert c["f"] // t == c["f_per_rank"]


@pytest.mark.parametrize("n_q,n_kv,t", [(64, 8, 16), (8, 2, 4), (8, 2, 8), (16, 8, 2), (4, 2, 2)])
def test_gqa_replica_matches_query_group(n_q, n_kv, t):
    """Rank r's KV head must be the one its own Q heads attend with (Q head j
    reads KV head j // (n_q // n_kv))."""
    qpr = n_q // t
    group = n_q // n_kv
    for r in range(t):
        first, count = oracle.kv_heads_for_rank(n_kv, r, t)
        need = sorted({j // group for j in range(r * qpr, (r + 1) * qpr)})
        assert list(range(first, first + count)) == need


def test_qkv_shard_outputs_are_slices_of_unsharded_projections():
    rng = np.random.default_rng(11)
    n, h, hd, nq, nkv, t = 5, 16, 4, 8, 2, 4
    x = rng.standard_normal((n, h))
    wq = rng.standard_normal((nq * hd, h))
    wk = rng.standard_normal((nkv * hd, h))
    wv = rng.standard_normal((nkv * hd, h))
    Q = F.linear(torch.from_numpy(x), torch.from_numpy(wq)).numpy()
    K = F.linear(torch.from_numpy(x), torch.from_numpy(wk)).numpy()
    V = F.linear(torch.from_numpy(x), torch.from_numpy(wv)).numpy()
    qpr = nq // t
    for r in range(t):
        first, count = oracle.kv_heads_for_rank(nkv, r, t)
        y = oracle.linear(x, oracle.shard_qkv(wq, wk, wv, nq, nkv, hd, r, t))
        qn = qpr * hd
        kn = count * hd
        assert np.allclose(y[:, :qn], Q[:, r * qn:(r + 1) * qn], rtol=1e-12, atol=1e-12)
        assert np.allclose(y[:, qn:qn + kn], K[:, first * hd:(first + count) * hd], rtol=1e-12, atol=1e-12)
        assert np.allclose(y[:, qn + kn:], V[:, first * hd:(first + count) * hd], rtol=1e-12, atol=1e-12)


def test_o_proj_row_parallel_partials_sum_to_full():
    """vLLM source analysis 13 §2.3: concatenating the heads' outputs and
    projecting equals summing each rank's projection of its own heads."""
    rng = np.random.default_rng(12)
    n, hd, nq, h, t = 6, 4, 8, 12, 4
    A = rng.standard_normal((n, nq * hd))
    Wo = rng.standard_normal((h, nq * hd))
    full = F.linear(torch.from_numpy(A), torch.from_numpy(Wo)).numpy()
    parts = [oracle.linear(oracle.shard(A, 1, r, t), oracle.shard(Wo, 1, r, t)) for r in range(t)]
    assert np.allclose(oracle.reduce_sum_f64(parts).reshape(n, h), full, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Vocab-parallel embedding and LM head
# --------------------------------------------------------------------------

def test_vocab_range_rule():
    assert [oracle.vocab_range(151936, r, 2) for r in range(2)] == [(0, 75968), (75968, 151936)]
    assert [oracle.vocab_range(11, r, 4) for r in range(4)] == [(0, 3), (3, 6), (6, 9), (9, 11)]
    assert [oracle.vocab_range(10, r, 2) for r in range(2)] == [(0, 5), (5, 10)]
    rs = [oracle.vocab_range(10, r, 8) for r in range(8)]
    assert rs[:5] == [(0, 2), (2, 4), (4, 6), (6, 8), (8, 10)]
    assert all(e - s == 0 for s, e in rs[5:])


def test_vocab_embedding_demo_structure():
    g = gold("vllm13_vocab_embedding.json")
    V, h, t = g["vocab"], g["hidden"], g["tp_size"]
    table = np.random.default_rng(42).standard_normal((V, h))
    ids = np.array(g["ids"], dtype=np.int64).reshape(-1)
    outs = []
    for r in range(t):
        s, e = oracle.vocab_range(V, r, t)
        assert [s, e] == g["ranges"][r]
        o = oracle.embed_rank(ids, table[s:e], V, r, t)
        nz = np.any(o != 0, axis=1).reshape(np.array(g["ids"]).shape)
        assert nz.tolist() == g[f"rank{r}_nonzero"]
        outs.append(o)
    assert np.array_equal(outs[0] + outs[1], table[ids])
    ref = F.embedding(torch.from_numpy(ids), torch.from_numpy(table)).numpy()
    assert np.array_equal(oracle.embed_full(ids, table), ref)


@pytest.mark.parametrize("V", [10, 11])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
def test_vocab_embedding_brute_force_edges(V, t):
    h = 3
    table = (np.arange(V * h, dtype=np.float32).reshape(V, h) + 1.0)
    ids_set = set()
    for r in range(t):
        s, e = oracle.vocab_range(V, r, t)
        ids_set |= {s - 1, s, e - 1, e}
    ids_set |= {-1, 0, V - 1, V, V + 7, -(1 << 40)}
    ids = np.array(sorted(ids_set), dtype=np.int64)
    total = np.zeros((ids.size, h), dtype=np.float64)
    owners = np.zeros(ids.size, dtype=np.int64)
    for r in range(t):
        s, e = oracle.vocab_range(V, r, t)
        o = oracle.embed_rank(ids, table[s:e], V, r, t)
        for i, v in enumerate(ids):
            if s <= v < e:
                assert np.array_equal(o[i], table[v])
                owners[i] += 1
            else:
                assert np.all(o[i].view(np.uint32) == 0)   # +0.0 bits, never -0.0
        total += o
    valid = (ids >= 0) & (ids < V)
    assert np.all(owners[valid] == 1) and np.all(owners[~valid] == 0)
    assert np.array_equal(total.astype(np.float32), oracle.embed_full(ids, table))


def test_masked_rows_do_not_read_the_table():
    """Out-of-shard rows are written without reading the table: a NaN in the
    table never leaks into a masked row (multiplying by a zero mask would)."""
    V, h, t = 8, 4, 2
    table = np.full((V, h), np.nan, dtype=np.float32)
    ids = np.array([0, 5, 7, 2], dtype=np.int64)
    o = oracle.embed_rank(ids, table[0:4], V, 0, t)
    assert np.all(np.isnan(o[[0, 3]]))
    assert np.all(o[[1, 2]].view(np.uint32) == 0)


@pytest.mark.parametrize("t", [1, 2, 3])
def test_lm_head_shards_concatenate_to_full_logits(t):
    rng = np.random.default_rng(9)
    n, h, V = 4, 8, 11
    x = rng.standard_normal((n, h))
    E = rng.standard_normal((V, h))
    full = F.linear(torch.from_numpy(x), torch.from_numpy(E)).numpy()
    cat = np.concatenate([oracle.lm_head_rank(x, E, r, t) for r in range(t)], axis=1)
    assert cat.shape == full.shape
    assert np.allclose(cat, full, rtol=1e-12, atol=1e-12)
    # one-hot rows pick table columns exactly
    onehot = np.eye(h)[[0, 3, 7]]
    cat1 = np.concatenate([oracle.lm_head_rank(onehot, E, r, t) for r in range(t)], axis=1)
    assert np.array_equal(cat1, E.T[[0, 3, 7]])


# --------------------------------------------------------------------------
# Ring all-reduce schedule and simulation
# --------------------------------------------------------------------------

def test_ring_rounds_and_traffic_from_pages():
    g = gold("vllm13_ring_cost.json")
    for N, rounds in g["rounds_at"].items():
        N = int(N)
        K = 8 * N * 1000
        sent, recv, got_rounds = oracle.ring_traffic(N, K)
        assert got_rounds == rounds
        assert all(s == 2 * (N - 1) * K // N for s in sent)
        assert all(r == 2 * (N - 1) * K // N for r in recv)
    for N, rs in g["rs_rounds_at"].items():
        sched = oracle.ring_schedule(int(N), 64)
        assert max(s["step"] for s in sched if s["phase"] == 0) + 1 == rs


@pytest.mark.parametrize("t,K", [(2, 16384 * 2), (4, 64 * 8192), (8, 8192 * 8192), (16, 8192 * 8192)])
def test_ring_traffic_config_sizes(t, K):
    sent, recv, rounds = oracle.ring_traffic(t, K)
    assert rounds == 2 * (t - 1)
    assert sent[0] == 2 * (t - 1) * K // t


@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 8])
def test_ring_schedule_structure(t):
    K = 37 * t + 5  # ragged chunk sizes
    sched = oracle.ring_schedule(t, K)
    assert len(sched) == 2 * t * (t - 1)
    # chunk bounds partition [0, K)
    bounds = [oracle.chunk_bounds(K, t, c) for c in range(t)]
    assert bounds[0][0] == 0 and bounds[-1][1] == K
    assert all(bounds[c][1] == bounds[c + 1][0] for c in range(t - 1))
    for phase in (0, 1):
        for s in range(t - 1):
            step = [x for x in sched if x["phase"] == phase and x["step"] == s]
            assert sorted(x["src"] for x in step) == list(range(t))
            assert sorted(x["chunk"] for x in step) == list(range(t))   # all chunks move each round
            assert all(x["dst"] == (x["src"] + 1) % t for x in step)
    # after reduce-scatter every chunk has been added into t-1 times
    adds = [0] * t
    for x in sched:
        if x["phase"] == 0:
            adds[x["chunk"]] += 1
    assert adds == [t - 1] * t


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
def test_ring_simulation_is_exact_on_representable_sums(t):
    # distinct power-of-two scales per rank: every partial sum is exact in fp32
    K = 10 * t + 3
    parts = [np.full(K, float(1 << r), dtype=np.float32) * (1 + np.arange(K) % 7) for r in range(t)]
    out = oracle.ring_allreduce_f32(parts)
    assert np.array_equal(out, sum(p.astype(np.float64) for p in parts).astype(np.float32))


def test_ring_chunk_accumulation_order():
    """Pins the order the reading derives: chunk c is summed as
    ((P_c + P_{c+1}) + P_{c+2}) ...  With 1 and two 2^-24 terms, 1 + 2^-24
    rounds back to 1 (tie to even) while 2^-24 + 2^-24 + 1 is 1 + 2^-23."""
    t, K = 3, 3
    e = np.float32(2.0 ** -24)
    one = np.float32(1.0)
    # element i lies in chunk i
    P0 = np.array([one, e, e], dtype=np.float32)
    P1 = np.array([e, one, e], dtype=np.float32)
    P2 = np.array([e, e, one], dtype=np.float32)
    out = oracle.ring_allreduce_f32([P0, P1, P2])
    # each chunk starts from the partial that holds the 1 -> result 1.0 everywhere
    assert out.tolist() == [1.0, 1.0, 1.0]
    # element i (chunk i) is summed (P_i + P_{i+1}) + P_{i+2}:
    #   element 0, the 1 in P1: (e + 1) + e = 1            (both ties round to even)
    #   element 1, the 1 in P0: (e + e) + 1 = 1 + 2^-23
    #   element 2, the 1 in P2: (1 + e) + e = 1
    # plain rank order (P0 + P1) + P2 would give [1, 1, 1 + 2^-23] and the
    # reverse ring direction (P_i + P_{i-1}) + P_{i-2} would give
    # [1 + 2^-23, 1, 1], so both slips fail.
    P0 = np.array([e, one, e], dtype=np.float32)
    P1 = np.array([one, e, e], dtype=np.float32)
    P2 = np.array([e, e, one], dtype=np.float32)
    out = oracle.ring_allreduce_f32([P0, P1, P2])
    assert out.tolist() == [1.0, 1.0 + 2.0 ** -23, 1.0]


@pytest.mark.parametrize("t", [2, 3, 4, 8, 16])
def test_ring_simulation_within_sequential_sum_bound(t):
    rng = np.random.default_rng(t)
    K = 4096 + 5
    parts = [rng.standard_normal(K).astype(np.float32) for _ in range(t)]
    out = oracle.ring_allreduce_f32(parts).astype(np.float64)
    exact = oracle.reduce_sum_f64(parts)
    bound = (t - 1) * 2.0 ** -24 * sum(np.abs(p.astype(np.float64)) for p in parts) * 1.0001
    assert np.all(np.abs(out - exact) <= bound)
    # a window simulation equals the same elements of the full simulation
    w = oracle.ring_allreduce_f32(parts, 1000, 3000)
    assert np.array_equal(w, out[1000:3000].astype(np.float32))


# --------------------------------------------------------------------------
# sequence-parallel epilogue: reduce-scatter + residual add + RMSNorm
# --------------------------------------------------------------------------

@pytest.mark.parametrize("t", [2, 3, 4, 8])
@pytest.mark.parametrize("n", [8, 13])
def test_sp_rank_owns_the_chunk_the_ring_completes_there(t, n):
    """Rank r ends the reduce-scatter holding the chunk that the ring
    schedule's last reduce-scatter round delivers to it, as whole token rows."""
    sched = oracle.ring_schedule(t, n)
    last = [s for s in sched if s["phase"] == 0 and s["step"] == t - 2]
    owner = {s["dst"]: s["chunk"] for s in last}
    # partial 0 carries each row's index, the others are zero
    parts = [np.zeros((n, 3), np.float32) for _ in range(t)]
    parts[0][:] = np.arange(n, dtype=np.float32)[:, None]
    for r in range(t):
        lo, hi = oracle.sp_rows(n, t, owner[r])
        res = np.zeros((hi - lo, 3), np.float32)
        got, _ = oracle.rs_add_rmsnorm(parts, r, res, np.ones(3), 1e-5, False)
        assert got[:, 0].tolist() == list(range(lo, hi)), (t, n, r)
        # whole rows: the chunks tile [0, n) in order
    cuts = [oracle.sp_rows(n, t, c) for c in range(t)]
    assert cuts[0][0] == 0 and cuts[-1][1] == n
    assert all(cuts[c][1] == cuts[c + 1][0] for c in range(t - 1))


def test_sp_sum_follows_ring_order():
    """Row c is summed ((P_c + P_{c+1}) + P_{c+2}).  With two 2^-24 terms
    first, 2^-24 + 2^-24 + 1 = 1 + 2^-23 exactly; any order that adds the 1
    earlier rounds 1 + 2^-24 back to 1 (tie to even)."""
    e = np.float32(2.0 ** -24)
    n, t = 3, 3
    parts = [np.zeros((n, 1), np.float32) for _ in range(t)]
    for c in range(n):
        parts[c][c, 0] = e
        parts[(c + 1) % t][c, 0] = e
        parts[(c + 2) % t][c, 0] = 1.0
    for r in range(t):
        got, _ = oracle.rs_add_rmsnorm(parts, r, np.zeros((1, 1), np.float32), np.ones(1), 0.0, False)
        assert got[0, 0] == np.float32(1.0 + 2.0 ** -23), r


def test_sp_residual_add_rounds_once():
    """fp32 sum then one bf16 rounding: 1 + 2^-8 + 2^-16 rounds up to
    1 + 2^-7.  Rounding the reduced sum first (1 + 2^-8 is a tie and goes to
    1) and then adding 2^-16 would give 1."""
    n, t = 2, 2
    parts = [np.zeros((n, 1), np.float32) for _ in range(t)]
    for c in range(n):
        parts[c][c, 0] = 1.0
        parts[(c + 1) % t][c, 0] = 2.0 ** -8
    for r in range(t):
        res = np.full((1, 1), 2.0 ** -16, np.float32)
        got, _ = oracle.rs_add_rmsnorm(parts, r, res, np.ones(1), 1e-5, True)
        assert got[0, 0] == np.float32(1.0 + 2.0 ** -7), r


def test_rmsnorm_closed_forms():
    t, n = 1, 3
    rows = np.array([[3.0, 4.0], [-2.5, -2.5], [0.0, 0.0]], np.float32)
    w = np.array([1.0, 0.5])
    _, out = oracle.rs_add_rmsnorm([rows], 0, np.zeros_like(rows), w, 0.0, False)
    # mean square of (3, 4) is 12.5: y = (3, 4) / (5 / sqrt 2) * w
    assert np.allclose(out[0], [3 * math.sqrt(2) / 5, 0.5 * 4 * math.sqrt(2) / 5], rtol=1e-15, atol=0)
    # a constant row normalises to sign * w
    assert out[1].tolist() == [-1.0, -0.5]
    # a zero row stays zero (eps keeps it finite): eps = 0 would divide by 0
    _, out2 = oracle.rs_add_rmsnorm([rows], 0, np.zeros_like(rows), w, 1e-5, False)
    assert out2[2].tolist() == [0.0, 0.0]


def test_rmsnorm_invariances():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    w = rng.standard_normal(64)
    z = np.zeros_like(x)
    _, y1 = oracle.rs_add_rmsnorm([x], 0, z, w, 0.0, False)
    _, y8 = oracle.rs_add_rmsnorm([x * np.float32(8.0)], 0, z, w, 0.0, False)
    assert np.allclose(y1, y8, rtol=1e-14, atol=0)            # scale invariant
    _, yu = oracle.rs_add_rmsnorm([x], 0, z, np.ones(64), 0.0, False)
    assert abs(float(np.mean(yu ** 2)) - 1.0) < 1e-13           # unit mean square
    assert np.allclose(yu * w, y1, rtol=1e-14, atol=0)          # gain is elementwise
    # eps acts inside the root: y = x / sqrt(ms + eps)
    eps = 0.25
    _, ye = oracle.rs_add_rmsnorm([x], 0, z, np.ones(64), eps, False)
    ms = float(np.mean(x.astype(np.float64) ** 2))
    assert np.allclose(ye, x.astype(np.float64) / math.sqrt(ms + eps), rtol=1e-14, atol=0)


def test_sp_single_rank_is_the_plain_add_norm():
    rng = np.random.default_rng(9)
    P = torch.randn(5, 16).to(torch.bfloat16).float().numpy()
    R = torch.randn(5, 16).to(torch.bfloat16).float().numpy()
    got, _ = oracle.rs_add_rmsnorm([P], 0, R, np.ones(16), 1e-5, True)
    # one fp32 add then torch's own RNE conversion to bf16
    ref = (torch.from_numpy(P) + torch.from_numpy(R)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)


def test_rmsnorm_reads_the_stored_residual():
    """The norm is taken of the new residual stream as stored (bf16-rounded),
    not of the unrounded fp32 sum: rows whose rounding moves the mean square
    tell the two apart."""
    n, t = 2, 2
    parts = [np.zeros((n, 2), np.float32) for _ in range(t)]
    for c in range(n):
        parts[c][c] = [1.0, 1.0]
        parts[(c + 1) % t][c] = [2.0 ** -8, 0.0]
    res = np.full((1, 2), 2.0 ** -16, np.float32)
    for r in range(t):
        stored, out = oracle.rs_add_rmsnorm(parts, r, res, np.ones(2), 0.0, True)
        assert stored[0].tolist() == [1.0 + 2.0 ** -7, 1.0]
        v = np.array([1.0 + 2.0 ** -7, 1.0])
        assert np.allclose(out[0], v / math.sqrt(np.mean(v * v)), rtol=1e-15, atol=0)
        u = np.array([1.0 + 2.0 ** -8 + 2.0 ** -16, 1.0 + 2.0 ** -16])
        assert not np.allclose(out[0], u / math.sqrt(np.mean(u * u)), rtol=1e-6, atol=0)


# --------------------------------------------------------------------------
# one-shot (rank-order) reduce; logits gather + greedy argmax
# --------------------------------------------------------------------------

def test_rank_order_reduce_ties_and_zero_start():
    """((0 + P_0) + P_1) + P_2: on the ring pin's data the 1 + 2^-23 lands on
    element 2 (ring order puts it on element 1); the zero start turns a sum
    of negative zeros into +0."""
    e = np.float32(2.0 ** -24)
    one = np.float32(1.0)
    P0 = np.array([e, one, e], dtype=np.float32)
    P1 = np.array([one, e, e], dtype=np.float32)
    P2 = np.array([e, e, one], dtype=np.float32)
    assert oracle.reduce_rank_f32([P0, P1, P2]).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -23]
    assert oracle.ring_allreduce_f32([P0, P1, P2]).tolist() == [1.0, 1.0 + 2.0 ** -23, 1.0]
    z = oracle.reduce_rank_f32([np.array([-0.0], np.float32)] * 3)
    assert z[0] == 0.0 and not np.signbit(z[0])


@pytest.mark.parametrize("t", [1, 2, 5, 8])
def test_rank_order_reduce_is_exact_on_representable_sums(t):
    K = 37
    parts = [np.full(K, float(1 << r), np.float32) * (1 + np.arange(K) % 5) for r in range(t)]
    out = oracle.reduce_rank_f32(parts)
    assert np.array_equal(out, sum(p.astype(np.float64) for p in parts).astype(np.float32))


@pytest.mark.parametrize("V,t", [(10, 3), (11, 4), (7, 8), (151936, 2)])
def test_logits_gather_is_the_full_logits_and_argmax_matches_torch(V, t):
    """Concatenating the rank shards gives X.E^T over the whole vocabulary
    (trailing ranks may be short or empty); the greedy pick is
    torch.argmax of that row (the call the pages' generation loop makes)."""
    rng = np.random.default_rng(V + t)
    n, h = 3, 8
    X = rng.standard_normal((n, h))
    E = rng.standard_normal((V, h))
    shards = [oracle.lm_head_rank(X, E, r, t) for r in range(t)]
    full, am = oracle.logits_gather_argmax(shards, V)
    assert np.allclose(full, X @ E.T, rtol=1e-12, atol=1e-12)
    assert am.tolist() == torch.argmax(torch.from_numpy(full), dim=1).tolist()


def test_argmax_ties_take_the_first_index_and_nan_wins():
    t, V = 3, 7                                   # shards of 3, 3, 1 columns
    row_tie = [[1.0, 5.0, 2.0], [5.0, 0.0, 5.0], [-1.0]]
    row_nan = [[1.0, 2.0, 3.0], [9.0, float("nan"), 10.0], [float("nan")]]
    row_neg = [[-3.0, -2.0, -2.0], [-7.0, -2.5, -9.0], [-2.0]]
    shards = [np.array([row_tie[r], row_nan[r], row_neg[r]]) for r in range(t)]
    _, am = oracle.logits_gather_argmax(shards, V)
    assert am.tolist() == [1, 4, 1]
    full = torch.tensor([[1.0, 5.0, 2.0, 5.0, 0.0, 5.0, -1.0], [1.0, 2.0, 3.0, 9.0, float("nan"), 10.0, float("nan")],
                         [-3.0, -2.0, -2.0, -7.0, -2.5, -9.0, -2.0]], dtype=torch.float64)
    assert torch.argmax(full, dim=1).tolist() == [1, 4, 1]


# --------------------------------------------------------------------------
# head-parallel attention core
# --------------------------------------------------------------------------

def _sdpa64(qkv, nq, nkv, d, causal):
    n = qkv.shape[0]
    t = torch.from_numpy(qkv)
    q = t[:, :nq * d].reshape(n, nq, d).transpose(0, 1)
    k = t[:, nq * d:(nq + nkv) * d].reshape(n, nkv, d).transpose(0, 1).repeat_interleave(nq // nkv, 0)
    v = t[:, (nq + nkv) * d:].reshape(n, nkv, d).transpose(0, 1).repeat_interleave(nq // nkv, 0)
    mask = torch.ones(n, n, dtype=torch.bool).tril() if causal else None
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask).transpose(0, 1).reshape(n, nq * d).numpy()


@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2), (4, 1), (8, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_torch_sdpa(nq, nkv, causal):
    """The library routine the pages' TP attention calls, in float64, with
    the KV heads repeated for GQA and the causal tril mask."""
    rng = np.random.default_rng(nq * 10 + nkv + causal)
    n, d = 23, 16
    qkv = rng.standard_normal((n, (nq + 2 * nkv) * d))
    got = oracle.attention_rank(qkv, nq, nkv, d, causal)
    assert np.allclose(got, _sdpa64(qkv, nq, nkv, d, causal), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    n, nq, nkv, d = 6, 2, 1, 4
    rng = np.random.default_rng(3)
    qkv = rng.standard_normal((n, (nq + 2 * nkv) * d))
    # identical keys: uniform weights, so each query averages the visible V rows
    qkv[:, nq * d:(nq + nkv) * d] = qkv[0, nq * d:(nq + nkv) * d]
    V = qkv[:, (nq + nkv) * d:]
    causal = oracle.attention_rank(qkv, nq, nkv, d, True)
    full = oracle.attention_rank(qkv, nq, nkv, d, False)
    for i in range(n):
        for h in range(nq):
            assert np.allclose(causal[i, h * d:(h + 1) * d], V[:i + 1].mean(axis=0), rtol=1e-14, atol=1e-14)
            assert np.allclose(full[i, h * d:(h + 1) * d], V.mean(axis=0), rtol=1e-14, atol=1e-14)
    # the first query sees only key 0: its output is V[0] exactly
    qkv2 = rng.standard_normal((n, (nq + 2 * nkv) * d))
    out = oracle.attention_rank(qkv2, nq, nkv, d, True)
    assert np.array_equal(out[0, :d], qkv2[0, (nq + nkv) * d:])
    # one dominant key: the output is (to fp64 rounding) that key's V row
    qkv3 = np.zeros((n, (nq + 2 * nkv) * d))
    qkv3[:, 0] = 1.0                                   # query head 0: e_0
    qkv3[4, nq * d] = 200.0                            # key 4 along e_0
    qkv3[:, (nq + nkv) * d:] = np.arange(n)[:, None]
    out3 = oracle.attention_rank(qkv3, nq, nkv, d, False)
    assert np.allclose(out3[:, :d], 4.0, rtol=0, atol=1e-12)


def test_attention_head_parallel_ranks_concatenate_to_full():
    """[VLLM13] §2.3.3: each rank computes attention for its own heads with no
    communication; the ranks' outputs side by side are the full output."""
    rng = np.random.default_rng(11)
    n, nq, nkv, d, t = 17, 8, 4, 8, 2
    qkv = rng.standard_normal((n, (nq + 2 * nkv) * d))
    full = oracle.attention_rank(qkv, nq, nkv, d, True)
    q, k, v = qkv[:, :nq * d], qkv[:, nq * d:(nq + nkv) * d], qkv[:, (nq + nkv) * d:]
    lq, lk = nq // t, nkv // t
    parts = []
    for r in range(t):
        sub = np.concatenate([q[:, r * lq * d:(r + 1) * lq * d], k[:, r * lk * d:(r + 1) * lk * d],
                              v[:, r * lk * d:(r + 1) * lk * d]], axis=1)
        parts.append(oracle.attention_rank(sub, lq, lk, d, True))
    assert np.allclose(np.concatenate(parts, axis=1), full, rtol=1e-13, atol=1e-14)


def test_attention_rows_are_independent():
    rng = np.random.default_rng(12)
    n, nq, nkv, d = 19, 4, 1, 8
    qkv = rng.standard_normal((n, (nq + 2 * nkv) * d))
    full = oracle.attention_rank(qkv, nq, nkv, d, True)
    rows = [18, 0, 7]
    assert np.array_equal(oracle.attention_rank(qkv, nq, nkv, d, True, rows=rows), full[rows])


# --------------------------------------------------------------------------
# Checkpoint-style loaders: [NANO22] §3-§5 weight_loader on the full tensor,
# shard selected before the dtype conversion ([MINISGL] §8)
# --------------------------------------------------------------------------

def _bits_to_f64(b):
    return oracle.bf16_bits_to_f64(b)


def test_loader_worked_examples():
    """The printed runs of [NANO22] §3 (column cut), §4 (row cut) and §5
    (merged q/k/v and gate/up, one projection per call), through the loaders
    with a float32 -> bfloat16 conversion (all values are exact in bf16)."""
    g = gold("nano22_column_parallel.json")
    full = np.array([[v] * g["in_features"] for v in g["full_row_labels"]], dtype=np.float32)
    for r, rows in g["rank_rows"].items():
        got = _bits_to_f64(oracle.load_shard(full, 0, int(r), g["tp_size"], True))
        assert got.shape == tuple(g["rank_weight_shape"]) and got[:, 0].tolist() == rows
    g = gold("nano22_row_parallel.json")
    w = np.array(g["weight"], dtype=np.float32)
    for r, cols in g["rank_cols"].items():
        assert _bits_to_f64(oracle.load_shard(w, 1, int(r), g["tp_size"], True)).tolist() == cols
    g = gold("nano22_merged_double_cut.json")
    q = g["qkv"]
    hd, hid, t = q["head_size"], q["hidden"], q["tp_size"]
    srcs = [_by_head(q["num_q_heads"], q["q_base"], hd, hid), _by_head(q["num_kv_heads"], q["k_base"], hd, hid),
            _by_head(q["num_kv_heads"], q["v_base"], hd, hid)]
    for r in range(t):
        table = np.zeros(((q["num_q_heads"] // t + 2 * (q["num_kv_heads"] // t)) * hd, hid), dtype=np.uint16)
        for sid in (2, 0, 1):                          # any order of the three calls
            oracle.load_qkv(table, srcs[sid], sid, q["num_q_heads"], q["num_kv_heads"], hd, r, t)
        c = _bits_to_f64(table)[:, 0].tolist()
        exp = q[f"rank{r}"]
        nq, nk = len(exp["q"]), len(exp["k"])
        assert c[:nq] == exp["q"] and c[nq:nq + nk] == exp["k"] and c[nq + nk:] == exp["v"]
    gu = g["gate_up"]
    table = np.zeros((2 * gu["intermediate"] // gu["tp_size"], gu["hidden"]), dtype=np.float32)
    oracle.load_gate_up(table, np.full((gu["intermediate"], gu["hidden"]), gu["gate_fill"], np.float32), 0, 0,
                        gu["tp_size"])
    oracle.load_gate_up(table, np.full((gu["intermediate"], gu["hidden"]), gu["up_fill"], np.float32), 1, 0,
                        gu["tp_size"])
    half = gu["intermediate"] // gu["tp_size"]
    assert table[:half, 0].tolist() == gu["rank0"]["gate_segment"]
    assert table[half:, 0].tolist() == gu["rank0"]["up_segment"]


def test_loader_conversion_is_torch_copy_into_bf16_param():
    """The pages' loaders end in param.data.copy_(loaded_weight): copying a
    float32 chunk into a bfloat16 parameter is torch's round to nearest even
    (ties, subnormals and infinities included; a NaN stays a NaN); bf16 ->
    fp32 is exact."""
    rng = np.random.default_rng(21)
    src = rng.standard_normal((16, 64)).astype(np.float32)
    src[0, :8] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, np.inf, -np.inf, np.nan, 0.0],
                          dtype=np.float32)
    src[1, :4] = np.array([3.0e38, -3.0e38, 1e-40, -0.0], dtype=np.float32)
    for dim in (0, 1):
        for r in range(4):
            got = oracle.load_shard(src, dim, r, 4, True)
            chunk = torch.from_numpy(src).chunk(4, dim)[r]
            param = torch.empty(chunk.shape, dtype=torch.bfloat16)
            param.copy_(chunk)
            ref = param.view(torch.int16).numpy().view(np.uint16)
            # a NaN stays a NaN (its payload bits are not fixed)
            nan_got = (got & 0x7F80) == 0x7F80
            nan_got &= (got & 0x007F) != 0
            assert np.array_equal(nan_got, torch.isnan(param).numpy())
            assert np.array_equal(got[~nan_got], ref[~nan_got])
    b = oracle.f32_to_bf16_bits(src)
    back = oracle.load_shard(b, 0, 1, 2, False)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).chunk(2, 0)[1].float().numpy()
    assert np.array_equal(back.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n_q,n_kv,t", [(8, 2, 2), (8, 2, 8), (64, 8, 16), (4, 4, 4)])
def test_loader_tables_equal_shard_then_convert(n_q, n_kv, t):
    """Loading the projections one at a time gives the merged table of the
    full tensors' shard selection ([NANO22] §5 / [GUIDE62] §2.2 replication),
    converted; the segment order is q, k, v and gate, up."""
    rng = np.random.default_rng(n_q * 100 + t)
    hd, h, f = 4, 6, 8 * t
    wq = rng.standard_normal((n_q * hd, h)).astype(np.float32)
    wk = rng.standard_normal((n_kv * hd, h)).astype(np.float32)
    wv = rng.standard_normal((n_kv * hd, h)).astype(np.float32)
    gate = rng.standard_normal((f, h)).astype(np.float32)
    up = rng.standard_normal((f, h)).astype(np.float32)
    for r in range(t):
        ref = oracle.shard_qkv(oracle.f32_to_bf16_bits(wq), oracle.f32_to_bf16_bits(wk), oracle.f32_to_bf16_bits(wv),
                               n_q, n_kv, hd, r, t)
        table = np.full(ref.shape, 0xFFFF, dtype=np.uint16)
        for sid, src in enumerate((wq, wk, wv)):
            oracle.load_qkv(table, src, sid, n_q, n_kv, hd, r, t)
        assert np.array_equal(table, ref)
        ref = oracle.shard_gate_up(oracle.f32_to_bf16_bits(gate), oracle.f32_to_bf16_bits(up), r, t)
        table = np.full(ref.shape, 0xFFFF, dtype=np.uint16)
        oracle.load_gate_up(table, up, 1, r, t)
        oracle.load_gate_up(table, gate, 0, r, t)
        assert np.array_equal(table, ref)


def test_loader_wrong_segment_or_chunk_is_caught():
    """Putting k where v belongs, or taking the chunk of the wrong rank, fails
    the comparison with the shard selection of the full tensors."""
    rng = np.random.default_rng(3)
    n_q, n_kv, hd, h, t = 4, 2, 2, 3, 2
    wq = rng.standard_normal((n_q * hd, h)).astype(np.float32)
    wk = rng.standard_normal((n_kv * hd, h)).astype(np.float32)
    wv = rng.standard_normal((n_kv * hd, h)).astype(np.float32)
    ref = oracle.shard_qkv(wq, wk, wv, n_q, n_kv, hd, 1, t)
    table = np.zeros_like(ref)
    oracle.load_qkv(table, wq, 0, n_q, n_kv, hd, 1, t)
    oracle.load_qkv(table, wv, 1, n_q, n_kv, hd, 1, t)      # v into k's segment
    oracle.load_qkv(table, wk, 2, n_q, n_kv, hd, 1, t)
    assert not np.array_equal(table, ref)
    other = np.zeros_like(ref)
    for sid, src in enumerate((wq, wk, wv)):
        oracle.load_qkv(other, src, sid, n_q, n_kv, hd, 0, t)   # rank 0's chunks
    assert not np.array_equal(other, ref)
