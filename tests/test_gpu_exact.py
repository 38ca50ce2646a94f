"""Bit-exact GPU checks of every production GEMM kernel at the shapes the
benchmark times, element by element over the whole output.

A linear layer computes y = x . W^T with weights stored [out, in] (Nano-vLLM
walkthrough no. 22, §2).  With one-hot token rows, x[i] = e_j(i), every
output is a single product 1.0 * W[c, j(i)] plus exact zeros, so
y[i, c] = W[c, j(i)] exactly in fp32 and after rounding to bf16: a wrong
element anywhere (a transposed operand, a misplaced fragment, a lost K
piece of a split or balanced-last-round tile, a bad store offset) shows up
as a mismatched bit pattern.

The gated product act = SiLU(x . G^T) * (x . U^T) (Tensor parallelism:
implemented from scratch, Implementation, class TPMLP) is made exact the
same way: the gate weights are integers in [20, 83], for which
1 + e^-g rounds to 1 in fp32, so SiLU(g) = g exactly and
act[i, c] = bf16(G[c, j] * U[c, j]), where the fp32 product of an integer
under 128 and a bf16 value is exact.  The gate values differ from row to
row and column to column, so a gate row read in place of another (or an up
row in place of a gate row) changes the result.

Shapes and the kernel the planner gives each (the launch configuration the
benchmark times):
  prefill gate_up   8192 x 8192 -> 2 x 3584   256x256 paired-stage tiles, balanced last round
  prefill down      8192 x 3584 -> 8192       256x256 paired-stage tiles, 4 full rounds
  decode gate_up      64 x 8192 -> 2 x 7168   register streaming, 8 K slices of 1024 + slice-order finish
  decode down         64 x 7168 -> 8192       register streaming, 7 K slices of 1024 + slice-order finish
  QKV (TP=16)       8192 x 8192 -> 768        256x192 paired-stage tiles, K split in two + split finish
  o_proj (TP=16)    8192 x  512 -> 8192       256x256 paired-stage tiles, K = 512
  LM head (TP=2)     512 x 1024 -> 75968 fp32 256x256 tiles, fp32 rows staged through LDS
  fp32 MLP (TP=2)     16 x 1024 -> 2 x 1536, 16 x 1536 -> 1024   fp32 small-M kernels
                      (8 act columns, and 4 output columns, per workgroup)
and the kernels other shapes take: the register-streaming kernel at
narrower outputs, the LDS-ring streaming decode kernel with its finish
pass, 64x128 split-K
tiles (the QKV projection of one decode step at TP=16), and the
element-wise register-staged tiles (K not a multiple of 8).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from rank_sharded_layer_amd import tpshard as T
from tests.helpers import bits, relf, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def one_hot_rows(n, k, dtype, salt=13):
    """x[i] = e_j(i) with j(i) = (7919 i + salt) mod k (7919 is an odd prime,
    so the columns spread over every K slice and tile)."""
    j = (np.arange(n, dtype=np.int64) * 7919 + salt) % k
    x = torch.zeros((n, k), dtype=dtype, device=DEV)
    x[torch.arange(n, device=DEV), torch.from_numpy(j).to(DEV)] = 1
    return x, j


def gate_values(rows, k, dtype):
    """Integers 20 .. 83 that vary along rows and columns."""
    c = torch.arange(rows, device=DEV, dtype=torch.int64)[:, None]
    kk = torch.arange(k, device=DEV, dtype=torch.int64)[None, :]
    return (20 + (c + 3 * kk) % 64).to(dtype)


def check_linear_exact(n, k, m, out_dtype, seed):
    x, j = one_hot_rows(n, k, torch.bfloat16)
    w = synth.normal((m, k), 0.02, seed, torch.bfloat16, device=DEV)
    y = T.tp_linear_rank_forward(x, w, out_dtype=out_dtype)
    torch.cuda.synchronize()
    wb = bits(w)                                  # [m, k] uint16
    ref = np.ascontiguousarray(wb[:, j].T)        # y[i, c] = w[c, j(i)]
    if out_dtype == torch.float32:
        ref = ref.astype(np.uint32) << 16         # bf16 -> fp32 is exact
    got = bits(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    # and the same rows through the fp64 oracle's product
    rows = synth.sample_rows(n, 3, seed + 1)
    assert relf(to_f64(y)[rows], oracle.linear(to_f64(x)[rows], to_f64(w))) == 0.0


def check_gate_up_exact(n, h, fl, seed):
    x, j = one_hot_rows(n, h, torch.bfloat16)
    gate = gate_values(fl, h, torch.bfloat16)
    up = synth.normal((fl, h), 0.02, seed, torch.bfloat16, device=DEV)
    wgu = torch.cat([gate, up], 0).contiguous()
    act = T.tp_gate_up_act_rank(x, wgu)
    torch.cuda.synchronize()
    g = to_f64(gate)[:, j].T.astype(np.float32)   # [n, fl], integers 20..83
    u = to_f64(up)[:, j].T.astype(np.float32)
    prod = g * u                                  # exact in fp32
    assert np.array_equal(prod.astype(np.float64), g.astype(np.float64) * u.astype(np.float64))
    ref = oracle.f32_to_bf16_bits(prod)
    got = bits(act)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    # the oracle's SiLU agrees up to the e^-20 it keeps
    rows = synth.sample_rows(n, 3, seed + 1)
    xr = to_f64(x)[rows]
    ref64 = oracle.silu_mul(oracle.linear(xr, to_f64(gate)), oracle.linear(xr, to_f64(up)))
    assert relf(to_f64(act)[rows], ref64) < 1e-2


# ---- prefill (one rank of TP=8, Llama-3.1-70B shapes) --------------------------

def test_prefill_gate_up_paired_tiles_balanced_round_bit_exact():
    w = synth.get("llama70b_prefill_tp8")
    check_gate_up_exact(w.n, w.h, w.f_local, w.seed(synth.T_UP))


def test_prefill_down_paired_tiles_bit_exact():
    w = synth.get("llama70b_prefill_tp8")
    check_linear_exact(w.n, w.f_local, w.h, torch.bfloat16, w.seed(synth.T_DOWN))


# ---- decode (one rank of TP=4) -------------------------------------------------

def test_decode_gate_up_register_streaming_bit_exact():
    w = synth.get("llama70b_decode_tp4")
    check_gate_up_exact(w.n, w.h, w.f_local, w.seed(synth.T_UP))


def test_decode_down_register_streaming_bit_exact():
    w = synth.get("llama70b_decode_tp4")
    check_linear_exact(w.n, w.f_local, w.h, torch.bfloat16, w.seed(synth.T_DOWN))


# ---- attention projections (one rank of TP=16) -----------------------------------

def test_qkv_projection_bit_exact():
    w = synth.get("llama70b_attnproj_tp16")
    rows = (w.n_q // w.tp + 2) * w.head_dim          # 4 q heads + 1 k + 1 v = 768
    check_linear_exact(w.n, w.h, rows, torch.bfloat16, w.seed(synth.T_WQ))


def test_o_proj_bit_exact():
    w = synth.get("llama70b_attnproj_tp16")
    check_linear_exact(w.n, w.n_q // w.tp * w.head_dim, w.h, torch.bfloat16, w.seed(synth.T_WO))


# ---- LM head (one rank of TP=2, Qwen3 vocab), fp32 logits ---------------------------

def test_lm_head_fp32_store_bit_exact():
    w = synth.get("qwen3_vocab_tp2")
    check_linear_exact(w.n, w.h, w.vocab // w.tp, torch.float32, w.seed(synth.T_TABLE))


# ---- fp32 MLP (one rank of TP=2, Qwen3-0.6B shapes) -------------------------------

def test_fp32_small_m_kernels_bit_exact():
    w = synth.get("qwen3_mlp_tp2_fp32")
    fl = w.f_local
    x, j = one_hot_rows(w.n, w.h, torch.float32)
    gate = gate_values(fl, w.h, torch.float32)
    up = synth.normal((fl, w.h), 0.02, w.seed(synth.T_UP), torch.float32, device=DEV)
    act = T.tp_gate_up_act_rank(x, torch.cat([gate, up], 0).contiguous())
    g = gate.cpu().numpy()[:, j].T
    u = up.cpu().numpy()[:, j].T
    assert np.array_equal(bits(act), (g * u).view(np.uint32))     # fp32 product, rounded once
    xd, jd = one_hot_rows(w.n, fl, torch.float32)
    down = synth.normal((w.h, fl), 0.02, w.seed(synth.T_DOWN), torch.float32, device=DEV)
    y = T.tp_linear_rank_forward(xd, down)
    assert np.array_equal(bits(y), np.ascontiguousarray(bits(down)[:, jd].T))


@pytest.mark.parametrize("m,k,n,gated", [
    (16, 1024, 1000, False),    # 4 columns per workgroup, ragged last block
    (20, 100, 2100, False),     # 8 columns, two token blocks, one K step per wave
    (16, 512, 4200, False),     # 16 columns
    (16, 1024, 100, True),      # gated, 8 act columns (8 gate + 8 up rows), ragged
    (32, 2048, 4100, True),     # gated, 16 act columns (two row blocks), two token blocks
])
def test_fp32_small_m_column_blocks_bit_exact(m, k, n, gated):
    """The fp32 small-M kernel at every column-block width it takes (16, 8
    or 4 output columns per workgroup) with ragged edges: one-hot tokens
    make each output a single exact product."""
    x, j = one_hot_rows(m, k, torch.float32, salt=5)
    if gated:
        gate = gate_values(n, k, torch.float32)
        up = synth.normal((n, k), 0.02, 409, torch.float32, device=DEV)
        y = T.tp_gate_up_act_rank(x, torch.cat([gate, up], 0).contiguous())
        ref = gate.cpu().numpy()[:, j].T * up.cpu().numpy()[:, j].T
    else:
        w = synth.normal((n, k), 0.02, 410, torch.float32, device=DEV)
        y = T.tp_linear_rank_forward(x, w)
        ref = np.ascontiguousarray(w.cpu().numpy()[:, j].T)
    torch.cuda.synchronize()
    bad = np.argwhere(bits(y) != np.ascontiguousarray(ref, dtype=np.float32).view(np.uint32))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


# ---- kernels of other decode-sized shapes ---------------------------------------

def test_register_streaming_narrow_outputs_bit_exact():
    """Narrower outputs with long K: K slices of 1024, fp32 partial tiles
    added in slice order by the finish pass."""
    check_linear_exact(64, 6144, 4000, torch.bfloat16, 401)
    check_gate_up_exact(64, 8192, 4096, 402)


def test_lds_ring_streaming_bit_exact():
    """Shorter K with few 16-row blocks: the persistent LDS-ring kernel."""
    check_gate_up_exact(64, 4000, 2040, 403)
    check_linear_exact(64, 2040, 4000, torch.float32, 404)


def test_split_k_64x128_tiles_bit_exact():
    """One decode step's QKV projection at TP=16 (64 x 8192 -> 768): 64x128
    deep-pipelined tiles with K split for occupancy and a split-order finish."""
    check_linear_exact(64, 8192, 768, torch.bfloat16, 405)


def test_element_wise_register_staged_tiles_bit_exact():
    """K = 1001 is not a multiple of 8: 128x128 (M > 64) and 64x128 tiles
    with element-wise loads."""
    check_linear_exact(300, 1001, 520, torch.bfloat16, 406)
    check_linear_exact(40, 1001, 520, torch.float32, 407)
    check_gate_up_exact(40, 1001, 200, 408)
