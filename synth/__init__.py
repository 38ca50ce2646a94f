"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module holds no arithmetic of the method: it only draws random numbers
(torch's counter-based Philox generator on either device) and states the
workload shapes.  Both sides receive the exact same bits.

Recipe (stated once here):
  * one generator per tensor, seeded by mix(42, config_id, tensor_id); 42 is
    the seed the pages' numpy demos use;
  * activations x ~ N(0, 1), weights and tables ~ N(0, 0.02), drawn in fp32;
  * bf16 workloads round the fp32 draws to bf16 (round-to-nearest-even, the
    rounding torch's .to(bfloat16) performs); fp32 workloads keep the draws;
  * token ids are uniform integers in [0, vocab) (int64);
  * generation may run on the GPU for the large shapes; the CPU and GPU
    generators give different streams, so a test always feeds one tensor to
    both sides rather than regenerating it.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

BASE_SEED = 42

# tensor ids within a workload
T_X, T_GATE, T_UP, T_DOWN, T_TABLE, T_IDS = 0, 1, 2, 3, 4, 5
T_WQ, T_WK, T_WV, T_WO = 6, 7, 8, 9
T_NORM_W = 10
T_ATTN_OUT = 100      # + rank
T_PARTIAL = 200       # + rank
T_RESIDUAL = 300      # + rank

W_STD = 0.02
X_STD = 1.0


def mix(config_id: int, tensor_id: int, base: int = BASE_SEED) -> int:
    s = (base * 1_000_003 + config_id) * 1_000_003 + tensor_id
    return s % (1 << 62)


def normal(shape, std: float, seed: int, dtype: torch.dtype = torch.bfloat16,
           device="cpu") -> torch.Tensor:
    """fp32 N(0, std^2) draws, rounded to `dtype` when it is bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    a = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        a.mul_(std)
    if dtype == torch.float32:
        return a
    return a.to(dtype)


def token_ids(n: int, vocab: int, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int64)


def sample_rows(n: int, count: int, seed: int):
    """Sorted distinct row indices for sampled checks (always includes the last row)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    count = min(count, n)
    idx = torch.randperm(n, generator=g)[:count].tolist()
    if n - 1 not in idx:
        idx[-1] = n - 1
    return sorted(set(idx))


@dataclass
class Workload:
    """Shapes of one synthetic workload shaped like the pages' examples."""
    config_id: int
    name: str
    kind: str                  # "mlp" | "vocab" | "attn_proj"
    dtype: torch.dtype
    tp: int
    n: int
    h: int
    f: int = 0                 # full MLP intermediate size
    vocab: int = 0
    n_q: int = 0
    n_kv: int = 0
    head_dim: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def f_local(self) -> int:
        return self.f // self.tp

    def seed(self, tensor_id: int) -> int:
        return mix(self.config_id, tensor_id)


WORKLOADS = {
    "qwen3_mlp_tp2_fp32": Workload(
        0, "qwen3_mlp_tp2_fp32", "mlp", torch.float32, tp=2, n=16, h=1024, f=3072,
        note="Qwen3-0.6B-shaped MLP, TP=2, fp32"),
    "qwen3_vocab_tp2": Workload(
        1, "qwen3_vocab_tp2", "vocab", torch.bfloat16, tp=2, n=512, h=1024, vocab=151936,
        note="Qwen3-0.6B-shaped vocab-parallel embedding + LM head, TP=2, bf16"),
    "llama70b_decode_tp4": Workload(
        2, "llama70b_decode_tp4", "mlp", torch.bfloat16, tp=4, n=64, h=8192, f=28672,
        note="Llama-3.1-70B-shaped decode MLP, one rank of TP=4, bf16"),
    "llama70b_prefill_tp8": Workload(
        3, "llama70b_prefill_tp8", "mlp", torch.bfloat16, tp=8, n=8192, h=8192, f=28672,
        note="Llama-3.1-70B-shaped prefill MLP chunk, one rank of TP=8, bf16"),
    "llama70b_attnproj_tp16": Workload(
        4, "llama70b_attnproj_tp16", "attn_proj", torch.bfloat16, tp=16, n=8192, h=8192,
        n_q=64, n_kv=8, head_dim=128,
        note="Llama-3.1-70B-shaped QKV/o_proj at TP=16 with GQA KV replication, bf16"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
