"""The compute entry points under stream capture: they launch kernels on the
caller's stream only (no allocation, synchronisation or memset), so a
captured sequence replays as a graph.  Every replay is compared bit for bit
with an eager call on the same inputs, with eager work and synchronisation
between the replays and the inputs rewritten in place before each one."""
import pytest
import torch

import synth
from rank_sharded_layer_amd import tpshard as T

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _mlp_case(n, h, fl, seed):
    x = synth.normal((n, h), 1.0, seed, torch.bfloat16, device=DEV)
    wgu = synth.normal((2 * fl, h), 0.02, seed + 1, torch.bfloat16, device=DEV)
    wd = synth.normal((h, fl), 0.02, seed + 2, torch.bfloat16, device=DEV)
    ws = torch.empty(max(T.tp_mlp_workspace_bytes(n, h, fl, torch.bfloat16), 256), dtype=torch.uint8, device=DEV)
    return x, wgu, wd, ws


@pytest.mark.parametrize("n,h,fl", [
    (64, 8192, 2048),     # decode: register-streaming split-K kernels and their finish passes
    (40, 1024, 392),      # tiled kernels, split-K, ragged tiles
    (1280, 2048, 1536),   # 128 x 128 tiles with K split in four and the split finish
    (2560, 8192, 7168),   # gate_up on 256 x 256 paired-stage tiles with a balanced last round
])
def test_mlp_share_replays_from_a_captured_graph(n, h, fl):
    x, wgu, wd, ws = _mlp_case(n, h, fl, 61)
    out = torch.empty((n, h), dtype=torch.bfloat16, device=DEV)
    T.tp_mlp_rank_forward(x, wgu, wd, partial=out, workspace=ws)     # warm-up, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        T.tp_mlp_rank_forward(x, wgu, wd, partial=out, workspace=ws)
    for rep in range(3):
        x.copy_(synth.normal((n, h), 1.0, 100 + rep, torch.bfloat16, device=DEV))
        ref = T.tp_mlp_rank_forward(x, wgu, wd, workspace=torch.empty_like(ws))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (n, h, fl, rep)


def test_attention_and_reduce_replay_from_a_captured_graph():
    """The attention core (split key chunks and their combine) followed by the
    t-way partial reduce, captured as one sequence."""
    n, nq, nkv, t = 1536, 4, 1, 4
    qkv = synth.normal((n, (nq + 2 * nkv) * 128), 1.0, 71, torch.bfloat16, device=DEV)
    att = torch.empty((n, nq * 128), dtype=torch.bfloat16, device=DEV)
    aws = torch.empty(max(T.tp_attention_workspace_bytes(n, nq, nkv, 128, True), 256), dtype=torch.uint8,
                      device=DEV)
    parts = [synth.normal((n, 512), 1.0, 80 + r, torch.bfloat16, device=DEV) for r in range(t)]
    red = torch.empty((n, 512), dtype=torch.bfloat16, device=DEV)
    T.tp_attention_rank(qkv, nq, nkv, causal=True, out=att, workspace=aws)
    T.tp_partial_reduce(parts, out=red)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        T.tp_attention_rank(qkv, nq, nkv, causal=True, out=att, workspace=aws)
        T.tp_partial_reduce(parts, out=red)
    for rep in range(3):
        qkv.copy_(synth.normal(tuple(qkv.shape), 1.0, 90 + rep, torch.bfloat16, device=DEV))
        parts[0].copy_(synth.normal((n, 512), 1.0, 95 + rep, torch.bfloat16, device=DEV))
        ref_att = T.tp_attention_rank(qkv, nq, nkv, causal=True, workspace=torch.empty_like(aws))
        ref_red = T.tp_partial_reduce(parts)
        att.zero_()
        red.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(att, ref_att), rep
        assert torch.equal(red, ref_red), rep
