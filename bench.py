"""Benchmark of one tensor-parallel rank's share of a Transformer layer on one MI355X.

Step (the timed unit): one rank's MLP share at the Llama-3.1-70B prefill
shape, one rank of TP=8 (n=8192 tokens, h=8192, f_local=3584, bf16):
  fused column-parallel gate_up GEMM with the SiLU(gate)*up epilogue,
  row-parallel down GEMM -> full-shape [8192, 8192] bf16 partial,
  ring-order reduce of that partial with the 7 other ranks' partials.
Inputs are resident in HBM before timing starts.  Before the W warmup
steps, the step runs untimed for --settle-ms of wall time: under sustained
MFMA load the GPU's power management takes tens of milliseconds to reach its
steady state (back-to-back gate_up launches fall from ~1.17 ms to ~0.71 ms
over the first ~70 ms), and the figure reported is the steady state.  `value` is the MLP's
TFLOP/s over its two launches (algorithmic FLOP / measured time);
`ms_per_step` covers the whole step, reduce included.

Further legs, each timed on its own with HIP events on the library's stream:
decode MLP (n=64, one rank of TP=4, HBM-bound, weights rotated over 3
copies so the 256 MB Infinity Cache cannot hold them), the reduce at 8 and 16
ranks, the vocab-parallel embedding + LM head (TP=2), the attention
projections at TP=16 and the fp32 Qwen3 MLP.  A bounded sample of the fp64
CPU oracle is timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--legs all|none|a,b]
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from rank_sharded_layer_amd import tpshard as T  # noqa: E402

METRIC = "rank-shard MLP TFLOP/s (n=8192) & HBM GB/s (n=64); partial-reduce GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
DEV = "cuda:0"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class EventTimer:
    """Accumulates elapsed time of bracketed regions with HIP events recorded
    on torch's current stream (the stream every library call is issued on)."""

    def __init__(self):
        self.pairs = {}

    def start(self, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs.setdefault(name, []).append([ev, None])

    def stop(self, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs[name][-1][1] = ev

    def all_ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs[name]]

    def ms(self, name):
        """Median milliseconds per region."""
        return median(self.all_ms(name))

    def stats(self, name):
        return stats(self.all_ms(name))


def median(v):
    s = sorted(v)
    m = len(s) // 2
    return s[m] if len(s) % 2 else 0.5 * (s[m - 1] + s[m])


def stats(v):
    """median / min / max (ms) of repeated measurements"""
    return {"median": round(median(v), 5), "min": round(min(v), 5), "max": round(max(v), 5), "n": len(v)}


def batched_ms(fn, n_calls, n_batches=7, prime=3):
    """Per-call milliseconds of `fn(i)` over n_batches batches of n_calls
    back-to-back calls, each batch between one event pair (the GPU never
    waits for the host inside a batch).  Returns the per-batch averages."""
    for i in range(prime):
        fn(i)
    torch.cuda.synchronize()
    out = []
    k = 0
    for _ in range(n_batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_calls):
            fn(k)
            k += 1
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n_calls)
    return out


def gen(w, tid, shape, std):
    return synth.normal(shape, std, w.seed(tid), w.dtype, device=DEV)


# ---------------------------------------------------------------------------
# main step: prefill MLP share + reduce
# ---------------------------------------------------------------------------

def prefill_setup():
    w = synth.get("llama70b_prefill_tp8")
    r = 0
    x = gen(w, synth.T_X, (w.n, w.h), 1.0)
    gate = gen(w, synth.T_GATE, (w.f, w.h), 0.02)
    up = gen(w, synth.T_UP, (w.f, w.h), 0.02)
    down = gen(w, synth.T_DOWN, (w.h, w.f), 0.02)
    wgu = T.tp_shard_gate_up(gate, up, r, w.tp)
    wd = T.tp_shard_weights(down, 1, r, w.tp)
    del gate, up, down
    fl = w.f_local
    act = torch.empty((w.n, fl), dtype=w.dtype, device=DEV)
    parts = [torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)]
    parts += [gen(w, synth.T_PARTIAL + q, (w.n, w.h), 1.0) for q in range(1, w.tp)]
    y = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)
    ws_gu = T.tp_gate_up_workspace_bytes(w.n, w.h, fl, w.dtype)
    ws_dn = T.tp_linear_workspace_bytes(w.n, fl, w.h, w.dtype)
    ws = torch.empty(max(ws_gu, ws_dn, 256), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    return dict(w=w, x=x, wgu=wgu, wd=wd, act=act, parts=parts, y=y, ws=ws)


def prefill_step(S, tm=None):
    if tm:
        tm.start("gate_up")
    T.tp_gate_up_act_rank(S["x"], S["wgu"], act=S["act"], workspace=S["ws"])
    if tm:
        tm.stop("gate_up")
        tm.start("down")
    T.tp_linear_rank_forward(S["act"], S["wd"], y=S["parts"][0], workspace=S["ws"])
    if tm:
        tm.stop("down")
        tm.start("reduce")
    T.tp_partial_reduce(S["parts"], out=S["y"])
    if tm:
        tm.stop("reduce")


def mlp_flops(n, h, fl):
    return 2.0 * n * h * (2 * fl) + 2.0 * n * fl * h


def measured_traffic():
    """HBM bytes per gate_up launch from the committed rocprofv3 counter
    summary (FETCH_SIZE/WRITE_SIZE, calibrated on a plain copy), or None if
    the GEMM source changed since those counters were taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "traffic_gate_up_llama70b_prefill_tp8.json")
    src_path = os.path.join(ROOT, "rank_sharded_layer_amd", "csrc", "gemm.hip")
    try:
        rec = json.load(open(rec_path))
        sha = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    except OSError:
        return None
    if rec.get("gemm_source_sha256") != sha:
        return None
    return rec["traffic_bytes_per_launch"]


# ---------------------------------------------------------------------------
# legs
# ---------------------------------------------------------------------------

def leg_decode(reps):
    w = synth.get("llama70b_decode_tp4")
    fl = w.f_local
    x = gen(w, synth.T_X, (w.n, w.h), 1.0)
    gate = gen(w, synth.T_GATE, (w.f, w.h), 0.02)
    up = gen(w, synth.T_UP, (w.f, w.h), 0.02)
    down = gen(w, synth.T_DOWN, (w.h, w.f), 0.02)
    # three ranks' shards as rotating copies: 3 x 352 MB, more than the 256 MB MALL
    copies = [(T.tp_shard_gate_up(gate, up, r, w.tp), T.tp_shard_weights(down, 1, r, w.tp)) for r in range(3)]
    del gate, up, down
    act = torch.empty((w.n, fl), dtype=w.dtype, device=DEV)
    part = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)
    ws = torch.empty(max(T.tp_mlp_workspace_bytes(w.n, w.h, fl, w.dtype),
                         T.tp_gate_up_workspace_bytes(w.n, w.h, fl, w.dtype),
                         T.tp_linear_workspace_bytes(w.n, fl, w.h, w.dtype), 256),
                     dtype=torch.uint8, device=DEV)
    # the 4 ranks' 1 MiB partials, 64 sets (320 MB) rotated for the cold figure
    psets = [[gen(w, synth.T_PARTIAL + q, (w.n, w.h), 1.0) for q in range(w.tp)]]
    psets += [[p.clone() for p in psets[0]] for _ in range(63)]
    y = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)

    # cold: weights rotate over the three copies; warm: one copy over and over
    def mlp(i):
        wgu, wd = copies[i % 3]
        T.tp_mlp_rank_forward(x, wgu, wd, partial=part, workspace=ws)

    def mlp_warm(i):
        T.tp_mlp_rank_forward(x, copies[0][0], copies[0][1], partial=part, workspace=ws)

    def gate_up(i):
        T.tp_gate_up_act_rank(x, copies[i % 3][0], act=act, workspace=ws)

    def down(i):
        T.tp_linear_rank_forward(act, copies[i % 3][1], y=part, workspace=ws)

    def reduce_warm(i):
        T.tp_partial_reduce(psets[0], out=y)

    def reduce_cold(i):
        T.tp_partial_reduce(psets[i % 64], out=y)

    mlp_v = batched_ms(mlp, reps)
    warm_v = batched_ms(mlp_warm, reps)
    gate_up_v = batched_ms(gate_up, reps)
    down_v = batched_ms(down, reps)
    red_warm = batched_ms(reduce_warm, reps)
    red_cold = batched_ms(reduce_cold, 64)
    torch.cuda.synchronize()
    wbytes = (2 * fl * w.h + w.h * fl) * 2
    io = (w.n * w.h + 2 * w.n * fl + w.n * w.h) * 2      # x, act write+read, partial
    red_bytes = (w.tp + 1) * w.n * w.h * 2
    mlp_ms, warm_ms = median(mlp_v), median(warm_v)

    return {
        "workload": w.name, "n": w.n, "h": w.h, "f_local": fl, "tp": w.tp,
        "mlp_ms": mlp_ms, "mlp_ms_stats": stats(mlp_v),
        "gate_up_ms": median(gate_up_v), "gate_up_ms_stats": stats(gate_up_v),
        "down_ms": median(down_v), "down_ms_stats": stats(down_v),
        "mlp_GBps": (wbytes + io) / mlp_ms / 1e6,
        "mlp_hbm_frac": (wbytes + io) / mlp_ms / 1e6 / PEAK_HBM_GBPS,
        "algorithmic_bytes": wbytes + io,
        "mlp_TFLOPs": mlp_flops(w.n, w.h, fl) / mlp_ms / 1e9,
        "warm_mlp_ms": warm_ms, "warm_mlp_ms_stats": stats(warm_v),
        "warm_mlp_GBps": (wbytes + io) / warm_ms / 1e6,
        "reduce_ms": median(red_cold), "reduce_ms_stats": stats(red_cold),
        "reduce_GBps": red_bytes / median(red_cold) / 1e6,
        "warm_reduce_ms": median(red_warm), "warm_reduce_ms_stats": stats(red_warm),
        "reduce_note": "4 x 1 MiB partials: launch bound, not an HBM-roofline claim; cold = 64 partial sets "
                       "(320 MB) rotated, warm = one set",
        "cold": "weights rotated over 3 rank copies (1.06 GB > 256 MB MALL); warm_* = one copy repeated",
        "timing": "median (min, max) over 7 batches of back-to-back calls, each batch between one event pair",
    }


def leg_reduce(name, reps):
    w = synth.get(name)
    parts = [gen(w, synth.T_PARTIAL + q, (w.n, w.h), 1.0) for q in range(w.tp)]
    y = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)
    tm = EventTimer()
    for i in range(2 + reps):
        if i >= 2:
            tm.start("reduce")
        T.tp_partial_reduce(parts, out=y)
        if i >= 2:
            tm.stop("reduce")
    for i in range(2 + reps):
        if i >= 2:
            tm.start("rank")
        T.tp_partial_reduce(parts, out=y, order=T.TP_ORDER_RANK)
        if i >= 2:
            tm.stop("rank")
    torch.cuda.synchronize()
    b = (w.tp + 1) * w.n * w.h * 2
    ms = tm.ms("reduce")
    msr = tm.ms("rank")
    del parts
    return {"workload": name, "t": w.tp, "K": w.n * w.h, "ms": ms, "ms_stats": tm.stats("reduce"),
            "GBps": b / ms / 1e6, "hbm_frac": b / ms / 1e6 / PEAK_HBM_GBPS, "algorithmic_bytes": b,
            "rank_order_ms": msr, "rank_order_ms_stats": tm.stats("rank"),
            "rank_order_hbm_frac": b / msr / 1e6 / PEAK_HBM_GBPS,
            "cold": f"working set {(b / 2**30):.2f} GiB > 1 GiB: every call streams from HBM"}


def leg_spnorm(reps):
    """Sequence-parallel epilogue at the 70B prefill shape: each rank's
    reduce-scatter rows (1024 of 8192) + residual add + RMSNorm.  Calls cycle
    over the 8 ranks, so consecutive calls read disjoint rows (8 x 151 MB
    between two visits of a chunk: cold in the MALL), back to back between
    one event pair; the library is called with pre-marshalled arguments so
    that the host keeps ahead of the ~25 us calls."""
    import ctypes
    w = synth.get("llama70b_prefill_tp8")
    t, n, h = w.tp, w.n, w.h
    parts = [gen(w, synth.T_PARTIAL + q, (n, h), 1.0) for q in range(t)]
    weight = gen(w, synth.T_NORM_W, (h,), 0.1) + 1.0
    rows = n // t
    res = [gen(w, synth.T_RESIDUAL + r, (rows, h), 1.0) for r in range(t)]
    ro = [torch.empty((rows, h), dtype=w.dtype, device=DEV) for _ in range(t)]
    out = [torch.empty((rows, h), dtype=w.dtype, device=DEV) for _ in range(t)]
    L = T.lib()
    ptrs = (ctypes.c_void_p * t)(*[p.data_ptr() for p in parts])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = 1 if w.dtype == torch.bfloat16 else 0
    args = [(ptrs, t, r, n, h, dt, ctypes.c_void_p(res[r].data_ptr()), ctypes.c_void_p(weight.data_ptr()),
             1e-5, ctypes.c_void_p(ro[r].data_ptr()), ctypes.c_void_p(out[r].data_ptr()), stream) for r in range(t)]
    for r in range(t):
        assert T.tp_sp_rows(n, r, t)[1] - T.tp_sp_rows(n, r, t)[0] == rows
        assert L.tp_rs_add_rmsnorm(*args[r]) == 0
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    calls = reps * t
    e0.record()
    for i in range(calls):
        L.tp_rs_add_rmsnorm(*args[i % t])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    b = (t * rows * h + rows * h + 2 * rows * h) * 2 + h * 2
    del parts, res, ro, out
    return {"workload": w.name, "t": t, "rows_per_rank": rows, "h": h, "ms_per_rank": ms, "GBps": b / ms / 1e6,
            "hbm_frac": b / ms / 1e6 / PEAK_HBM_GBPS, "algorithmic_bytes": b,
            "timing": "calls cycling over the 8 ranks, back to back between one event pair"}


def leg_vocab(reps):
    w = synth.get("qwen3_vocab_tp2")
    table = gen(w, synth.T_TABLE, (w.vocab, w.h), 0.02)
    ids = synth.token_ids(w.n, w.vocab, w.seed(synth.T_IDS), device=DEV)
    shards = [T.tp_shard_weights(table, 0, r, w.tp) for r in range(w.tp)]
    del table
    outs = [torch.empty((w.n, w.h), dtype=w.dtype, device=DEV) for _ in range(w.tp)]
    xemb = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)
    v_local = shards[0].shape[0]
    tm = EventTimer()
    for i in range(2 + reps):
        t_ = tm if i >= 2 else None
        if t_:
            t_.start("embed")
        for r in range(w.tp):
            T.tp_vocab_embed_rank(ids, shards[r], w.vocab, r, w.tp, out=outs[r])
        if t_:
            t_.stop("embed")
            t_.start("reduce")
        T.tp_partial_reduce(outs, out=xemb)
        if t_:
            t_.stop("reduce")
    # LM head: 156 MB table shard + 156 MB fp32 logits per call.  Cold: three
    # table copies and three logits buffers in rotation (936 MB, more than
    # the 256 MB MALL); warm: one table and one logits buffer.
    tabs = [shards[1]] + [shards[1].clone() for _ in range(2)]
    logits = [torch.empty((w.n, v_local), dtype=torch.float32, device=DEV) for _ in range(3)]

    def lm_cold(i):
        T.tp_lm_head_rank(xemb, tabs[i % 3], logits=logits[i % 3])

    def lm_warm(i):
        T.tp_lm_head_rank(xemb, tabs[0], logits=logits[0])

    cold_v = batched_ms(lm_cold, reps)
    warm_v = batched_ms(lm_warm, reps)
    del tabs, logits
    torch.cuda.synchronize()
    fl = 2.0 * w.n * w.h * v_local
    by = v_local * w.h * 2 + w.n * w.h * 2 + w.n * v_local * 4
    ms = median(cold_v)
    # gather of both ranks' logits into [n, V] and the greedy pick (622 MB
    # moved per call with the full copy: consecutive calls stream from HBM)
    rank_logits = [T.tp_lm_head_rank(xemb, shards[r]) for r in range(w.tp)]
    full = torch.empty((w.n, w.vocab), dtype=torch.float32, device=DEV)
    am = torch.empty((w.n,), dtype=torch.int64, device=DEV)
    tg = EventTimer()
    for i in range(2 + reps):
        if i >= 2:
            tg.start("gather")
        T.tp_logits_gather_argmax(rank_logits, w.vocab, full=full, argmax=am)
        if i >= 2:
            tg.stop("gather")
            tg.start("argmax")
        T.tp_logits_gather_argmax(rank_logits, w.vocab, argmax=am, want_full=False)
        if i >= 2:
            tg.stop("argmax")
    torch.cuda.synchronize()
    gb = w.n * w.vocab * 4
    return {"workload": w.name, "embed_ms_all_ranks": tm.ms("embed"), "embed_ms_stats": tm.stats("embed"),
            "reduce_ms": tm.ms("reduce"), "reduce_ms_stats": tm.stats("reduce"),
            "lm_head_ms": ms, "lm_head_ms_stats": stats(cold_v),
            "lm_head_TFLOPs": fl / ms / 1e9, "lm_head_GBps": by / ms / 1e6,
            "lm_head_hbm_frac": by / ms / 1e6 / PEAK_HBM_GBPS,
            "lm_head_mfma_frac": fl / ms / 1e9 / PEAK_BF16_TFLOPS,
            "warm_lm_head_ms": median(warm_v), "warm_lm_head_ms_stats": stats(warm_v),
            "lm_head_cold": "3 table shards + 3 logits buffers rotated (936 MB); warm = one of each",
            "embed_note": "embedding and its shard sum: 1-3 MiB per call, launch bound (warm)",
            "gather_argmax_ms": tg.ms("gather"), "gather_argmax_ms_stats": tg.stats("gather"),
            "gather_argmax_GBps": 2 * gb / tg.ms("gather") / 1e6,
            "gather_argmax_hbm_frac": 2 * gb / tg.ms("gather") / 1e6 / PEAK_HBM_GBPS,
            "argmax_only_ms": tg.ms("argmax"), "argmax_only_ms_stats": tg.stats("argmax"),
            "argmax_only_GBps": gb / tg.ms("argmax") / 1e6,
            "argmax_only_hbm_frac": gb / tg.ms("argmax") / 1e6 / PEAK_HBM_GBPS}


def leg_attnproj(reps):
    w = synth.get("llama70b_attnproj_tp16")
    hd, t = w.head_dim, w.tp
    r = 5
    wq = gen(w, synth.T_WQ, (w.n_q * hd, w.h), 0.02)
    wk = gen(w, synth.T_WK, (w.n_kv * hd, w.h), 0.02)
    wv = gen(w, synth.T_WV, (w.n_kv * hd, w.h), 0.02)
    wo = gen(w, synth.T_WO, (w.h, w.n_q * hd), 0.02)
    wqkv = T.tp_shard_qkv(wq, wk, wv, w.n_q, w.n_kv, hd, r, t)
    wo_r = T.tp_shard_weights(wo, 1, r, t)
    del wq, wk, wv, wo
    nq_r, nkv_r = w.n_q // t, max(w.n_kv // t, 1)
    # cold: three token inputs and three output partials in rotation (768 MiB
    # of x and partials, more than the 256 MB MALL); warm: one of each
    xs = [gen(w, synth.T_X, (w.n, w.h), 1.0)] + [None, None]
    xs[1], xs[2] = xs[0].clone(), xs[0].clone()
    parts = [torch.empty((w.n, w.h), dtype=w.dtype, device=DEV) for _ in range(3)]
    qkv = torch.empty((w.n, wqkv.shape[0]), dtype=w.dtype, device=DEV)
    a_r = torch.empty((w.n, nq_r * hd), dtype=w.dtype, device=DEV)
    aws = torch.empty(max(T.tp_attention_workspace_bytes(w.n, nq_r, nkv_r, hd, causal=True), 16),
                      dtype=torch.uint8, device=DEV)
    res = {}
    for mode in ("cold", "warm"):
        tm = EventTimer()
        for i in range(2 + reps):
            j = i % 3 if mode == "cold" else 0
            t_ = tm if i >= 2 else None
            if t_:
                t_.start("qkv")
            T.tp_linear_rank_forward(xs[j], wqkv, y=qkv)
            if t_:
                t_.stop("qkv")
                t_.start("attn")
            T.tp_attention_rank(qkv, nq_r, nkv_r, head_dim=hd, causal=True, out=a_r, workspace=aws)
            if t_:
                t_.stop("attn")
                t_.start("o_proj")
            T.tp_linear_rank_forward(a_r, wo_r, y=parts[j])
            if t_:
                t_.stop("o_proj")
        torch.cuda.synchronize()
        res[mode] = tm
    tm = res["cold"]
    fq = 2.0 * w.n * w.h * wqkv.shape[0]
    fo = 2.0 * w.n * a_r.shape[1] * w.h
    fa = 4.0 * nq_r * hd * w.n * (w.n + 1) / 2        # causal: QK^T and PV over s <= i
    out = {"workload": w.name, "qkv_ms": tm.ms("qkv"), "qkv_ms_stats": tm.stats("qkv"),
           "qkv_TFLOPs": fq / tm.ms("qkv") / 1e9,
           "attn_ms": tm.ms("attn"), "attn_ms_stats": tm.stats("attn"), "attn_TFLOPs": fa / tm.ms("attn") / 1e9,
           "attn_mfma_frac": fa / tm.ms("attn") / 1e9 / PEAK_BF16_TFLOPS,
           "o_proj_ms": tm.ms("o_proj"), "o_proj_ms_stats": tm.stats("o_proj"),
           "o_proj_TFLOPs": fo / tm.ms("o_proj") / 1e9,
           "qkv_mfma_frac": fq / tm.ms("qkv") / 1e9 / PEAK_BF16_TFLOPS,
           "o_proj_mfma_frac": fo / tm.ms("o_proj") / 1e9 / PEAK_BF16_TFLOPS,
           "chain": "x -> QKV projection -> attention core (causal, 4 q heads / 1 kv head) -> o_proj partial",
           "cold": "3 token inputs and 3 partials rotated; warm_* = one of each"}
    wt = res["warm"]
    for k in ("qkv", "attn", "o_proj"):
        out[f"warm_{k}_ms"] = wt.ms(k)
        out[f"warm_{k}_ms_stats"] = wt.stats(k)
    return out


def leg_qwen_fp32(reps):
    w = synth.get("qwen3_mlp_tp2_fp32")
    x = gen(w, synth.T_X, (w.n, w.h), 1.0)
    gate = gen(w, synth.T_GATE, (w.f, w.h), 0.02)
    up = gen(w, synth.T_UP, (w.f, w.h), 0.02)
    down = gen(w, synth.T_DOWN, (w.h, w.f), 0.02)
    shards = [(T.tp_shard_gate_up(gate, up, r, w.tp), T.tp_shard_weights(down, 1, r, w.tp)) for r in range(w.tp)]
    # cold: 16 copies of both ranks' weights in rotation (605 MB > 256 MB MALL)
    sets = [shards] + [[(a.clone(), b.clone()) for a, b in shards] for _ in range(15)]
    ws = torch.empty(T.tp_mlp_workspace_bytes(w.n, w.h, w.f_local, w.dtype), dtype=torch.uint8, device=DEV)
    parts = [torch.empty((w.n, w.h), dtype=w.dtype, device=DEV) for _ in range(w.tp)]
    y = torch.empty((w.n, w.h), dtype=w.dtype, device=DEV)

    def layer(i, cold):
        sh = sets[i % 16] if cold else shards
        for r in range(w.tp):
            T.tp_mlp_rank_forward(x, sh[r][0], sh[r][1], partial=parts[r], workspace=ws)
        T.tp_partial_reduce(parts, out=y)

    cold_v = batched_ms(lambda i: layer(i, True), reps)
    warm_v = batched_ms(lambda i: layer(i, False), reps)
    torch.cuda.synchronize()
    wb = (3 * w.f_local * w.h) * 4
    return {"workload": w.name, "all_ranks_plus_reduce_us": median(cold_v) * 1e3,
            "all_ranks_plus_reduce_us_stats": {k: (v * 1e3 if k != "n" else v) for k, v in stats(cold_v).items()},
            "warm_all_ranks_plus_reduce_us": median(warm_v) * 1e3,
            "warm_all_ranks_plus_reduce_us_stats": {k: (v * 1e3 if k != "n" else v)
                                                    for k, v in stats(warm_v).items()},
            "weight_bytes_per_rank": wb,
            "cold": "16 copies of both ranks' weights rotated; warm = one copy",
            "note": "latency bound at this size (19 MB of fp32 weights per rank)"}


def leg_load(reps):
    """Checkpoint-style loading of one rank's MLP weights: rank 5 of TP=8
    takes its gate and up rows and its down columns from fp32 tensors in host
    memory into bf16 tables (only the shard crosses the host link)."""
    w = synth.get("llama70b_prefill_tp8")
    r, t = 5, w.tp
    fl = w.f // t
    g = torch.Generator().manual_seed(w.seed(synth.T_GATE))
    full = [torch.empty((w.f, w.h), dtype=torch.float32).uniform_(-0.05, 0.05, generator=g) for _ in range(2)]
    down = torch.empty((w.h, w.f), dtype=torch.float32).uniform_(-0.05, 0.05, generator=g)
    gu = torch.empty((2 * fl, w.h), dtype=torch.bfloat16, device=DEV)
    dn = torch.empty((w.h, fl), dtype=torch.bfloat16, device=DEV)
    staging = torch.empty(T.tp_load_staging_bytes(fl, w.h, torch.float32, torch.bfloat16), dtype=torch.uint8,
                          device=DEV)
    host_bytes = 3 * fl * w.h * 4

    def load(srcs):
        T.tp_load_gate_up(srcs[0], 0, r, t, out=gu, staging=staging)
        T.tp_load_gate_up(srcs[1], 1, r, t, out=gu, staging=staging)
        T.tp_load_shard(srcs[2], 1, r, t, out=dn, staging=staging)

    def timed(srcs):
        load(srcs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            load(srcs)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    ms_pageable = timed((full[0], full[1], down))
    pinned = [a.pin_memory() for a in (full[0], full[1], down)]
    ms_pinned = timed(pinned)
    # context: one plain contiguous pinned host -> device copy of the same bytes
    chunk = pinned[0][r * fl:(r + 1) * fl]
    buf = torch.empty(chunk.shape, dtype=torch.float32, device=DEV)
    buf.copy_(chunk, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        buf.copy_(chunk, non_blocking=True)
    torch.cuda.synchronize()
    ms_copy = (time.perf_counter() - t0) / reps * 1e3
    copy_gbps = chunk.numel() * 4 / ms_copy / 1e6
    chunk_pg = full[0][r * fl:(r + 1) * fl]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        buf.copy_(chunk_pg)
    torch.cuda.synchronize()
    pageable_copy_gbps = chunk_pg.numel() * 4 / ((time.perf_counter() - t0) / reps * 1e3) / 1e6
    return {"workload": w.name, "host_bytes": host_bytes,
            "pageable_ms": ms_pageable, "pageable_GBps": host_bytes / ms_pageable / 1e6,
            "pinned_ms": ms_pinned, "pinned_GBps": host_bytes / ms_pinned / 1e6,
            "plain_pinned_copy_GBps": copy_gbps, "plain_pageable_copy_GBps": pageable_copy_gbps,
            "pinned_frac_of_plain_copy": host_bytes / ms_pinned / 1e6 / copy_gbps,
            "what": "gate + up rows and down columns of rank 5/8 from fp32 host tensors to bf16 device tables "
                    "(wall clock, host link bound)"}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(S, budget_s=12.0):
    """Times the fp64 oracle's rank-partial MLP on sampled token rows of the
    same prefill workload.  Row-independent, so the rate (FLOP/s) carries
    over to the full workload."""
    import numpy as np  # noqa: F401

    import oracle
    from tests.helpers import to_f64
    w = S["w"]
    fl = w.f_local
    G = to_f64(S["wgu"][:fl])
    U = to_f64(S["wgu"][fl:])
    D = to_f64(S["wd"])
    cap = 4096
    X = to_f64(S["x"][:cap])
    cores = oracle_cores()
    rows = max(1, min(cores, cap))
    t0 = time.perf_counter()
    oracle.mlp_rank(X[:rows], G, U, D, 0, 1)
    dt = time.perf_counter() - t0
    # scale the sample to the time budget (rows in multiples of the thread count)
    more = int(budget_s / max(dt, 1e-3)) * rows
    more = max(rows, min(more - more % rows, cap))
    t0 = time.perf_counter()
    oracle.mlp_rank(X[:more], G, U, D, 0, 1)
    dt2 = time.perf_counter() - t0
    flops = mlp_flops(more, w.h, fl)
    return {"value": flops / dt2 / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{more} of {w.n} token rows of the rank's MLP share (fp64, {dt2:.1f} s)",
            "full_workload_extrapolated_s": dt2 * w.n / more}


def oracle_cores():
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def host_bf16_f64(shape, std, seed):
    """seeded N(0, std^2) draws on the host, rounded to bf16, widened to fp64"""
    return synth.normal(shape, std, seed, torch.bfloat16).to(torch.float64).numpy()


def host_bf16_f32(shape, std, seed):
    return synth.normal(shape, std, seed, torch.bfloat16).to(torch.float32).numpy()


def cpu_oracle_legs():
    """The fp64 oracle beside the decode and reduce legs, at full size, on
    host-generated inputs of the same shapes and distributions (the oracle's
    time does not depend on the values): the decode rank share (64 tokens,
    f_local 7168) and its ring-order reduce of 4 partials of 1 MiB, and the
    8- and 16-rank reduces of 128 MiB partials (fp32 ring simulation and the
    fp64 sum)."""
    import oracle
    out = {"cores": oracle_cores()}
    w = synth.get("llama70b_decode_tp4")
    fl = w.f_local
    X = host_bf16_f64((w.n, w.h), 1.0, w.seed(synth.T_X))
    G = host_bf16_f64((fl, w.h), 0.02, w.seed(synth.T_GATE))
    U = host_bf16_f64((fl, w.h), 0.02, w.seed(synth.T_UP))
    D = host_bf16_f64((w.h, fl), 0.02, w.seed(synth.T_DOWN))
    t0 = time.perf_counter()
    oracle.mlp_rank(X, G, U, D, 0, 1)
    dt = time.perf_counter() - t0
    del X, G, U, D
    parts = [host_bf16_f32((w.n, w.h), 1.0, w.seed(synth.T_PARTIAL + q)) for q in range(w.tp)]
    t0 = time.perf_counter()
    oracle.ring_allreduce_f32(parts)
    dr = time.perf_counter() - t0
    out["decode"] = {"mlp_rank_s": round(dt, 4), "mlp_rank_GFLOPs": round(mlp_flops(w.n, w.h, fl) / dt / 1e9, 2),
                     "ring_reduce_s": round(dr, 5),
                     "what": "fp64 rank share at full size (64 tokens) + fp32 ring-order reduce of 4 x 1 MiB"}
    for name, key in (("llama70b_prefill_tp8", "reduce8"), ("llama70b_attnproj_tp16", "reduce16")):
        w = synth.get(name)
        parts = [host_bf16_f32((w.n, w.h), 1.0, w.seed(synth.T_PARTIAL + q)) for q in range(w.tp)]
        t0 = time.perf_counter()
        oracle.ring_allreduce_f32(parts)
        d_ring = time.perf_counter() - t0
        parts = [p.astype("float64") for p in parts]
        t0 = time.perf_counter()
        oracle.reduce_sum_f64(parts)
        d64 = time.perf_counter() - t0
        b = (w.tp + 1) * w.n * w.h * 2
        out[key] = {"ring_f32_s": round(d_ring, 3), "ring_f32_GBps": round(b / d_ring / 1e9, 2),
                    "sum_f64_s": round(d64, 3),
                    "what": f"{w.tp} partials of [{w.n}, {w.h}] at full size: fp32 ring-order simulation and fp64 sum"}
        del parts
    return out


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps before the warmup, for this much wall time (clock settling)")
    ap.add_argument("--legs", default="all")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 512 MiB device copy (tp_shard_weights, t=1) to calibrate HBM counters")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every tensor-parallel rank is emulated on a single device; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    T.lib()

    log("bench: setup prefill workload")
    S = prefill_setup()
    w = S["w"]
    log(f"bench: settle {a.settle_ms:.0f} ms")
    n_settle = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < a.settle_ms:
        for _ in range(8):
            prefill_step(S)
        n_settle += 8
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(a.warmup):
        prefill_step(S)
    torch.cuda.synchronize()
    tm = EventTimer()
    log(f"bench: timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tm.start("step")
    for _ in range(a.steps):
        prefill_step(S, tm)
    tm.stop("step")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = tm.all_ms("step")[0] / a.steps
    gu_ms, dn_ms, rd_ms = tm.ms("gate_up"), tm.ms("down"), tm.ms("reduce")
    mlp_v = [g + d for g, d in zip(tm.all_ms("gate_up"), tm.all_ms("down"))]
    gu_mean = sum(tm.all_ms("gate_up")) / len(tm.all_ms("gate_up"))
    fl = w.f_local
    mlp_ms = median(mlp_v)
    flops = mlp_flops(w.n, w.h, fl)
    value = flops / mlp_ms / 1e9
    gu_flops = 2.0 * w.n * w.h * 2 * fl
    red_bytes = (w.tp + 1) * w.n * w.h * 2
    log(f"bench: step {ms_step:.3f} ms (wall {wall * 1e3 / a.steps:.3f} ms): gate_up {gu_ms:.3f} "
        f"down {dn_ms:.3f} reduce {rd_ms:.3f} -> {value:.1f} TFLOP/s")

    legs = {}
    names = ["decode", "reduce8", "reduce16", "spnorm", "vocab", "attnproj", "qwen_fp32", "load"] if a.legs == "all" else \
        ([] if a.legs == "none" else a.legs.split(","))
    for nm in names:
        log(f"bench: leg {nm}")
        if nm == "decode":
            legs[nm] = leg_decode(20)
        elif nm == "reduce8":
            legs[nm] = leg_reduce("llama70b_prefill_tp8", 20)
        elif nm == "reduce16":
            legs[nm] = leg_reduce("llama70b_attnproj_tp16", 10)
        elif nm == "spnorm":
            legs[nm] = leg_spnorm(10)
        elif nm == "vocab":
            legs[nm] = leg_vocab(20)
        elif nm == "attnproj":
            legs[nm] = leg_attnproj(10)
        elif nm == "qwen_fp32":
            legs[nm] = leg_qwen_fp32(50)
        elif nm == "load":
            legs[nm] = leg_load(3)
        torch.cuda.empty_cache()

    if a.copy_calib:
        # a [4096, 65536] bf16 copy (dim-1 shard with t=1): 512 MiB read and
        # 512 MiB written by one copy2d_kernel launch of grid 32 x 4096
        src = torch.empty((4096, 65536), dtype=torch.bfloat16, device=DEV)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        T.tp_shard_weights(src, 1, 0, 1, out=dst)
        torch.cuda.synchronize()
        log("bench: copy calibration: 512 MiB read + 512 MiB written by copy2d_kernel (grid 32x4096)")
        del src, dst

    cpu = None
    if not a.no_cpu:
        log("bench: cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(S)
        if legs:
            log("bench: cpu oracle beside the decode and reduce legs")
            cpu["legs"] = cpu_oracle_legs()
            for k in ("decode", "reduce8", "reduce16"):
                if k in legs:
                    legs[k]["cpu_oracle"] = cpu["legs"][k]

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "settle": {"steps": n_settle, "ms": round(settle_ms, 1)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "h": w.h, "f_local": fl, "tp": w.tp,
                   "step": "gate_up+SiLU*up GEMM, down GEMM, ring-order reduce of 8 partials",
                   "value_over": "median over the timed steps of the MLP launches (gate_up + down)"},
        "mlp_ms": round(mlp_ms, 4), "gate_up_ms": round(gu_ms, 4), "down_ms": round(dn_ms, 4),
        "reduce_ms": round(rd_ms, 4), "reduce_GBps": round(red_bytes / rd_ms / 1e6, 1),
        "timing": "medians over the timed steps (HIP events around each launch); *_stats give median, min, max",
        "mlp_ms_stats": stats(mlp_v), "gate_up_ms_stats": tm.stats("gate_up"), "down_ms_stats": tm.stats("down"),
        "reduce_ms_stats": tm.stats("reduce"),
        "cold": "each step streams 1.2 GB of partials through the reduce, so every step starts cold in the MALL",
        "step_TFLOPs_incl_reduce": round(flops / ms_step / 1e9, 2),
        "roofline": {"kernel": "gate_up GEMM + SiLU*up epilogue", "bound": "mfma",
                     "achieved": round(gu_flops / gu_mean / 1e9, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gu_flops / gu_mean / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "duration": "mean gate_up launch time over the timed steps (HIP events)"},
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
