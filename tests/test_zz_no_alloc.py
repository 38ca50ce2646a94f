"""tp_mlp_rank_forward_noalloc: the MLP share for callers that cannot
allocate device memory.  Called through the C ABI (ctypes on raw device
pointers, the library's own scratch instead of a workspace) and compared bit
for bit with tp_mlp_rank_forward on the same inputs, on two calls in a row
with the second one smaller, so that the second call runs on scratch the
first one left behind.
"""
import ctypes

import pytest
import torch

import synth
from rank_sharded_layer_amd import tpshard as T

DEV = "cuda:0"
NULL = ctypes.c_void_p(0)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(x, wgu, wd, partial, out_dt):
    n, h = x.shape
    fl = wgu.shape[0] // 2
    L = T.lib()
    st = L.tp_mlp_rank_forward_noalloc(_p(x), n, h, _p(wgu), _p(wd), fl, T.TP_BF16, _p(partial),
                                       T.TP_BF16 if out_dt == torch.bfloat16 else T.TP_F32,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, T.tp_last_error()


@pytest.mark.gpu
def test_noalloc_mlp_equals_workspace_mlp_on_two_calls():
    cases = [
        # the Llama-3.1-70B decode share (one rank of TP=4): register-streaming split-K, ~16 MB of scratch
        (64, 8192, 7168, torch.bfloat16, 11),
        # smaller second call: tiled kernels with split-K, ragged tiles, fp32 output
        (17, 1024, 392, torch.float32, 12),
    ]
    for n, h, fl, out_dt, seed in cases:
        x = synth.normal((n, h), 1.0, seed, torch.bfloat16, device=DEV)
        wgu = synth.normal((2 * fl, h), 0.02, seed + 1, torch.bfloat16, device=DEV)
        wd = synth.normal((h, fl), 0.02, seed + 2, torch.bfloat16, device=DEV)
        ref = T.tp_mlp_rank_forward(x, wgu, wd, out_dtype=out_dt)
        got = torch.full((n, h), float("nan"), dtype=out_dt, device=DEV)
        st, msg = _noalloc(x, wgu, wd, got, out_dt)
        assert st == 0, msg
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (n, h, fl)


@pytest.mark.gpu
def test_noalloc_mlp_rejects_shapes_beyond_its_scratch():
    """The 8192-token prefill share at TP=8 needs about 123 MB: TP_EWORKSPACE,
    nothing launched (the output keeps its contents)."""
    n, h, fl = 8192, 8192, 3584
    need = T.tp_mlp_workspace_bytes(n, h, fl, torch.bfloat16)
    assert need > 64 << 20
    x = torch.zeros((n, h), dtype=torch.bfloat16, device=DEV)
    wgu = torch.zeros((2 * fl, h), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((h, fl), dtype=torch.bfloat16, device=DEV)
    out = torch.full((n, h), 7.0, dtype=torch.bfloat16, device=DEV)
    st, msg = _noalloc(x, wgu, wd, out, torch.bfloat16)
    assert st == 6 and "scratch" in msg
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.skipif(torch.cuda.is_available(), reason="dummy-pointer error paths run on a GPU-less host only")
def test_noalloc_mlp_argument_errors_on_host():
    L = T.lib()
    d = ctypes.c_void_p(0x1000)
    assert L.tp_mlp_rank_forward_noalloc(NULL, 4, 8, d, d, 6, 1, d, 1, NULL) == 1
    assert L.tp_mlp_rank_forward_noalloc(d, 4, 8, d, d, 6, 0, d, 1, NULL) == 3       # f32 -> bf16
    assert L.tp_mlp_rank_forward_noalloc(d, 8192, 8192, d, d, 3584, 1, d, 1, NULL) == 6
    assert "scratch" in T.tp_last_error()
