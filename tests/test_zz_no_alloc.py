"""The allocation-free decode (gqa_attn_decode_noalloc) against gqa_attn_decode.

Both entry points run the same kernels; the allocation-free one keeps its split
partials in the library's fixed per-GPU array instead of a caller's workspace.
Two calls in a row, the second smaller (the array keeps the first call's
partials, which the second must not read), each compared with the workspace
entry point's output: bit for bit (same kernels, same split plan) and against
the fp64 oracle to the bf16 bar.  A size beyond the array is rejected on the
host, before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
from gpu_helpers import assert_bf16_close, dev_f32, dev_i32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


def run_both(d, window, sink_tokens=0):
    q, k, v, s = (dev_tensor(d.q, "cuda"), dev_tensor(d.k, "cuda"), dev_tensor(d.v, "cuda"),
                  dev_f32(d.sinks, "cuda"))
    sl = dev_i32(d.seqlens, "cuda")
    ref, l_ref = gq.attn_decode(q, (k, v), sl, s, window=window, sink_tokens=sink_tokens, return_lse=True)
    out = torch.empty_like(q)
    got, l_got = gq.attn_decode_noalloc(q, (k, v), sl, s, window=window, sink_tokens=sink_tokens, return_lse=True,
                                        out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return got, l_got, ref, l_ref


def test_noalloc_decode_two_calls_second_smaller():
    # 1: the batched decode workload (B64, cache 8192, 64/8 heads): 8 split partials per head, 8.65 MB
    B, L = 64, 8192
    assert gq.decode_workspace_size(B, L, 64, 8) > 0
    say("noalloc decode call 1: B64 x 8192 dense")
    d = gi.c3_decode()
    got, l_got, ref, l_ref = run_both(d, 0)
    assert torch.equal(got, ref) and torch.equal(l_got, l_ref)
    rows = np.arange(0, B, 9)
    o_ref, _ = oracle.decode_ref(d.q.f64[rows], d.k.f64[rows], d.v.f64[rows], d.seqlens[rows], d.sinks, 0, d.scale)
    assert_bf16_close(to_f64(got)[rows], o_ref, "noalloc call 1 vs oracle")
    # 2: smaller, windowed with sink tokens, ragged lengths; split partials again (fewer of them)
    say("noalloc decode call 2: B8 x 20000, window 128 + 4 sink tokens, and dense")
    d2 = gi.decode_problem(46, 8, 20000, 64, 8, 64, "bf16",
                           seqlens=[20000, 1, 129, 4097, 15000, 7, 300, 19999])
    for W, st in ((128, 4), (0, 0)):
        got2, l_got2, ref2, l_ref2 = run_both(d2, W, st)
        assert torch.equal(got2, ref2) and torch.equal(l_got2, l_ref2), (W, st)
        o2, _ = oracle.decode_ref(d2.q.f64, d2.k.f64, d2.v.f64, d2.seqlens, d2.sinks, W, d2.scale, sink_tokens=st)
        assert_bf16_close(to_f64(got2), o2, f"noalloc call 2 (W={W}) vs oracle")


def test_noalloc_decode_rejects_beyond_the_array():
    # 64 query heads over 4 KV heads at B16 x 65536: 64 splits per head, 17.3 MB of partials
    need = gq.decode_workspace_size(16, 65536, 64, 4)
    assert need > 16 << 20
    L = gq.lib()
    dummy = ctypes.c_void_p(16)
    rc = L.gqa_attn_decode_noalloc(dummy, dummy, dummy, dummy, None, dummy, None, 16, 65536, 64, 4, 64, 0, 0,
                                   0.0, gq.GQA_BF16, None)
    assert rc == -3, rc
    assert b"allocation-free" in L.gqa_attn_last_error()
