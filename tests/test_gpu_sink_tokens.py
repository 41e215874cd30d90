"""GPU parity of the start-of-sequence sink tokens (the first n positions stay
visible past the window edge), through the C ABI, against the fp64 oracle.

Covered: prefill with sink tiles before the window (n within one tile, n over
several tiles, n beyond the sequence, window 1), decode over the split plan and
the one-unit-per-wave plan, ragged + paged batches, and the fp32 path.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
from gpu_helpers import (assert_bf16_close, assert_fp32_close, assert_lse_close, dev_f32, dev_i32, dev_tensor, say,
                         to_f64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,S,W,n", [
    (1, 300, 128, 4),
    (1, 700, 64, 100),
    (2, 257, 16, 1),
    (1, 520, 1, 3),
    (1, 200, 128, 500),
    (1, 1000, 128, 64),
    (1, 33, 8, 40),
    (1, 600, 128, 32),   # the most sink tokens whose tile runs key half 0 only
    (1, 600, 100, 33),   # one more: the sink tile runs both halves
])
def test_prefill_sink_tokens(device, B, S, W, n):
    say(f"prefill sink tokens B{B} S{S} W={W} n={n}")
    p = gi.prefill_problem(80, B, S, 64, 8, 64, dtype="bf16")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               dev_f32(p.sinks, device), window=W, sink_tokens=n, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, window=W, scale=p.scale, sink_tokens=n)
    assert_bf16_close(to_f64(out), o_ref, "prefill")
    assert_lse_close(to_f64(lse), l_ref, "prefill lse")


def test_prefill_sink_tokens_layer_shape_sampled(device):
    p = gi.c2_layer()
    W, n = 128, 4
    say(f"prefill sink tokens layer-shaped S4096 W={W} n={n}")
    out = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                          dev_f32(p.sinks, device), window=W, sink_tokens=n)
    torch.cuda.synchronize()
    rows = [0, 3, 4, 127, 128, 131, 132, 1000, 2047, 4095]
    o_ref, _ = oracle.prefill_rows_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, p.scale, rows=rows, sink_tokens=n)
    assert_bf16_close(to_f64(out)[:, rows], o_ref, "sampled rows")


@pytest.mark.parametrize("B,Lmax,W,n,solo", [
    (8, 3000, 128, 4, False),
    (8, 3000, 128, 200, False),
    (2, 40000, 4096, 64, False),   # several splits over the virtual key range
    (300, 400, 128, 4, True),      # one unit per wave
])
def test_decode_sink_tokens(device, monkeypatch, B, Lmax, W, n, solo):
    monkeypatch.setenv("GQA_DECODE_ROWS", "0")  # per-head forms; the whole-row form's sink-token cases are in the parity tests
    monkeypatch.setenv("GQA_DECODE_SOLO", "1" if solo else "0")
    say(f"decode sink tokens B{B} Lmax{Lmax} W={W} n={n} solo={solo}")
    d = gi.decode_problem(81, B, Lmax, 64, 8, 64, dtype="bf16", seqlens="random")
    out, lse = gq.attn_decode(dev_tensor(d.q, device), (dev_tensor(d.k, device), dev_tensor(d.v, device)),
                              dev_i32(d.seqlens, device), dev_f32(d.sinks, device), window=W, sink_tokens=n,
                              return_lse=True)
    torch.cuda.synchronize()
    got, got_l = to_f64(out), to_f64(lse)
    pick = range(B) if B <= 8 else [0, 1, 2, 150, B - 1]
    for b in pick:
        sl = slice(b, b + 1)
        o_ref, l_ref = oracle.decode_ref(d.q.f64[sl], d.k.f64[sl], d.v.f64[sl], d.seqlens[sl], d.sinks, W, d.scale,
                                         sink_tokens=n)
        assert_bf16_close(got[sl], o_ref, f"sequence {b} (L={d.seqlens[b]})")
        assert_lse_close(got_l[sl], l_ref, "lse")


def test_varlen_paged_sink_tokens(device):
    r = gi.c5_ragged()
    W, n = 128, 4
    say(f"varlen paged sink tokens W={W} n={n}")
    out = gq.attn_varlen_paged(dev_tensor(r.q, device), (dev_tensor(r.k, device), dev_tensor(r.v, device)),
                               dev_i32(r.block_table, device), dev_i32(r.cu_seqlens_q, device),
                               dev_i32(r.seqlens_k, device), dev_f32(r.sinks, device), window=W, sink_tokens=n,
                               max_q_len=r.max_q_len, max_kv_len=r.max_kv_len)
    torch.cuda.synchronize()
    got = to_f64(out)
    cu = r.cu_seqlens_q
    rows = sorted(set([int(cu[b]) for b in range(len(cu) - 1) if cu[b + 1] > cu[b]] +
                      [int(cu[b + 1]) - 1 for b in range(len(cu) - 1) if cu[b + 1] > cu[b]] + [5, 300, 1000]))
    o_ref, _ = oracle.varlen_ref(r.q.f64, r.k.f64, r.v.f64, cu, r.seqlens_k, r.sinks, W, r.scale,
                                 block_table=r.block_table, block_size=r.block_size, rows=rows, sink_tokens=n)
    assert_bf16_close(got[rows], o_ref[rows], "varlen rows")


def test_fp32_sink_tokens(device):
    p = gi.prefill_problem(82, 1, 200, 8, 2, 64, dtype="fp32")
    W, n = 16, 5
    say(f"fp32 prefill sink tokens W={W} n={n}")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               dev_f32(p.sinks, device), window=W, sink_tokens=n, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, window=W, scale=p.scale, sink_tokens=n)
    assert_fp32_close(to_f64(out), o_ref, "fp32 prefill")
    assert_lse_close(to_f64(lse), l_ref, "fp32 lse", fp32=True)
    d = gi.decode_problem(83, 4, 300, 8, 2, 64, dtype="fp32", seqlens=[1, 10, 150, 300])
    o = gq.attn_decode(dev_tensor(d.q, device), (dev_tensor(d.k, device), dev_tensor(d.v, device)),
                       dev_i32(d.seqlens, device), dev_f32(d.sinks, device), window=W, sink_tokens=n)
    torch.cuda.synchronize()
    o_ref, _ = oracle.decode_ref(d.q.f64, d.k.f64, d.v.f64, d.seqlens, d.sinks, W, d.scale, sink_tokens=n)
    assert_fp32_close(to_f64(o), o_ref, "fp32 decode")
