"""GPU parity on the long-context workloads: prefill at S32768 and decode at
B8 x 131072, both 64/8 heads bf16 N(0,1), dense and window 128.

The oracle computes sampled outputs one by one (every head of the sampled
query rows; every head of two whole decode sequences); properties that hold at
any size (finite outputs, the convexity bound) are checked everywhere.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
from gpu_helpers import assert_bf16_close, assert_lse_close, dev_f32, dev_i32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def long_prefill():
    return gi.c4_prefill()


@pytest.fixture(scope="module")
def long_decode():
    return gi.c4_decode()


@pytest.mark.parametrize("W", [0, 128])
def test_prefill_long_context_sampled(device, long_prefill, W):
    p = long_prefill
    S = p.q.shape[1]
    say(f"prefill long context S{S} W={W}")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               dev_f32(p.sinks, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.isfinite(got).all()
    assert np.abs(got).max() <= np.abs(gi.bf16_to_f32(p.v.store)).max() + 1e-2
    rng = np.random.default_rng(100 + W)
    rows = sorted(set([0, 1, 63, 64, 127, 128, 129, S // 2, S - 65, S - 64, S - 2, S - 1]
                      + [int(r) for r in rng.integers(0, S, size=24)]))
    # the oracle's single-head routine on the sampled query rows, every head
    q = gi.bf16_to_f64(p.q.store[0, rows])  # [rows, Hq, D]
    kf, vf = p.k.f64[0], p.v.f64[0]
    o_ref = np.zeros((1, len(rows), 64, 64))
    l_ref = np.zeros((1, 64, len(rows)))
    k_pos = np.arange(S)
    for h in range(64):
        g = oracle.kv_head(h, 64, 8)
        o_h, l_h = oracle.attend(q[:, h], kf[:, g], vf[:, g], rows, k_pos, p.sinks[h], W, p.scale)
        o_ref[0, :, h], l_ref[0, h] = o_h, l_h
    assert_bf16_close(got[:, rows], o_ref, "sampled rows")
    assert_lse_close(to_f64(lse)[:, :, rows], l_ref, "sampled lse")


@pytest.mark.parametrize("W", [0, 128])
def test_decode_long_context(device, long_decode, W):
    d = long_decode
    say(f"decode long context B8 x 131072 W={W}")
    out, lse = gq.attn_decode(dev_tensor(d.q, device), (dev_tensor(d.k, device), dev_tensor(d.v, device)),
                              dev_i32(d.seqlens, device), dev_f32(d.sinks, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    got, got_l = to_f64(out), to_f64(lse)
    assert np.isfinite(got).all()
    for b in (0, 7):
        sl = slice(b, b + 1)
        o_ref, l_ref = oracle.decode_ref(gi.bf16_to_f64(d.q.store[sl]), gi.bf16_to_f64(d.k.store[sl]),
                                         gi.bf16_to_f64(d.v.store[sl]), d.seqlens[sl], d.sinks, W, d.scale)
        assert_bf16_close(got[sl], o_ref, f"sequence {b}")
        assert_lse_close(got_l[sl], l_ref, "lse")
