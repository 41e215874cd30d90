"""GPU parity on the long-context workloads: prefill (and its backward) at
S32768 and decode at B8 x 131072, all 64/8 heads bf16 N(0,1), dense and window
128.

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


@pytest.mark.parametrize("W", [0, 128])
def test_backward_long_context_sampled(device, long_prefill, W):
    """Backward at S32768 (one slab per key block at this size).  The oracle's
    single-head gradient routine on a subset of query rows is exact for dq of
    those rows, and for dk, dv of the keys that only those rows see: the last
    64 positions (every query that sees key j sits at j or later).  Other
    sampled query rows check dq on their own."""
    import oracle.backward as BW
    from gpu_helpers import assert_grad_close

    p = long_prefill
    S = p.q.shape[1]
    say(f"backward long context S{S} W={W}")
    q, k, v = dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device)
    sinks = dev_f32(p.sinks, device)
    dout = gi.make_tensor(4, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    out, lse = gq.attn_prefill(q, k, v, sinks, window=W, return_lse=True)
    dq, dk, dv, _ = gq.attn_prefill_backward(q, k, v, sinks, out, lse, dev_tensor(dout, device), window=W)
    torch.cuda.synchronize()
    dq, dk, dv = to_f64(dq)[0], to_f64(dk)[0], to_f64(dv)[0]
    for t in (dq, dk, dv):
        assert np.isfinite(t).all()
    tail = np.arange(S - 64, S)
    rng = np.random.default_rng(200 + W)
    early = sorted(set([0, 1, 127, 128, 4095] + [int(r) for r in rng.integers(0, S - 64, size=6)]))
    qf, kf, vf, gf = p.q.f64[0], p.k.f64[0], p.v.f64[0], dout.f64[0]
    k_pos = np.arange(S)
    dq_ref_tail = np.zeros((64, 64, 64))
    dq_ref_early = np.zeros((len(early), 64, 64))
    dk_ref = np.zeros((64, 8, 64))
    dv_ref = np.zeros((64, 8, 64))
    for h in range(64):
        g = oracle.kv_head(h, 64, 8)
        gq_t, gk_t, gv_t, _, _, _ = BW.row_grads(qf[tail, h], kf[:, g], vf[:, g], tail, k_pos, p.sinks[h],
                                                 gf[tail, h], W, p.scale)
        dq_ref_tail[:, h] = gq_t
        dk_ref[:, g] += gk_t[tail]
        dv_ref[:, g] += gv_t[tail]
        gq_e, _, _, _, _, _ = BW.row_grads(qf[early, h], kf[:, g], vf[:, g], early, k_pos, p.sinks[h],
                                           gf[early, h], W, p.scale)
        dq_ref_early[:, h] = gq_e
    assert_grad_close(dq[tail], dq_ref_tail, "dq last 64 rows")
    assert_grad_close(dq[early], dq_ref_early, "dq sampled rows")
    assert_grad_close(dk[tail], dk_ref, "dk last 64 keys")
    assert_grad_close(dv[tail], dv_ref, "dv last 64 keys")
