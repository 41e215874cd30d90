"""GPU parity on seeded random shapes: prefill, decode, varlen (paged and packed) and the prefill backward.

The fixed case lists elsewhere pin chosen shapes; this file draws the shape of
each case from a seeded generator instead, so that combinations nobody listed
meet: odd head ratios with windows and start-of-sequence sink tokens, scales
other than 1/sqrt(D), block sizes from 1 to 64, empty query chunks, sequences
shorter than one tile.  Every case is small enough for the fp64 oracle to run
element by element, and is compared at the bf16 bound of the other parity
tests.  The shapes are the test's own choice; the inputs come from
``gqa_inputs`` as everywhere else.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
import oracle.backward as obw
from gpu_helpers import (assert_bf16_close, assert_dsinks_close, assert_grad_close, assert_lse_close, dev_f32, dev_i32,
                         dev_tensor, say, to_f64)

pytestmark = pytest.mark.gpu

# (Hq, Hkv): group sizes 1 to 32, including ones that are not a power of two
HEADS = [(64, 8), (32, 8), (16, 4), (8, 8), (8, 2), (24, 8), (32, 2), (16, 1), (48, 8), (12, 4), (32, 1)]
SINK_KINDS = ["normal", "normal", "none", "zero"]


def draw_common(rng, max_len):
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    W = 0 if rng.random() < 0.4 else int(rng.integers(1, max_len + 20))
    n_st = int(rng.integers(1, 41)) if W > 0 and rng.random() < 0.35 else 0
    sk = SINK_KINDS[rng.integers(len(SINK_KINDS))]
    scale = None if rng.random() < 0.6 else float(rng.uniform(0.05, 0.3))
    std = float(rng.choice([1.0 / np.sqrt(2.0), 1.0]))
    return Hq, Hkv, W, n_st, sk, scale, std


def prefill_case(i):
    rng = np.random.default_rng(7100 + i)
    B = int(rng.integers(1, 4))
    S = int(rng.integers(1, 301))
    Hq, Hkv, W, n_st, sk, scale, std = draw_common(rng, S)
    return B, S, Hq, Hkv, W, n_st, sk, scale, std


def decode_case(i):
    rng = np.random.default_rng(7200 + i)
    B = int(rng.integers(1, 7))
    Lmax = int(rng.integers(1, 1501))
    Hq, Hkv, W, n_st, sk, scale, std = draw_common(rng, Lmax)
    return B, Lmax, Hq, Hkv, W, n_st, sk, scale, std


def backward_case(i):
    rng = np.random.default_rng(7400 + i)
    B = int(rng.integers(1, 3))
    S = int(rng.integers(1, 201))
    Hq, Hkv, W, n_st, sk, scale, std = draw_common(rng, S)
    return B, S, Hq, Hkv, W, n_st, sk, scale, std


def varlen_case(i):
    rng = np.random.default_rng(7300 + i)
    B = int(rng.integers(1, 7))
    kv = [int(x) for x in rng.integers(1, 801, size=B)]
    ql = []
    for L in kv:
        r = rng.random()
        ql.append(1 if r < 0.4 else (0 if r < 0.5 else int(rng.integers(1, L + 1))))
    bs = int(2 ** rng.integers(0, 7))  # 1 .. 64
    packed = bool(rng.random() < 0.25)
    Hq, Hkv, W, n_st, sk, scale, std = draw_common(rng, max(kv))
    return kv, ql, bs, packed, Hq, Hkv, W, n_st, sk, scale, std


@pytest.mark.parametrize("i", range(48))
def test_prefill_random_shape(device, i):
    B, S, Hq, Hkv, W, n_st, sk, scale, std = prefill_case(i)
    p = gi.prefill_problem(7100 + i, B, S, Hq, Hkv, 64, "bf16", std=std, sink_kind=sk, scale=scale)
    say(f"random prefill #{i}: B={B} S={S} Hq={Hq} Hkv={Hkv} W={W} sink_tokens={n_st} sink={sk} scale={scale}")
    sinks = None if sk == "none" else dev_f32(p.sinks, device)
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device), sinks,
                               window=W, scale=scale, sink_tokens=n_st, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, p.scale, sink_tokens=n_st)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


@pytest.mark.parametrize("i", range(32))
def test_decode_random_shape(device, i):
    B, Lmax, Hq, Hkv, W, n_st, sk, scale, std = decode_case(i)
    p = gi.decode_problem(7200 + i, B, Lmax, Hq, Hkv, 64, "bf16", std=std, sink_kind=sk, seqlens="random",
                          scale=scale)
    say(f"random decode #{i}: B={B} Lmax={Lmax} Hq={Hq} Hkv={Hkv} W={W} sink_tokens={n_st} sink={sk} scale={scale}")
    sinks = None if sk == "none" else dev_f32(p.sinks, device)
    out, lse = gq.attn_decode(dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                              dev_i32(p.seqlens, device), sinks, window=W, scale=scale, sink_tokens=n_st,
                              return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_ref(p.q.f64, p.k.f64, p.v.f64, p.seqlens, p.sinks, W, p.scale, sink_tokens=n_st)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


@pytest.mark.parametrize("i", range(32))
def test_varlen_random_shape(device, i):
    kv, ql, bs, packed, Hq, Hkv, W, n_st, sk, scale, std = varlen_case(i)
    p = gi.varlen_problem(7300 + i, kv, ql, Hq, Hkv, 64, block_size=bs, dtype="bf16", std=std, sink_kind=sk,
                          spare_blocks=2, scale=scale)
    say(f"random varlen #{i}: kv={kv} q={ql} bs={bs} packed={packed} Hq={Hq} Hkv={Hkv} W={W} sink_tokens={n_st} "
        f"sink={sk} scale={scale}")
    sinks = None if sk == "none" else dev_f32(p.sinks, device)
    q = dev_tensor(p.q, device)
    if packed:
        ks, vs, cu = [], [], [0]
        for b in range(len(kv)):
            L = int(p.seqlens_k[b])
            ks.append(oracle.gather_paged(p.k.store, p.block_table[b], p.block_size, L))
            vs.append(oracle.gather_paged(p.v.store, p.block_table[b], p.block_size, L))
            cu.append(cu[-1] + L)
        kc = gi.Tensor(np.concatenate(ks), p.k.dtype)
        vc = gi.Tensor(np.concatenate(vs), p.v.dtype)
        out, lse = gq.attn_varlen_paged(q, (dev_tensor(kc, device), dev_tensor(vc, device)), None,
                                        dev_i32(p.cu_seqlens_q, device), dev_i32(p.seqlens_k, device), sinks,
                                        window=W, scale=scale, max_q_len=p.max_q_len, max_kv_len=p.max_kv_len,
                                        cu_seqlens_k=dev_i32(cu, device), sink_tokens=n_st, return_lse=True)
    else:
        out, lse = gq.attn_varlen_paged(q, (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                                        dev_i32(p.block_table, device), dev_i32(p.cu_seqlens_q, device),
                                        dev_i32(p.seqlens_k, device), sinks, window=W, scale=scale,
                                        max_q_len=p.max_q_len, max_kv_len=p.max_kv_len, sink_tokens=n_st,
                                        return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.varlen_ref(p.q.f64, p.k.f64, p.v.f64, p.cu_seqlens_q, p.seqlens_k, p.sinks, W, p.scale,
                                     block_table=p.block_table, block_size=p.block_size, sink_tokens=n_st)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


@pytest.mark.parametrize("i", range(16))
def test_backward_random_shape(device, i):
    B, S, Hq, Hkv, W, n_st, sk, scale, std = backward_case(i)
    p = gi.prefill_problem(7400 + i, B, S, Hq, Hkv, 64, "bf16", std=std, sink_kind=sk, scale=scale)
    dout = gi.make_tensor(7400 + i, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    say(f"random backward #{i}: B={B} S={S} Hq={Hq} Hkv={Hkv} W={W} sink_tokens={n_st} sink={sk} scale={scale}")
    q, k, v = dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device)
    sinks = None if sk == "none" else dev_f32(p.sinks, device)
    out, lse = gq.attn_prefill(q, k, v, sinks, window=W, scale=scale, sink_tokens=n_st, return_lse=True)
    g = gq.attn_prefill_backward(q, k, v, sinks, out, lse, dev_tensor(dout, device), window=W, scale=scale,
                                 sink_tokens=n_st)
    torch.cuda.synchronize()
    dq, dk, dv, ds = (to_f64(t) for t in g)
    rq, rk, rv, rs, ra = obw.prefill_grad_ref(p.q.f64, p.k.f64, p.v.f64, None if sk == "none" else p.sinks,
                                              dout.f64, W, p.scale, n_st, dsink_abs=True)
    assert_grad_close(dq, rq, "dq")
    assert_grad_close(dk, rk, "dk")
    assert_grad_close(dv, rv, "dv")
    if ra.max() > 0:
        assert_dsinks_close(ds, rs, ra, "dsinks")
    else:
        assert not ds.any(), "dsinks must be zero without a sink"
