"""GPU parity of the prefill that rotates its queries as it loads them (gqa_attn_prefill_rope).

* Against the two separate calls it replaces: the rotary append's rotated queries
  (q_out) passed to gqa_attn_prefill give, bit for bit, the same output and
  log-sum-exp (the kernel forms the angles and the rotation with the same code).
* Against the oracle: ``rope_ref`` on the unrotated queries (positions 0..S-1), then
  the prefill oracle, to the bf16 bar (sampled rows at S4096, all rows otherwise).
* The rotary append's keys-only form (q = q_out = NULL) writes the same cache bits
  as the full call.
Dense and windowed layers, sink tokens, both
pairings, the default and a custom table, mscale, and 8, 4, 3 and 1 query heads
per KV head (with 3 and 1 the two N-tiles of a wave sit at different positions).
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
import oracle.rope as R
from gpu_helpers import assert_bf16_close, dev_f32, dev_i32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def run_case(cfg, B, S, Hq, Hkv, window=0, sink_tokens=0, pairing=0, inv=None, mscale=1.0, n_rows=None):
    say(f"prefill rope B{B} S{S} heads {Hq}/{Hkv} W={window} sink tokens {sink_tokens} pairing {pairing} "
        f"table {'custom' if inv is not None else 'default'} mscale {mscale}")
    p = gi.prefill_problem(cfg, B, S, Hq, Hkv)
    q, k, v = dev_tensor(p.q, "cuda"), dev_tensor(p.k, "cuda"), dev_tensor(p.v, "cuda")
    sinks = dev_f32(p.sinks, "cuda")
    inv_t = None if inv is None else dev_f32(inv, "cuda")
    out_a, lse_a = gq.attn_prefill_rope(q, k, v, sinks, window=window, sink_tokens=sink_tokens, inv_freq=inv_t,
                                        mscale=mscale, pairing=pairing, return_lse=True)
    # the two separate calls: the rotary append's q_out, then the prefill
    cu = dev_i32(np.arange(B + 1) * S, "cuda")
    sl = dev_i32(np.full(B, S), "cuda")
    kc = torch.empty((B, S, Hkv, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    q_rot = gq.rope_append(q.view(B * S, Hq, 64), k.view(B * S, Hkv, 64), v.view(B * S, Hkv, 64), sl, (kc, vc),
                           inv_freq=inv_t, cu_seqlens_q=cu, pairing=pairing, mscale=mscale)
    out_b, lse_b = gq.attn_prefill(q_rot.view(B, S, Hq, 64), k, v, sinks, window=window, sink_tokens=sink_tokens,
                                   return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_a), bits(out_b)), "output differs from rope_append + prefill"
    assert torch.equal(lse_a, lse_b), "lse differs from rope_append + prefill"
    # the oracle composition: rotate in fp64, then attend
    inv_np = R.default_inv_freq(64) if inv is None else inv
    qr = R.rope_ref(p.q.f64, np.arange(S), inv_np, pairing, mscale)
    rows = None if n_rows is None else np.unique(np.concatenate([
        [0, 1, 31, 32, S - 1], np.random.default_rng(cfg).choice(S, n_rows, replace=False)]))
    o_ref, _ = oracle.prefill_rows_ref(qr, p.k.f64, p.v.f64, p.sinks, window, p.scale, rows=rows,
                                       sink_tokens=sink_tokens)
    got = to_f64(out_a) if rows is None else to_f64(out_a)[:, rows]
    assert_bf16_close(got, o_ref, "prefill rope vs oracle composition")


def test_dense_layer():
    # the layer-shaped B1 S4096 64/8
    run_case(100, 1, 4096, 64, 8, n_rows=40)


def test_window_layer_halves_custom_table():
    inv = (R.default_inv_freq(64, base=150000.0) * np.float32(0.5)).astype(np.float32)
    run_case(101, 1, 4096, 64, 8, window=128, pairing=1, inv=inv, mscale=1.1, n_rows=40)


def test_window_sink_tokens():
    run_case(102, 1, 1000, 64, 8, window=128, sink_tokens=4)


@pytest.mark.parametrize("Hq,Hkv,S,W,pairing", [(12, 4, 333, 0, 1), (8, 8, 200, 64, 0), (16, 4, 517, 0, 0),
                                                (24, 8, 130, 0, 0), (64, 8, 300, 128, 0), (64, 4, 200, 100, 1)])
def test_group_sizes(Hq, Hkv, S, W, pairing):
    run_case(103, 2, S, Hq, Hkv, window=W, pairing=pairing)


def test_keys_only_append_matches_full_call():
    T, Hq, Hkv, L = 300, 64, 8, 512
    q, k, v = (dev_tensor(gi.make_tensor(104, t, (T, h, 64), 1.0, "bf16"), "cuda")
               for t, h in ((gi.T_Q, Hq), (gi.T_K, Hkv), (gi.T_V, Hkv)))
    cu = dev_i32([0, 100, 300], "cuda")
    sl = dev_i32([100, 450], "cuda")
    say("rope append keys only vs full call")
    kc_a = torch.zeros((2, L, Hkv, 64), dtype=torch.bfloat16, device="cuda")
    vc_a = torch.zeros_like(kc_a)
    kc_b, vc_b = kc_a.clone(), vc_a.clone()
    gq.rope_append(q, k, v, sl, (kc_a, vc_a), cu_seqlens_q=cu, pairing=1)
    assert gq.rope_append(None, k, v, sl, (kc_b, vc_b), cu_seqlens_q=cu, pairing=1) is None
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc_a), bits(kc_b)) and np.array_equal(bits(vc_a), bits(vc_b))


def test_fp32_is_rejected():
    q = torch.zeros((1, 64, 8, 64), dtype=torch.float32, device="cuda")
    k = torch.zeros((1, 64, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(gq.GqaError):
        gq.attn_prefill_rope(q, k, k)
