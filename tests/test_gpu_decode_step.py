"""GPU parity of the fused decode step (gqa_attn_decode_step), through the C ABI.

One launch rotates each sequence's new query and key, appends the rotated key
and the value to the cache, and attends.  Checked against the two separate
calls it replaces and against the fp64 oracle:
* the cache after the step and the rotated queries equal, bit for bit, what
  gqa_rope_append writes (the rotation is the same shared code, rounded to
  bf16 once), and no other cache row changes;
* the output and log-sum-exp match the oracle decode evaluated on exactly those
  bf16 rotated queries and cache rows, to the bf16 bar (max 2e-2, mean 2e-3;
  lse: the derived 1e-3 / 1e-4);
* end to end, the output matches the oracle composition from the unrotated
  inputs (rope_append_ref, then decode_ref / decode_ring_ref), to the bf16 bar.
Contiguous, paged and ring caches; dense and windowed layers, sink tokens,
custom frequency tables, both pairings, 16, 8 and 4 query heads per KV head,
sequences of one token, shorter than the window, and far longer.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
import oracle.ring as ORING
import oracle.rope as R
from gpu_helpers import assert_bf16_close, assert_lse_close, dev_f32, dev_i32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def new_rows(cfg, B, Hq, Hkv):
    return (gi.make_tensor(cfg, gi.T_Q, (B, Hq, 64), 1.0, "bf16"),
            gi.make_tensor(cfg, gi.T_K, (B, Hkv, 64), 1.0, "bf16"),
            gi.make_tensor(cfg, gi.T_V, (B, Hkv, 64), 1.0, "bf16"))


def run_case(kind, B, Hq, Hkv, cache_shape, seqlens, window=0, sink_tokens=0, inv=None, pairing=0, mscale=1.0,
             block_table=None, cfg=80):
    """Fused step vs rope_append (bits) and vs the oracle (values); returns nothing, asserts."""
    dev = "cuda"
    q, k, v = new_rows(cfg, B, Hq, Hkv)
    kc0 = gi.make_tensor(cfg + 1, gi.T_K, cache_shape, 1.0, "bf16")
    vc0 = gi.make_tensor(cfg + 1, gi.T_V, cache_shape, 1.0, "bf16")
    sinks = gi.make_sinks(cfg, Hq, "normal")
    sl = dev_i32(seqlens, dev)
    inv_t = None if inv is None else dev_f32(inv, dev)
    bt = None if block_table is None else dev_i32(block_table, dev)
    ring = kind == R.CACHE_RING
    # the two separate calls: rope_append, then (below) the oracle on what it wrote
    kc_a, vc_a = dev_tensor(kc0, dev), dev_tensor(vc0, dev)
    q_a = gq.rope_append(dev_tensor(q, dev), dev_tensor(k, dev), dev_tensor(v, dev), sl, (kc_a, vc_a), inv_freq=inv_t,
                         pairing=pairing, mscale=mscale, block_table=bt, ring=ring)
    # the fused step
    kc_b, vc_b = dev_tensor(kc0, dev), dev_tensor(vc0, dev)
    q_b = torch.empty_like(q_a)
    out, lse = gq.attn_decode_step(dev_tensor(q, dev), dev_tensor(k, dev), dev_tensor(v, dev), sl, (kc_b, vc_b),
                                   dev_f32(sinks, dev), window=window, sink_tokens=sink_tokens, inv_freq=inv_t,
                                   mscale=mscale, pairing=pairing, block_table=bt, ring=ring, q_out=q_b,
                                   return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(q_b), bits(q_a)), "rotated queries differ from the rotary append's"
    assert np.array_equal(bits(kc_b), bits(kc_a)), "key cache differs from the rotary append's"
    assert np.array_equal(bits(vc_b), bits(vc_a)), "value cache differs from the rotary append's"
    # the oracle decode on exactly the bf16 rotated queries and cache rows
    qr, kcr, vcr = to_f64(q_b), to_f64(kc_b), to_f64(vc_b)
    scale = 1.0 / 8.0
    if kind == R.CACHE_RING:
        o_ref, l_ref = ORING.decode_ring_ref(qr, kcr, vcr, seqlens, sinks, cache_shape[1], scale)
    elif kind == R.CACHE_PAGED:
        Lmax = block_table.shape[1] * cache_shape[1]
        kf = np.stack([oracle.gather_paged(kcr, block_table[b], cache_shape[1], Lmax) for b in range(B)])
        vf = np.stack([oracle.gather_paged(vcr, block_table[b], cache_shape[1], Lmax) for b in range(B)])
        o_ref, l_ref = oracle.decode_ref(qr, kf, vf, seqlens, sinks, window, scale, sink_tokens=sink_tokens)
    else:
        o_ref, l_ref = oracle.decode_ref(qr, kcr, vcr, seqlens, sinks, window, scale, sink_tokens=sink_tokens)
    assert_bf16_close(to_f64(out), o_ref, "step output vs oracle on its bf16 inputs")
    assert_lse_close(to_f64(lse), l_ref, "step lse")
    # end to end from the unrotated inputs
    inv_np = R.default_inv_freq(64) if inv is None else inv
    q_ref, kc_ref, vc_ref = R.rope_append_ref(q.f64, k.f64, v.f64, seqlens, inv_np, kc0.f64, vc0.f64, kind,
                                              cache_len=cache_shape[1] if kind != R.CACHE_PAGED else 0,
                                              block_table=block_table, block_size=cache_shape[1],
                                              pairing=pairing, mscale=mscale)
    if kind == R.CACHE_RING:
        o_e2e, _ = ORING.decode_ring_ref(q_ref, kc_ref, vc_ref, seqlens, sinks, cache_shape[1], scale)
    elif kind == R.CACHE_PAGED:
        Lmax = block_table.shape[1] * cache_shape[1]
        kf = np.stack([oracle.gather_paged(kc_ref, block_table[b], cache_shape[1], Lmax) for b in range(B)])
        vf = np.stack([oracle.gather_paged(vc_ref, block_table[b], cache_shape[1], Lmax) for b in range(B)])
        o_e2e, _ = oracle.decode_ref(q_ref, kf, vf, seqlens, sinks, window, scale, sink_tokens=sink_tokens)
    else:
        o_e2e, _ = oracle.decode_ref(q_ref, kc_ref, vc_ref, seqlens, sinks, window, scale, sink_tokens=sink_tokens)
    assert_bf16_close(to_f64(out), o_e2e, "step output vs oracle composition from unrotated inputs")


@pytest.mark.parametrize("window,sink_tokens", [(128, 0), (128, 4), (0, 0), (300, 2)])
def test_step_contiguous(window, sink_tokens):
    B, Hq, Hkv, Lmax = 6, 64, 8, 1024
    seqlens = np.array([1, 2, 129, 700, 1000, 1024], dtype=np.int32)
    say(f"decode step contiguous W={window} sink tokens {sink_tokens}")
    run_case(R.CACHE_CONTIGUOUS, B, Hq, Hkv, (B, Lmax, Hkv, 64), seqlens, window, sink_tokens)


def test_step_contiguous_custom_table_halves_g4():
    B, Hq, Hkv, Lmax = 5, 16, 4, 512
    seqlens = np.array([3, 64, 65, 200, 512], dtype=np.int32)
    inv = (R.default_inv_freq(64, base=500000.0) * np.float32(0.25)).astype(np.float32)
    say("decode step contiguous, custom table, halves pairing, mscale 1.1, 16/4 heads")
    run_case(R.CACHE_CONTIGUOUS, B, Hq, Hkv, (B, Lmax, Hkv, 64), seqlens, 128, 0, inv=inv, pairing=1, mscale=1.1,
             cfg=82)


def test_step_sixteen_heads_per_kv_head():
    # 32 query heads over 2 KV heads: the 16 columns of the step's matrix products all in use
    B, Hq, Hkv, Lmax = 4, 32, 2, 700
    seqlens = np.array([1, 33, 640, 700], dtype=np.int32)
    say("decode step contiguous, 32/2 heads, window 256, pairing halves")
    run_case(R.CACHE_CONTIGUOUS, B, Hq, Hkv, (B, Lmax, Hkv, 64), seqlens, 256, 0, pairing=1, cfg=88)


@pytest.mark.parametrize("window", [128, 0])
def test_step_paged(window):
    r = gi.varlen_problem(84, [40, 1, 600, 1500], [1, 1, 1, 1], 64, 8, block_size=16, maxblk=128)
    say(f"decode step paged W={window}")
    run_case(R.CACHE_PAGED, 4, 64, 8, r.k.shape, np.asarray(r.seqlens_k, dtype=np.int32), window, 0,
             block_table=np.asarray(r.block_table, dtype=np.int32), cfg=85)


def test_step_ring():
    B, W = 6, 128
    seqlens = np.array([1, 5, 128, 129, 8192, 131072], dtype=np.int32)
    say("decode step ring W128 (positions to 131071)")
    run_case(R.CACHE_RING, B, 64, 8, (B, W, 8, 64), seqlens, 0, 0, cfg=86)


def test_step_rejects_long_ranges_and_fp32():
    dev = "cuda"
    q, k, v = (dev_tensor(t, dev) for t in new_rows(87, 2, 64, 8))
    kc = torch.zeros((2, 4096, 8, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(gq.GqaError):
        gq.attn_decode_step(q, k, v, dev_i32([10, 20], dev), (kc, torch.zeros_like(kc)), window=0)
