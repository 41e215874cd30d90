"""GPU parity of chunked prefill over a ring (gqa_attn_prefill_ring), through the C ABI.

A chunk of new tokens of a windowed layer attends over the positions its W-slot
ring still holds plus its own rows, then (append) joins the ring.  Checked
against the oracle's ``prefill_ring_ref`` on the same bf16 / fp32 values, to the
bf16 bar (max 2e-2, mean 2e-3; lse: the derived 1e-3 / 1e-4) or the fp32 bar;
ring slots never written hold NaN, so reading one shows; the rings after the
call equal the oracle's append bit for bit (or are untouched without append).
Chunks shorter than, equal to and longer than W, fresh prompts, partly filled
and full rings, one-row chunks (decode steps), empty chunks, positions past
131072, and a prompt prefilled chunk by chunk against the windowed prefill of
the whole prompt.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
import oracle.ring as ORING
from gpu_helpers import (assert_bf16_close, assert_fp32_close, assert_lse_close, dev_f32, dev_i32, dev_tensor, say,
                         to_f64)

pytestmark = pytest.mark.gpu

NAN_BITS = {"bf16": np.uint16(0x7FC0), "fp32": np.float32(np.nan)}


def raw(t: torch.Tensor) -> np.ndarray:
    h = t.detach().cpu().contiguous()
    return h.view(torch.int16).numpy().view(np.uint16) if h.dtype == torch.bfloat16 else h.view(torch.int32).numpy()


def store_bits(t: gi.Tensor) -> np.ndarray:
    return t.store if t.dtype == "bf16" else t.store.view(np.uint32).view(np.int32)


def rings_before(cfg, B, W, Hkv, L0s, dtype):
    """Rings holding positions 0..L0-1 (values drawn directly); slots never written are NaN."""
    kr = gi.make_tensor(cfg, gi.T_K, (B, W, Hkv, 64), 1.0, dtype)
    vr = gi.make_tensor(cfg, gi.T_V, (B, W, Hkv, 64), 1.0, dtype)
    for b, L0 in enumerate(L0s):
        if L0 < W:
            kr.store[b, L0:] = NAN_BITS[dtype]
            vr.store[b, L0:] = NAN_BITS[dtype]
    return kr, vr


def run_chunks(cfg, W, pairs, Hq=64, Hkv=8, dtype="bf16", append=True, sink_kind="normal", scale=None):
    L0s = np.array([p[0] for p in pairs], dtype=np.int64)
    q_lens = np.array([p[1] for p in pairs], dtype=np.int64)
    B, T = len(pairs), int(q_lens.sum())
    seqlens = (L0s + q_lens).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kr, vr = rings_before(cfg, B, W, Hkv, L0s, dtype)
    q = gi.make_tensor(cfg + 1, gi.T_Q, (T, Hq, 64), 1.0, dtype)
    kn = gi.make_tensor(cfg + 1, gi.T_K, (T, Hkv, 64), 1.0, dtype)
    vn = gi.make_tensor(cfg + 1, gi.T_V, (T, Hkv, 64), 1.0, dtype)
    sinks = gi.make_sinks(cfg, Hq, sink_kind)
    say(f"ring prefill {dtype} W={W} heads {Hq}/{Hkv} append={append} (L0, q_len)={pairs}")
    kr_d, vr_d = dev_tensor(kr, "cuda"), dev_tensor(vr, "cuda")
    out, lse = gq.attn_prefill_ring(dev_tensor(q, "cuda"), dev_tensor(kn, "cuda"), dev_tensor(vn, "cuda"),
                                    dev_i32(cu, "cuda"), dev_i32(seqlens, "cuda"), (kr_d, vr_d),
                                    sinks=dev_f32(sinks, "cuda"), scale=scale, append=append, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = ORING.prefill_ring_ref(q.f64, kn.f64, vn.f64, cu, seqlens, kr.f64, vr.f64, sinks, W, scale)
    if dtype == "bf16":
        assert_bf16_close(to_f64(out), o_ref, "ring prefill output")
    else:
        assert_fp32_close(to_f64(out), o_ref, "ring prefill output")
    assert_lse_close(to_f64(lse), l_ref, "ring prefill lse", fp32=dtype == "fp32")
    if append:
        k_ref, v_ref = ORING.ring_append_ref(store_bits(kr), store_bits(vr), store_bits(kn), store_bits(vn), seqlens, W,
                                             cu_seqlens_q=cu)
    else:
        k_ref, v_ref = store_bits(kr), store_bits(vr)
    assert np.array_equal(raw(kr_d), k_ref) and np.array_equal(raw(vr_d), v_ref), "rings after the call"


# (L0, q_len): fresh prompts, partly filled and full rings; chunks shorter than,
# equal to and longer than the ring; one-row chunks; an empty chunk
PAIRS_128 = [(0, 1), (0, 100), (0, 128), (0, 300), (50, 78), (50, 128), (127, 129), (128, 1), (500, 64),
             (500, 128), (500, 129), (500, 700), (10, 0), (3000, 33)]


@pytest.mark.parametrize("append", [True, False])
def test_ring_prefill_w128(append):
    run_chunks(90, 128, PAIRS_128, append=append)


def test_ring_prefill_far_positions():
    run_chunks(91, 128, [(131000, 513), (131071, 1), (262144, 128), (1 << 20, 200)])


def test_ring_prefill_small_ring_g4():
    # a ring that is not a power of two, 16 query heads over 4 KV heads, no sink
    run_chunks(92, 5, [(0, 1), (0, 7), (2, 3), (4, 5), (9, 70), (33, 1)], Hq=16, Hkv=4, sink_kind="none")


def test_ring_prefill_one_slot():
    run_chunks(93, 1, [(0, 40), (7, 1), (7, 65)], Hq=8, Hkv=1, scale=0.3)


def test_ring_prefill_fp32():
    run_chunks(94, 16, [(0, 5), (0, 16), (3, 40), (20, 16), (20, 17), (100, 1)], Hq=16, Hkv=2, dtype="fp32")


def test_prompt_in_chunks_equals_windowed_prefill():
    """Three prompts prefilled chunk by chunk through their rings (attend, then append)
    give the rows of the windowed prefill of the whole prompts."""
    W, Hq, Hkv = 128, 64, 8
    schedule = [[1, 128, 300], [127, 0, 128], [129, 64, 1], [1, 500, 40], [260, 1, 128]]
    S = [sum(c[b] for c in schedule) for b in range(3)]
    Smax = max(S)
    p = gi.prefill_problem(95, 3, Smax, Hq, Hkv)
    qf, kf, vf = (dev_tensor(t, "cuda") for t in (p.q, p.k, p.v))
    kr = torch.full((3, W, Hkv, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    vr = torch.full_like(kr, float("nan"))
    sinks = dev_f32(p.sinks, "cuda")
    got = torch.zeros((3, Smax, Hq, 64), dtype=torch.bfloat16, device="cuda")
    done = [0, 0, 0]
    for lens in schedule:
        ends = [done[b] + lens[b] for b in range(3)]
        say(f"prompt in chunks: chunk lengths {lens}, positions {done} -> {ends}")
        cu = dev_i32(np.concatenate([[0], np.cumsum(lens)]), "cuda")
        q = torch.cat([qf[b, done[b]:ends[b]] for b in range(3)]).contiguous()
        k = torch.cat([kf[b, done[b]:ends[b]] for b in range(3)]).contiguous()
        v = torch.cat([vf[b, done[b]:ends[b]] for b in range(3)]).contiguous()
        o = gq.attn_prefill_ring(q, k, v, cu, dev_i32(ends, "cuda"), (kr, vr), sinks=sinks)
        r = 0
        for b in range(3):
            got[b, done[b]:ends[b]] = o[r:r + lens[b]]
            r += lens[b]
        done = ends
    torch.cuda.synchronize()
    for b in range(3):
        ref, _ = oracle.prefill_ref(p.q.f64[b:b + 1, :S[b]], p.k.f64[b:b + 1, :S[b]], p.v.f64[b:b + 1, :S[b]],
                                    p.sinks, window=W, scale=p.scale)
        assert_bf16_close(to_f64(got[b, :S[b]]), ref[0], f"prompt {b} in chunks vs windowed prefill")
        held = [q % W for q in range(max(0, S[b] - W), S[b])]
        want = kf[b, max(0, S[b] - W):S[b]]
        assert torch.equal(kr[b, held].view(torch.int16), want.view(torch.int16)), f"ring of prompt {b}"


def test_ring_prefill_rejects_bad_args():
    kr = torch.zeros((2, 8, 8, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda")
    cu = dev_i32([0, 2, 4], "cuda")
    sl = dev_i32([2, 2], "cuda")
    with pytest.raises(ValueError):   # k_new of the wrong shape (the binding checks shapes)
        gq.attn_prefill_ring(q, k[:3], k[:3], cu, sl, (kr, kr))
    with pytest.raises(ValueError):   # cu_seqlens_q of the wrong length
        gq.attn_prefill_ring(q, k, k, dev_i32([0, 4], "cuda"), sl, (kr, kr))
