"""GPU parity of the ring cache of windowed layers, through the C ABI.

* ``gqa_kv_ring_append`` is byte work: compared bit for bit with the oracle's
  append, for one-token decode steps and for ragged chunks (empty chunks, chunks
  shorter than, equal to and longer than the ring).
* ``gqa_attn_decode_ring`` is compared with the windowed definition of the full
  history (``oracle.decode_ref`` with window W) after the ring was filled on the
  GPU, and with the oracle's decode from the ring contents at full size.
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


def raw(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a device tensor (uint16 for bf16, uint32 for fp32)."""
    h = t.detach().cpu().contiguous()
    return h.view(torch.int16).numpy().view(np.uint16) if h.dtype == torch.bfloat16 else h.view(torch.int32).numpy()


def store_bits(t: gi.Tensor) -> np.ndarray:
    return t.store if t.dtype == "bf16" else t.store.view(np.uint32).view(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [128, 5, 1])
def test_ring_append_decode_step_bit_exact(device, dtype, W):
    B, Hkv, D = 9, 8, 64
    say(f"ring append decode step {dtype} W={W}")
    r = gi.ring_problem(61, B, W, "random", Hkv=Hkv, dtype=dtype)
    new = gi.make_tensor(62, gi.T_K, (B, Hkv, D), 1.0, dtype)
    newv = gi.make_tensor(62, gi.T_V, (B, Hkv, D), 1.0, dtype)
    seqlens = r.seqlens.copy()
    seqlens[0] = 1          # first token of a sequence
    seqlens[1] = W          # fills the last slot
    seqlens[2] = W + 1      # wraps to slot 0
    kr, vr = dev_tensor(r.k_ring, device), dev_tensor(r.v_ring, device)
    gq.kv_ring_append(dev_tensor(new, device), dev_tensor(newv, device), (kr, vr), dev_i32(seqlens, device))
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.ring_append_ref(store_bits(r.k_ring), store_bits(r.v_ring), store_bits(new),
                                          store_bits(newv), seqlens, W)
    assert np.array_equal(raw(kr), k_ref) and np.array_equal(raw(vr), v_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ring_append_chunks_bit_exact(device, dtype):
    W, Hkv, D = 16, 8, 64
    q_lens = np.array([0, 1, 15, 16, 17, 40, 3, 0, 48], dtype=np.int32)
    before = np.array([5, 0, 0, 7, 30, 1, 100, 2, 16], dtype=np.int32)
    seqlens = before + q_lens
    B = len(q_lens)
    say(f"ring append chunks {dtype} W={W} q_lens={list(q_lens)}")
    r = gi.ring_problem(63, B, W, seqlens, Hkv=Hkv, dtype=dtype)
    T = int(q_lens.sum())
    kn = gi.make_tensor(64, gi.T_K, (T, Hkv, D), 1.0, dtype)
    vn = gi.make_tensor(64, gi.T_V, (T, Hkv, D), 1.0, dtype)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kr, vr = dev_tensor(r.k_ring, device), dev_tensor(r.v_ring, device)
    gq.kv_ring_append(dev_tensor(kn, device), dev_tensor(vn, device), (kr, vr), dev_i32(seqlens, device),
                      cu_seqlens_q=dev_i32(cu, device))
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.ring_append_ref(store_bits(r.k_ring), store_bits(r.v_ring), store_bits(kn), store_bits(vn),
                                          seqlens, W, cu_seqlens_q=cu)
    assert np.array_equal(raw(kr), k_ref) and np.array_equal(raw(vr), v_ref)


def _history(cfg, lens, Hq, Hkv, D, dtype):
    p = gi.decode_problem(cfg, len(lens), int(max(lens)), Hq, Hkv, D, dtype=dtype, seqlens=lens)
    return p


@pytest.mark.parametrize("dtype,W,lens", [
    ("bf16", 128, [1, 2, 127, 128, 129, 300, 1000, 77]),
    ("bf16", 64, [64, 65, 500, 3]),
    ("bf16", 1, [1, 9, 200]),
    ("fp32", 128, [1, 128, 129, 400]),
    ("fp32", 16, [5, 16, 33]),
])
def test_ring_decode_matches_windowed_definition(device, dtype, W, lens):
    lens = np.asarray(lens, dtype=np.int32)
    B, Hq, Hkv, D = len(lens), 64, 8, 64
    say(f"ring decode {dtype} W={W} lens={list(lens)}")
    h = _history(65, lens, Hq, Hkv, D, dtype)
    # fill the rings on the GPU with the whole history as one chunk per sequence
    Lmax = int(lens.max())
    rows_k = np.concatenate([h.k.store[b, :lens[b]] for b in range(B)])
    rows_v = np.concatenate([h.v.store[b, :lens[b]] for b in range(B)])
    to = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)) \
        if dtype == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kr = torch.zeros((B, W, Hkv, D), dtype=tdt, device=device)
    vr = torch.zeros_like(kr)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seq_d = dev_i32(lens, device)
    gq.kv_ring_append(to(rows_k), to(rows_v), (kr, vr), seq_d, cu_seqlens_q=dev_i32(cu, device))
    out, lse = gq.attn_decode_ring(dev_tensor(h.q, device), (kr, vr), seq_d, dev_f32(h.sinks, device),
                                   return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_ref(h.q.f64, h.k.f64, h.v.f64, lens, h.sinks, window=W)
    got = to_f64(out)
    if dtype == "bf16":
        assert_bf16_close(got, o_ref, "ring decode")
        assert_lse_close(to_f64(lse), l_ref, "ring lse")
    else:
        assert_fp32_close(got, o_ref, "ring decode")
        assert_lse_close(to_f64(lse), l_ref, "ring lse", fp32=True)
    assert Lmax >= 1


def test_ring_generation_steps(device):
    # prompt appended as chunks, then decode steps: append the new token, attend
    W, Hq, Hkv, D = 32, 64, 8, 64
    prompt = np.array([40, 7, 32, 1], dtype=np.int32)
    steps = 4
    B = len(prompt)
    total = prompt + steps
    say(f"ring generation W={W} prompts={list(prompt)} steps={steps}")
    h = _history(66, total, Hq, Hkv, D, "bf16")
    kr = torch.zeros((B, W, Hkv, D), dtype=torch.bfloat16, device=device)
    vr = torch.zeros_like(kr)
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    cu = np.concatenate([[0], np.cumsum(prompt)]).astype(np.int32)
    gq.kv_ring_append(tb(np.concatenate([h.k.store[b, :prompt[b]] for b in range(B)])),
                      tb(np.concatenate([h.v.store[b, :prompt[b]] for b in range(B)])),
                      (kr, vr), dev_i32(prompt, device), cu_seqlens_q=dev_i32(cu, device))
    qs = gi.make_tensor(67, gi.T_Q, (steps, B, Hq, D), 1.0, "bf16")
    for s in range(steps):
        L = prompt + s + 1
        gq.kv_ring_append(tb(np.stack([h.k.store[b, L[b] - 1] for b in range(B)])),
                          tb(np.stack([h.v.store[b, L[b] - 1] for b in range(B)])),
                          (kr, vr), dev_i32(L, device))
        out = gq.attn_decode_ring(tb(qs.store[s]), (kr, vr), dev_i32(L, device), dev_f32(h.sinks, device))
        torch.cuda.synchronize()
        o_ref, _ = oracle.decode_ref(qs.f64[s], h.k.f64, h.v.f64, L, h.sinks, window=W)
        assert_bf16_close(to_f64(out), o_ref, f"generation step {s}")


def test_ring_decode_full_size(device):
    # windowed-layer decode at the batched-decode shape: B64 at position 8191, 128-slot rings
    r = gi.c6_ring()
    say("ring decode B64 W128 at position 8191")
    out, lse = gq.attn_decode_ring(dev_tensor(r.q, device), (dev_tensor(r.k_ring, device),
                                   dev_tensor(r.v_ring, device)), dev_i32(r.seqlens, device),
                                   dev_f32(r.sinks, device), return_lse=True)
    torch.cuda.synchronize()
    got, got_l = to_f64(out), to_f64(lse)
    assert np.isfinite(got).all()
    for b in (0, 17, 63):
        sl = slice(b, b + 1)
        o_ref, l_ref = oracle.decode_ring_ref(r.q.f64[sl], r.k_ring.f64[sl], r.v_ring.f64[sl], r.seqlens[sl],
                                              r.sinks, r.W, r.scale)
        assert_bf16_close(got[sl], o_ref, f"sequence {b}")
        assert_lse_close(got_l[sl], l_ref, "lse")


# ----------------------------------------------------------------------------- one unit per wave ("solo" plan)
# Short key ranges with at least 8 (sequence, KV head) units per CU are planned
# with one unit per wave; these cases reach that plan (2048+ units).

def _solo_env(monkeypatch, on: bool):
    # the per-head forms only (at 256+ sequences the whole-row form would take these shapes)
    monkeypatch.setenv("GQA_DECODE_ROWS", "0")
    monkeypatch.setenv("GQA_DECODE_SOLO", "1" if on else "0")


@pytest.mark.parametrize("form", ["solo", "split", "rows"])
def test_ring_decode_many_sequences(device, monkeypatch, form):
    if form == "rows":
        monkeypatch.setenv("GQA_DECODE_ROWS", "1")  # the plan's own choice at 512 sequences
    else:
        _solo_env(monkeypatch, form == "solo")
    r = gi.ring_problem(69, 512, 128, "random")
    say(f"ring decode B512 W128 random lengths form={form}")
    out, lse = gq.attn_decode_ring(dev_tensor(r.q, device), (dev_tensor(r.k_ring, device),
                                   dev_tensor(r.v_ring, device)), dev_i32(r.seqlens, device),
                                   dev_f32(r.sinks, device), return_lse=True)
    torch.cuda.synchronize()
    got, got_l = to_f64(out), to_f64(lse)
    assert np.isfinite(got).all()
    pick = [0, 1, 2, 100, 255, 256, 511] + [int(b) for b in np.flatnonzero(r.seqlens < 128)[:4]]
    for b in sorted(set(pick)):
        sl = slice(b, b + 1)
        o_ref, l_ref = oracle.decode_ring_ref(r.q.f64[sl], r.k_ring.f64[sl], r.v_ring.f64[sl], r.seqlens[sl],
                                              r.sinks, r.W, r.scale)
        assert_bf16_close(got[sl], o_ref, f"sequence {b} (L={r.seqlens[b]})")
        assert_lse_close(got_l[sl], l_ref, "lse")


def test_windowed_decode_many_sequences_solo(device, monkeypatch):
    # the same plan on an ordinary windowed decode over a longer cache
    _solo_env(monkeypatch, True)
    d = gi.decode_problem(70, 300, 400, 64, 8, 64, dtype="bf16", seqlens="random")
    say("decode B300 Lmax400 window 128 (solo plan)")
    out = gq.attn_decode(dev_tensor(d.q, device), (dev_tensor(d.k, device), dev_tensor(d.v, device)),
                         dev_i32(d.seqlens, device), dev_f32(d.sinks, device), window=128)
    torch.cuda.synchronize()
    got = to_f64(out)
    for b in (0, 1, 150, 299):
        sl = slice(b, b + 1)
        o_ref, _ = oracle.decode_ref(d.q.f64[sl], d.k.f64[sl], d.v.f64[sl], d.seqlens[sl], d.sinks, 128, d.scale)
        assert_bf16_close(got[sl], o_ref, f"sequence {b}")


def test_paged_decode_steps_many_sequences_solo(device, monkeypatch):
    # a varlen batch of single-token steps over a paged cache, window 64 -> solo plan, paged addressing
    _solo_env(monkeypatch, True)
    B = 260
    kv = gi.rng_for(71, gi.T_LEN).integers(1, 300, size=B)
    r = gi.varlen_problem(71, kv, np.ones(B, dtype=np.int32), 64, 8, 64, block_size=16, dtype="bf16")
    say("varlen B260 decode steps, paged, window 64 (solo plan)")
    out = gq.attn_varlen_paged(dev_tensor(r.q, device), (dev_tensor(r.k, device), dev_tensor(r.v, device)),
                               dev_i32(r.block_table, device), dev_i32(r.cu_seqlens_q, device),
                               dev_i32(r.seqlens_k, device), dev_f32(r.sinks, device), window=64,
                               max_q_len=1, max_kv_len=r.max_kv_len)
    torch.cuda.synchronize()
    got = to_f64(out)
    rows = [0, 1, 77, 259]
    o_ref, _ = oracle.varlen_ref(r.q.f64, r.k.f64, r.v.f64, r.cu_seqlens_q, r.seqlens_k, r.sinks, 64, r.scale,
                                 block_table=r.block_table, block_size=r.block_size, rows=rows)
    assert_bf16_close(got[rows], o_ref[rows], "paged decode steps")
