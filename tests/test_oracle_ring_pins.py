"""Pins of the ring-cache oracle (CPU).

The ring layout is a reading (position p in slot p mod W of a W-slot ring); what
the pages fix is that a windowed layer sees only the last W tokens («GPT-OSS vs
Qwen3», "Utilisation de Sliding Window Attention").  So the pins are:

* the slot contents in closed form: after positions 0..L-1, slot s holds the
  largest p < L with p = s (mod W), written out by hand with the positions
  themselves as the data;
* appending a chunk at once equals appending its rows one by one;
* decode from the ring equals the windowed decode of the full history
  (``decode_ref``, itself pinned by brute force and SDPA in test_oracle_pins),
  for rings shorter than, equal to and longer than the history, and equals the
  pure-Python brute force;
* planted mistakes (a wrong slot rule, a stale slot) fail those identities.
"""
import numpy as np
import pytest

import oracle
import oracle.ring as OR
from oracle.brute import brute_row


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_slot_contents_closed_form():
    # data = the position itself, so the ring must read back the expected positions
    for W in (1, 2, 3, 5, 8):
        for L in range(0, 3 * W + 2):
            full = np.arange(L, dtype=np.float64).reshape(1, L, 1, 1) if L else np.zeros((1, 0, 1, 1))
            full_pad = np.zeros((1, max(L, 1), 1, 1))
            full_pad[:, :L] = full
            kr, vr = OR.ring_from_history(full_pad, full_pad, [L], W)
            for s in range(W):
                cands = [p for p in range(L) if p % W == s]
                want = max(cands) if cands else 0.0
                assert kr[0, s, 0, 0] == want and vr[0, s, 0, 0] == want, (W, L, s)
            assert list(OR.ring_positions(L, W)) == list(range(max(0, L - W), L))


@pytest.mark.parametrize("W", [1, 4, 7])
def test_chunk_append_equals_row_by_row(W):
    B, Hkv, D = 3, 2, 4
    rng = np.random.default_rng(W)
    L0 = [0, 5, 2 * W + 3]       # positions before the chunk
    q_lens = [W + 3, 1, 2 * W]   # chunk lengths, some longer than the ring
    kr0 = rng.standard_normal((B, W, Hkv, D))
    vr0 = rng.standard_normal((B, W, Hkv, D))
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    T = int(cu[-1])
    kn = rng.standard_normal((T, Hkv, D))
    vn = rng.standard_normal((T, Hkv, D))
    seqlens = [L0[b] + q_lens[b] for b in range(B)]
    k_all, v_all = OR.ring_append_ref(kr0, vr0, kn, vn, seqlens, W, cu_seqlens_q=cu)
    # one row at a time, in position order, each as a one-token decode-style append
    k1, v1 = kr0.copy(), vr0.copy()
    for b in range(B):
        for t in range(q_lens[b]):
            L = L0[b] + t + 1
            kb = np.zeros((B, Hkv, D)); vb = np.zeros((B, Hkv, D))
            kb[b] = kn[cu[b] + t]; vb[b] = vn[cu[b] + t]
            sl = [0] * B
            sl[b] = L
            k_step, v_step = OR.ring_append_ref(k1, v1, kb, vb, sl, W)
            # only sequence b moved (the others had position -1: skipped)
            k1[b], v1[b] = k_step[b], v_step[b]
    assert np.array_equal(k_all, k1) and np.array_equal(v_all, v1)


@pytest.mark.parametrize("W,lens", [(8, [1, 5, 8, 9, 30]), (1, [1, 2, 7]), (16, [16, 17, 3])])
def test_ring_decode_equals_windowed_decode(W, lens):
    B, Hq, Hkv, D = len(lens), 4, 2, 8
    Lmax = max(lens)
    q = rand((B, Hq, D), 1)
    k = rand((B, Lmax, Hkv, D), 2)
    v = rand((B, Lmax, Hkv, D), 3)
    sinks = rand((Hq,), 4)
    kr, vr = OR.ring_from_history(k, v, lens, W)
    o_r, l_r = OR.decode_ring_ref(q, kr, vr, lens, sinks, W)
    o_w, l_w = oracle.decode_ref(q, k, v, lens, sinks, window=W)
    np.testing.assert_allclose(o_r, o_w, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_r, l_w, rtol=0, atol=1e-13)


def test_ring_decode_brute_force():
    W, lens = 5, [3, 5, 12]
    B, Hq, Hkv, D = 3, 2, 1, 3
    q = rand((B, Hq, D), 11)
    k = rand((B, 12, Hkv, D), 12)
    v = rand((B, 12, Hkv, D), 13)
    sinks = [0.5, -1.0]
    kr, vr = OR.ring_from_history(k, v, lens, W)
    o, lse = OR.decode_ring_ref(q, kr, vr, lens, sinks, W, scale=0.7)
    for b, L in enumerate(lens):
        for h in range(Hq):
            ob, lb, _, _ = brute_row(list(q[b, h]), [list(k[b, j, 0]) for j in range(L)],
                                     [list(v[b, j, 0]) for j in range(L)], L - 1, sinks[h], W, 0.7)
            np.testing.assert_allclose(o[b, h], ob, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, h] - lb) < 1e-12


def test_ring_longer_than_history_is_dense():
    W, lens = 64, [1, 10, 40]
    q = rand((3, 4, 8), 21)
    k = rand((3, 40, 2, 8), 22)
    v = rand((3, 40, 2, 8), 23)
    kr, vr = OR.ring_from_history(k, v, lens, W)
    o_r, _ = OR.decode_ring_ref(q, kr, vr, lens, None, W)
    o_d, _ = oracle.decode_ref(q, k, v, lens, None, window=0)
    np.testing.assert_allclose(o_r, o_d, rtol=0, atol=1e-13)


def test_planted_slot_rule_mistake_is_caught(monkeypatch):
    W, lens = 6, [20]
    q = rand((1, 2, 4), 31)
    k = rand((1, 20, 1, 4), 32)
    v = rand((1, 20, 1, 4), 33)
    o_w, _ = oracle.decode_ref(q, k, v, lens, None, window=W)
    # a slot rule off by one: the ring is filled modulo W - 1, so it holds one position fewer
    # (a rule that only permutes the last W positions would not change the result: keys are a set)
    monkeypatch.setattr(OR, "ring_slot", lambda p, W_: p % (W_ - 1))
    kr, vr = OR.ring_from_history(k, v, lens, W)
    monkeypatch.undo()
    o_r, _ = OR.decode_ring_ref(q, kr, vr, lens, None, W)
    assert np.abs(o_r - o_w).max() > 1e-3


def test_stale_slot_is_caught():
    W, lens = 4, [9]
    q = rand((1, 2, 4), 41)
    k = rand((1, 9, 1, 4), 42)
    v = rand((1, 9, 1, 4), 43)
    kr, vr = OR.ring_from_history(k, v, [8], W)  # the newest token never appended
    o_r, _ = OR.decode_ring_ref(q, kr, vr, lens, None, W)
    o_w, _ = oracle.decode_ref(q, k, v, lens, None, window=W)
    assert np.abs(o_r - o_w).max() > 1e-3
