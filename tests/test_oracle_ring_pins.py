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
* planted mistakes (a wrong slot rule, a stale slot) fail those identities;
* chunked prefill over the ring equals the windowed definition on the whole
  history (``varlen_ref`` over packed KV) and the brute force, for chunks
  shorter than, equal to and longer than the ring, with never-written slots
  NaN; a prompt prefilled chunk by chunk (attend, then append) equals the
  windowed prefill of the whole prompt; appending before attending and a wrong
  slot read are caught.
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


# ---------------------------------------------------------------------------
# Chunked prefill over a ring: the chunk's queries attend over the positions the
# ring holds plus the chunk's own rows, and the chunk is appended afterwards.
# Pinned against the windowed definition on the whole history (varlen_ref over
# packed KV, itself pinned by brute force and SDPA), against the pure-Python
# brute force, and by prefilling a prompt in chunks of every length class.

def chunk_problem(W, L0s, q_lens, Hq=4, Hkv=2, D=8, seed=0):
    """A history per sequence, the rings holding positions 0..L0-1 (never-written
    slots NaN, so reading one shows), and the chunk rows packed by cu_seqlens_q."""
    rng = np.random.default_rng(seed)
    B = len(L0s)
    Ls = [L0s[b] + q_lens[b] for b in range(B)]
    Lmax = max(max(Ls), 1)
    q_full = rng.standard_normal((B, Lmax, Hq, D))
    k_full = rng.standard_normal((B, Lmax, Hkv, D))
    v_full = rng.standard_normal((B, Lmax, Hkv, D))
    kr = np.full((B, W, Hkv, D), np.nan)
    vr = np.full((B, W, Hkv, D), np.nan)
    for b in range(B):
        for p in range(L0s[b]):
            kr[b, p % W] = k_full[b, p]
            vr[b, p % W] = v_full[b, p]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    q = np.concatenate([q_full[b, L0s[b]:Ls[b]] for b in range(B)])
    kn = np.concatenate([k_full[b, L0s[b]:Ls[b]] for b in range(B)])
    vn = np.concatenate([v_full[b, L0s[b]:Ls[b]] for b in range(B)])
    sinks = rng.standard_normal((Hq,))
    return q_full, k_full, v_full, kr, vr, q, kn, vn, cu, np.array(Ls), sinks


def history_ref(k_full, v_full, q, cu, Ls, sinks, W):
    """The windowed definition over each sequence's whole history (packed KV rows)."""
    B = len(Ls)
    kp = np.concatenate([k_full[b, :Ls[b]] for b in range(B)])
    vp = np.concatenate([v_full[b, :Ls[b]] for b in range(B)])
    cu_k = np.concatenate([[0], np.cumsum(Ls)]).astype(np.int64)
    return oracle.varlen_ref(q, kp, vp, cu, Ls, sinks, window=W, cu_seqlens_k=cu_k)


# (L0, q_len) pairs: fresh prompts, partly filled rings, full rings; chunks shorter
# than, equal to and longer than the ring; empty chunks between them
CASES = {
    1: [(0, 1), (0, 5), (3, 1), (3, 4), (9, 0), (9, 2)],
    4: [(0, 3), (0, 4), (0, 11), (2, 1), (2, 4), (3, 9), (4, 4), (13, 1), (13, 3), (13, 4), (13, 10), (6, 0)],
    8: [(0, 8), (5, 2), (5, 8), (7, 20), (8, 1), (30, 7), (30, 8), (30, 9), (30, 25)],
}


@pytest.mark.parametrize("W", sorted(CASES))
def test_ring_prefill_equals_history(W):
    L0s, q_lens = zip(*CASES[W])
    q_full, k_full, v_full, kr, vr, q, kn, vn, cu, Ls, sinks = chunk_problem(W, list(L0s), list(q_lens), seed=W)
    o, lse = OR.prefill_ring_ref(q, kn, vn, cu, Ls, kr, vr, sinks, W)
    o_h, lse_h = history_ref(k_full, v_full, q, cu, Ls, sinks, W)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, o_h, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_h, rtol=0, atol=1e-13)


def test_ring_prefill_brute_force():
    W, scale = 3, 0.7
    L0s, q_lens = [0, 2, 7, 4], [4, 2, 5, 1]
    q_full, k_full, v_full, kr, vr, q, kn, vn, cu, Ls, _ = chunk_problem(W, L0s, q_lens, Hq=2, Hkv=1, D=3, seed=5)
    sinks = [0.3, -np.inf]
    o, lse = OR.prefill_ring_ref(q, kn, vn, cu, Ls, kr, vr, sinks, W, scale=scale)
    for b in range(len(L0s)):
        keys = [list(k_full[b, j, 0]) for j in range(Ls[b])]
        vals = [list(v_full[b, j, 0]) for j in range(Ls[b])]
        for t in range(q_lens[b]):
            r, p = cu[b] + t, L0s[b] + t
            for h in range(2):
                ob, lb, _, _ = brute_row(list(q[r, h]), keys, vals, p, sinks[h], W, scale)
                np.testing.assert_allclose(o[r, h], ob, rtol=1e-12, atol=1e-12)
                assert abs(lse[h, r] - lb) < 1e-12


@pytest.mark.parametrize("W,schedule", [
    (4, [[1, 4], [2, 1], [4, 9], [9, 0], [1, 1], [0, 3]]),   # per call: chunk lengths of the two sequences
    (8, [[8, 3], [20, 8], [1, 9], [7, 16]]),
])
def test_prompt_in_chunks_equals_full_prefill(W, schedule):
    """A prompt prefilled chunk by chunk through the ring (attend, then append) gives
    the rows of the windowed prefill of the whole prompt, and leaves the ring of the
    whole prompt."""
    Hq, Hkv, D = 4, 2, 8
    S = [sum(c[b] for c in schedule) for b in range(2)]
    rng = np.random.default_rng(W + 100)
    Smax = max(S)
    q_full = rng.standard_normal((2, Smax, Hq, D))
    k_full = rng.standard_normal((2, Smax, Hkv, D))
    v_full = rng.standard_normal((2, Smax, Hkv, D))
    sinks = rng.standard_normal((Hq,))
    kr = np.full((2, W, Hkv, D), np.nan)
    vr = np.full((2, W, Hkv, D), np.nan)
    got = np.zeros((2, Smax, Hq, D))
    done = [0, 0]
    for lens in schedule:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        Ls = np.array([done[b] + lens[b] for b in range(2)])
        q = np.concatenate([q_full[b, done[b]:Ls[b]] for b in range(2)])
        kn = np.concatenate([k_full[b, done[b]:Ls[b]] for b in range(2)])
        vn = np.concatenate([v_full[b, done[b]:Ls[b]] for b in range(2)])
        o, _, kr, vr = OR.prefill_ring_append_ref(q, kn, vn, cu, Ls, kr, vr, sinks, W)
        for b in range(2):
            got[b, done[b]:Ls[b]] = o[cu[b]:cu[b + 1]]
        done = list(Ls)
    for b in range(2):
        ref, _ = oracle.prefill_ref(q_full[b:b + 1, :S[b]], k_full[b:b + 1, :S[b]], v_full[b:b + 1, :S[b]], sinks,
                                    window=W)
        np.testing.assert_allclose(got[b, :S[b]], ref[0], rtol=0, atol=1e-13)
        kw, vw = OR.ring_from_history(k_full[b:b + 1], v_full[b:b + 1], [S[b]], W)
        held = [p % W for p in range(max(0, S[b] - W), S[b])]
        assert np.array_equal(kr[b, held], kw[0, held]) and np.array_equal(vr[b, held], vw[0, held])


def test_fresh_prompt_is_the_windowed_prefill():
    W = 5
    q_full, k_full, v_full, kr, vr, q, kn, vn, cu, Ls, sinks = chunk_problem(W, [0], [17], seed=9)
    o, lse = OR.prefill_ring_ref(q, kn, vn, cu, Ls, kr, vr, sinks, W)
    ref, lse_ref = oracle.prefill_ref(q_full[:, :17], k_full[:, :17], v_full[:, :17], sinks, window=W)
    np.testing.assert_allclose(o, ref[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref[0], rtol=0, atol=1e-13)


def test_planted_append_before_attend_is_caught():
    # appending the chunk first overwrites slots the chunk's first queries still read
    W = 4
    L0s, q_lens = [6, 6], [2, 7]
    q_full, k_full, v_full, kr, vr, q, kn, vn, cu, Ls, sinks = chunk_problem(W, L0s, q_lens, seed=13)
    o_h, _ = history_ref(k_full, v_full, q, cu, Ls, sinks, W)
    k2, v2 = OR.ring_append_ref(kr, vr, kn, vn, Ls, W, cu_seqlens_q=cu)
    o_bad, _ = OR.prefill_ring_ref(q, kn, vn, cu, Ls, k2, v2, sinks, W)
    for b in range(2):
        assert np.abs(o_bad[cu[b]:cu[b + 1]] - o_h[cu[b]:cu[b + 1]]).max() > 1e-3, b


def test_planted_slot_read_mistake_is_caught(monkeypatch):
    W = 4
    q_full, k_full, v_full, kr, vr, q, kn, vn, cu, Ls, sinks = chunk_problem(W, [10], [3], seed=17)
    o_h, _ = history_ref(k_full, v_full, q, cu, Ls, sinks, W)
    monkeypatch.setattr(OR, "ring_slot", lambda p, W_: (p + 1) % W_)
    o_bad, _ = OR.prefill_ring_ref(q, kn, vn, cu, Ls, kr, vr, sinks, W)
    assert np.abs(o_bad - o_h).max() > 1e-3
