"""Pins of the RoPE oracle (CPU).

What the pages fix: θ_i = 10000^(-2i/d) and a rotation of q and k by the
position m («GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §3.4).
Pins: hand values of the table; a worked quarter-turn; the identity at m = 0;
norm preservation per pair; the relative-position identity that makes RoPE
useful for attention (<R(m)q, R(n)k> depends on m - n only); the two pairings
are the same rotation under a coordinate permutation; a pure-Python scalar
enumeration; the cache append rules (contiguous, paged, ring) by hand; and
planted mistakes (wrong sign, wrong frequency index) caught.
"""
import math

import numpy as np
import pytest

import oracle.rope as R


def test_default_table_hand_values():
    t = R.default_inv_freq(4)
    assert t.dtype == np.float32 and t.shape == (2,)
    assert t[0] == 1.0 and abs(t[1] - 0.01) < 1e-9          # 10000^0, 10000^(-1/2)
    t64 = R.default_inv_freq(64)
    assert t64[0] == 1.0 and abs(t64[16] - 0.01) < 1e-9      # i = d/4: 10000^(-1/2)
    assert abs(t64[31] / np.float32(10000.0 ** (-62 / 64)) - 1) < 1e-7


def test_quarter_turn_worked_example():
    # d = 2, θ_0 = 1: position π/2 is not an integer, so use a table of π/2 at position 1
    x = np.array([[[1.0, 0.0]]])
    out = R.rope_ref(x, [1], np.array([math.pi / 2], dtype=np.float32))
    c, s = math.cos(float(np.float32(math.pi / 2))), math.sin(float(np.float32(math.pi / 2)))
    np.testing.assert_allclose(out[0, 0], [c, s], atol=1e-15)   # (1, 0) -> (cos, sin): counter-clockwise
    y = R.rope_ref(np.array([[[0.0, 1.0]]]), [1], np.array([math.pi / 2], dtype=np.float32))
    np.testing.assert_allclose(y[0, 0], [-s, c], atol=1e-15)


@pytest.mark.parametrize("pairing", [R.PAIR_INTERLEAVED, R.PAIR_HALVES])
def test_position_zero_is_identity_and_norms_kept(pairing):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 64))
    inv = R.default_inv_freq(64)
    assert np.array_equal(R.rope_ref(x, np.zeros(5), inv, pairing), x)
    y = R.rope_ref(x, [0, 1, 17, 4095, 131071], inv, pairing)
    a, b = R.pair_index(64, pairing)
    np.testing.assert_allclose(y[..., a] ** 2 + y[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-12)


@pytest.mark.parametrize("pairing", [R.PAIR_INTERLEAVED, R.PAIR_HALVES])
def test_relative_position_identity(pairing):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    inv = R.default_inv_freq(64)
    for m, n in ((5, 2), (100, 97), (1000, 997), (7, 7)):
        lhs = float((R.rope_ref(q, [m], inv, pairing) * R.rope_ref(k, [n], inv, pairing)).sum())
        rhs = float((R.rope_ref(q, [m - n], inv, pairing) * k).sum())
        assert abs(lhs - rhs) < 1e-10, (m, n)


def test_pairings_are_a_coordinate_permutation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, 8))
    inv = R.default_inv_freq(8)
    pos = [0, 3, 11, 200]
    perm = np.array([0, 4, 1, 5, 2, 6, 3, 7])  # halves layout -> interleaved layout
    a = R.rope_ref(x, pos, inv, R.PAIR_HALVES)
    b = R.rope_ref(x[..., perm], pos, inv, R.PAIR_INTERLEAVED)
    np.testing.assert_allclose(a[..., perm], b, rtol=0, atol=1e-15)


def test_brute_force_scalar_loop():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 2, 6))
    pos = [2, 9, 40]
    inv = R.default_inv_freq(6)
    got = R.rope_ref(x, pos, inv, R.PAIR_INTERLEAVED, mscale=0.9)
    for r in range(3):
        for h in range(2):
            for i in range(3):
                th = float(inv[i]) * pos[r]
                a, b = x[r, h, 2 * i], x[r, h, 2 * i + 1]
                want_a = 0.9 * (a * math.cos(th) - b * math.sin(th))
                want_b = 0.9 * (a * math.sin(th) + b * math.cos(th))
                assert abs(got[r, h, 2 * i] - want_a) < 1e-13 and abs(got[r, h, 2 * i + 1] - want_b) < 1e-13


def test_new_positions():
    seq, pos = R.new_positions([5, 1, 9])
    assert list(seq) == [0, 1, 2] and list(pos) == [4, 0, 8]
    seq, pos = R.new_positions([5, 3, 9], cu_seqlens_q=[0, 2, 2, 5])
    assert list(seq) == [0, 0, 2, 2, 2] and list(pos) == [3, 4, 6, 7, 8]


def test_cache_rules_by_hand():
    d, Hkv, Hq = 4, 1, 1
    inv = R.default_inv_freq(d)
    k = np.arange(3 * d, dtype=np.float64).reshape(3, Hkv, d) + 1.0
    v = -k
    q = np.zeros((3, Hq, d))
    seqlens = [2, 1, 6]   # rows at positions 1, 0, 5
    # contiguous, length 4: the row at position 5 does not fit and is dropped
    _, kc, vc = R.rope_append_ref(q, k, v, seqlens, inv, np.zeros((3, 4, 1, d)), np.zeros((3, 4, 1, d)),
                                  R.CACHE_CONTIGUOUS, cache_len=4)
    assert np.array_equal(vc[0, 1, 0], v[0, 0]) and np.array_equal(vc[1, 0, 0], v[1, 0])
    assert not vc[2].any()
    np.testing.assert_allclose(kc[1, 0, 0], k[1, 0], atol=0)            # position 0: no rotation
    # ring of 2 slots: position 5 -> slot 1
    _, kc, vc = R.rope_append_ref(q, k, v, seqlens, inv, np.zeros((3, 2, 1, d)), np.zeros((3, 2, 1, d)),
                                  R.CACHE_RING, cache_len=2)
    assert np.array_equal(vc[2, 1, 0], v[2, 0]) and not vc[2, 0].any()
    # paged, block size 2: sequence 2's block 2 is physical block 0
    table = np.array([[3, 1, -1], [2, -1, -1], [4, 5, 0]])
    _, kc, vc = R.rope_append_ref(q, k, v, seqlens, inv, np.zeros((6, 2, 1, d)), np.zeros((6, 2, 1, d)),
                                  R.CACHE_PAGED, block_table=table, block_size=2)
    assert np.array_equal(vc[3, 1, 0], v[0, 0]) and np.array_equal(vc[2, 0, 0], v[1, 0])
    assert np.array_equal(vc[0, 1, 0], v[2, 0])


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((1, 1, 8))
    inv = R.default_inv_freq(8)

    def rel_gap():
        lhs = float((R.rope_ref(q, [9], inv) * R.rope_ref(k, [4], inv)).sum())
        rhs = float((R.rope_ref(q, [5], inv) * k).sum())
        return abs(lhs - rhs)

    assert rel_gap() < 1e-12
    # a rotation whose two coordinates turn opposite ways is no longer relative
    orig = R.rope_ref

    def wrong_sign(x, pos, inv_freq, pairing=0, mscale=1.0):
        y = orig(x, pos, inv_freq, pairing, mscale)
        a, b = R.pair_index(x.shape[-1], pairing)
        xx = np.asarray(x, dtype=np.float64)
        ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq.astype(np.float64)[None, :]
        y[..., b] = (xx[..., a] * np.sin(ang)[:, None, :] * -1) + xx[..., b] * np.cos(ang)[:, None, :]
        return y

    monkeypatch.setattr(R, "rope_ref", wrong_sign)
    assert rel_gap() > 1e-3
    monkeypatch.undo()
    # a table with the index off by one fails the hand values of the table pin
    monkeypatch.setattr(R, "default_inv_freq",
                        lambda d, base=10000.0: (base ** (-2.0 * (np.arange(d // 2) + 1) / d)).astype(np.float32))
    with pytest.raises(AssertionError):
        test_default_table_hand_values()
