"""Pins of the oracle's start-of-sequence sink tokens (CPU).

«GPT-OSS vs Qwen3», section "Attention Bias et Sinks", describes the classical
attention sink as a special token at the start of the sequence that is always
attended (gpt-oss itself uses a learned logit per head instead; both are
supported and combine).  Reading: with a window W > 0, the first n positions
stay visible past the window edge, still causally (j <= p).

Pins: the independent pure-Python enumeration, a closed form (window 1, one
sink token), the special cases that reduce to known results (n = 0 is the
windowed oracle, n >= p + 1 and W <= 0 are dense), cross-shape identities
(decode = last prefill row, chunk = rows of the full prefill), and a planted
off-by-one that the brute force catches.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from oracle.brute import brute_prefill, brute_row


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CASES = [(S, W, n) for S in (1, 5, 12) for W in (1, 2, 3, 5) for n in (1, 2, 4, 20)]


@pytest.mark.parametrize("S,W,n", CASES)
def test_brute_force(S, W, n):
    B, Hq, Hkv, D = 1, 4, 2, 3
    q, k, v = rand((B, S, Hq, D), S), rand((B, S, Hkv, D), S + 1), rand((B, S, Hkv, D), S + 2)
    sinks = [-math.inf, 0.0, 1.5, -2.0]
    o, lse = oracle.prefill_ref(q, k, v, sinks, window=W, scale=0.6, sink_tokens=n)
    ob, lb = brute_prefill(q.tolist(), k.tolist(), v.tolist(), sinks, W, 0.6, n)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-12)


def test_closed_form_window_one_sink_one():
    # W = 1, n = 1: a query at p >= 1 sees exactly keys 0 and p
    S, D = 7, 4
    q, k, v = rand((S, D), 3), rand((S, D), 4), rand((S, D), 5)
    s, sc = 0.3, 0.5
    o, lse = OA.attend(q, k, v, np.arange(S), np.arange(S), s, 1, sc, sink_tokens=1)
    for p in range(1, S):
        x0 = sc * float(q[p] @ k[0])
        xp = sc * float(q[p] @ k[p])
        z = math.exp(s) + math.exp(x0) + math.exp(xp)
        want = (math.exp(x0) * v[0] + math.exp(xp) * v[p]) / z
        np.testing.assert_allclose(o[p], want, rtol=1e-12, atol=1e-14)
        assert abs(lse[p] - math.log(z)) < 1e-12
    # p = 0 sees only itself
    z0 = math.exp(s) + math.exp(sc * float(q[0] @ k[0]))
    np.testing.assert_allclose(o[0], math.exp(sc * float(q[0] @ k[0])) / z0 * v[0], rtol=1e-12)


def test_zero_sink_tokens_is_the_windowed_oracle():
    q, k, v = rand((2, 40, 8, 16), 6), rand((2, 40, 2, 16), 7), rand((2, 40, 2, 16), 8)
    sinks = rand((8,), 9)
    a = oracle.prefill_ref(q, k, v, sinks, window=9)
    b = oracle.prefill_ref(q, k, v, sinks, window=9, sink_tokens=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_many_sink_tokens_or_dense_is_dense():
    q, k, v = rand((1, 30, 4, 8), 10), rand((1, 30, 1, 8), 11), rand((1, 30, 1, 8), 12)
    sinks = rand((4,), 13)
    dense = oracle.prefill_ref(q, k, v, sinks, window=0)
    for W, n in ((3, 30), (1, 100), (0, 5)):
        got = oracle.prefill_ref(q, k, v, sinks, window=W, sink_tokens=n)
        assert np.array_equal(got[0], dense[0]) and np.array_equal(got[1], dense[1]), (W, n)


def test_decode_is_last_prefill_row_with_sink_tokens():
    S, W, n = 50, 8, 3
    q, k, v = rand((1, S, 8, 16), 14), rand((1, S, 2, 16), 15), rand((1, S, 2, 16), 16)
    sinks = rand((8,), 17)
    o_p, l_p = oracle.prefill_ref(q, k, v, sinks, window=W, sink_tokens=n)
    o_d, l_d = oracle.decode_ref(q[:, -1], k, v, [S], sinks, window=W, sink_tokens=n)
    np.testing.assert_allclose(o_d, o_p[:, -1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l_d, l_p[:, :, -1], rtol=0, atol=1e-14)


def test_chunk_is_rows_of_full_prefill_with_sink_tokens():
    S, W, n, qlen = 60, 10, 4, 17
    q, k, v = rand((1, S, 4, 8), 18), rand((1, S, 2, 8), 19), rand((1, S, 2, 8), 20)
    sinks = rand((4,), 21)
    o_p, _ = oracle.prefill_ref(q, k, v, sinks, window=W, sink_tokens=n)
    cu = np.array([0, qlen])
    o_v, _ = oracle.varlen_ref(q[0, S - qlen:], k[0], v[0], cu, [S], sinks, W, block_table=None,
                               cu_seqlens_k=[0, S], sink_tokens=n)
    np.testing.assert_allclose(o_v, o_p[0, S - qlen:], rtol=0, atol=1e-14)


def test_planted_off_by_one_is_caught(monkeypatch):
    # a sink-token rule j <= n (one key too many) must disagree with the brute force
    def wrong(q_pos, k_pos, window, sink_tokens=0):
        p = np.asarray(q_pos, dtype=np.int64)[:, None]
        j = np.asarray(k_pos, dtype=np.int64)[None, :]
        vis = j <= p
        if window > 0:
            vis &= (j > p - window) | (j <= sink_tokens)
        return vis

    monkeypatch.setattr(OA, "visible_mask", wrong)
    S, W, n = 12, 2, 3
    q, k, v = rand((1, S, 2, 4), 22), rand((1, S, 1, 4), 23), rand((1, S, 1, 4), 24)
    o, _ = oracle.prefill_ref(q, k, v, None, window=W, sink_tokens=n)
    ob, _ = brute_prefill(q.tolist(), k.tolist(), v.tolist(), [-math.inf] * 2, W, 0.5, n)
    assert np.abs(o - np.array(ob)).max() > 1e-3
