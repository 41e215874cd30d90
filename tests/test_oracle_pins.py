"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (a dropped or
mis-scaled sink, a window one key too wide, the other query-head grouping, a
transposed operand, a wrong causal alignment) fails at least one of them; the
mutation tests at the end plant such mistakes in the oracle and check that.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as OA
from oracle.brute import brute_prefill, brute_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_problem(seed, B, S, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    return q, k, v


# ---------------------------------------------------------------- hand-derived worked examples

def _val(sv):
    sv = sv.strip()
    if sv == "-inf":
        return -math.inf
    if sv.startswith("ln "):
        rest = sv[3:]
        if "/" in rest:
            n, d = rest.split("/")
            return math.log(float(n)) / float(d)
        return math.log(float(rest))
    return float(Fraction(sv))


def _arr(x):
    return np.vectorize(_val, otypes=[np.float64])(np.array(x, dtype=object))


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def check_golden(case):
    q = _arr(case["q"])[None]
    k = _arr(case["k"])[None]
    v = _arr(case["v"])[None]
    sinks = _arr(case["sinks"])
    scale = None if case["scale"] == "default" else _val(case["scale"])
    o, lse = oracle.prefill_ref(q, k, v, sinks, case["window"], scale)
    ok_o = np.allclose(o[0], _arr(case["o"]), rtol=1e-13, atol=1e-14)
    ok_l = np.allclose(lse[0], _arr(case["lse"]), rtol=1e-13, atol=1e-14)
    return ok_o and ok_l


@pytest.mark.parametrize("idx", range(len(golden_cases())))
def test_golden_hand_examples(idx):
    assert check_golden(golden_cases()[idx])


# ---------------------------------------------------------------- P1 brute force

BRUTE_GRID = [
    (S, D, hq, hkv, W, s)
    for S in (1, 2, 5, 12)
    for D in (1, 4, 8)
    for (hq, hkv) in ((1, 1), (2, 1), (4, 2), (8, 2))
    for W in (0, 1, 2, 3, 12, 17)
    for s in (-math.inf, -3.0, 0.0, 2.5)
]


def brute_agrees(S, D, hq, hkv, W, s, seed=0):
    q, k, v = rand_problem(seed + 1000 * S + D, 1, S, hq, hkv, D)
    sinks = np.full((hq,), s)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.prefill_ref(q, k, v, sinks, W, scale)
    ob, lb = brute_prefill(q.tolist(), k.tolist(), v.tolist(), sinks.tolist(), W, scale)
    return np.allclose(o, np.array(ob), rtol=1e-12, atol=1e-13) and np.allclose(lse, np.array(lb), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S,D,hq,hkv,W,s", BRUTE_GRID[::7])
def test_brute_force_grid(S, D, hq, hkv, W, s):
    assert brute_agrees(S, D, hq, hkv, W, s)


def test_brute_force_per_head_sinks():
    q, k, v = rand_problem(7, 2, 9, 8, 2, 4)
    sinks = np.array([-math.inf, -3.0, 0.0, 2.5, 1.0, -0.5, -math.inf, 4.0])
    for W in (0, 1, 4, 9):
        o, lse = oracle.prefill_ref(q, k, v, sinks, W, 0.37)
        ob, lb = brute_prefill(q.tolist(), k.tolist(), v.tolist(), sinks.tolist(), W, 0.37)
        np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P2 closed forms

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def test_closed_form_window_one():
    """W = 1: only the query's own key is visible, so o_p = v_p * sigmoid(x_pp - s)."""
    q, k, v = rand_problem(3, 1, 10, 4, 2, 8)
    sinks = np.array([-1.0, 0.5, 2.0, -math.inf])
    sc = 0.3
    o, lse = oracle.prefill_ref(q, k, v, sinks, 1, sc)
    for h in range(4):
        g = h // 2
        x = sc * np.einsum("sd,sd->s", q[0, :, h], k[0, :, g])
        w = sigmoid(x - sinks[h])
        np.testing.assert_allclose(o[0, :, h], v[0, :, g] * w[:, None], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[0, h], np.logaddexp(x, sinks[h]), rtol=1e-13)


def test_closed_form_first_row():
    """Row 0 of a dense causal prefill sees only key 0: same logistic form."""
    q, k, v = rand_problem(4, 1, 6, 2, 1, 4)
    sinks = np.array([0.7, -2.0])
    o, _ = oracle.prefill_ref(q, k, v, sinks, 0, None)
    for h in range(2):
        x = 0.5 * q[0, 0, h] @ k[0, 0, 0]
        np.testing.assert_allclose(o[0, 0, h], v[0, 0, 0] * sigmoid(x - sinks[h]), rtol=1e-13)


def test_off_by_one_softmax():
    """s = 0: weights exp(x_j) / (1 + sum_k exp(x_k)), evaluated without any max shift."""
    rng = np.random.default_rng(11)
    S, D = 7, 4
    q = rng.uniform(-1, 1, (1, S, 1, D))
    k = rng.uniform(-1, 1, (1, S, 1, D))
    v = rng.standard_normal((1, S, 1, D))
    o, lse = oracle.prefill_ref(q, k, v, np.zeros(1), 0, 1.0)
    for t in range(S):
        e = [math.exp(float(q[0, t, 0] @ k[0, j, 0])) for j in range(t + 1)]
        den = 1.0 + sum(e)
        want = sum(e[j] * v[0, j, 0] for j in range(t + 1)) / den
        np.testing.assert_allclose(o[0, t, 0], want, rtol=1e-13)
        np.testing.assert_allclose(lse[0, 0, t], math.log(den), rtol=1e-13)


# ---------------------------------------------------------------- P3 library routine (torch SDPA, fp64, CPU)

def sdpa_reference(q, k, v, sinks, window, scale):
    """torch SDPA on repeated K/V with a band mask; a finite sink becomes one extra key
    with k = 0, v = 0 and additive bias s_h."""
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    keep = j <= i
    if window > 0:
        keep &= j > i - window
    bias = torch.zeros((1, Hq, S, S + 1), dtype=torch.float64)
    bias[..., :S] = torch.where(keep, 0.0, -math.inf)
    bias[..., S] = torch.from_numpy(np.asarray(sinks, dtype=np.float64))[:, None]
    zk = torch.zeros((B, Hq, 1, D), dtype=torch.float64)
    # the extra key has logit scale*q.0 + bias = s_h and value 0
    tk = torch.cat([tk, zk], dim=2)
    tv = torch.cat([tv, zk], dim=2)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=bias, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("hq,hkv,S,W", [(8, 2, 33, 0), (8, 2, 33, 5), (4, 4, 20, 0), (6, 1, 17, 3), (8, 8, 40, 16)])
def test_sdpa_no_sink(hq, hkv, S, W):
    q, k, v = rand_problem(hq * 100 + S, 2, S, hq, hkv, 16)
    sinks = np.full((hq,), -math.inf)
    o, _ = oracle.prefill_ref(q, k, v, sinks, W, 0.25)
    # the extra sink key gets bias -inf: plain softmax attention
    np.testing.assert_allclose(o, sdpa_reference(q, k, v, sinks, W, 0.25), rtol=1e-11, atol=1e-12)
    # and without the extra column at all, using torch's own causal flag when W = 0
    if W == 0:
        G = hq // hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.25)
        np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("W", [0, 1, 7, 64])
def test_sdpa_with_sink(W):
    q, k, v = rand_problem(77 + W, 1, 50, 8, 2, 8)
    sinks = np.random.default_rng(5).standard_normal(8) * 2
    o, _ = oracle.prefill_ref(q, k, v, sinks, W, None)
    np.testing.assert_allclose(o, sdpa_reference(q, k, v, sinks, W, 1 / math.sqrt(8)), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P5..P9 invariants

def test_window_at_least_length_is_dense():
    q, k, v = rand_problem(8, 1, 30, 4, 2, 8)
    sinks = np.array([0.1, -0.2, 1.5, -math.inf])
    o0, l0 = oracle.prefill_ref(q, k, v, sinks, 0, None)
    for W in (30, 31, 1000):
        o1, l1 = oracle.prefill_ref(q, k, v, sinks, W, None)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, _ = oracle.prefill_ref(q, k, v, sinks, 29, None)
    assert not np.allclose(o0[0, -1], o2[0, -1])


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = rand_problem(9, 2, 16, 8, 2, 8)
    sinks = np.linspace(-2, 2, 8)
    for W in (0, 5):
        o_g, l_g = oracle.prefill_ref(q, k, v, sinks, W, None)
        o_m, l_m = oracle.prefill_ref(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), sinks, W, None)
        np.testing.assert_array_equal(o_g, o_m)
        np.testing.assert_array_equal(l_g, l_m)


def test_probability_mass_is_one():
    q, k, v = rand_problem(10, 1, 25, 4, 1, 8)
    sinks = np.array([-math.inf, -1.0, 0.0, 3.0])
    for W in (0, 6):
        P, SM = oracle.probabilities(q, k, v, sinks, W, None)
        total = P.sum(axis=-1) + SM
        np.testing.assert_allclose(total, 1.0, rtol=0, atol=1e-15)
        assert (P >= 0).all() and (SM >= 0).all()
        # zero mass outside the visible set
        vis = OA.visible_mask(np.arange(25), np.arange(25), W)
        assert (P[..., ~vis] == 0).all()


def test_output_bounded_by_visible_values():
    q, k, v = rand_problem(12, 1, 20, 2, 1, 8)
    sinks = np.array([0.5, -math.inf])
    P, SM = oracle.probabilities(q, k, v, sinks, 4, None)
    o, _ = oracle.prefill_ref(q, k, v, sinks, 4, None)
    for h in range(2):
        for t in range(20):
            vis = [j for j in range(20) if t - 4 < j <= t]
            bound = (1 - SM[0, h, t]) * np.abs(v[0, vis, 0]).max(axis=0)
            assert (np.abs(o[0, t, h]) <= bound + 1e-14).all()


def test_key_permutation_and_value_linearity():
    rng = np.random.default_rng(13)
    L, D = 20, 8
    qv = rng.standard_normal((3, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    q_pos = np.array([5, 12, 19])
    k_pos = np.arange(L)
    o, lse = OA.attend(qv, k, v, q_pos, k_pos, 0.4, 8, 0.3)
    perm = rng.permutation(L)
    o_p, lse_p = OA.attend(qv, k[perm], v[perm], q_pos, k_pos[perm], 0.4, 8, 0.3)
    np.testing.assert_allclose(o, o_p, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse_p, rtol=1e-14)
    v2 = rng.standard_normal((L, D))
    o2, _ = OA.attend(qv, k, v2, q_pos, k_pos, 0.4, 8, 0.3)
    o3, _ = OA.attend(qv, k, 2.0 * v - 3.0 * v2, q_pos, k_pos, 0.4, 8, 0.3)
    np.testing.assert_allclose(o3, 2.0 * o - 3.0 * o2, rtol=1e-12, atol=1e-13)


def test_sink_limits():
    """s -> -inf approaches plain softmax; s -> +inf drives every output to zero."""
    q, k, v = rand_problem(14, 1, 12, 2, 1, 4)
    o_none, _ = oracle.prefill_ref(q, k, v, np.full(2, -math.inf), 0, None)
    o_low, _ = oracle.prefill_ref(q, k, v, np.full(2, -60.0), 0, None)
    np.testing.assert_allclose(o_low, o_none, rtol=1e-20, atol=1e-20)
    o_high, _ = oracle.prefill_ref(q, k, v, np.full(2, 80.0), 0, None)
    assert np.abs(o_high).max() < 1e-30
    o_inf, lse_inf = oracle.prefill_ref(q, k, v, np.full(2, math.inf), 0, None)
    assert (o_inf == 0).all() and (lse_inf == math.inf).all()
    o_nan, _ = oracle.prefill_ref(q, k, v, np.array([math.nan, 0.0]), 0, None)
    assert np.isnan(o_nan[0, :, 0]).all() and np.isfinite(o_nan[0, :, 1]).all()


def test_empty_visible_set():
    """No visible key and no sink: o = 0, lse = s (here -inf); with a sink, lse = s."""
    o, lse = OA.attend(np.ones((1, 4)), np.ones((3, 4)), np.ones((3, 4)), [1], [5, 6, 7], -math.inf, 0, 1.0)
    assert (o == 0).all() and lse[0] == -math.inf
    o, lse = OA.attend(np.ones((1, 4)), np.ones((3, 4)), np.ones((3, 4)), [1], [5, 6, 7], 0.25, 0, 1.0)
    assert (o == 0).all() and lse[0] == 0.25
    o, lse = OA.attend(np.ones((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), [0], [], 0.25, 0, 1.0)
    assert (o == 0).all() and lse[0] == 0.25


# ---------------------------------------------------------------- P10 cross-shape identities

def test_decode_is_last_prefill_row():
    q, k, v = rand_problem(15, 3, 23, 8, 2, 8)
    sinks = np.linspace(-1, 1, 8)
    for W in (0, 4):
        o_p, l_p = oracle.prefill_ref(q, k, v, sinks, W, None)
        # decode with caches padded beyond the valid length (garbage after seqlen)
        kc = np.concatenate([k, np.full((3, 5, 2, 8), 1e6)], axis=1)
        vc = np.concatenate([v, np.full((3, 5, 2, 8), 1e6)], axis=1)
        o_d, l_d = oracle.decode_ref(q[:, -1], kc, vc, np.array([23, 23, 23]), sinks, W, None)
        np.testing.assert_allclose(o_d, o_p[:, -1], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(l_d, l_p[:, :, -1], rtol=1e-13)
        # a shorter seqlen is the prefill of the truncated sequence
        o_d2, _ = oracle.decode_ref(q[:, 10], kc, vc, np.array([11, 11, 11]), sinks, W, None)
        np.testing.assert_allclose(o_d2, o_p[:, 10], rtol=1e-13, atol=1e-15)


def test_brute_decode_row():
    q, k, v = rand_problem(16, 1, 9, 2, 1, 4)
    o_d, l_d = oracle.decode_ref(q[:, 8], k, v, np.array([9]), np.array([0.3, -0.3]), 3, 0.5)
    for h in range(2):
        ob, lb, _, _ = brute_row(q[0, 8, h].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 8,
                                 [0.3, -0.3][h], 3, 0.5)
        np.testing.assert_allclose(o_d[0, h], ob, rtol=1e-12)
        np.testing.assert_allclose(l_d[0, h], lb, rtol=1e-12)


def test_chunked_prefill_is_rows_of_full_prefill():
    """Queries that are the newest q_len positions (bottom-right alignment) give the
    same rows as the full prefill."""
    q, k, v = rand_problem(17, 1, 40, 8, 2, 8)
    sinks = np.linspace(-1, 1, 8)
    for W in (0, 6):
        o_full, l_full = oracle.prefill_ref(q, k, v, sinks, W, None)
        for qlen in (1, 7, 40):
            cu_q = np.array([0, qlen])
            cu_k = np.array([0, 40])
            o_c, l_c = oracle.varlen_ref(q[0, 40 - qlen:], k[0], v[0], cu_q, np.array([40]), sinks, W, None,
                                         block_table=None, cu_seqlens_k=cu_k)
            np.testing.assert_allclose(o_c, o_full[0, 40 - qlen:], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(l_c, l_full[0][:, 40 - qlen:], rtol=1e-13)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(18)
    Hq, Hkv, D, bs = 4, 2, 8, 4
    lens = [13, 1, 8, 21]
    qlens = [5, 1, 8, 1]
    seqs_k = [rng.standard_normal((L, Hkv, D)) for L in lens]
    seqs_v = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((sum(qlens), Hq, D))
    sinks = rng.standard_normal(Hq)
    nb = [(L + bs - 1) // bs for L in lens]
    perm = rng.permutation(sum(nb) + 3)
    kc = rng.standard_normal((len(perm), bs, Hkv, D)) * 1e6  # garbage in unused slots
    vc = rng.standard_normal((len(perm), bs, Hkv, D)) * 1e6
    table = np.full((4, 8), -1)
    off = 0
    for b, L in enumerate(lens):
        for i in range(nb[b]):
            blk = perm[off + i]
            table[b, i] = blk
            n = min(bs, L - i * bs)
            kc[blk, :n] = seqs_k[b][i * bs:i * bs + n]
            vc[blk, :n] = seqs_v[b][i * bs:i * bs + n]
        off += nb[b]
    cu_q = np.concatenate([[0], np.cumsum(qlens)])
    cu_k = np.concatenate([[0], np.cumsum(lens)])
    for W in (0, 3):
        o_p, l_p = oracle.varlen_ref(q, kc, vc, cu_q, np.array(lens), sinks, W, None, block_table=table, block_size=bs)
        o_c, l_c = oracle.varlen_ref(q, np.concatenate(seqs_k), np.concatenate(seqs_v), cu_q, np.array(lens), sinks,
                                     W, None, cu_seqlens_k=cu_k)
        np.testing.assert_array_equal(o_p, o_c)
        np.testing.assert_array_equal(l_p, l_c)
        # and each sequence against the brute force
        for b in range(4):
            for t in range(qlens[b]):
                p = lens[b] - qlens[b] + t
                for h in range(Hq):
                    ob, lb, _, _ = brute_row(q[cu_q[b] + t, h].tolist(), seqs_k[b][:, h // 2].tolist(),
                                             seqs_v[b][:, h // 2].tolist(), p, sinks[h], W, 1 / math.sqrt(D))
                    np.testing.assert_allclose(o_p[cu_q[b] + t, h], ob, rtol=1e-12, atol=1e-14)


def test_row_subset_matches_full():
    q, k, v = rand_problem(19, 1, 30, 4, 2, 8)
    sinks = np.array([0.0, 1.0, -1.0, -math.inf])
    o, lse = oracle.prefill_ref(q, k, v, sinks, 7, None)
    rows = np.array([0, 3, 17, 29])
    o_r, l_r = oracle.prefill_rows_ref(q, k, v, sinks, 7, None, rows=rows)
    np.testing.assert_array_equal(o_r, o[:, rows])
    np.testing.assert_array_equal(l_r, lse[:, :, rows])


# ---------------------------------------------------------------- planted mistakes must be caught

def core_pins_pass():
    """A compact run of the independent pins; False as soon as one disagrees.

    Any exception propagates: a planted mistake counts as caught only when a
    pin compares values and finds them different, never because the mutated
    oracle crashed.
    """
    for case in golden_cases():
        if not check_golden(case):
            return False
    for args in [(5, 4, 4, 2, 0, 0.5), (6, 4, 8, 2, 2, -1.0), (7, 2, 2, 1, 3, -math.inf), (4, 8, 4, 2, 1, 1.5)]:
        if not brute_agrees(*args):
            return False
    q, k, v = rand_problem(99, 1, 12, 4, 2, 4)
    sinks = np.array([0.3, -0.7, 1.1, -math.inf])
    o, _ = oracle.prefill_ref(q, k, v, sinks, 3, None)
    if not np.allclose(o, sdpa_reference(q, k, v, sinks, 3, 0.5), rtol=1e-11, atol=1e-12):
        return False
    return True


def test_unmutated_oracle_passes_core_pins():
    assert core_pins_pass()


MUTATIONS = {}


def mutation(fn):
    MUTATIONS[fn.__name__] = fn
    return fn


@mutation
def window_one_too_wide(mp):
    # W + 1 keys instead of W (j >= p - W); the sink-token rule is kept
    def vm(q_pos, k_pos, window, sink_tokens=0):
        p = np.asarray(q_pos, dtype=np.int64)[:, None]
        j = np.asarray(k_pos, dtype=np.int64)[None, :]
        vis = j <= p
        if window > 0:
            vis &= (j >= p - window) | (j < sink_tokens)
        return vis
    mp.setattr(OA, "visible_mask", vm)


@mutation
def not_causal(mp):
    # every key visible (no causal bound); the window and sink-token rules are kept
    def vm(q_pos, k_pos, window, sink_tokens=0):
        p = np.asarray(q_pos, dtype=np.int64)[:, None]
        j = np.asarray(k_pos, dtype=np.int64)[None, :]
        vis = np.ones(np.broadcast_shapes(p.shape, j.shape), dtype=bool)
        if window > 0:
            vis &= (j > p - window) | (j < sink_tokens)
        return vis
    mp.setattr(OA, "visible_mask", vm)


@mutation
def interleaved_head_map(mp):
    mp.setattr(OA, "kv_head", lambda h, hq, hkv: h % hkv)


_attend = OA.attend


@mutation
def sink_times_scale(mp):
    mp.setattr(OA, "attend", lambda q, k, v, qp, kp, s, w, sc, **kw: _attend(q, k, v, qp, kp, s * sc, w, sc, **kw))


@mutation
def sink_dropped(mp):
    mp.setattr(OA, "attend", lambda q, k, v, qp, kp, s, w, sc, **kw: _attend(q, k, v, qp, kp, -math.inf, w, sc, **kw))


@mutation
def sink_as_value_token(mp):
    # a sink that behaves like a token with v = 1 instead of a pure denominator term
    def att(q, k, v, qp, kp, s, w, sc, **kw):
        o, lse, *rest = _attend(q, k, v, qp, kp, s, w, sc, return_probs=True)
        p, sm = rest
        out = o + sm[:, None]
        return (out, lse, p, sm) if kw.get("return_probs") else (out, lse)
    mp.setattr(OA, "attend", att)


@mutation
def scale_not_applied(mp):
    mp.setattr(OA, "attend", lambda q, k, v, qp, kp, s, w, sc, **kw: _attend(q, k, v, qp, kp, s, w, 1.0, **kw))


@mutation
def keys_transposed_with_queries(mp):
    # use q as keys and k as queries (S^T instead of S); same shapes in the MHA case
    def att(q, k, v, qp, kp, s, w, sc, **kw):
        if q.shape == k.shape:
            return _attend(k, q, v, qp, kp, s, w, sc, **kw)
        return _attend(q, k, v, qp, kp, s, w, sc, **kw)
    mp.setattr(OA, "attend", att)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    assert not core_pins_pass(), f"mutation {name} slipped through the pins"
