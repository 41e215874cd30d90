"""Pins of the attention-gradient oracle (CPU).

The gradients are the derivative of the forward definition, so they are pinned
to the (already pinned) forward oracle by central finite differences, to torch
autograd through an independently written fp64 forward (the sink as an extra
zero-value column of the softmax), to torch's own SDPA backward where the sink
is absent, to a hand-derived closed form for a single visible key, and to
invariants of the softmax Jacobian.  Planted mistakes in the gradient formulas
(dropped Dp term, sink sign, transposed weights, dropped scale) are each caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as BW


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def loss(q, k, v, sinks, dout, window, scale, sink_tokens):
    o, _ = oracle.prefill_ref(q, k, v, sinks, window=window, scale=scale, sink_tokens=sink_tokens)
    return float((o * dout).sum())


def fd_max_error(q, k, v, sinks, dout, window, scale, sink_tokens, grads, eps=1e-6):
    """Largest |analytic - central difference| over every input element."""
    worst = 0.0
    args = {"q": q, "k": k, "v": v}
    if sinks is not None:
        args["s"] = sinks
    names = {"q": 0, "k": 1, "v": 2, "s": 3}
    for name, x in args.items():
        g = grads[names[name]]
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a = dict(q=q, k=k, v=v, s=sinks)
            a[name] = xp
            lp = loss(a["q"], a["k"], a["v"], a["s"], dout, window, scale, sink_tokens)
            a[name] = xm
            lm = loss(a["q"], a["k"], a["v"], a["s"], dout, window, scale, sink_tokens)
            worst = max(worst, abs((lp - lm) / (2 * eps) - g[idx]))
    return worst


TINY = [  # (window, sink_tokens, sinks kind)
    (0, 0, "normal"),
    (0, 0, "none"),
    (0, 0, "zero"),
    (2, 0, "normal"),
    (3, 1, "normal"),
    (1, 2, "none"),
]


@pytest.mark.parametrize("window,sink_tokens,kind", TINY)
def test_finite_differences(window, sink_tokens, kind):
    B, S, Hq, Hkv, D = 1, 6, 4, 2, 3
    q, k, v, dout = rnd(1, B, S, Hq, D), rnd(2, B, S, Hkv, D), rnd(3, B, S, Hkv, D), rnd(4, B, S, Hq, D)
    sinks = {"normal": rnd(5, Hq), "none": None, "zero": np.zeros(Hq)}[kind]
    scale = 0.7
    grads = BW.prefill_grad_ref(q, k, v, sinks, dout, window, scale, sink_tokens)
    err = fd_max_error(q, k, v, sinks, dout, window, scale, sink_tokens, grads)
    assert err < 1e-7, err
    if sinks is None:
        assert not grads[3].any()


def torch_forward(q, k, v, sinks, window, scale, sink_tokens):
    """fp64 forward written independently of the oracle: the sink is one extra
    column of logits with no value; visibility from explicit position grids."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=2)            # [B, S, Hq, D]
    vv = v.repeat_interleave(G, dim=2)
    x = scale * torch.einsum("bqhd,bkhd->bhqk", q, kk)
    p = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    vis = j <= p
    if window > 0:
        vis = vis & ((j > p - window) | (j < sink_tokens))
    x = x.masked_fill(~vis, float("-inf"))
    col = sinks.view(1, Hq, 1, 1).expand(B, Hq, S, 1)
    w = torch.softmax(torch.cat([x, col], dim=-1), dim=-1)[..., :S]
    return torch.einsum("bhqk,bkhd->bqhd", w, vv)


@pytest.mark.parametrize("window,sink_tokens,with_sink", [(0, 0, True), (5, 0, True), (5, 3, True), (40, 0, True),
                                                          (0, 0, False), (7, 2, False)])
def test_autograd_of_independent_forward(window, sink_tokens, with_sink):
    B, S, Hq, Hkv, D = 2, 37, 8, 2, 16
    q, k, v, dout = rnd(11, B, S, Hq, D), rnd(12, B, S, Hkv, D), rnd(13, B, S, Hkv, D), rnd(14, B, S, Hq, D)
    s = rnd(15, Hq) if with_sink else np.full(Hq, -np.inf)
    scale = 1 / 4
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    ts = torch.tensor(s, requires_grad=with_sink)
    out = torch_forward(tq, tk, tv, ts, window, scale, sink_tokens)
    out.backward(torch.tensor(dout))
    dq, dk, dv, ds = BW.prefill_grad_ref(q, k, v, s if with_sink else None, dout, window, scale, sink_tokens)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    if with_sink:
        np.testing.assert_allclose(ds, ts.grad.numpy(), rtol=0, atol=1e-12)


def test_no_sink_matches_sdpa_backward():
    B, S, Hq, Hkv, D = 1, 50, 6, 3, 8
    q, k, v, dout = rnd(21, B, S, Hq, D), rnd(22, B, S, Hkv, D), rnd(23, B, S, Hkv, D), rnd(24, B, S, Hq, D)
    G = Hq // Hkv
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    kk = tk.repeat_interleave(G, dim=2).transpose(1, 2)
    vv = tv.repeat_interleave(G, dim=2).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(1, 2), kk, vv, is_causal=True)
    o.transpose(1, 2).backward(torch.tensor(dout))
    dq, dk, dv, ds = BW.prefill_grad_ref(q, k, v, None, dout, 0, None, 0)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)
    assert not ds.any()


def test_single_visible_key_closed_form():
    # position 0 sees only itself: P = logistic(x - s); L = P <dO, v>
    q, k, v, dO = np.array([0.5, -1.0]), np.array([2.0, 0.25]), np.array([1.5, -0.5]), np.array([0.3, 0.8])
    s, scale = 0.4, 0.5
    x = scale * q @ k                                      # 0.375
    P = 1 / (1 + math.exp(s - x))
    c = P * (1 - P) * (dO @ v)                             # dL/dx
    dq, dk, dv, ds = BW.prefill_grad_ref(q[None, None, None], k[None, None, None], v[None, None, None],
                                         [s], dO[None, None, None], 0, scale, 0)
    np.testing.assert_allclose(dq[0, 0, 0], scale * c * k, rtol=1e-14)
    np.testing.assert_allclose(dk[0, 0, 0], scale * c * q, rtol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 0], P * dO, rtol=1e-14)
    np.testing.assert_allclose(ds, [-c], rtol=1e-14)


@pytest.mark.parametrize("window,sink_tokens", [(0, 0), (4, 2)])
def test_softmax_jacobian_invariants(window, sink_tokens):
    n = 20
    q, k, v, dO = rnd(31, n, 8), rnd(32, n, 8), rnd(33, n, 5), rnd(34, n, 5)
    pos = np.arange(n)
    dq, dk, dv, ds, dx, ds_rows = BW.row_grads(q, k, v, pos, pos, 0.3, dO, window, 0.35, sink_tokens)
    # logit gradients plus the sink's sum to zero in every row
    np.testing.assert_allclose(dx.sum(axis=1) + ds_rows, 0.0, atol=1e-13)
    # value gradients sum to the non-sink mass times dO
    _, _, P, P_s = oracle.attend(q, k, v, pos, pos, 0.3, window, 0.35, return_probs=True, sink_tokens=sink_tokens)
    np.testing.assert_allclose(dv.sum(axis=0), ((1 - P_s)[:, None] * dO).sum(axis=0), atol=1e-12)
    # invisible pairs get no gradient
    vis = oracle.visible_mask(pos, pos, window, sink_tokens)
    assert not dx[~vis].any()


def test_gqa_is_mha_summed_over_the_group():
    B, S, Hq, Hkv, D = 1, 24, 8, 2, 4
    q, k, v, dout = rnd(41, B, S, Hq, D), rnd(42, B, S, Hkv, D), rnd(43, B, S, Hkv, D), rnd(44, B, S, Hq, D)
    sinks = rnd(45, Hq)
    g_gqa = BW.prefill_grad_ref(q, k, v, sinks, dout, 6, None, 1)
    G = Hq // Hkv
    g_mha = BW.prefill_grad_ref(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), sinks, dout, 6, None, 1)
    np.testing.assert_array_equal(g_gqa[0], g_mha[0])
    np.testing.assert_allclose(g_gqa[1], g_mha[1].reshape(B, S, Hkv, G, D).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(g_gqa[2], g_mha[2].reshape(B, S, Hkv, G, D).sum(axis=3), atol=1e-13)
    np.testing.assert_array_equal(g_gqa[3], g_mha[3])


def test_dout_dot_out_is_the_row_sum_of_p_dp():
    B, S, Hq, Hkv, D = 1, 16, 4, 2, 8
    q, k, v, dout = rnd(51, B, S, Hq, D), rnd(52, B, S, Hkv, D), rnd(53, B, S, Hkv, D), rnd(54, B, S, Hq, D)
    sinks = rnd(55, Hq)
    o, _ = oracle.prefill_ref(q, k, v, sinks, 0, None)
    Dm = BW.dout_dot_out(o, dout)
    P, _ = oracle.probabilities(q, k, v, sinks, 0, None)
    for h in range(Hq):
        dP = dout[0, :, h] @ v[0, :, h // 2].T
        np.testing.assert_allclose(Dm[0, h], (P[0, h] * dP).sum(axis=1), atol=1e-13)


def _planted(kind):
    def wrong(q, k, v, q_pos, k_pos, sink, dout, window, scale, sink_tokens=0):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        dout = np.asarray(dout, dtype=np.float64)
        o, _, P, P_s = oracle.attend(q, k, v, q_pos, k_pos, sink, window, scale, return_probs=True,
                                     sink_tokens=sink_tokens)
        dP = dout @ v.T
        Dp = (dout * o).sum(axis=1)
        dx = P * dP if kind == "no_Dp" else P * (dP - Dp[:, None])
        ds_rows = P_s * Dp if kind == "sink_sign" else -P_s * Dp
        sc = 1.0 if kind == "no_scale" else scale
        dq, dk = sc * (dx @ k), scale * (dx.T @ q)
        dv = P @ dout if kind == "transposed_P" else P.T @ dout
        return dq, dk, dv, float(ds_rows.sum()), dx, ds_rows
    return wrong


@pytest.mark.parametrize("kind", ["no_Dp", "sink_sign", "transposed_P", "no_scale"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 3
    q, k, v, dout = rnd(61, B, S, Hq, D), rnd(62, B, S, Hkv, D), rnd(63, B, S, Hkv, D), rnd(64, B, S, Hq, D)
    sinks = rnd(65, Hq)
    monkeypatch.setattr(BW, "row_grads", _planted(kind))
    grads = BW.prefill_grad_ref(q, k, v, sinks, dout, 0, 0.6, 0)
    assert fd_max_error(q, k, v, sinks, dout, 0, 0.6, 0, grads) > 1e-3


def test_kv_head_subset_is_a_restriction():
    B, S, Hq, Hkv, D = 1, 12, 8, 4, 4
    q, k, v, dout = rnd(71, B, S, Hq, D), rnd(72, B, S, Hkv, D), rnd(73, B, S, Hkv, D), rnd(74, B, S, Hq, D)
    sinks = rnd(75, Hq)
    full = BW.prefill_grad_ref(q, k, v, sinks, dout, 5, None, 2)
    part = BW.prefill_grad_ref(q, k, v, sinks, dout, 5, None, 2, kv_heads=[1, 3])
    heads = [2, 3, 6, 7]
    np.testing.assert_array_equal(part[0][:, :, heads], full[0][:, :, heads])
    np.testing.assert_array_equal(part[1][:, :, [1, 3]], full[1][:, :, [1, 3]])
    np.testing.assert_array_equal(part[2][:, :, [1, 3]], full[2][:, :, [1, 3]])
    np.testing.assert_array_equal(part[3][heads], full[3][heads])
    assert not part[0][:, :, [0, 1, 4, 5]].any() and not part[1][:, :, [0, 2]].any()


def test_dsink_abs_is_the_sum_of_term_magnitudes():
    B, S, Hq, Hkv, D = 1, 9, 4, 2, 4
    q, k, v, dout = rnd(81, B, S, Hq, D), rnd(82, B, S, Hkv, D), rnd(83, B, S, Hkv, D), rnd(84, B, S, Hq, D)
    sinks = rnd(85, Hq)
    *_, ds, ds_abs = BW.prefill_grad_ref(q, k, v, sinks, dout, 0, None, 0, dsink_abs=True)
    assert (ds_abs >= np.abs(ds) - 1e-15).all()
    for h in range(Hq):
        _, _, _, _, _, rows = BW.row_grads(q[0, :, h], k[0, :, h // 2], v[0, :, h // 2], np.arange(S), np.arange(S),
                                           sinks[h], dout[0, :, h], 0, 1 / 2, 0)
        np.testing.assert_allclose(ds_abs[h], np.abs(rows).sum(), rtol=1e-14)
    *_, ds1, abs1 = BW.prefill_grad_ref(q[:, :1], k[:, :1], v[:, :1], sinks, dout[:, :1], 0, None, 0, dsink_abs=True)
    np.testing.assert_allclose(abs1, np.abs(ds1), rtol=1e-14)   # one row: one term per head
