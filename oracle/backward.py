"""Gradients of sink + window causal GQA attention (test infrastructure only).

The pages describe how the model is trained («GPT-OSS-20B : Architecture MoE &
Résumé du Model Card», §5 "Entraînement": next-token prediction; «GPT-OSS vs
Qwen3», "Entraînement et optimisation": pre-training, supervised fine-tuning,
RL) but print no backward pass.  Training needs the derivative of the forward
definition in ``oracle.attention``, which is what this module writes out, by
the chain rule, with no blocking or reordering.

For one sequence, query head h (KV head g = h // G) and the query at position p
with visible set J, the forward gives the weights

    P_j = exp(x_j - lse),   P_s = exp(s_h - lse)      (P_s: the sink's share)
    o   = sum_{j in J} P_j v_j,                 x_j = scale * <q, k_j>

Given the upstream gradient dO = dL/do of that row:

    dP_j   = <dO, v_j>                     (dL/dP_j; the sink has no value, dP_s = 0)
    Dp     = sum_{j in J} P_j dP_j = <dO, o>
    dx_j   = P_j (dP_j - Dp)               (softmax Jacobian, the sink a column of it)
    ds     = P_s (0 - Dp) = -P_s Dp        (gradient of the sink logit from this row)
    dq    += scale * sum_j dx_j k_j
    dk_j  += scale * dx_j q                (summed over every row and query head of g)
    dv_j  += P_j dO                        (likewise)
    dsinks[h] = sum over rows and sequences of ds

Pins: ``tests/test_oracle_backward_pins.py`` (central finite differences of the
forward oracle, autograd of an independently written forward, closed forms,
invariants, planted mistakes).
"""
from __future__ import annotations

import numpy as np

from .attention import _default_scale, attend, kv_head


def row_grads(q, k, v, q_pos, k_pos, sink: float, dout, window: int, scale: float, sink_tokens: int = 0):
    """Gradients of single-head attention for rows q [n, D] against keys k [L, D], v [L, Dv].

    Returns (dq [n, D], dk [L, D], dv [L, Dv], dsink scalar, dx [n, L], dsink_rows [n]):
    dx are the gradients of the logits x (zero off the visible set), dsink_rows
    the per-row gradients of the sink logit.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    o, _, P, P_s = attend(q, k, v, q_pos, k_pos, sink, window, scale, return_probs=True, sink_tokens=sink_tokens)
    dP = dout @ v.T                                # [n, L]
    Dp = (dout * o).sum(axis=1)                    # [n]
    dx = P * (dP - Dp[:, None])                    # zero where P is zero (masked)
    ds_rows = -P_s * Dp
    dq = scale * (dx @ k)
    dk = scale * (dx.T @ q)
    dv = P.T @ dout
    return dq, dk, dv, float(ds_rows.sum()), dx, ds_rows


def prefill_grad_ref(q, k, v, sinks, dout, window: int = 0, scale=None, sink_tokens: int = 0, kv_heads=None,
                     dsink_abs: bool = False):
    """Gradients of the prefill (self-attention of whole sequences).

    q, dout: [B, S, Hq, D]; k, v: [B, S, Hkv, D]; sinks: [Hq] or None (no sink).
    Returns dq [B, S, Hq, D], dk [B, S, Hkv, D], dv [B, S, Hkv, D], dsinks [Hq]
    (zeros when sinks is None), all fp64.  kv_heads (optional): compute only the
    query heads of these KV heads (the rest of every output stays zero).
    dsink_abs: also return, per head, the sum over rows of |ds| (the magnitude
    of the terms that dsinks adds up, a scale for comparing it).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = _default_scale(D, scale)
    has_sink = sinks is not None
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.zeros((Hq,))
    ds_abs = np.zeros((Hq,))
    pos = np.arange(S)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            if kv_heads is not None and g not in kv_heads:
                continue
            gq, gk, gv, gs, _, ds_rows = row_grads(q[b, :, h], k[b, :, g], v[b, :, g], pos, pos, sinks[h],
                                                   dout[b, :, h], window, scale, sink_tokens)
            dq[b, :, h] = gq
            dk[b, :, g] += gk
            dv[b, :, g] += gv
            dsinks[h] += gs
            ds_abs[h] += np.abs(ds_rows).sum()
    if not has_sink:
        dsinks[:] = 0.0
        ds_abs[:] = 0.0
    if dsink_abs:
        return dq, dk, dv, dsinks, ds_abs
    return dq, dk, dv, dsinks


def dout_dot_out(o, dout):
    """D = <dO, o> per row and head: [B, Hq, S] from o, dout [B, S, Hq, D]."""
    return np.einsum("bshd,bshd->bhs", np.asarray(dout, dtype=np.float64), np.asarray(o, dtype=np.float64))
