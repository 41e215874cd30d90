"""Pure-Python scalar enumeration of the same attention definition (test infrastructure only).

Written independently of ``oracle.attention``: plain nested lists, ``math.exp``
and ``math.fsum``, the visible keys enumerated as the integer range of the
"last W tokens up to and including the query" («GPT-OSS vs Qwen3»,
"Utilisation de Sliding Window Attention") with the first sink_tokens
positions prepended when asked (the start-of-sequence sink tokens of «GPT-OSS
vs Qwen3», "Attention Bias et Sinks"), and the softmax taken over the
list formed by the sink logit («GPT-OSS vs Qwen3», "Attention Bias et Sinks")
followed by the visible scaled logits.  Only for tiny inputs.
"""
from __future__ import annotations

import math


def _visible_keys(p: int, window: int, sink_tokens: int = 0):
    lo = 0 if window <= 0 else max(0, p - window + 1)
    # the first sink_tokens positions join the window (at most up to the query itself)
    head = [j for j in range(min(sink_tokens, lo, p + 1))]
    return head + list(range(lo, p + 1))


def brute_row(qv, keys, vals, p: int, sink: float, window: int, scale: float, sink_tokens: int = 0):
    """One query vector qv at position p against keys[j], vals[j] (lists of floats).

    Returns (o list, lse float, weights dict j -> prob, sink_prob).
    """
    js = [j for j in _visible_keys(p, window, sink_tokens) if j < len(keys)]
    logits = [sink] + [scale * math.fsum(a * b for a, b in zip(qv, keys[j])) for j in js]
    top = max(logits)
    if top == -math.inf:
        return [0.0] * len(vals[0] if vals else qv), -math.inf, {}, 0.0
    w = [math.exp(x - top) for x in logits]
    z = math.fsum(w)
    probs = [x / z for x in w]
    dv = len(vals[0]) if vals else len(qv)
    o = [math.fsum(probs[1 + i] * vals[j][d] for i, j in enumerate(js)) for d in range(dv)]
    return o, top + math.log(z), {j: probs[1 + i] for i, j in enumerate(js)}, probs[0]


def brute_prefill(q, k, v, sinks, window: int, scale: float, sink_tokens: int = 0):
    """q: nested list [B][S][Hq][D]; k, v: [B][S][Hkv][D]; sinks: [Hq] floats.

    Returns o [B][S][Hq][D] and lse [B][Hq][S] as nested lists.
    """
    B, S, Hq = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0][0])
    group = Hq // Hkv
    o = [[[None] * Hq for _ in range(S)] for _ in range(B)]
    lse = [[[None] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            keys = [k[b][j][g] for j in range(S)]
            vals = [v[b][j][g] for j in range(S)]
            for t in range(S):
                o[b][t][h], lse[b][h][t], _, _ = brute_row(q[b][t][h], keys, vals, t, sinks[h], window, scale,
                                                           sink_tokens)
    return o, lse
