"""fp64 NumPy definition of sink + window causal GQA attention (test infrastructure only).

The definition, for one sequence, query head h and a query at position p:

    G   = Hq / Hkv,  g = h // G                       (grouped KV heads)
    J   = { j : j <= p  and  (W <= 0  or  j > p - W  or  j < n) }
                                                       (causal, last W keys, plus the
                                                        first n "sink tokens" when asked)
    x_j = scale * <q, k_j[g]>                          (scaled dot product)
    s   = sinks[h]                                     (learned sink logit)
    m   = max(s, max_{j in J} x_j)
    Z   = exp(s - m) + sum_{j in J} exp(x_j - m)
    o   = sum_{j in J} exp(x_j - m) / Z * v_j[g]
    lse = m + ln Z

The sink enters the denominator only (it has no value vector), which is how
the "Attention Bias et Sinks" section of «GPT-OSS vs Qwen3» describes it: a
learned bias logit per head that does not change the input tokens.  With
s = 0 this is off-by-one attention, cited in the "Pour aller plus loin" list
of «gpt-oss Deep Dive with Xiaoli Alex Shen»; with s = -inf it is ordinary
softmax attention.  The 64-query / 8-KV head grouping is §3.3 of «GPT-OSS-20B :
Architecture MoE & Résumé du Model Card»; the 128-token window is the "Utilisation
de Sliding Window Attention" section of «GPT-OSS vs Qwen3».  The matrix product
and exp are library primitives; there is no blocking, fusion or reordering.
"""
from __future__ import annotations

import math

import numpy as np


def kv_head(h: int, hq: int, hkv: int) -> int:
    """KV head used by query head h: contiguous groups of G = hq/hkv query heads.

    «GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §3.3: each KV head
    is shared by 8 query heads.  Which 8 is not printed; the contiguous grouping
    h // G is the reading taken.
    """
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def visible_mask(q_pos: np.ndarray, k_pos: np.ndarray, window: int, sink_tokens: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k]: key position j is visible from query position p.

    Causal (decoder-only, autoregressive: «OpenAI lance gpt-oss-20b, qui tient
    sur 16 Go», opening section): j <= p.  Sliding window («GPT-OSS vs Qwen3»,
    "Utilisation de Sliding Window Attention"): only the last W tokens,
    read as j > p - W, i.e. exactly W keys counting the query's own position.
    W <= 0 means dense.  Sink tokens («GPT-OSS vs Qwen3», "Attention Bias et
    Sinks": the classical sink is a token at the start of the sequence that is
    always attended): the first ``sink_tokens`` positions stay visible past the
    window edge (still causal).
    """
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(k_pos, dtype=np.int64)[None, :]
    vis = j <= p
    if window > 0:
        vis &= (j > p - window) | (j < sink_tokens)
    return vis


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos, k_pos, sink: float,
           window: int, scale: float, return_probs: bool = False, sink_tokens: int = 0):
    """Single-head attention of query rows against a set of keys.

    q: [n, D], k: [L, D], v: [L, Dv] (fp64), q_pos: [n], k_pos: [L].
    Returns (o [n, Dv], lse [n]) and, if asked, (p [n, L], sink_mass [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, L = q.shape[0], k.shape[0]
    s = float(sink)
    vis = visible_mask(q_pos, k_pos, window, sink_tokens)
    x = scale * (q @ k.T) if L else np.zeros((n, 0))
    xm = np.where(vis, x, -np.inf)
    row_max = xm.max(axis=1) if L else np.full((n,), -np.inf)
    m = np.maximum(row_max, s)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(vis, np.exp(xm - m_safe[:, None]), 0.0)
    e_sink = np.exp(s - m_safe)
    Z = e_sink + e.sum(axis=1)
    o = np.zeros((n, v.shape[1]))
    # rows with m = +-inf: nothing visible and no sink (o = 0, lse = s = -inf), or
    # an infinite sink that takes all the mass (o = 0, lse = s = +inf)
    lse = np.full((n,), s)
    ok = finite
    o[ok] = (e[ok] @ v) / Z[ok, None]
    lse[ok] = m[ok] + np.log(Z[ok])
    if np.isnan(s):
        o[:] = np.nan
        lse[:] = np.nan
    if return_probs:
        p = np.zeros_like(e)
        p[ok] = e[ok] / Z[ok, None]
        sink_mass = np.zeros((n,))
        sink_mass[ok] = e_sink[ok] / Z[ok]
        return o, lse, p, sink_mass
    return o, lse


def _default_scale(D: int, scale) -> float:
    return 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)


def prefill_rows_ref(q, k, v, sinks, window: int = 0, scale=None, rows=None, heads=None, sink_tokens: int = 0):
    """Prefill (self-attention of a whole sequence), optionally on a subset of query rows.

    q: [B, S, Hq, D], k/v: [B, S, Hkv, D], sinks: [Hq] (or None = no sink).
    rows: positions to compute (default all).  Returns o [B, len(rows), Hq, D]
    and lse [B, Hq, len(rows)] (heads outside ``heads`` are left at zero).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    o = np.zeros((B, len(rows), Hq, v.shape[3]))
    lse = np.zeros((B, Hq, len(rows)))
    k_pos = np.arange(S)
    for b in range(B):
        for h in heads:
            g = kv_head(h, Hq, Hkv)
            o[b, :, h], lse[b, h] = attend(q[b, rows, h], k[b, :, g], v[b, :, g], rows, k_pos,
                                           sinks[h], window, scale, sink_tokens=sink_tokens)
    return o, lse


def prefill_ref(q, k, v, sinks, window: int = 0, scale=None, sink_tokens: int = 0):
    """Full prefill: o [B, S, Hq, D], lse [B, Hq, S]."""
    return prefill_rows_ref(q, k, v, sinks, window, scale, sink_tokens=sink_tokens)


def decode_ref(q, k_cache, v_cache, seqlens, sinks, window: int = 0, scale=None, sink_tokens: int = 0):
    """One new query token per sequence against a contiguous KV cache.

    q: [B, Hq, D]; caches [B, Lmax, Hkv, D]; seqlens[b] counts the cached
    positions including the new token, so the query sits at position
    seqlens[b] - 1 and sees positions 0..seqlens[b]-1 (within the window).
    Returns o [B, Hq, D], lse [B, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    o = np.zeros((B, Hq, v_cache.shape[3]))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seqlens[b])
        k_pos = np.arange(L)
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            ob, lb = attend(q[b, h][None], k_cache[b, :L, g], v_cache[b, :L, g], [L - 1], k_pos,
                            sinks[h], window, scale, sink_tokens=sink_tokens)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def gather_paged(cache, block_table_row, block_size: int, L: int):
    """Rows 0..L-1 of one sequence from a paged cache [Nblk, bs, Hkv, D].

    Position p lives in physical block block_table_row[p // bs], slot p % bs.
    """
    cache = np.asarray(cache)
    pos = np.arange(L)
    blocks = np.asarray(block_table_row, dtype=np.int64)[pos // block_size]
    return cache[blocks, pos % block_size]


def varlen_ref(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, sinks, window: int = 0, scale=None,
               block_table=None, block_size: int = 16, cu_seqlens_k=None, rows=None, sink_tokens: int = 0):
    """Packed variable-length queries against a paged (or packed) KV cache.

    q: [Tq, Hq, D].  Sequence b owns query rows cu_seqlens_q[b]..cu_seqlens_q[b+1]-1
    and KV positions 0..seqlens_k[b]-1.  Its q_len queries are the newest
    positions: query t sits at seqlens_k[b] - q_len + t.  With block_table the
    caches are [Nblk, bs, Hkv, D]; without it they are packed [Tk, Hkv, D] and
    sequence b's positions start at row cu_seqlens_k[b].
    rows (optional): global query row indices to compute; other rows stay zero.
    Returns o [Tq, Hq, D], lse [Hq, Tq].
    """
    q = np.asarray(q, dtype=np.float64)
    Tq, Hq, D = q.shape
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    Hkv = kc.shape[-2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    o = np.zeros((Tq, Hq, vc.shape[-1]))
    lse = np.zeros((Hq, Tq))
    want = None if rows is None else set(int(r) for r in rows)
    B = len(seqlens_k)
    for b in range(B):
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        L = int(seqlens_k[b])
        qlen = r1 - r0
        sel = [r for r in range(r0, r1) if want is None or r in want]
        if not sel:
            continue
        if block_table is not None:
            kb = gather_paged(kc, block_table[b], block_size, L)
            vb = gather_paged(vc, block_table[b], block_size, L)
        else:
            c0 = int(cu_seqlens_k[b])
            kb, vb = kc[c0:c0 + L], vc[c0:c0 + L]
        q_pos = np.array([L - qlen + (r - r0) for r in sel])
        k_pos = np.arange(L)
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            ob, lb = attend(q[sel, h], kb[:, g], vb[:, g], q_pos, k_pos, sinks[h], window, scale,
                            sink_tokens=sink_tokens)
            o[sel, h] = ob
            lse[h, sel] = lb
    return o, lse


def probabilities(q, k, v, sinks, window: int = 0, scale=None, sink_tokens: int = 0):
    """Attention weights of a prefill: p [B, Hq, S, S] (zero off the visible set) and
    sink_mass [B, Hq, S]; p summed over keys plus sink_mass is one in every row."""
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    P = np.zeros((B, Hq, S, S))
    SM = np.zeros((B, Hq, S))
    pos = np.arange(S)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            _, _, P[b, h], SM[b, h] = attend(q[b, :, h], np.asarray(k, dtype=np.float64)[b, :, g],
                                             np.asarray(v, dtype=np.float64)[b, :, g], pos, pos,
                                             sinks[h], window, scale, return_probs=True,
                                             sink_tokens=sink_tokens)
    return P, SM
