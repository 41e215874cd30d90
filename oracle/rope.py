"""Rotary position encoding of new tokens and their KV-cache append (test infrastructure only).

«GPT-OSS-20B : Architecture MoE & Résumé du Model Card», §3.4 "Encodage de
Position (RoPE)": m is the token position and θ_i = 10000^(-2i/d); the rotation
formula itself did not survive on the page.  «OpenAI lance gpt-oss-20b, qui
tient sur 16 Go», "gpt-oss remplace plusieurs composants", and «GPT-OSS vs
Qwen3», "Adoption de RoPE": RoPE turns the query and key vectors by an angle
that depends on the token's position.

Readings (the plainest consistent with those lines):

* pair i of a head is rotated by the angle m·θ_i, counter-clockwise:
  (a, b) -> (a cos - b sin, a sin + b cos);
* the pairs are (2i, 2i+1) ("interleaved", the default) or (i, i + d/2)
  ("halves"); the pages do not say which, so both are offered;
* the frequency table is an input, θ_i by default; the page's YaRN line
  (131 072 tokens, "24×") gives too little to define YaRN's blend of
  frequencies, so a caller who wants it passes its own table, and an optional
  factor scales cos and sin alike.

Angles are formed in fp64 from the fp32 table the kernels receive (position
times an fp32 frequency is exact in fp64).
"""
from __future__ import annotations

import numpy as np

PAIR_INTERLEAVED = 0
PAIR_HALVES = 1


def default_inv_freq(d: int, base: float = 10000.0) -> np.ndarray:
    """θ_i = base^(-2i/d), i = 0 .. d/2 - 1, rounded to fp32 (the table the kernels take)."""
    i = np.arange(d // 2, dtype=np.float64)
    return (base ** (-2.0 * i / d)).astype(np.float32)


def pair_index(d: int, pairing: int):
    """(first, second) coordinate of every pair i."""
    i = np.arange(d // 2)
    if pairing == PAIR_INTERLEAVED:
        return 2 * i, 2 * i + 1
    if pairing == PAIR_HALVES:
        return i, i + d // 2
    raise ValueError(pairing)


def rope_ref(x, pos, inv_freq, pairing: int = PAIR_INTERLEAVED, mscale: float = 1.0):
    """Rotate x [..., n, H, d] whose leading rows sit at positions pos [n].

    Returns fp64 [..., n, H, d].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a_idx, b_idx = pair_index(d, pairing)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * np.asarray(inv_freq, dtype=np.float32).astype(np.float64)[None, :]
    c = (np.cos(ang) * mscale)[:, None, :]   # [n, 1, d/2]
    s = (np.sin(ang) * mscale)[:, None, :]
    a = x[..., a_idx]
    b = x[..., b_idx]
    out = np.empty_like(x)
    out[..., a_idx] = a * c - b * s
    out[..., b_idx] = a * s + b * c
    return out


def new_positions(seqlens, cu_seqlens_q=None):
    """Positions of the new rows: row b at seqlens[b]-1 (one per sequence), or the newest
    q_len positions of each sequence (chunks by cu_seqlens_q).  Returns (seq [T], pos [T])."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    if cu_seqlens_q is None:
        return np.arange(len(seqlens)), seqlens - 1
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    seq, pos = [], []
    for b in range(len(seqlens)):
        n = int(cu[b + 1] - cu[b])
        for t in range(n):
            seq.append(b)
            pos.append(int(seqlens[b]) - n + t)
    return np.array(seq, dtype=np.int64), np.array(pos, dtype=np.int64)


CACHE_CONTIGUOUS = 0
CACHE_PAGED = 1
CACHE_RING = 2


def rope_append_ref(q, k, v, seqlens, inv_freq, k_cache, v_cache, kind: int, cache_len: int = 0,
                    cu_seqlens_q=None, block_table=None, block_size: int = 16, pairing: int = PAIR_INTERLEAVED,
                    mscale: float = 1.0):
    """Rotated queries and the caches after the append (copies; fp64 values).

    q [T, Hq, d], k/v [T, Hkv, d] are the new rows.  Caches: contiguous
    [B, cache_len, Hkv, d] (position p of sequence b in row p; p >= cache_len is
    not stored), paged [Nblk, bs, Hkv, d] (block_table[b][p // bs], slot p % bs),
    or a ring of cache_len slots [B, W, Hkv, d] (slot p % W, last W positions).
    Rows with a negative position are not stored.
    """
    seq, pos = new_positions(seqlens, cu_seqlens_q)
    q_rot = rope_ref(q, pos, inv_freq, pairing, mscale)
    k_rot = rope_ref(k, pos, inv_freq, pairing, mscale)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    v = np.asarray(v, dtype=np.float64)
    L = np.asarray(seqlens, dtype=np.int64)
    for r in range(len(pos)):
        b, p = int(seq[r]), int(pos[r])
        if p < 0:
            continue
        if kind == CACHE_CONTIGUOUS:
            if p >= cache_len:
                continue
            kc[b, p], vc[b, p] = k_rot[r], v[r]
        elif kind == CACHE_PAGED:
            blk = int(block_table[b][p // block_size])
            kc[blk, p % block_size], vc[blk, p % block_size] = k_rot[r], v[r]
        elif kind == CACHE_RING:
            if p < int(L[b]) - cache_len:
                continue
            kc[b, p % cache_len], vc[b, p % cache_len] = k_rot[r], v[r]
        else:
            raise ValueError(kind)
    return q_rot, kc, vc
