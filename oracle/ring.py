"""Ring-buffer KV cache of sliding-window layers (test infrastructure only).

«GPT-OSS vs Qwen3», section "Utilisation de Sliding Window Attention": some
layers attend only to the most recent 128 tokens, so as to use less memory.
A windowed layer therefore never needs more than its last W positions; the
plainest store for them is a ring of W slots per sequence, position p in slot
p mod W (the slot rule is this reading; the pages name no layout).

Everything here is plain NumPy.  ``decode_ring_ref`` does not trust the ring
to hold the right positions: it recovers each slot's position from the slot
rule, keeps the positions the window allows, and calls the windowed
definition ``attention.attend`` with those positions.  ``prefill_ring_ref``
does the same for a chunk of new tokens, whose queries see the positions the
ring still holds plus the chunk's own rows; the chunk is appended afterwards
(``prefill_ring_append_ref``).
"""
from __future__ import annotations

import numpy as np

from .attention import _default_scale, attend, kv_head


def ring_slot(p: int, W: int) -> int:
    """Slot of position p in a ring of W slots."""
    return p % W


def ring_positions(L: int, W: int) -> np.ndarray:
    """Positions a ring of W slots holds after positions 0..L-1 were appended in order:
    the last min(L, W) of them."""
    return np.arange(max(0, L - W), L, dtype=np.int64)


def ring_append_ref(k_ring, v_ring, k_new, v_new, seqlens, W: int, cu_seqlens_q=None):
    """Rings after appending new rows (copies; inputs are not modified).

    k_ring/v_ring [B, W, Hkv, D]; k_new/v_new [T, Hkv, D].  Without cu_seqlens_q
    row b is the newest token of sequence b (position seqlens[b] - 1); with it,
    sequence b's rows are its newest q_len positions.  Rows are applied in
    position order, so of a chunk longer than W the newest rows remain.
    """
    k_ring = np.array(k_ring, copy=True)
    v_ring = np.array(v_ring, copy=True)
    B = k_ring.shape[0]
    for b in range(B):
        L = int(seqlens[b])
        if cu_seqlens_q is None:
            rows = [b]
        else:
            rows = list(range(int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])))
        q_len = len(rows)
        for t, r in enumerate(rows):
            p = L - q_len + t
            if p < 0:
                continue
            s = ring_slot(p, W)
            k_ring[b, s] = k_new[r]
            v_ring[b, s] = v_new[r]
    return k_ring, v_ring


def ring_from_history(k_full, v_full, seqlens, W: int):
    """Rings of W slots built by appending positions 0..L-1 of each sequence one at a time.

    k_full/v_full [B, Lmax, Hkv, D].  Slots never written stay zero.
    """
    B, _, Hkv, D = k_full.shape
    k_ring = np.zeros((B, W, Hkv, D), dtype=k_full.dtype)
    v_ring = np.zeros((B, W, Hkv, D), dtype=v_full.dtype)
    for b in range(B):
        for p in range(int(seqlens[b])):
            k_ring[b, ring_slot(p, W)] = k_full[b, p]
            v_ring[b, ring_slot(p, W)] = v_full[b, p]
    return k_ring, v_ring


def decode_ring_ref(q, k_ring, v_ring, seqlens, sinks, W: int, scale=None):
    """Decode on a windowed layer from its ring.

    q [B, Hq, D]; rings [B, W, Hkv, D]; seqlens[b] counts the new token (query at
    position seqlens[b] - 1).  The keys are the positions the ring holds, each
    read from its slot, under the window-W causal mask of the definition.
    Returns o [B, Hq, D], lse [B, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    k_ring = np.asarray(k_ring, dtype=np.float64)
    v_ring = np.asarray(v_ring, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_ring.shape[2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    o = np.zeros((B, Hq, v_ring.shape[3]))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(seqlens[b])
        pos = ring_positions(L, W)
        slots = pos % W
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            ob, lb = attend(q[b, h][None], k_ring[b, slots, g], v_ring[b, slots, g], [L - 1], pos,
                            sinks[h], W, scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def prefill_ring_ref(q, k_new, v_new, cu_seqlens_q, seqlens, k_ring, v_ring, sinks, W: int, scale=None):
    """Chunked prefill of a windowed layer over its ring: the chunk attends before it is appended.

    Sequence b owns query rows cu_seqlens_q[b]..cu_seqlens_q[b+1]-1 of q [T, Hq, D]
    and of its own key and value rows k_new/v_new [T, Hkv, D]: they are its newest
    q_len positions L0..L-1, with L = seqlens[b] counting the chunk and L0 = L - q_len.
    The rings [B, W, Hkv, D] still hold the positions before the chunk (the last
    min(L0, W) of 0..L0-1, each in its slot).  The keys of the chunk's queries are
    those ring positions, read from their slots, and the chunk's own positions,
    read from its rows, under the window-W causal mask of the definition («GPT-OSS
    vs Qwen3», "Utilisation de Sliding Window Attention": the last W tokens).  A
    query at position p >= L0 needs positions above p - W >= L0 - W, all of which
    the ring or the chunk holds, whatever the chunk's length.
    Returns o [T, Hq, D], lse [Hq, T] (the layout of varlen_ref).
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    k_ring = np.asarray(k_ring, dtype=np.float64)
    v_ring = np.asarray(v_ring, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k_ring.shape[2]
    scale = _default_scale(D, scale)
    sinks = np.full((Hq,), -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    o = np.zeros((T, Hq, v_ring.shape[3]))
    lse = np.zeros((Hq, T))
    for b in range(len(seqlens)):
        r0, r1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        if r1 == r0:
            continue
        L = int(seqlens[b])
        L0 = L - (r1 - r0)
        old = ring_positions(L0, W)                 # held by the ring
        slots = np.array([ring_slot(int(p), W) for p in old], dtype=np.int64)
        new = np.arange(L0, L, dtype=np.int64)      # the chunk's own rows
        k_pos = np.concatenate([old, new])
        q_pos = new
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            keys = np.concatenate([k_ring[b, slots, g], k_new[r0:r1, g]])
            vals = np.concatenate([v_ring[b, slots, g], v_new[r0:r1, g]])
            o[r0:r1, h], lse[h, r0:r1] = attend(q[r0:r1, h], keys, vals, q_pos, k_pos, sinks[h], W, scale)
    return o, lse


def prefill_ring_append_ref(q, k_new, v_new, cu_seqlens_q, seqlens, k_ring, v_ring, sinks, W: int, scale=None):
    """prefill_ring_ref, then the chunk appended to the rings (ring_append_ref).

    Returns o [T, Hq, D], lse [Hq, T] and the new rings (copies)."""
    o, lse = prefill_ring_ref(q, k_new, v_new, cu_seqlens_q, seqlens, k_ring, v_ring, sinks, W, scale)
    k2, v2 = ring_append_ref(k_ring, v_ring, k_new, v_new, seqlens, W, cu_seqlens_q=cu_seqlens_q)
    return o, lse, k2, v2
