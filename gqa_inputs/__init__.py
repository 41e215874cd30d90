"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and lays them out.  It holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method's code.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([cfg,
tensor_id]))`` with tensor ids q=0, k=1, v=2, sinks=3, lengths=4, block
permutation=5.  Floating-point tensors are drawn in fp32; tensors that the
GPU path consumes in bf16 are rounded to bf16 on the CPU (round to nearest,
ties to even) and handed out as raw 16-bit patterns, so that the GPU and the
oracle see the very same bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

T_Q, T_K, T_V, T_SINK, T_LEN, T_PERM, T_DOUT = range(7)


def rng_for(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(tensor_id)]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even (finite inputs).

    Works in place-sized uint32 chunks so that gigabyte tensors convert without
    large temporaries (finite values never carry past bit 31)."""
    u = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, u.size, step):
        c = u[i:i + step]
        r = c + (((c >> 16) & 1) + np.uint32(0x7FFF))
        out[i:i + step] = (r >> 16).astype(np.uint16)
    return out.reshape(np.shape(x))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def normal(cfg: int, tensor_id: int, shape, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) draw."""
    x = rng_for(cfg, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return x


@dataclass
class Tensor:
    """One synthetic input: fp64 values for the oracle, device-ready storage for the GPU.

    ``store`` is uint16 bf16 bits when ``dtype == 'bf16'`` and float32 otherwise;
    ``f64`` is its exact value in float64.
    """

    store: np.ndarray
    dtype: str

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_to_f64(self.store)
        return self.store.astype(np.float64)

    @property
    def shape(self):
        return self.store.shape


def make_tensor(cfg: int, tensor_id: int, shape, std: float, dtype: str) -> Tensor:
    x = normal(cfg, tensor_id, shape, std)
    if dtype == "bf16":
        return Tensor(bf16_bits(x), "bf16")
    if dtype == "fp32":
        return Tensor(x, "fp32")
    raise ValueError(dtype)


def make_sinks(cfg: int, hq: int, kind: str = "normal") -> np.ndarray:
    """Per-query-head sink logits, fp32 ``[hq]``.

    kind: 'normal' (N(0,1)), 'none' (all -inf, i.e. no sink), 'zero'.
    """
    if kind == "normal":
        return normal(cfg, T_SINK, (hq,))
    if kind == "none":
        return np.full((hq,), -np.inf, dtype=np.float32)
    if kind == "zero":
        return np.zeros((hq,), dtype=np.float32)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# prefill / decode / ragged-paged problems


@dataclass
class Prefill:
    q: Tensor  # [B, S, Hq, D]
    k: Tensor  # [B, S, Hkv, D]
    v: Tensor  # [B, S, Hkv, D]
    sinks: np.ndarray  # [Hq] fp32
    scale: float

    @property
    def dims(self):
        B, S, Hq, D = self.q.shape
        return B, S, Hq, self.k.shape[2], D


def prefill_problem(cfg: int, B: int, S: int, Hq: int, Hkv: int, D: int = 64, dtype: str = "bf16",
                    std: float = 1.0, sink_kind: str = "normal", scale: float | None = None) -> Prefill:
    return Prefill(
        q=make_tensor(cfg, T_Q, (B, S, Hq, D), std, dtype),
        k=make_tensor(cfg, T_K, (B, S, Hkv, D), std, dtype),
        v=make_tensor(cfg, T_V, (B, S, Hkv, D), std, dtype),
        sinks=make_sinks(cfg, Hq, sink_kind),
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
    )


@dataclass
class Decode:
    q: Tensor  # [B, Hq, D]
    k: Tensor  # [B, Lmax, Hkv, D]
    v: Tensor  # [B, Lmax, Hkv, D]
    seqlens: np.ndarray  # [B] int32, cache length including the new token
    sinks: np.ndarray
    scale: float


def decode_problem(cfg: int, B: int, Lmax: int, Hq: int, Hkv: int, D: int = 64, dtype: str = "bf16",
                   std: float = 1.0, sink_kind: str = "normal", seqlens=None,
                   scale: float | None = None) -> Decode:
    if seqlens is None:
        seqlens = np.full((B,), Lmax, dtype=np.int32)
    elif isinstance(seqlens, str) and seqlens == "random":
        seqlens = rng_for(cfg, T_LEN).integers(1, Lmax + 1, size=B).astype(np.int32)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    return Decode(
        q=make_tensor(cfg, T_Q, (B, Hq, D), std, dtype),
        k=make_tensor(cfg, T_K, (B, Lmax, Hkv, D), std, dtype),
        v=make_tensor(cfg, T_V, (B, Lmax, Hkv, D), std, dtype),
        seqlens=seqlens,
        sinks=make_sinks(cfg, Hq, sink_kind),
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
    )


@dataclass
class Varlen:
    """Packed queries over a paged KV cache.

    Sequence b owns query rows ``cu_seqlens_q[b]:cu_seqlens_q[b+1]`` and KV
    positions ``0..seqlens_k[b]-1``; position p lives in physical block
    ``block_table[b, p // block_size]`` at slot ``p % block_size``.
    """

    q: Tensor  # [Tq, Hq, D]
    k: Tensor  # [Nblk, bs, Hkv, D]
    v: Tensor  # [Nblk, bs, Hkv, D]
    cu_seqlens_q: np.ndarray  # [B+1] int32
    seqlens_k: np.ndarray  # [B] int32
    block_table: np.ndarray  # [B, maxblk] int32, -1 padded
    block_size: int
    sinks: np.ndarray
    scale: float
    q_lens: np.ndarray = field(default=None)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if len(self.q_lens) else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.block_table.shape[1] * self.block_size)


def varlen_problem(cfg: int, kv_lens, q_lens, Hq: int, Hkv: int, D: int = 64, block_size: int = 16,
                   maxblk: int | None = None, dtype: str = "bf16", std: float = 1.0,
                   sink_kind: str = "normal", permute: bool = True, spare_blocks: int = 0,
                   scale: float | None = None) -> Varlen:
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    assert np.all(q_lens <= kv_lens) and np.all(q_lens >= 0)
    B = len(kv_lens)
    nblk = [(int(L) + block_size - 1) // block_size for L in kv_lens]
    total = int(sum(nblk)) + spare_blocks
    if maxblk is None:
        maxblk = max(nblk) if nblk else 1
    perm = rng_for(cfg, T_PERM).permutation(total).astype(np.int32) if permute else np.arange(total, dtype=np.int32)
    table = np.full((B, maxblk), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    cu = np.zeros((B + 1,), dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    Tq = int(cu[-1])
    return Varlen(
        q=make_tensor(cfg, T_Q, (Tq, Hq, D), std, dtype),
        k=make_tensor(cfg, T_K, (max(total, 1), block_size, Hkv, D), std, dtype),
        v=make_tensor(cfg, T_V, (max(total, 1), block_size, Hkv, D), std, dtype),
        cu_seqlens_q=cu,
        seqlens_k=kv_lens,
        block_table=table,
        block_size=block_size,
        sinks=make_sinks(cfg, Hq, sink_kind),
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        q_lens=q_lens,
    )


# ---------------------------------------------------------------------------
# the five workloads the measurements are quoted on

def c1_tiny(dtype: str = "fp32") -> Prefill:
    """Tiny prefill: B1, S256, 8 q heads / 2 KV heads, D64, fp32, N(0,1), scale 1/8."""
    return prefill_problem(1, 1, 256, 8, 2, 64, dtype=dtype, std=1.0)


def c2_layer() -> Prefill:
    """Layer-shaped prefill: B1, S4096, 64/8 heads, D64, bf16 N(0,1)/sqrt2, fp32 N(0,1) sinks."""
    return prefill_problem(2, 1, 4096, 64, 8, 64, dtype="bf16", std=1.0 / math.sqrt(2.0))


def c3_decode() -> Decode:
    """Batched decode: B64, cache 8192, 64/8 heads, D64, bf16 N(0,1), fp32 sinks."""
    return decode_problem(3, 64, 8192, 64, 8, 64, dtype="bf16", std=1.0)


def c4_prefill() -> Prefill:
    """Long-context prefill: B1, S32768, 64/8 heads, D64, bf16 N(0,1)."""
    return prefill_problem(4, 1, 32768, 64, 8, 64, dtype="bf16", std=1.0)


def c4_decode() -> Decode:
    """Long-context decode: B8, cache 131072, 64/8 heads, D64, bf16 N(0,1)."""
    return decode_problem(40, 8, 131072, 64, 8, 64, dtype="bf16", std=1.0)


def c5_lengths(cfg: int = 5, B: int = 16):
    """Sequence lengths U{128..8192}; even b is a 512-token prefill chunk, odd b a decode step."""
    kv = rng_for(cfg, T_LEN).integers(128, 8193, size=B).astype(np.int32)
    q = np.array([min(512, int(L)) if b % 2 == 0 else 1 for b, L in enumerate(kv)], dtype=np.int32)
    return kv, q


def c5_ragged(cfg: int = 5) -> Varlen:
    """Ragged + paged: 16 sequences, 16-token blocks, permuted block table [16, 512]."""
    kv, q = c5_lengths(cfg)
    return varlen_problem(cfg, kv, q, 64, 8, 64, block_size=16, maxblk=512, dtype="bf16", std=1.0)


@dataclass
class Ring:
    """Decode step of a windowed layer against its ring cache of W slots per sequence."""

    q: Tensor        # [B, Hq, D]
    k_ring: Tensor   # [B, W, Hkv, D]
    v_ring: Tensor
    seqlens: np.ndarray  # [B] int32, positions including the new token
    sinks: np.ndarray
    scale: float
    W: int


def ring_problem(cfg: int, B: int, W: int, seqlens, Hq: int = 64, Hkv: int = 8, D: int = 64, dtype: str = "bf16",
                 std: float = 1.0, sink_kind: str = "normal", scale: float | None = None) -> Ring:
    """Ring contents drawn directly (every slot filled); seqlens given, or 'random' in [1, 3W]."""
    if isinstance(seqlens, str) and seqlens == "random":
        seqlens = rng_for(cfg, T_LEN).integers(1, 3 * W + 1, size=B)
    seqlens = np.broadcast_to(np.asarray(seqlens, dtype=np.int32), (B,)).copy()
    return Ring(
        q=make_tensor(cfg, T_Q, (B, Hq, D), std, dtype),
        k_ring=make_tensor(cfg, T_K, (B, W, Hkv, D), std, dtype),
        v_ring=make_tensor(cfg, T_V, (B, W, Hkv, D), std, dtype),
        seqlens=seqlens,
        sinks=make_sinks(cfg, Hq, sink_kind),
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        W=W,
    )


def c6_ring(B: int = 64) -> Ring:
    """Windowed-layer decode from a 128-slot ring: B sequences at position 8191, 64/8 heads, bf16 N(0,1)."""
    return ring_problem(6, B, 128, 8192)


def to_torch(t: Tensor, device):
    """Device tensor holding exactly the bits of ``t`` (bf16 or fp32)."""
    import torch

    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)
