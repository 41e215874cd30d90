"""Python binding of the MI355X attention library (``libgqa_attn.so``).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is not built, every call raises.

Functions (names follow the C ABI in ``include/gqa_attn.h``):

* ``attn_prefill(q, k, v, sinks, window=0, scale=None, sink_tokens=0)``
* ``attn_decode(q, kv_cache, seqlens, sinks, window=0, scale=None, sink_tokens=0)``
* ``attn_varlen_paged(q, kv_cache, block_table, cu_seqlens_q, seqlens_k, sinks, ...)``
* ``rope_append(q, k, v, seqlens, kv_cache, inv_freq=None, ...)``: rotary
  encoding of new rows fused with their KV-cache append (contiguous, paged or
  ring cache); inv_freq=None selects the library's default table θ_i = 10000^(-2i/D)
* ``kv_ring_append(k_new, v_new, kv_ring, seqlens, cu_seqlens_q=None)`` and
  ``attn_decode_ring(q, kv_ring, seqlens, sinks, scale=None)``: the W-slot ring
  cache of sliding-window layers (position p in slot p % W)
* ``attn_prefill_backward(q, k, v, sinks, out, lse, dout, ...)``: gradients of
  the prefill with respect to q, k, v and the sink logits

The computation is causal grouped-query attention with a learned per-head sink
logit and an optional sliding window (0 = dense), as described on the pages
«GPT-OSS vs Qwen3» (sections "Introduction de Grouped Query Attention",
"Utilisation de Sliding Window Attention", "Attention Bias et Sinks") and
«GPT-OSS-20B : Architecture MoE & Résumé du Model Card» (§3.3).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "attn_prefill",
    "attn_prefill_rope",
    "attn_decode",
    "attn_varlen_paged",
    "kv_ring_append",
    "rope_append",
    "attn_decode_ring",
    "attn_prefill_ring",
    "attn_decode_noalloc",
    "attn_decode_step",
    "attn_prefill_backward",
    "backward_workspace_size",
    "decode_workspace_size",
    "varlen_workspace_size",
    "lib",
    "lib_path",
    "GQA_BF16",
    "GQA_FP32",
    "GqaError",
    "debug_flags",
]

GQA_BF16 = 0
GQA_FP32 = 1
GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_UNSUPPORTED = -2
GQA_ERR_WORKSPACE = -3
GQA_ERR_HIP = -4

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgqa_attn.so"
_lib = None


class GqaError(RuntimeError):
    """A nonzero status returned by the C library."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status


def lib_path() -> str:
    return os.environ.get("GQA_ATTN_LIB") or os.path.join(_PKG, _LIB_NAME)


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "gqa_attn_version": (_I, []),
    "gqa_attn_status_string": (ctypes.c_char_p, [_I]),
    "gqa_attn_last_error": (ctypes.c_char_p, []),
    "gqa_attn_debug_flags": (_I, [ctypes.POINTER(ctypes.c_uint), _I]),
    "gqa_attn_prefill": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_attn_prefill_rope": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _F, _I, _I, _P]),
    "gqa_attn_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "gqa_attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "gqa_attn_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_attn_varlen_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "gqa_attn_varlen_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _P, _P, _P,
                                   _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "gqa_kv_ring_append": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gqa_attn_decode_ring_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gqa_attn_decode_ring": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "gqa_attn_prefill_ring": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                   _P]),
    "gqa_rope_append": (_I, [_P, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _I, _I, _P, _I, _I, _I,
                             _I, _I, _I, _I, _I, _I, _P]),
    "gqa_attn_decode_step": (_I, [_P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P,
                                  _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_attn_prefill_backward_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gqa_attn_prefill_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
}


def lib() -> ctypes.CDLL:
    """Load the C library (after torch, so that one HIP runtime serves both)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run `python -m attention_gqa_causal_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# device-side metadata clamp records (gqa_attn_debug_flags, libraries built with GQA_DEBUG)
GQA_DBG_SEQLENS_K = 1
GQA_DBG_BLOCK_TABLE = 2
GQA_DBG_CU_SEQLENS_Q = 4
GQA_DBG_PACKED_ROW = 8
GQA_DBG_Q_LEN = 16


def debug_flags(reset: bool = True) -> int:
    """OR of the GQA_DBG_* kinds of device-side metadata the kernels had to clamp
    since the last reset (synchronises the device).  Needs the library built with
    GQA_DEBUG (``python -m attention_gqa_causal_amd.build --debug``, then
    GQA_ATTN_LIB pointing at libgqa_attn_debug.so); a release library raises
    GqaError (GQA_ERR_UNSUPPORTED)."""
    flags = ctypes.c_uint(0)
    _check(lib().gqa_attn_debug_flags(ctypes.byref(flags), 1 if reset else 0))
    return int(flags.value)


def _check(status: int):
    if status != GQA_OK:
        L = lib()
        raise GqaError(status, L.gqa_attn_status_string(status).decode(), L.gqa_attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _out_arg(out, q):
    """A caller's output tensor (checked against q), or a new one."""
    if out is None:
        return torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, q.device, q.dim())
    _need(out.shape == q.shape, "out must match q")
    return out


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_FP32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name, dtype, device, ndim):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.device == device, f"{name} must be on {device}")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.dim() == ndim, f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _sinks_arg(sinks, hq, device):
    if sinks is None:
        return None
    _check_tensor(sinks, "sinks", torch.float32, device, 1)
    _need(sinks.shape[0] == hq, f"sinks must have Hq={hq} entries")
    return sinks


def _scale(scale) -> float:
    return 0.0 if scale is None else float(scale)


def _split_cache(kv_cache):
    if isinstance(kv_cache, (tuple, list)):
        _need(len(kv_cache) == 2, "kv_cache must be (k_cache, v_cache)")
        return kv_cache[0], kv_cache[1]
    _need(kv_cache.shape[0] == 2, "a single kv_cache tensor must stack K and V on dim 0")
    return kv_cache[0], kv_cache[1]


def attn_prefill(q, k, v, sinks=None, window: int = 0, scale=None, return_lse: bool = False, out=None,
                 sink_tokens: int = 0):
    """Causal self-attention over whole sequences.

    q [B, S, Hq, 64], k/v [B, S, Hkv, 64] (bf16 or fp32, same dtype, on the GPU);
    sinks [Hq] fp32 or None.  Returns out [B, S, Hq, 64] (and lse [B, Hq, S] fp32).
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 4)
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    _check_tensor(k, "k", q.dtype, dev, 4)
    _check_tensor(v, "v", q.dtype, dev, 4)
    _need(k.shape[:2] == (B, S) and k.shape[3] == D and v.shape == k.shape, "k/v must be [B, S, Hkv, D] matching q")
    Hkv = k.shape[2]
    sinks = _sinks_arg(sinks, Hq, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.dtype, dev, 4)
        _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().gqa_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), _ptr(lse),
                                  B, S, Hq, Hkv, D, int(window), int(sink_tokens), _scale(scale), dt, _stream(dev)))
    return (out, lse) if return_lse else out


def attn_prefill_rope(q, k, v, sinks=None, window: int = 0, scale=None, inv_freq=None, mscale: float = 1.0,
                      pairing=0, return_lse: bool = False, out=None, sink_tokens: int = 0):
    """Prefill whose queries arrive unrotated: the kernel rotates each query row at its
    position as it loads it (the rotary append's angles and rotation, bit for bit).

    q [B, S, Hq, 64] unrotated, k [B, S, Hkv, 64] already rotated, v [B, S, Hkv, 64]
    (bf16); inv_freq [32] fp32 or None (the default table); pairing 0: (2i, 2i+1),
    1: (i, i + 32).  Returns out (and lse) as ``attn_prefill``.
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 4)
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    _check_tensor(k, "k", q.dtype, dev, 4)
    _check_tensor(v, "v", q.dtype, dev, 4)
    _need(k.shape[:2] == (B, S) and k.shape[3] == D and v.shape == k.shape, "k/v must be [B, S, Hkv, D] matching q")
    Hkv = k.shape[2]
    if inv_freq is not None:
        _check_tensor(inv_freq, "inv_freq", torch.float32, dev, 1)
        _need(inv_freq.shape[0] == D // 2, "inv_freq must have D/2 entries")
    sinks = _sinks_arg(sinks, Hq, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.dtype, dev, 4)
        _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().gqa_attn_prefill_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), _ptr(lse), B, S, Hq, Hkv,
                                       D, int(window), int(sink_tokens), _scale(scale), _ptr(inv_freq),
                                       float(mscale), int(pairing), dt, _stream(dev)))
    return (out, lse) if return_lse else out


def backward_workspace_size(B, S, Hq, Hkv, D=64, dtype=GQA_BF16) -> int:
    return int(lib().gqa_attn_prefill_backward_workspace_size(B, S, Hq, Hkv, D, dtype))


def attn_prefill_backward(q, k, v, sinks, out, lse, dout, window: int = 0, scale=None, sink_tokens: int = 0,
                          workspace=None, grads=None):
    """Gradients of the prefill: returns (dq, dk, dv, dsinks).

    q, out, dout [B, S, Hq, 64]; k, v [B, S, Hkv, 64] (one dtype, bf16 or fp32);
    lse [B, Hq, S] fp32 as ``attn_prefill(..., return_lse=True)`` returned it;
    sinks [Hq] fp32 or None (then dsinks is all zeros).  ``grads``: optional
    preallocated (dq, dk, dv, dsinks).  ``workspace``: optional uint8 tensor of
    at least ``backward_workspace_size`` bytes.
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 4)
    dt = _dtype_code(q)
    B, S, Hq, D = q.shape
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(t, name, q.dtype, dev, 4)
    _need(k.shape[:2] == (B, S) and k.shape[3] == D and v.shape == k.shape, "k/v must be [B, S, Hkv, D] matching q")
    _need(out.shape == q.shape and dout.shape == q.shape, "out and dout must match q")
    Hkv = k.shape[2]
    _check_tensor(lse, "lse", torch.float32, dev, 3)
    _need(tuple(lse.shape) == (B, Hq, S), "lse must be [B, Hq, S]")
    sinks = _sinks_arg(sinks, Hq, dev)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsinks = torch.empty((Hq,), dtype=torch.float32, device=dev)
    else:
        dq, dk, dv, dsinks = grads
        _check_tensor(dq, "dq", q.dtype, dev, 4)
        _check_tensor(dk, "dk", q.dtype, dev, 4)
        _check_tensor(dv, "dv", q.dtype, dev, 4)
        _need(dq.shape == q.shape and dk.shape == k.shape and dv.shape == k.shape, "gradients must match q, k, v")
        if dsinks is not None:
            _check_tensor(dsinks, "dsinks", torch.float32, dev, 1)
            _need(dsinks.shape[0] == Hq, f"dsinks must have Hq={Hq} entries")
    need = backward_workspace_size(B, S, Hq, Hkv, D, dt)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check_tensor(workspace, "workspace", torch.uint8, dev, 1)
    _check(lib().gqa_attn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(dout),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), B, S, Hq, Hkv, D, int(window),
                                           int(sink_tokens), _scale(scale), dt, _ptr(workspace),
                                           workspace.numel(), _stream(dev)))
    return dq, dk, dv, dsinks


def decode_workspace_size(B, Lmax, Hq, Hkv, D=64, window=0, dtype=GQA_BF16, sink_tokens=0) -> int:
    return int(lib().gqa_attn_decode_workspace_size(B, Lmax, Hq, Hkv, D, int(window), int(sink_tokens), dtype))


def attn_decode(q, kv_cache, seqlens, sinks=None, window: int = 0, scale=None, return_lse: bool = False,
                workspace=None, sink_tokens: int = 0, out=None):
    """One new query token per sequence against a contiguous KV cache.

    q [B, Hq, 64]; kv_cache = (k_cache, v_cache) each [B, Lmax, Hkv, 64], or one
    [2, B, Lmax, Hkv, 64] tensor; seqlens [B] int32 on the GPU (cached positions
    including the new token).  Returns out [B, Hq, 64] (and lse [B, Hq]); out
    may be given (a contiguous tensor like q).
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 3)
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    kc, vc = _split_cache(kv_cache)
    _check_tensor(kc, "k_cache", q.dtype, dev, 4)
    _check_tensor(vc, "v_cache", q.dtype, dev, 4)
    _need(kc.shape[0] == B and kc.shape[3] == D and vc.shape == kc.shape, "caches must be [B, Lmax, Hkv, D]")
    Lmax, Hkv = kc.shape[1], kc.shape[2]
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B, "seqlens must have B entries")
    sinks = _sinks_arg(sinks, Hq, dev)
    out = _out_arg(out, q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    ws_bytes = int(lib().gqa_attn_decode_workspace_size(B, Lmax, Hq, Hkv, D, int(window), int(sink_tokens), dt))
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gqa_attn_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(seqlens), _ptr(sinks), _ptr(out), _ptr(lse),
                                 B, Lmax, Hq, Hkv, D, int(window), int(sink_tokens), _scale(scale), dt,
                                 _ptr(workspace), ws_have, _stream(dev)))
    return (out, lse) if return_lse else out


def attn_decode_noalloc(q, kv_cache, seqlens, sinks=None, window: int = 0, scale=None, return_lse: bool = False,
                        sink_tokens: int = 0, out=None):
    """attn_decode through the allocation-free entry point: the split partials live in
    the library's fixed per-GPU array (GQA_NOALLOC_SCRATCH_BYTES), not in a workspace.

    Arguments as attn_decode.  Pass `out` (and nothing that needs lse) for a call that
    allocates no device memory at all; calls that overlap on one GPU share the array.
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 3)
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    kc, vc = _split_cache(kv_cache)
    _check_tensor(kc, "k_cache", q.dtype, dev, 4)
    _check_tensor(vc, "v_cache", q.dtype, dev, 4)
    _need(kc.shape[0] == B and kc.shape[3] == D and vc.shape == kc.shape, "caches must be [B, Lmax, Hkv, D]")
    Lmax, Hkv = kc.shape[1], kc.shape[2]
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B, "seqlens must have B entries")
    sinks = _sinks_arg(sinks, Hq, dev)
    out = _out_arg(out, q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().gqa_attn_decode_noalloc(_ptr(q), _ptr(kc), _ptr(vc), _ptr(seqlens), _ptr(sinks), _ptr(out),
                                         _ptr(lse), B, Lmax, Hq, Hkv, D, int(window), int(sink_tokens), _scale(scale),
                                         dt, _stream(dev)))
    return (out, lse) if return_lse else out


def varlen_workspace_size(B, max_q_len, max_kv_len, Hq, Hkv, D=64, window=0, dtype=GQA_BF16, sink_tokens=0) -> int:
    return int(lib().gqa_attn_varlen_workspace_size(B, max_q_len, max_kv_len, Hq, Hkv, D, int(window),
                                                    int(sink_tokens), dtype))


def attn_varlen_paged(q, kv_cache, block_table, cu_seqlens_q, seqlens_k, sinks=None, window: int = 0, scale=None,
                      max_q_len: int | None = None, max_kv_len: int | None = None, cu_seqlens_k=None,
                      return_lse: bool = False, workspace=None, sink_tokens: int = 0, out=None):
    """Packed variable-length queries over a paged KV cache (mixed prefill chunks and decode steps).

    q [Tq, Hq, 64]; kv_cache = (k_cache, v_cache) each [num_blocks, block_size, Hkv, 64]
    with block_table [B, max_blocks] int32, or, with block_table None, packed
    [num_rows, Hkv, 64] caches addressed by cu_seqlens_k [B+1].  cu_seqlens_q [B+1]
    and seqlens_k [B] are int32 on the GPU.  max_q_len / max_kv_len are host-side
    bounds; when omitted they are read back from the GPU (a synchronising copy).
    Returns out [Tq, Hq, 64] (and lse [Hq, Tq]); out may be given (a contiguous
    tensor like q).
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 3)
    dt = _dtype_code(q)
    Tq, Hq, D = q.shape
    kc, vc = _split_cache(kv_cache)
    _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _check_tensor(seqlens_k, "seqlens_k", torch.int32, dev, 1)
    B = seqlens_k.shape[0]
    _need(cu_seqlens_q.shape[0] == B + 1, "cu_seqlens_q must have B+1 entries")
    if block_table is not None:
        _check_tensor(kc, "k_cache", q.dtype, dev, 4)
        _check_tensor(vc, "v_cache", q.dtype, dev, 4)
        _need(vc.shape == kc.shape and kc.shape[3] == D, "paged caches must be [num_blocks, block_size, Hkv, D]")
        _check_tensor(block_table, "block_table", torch.int32, dev, 2)
        _need(block_table.shape[0] == B, "block_table must have B rows")
        num_blocks, block_size, Hkv = kc.shape[0], kc.shape[1], kc.shape[2]
        max_blocks = block_table.shape[1]
        cap = max_blocks * block_size
    else:
        _check_tensor(kc, "k_cache", q.dtype, dev, 3)
        _check_tensor(vc, "v_cache", q.dtype, dev, 3)
        _need(vc.shape == kc.shape and kc.shape[2] == D, "packed caches must be [num_rows, Hkv, D]")
        _need(cu_seqlens_k is not None, "cu_seqlens_k is required without a block table")
        _check_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev, 1)
        _need(cu_seqlens_k.shape[0] == B + 1, "cu_seqlens_k must have B+1 entries")
        num_blocks, block_size, Hkv = kc.shape[0], 1, kc.shape[1]
        max_blocks = 0
        cap = None
    if max_q_len is None:
        max_q_len = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B else 0
    if max_kv_len is None:
        max_kv_len = cap if cap is not None else (int(seqlens_k.max().item()) if B else 0)
    sinks = _sinks_arg(sinks, Hq, dev)
    out = _out_arg(out, q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev) if return_lse else None
    ws_bytes = int(lib().gqa_attn_varlen_workspace_size(B, max_q_len, max_kv_len, Hq, Hkv, D, int(window),
                                                        int(sink_tokens), dt))
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gqa_attn_varlen_paged(_ptr(q), _ptr(kc), _ptr(vc), _ptr(cu_seqlens_q), _ptr(seqlens_k),
                                       _ptr(block_table), max_blocks, block_size, _ptr(cu_seqlens_k), num_blocks,
                                       _ptr(sinks), _ptr(out), _ptr(lse), B, Tq, int(max_q_len), int(max_kv_len),
                                       Hq, Hkv, D, int(window), int(sink_tokens), _scale(scale), dt,
                                       _ptr(workspace), ws_have, _stream(dev)))
    return (out, lse) if return_lse else out


def kv_ring_append(k_new, v_new, kv_ring, seqlens, cu_seqlens_q=None):
    """Write new tokens' K/V rows into the W-slot rings of a sliding-window layer (in place).

    kv_ring = (k_ring, v_ring) each [B, W, Hkv, 64]; k_new/v_new [T, Hkv, 64] of the
    same dtype.  Without cu_seqlens_q, T == B and row b is sequence b's newest token
    (position seqlens[b] - 1); with cu_seqlens_q [B+1] int32 the rows of sequence b
    are its newest q_len positions.  seqlens [B] int32 counts the new rows.
    """
    kr, vr = _split_cache(kv_ring)
    dev = kr.device
    dt = _dtype_code(kr)
    _check_tensor(kr, "k_ring", kr.dtype, dev, 4)
    _check_tensor(vr, "v_ring", kr.dtype, dev, 4)
    _need(vr.shape == kr.shape, "k_ring and v_ring must have the same shape")
    B, W, Hkv, D = kr.shape
    _check_tensor(k_new, "k_new", kr.dtype, dev, 3)
    _check_tensor(v_new, "v_new", kr.dtype, dev, 3)
    _need(v_new.shape == k_new.shape and k_new.shape[1:] == (Hkv, D), "k_new/v_new must be [T, Hkv, D]")
    T = k_new.shape[0]
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B, "seqlens must have B entries")
    if cu_seqlens_q is not None:
        _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
        _need(cu_seqlens_q.shape[0] == B + 1, "cu_seqlens_q must have B+1 entries")
    _check(lib().gqa_kv_ring_append(_ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q), _ptr(seqlens), _ptr(kr), _ptr(vr),
                                    B, T, W, Hkv, D, dt, _stream(dev)))


def attn_decode_ring(q, kv_ring, seqlens, sinks=None, scale=None, return_lse: bool = False, workspace=None):
    """Decode on a sliding-window layer against its ring cache.

    q [B, Hq, 64]; kv_ring = (k_ring, v_ring) each [B, W, Hkv, 64] holding the last
    min(seqlens[b], W) positions (slot p % W); seqlens [B] int32 counts the new token.
    The window is the ring size W.  Returns out [B, Hq, 64] (and lse [B, Hq]).
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 3)
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    kr, vr = _split_cache(kv_ring)
    _check_tensor(kr, "k_ring", q.dtype, dev, 4)
    _check_tensor(vr, "v_ring", q.dtype, dev, 4)
    _need(kr.shape[0] == B and kr.shape[3] == D and vr.shape == kr.shape, "rings must be [B, W, Hkv, D]")
    W, Hkv = kr.shape[1], kr.shape[2]
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B, "seqlens must have B entries")
    sinks = _sinks_arg(sinks, Hq, dev)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    ws_bytes = int(lib().gqa_attn_decode_ring_workspace_size(B, W, Hq, Hkv, D, dt))
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gqa_attn_decode_ring(_ptr(q), _ptr(kr), _ptr(vr), _ptr(seqlens), _ptr(sinks), _ptr(out), _ptr(lse),
                                      B, W, Hq, Hkv, D, _scale(scale), dt, _ptr(workspace), ws_have, _stream(dev)))
    return (out, lse) if return_lse else out


def attn_prefill_ring(q, k_new, v_new, cu_seqlens_q, seqlens, kv_ring, sinks=None, scale=None, append: bool = True,
                      max_q_len: int | None = None, return_lse: bool = False, out=None):
    """Chunked prefill of a sliding-window layer over its ring: attend, then append.

    q [Tq, Hq, 64], k_new/v_new [Tq, Hkv, 64]: the chunks' rows, sequence b's at
    cu_seqlens_q[b]..cu_seqlens_q[b+1]-1 (int32 [B+1]), its newest positions;
    seqlens [B] int32 counts each sequence's chunk.  kv_ring = (k_ring, v_ring) each
    [B, W, Hkv, 64] holding the positions before the chunks; the window is W.  With
    append the chunks are written to the rings after the attention.  max_q_len is a
    host-side bound (read back from the GPU when omitted).  Returns out [Tq, Hq, 64]
    (and lse [Hq, Tq]).
    """
    dev = q.device
    _check_tensor(q, "q", q.dtype, dev, 3)
    dt = _dtype_code(q)
    Tq, Hq, D = q.shape
    kr, vr = _split_cache(kv_ring)
    _check_tensor(kr, "k_ring", q.dtype, dev, 4)
    _check_tensor(vr, "v_ring", q.dtype, dev, 4)
    _need(kr.shape[3] == D and vr.shape == kr.shape, "rings must be [B, W, Hkv, D]")
    B, W, Hkv = kr.shape[0], kr.shape[1], kr.shape[2]
    _check_tensor(k_new, "k_new", q.dtype, dev, 3)
    _check_tensor(v_new, "v_new", q.dtype, dev, 3)
    _need(k_new.shape == (Tq, Hkv, D) and v_new.shape == k_new.shape, "k_new/v_new must be [Tq, Hkv, D]")
    _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B and cu_seqlens_q.shape[0] == B + 1,
          "seqlens must have B entries and cu_seqlens_q B+1")
    if max_q_len is None:
        max_q_len = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B else 0
    sinks = _sinks_arg(sinks, Hq, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.dtype, dev, 3)
        _need(out.shape == q.shape, "out must have q's shape")
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=dev) if return_lse else None
    _check(lib().gqa_attn_prefill_ring(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q), _ptr(seqlens), _ptr(kr),
                                       _ptr(vr), int(bool(append)), _ptr(sinks), _ptr(out), _ptr(lse), B, Tq,
                                       int(max_q_len), W, Hq, Hkv, D, _scale(scale), dt, _stream(dev)))
    return (out, lse) if return_lse else out


ROPE_INTERLEAVED = 0
ROPE_HALVES = 1


def attn_decode_step(q, k_new, v_new, seqlens, kv_cache, sinks=None, window: int = 0, scale=None,
                     sink_tokens: int = 0, inv_freq=None, mscale: float = 1.0, pairing=ROPE_INTERLEAVED,
                     block_table=None, ring: bool = False, q_out=None, return_lse: bool = False, out=None):
    """One decode step in one launch: rotate the new token's query and key, append the
    rotated key and the value to the cache, attend.

    q [B, Hq, 64], k_new/v_new [B, Hkv, 64] bf16 (not rotated); seqlens [B] int32 counts
    the new token.  kv_cache = (k_cache, v_cache): contiguous [B, L, Hkv, 64]; paged
    [num_blocks, block_size, Hkv, 64] with block_table; or, with ring=True, rings
    [B, W, Hkv, 64] (the window is W).  Returns out [B, Hq, 64] (and lse [B, Hq]);
    q_out, if given, receives the rotated queries.
    """
    dev = q.device
    _check_tensor(q, "q", torch.bfloat16, dev, 3)
    B, Hq, D = q.shape
    _check_tensor(k_new, "k_new", torch.bfloat16, dev, 3)
    _check_tensor(v_new, "v_new", torch.bfloat16, dev, 3)
    _need(k_new.shape[0] == B and k_new.shape[2] == D and v_new.shape == k_new.shape, "k_new/v_new must be [B, Hkv, D]")
    Hkv = k_new.shape[1]
    kc, vc = _split_cache(kv_cache)
    _check_tensor(kc, "k_cache", torch.bfloat16, dev, 4)
    _check_tensor(vc, "v_cache", torch.bfloat16, dev, 4)
    _need(vc.shape == kc.shape and kc.shape[2] == Hkv and kc.shape[3] == D, "caches must be [.., .., Hkv, D]")
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    _need(seqlens.shape[0] == B, "seqlens must have B entries")
    if inv_freq is not None:
        _check_tensor(inv_freq, "inv_freq", torch.float32, dev, 1)
        _need(inv_freq.shape[0] == D // 2, "inv_freq must have D/2 entries")
    if q_out is not None:
        _check_tensor(q_out, "q_out", torch.bfloat16, dev, 3)
        _need(q_out.shape == q.shape, "q_out must match q")
    sinks = _sinks_arg(sinks, Hq, dev)
    out = _out_arg(out, q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    if block_table is not None:
        _check_tensor(block_table, "block_table", torch.int32, dev, 2)
        _need(block_table.shape[0] == B, "block_table must have B rows")
        kind, cache_len = 1, 0
        max_blocks, block_size, num_blocks = block_table.shape[1], kc.shape[1], kc.shape[0]
    else:
        _need(kc.shape[0] == B, "a contiguous or ring cache has B rows")
        kind, cache_len = (2 if ring else 0), kc.shape[1]
        max_blocks, block_size, num_blocks = 0, 0, 0
    _check(lib().gqa_attn_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(q_out), _ptr(seqlens), _ptr(inv_freq),
                                      float(mscale), int(pairing), _ptr(kc), _ptr(vc), kind, cache_len,
                                      _ptr(block_table), max_blocks, block_size, num_blocks, _ptr(sinks), _ptr(out),
                                      _ptr(lse), B, Hq, Hkv, D, int(window), int(sink_tokens), _scale(scale),
                                      GQA_BF16, _stream(dev)))
    return (out, lse) if return_lse else out


def rope_append(q, k, v, seqlens, kv_cache, inv_freq=None, q_out=None, cu_seqlens_q=None, pairing=ROPE_INTERLEAVED,
                mscale: float = 1.0, block_table=None, ring: bool = False):
    """Rotate new rows' queries and keys and append keys and values to the cache.

    q [T, Hq, 64], k/v [T, Hkv, 64] (bf16 or fp32); seqlens [B] int32 counts the new rows;
    without cu_seqlens_q, T == B (one row per sequence).  kv_cache = (k_cache, v_cache):
    contiguous [B, L, Hkv, 64]; paged [num_blocks, block_size, Hkv, 64] with block_table
    [B, max_blocks]; or, with ring=True, rings [B, W, Hkv, 64].  Returns q_out [T, Hq, 64]
    (pass q_out=q to rotate in place).  q=None: keys only (for attn_prefill_rope, which
    rotates its queries itself); returns None.
    """
    dev = k.device
    dt = _dtype_code(k)
    _check_tensor(k, "k", k.dtype, dev, 3)
    _check_tensor(v, "v", k.dtype, dev, 3)
    T, Hkv, D = k.shape
    _need(v.shape == k.shape, "k/v must be [T, Hkv, D]")
    if q is None:
        _need(q_out is None, "q_out needs q")
        Hq = 1
    else:
        _check_tensor(q, "q", k.dtype, dev, 3)
        _need(q.shape[0] == T and q.shape[2] == D, "q must be [T, Hq, D]")
        Hq = q.shape[1]
    q_dtype = k.dtype
    Hkv = k.shape[1]
    kc, vc = _split_cache(kv_cache)
    _check_tensor(kc, "k_cache", q_dtype, dev, 4)
    _check_tensor(vc, "v_cache", q_dtype, dev, 4)
    _need(vc.shape == kc.shape and kc.shape[2] == Hkv and kc.shape[3] == D, "caches must be [.., .., Hkv, D]")
    _check_tensor(seqlens, "seqlens", torch.int32, dev, 1)
    B = seqlens.shape[0]
    if cu_seqlens_q is not None:
        _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
        _need(cu_seqlens_q.shape[0] == B + 1, "cu_seqlens_q must have B+1 entries")
    if inv_freq is not None:  # None: the library's default table θ_i = 10000^(-2i/D)
        _check_tensor(inv_freq, "inv_freq", torch.float32, dev, 1)
        _need(inv_freq.shape[0] == D // 2, "inv_freq must have D/2 entries")
    if q is None:
        pass
    elif q_out is None:
        q_out = torch.empty_like(q)
    else:
        _check_tensor(q_out, "q_out", q_dtype, dev, 3)
        _need(q_out.shape == q.shape, "q_out must match q")
    if block_table is not None:
        _check_tensor(block_table, "block_table", torch.int32, dev, 2)
        _need(block_table.shape[0] == B, "block_table must have B rows")
        kind, cache_len = 1, 0
        max_blocks, block_size, num_blocks = block_table.shape[1], kc.shape[1], kc.shape[0]
    else:
        _need(kc.shape[0] == B, "a contiguous or ring cache has B rows")
        kind, cache_len = (2 if ring else 0), kc.shape[1]
        max_blocks, block_size, num_blocks = 0, 0, 0
    _check(lib().gqa_rope_append(_ptr(q), _ptr(k), _ptr(v), _ptr(q_out), _ptr(cu_seqlens_q), _ptr(seqlens),
                                 _ptr(inv_freq), float(mscale), int(pairing), _ptr(kc), _ptr(vc), kind, cache_len,
                                 _ptr(block_table), max_blocks, block_size, num_blocks, B, T, Hq, Hkv, D, dt,
                                 _stream(dev)))
    return q_out
