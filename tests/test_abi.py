"""The C-ABI library: it loads, exports every symbol its header declares, and
rejects bad arguments with the documented status before launching anything.
CPU only: no call here reaches a kernel."""
import ctypes
import math
import os
import re

import pytest

import attention_gqa_causal_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

P = ctypes.c_void_p
DUMMY = P(256)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return gq.lib()


def test_library_loads(L):
    assert L.gqa_attn_version() == 600


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.gqa_attn_status_string(0) == b"GQA_OK"
    assert L.gqa_attn_status_string(-1) == b"GQA_ERR_INVALID_ARG"
    assert L.gqa_attn_status_string(-2) == b"GQA_ERR_UNSUPPORTED"
    assert L.gqa_attn_status_string(-3) == b"GQA_ERR_WORKSPACE"
    assert L.gqa_attn_status_string(-4) == b"GQA_ERR_HIP"
    assert L.gqa_attn_status_string(-99) == b"GQA_ERR_UNKNOWN"


def prefill(L, q=DUMMY, k=DUMMY, v=DUMMY, out=DUMMY, B=1, S=16, Hq=64, Hkv=8, D=64, window=0, scale=0.0, dt=0,
            sink_tokens=0):
    return L.gqa_attn_prefill(q, k, v, None, out, None, B, S, Hq, Hkv, D, window, sink_tokens, scale, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=32), -2),
    (dict(D=128), -2),
    (dict(Hq=12, Hkv=8), -2),
    (dict(Hq=0), -1),
    (dict(Hkv=-1), -1),
    (dict(window=-1), -1),
    (dict(sink_tokens=-1), -1),
    (dict(window=128, sink_tokens=-4), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=-0.5), -1),
    (dict(dt=7), -2),
    (dict(B=-1), -1),
    (dict(S=-3), -1),
    (dict(q=None), -1),
    (dict(k=None), -1),
    (dict(out=None), -1),
])
def test_prefill_rejects(L, kw, code):
    assert prefill(L, **kw) == code
    assert len(L.gqa_attn_last_error()) > 0


def test_prefill_empty_is_noop(L):
    assert prefill(L, q=None, k=None, v=None, out=None, B=0) == 0
    assert prefill(L, q=None, k=None, v=None, out=None, S=0) == 0
    assert L.gqa_attn_last_error() == b""


def decode(L, ws=None, ws_bytes=0, seqlens=DUMMY, B=64, Lmax=8192, Hq=64, Hkv=8, D=64, window=0, dt=0,
           sink_tokens=0):
    return L.gqa_attn_decode(DUMMY, DUMMY, DUMMY, seqlens, None, DUMMY, None, B, Lmax, Hq, Hkv, D, window, sink_tokens,
                             0.0, dt, ws, ws_bytes, None)


def test_decode_workspace_rules(L):
    # a long single-batch decode is split, so it needs a workspace
    need = L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 0, 0, 0)
    assert need > 0 and need % 4 == 0
    assert decode(L, B=8, Lmax=131072) == -3
    assert decode(L, ws=DUMMY, ws_bytes=need - 4, B=8, Lmax=131072) == -3
    # fp32 and invalid shapes need none
    assert L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 0, 0, 1) == 0
    assert L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 32, 0, 0, 0) == 0
    assert L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 128, -1, 0) == 0
    # a sliding window caps the work per sequence: never more partials than dense
    assert L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 128, 0, 0) <= need
    # sink tokens add keys to a windowed layer's range (never beyond the dense plan)
    assert L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 4096, 0, 0) <= \
        L.gqa_attn_decode_workspace_size(8, 131072, 64, 8, 64, 4096, 60000, 0) <= need


def test_decode_rejects(L):
    assert decode(L, seqlens=None) == -1
    assert decode(L, D=80) == -2
    assert decode(L, Lmax=0) == -1
    assert decode(L, window=-5) == -1
    assert decode(L, window=128, sink_tokens=-1) == -1
    assert decode(L, B=0) == 0


def varlen(L, table=DUMMY, cu_k=None, bs=16, maxblk=512, nblk=100, B=16, Tq=100, mq=64, mk=8192, window=0,
           cu_q=DUMMY, ws=None, ws_bytes=0, D=64):
    return L.gqa_attn_varlen_paged(DUMMY, DUMMY, DUMMY, cu_q, DUMMY, table, maxblk, bs, cu_k, nblk, None, DUMMY, None,
                                   B, Tq, mq, mk, 64, 8, D, window, 0, 0.0, 0, ws, ws_bytes, None)


def test_varlen_rejects(L):
    need = L.gqa_attn_varlen_workspace_size(16, 64, 8192, 64, 8, 64, 0, 0, 0)
    assert varlen(L, bs=12, ws=DUMMY, ws_bytes=need) == -2          # block size not a power of two
    assert varlen(L, bs=2048, ws=DUMMY, ws_bytes=need) == -2
    assert varlen(L, table=None, cu_k=None) == -1                 # packed needs cu_seqlens_k
    assert varlen(L, maxblk=4, bs=16, mk=8192) == -1               # table too small for max_kv_len
    assert varlen(L, mq=9000, mk=8192) == -1                       # more queries than positions
    assert varlen(L, cu_q=None) == -1
    assert varlen(L, nblk=0) == -1
    assert varlen(L, D=48) == -2
    assert varlen(L, B=0) == 0 and varlen(L, Tq=0) == 0 and varlen(L, mq=0) == 0
    if need:
        assert varlen(L, ws=None) == -3


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gq.attn_prefill(q, k, k.clone(), None)
    with pytest.raises(ValueError):
        gq.attn_decode(q[:, 0], (k, k), torch.ones(1, dtype=torch.int32), None)


def test_header_documents_each_entry_point():
    text = open(HEADER).read()
    for n in ("gqa_attn_prefill", "gqa_attn_decode", "gqa_attn_varlen_paged"):
        assert n in text
    # every entry point states layouts, ownership and error behaviour
    for word in ("[B, S, Hq, D]", "[B, Lmax, Hkv, D]", "block_table", "caller owns", "GQA_ERR_WORKSPACE"):
        assert word in text


def test_no_oracle_on_product_path():
    """The package must not import, call or link the CPU oracle."""
    pkg = os.path.join(ROOT, "attention_gqa_causal_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in src and "from oracle" not in src, f


def ring_append(L, B=4, T=4, W=128, Hkv=8, D=64, dt=0, cu=None, seqlens=DUMMY, kn=DUMMY, vn=DUMMY,
                kr=DUMMY, vr=DUMMY):
    return L.gqa_kv_ring_append(kn, vn, cu, seqlens, kr, vr, B, T, W, Hkv, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=128), -2),
    (dict(dt=7), -2),
    (dict(W=0), -1),
    (dict(W=-5), -1),
    (dict(T=3), -1),           # one new row per sequence without cu_seqlens_q
    (dict(B=-1), -1),
    (dict(Hkv=0), -1),
    (dict(seqlens=None), -1),
    (dict(kr=None), -1),
])
def test_ring_append_rejects(L, kw, code):
    assert ring_append(L, **kw) == code
    assert L.gqa_attn_last_error() != b""


def test_ring_append_empty_is_ok(L):
    assert ring_append(L, B=0, T=0, seqlens=None, kn=None, vn=None, kr=None, vr=None) == 0
    assert ring_append(L, B=3, T=0, cu=DUMMY, seqlens=None, kn=None, vn=None, kr=None, vr=None) == 0


def ring_decode(L, B=2, W=128, Hq=64, Hkv=8, D=64, scale=0.0, dt=0, q=DUMMY, seqlens=DUMMY, ws=None, ws_bytes=0):
    return L.gqa_attn_decode_ring(q, DUMMY, DUMMY, seqlens, None, DUMMY, None, B, W, Hq, Hkv, D, scale, dt,
                                  ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=0), -1),
    (dict(D=32), -2),
    (dict(Hq=12), -2),
    (dict(scale=-1.0), -1),
    (dict(seqlens=None), -1),
    (dict(q=None), -1),
])
def test_ring_decode_rejects(L, kw, code):
    assert ring_decode(L, **kw) == code


def prefill_rope(L, B=1, S=64, Hq=8, Hkv=2, D=64, window=0, st=0, scale=0.0, mscale=1.0, pairing=0, dt=0,
                 q=DUMMY, out=DUMMY):
    return L.gqa_attn_prefill_rope(q, DUMMY, DUMMY, None, out, None, B, S, Hq, Hkv, D, window, st, scale, None,
                                   mscale, pairing, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=1), -2),             # bf16 only
    (dict(pairing=2), -1),
    (dict(mscale=float("inf")), -1),
    (dict(D=128), -2),
    (dict(Hq=6, Hkv=4), -2),
    (dict(window=-1), -1),
    (dict(q=None), -1),
])
def test_prefill_rope_rejects(L, kw, code):
    assert prefill_rope(L, **kw) == code
    assert L.gqa_attn_last_error() != b""


def test_prefill_rope_empty_is_ok(L):
    assert prefill_rope(L, B=0, q=None, out=None) == 0
    assert prefill_rope(L, S=0, q=None, out=None) == 0


def test_rope_append_keys_only_needs_both_null(L):
    # q without q_out (or the reverse) is an error; both NULL is the keys-only form
    rc = L.gqa_rope_append(DUMMY, DUMMY, DUMMY, None, None, DUMMY, None, 1.0, 0, DUMMY, DUMMY, 0, 16, None, 0, 0, 0,
                           2, 2, 8, 2, 64, 0, None)
    assert rc == -1
    assert L.gqa_rope_append(None, DUMMY, DUMMY, None, None, DUMMY, None, 1.0, 0, DUMMY, DUMMY, 0, 16, None, 0, 0, 0,
                             0, 0, 8, 2, 64, 0, None) == 0


def ring_prefill(L, B=2, Tq=4, max_q_len=2, W=128, Hq=64, Hkv=8, D=64, scale=0.0, dt=0, q=DUMMY, kn=DUMMY,
                 cu=DUMMY, seqlens=DUMMY, kr=DUMMY, out=DUMMY, append=1):
    return L.gqa_attn_prefill_ring(q, kn, DUMMY, cu, seqlens, kr, DUMMY, append, None, out, None, B, Tq, max_q_len,
                                   W, Hq, Hkv, D, scale, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=0), -1),
    (dict(W=-3), -1),
    (dict(D=128), -2),
    (dict(dt=5), -2),
    (dict(Hq=12), -2),
    (dict(scale=float("nan")), -1),
    (dict(B=-1), -1),
    (dict(max_q_len=-1), -1),
    (dict(cu=None), -1),
    (dict(seqlens=None), -1),
    (dict(kn=None), -1),
    (dict(kr=None), -1),
    (dict(out=None), -1),
])
def test_ring_prefill_rejects(L, kw, code):
    assert ring_prefill(L, **kw) == code
    assert L.gqa_attn_last_error() != b""


def test_ring_prefill_empty_is_ok(L):
    # nothing to do: no pointer is looked at, no launch
    for kw in (dict(B=0), dict(Tq=0), dict(max_q_len=0)):
        assert ring_prefill(L, q=None, kn=None, cu=None, seqlens=None, kr=None, out=None, **kw) == 0


def test_ring_decode_workspace(L):
    # one split for a 128-slot ring; a long ring needs split partials
    assert L.gqa_attn_decode_ring_workspace_size(64, 128, 64, 8, 64, 0) == 0
    assert L.gqa_attn_decode_ring_workspace_size(8, 65536, 64, 8, 64, 0) > 0
    big = L.gqa_attn_decode_ring_workspace_size(8, 65536, 64, 8, 64, 0)
    assert ring_decode(L, B=8, W=65536, ws=None, ws_bytes=0) == -3
    assert ring_decode(L, B=8, W=65536, ws=DUMMY, ws_bytes=big - 1) == -3


def rope(L, B=4, T=4, Hq=64, Hkv=8, D=64, dt=0, cu=None, pairing=0, mscale=1.0, kind=0, cache_len=128,
         table=None, maxblk=0, bs=0, nblk=0, seqlens=DUMMY, inv=DUMMY, q=DUMMY, kc=DUMMY, q_out=DUMMY):
    return L.gqa_rope_append(q, DUMMY, DUMMY, q_out, cu, seqlens, inv, mscale, pairing, kc, DUMMY, kind, cache_len,
                             table, maxblk, bs, nblk, B, T, Hq, Hkv, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=128), -2),
    (dict(dt=5), -2),
    (dict(pairing=2), -1),
    (dict(mscale=float("nan")), -1),
    (dict(mscale=float("inf")), -1),
    (dict(T=3), -1),
    (dict(kind=3), -1),
    (dict(kind=0, cache_len=0), -1),
    (dict(kind=2, cache_len=-1), -1),
    (dict(kind=1, bs=12, maxblk=4, nblk=9, table=DUMMY), -2),
    (dict(kind=1, bs=16, maxblk=0, nblk=9, table=DUMMY), -1),
    (dict(kind=1, bs=16, maxblk=4, nblk=9, table=None), -1),
    (dict(seqlens=None), -1),
    (dict(q=None), -1),
    (dict(kc=None), -1),
    (dict(Hq=0), -1),
])
def test_rope_append_rejects(L, kw, code):
    assert rope(L, **kw) == code
    assert L.gqa_attn_last_error() != b""


def test_rope_append_null_table_is_the_default(L):
    # inv_freq NULL selects the library's own table: it is not an argument
    # error (the call below fails only on the missing cache)
    assert rope(L, inv=None, kc=None) == -1
    err = L.gqa_attn_last_error()
    assert b"k_cache" in err and b"inv_freq" not in err


def test_rope_append_empty_is_ok(L):
    assert rope(L, B=0, T=0, seqlens=None, inv=None, q=None, q_out=None, kc=None) == 0
    assert rope(L, B=0, T=0, seqlens=None, inv=None, q=None, kc=None) == -1  # q_out without q


def backward(L, B=1, S=16, Hq=64, Hkv=8, D=64, window=0, sink_tokens=0, scale=0.0, dt=0, q=DUMMY, lse=DUMMY,
             dout=DUMMY, dq=DUMMY, dsinks=None, ws=DUMMY, ws_bytes=1 << 20):
    return L.gqa_attn_prefill_backward(q, DUMMY, DUMMY, None, DUMMY, lse, dout, dq, DUMMY, DUMMY, dsinks,
                                       B, S, Hq, Hkv, D, window, sink_tokens, scale, dt, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=128), -2),
    (dict(dt=3), -2),
    (dict(Hq=12, Hkv=8), -2),
    (dict(Hq=0), -1),
    (dict(B=-1), -1),
    (dict(window=-1), -1),
    (dict(sink_tokens=-2), -1),
    (dict(scale=-1.0), -1),
    (dict(scale=float("nan")), -1),
    (dict(q=None), -1),
    (dict(lse=None), -1),
    (dict(dout=None), -1),
    (dict(dq=None), -1),
    (dict(ws=None), -3),
    (dict(ws_bytes=1024), -3),
])
def test_backward_rejects(L, kw, code):
    assert backward(L, **kw) == code
    assert L.gqa_attn_last_error() != b""


def test_backward_workspace_size(L):
    # two fp32 per (sequence, head, position) and one per (head, sequence, 1024
    # positions), each array rounded up to 256 bytes; with few
    # 64-key blocks (under 1024 per call) bf16 adds fp32 dK/dV partials for up
    # to 4 query slabs of every block (enough slabs for about 1024 jobs)
    part = 2 * 64 * 64 * 4
    ws = L.gqa_attn_prefill_backward_workspace_size
    assert ws(1, 16, 64, 8, 64, 1) == 2 * 16 * 64 * 4 + 256
    assert ws(1, 4096, 64, 8, 64, 0) == 2 * 4096 * 64 * 4 + 4 * 64 * 4 + 8 * 64 * 2 * part  # 512 blocks: 2 slabs
    assert ws(8, 4096, 64, 8, 64, 0) == 2 * 8 * 4096 * 64 * 4 + 8 * 4 * 64 * 4  # 4096 key blocks: no slabs
    assert ws(1, 100, 64, 8, 64, 0) == 2 * 100 * 64 * 4 + 256 + 8 * 2 * 4 * part
    assert ws(1, 3, 1, 1, 64, 1) == 3 * 256
    assert L.gqa_attn_prefill_backward_workspace_size(1, 16, 64, 8, 32, 0) == 0
    assert L.gqa_attn_prefill_backward_workspace_size(1, 16, 12, 8, 64, 0) == 0


def test_backward_empty_is_ok(L):
    assert backward(L, B=0, q=None, lse=None, dout=None, dq=None, ws=None, ws_bytes=0) == 0
    assert backward(L, S=0, q=None, lse=None, dout=None, dq=None, ws=None, ws_bytes=0) == 0


def test_release_library_reports_no_debug_records(L):
    # release builds clamp device-side metadata without recording it: the call
    # says so and touches no device
    flags = ctypes.c_uint(123)
    assert L.gqa_attn_debug_flags(ctypes.byref(flags), 1) == gq.GQA_ERR_UNSUPPORTED
    assert flags.value == 0
    assert L.gqa_attn_debug_flags(None, 0) == gq.GQA_ERR_INVALID_ARG


def test_debug_library_exports_the_same_symbols():
    path = os.path.join(ROOT, "attention_gqa_causal_amd", "libgqa_attn_debug.so")
    if not os.path.exists(path):
        pytest.skip("debug library not built (python -m attention_gqa_causal_amd.build --debug)")
    D = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(D, n), n
    D.gqa_attn_version.restype = ctypes.c_int
    assert D.gqa_attn_version() == 600
    # a NULL flags pointer is rejected before any device access
    D.gqa_attn_debug_flags.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert D.gqa_attn_debug_flags(None, 0) == gq.GQA_ERR_INVALID_ARG


def test_noalloc_decode_rejects_beyond_its_array_on_the_host(L):
    # 64 query heads over 4 KV heads at B16 x 65536 needs 17.3 MB of split partials, more than the
    # 16 MiB array; the call is refused before the device is touched (no GPU needed here)
    L.gqa_attn_decode_workspace_size.restype = ctypes.c_size_t
    assert L.gqa_attn_decode_workspace_size(16, 65536, 64, 4, 64, 0, 0, 0) > 16 << 20
    L.gqa_attn_decode_noalloc.restype = ctypes.c_int
    L.gqa_attn_decode_noalloc.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                                                                                         ctypes.c_void_p]
    rc = L.gqa_attn_decode_noalloc(DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, None, 16, 65536, 64, 4, 64, 0, 0, 0.0, 0,
                                   None)
    assert rc == -3
    assert b"allocation-free" in L.gqa_attn_last_error()
    # argument errors come first, as for every entry point
    assert L.gqa_attn_decode_noalloc(DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, None, 4, 64, 64, 8, 128, 0, 0, 0.0, 0,
                                     None) == -2
