"""GPU parity of the rotary encoding fused with the KV-cache append, through the C ABI.

The rotated queries and the cache rows written are compared with the fp64
oracle (``oracle.rope``) at the rounding of the output dtype: bf16 results are
within one bf16 step of the exact value (2^-8 relative) plus the fp32 rounding
of the rotation; fp32 results within 2e-6 absolute (inputs N(0,1)).  Cache rows
the call must not touch are compared bit for bit.  Positions reach the
131 072-token context.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
import oracle.rope as R
from gpu_helpers import assert_bf16_close, dev_f32, dev_i32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


def close_to_dtype(got, ref, dtype, what):
    err = np.abs(got - ref)
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 2e-5
    else:
        bound = np.full_like(ref, 2e-6)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} beyond the dtype bound, worst {err.max():.3e}"


def bits(t: torch.Tensor) -> np.ndarray:
    h = t.detach().cpu().contiguous()
    return h.view(torch.int16).numpy() if h.dtype == torch.bfloat16 else h.view(torch.int32).numpy()


def make_rows(cfg, T, Hq, Hkv, dtype):
    q = gi.make_tensor(cfg, gi.T_Q, (T, Hq, 64), 1.0, dtype)
    k = gi.make_tensor(cfg, gi.T_K, (T, Hkv, 64), 1.0, dtype)
    v = gi.make_tensor(cfg, gi.T_V, (T, Hkv, 64), 1.0, dtype)
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("pairing", [0, 1])
def test_rope_decode_step_contiguous(device, dtype, pairing):
    B, Hq, Hkv, Lmax = 6, 64, 8, 300
    seqlens = np.array([1, 2, 100, 299, 300, 301], dtype=np.int32)  # the last does not fit the cache
    say(f"rope decode step contiguous {dtype} pairing={pairing}")
    q, k, v = make_rows(90, B, Hq, Hkv, dtype)
    cache = gi.make_tensor(91, gi.T_K, (B, Lmax, Hkv, 64), 1.0, dtype)
    vcache = gi.make_tensor(91, gi.T_V, (B, Lmax, Hkv, 64), 1.0, dtype)
    kc, vc = dev_tensor(cache, device), dev_tensor(vcache, device)
    k0, v0 = bits(kc), bits(vc)
    # the oracle's default table passed explicitly (the other cases take the library's own: inv_freq NULL)
    inv = R.default_inv_freq(64)
    qo = gq.rope_append(dev_tensor(q, device), dev_tensor(k, device), dev_tensor(v, device), dev_i32(seqlens, device),
                        (kc, vc), inv_freq=dev_f32(inv, device), pairing=pairing)
    torch.cuda.synchronize()
    q_ref, kc_ref, vc_ref = R.rope_append_ref(q.f64, k.f64, v.f64, seqlens, inv, cache.f64, vcache.f64,
                                              R.CACHE_CONTIGUOUS, cache_len=Lmax, pairing=pairing)
    close_to_dtype(to_f64(qo), q_ref, dtype, "q")
    got_k, got_v = to_f64(kc), to_f64(vc)
    k1, v1 = bits(kc), bits(vc)
    for b in range(B):
        p = int(seqlens[b]) - 1
        if p < Lmax:
            close_to_dtype(got_k[b, p], kc_ref[b, p], dtype, f"k row b={b} p={p}")
            assert np.array_equal(v1[b, p], bits(dev_tensor(v, device))[b]), "v row copied bit for bit"
        keep = np.ones(Lmax, dtype=bool)
        if p < Lmax:
            keep[p] = False
        assert np.array_equal(k1[b, keep], k0[b, keep]) and np.array_equal(v1[b, keep], v0[b, keep]), b


@pytest.mark.parametrize("dtype,pairing", [("bf16", 0), ("bf16", 1), ("fp32", 0)])
def test_rope_chunks_paged(device, dtype, pairing):
    r = gi.varlen_problem(92, [40, 600, 131072, 17], [40, 100, 64, 1], 64, 8, block_size=16, dtype=dtype,
                          maxblk=8192)
    say(f"rope chunks paged {dtype} pairing={pairing} (positions to 131071)")
    T = int(r.cu_seqlens_q[-1])
    q, k, v = make_rows(93, T, 64, 8, dtype)
    kc, vc = dev_tensor(r.k, device), dev_tensor(r.v, device)
    qo = gq.rope_append(dev_tensor(q, device), dev_tensor(k, device), dev_tensor(v, device),
                        dev_i32(r.seqlens_k, device), (kc, vc), cu_seqlens_q=dev_i32(r.cu_seqlens_q, device),
                        pairing=pairing, block_table=dev_i32(r.block_table, device))
    torch.cuda.synchronize()
    inv = R.default_inv_freq(64)
    q_ref, kc_ref, vc_ref = R.rope_append_ref(q.f64, k.f64, v.f64, r.seqlens_k, inv, r.k.f64, r.v.f64,
                                              R.CACHE_PAGED, cu_seqlens_q=r.cu_seqlens_q,
                                              block_table=r.block_table, block_size=16, pairing=pairing)
    close_to_dtype(to_f64(qo), q_ref, dtype, "q")
    seq, pos = R.new_positions(r.seqlens_k, r.cu_seqlens_q)
    got_k, got_v = to_f64(kc), to_f64(vc)
    for rr in range(T):
        b, p = int(seq[rr]), int(pos[rr])
        blk, slot = int(r.block_table[b][p // 16]), p % 16
        close_to_dtype(got_k[blk, slot], kc_ref[blk, slot], dtype, f"k row {rr}")
        assert np.array_equal(got_v[blk, slot], vc_ref[blk, slot])


def test_rope_ring_in_place_custom_table(device):
    # ring cache, queries rotated in place, a non-default table and cos/sin scale
    B, W = 5, 16
    seqlens = np.array([1, 16, 17, 40, 131072], dtype=np.int32)
    say("rope ring in place, custom table, mscale 1.1")
    q, k, v = make_rows(94, B, 64, 8, "bf16")
    ring_k = gi.make_tensor(95, gi.T_K, (B, W, 8, 64), 1.0, "bf16")
    ring_v = gi.make_tensor(95, gi.T_V, (B, W, 8, 64), 1.0, "bf16")
    kr, vr = dev_tensor(ring_k, device), dev_tensor(ring_v, device)
    inv = (R.default_inv_freq(64, base=500000.0) * np.float32(0.25)).astype(np.float32)
    qd = dev_tensor(q, device)
    out = gq.rope_append(qd, dev_tensor(k, device), dev_tensor(v, device), dev_i32(seqlens, device), (kr, vr),
                         inv_freq=dev_f32(inv, device), q_out=qd, mscale=1.1, ring=True)
    torch.cuda.synchronize()
    assert out.data_ptr() == qd.data_ptr()
    q_ref, kr_ref, vr_ref = R.rope_append_ref(q.f64, k.f64, v.f64, seqlens, inv, ring_k.f64, ring_v.f64, R.CACHE_RING,
                                              cache_len=W, mscale=1.1)
    close_to_dtype(to_f64(qd), q_ref, "bf16", "q in place")
    close_to_dtype(to_f64(kr), kr_ref, "bf16", "ring k")
    assert np.array_equal(to_f64(vr), vr_ref)


def test_rope_then_decode_end_to_end(device):
    # a decode step: rotate the new token, append it, attend; against the oracle doing the same in fp64
    B, Lmax, Hq, Hkv = 4, 700, 64, 8
    seqlens = np.array([1, 2, 513, 700], dtype=np.int32)
    say("rope append then decode, contiguous cache")
    d = gi.decode_problem(96, B, Lmax, Hq, Hkv, 64, dtype="bf16", seqlens=seqlens)
    q, k, v = make_rows(97, B, Hq, Hkv, "bf16")
    kc, vc = dev_tensor(d.k, device), dev_tensor(d.v, device)
    qo = gq.rope_append(dev_tensor(q, device), dev_tensor(k, device), dev_tensor(v, device), dev_i32(seqlens, device),
                        (kc, vc))
    out = gq.attn_decode(qo, (kc, vc), dev_i32(seqlens, device), dev_f32(d.sinks, device), window=128)
    torch.cuda.synchronize()
    inv = R.default_inv_freq(64)
    q_ref, kc_ref, vc_ref = R.rope_append_ref(q.f64, k.f64, v.f64, seqlens, inv, d.k.f64, d.v.f64,
                                              R.CACHE_CONTIGUOUS, cache_len=Lmax)
    o_ref, _ = oracle.decode_ref(q_ref, kc_ref, vc_ref, seqlens, d.sinks, 128, d.scale)
    assert_bf16_close(to_f64(out), o_ref, "decode after rope append")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rope_default_table_is_the_oracles(device, dtype):
    # inv_freq=None: the library forms θ_i = 10000^(-2i/64) itself; the results equal those
    # of the oracle's fp32 table passed explicitly, bit for bit, out to position 131071
    B, Lmax = 4, 64
    seqlens = np.array([1, 4097, 65536, 131072], dtype=np.int32)
    say(f"rope default table vs explicit oracle table {dtype}")
    q, k, v = make_rows(98, B, 64, 8, dtype)
    outs = []
    for table in (None, dev_f32(R.default_inv_freq(64), device)):
        ring_k = torch.zeros((B, Lmax, 8, 64), dtype=dev_tensor(q, device).dtype, device=device)
        ring_v = torch.zeros_like(ring_k)
        qo = gq.rope_append(dev_tensor(q, device), dev_tensor(k, device), dev_tensor(v, device),
                            dev_i32(seqlens, device), (ring_k, ring_v), inv_freq=table, ring=True)
        torch.cuda.synchronize()
        outs.append((bits(qo), bits(ring_k)))
    assert np.array_equal(outs[0][0], outs[1][0]), "queries"
    assert np.array_equal(outs[0][1], outs[1][1]), "keys"
