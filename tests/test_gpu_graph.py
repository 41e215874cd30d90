"""The decode path captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI).

A serving loop replays one decode step per token; the library allocates
nothing and never synchronises, so its calls can be captured.  Captured: the
one-launch decode step of a windowed layer (rotate, append, attend) and the
allocation-free dense decode.  The graph is replayed several times with the
program's own eager work and synchronisations between the replays, and every
replay is compared bit for bit with the eager calls (the kernels are
deterministic), and the step's output with the oracle.
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


def test_decode_step_and_noalloc_decode_in_a_graph():
    B, Hq, Hkv, Lc = 8, 64, 8, 1024
    seqlens_np = np.array([1, 2, 127, 128, 129, 600, 1000, 1024], dtype=np.int32)
    q = gi.make_tensor(120, gi.T_Q, (B, Hq, 64), 1.0, "bf16")
    kn = gi.make_tensor(120, gi.T_K, (B, Hkv, 64), 1.0, "bf16")
    vn = gi.make_tensor(120, gi.T_V, (B, Hkv, 64), 1.0, "bf16")
    kc0 = gi.make_tensor(121, gi.T_K, (B, Lc, Hkv, 64), 1.0, "bf16")
    vc0 = gi.make_tensor(121, gi.T_V, (B, Lc, Hkv, 64), 1.0, "bf16")
    sinks_np = gi.make_sinks(120, Hq)
    d = gi.decode_problem(122, B, 4096, Hq, Hkv, seqlens=[4096, 1, 3000, 77, 4096, 2048, 5, 1000])
    qd, kd, vd = dev_tensor(d.q, "cuda"), dev_tensor(d.k, "cuda"), dev_tensor(d.v, "cuda")
    sld = dev_i32(d.seqlens, "cuda")
    qs, kns, vns = dev_tensor(q, "cuda"), dev_tensor(kn, "cuda"), dev_tensor(vn, "cuda")
    sl = dev_i32(seqlens_np, "cuda")
    sinks = dev_f32(sinks_np, "cuda")

    # eager reference, on its own copy of the cache
    kc_e, vc_e = dev_tensor(kc0, "cuda"), dev_tensor(vc0, "cuda")
    say("graph: eager decode step and allocation-free decode")
    o_step_e = gq.attn_decode_step(qs, kns, vns, sl, (kc_e, vc_e), sinks, window=128)
    o_dec_e = gq.attn_decode_noalloc(qd, (kd, vd), sld, sinks, window=0)
    torch.cuda.synchronize()

    # static buffers of the captured calls
    kc, vc = dev_tensor(kc0, "cuda"), dev_tensor(vc0, "cuda")
    o_step = torch.empty_like(qs)
    o_dec = torch.empty_like(qd)

    def calls():
        gq.attn_decode_step(qs, kns, vns, sl, (kc, vc), sinks, window=128, out=o_step)
        gq.attn_decode_noalloc(qd, (kd, vd), sld, sinks, window=0, out=o_dec)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (the step's append is idempotent)
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        o_step.fill_(0)
        o_dec.fill_(0)
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_step.view(torch.int16), o_step_e.view(torch.int16)), f"replay {rep}: decode step"
        assert torch.equal(o_dec.view(torch.int16), o_dec_e.view(torch.int16)), f"replay {rep}: decode"
        assert torch.equal(kc.view(torch.int16), kc_e.view(torch.int16)), f"replay {rep}: cache"
    # and the captured step against the oracle composition
    q_ref, kc_ref, vc_ref = R.rope_append_ref(q.f64, kn.f64, vn.f64, seqlens_np, R.default_inv_freq(64), kc0.f64,
                                              vc0.f64, R.CACHE_CONTIGUOUS, cache_len=Lc)
    o_ref, _ = oracle.decode_ref(q_ref, kc_ref, vc_ref, seqlens_np, sinks_np, 128, 1.0 / 8.0)
    assert_bf16_close(to_f64(o_step), o_ref, "graph-replayed decode step vs oracle")


def test_mixed_varlen_call_in_a_graph():
    # A ragged batch of prefill chunks and decode rows (a prefill launch and a
    # decode launch) captured as one graph.
    kv, ql = [300, 1, 700, 129, 2000, 1, 64, 5], [64, 1, 100, 1, 33, 1, 64, 5]
    p = gi.varlen_problem(130, kv, ql, 64, 8, 64, block_size=16, dtype="bf16")
    q = dev_tensor(p.q, "cuda")
    cache = (dev_tensor(p.k, "cuda"), dev_tensor(p.v, "cuda"))
    bt, cu, sk = dev_i32(p.block_table, "cuda"), dev_i32(p.cu_seqlens_q, "cuda"), dev_i32(p.seqlens_k, "cuda")
    sinks = dev_f32(p.sinks, "cuda")
    B = len(kv)
    ws = torch.empty((gq.varlen_workspace_size(B, p.max_q_len, p.max_kv_len, 64, 8),), dtype=torch.uint8,
                     device="cuda")

    def call(out):
        return gq.attn_varlen_paged(q, cache, bt, cu, sk, sinks, window=0, max_q_len=p.max_q_len,
                                    max_kv_len=p.max_kv_len, workspace=ws, out=out)

    say("graph: mixed varlen eager")
    o_eager = call(torch.empty_like(q))
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: mixed varlen capture")
    with torch.cuda.graph(g):
        call(o)
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(0)
        torch.cuda.synchronize()
        say(f"graph: mixed varlen replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_eager.view(torch.int16)), f"replay {rep}"
    o_ref, _ = oracle.varlen_ref(p.q.f64, p.k.f64, p.v.f64, p.cu_seqlens_q, p.seqlens_k, p.sinks, 0, p.scale,
                                 block_table=p.block_table, block_size=p.block_size)
    assert_bf16_close(to_f64(o), o_ref, "graph-replayed mixed varlen vs oracle")
