"""GPU parity of the prefill backward (dq, dk, dv, dsinks) through the C ABI,
against the fp64 gradient oracle (``oracle.backward``).

The backward takes the forward's output and log-sum-exp from the GPU forward,
as a training step would; the oracle differentiates the exact definition on
the same bf16 input values.  Covered: several tiles with ragged tails, group
sizes 1, 3, 4, 8 and 16 (odd groups leave a head pair half empty), windows
1 .. 128 with and without sink tokens, sinks normal / absent / zero / NULL, a
sequence shorter than a tile, the layer-shaped S4096 64/8 workload (dense and
window 128, two KV heads' worth of outputs against the full oracle), the fp32
path, determinism, and window >= S equal to dense.
"""
import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle.backward as BW
from gpu_helpers import assert_dsinks_close, assert_grad_close, dev_f32, dev_tensor, say, to_f64

pytestmark = pytest.mark.gpu


def run_backward(p, dout, device, window, sink_tokens, sinks_null=False):
    q, k, v = dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device)
    sinks = None if sinks_null else dev_f32(p.sinks, device)
    out, lse = gq.attn_prefill(q, k, v, sinks, window=window, sink_tokens=sink_tokens, return_lse=True)
    g = gq.attn_prefill_backward(q, k, v, sinks, out, lse, dev_tensor(dout, device), window=window,
                                 sink_tokens=sink_tokens)
    torch.cuda.synchronize()
    return g


def check(g, ref, what, fp32=False, heads=None, kv=None):
    dq, dk, dv, ds = (to_f64(t) for t in g)
    rq, rk, rv, rs, ra = ref
    if heads is not None:
        dq, rq, ds, rs, ra = dq[:, :, heads], rq[:, :, heads], ds[heads], rs[heads], ra[heads]
        dk, rk, dv, rv = dk[:, :, kv], rk[:, :, kv], dv[:, :, kv], rv[:, :, kv]
    assert_grad_close(dq, rq, f"{what} dq", fp32)
    assert_grad_close(dk, rk, f"{what} dk", fp32)
    assert_grad_close(dv, rv, f"{what} dv", fp32)
    if ra.max() > 0:
        assert_dsinks_close(ds, rs, ra, f"{what} dsinks", fp32)
    else:
        assert not ds.any(), f"{what}: dsinks must be zero without a sink"


CASES = [  # B, S, Hq, Hkv, window, sink_tokens, sink kind
    (1, 200, 8, 1, 0, 0, "normal"),
    (2, 130, 8, 2, 0, 0, "normal"),
    (1, 300, 8, 8, 64, 0, "none"),      # G = 1: every head pair half empty
    (1, 257, 6, 2, 16, 0, "normal"),    # G = 3
    (1, 333, 16, 2, 33, 0, "zero"),
    (1, 250, 8, 1, 128, 4, "normal"),   # sink tokens
    (1, 190, 8, 2, 1, 3, "normal"),     # window 1 + sink tokens
    (1, 300, 8, 1, 64, 100, "normal"),  # sink tokens over more than one key block
    (1, 100, 16, 1, 0, 0, "normal"),    # G = 16
    (1, 64, 8, 1, 0, 0, "normal"),      # exactly one key block
    (1, 5, 8, 1, 0, 0, "normal"),       # shorter than a tile
]


@pytest.mark.parametrize("B,S,Hq,Hkv,W,n,kind", CASES)
def test_backward_small(device, B, S, Hq, Hkv, W, n, kind):
    say(f"backward B{B} S{S} {Hq}/{Hkv} W={W} sink_tokens={n} sinks={kind}")
    p = gi.prefill_problem(100 + S, B, S, Hq, Hkv, 64, dtype="bf16", sink_kind=kind)
    dout = gi.make_tensor(100 + S, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    g = run_backward(p, dout, device, W, n)
    ref = BW.prefill_grad_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, dout.f64, W, p.scale, n, dsink_abs=True)
    check(g, ref, "small")


def test_backward_null_sinks(device):
    say("backward without a sink argument (NULL): dsinks all zero")
    p = gi.prefill_problem(140, 1, 150, 8, 2, 64, dtype="bf16")
    dout = gi.make_tensor(140, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    g = run_backward(p, dout, device, 0, 0, sinks_null=True)
    ref = BW.prefill_grad_ref(p.q.f64, p.k.f64, p.v.f64, None, dout.f64, 0, p.scale, 0, dsink_abs=True)
    check(g, ref, "null sinks")


@pytest.mark.parametrize("W,kv", [(0, [0]), (128, [5])])
def test_backward_layer_shape(device, W, kv):
    p = gi.c2_layer()
    say(f"backward layer-shaped B1 S4096 64/8 W={W} (oracle on KV head {kv})")
    dout = gi.make_tensor(2, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    g = run_backward(p, dout, device, W, 0)
    ref = BW.prefill_grad_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, dout.f64, W, p.scale, 0, kv_heads=kv,
                               dsink_abs=True)
    heads = [h for h in range(64) if h // 8 in kv]
    check(g, ref, f"S4096 W{W}", heads=heads, kv=kv)


def test_backward_fp32_tiny(device):
    p = gi.c1_tiny("fp32")
    dout = gi.make_tensor(1, gi.T_DOUT, p.q.shape, 1.0, "fp32")
    for W, n in ((0, 0), (128, 0), (16, 5)):
        say(f"backward fp32 tiny B1 S256 8/2 W={W} sink_tokens={n}")
        g = run_backward(p, dout, device, W, n)
        ref = BW.prefill_grad_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, dout.f64, W, p.scale, n, dsink_abs=True)
        check(g, ref, f"fp32 W{W}", fp32=True)


def test_backward_deterministic_and_window_ge_length(device):
    say("backward determinism, window >= S equals dense")
    p = gi.prefill_problem(141, 1, 500, 64, 8, 64, dtype="bf16")
    dout = gi.make_tensor(141, gi.T_DOUT, p.q.shape, 1.0, "bf16")
    a = run_backward(p, dout, device, 0, 0)
    b = run_backward(p, dout, device, 0, 0)
    c = run_backward(p, dout, device, 500, 7)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y), "two runs differ"
        assert torch.equal(x, z), "window >= S differs from dense"
