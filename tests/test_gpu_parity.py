"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 oracle.

Every input is seeded and synthetic (``gqa_inputs``) and goes bit-identical to
both sides.  Small cases span several tiles and a ragged tail and are compared
element by element; the full-size workloads are compared on sampled rows that
the oracle computes one by one, plus properties that hold at any size.
"""
import math
import os

import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
import oracle
from gpu_helpers import (assert_bf16_close, assert_fp32_close, assert_lse_close, dev_f32, dev_i32, dev_tensor, say,
                         to_f64)

pytestmark = pytest.mark.gpu

SQRT_HALF = 1.0 / math.sqrt(2.0)


def sinks_dev(p, kind, device):
    return None if kind == "none" else dev_f32(p.sinks, device)


# ----------------------------------------------------------------------------- prefill, bf16

PREFILL_CASES = [
    # B, S, Hq, Hkv, window, sink kind
    (1, 1, 64, 8, 0, "normal"),
    (1, 7, 64, 8, 0, "normal"),
    (2, 100, 64, 8, 0, "normal"),
    (1, 257, 64, 8, 0, "none"),
    (1, 257, 64, 8, 128, "normal"),
    (2, 200, 64, 8, 16, "zero"),
    (1, 130, 64, 8, 1, "normal"),
    (1, 333, 64, 8, 300, "normal"),
    (1, 96, 8, 8, 0, "normal"),
    (1, 150, 16, 4, 0, "normal"),
    (1, 150, 24, 8, 33, "normal"),
    (1, 77, 32, 2, 0, "normal"),
    (1, 300, 8, 1, 64, "normal"),
    (3, 65, 64, 8, 0, "normal"),
    (1, 333, 64, 4, 128, "normal"),  # G = 16, windowed: two tile groups per workgroup
    (1, 190, 32, 1, 100, "none"),    # G = 32, windowed, no sink
]


@pytest.mark.parametrize("B,S,Hq,Hkv,W,sk", PREFILL_CASES)
def test_prefill_bf16_small(device, B, S, Hq, Hkv, W, sk):
    cfg = 1000 + B * 7 + S * 13 + Hq * 17 + Hkv * 19 + W
    p = gi.prefill_problem(cfg, B, S, Hq, Hkv, 64, "bf16", std=SQRT_HALF, sink_kind=sk)
    say(f"prefill bf16 B={B} S={S} Hq={Hq} Hkv={Hkv} W={W} sink={sk}")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               sinks_dev(p, sk, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, p.scale)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


@pytest.mark.parametrize("B,S,Hq,Hkv,W", [(1, 257, 64, 8, 128), (2, 200, 64, 8, 16), (1, 333, 64, 4, 128),
                                        (1, 4096, 64, 8, 128)])
def test_prefill_two_step_equals_one_step(device, monkeypatch, B, S, Hq, Hkv, W):
    # windowed whole-sequence layers run two tile groups per workgroup over the
    # same key tiles; the result is the one-group-per-workgroup kernel's, bit for bit
    p = gi.prefill_problem(2100 + S + W, B, S, Hq, Hkv, 64, "bf16", std=SQRT_HALF)
    args = (dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device), dev_f32(p.sinks, device))
    say(f"prefill two tile groups per workgroup vs one: B={B} S={S} Hq={Hq} Hkv={Hkv} W={W}")
    res = {}
    for flag in ("0", "1"):
        monkeypatch.setenv("GQA_PREFILL_TWO_STEP", flag)
        res[flag] = gq.attn_prefill(*args, window=W, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(res["0"][0], res["1"][0]) and torch.equal(res["0"][1], res["1"][1])


def test_prefill_two_step_random_shapes(device, monkeypatch):
    # two tile groups per workgroup forced on every windowed layer: where the job's
    # key tiles fit the three LDS buffers (windows up to 128, G = 8, 16, 32) the
    # second step reuses them, elsewhere it streams them again; either way the
    # result is the one-group kernel's, bit for bit
    rng = np.random.default_rng(2200)
    for case in range(16):
        G = int(rng.choice([8, 16, 32] if case < 10 else [1, 3, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        B = int(rng.integers(1, 3))
        S = int(rng.integers(1, 700))
        W = int(rng.integers(1, 129 if case < 10 else 400))
        p = gi.prefill_problem(2200 + case, B, S, G * Hkv, Hkv, 64, "bf16", std=SQRT_HALF)
        args = (dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device), dev_f32(p.sinks, device))
        say(f"two-step random case {case}: B={B} S={S} G={G} Hkv={Hkv} W={W}")
        res = {}
        for flag in ("0", "2"):
            monkeypatch.setenv("GQA_PREFILL_TWO_STEP", flag)
            res[flag] = gq.attn_prefill(*args, window=W, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(res["0"][0], res["2"][0]) and torch.equal(res["0"][1], res["2"][1]), (B, S, G, Hkv, W)


def test_prefill_bf16_window_covering_sequence_equals_dense(device):
    p = gi.prefill_problem(2001, 1, 200, 64, 8, 64, "bf16", std=SQRT_HALF)
    args = (dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device), dev_f32(p.sinks, device))
    say("prefill bf16 window >= S vs dense")
    o0 = gq.attn_prefill(*args, window=0)
    o1 = gq.attn_prefill(*args, window=200)
    o2 = gq.attn_prefill(*args, window=5000)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(o0, o2)


def test_prefill_bf16_deterministic(device):
    p = gi.prefill_problem(2002, 1, 600, 64, 8, 64, "bf16", std=SQRT_HALF)
    args = (dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device), dev_f32(p.sinks, device))
    say("prefill bf16 repeatability")
    outs = [gq.attn_prefill(*args, window=w) for w in (0, 0, 0, 128, 128)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]) and torch.equal(outs[3], outs[4])


def test_prefill_empty(device):
    q = torch.empty((0, 16, 64, 64), dtype=torch.bfloat16, device=device)
    k = torch.empty((0, 16, 8, 64), dtype=torch.bfloat16, device=device)
    say("prefill empty batch")
    out = gq.attn_prefill(q, k, k.clone(), None)
    assert out.shape == q.shape


def sample_rows(S, W, rng, n_rand=48):
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, S // 2, S - 65, S - 64, S - 33, S - 32, S - 1]
    if W > 0:
        edges += [W - 1, W, W + 1, 2 * W]
    rows = set(r for r in edges if 0 <= r < S)
    rows |= set(range(min(16, S)))
    rows |= set(range(max(0, S - 16), S))
    rows |= set(int(r) for r in rng.integers(0, S, size=n_rand))
    return np.array(sorted(rows))


@pytest.mark.parametrize("W", [0, 128])
def test_prefill_layer_shaped_sampled(device, W):
    """B1 S4096 64/8 heads bf16 N(0,1)/sqrt2 (the layer-shaped workload), dense then window 128."""
    p = gi.c2_layer()
    say(f"prefill layer-shaped S4096 W={W}")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               dev_f32(p.sinks, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.isfinite(got).all()
    # convexity bound at every row: |o| <= max |v| over the group's values
    vmax = np.abs(p.v.f64).max()
    assert np.abs(got).max() <= vmax + 1e-2
    rows = sample_rows(4096, W, np.random.default_rng(W))
    o_ref, l_ref = oracle.prefill_rows_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, p.scale, rows=rows)
    assert_bf16_close(got[:, rows], o_ref, "sampled rows")
    assert_lse_close(to_f64(lse)[:, :, rows], l_ref, "sampled lse")


# ----------------------------------------------------------------------------- fp32 path

@pytest.mark.parametrize("W", [0, 128])
def test_prefill_fp32_tiny(device, W):
    """B1 S256 8/2 heads fp32 N(0,1), scale 1/8 (the tiny fp32 workload), dense and window 128."""
    p = gi.c1_tiny()
    say(f"prefill fp32 tiny W={W}")
    out, lse = gq.attn_prefill(dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device),
                               dev_f32(p.sinks, device), window=W, scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.prefill_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, 0.125)
    assert_fp32_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse", fp32=True)


def test_decode_fp32(device):
    p = gi.decode_problem(3001, 3, 400, 16, 4, 64, "fp32", seqlens=[400, 1, 237])
    say("decode fp32")
    for W in (0, 100):
        out, lse = gq.attn_decode(dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                                  dev_i32(p.seqlens, device), dev_f32(p.sinks, device), window=W, return_lse=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.decode_ref(p.q.f64, p.k.f64, p.v.f64, p.seqlens, p.sinks, W, p.scale)
        assert_fp32_close(to_f64(out), o_ref, f"decode fp32 W={W}")
        assert_lse_close(to_f64(lse), l_ref, "lse", fp32=True)


def test_varlen_fp32(device):
    p = gi.varlen_problem(3002, [40, 7, 130], [40, 1, 20], 8, 2, 64, block_size=16, dtype="fp32")
    say("varlen fp32")
    for W in (0, 16):
        out, lse = run_varlen(p, device, W)
        o_ref, l_ref = oracle.varlen_ref(p.q.f64, p.k.f64, p.v.f64, p.cu_seqlens_q, p.seqlens_k, p.sinks, W, p.scale,
                                         block_table=p.block_table, block_size=p.block_size)
        assert_fp32_close(to_f64(out), o_ref, f"varlen fp32 W={W}")
        assert_lse_close(to_f64(lse), l_ref, "lse", fp32=True)


# ----------------------------------------------------------------------------- decode, bf16

DECODE_CASES = [
    # B, Lmax, Hq, Hkv, window, seqlens
    (4, 100, 64, 8, 0, "full"),
    (5, 300, 64, 8, 0, "random"),
    (3, 1, 64, 8, 0, "full"),
    (6, 1000, 64, 8, 128, "random"),
    (2, 700, 8, 8, 0, "random"),
    (2, 513, 32, 2, 0, "random"),
    (2, 2000, 48, 1, 0, "random"),
    (1, 5000, 64, 8, 0, "full"),
    (1, 5000, 64, 8, 128, "full"),
    (3, 4097, 64, 8, 1, "random"),
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,W,sl", DECODE_CASES)
def test_decode_bf16_small(device, B, Lmax, Hq, Hkv, W, sl):
    cfg = 4000 + B * 7 + Lmax * 13 + Hq * 17 + Hkv + W
    p = gi.decode_problem(cfg, B, Lmax, Hq, Hkv, 64, "bf16", seqlens=None if sl == "full" else "random")
    say(f"decode bf16 B={B} Lmax={Lmax} Hq={Hq} Hkv={Hkv} W={W} seqlens={sl}")
    out, lse = gq.attn_decode(dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                              dev_i32(p.seqlens, device), dev_f32(p.sinks, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_ref(p.q.f64, p.k.f64, p.v.f64, p.seqlens, p.sinks, W, p.scale)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


def test_decode_split_counts_agree(device, monkeypatch):
    """The split-K count changes only rounding: 1, 3, 8 and 64 splits all match the oracle."""
    p = gi.decode_problem(4100, 2, 6000, 64, 8, 64, "bf16", seqlens=[6000, 3333])
    args = (dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)), dev_i32(p.seqlens, device),
            dev_f32(p.sinks, device))
    o_ref, _ = oracle.decode_ref(p.q.f64, p.k.f64, p.v.f64, p.seqlens, p.sinks, 0, p.scale)
    outs = []
    for n in ("1", "3", "8", "64"):
        monkeypatch.setenv("GQA_DECODE_SPLITS", n)
        say(f"decode forced splits={n}")
        outs.append(gq.attn_decode(*args))
        torch.cuda.synchronize()
        assert_bf16_close(to_f64(outs[-1]), o_ref, f"splits={n}")
    monkeypatch.delenv("GQA_DECODE_SPLITS")


ROWS_CASES = [
    # B, Lmax, Hq, window, sink tokens, seqlens, forced splits (None: the plan's)
    (4, 100, 64, 0, 0, "full", None),        # one split: the workgroup finishes the rows itself
    (3, 1, 64, 0, 0, "full", None),          # one position: an odd tile count, the pair's second tile masked
    (5, 300, 64, 0, 0, "random", None),
    (6, 1000, 64, 128, 0, "random", None),   # window: only the last 128 positions
    (6, 1000, 64, 128, 4, "random", 3),      # window plus sink tokens, over three splits
    (2, 700, 32, 0, 0, "random", 2),         # 4 query heads per KV head: half the columns idle
    (2, 6000, 64, 0, 0, [6000, 3333], 64),   # splits past the shorter sequence are empty
    (3, 4097, 64, 1, 0, "random", None),     # window 1
    (4, 2500, 64, 0, 0, "random", 5),
]


@pytest.mark.parametrize("B,Lmax,Hq,W,n,sl,splits", ROWS_CASES)
def test_decode_rows_form(device, monkeypatch, B, Lmax, Hq, W, n, sl, splits):
    """The whole-row decode form (8 KV heads, every head of a position in one
    workgroup), forced on for small shapes it would not pick by itself."""
    monkeypatch.setenv("GQA_DECODE_ROWS", "2")
    if splits:
        monkeypatch.setenv("GQA_DECODE_SPLITS", str(splits))
    cfg = 4300 + B * 7 + Lmax * 13 + Hq + W + n
    p = gi.decode_problem(cfg, B, Lmax, Hq, 8, 64, "bf16", seqlens=None if sl == "full" else sl)
    say(f"decode rows form B={B} Lmax={Lmax} Hq={Hq} W={W} n={n} seqlens={sl} splits={splits}")
    out, lse = gq.attn_decode(dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                              dev_i32(p.seqlens, device), dev_f32(p.sinks, device), window=W, sink_tokens=n,
                              return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_ref(p.q.f64, p.k.f64, p.v.f64, p.seqlens, p.sinks, W, p.scale, sink_tokens=n)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


def test_decode_is_last_prefill_row(device):
    p = gi.prefill_problem(4200, 2, 300, 64, 8, 64, "bf16", std=SQRT_HALF)
    q, k, v = dev_tensor(p.q, device), dev_tensor(p.k, device), dev_tensor(p.v, device)
    s = dev_f32(p.sinks, device)
    for W in (0, 128):
        say(f"decode vs last prefill row W={W}")
        op = gq.attn_prefill(q, k, v, s, window=W)
        od = gq.attn_decode(q[:, -1].contiguous(), (k, v), dev_i32([300, 300], device), s, window=W)
        torch.cuda.synchronize()
        o_ref, _ = oracle.prefill_rows_ref(p.q.f64, p.k.f64, p.v.f64, p.sinks, W, p.scale, rows=[299])
        assert_bf16_close(to_f64(od), o_ref[:, 0], "decode")
        assert_bf16_close(to_f64(op[:, -1]), o_ref[:, 0], "prefill last row")


@pytest.mark.parametrize("W,rows", [(0, "1"), (128, "1"), (0, "0")])
def test_decode_batched_full(device, monkeypatch, W, rows):
    """B64 cache 8192 64/8 heads bf16 N(0,1) (the batched-decode workload), every sequence checked; the
    plan's own form (whole rows on the dense layer) and the per-head form."""
    monkeypatch.setenv("GQA_DECODE_ROWS", rows)
    p = gi.c3_decode()
    say(f"decode batched B64 L8192 W={W} rows={rows}")
    out, lse = gq.attn_decode(dev_tensor(p.q, device), (dev_tensor(p.k, device), dev_tensor(p.v, device)),
                              dev_i32(p.seqlens, device), dev_f32(p.sinks, device), window=W, return_lse=True)
    torch.cuda.synchronize()
    got, got_l = to_f64(out), to_f64(lse)
    for b0 in range(0, 64, 16):
        sl = slice(b0, b0 + 16)
        o_ref, l_ref = oracle.decode_ref(gi.bf16_to_f64(p.q.store[sl]), gi.bf16_to_f64(p.k.store[sl]),
                                         gi.bf16_to_f64(p.v.store[sl]), p.seqlens[sl], p.sinks, W, p.scale)
        assert_bf16_close(got[sl], o_ref, f"batch {b0}")
        assert_lse_close(got_l[sl], l_ref, "lse")


# ----------------------------------------------------------------------------- varlen / paged

def run_varlen(p, device, W, packed=False, table=None):
    q = dev_tensor(p.q, device)
    if packed:
        # packed caches: gather each sequence's rows contiguously
        ks, vs, cu = [], [], [0]
        for b in range(len(p.seqlens_k)):
            L = int(p.seqlens_k[b])
            ks.append(oracle.gather_paged(p.k.store, p.block_table[b], p.block_size, L))
            vs.append(oracle.gather_paged(p.v.store, p.block_table[b], p.block_size, L))
            cu.append(cu[-1] + L)
        kc = gi.Tensor(np.concatenate(ks), p.k.dtype)
        vc = gi.Tensor(np.concatenate(vs), p.v.dtype)
        return gq.attn_varlen_paged(q, (dev_tensor(kc, device), dev_tensor(vc, device)), None,
                                    dev_i32(p.cu_seqlens_q, device), dev_i32(p.seqlens_k, device),
                                    dev_f32(p.sinks, device), window=W, max_q_len=p.max_q_len,
                                    max_kv_len=int(max(p.seqlens_k)), cu_seqlens_k=dev_i32(cu, device),
                                    return_lse=True)
    bt = p.block_table if table is None else table
    res = gq.attn_varlen_paged(q, (dev_tensor(p.k, device), dev_tensor(p.v, device)), dev_i32(bt, device),
                               dev_i32(p.cu_seqlens_q, device), dev_i32(p.seqlens_k, device),
                               dev_f32(p.sinks, device), window=W, max_q_len=p.max_q_len, max_kv_len=p.max_kv_len,
                               return_lse=True)
    torch.cuda.synchronize()
    return res


VARLEN_CASES = [
    # kv_lens, q_lens, block_size, window
    ([13, 1, 70, 300, 64, 129], [5, 1, 70, 1, 33, 2], 16, 0),
    ([13, 1, 70, 300, 64, 129], [5, 1, 70, 1, 33, 2], 16, 7),
    ([500, 40, 1000, 17], [1, 40, 1, 17], 16, 128),
    ([257, 3000, 1, 99], [257, 1, 1, 0], 64, 0),
    ([100, 200], [37, 1], 1, 0),
    ([2048, 4096, 700], [512, 1, 512], 16, 128),
]


@pytest.mark.parametrize("kv,ql,bs,W", VARLEN_CASES)
def test_varlen_paged_small(device, kv, ql, bs, W):
    p = gi.varlen_problem(5000 + sum(kv) + bs + W, kv, ql, 64, 8, 64, block_size=bs, dtype="bf16", spare_blocks=3)
    say(f"varlen paged kv={kv} q={ql} bs={bs} W={W}")
    out, lse = run_varlen(p, device, W)
    o_ref, l_ref = oracle.varlen_ref(p.q.f64, p.k.f64, p.v.f64, p.cu_seqlens_q, p.seqlens_k, p.sinks, W, p.scale,
                                     block_table=p.block_table, block_size=p.block_size)
    assert_bf16_close(to_f64(out), o_ref, "out")
    assert_lse_close(to_f64(lse), l_ref, "lse")


def test_varlen_packed_and_permutation(device):
    """Packed caches, and a paged cache under a different block permutation, give
    the very same bits as the paged run."""
    kv, ql = [13, 1, 70, 300, 64, 129], [5, 1, 70, 1, 33, 2]
    p = gi.varlen_problem(5100, kv, ql, 64, 8, 64, block_size=16, dtype="bf16")
    say("varlen packed vs paged")
    out_p, _ = run_varlen(p, device, 0)
    out_k, _ = run_varlen(p, device, 0, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_k)
    # move every block to a new physical slot
    perm = np.random.default_rng(1).permutation(p.k.shape[0]).astype(np.int32)
    inv = np.argsort(perm).astype(np.int32)
    k2 = gi.Tensor(p.k.store[inv], p.k.dtype)
    v2 = gi.Tensor(p.v.store[inv], p.v.dtype)
    t2 = np.where(p.block_table >= 0, perm[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    p2 = gi.Varlen(p.q, k2, v2, p.cu_seqlens_q, p.seqlens_k, t2, p.block_size, p.sinks, p.scale, p.q_lens)
    out_2, _ = run_varlen(p2, device, 0)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_2)


@pytest.mark.parametrize("W", [0, 128])
def test_varlen_longest_first_equals_batch_order(device, monkeypatch, W):
    # ragged batches are dispatched longest sequence first; the batch order
    # computes the same jobs, so the bits agree
    p = gi.c5_ragged()
    say(f"varlen longest-first vs batch order W={W}")
    monkeypatch.setenv("GQA_VARLEN_SORT", "0")
    o0, l0 = run_varlen(p, device, W)
    monkeypatch.setenv("GQA_VARLEN_SORT", "1")
    o1, l1 = run_varlen(p, device, W)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("W", [0, 128])
def test_varlen_ragged_paged_sampled(device, W):
    """16 sequences, lengths U{128..8192}, 512-token chunks and decode steps, 16-token
    blocks under a permuted table (the ragged + paged workload)."""
    p = gi.c5_ragged()
    say(f"varlen ragged paged 16 seqs W={W}")
    out, lse = run_varlen(p, device, W)
    got = to_f64(out)
    assert np.isfinite(got).all()
    rows = []
    cu = p.cu_seqlens_q
    rng = np.random.default_rng(7 + W)
    for b in range(16):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        n = r1 - r0
        pick = set(range(r0, min(r1, r0 + 8))) | set(range(max(r0, r1 - 8), r1))
        if n > 16:
            pick |= set(int(x) for x in rng.integers(r0, r1, size=8))
        rows += sorted(pick)
    o_ref, l_ref = oracle.varlen_ref(p.q.f64, p.k.f64, p.v.f64, cu, p.seqlens_k, p.sinks, W, p.scale,
                                     block_table=p.block_table, block_size=p.block_size, rows=rows)
    assert_bf16_close(got[rows], o_ref[rows], "sampled rows")
    assert_lse_close(to_f64(lse)[:, rows], l_ref[:, rows], "lse")
