"""The metadata-checking build (GQA_DEBUG, libgqa_attn_debug.so) on the GPU.

Metadata the kernels read from device memory cannot be validated on the host
without a synchronisation, so the kernels clamp it; the debug build also
records each kind of value it clamped.  Checked here: on valid metadata the
debug build records nothing and returns the release build's results bit for
bit; block ids, sequence lengths, query offsets and query counts out of range
are recorded by kind; every write stays inside the output (guard rows behind
it are untouched), results stay finite, and sequences whose own metadata is
valid get the same rows as in a call with all metadata valid.  The release
build, given the same metadata, stays inside its buffers too.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import attention_gqa_causal_amd as gq
import gqa_inputs as gi
from gpu_helpers import dev_f32, dev_i32, dev_tensor, say

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(gq.__file__), "libgqa_attn_debug.so")
GUARD = 3  # guard rows behind each output
SENTINEL = 12288.0  # exact in bf16


@pytest.fixture(scope="module")
def libs():
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} missing: python -m attention_gqa_causal_amd.build --debug")
    rel = gq.lib()
    dbg = ctypes.CDLL(DEBUG_LIB)
    for name, (res, args) in gq._SIGNATURES.items():
        fn = getattr(dbg, name)
        fn.restype = res
        fn.argtypes = args
    return rel, dbg


@pytest.fixture
def use(monkeypatch, libs):
    """use("release") / use("debug"): route the binding's calls to that library."""
    def _use(which):
        monkeypatch.setattr(gq, "_lib", libs[0] if which == "release" else libs[1])
    return _use


def guarded(rows, Hq, D, dtype=torch.bfloat16):
    """An output of `rows` rows with GUARD rows of a sentinel pattern behind it."""
    big = torch.full((rows + GUARD, Hq, D), SENTINEL, dtype=dtype, device="cuda")
    return big, big[:rows]


def assert_guard_intact(big, rows, what):
    tail = big[rows:].float()
    assert torch.all(tail == SENTINEL), f"{what}: write past the output"


def varlen_case(cfg=41):
    return gi.varlen_problem(cfg, [300, 40, 129, 77], [30, 1, 129, 5], 16, 4, 64, block_size=16, maxblk=24)


def run_varlen(p, W=0, table=None, cu=None, seqlens=None, max_q_len=None, max_kv_len=None):
    Tq = p.q.shape[0]
    big, out = guarded(Tq, p.q.shape[1], p.q.shape[2])
    o, lse = gq.attn_varlen_paged(
        dev_tensor(p.q, "cuda"), (dev_tensor(p.k, "cuda"), dev_tensor(p.v, "cuda")),
        dev_i32(p.block_table if table is None else table, "cuda"),
        dev_i32(p.cu_seqlens_q if cu is None else cu, "cuda"),
        dev_i32(p.seqlens_k if seqlens is None else seqlens, "cuda"),
        dev_f32(p.sinks, "cuda"), window=W,
        max_q_len=int(p.q_lens.max()) if max_q_len is None else max_q_len,
        max_kv_len=int(p.seqlens_k.max()) if max_kv_len is None else max_kv_len,
        out=out, return_lse=True)
    torch.cuda.synchronize()
    assert_guard_intact(big, Tq, "varlen")
    return o.clone(), lse.clone()


def seq_rows(p, b):
    return slice(int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1]))


@pytest.mark.parametrize("W", [0, 16])
def test_valid_metadata_records_nothing_and_matches_release(use, W):
    p = varlen_case()
    use("release")
    o_r, l_r = run_varlen(p, W)
    use("debug")
    gq.debug_flags(reset=True)
    o_d, l_d = run_varlen(p, W)
    flags = gq.debug_flags()
    say(f"valid varlen W={W}: flags {flags}")
    assert flags == 0
    assert torch.equal(o_r, o_d) and torch.equal(l_r, l_d)
    # batched prefill and decode too
    pp = gi.prefill_problem(42, 2, 200, 8, 2, 64)
    q, k, v, s = (dev_tensor(pp.q, "cuda"), dev_tensor(pp.k, "cuda"), dev_tensor(pp.v, "cuda"),
                  dev_f32(pp.sinks, "cuda"))
    a = gq.attn_prefill(q, k, v, s, window=W).clone()
    use("release")
    b = gq.attn_prefill(q, k, v, s, window=W).clone()
    assert torch.equal(a, b)
    use("debug")
    assert gq.debug_flags() == 0


def test_block_ids_out_of_range(use):
    p = varlen_case()
    use("release")
    o_ok, _ = run_varlen(p)
    bad = p.block_table.copy()
    n_blocks = p.k.shape[0]
    bad[0, 2] = n_blocks + 1000
    bad[2, 0] = -7
    use("debug")
    gq.debug_flags(reset=True)
    o, lse = run_varlen(p, table=bad)
    flags = gq.debug_flags()
    say(f"block ids out of range: flags {flags}")
    assert flags & gq.GQA_DBG_BLOCK_TABLE
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b in (1, 3):  # their own tables are valid
        assert torch.equal(o[seq_rows(p, b)], o_ok[seq_rows(p, b)])


def test_sequence_length_out_of_range(use):
    p = varlen_case()
    use("release")
    o_ok, _ = run_varlen(p)
    bad = p.seqlens_k.copy()
    bad[1] = p.block_table.shape[1] * p.block_size + 50  # past the table's capacity
    use("debug")
    gq.debug_flags(reset=True)
    o, _ = run_varlen(p, seqlens=bad)
    flags = gq.debug_flags()
    say(f"sequence length past capacity: flags {flags}")
    assert flags & gq.GQA_DBG_SEQLENS_K
    assert torch.isfinite(o.float()).all()
    for b in (0, 2, 3):
        assert torch.equal(o[seq_rows(p, b)], o_ok[seq_rows(p, b)])
    # a negative length: the sequence has no positions, so no query of it is computed
    bad = p.seqlens_k.copy()
    bad[3] = -5
    gq.debug_flags(reset=True)
    run_varlen(p, seqlens=bad)
    assert gq.debug_flags() & gq.GQA_DBG_SEQLENS_K


def test_query_offsets_out_of_range(use):
    p = varlen_case()
    use("release")
    o_ok, _ = run_varlen(p)
    Tq = p.q.shape[0]
    cu = p.cu_seqlens_q.copy()
    cu[-1] = Tq + 100      # the last sequence would run past the packed rows
    use("debug")
    gq.debug_flags(reset=True)
    o, _ = run_varlen(p, cu=cu, max_q_len=int(p.q_lens.max()) + 100)
    flags = gq.debug_flags()
    say(f"cu_seqlens_q past Tq: flags {flags}")
    assert flags & gq.GQA_DBG_CU_SEQLENS_Q
    assert torch.isfinite(o.float()).all()
    for b in (0, 1, 2):
        assert torch.equal(o[seq_rows(p, b)], o_ok[seq_rows(p, b)])
    # decreasing offsets
    cu = p.cu_seqlens_q.copy()
    cu[2] = cu[1] - 1
    gq.debug_flags(reset=True)
    run_varlen(p, cu=cu)
    assert gq.debug_flags() & gq.GQA_DBG_CU_SEQLENS_Q


def test_more_queries_than_positions(use):
    p = varlen_case()
    bad = p.seqlens_k.copy()
    bad[0] = 10  # sequence 0 brings 30 new queries
    use("debug")
    gq.debug_flags(reset=True)
    o, _ = run_varlen(p, seqlens=bad)
    flags = gq.debug_flags()
    say(f"q_len > seqlens_k: flags {flags}")
    assert flags & gq.GQA_DBG_Q_LEN
    assert torch.isfinite(o[seq_rows(p, 1)].float()).all()


def test_decode_lengths_out_of_range_and_reset(use):
    d = gi.decode_problem(43, 4, 256, 8, 2, 64, seqlens=[256, 100, 1, 37])
    q, k, v, s = (dev_tensor(d.q, "cuda"), dev_tensor(d.k, "cuda"), dev_tensor(d.v, "cuda"),
                  dev_f32(d.sinks, "cuda"))
    bad = np.array([300, 100, -2, 37], dtype=np.int32)  # past Lmax, valid, negative, valid
    use("debug")
    gq.debug_flags(reset=True)
    big, out = guarded(4, 8, 64)
    o = gq.attn_decode(q, (k, v), dev_i32(bad, "cuda"), s, out=out)
    torch.cuda.synchronize()
    assert_guard_intact(big, 4, "decode")
    first = gq.debug_flags(reset=True)
    second = gq.debug_flags()
    say(f"decode lengths out of range: flags {first}, after reset {second}")
    assert first & gq.GQA_DBG_SEQLENS_K and second == 0
    assert torch.isfinite(o.float()).all()
    ok = gq.attn_decode(q, (k, v), dev_i32(d.seqlens, "cuda"), s)
    assert torch.equal(o[1], ok[1]) and torch.equal(o[3], ok[3])


@pytest.mark.parametrize("rows", ["0", "2"])
def test_decode_lengths_out_of_range_64_8_heads(use, monkeypatch, rows):
    """64/8 heads: the per-head form and the whole-row form (forced on) with lengths past Lmax and negative."""
    monkeypatch.setenv("GQA_DECODE_ROWS", rows)
    d = gi.decode_problem(44, 4, 256, 64, 8, 64, seqlens=[256, 100, 1, 37])
    q, k, v, s = (dev_tensor(d.q, "cuda"), dev_tensor(d.k, "cuda"), dev_tensor(d.v, "cuda"),
                  dev_f32(d.sinks, "cuda"))
    bad = np.array([300, 100, -2, 37], dtype=np.int32)
    use("debug")
    gq.debug_flags(reset=True)
    big, out = guarded(4, 64, 64)
    o = gq.attn_decode(q, (k, v), dev_i32(bad, "cuda"), s, out=out)
    torch.cuda.synchronize()
    assert_guard_intact(big, 4, "decode")
    flags = gq.debug_flags(reset=True)
    say(f"decode 64/8 heads rows={rows}: lengths out of range, flags {flags}")
    assert flags & gq.GQA_DBG_SEQLENS_K
    assert torch.isfinite(o.float()).all()
    use("release")
    ok = gq.attn_decode(q, (k, v), dev_i32(d.seqlens, "cuda"), s)
    assert torch.equal(o[1], ok[1]) and torch.equal(o[3], ok[3])


def test_release_build_stays_in_bounds(use):
    p = varlen_case()
    use("release")
    bad_t = p.block_table.copy()
    bad_t[0, 1] = 10 ** 6
    bad_l = p.seqlens_k.copy()
    bad_l[1] = 10 ** 6
    cu = p.cu_seqlens_q.copy()
    cu[-1] = p.q.shape[0] + 7
    o, _ = run_varlen(p, table=bad_t, seqlens=bad_l, cu=cu, max_kv_len=int(p.seqlens_k.max()))
    say("release build with out-of-range metadata: outputs finite, guard rows intact")
    assert torch.isfinite(o.float()).all()
    with pytest.raises(gq.GqaError):
        gq.debug_flags()


@pytest.mark.parametrize("rows,dtype", [("0", "bf16"), ("2", "bf16"), ("0", "fp32")])
def test_valid_ring_decode_records_nothing(use, monkeypatch, rows, dtype):
    """A ring decode whose histories are longer than, equal to and shorter than the ring is
    within its contract: the kernels bound the key count by W themselves, so the debug build
    records no flag, and its results are the release build's bit for bit."""
    monkeypatch.setenv("GQA_DECODE_ROWS", rows)
    r = gi.ring_problem(45, 4, 128, [8192, 128, 5, 129], dtype=dtype)
    q, kr, vr, s = (dev_tensor(r.q, "cuda"), dev_tensor(r.k_ring, "cuda"), dev_tensor(r.v_ring, "cuda"),
                    dev_f32(r.sinks, "cuda"))
    sl = dev_i32(r.seqlens, "cuda")
    use("debug")
    gq.debug_flags(reset=True)
    o_d, l_d = gq.attn_decode_ring(q, (kr, vr), sl, s, return_lse=True)
    torch.cuda.synchronize()
    flags = gq.debug_flags(reset=True)
    say(f"valid ring decode rows={rows} {dtype}: flags {flags}")
    assert flags == 0
    use("release")
    o_r, l_r = gq.attn_decode_ring(q, (kr, vr), sl, s, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_r) and torch.equal(l_d, l_r)


def test_varlen_length_above_max_kv_len(use):
    """A seqlens_k[b] above max_kv_len but within the block table's capacity is metadata out
    of range: recorded, and clamped to max_kv_len by the decode rows and the prefill-style
    rows alike (the split plan of decode rows covers max_kv_len keys, so no key the
    sequence would read is silently dropped)."""
    p = varlen_case()
    max_kv = int(p.seqlens_k.max())
    cap = p.block_table.shape[1] * p.block_size
    assert max_kv + 40 <= cap
    bad = p.seqlens_k.copy()
    bad[1] = max_kv + 40   # a decode row (q_len 1)
    bad[3] = max_kv + 30   # prefill-style rows (q_len 5)
    clamped = p.seqlens_k.copy()
    clamped[1] = max_kv
    clamped[3] = max_kv
    use("release")
    o_ok, l_ok = run_varlen(p, seqlens=clamped, max_kv_len=max_kv)
    use("debug")
    gq.debug_flags(reset=True)
    o, lse = run_varlen(p, seqlens=bad, max_kv_len=max_kv)
    flags = gq.debug_flags(reset=True)
    say(f"varlen lengths above max_kv_len: flags {flags}")
    assert flags & gq.GQA_DBG_SEQLENS_K
    assert torch.equal(o, o_ok) and torch.equal(lse, l_ok)


def _ring_chunks(cfg=46):
    """A ragged batch of chunks over 128-slot rings: fresh, partly filled and full rings."""
    L0s, q_lens, W = np.array([0, 50, 500, 3000]), np.array([130, 78, 129, 1]), 128
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = dev_tensor(gi.make_tensor(cfg, gi.T_Q, (T, 64, 64), 1.0, "bf16"), "cuda")
    k = dev_tensor(gi.make_tensor(cfg, gi.T_K, (T, 8, 64), 1.0, "bf16"), "cuda")
    v = dev_tensor(gi.make_tensor(cfg, gi.T_V, (T, 8, 64), 1.0, "bf16"), "cuda")
    kr = dev_tensor(gi.make_tensor(cfg + 1, gi.T_K, (4, W, 8, 64), 1.0, "bf16"), "cuda")
    vr = dev_tensor(gi.make_tensor(cfg + 1, gi.T_V, (4, W, 8, 64), 1.0, "bf16"), "cuda")
    return q, k, v, kr, vr, cu, (L0s + q_lens).astype(np.int32), dev_f32(gi.make_sinks(cfg, 64), "cuda")


def test_valid_calls_of_the_fused_entry_points_record_nothing(use):
    """Chunked prefill over rings, the one-launch decode step (contiguous, paged, ring) and the
    prefill that rotates its queries, on valid metadata: the debug build records no flag and
    gives the release build's results (and cache contents) bit for bit."""
    q, k, v, kr, vr, cu, sl, s = _ring_chunks()
    p = gi.prefill_problem(47, 1, 700, 64, 8)
    pq, pk, pv = dev_tensor(p.q, "cuda"), dev_tensor(p.k, "cuda"), dev_tensor(p.v, "cuda")
    d = gi.decode_problem(48, 3, 400, 64, 8, seqlens=[1, 250, 400])
    r = gi.varlen_problem(49, [40, 300], [1, 1], 64, 8, block_size=16, maxblk=32)
    ring = gi.ring_problem(50, 3, 128, [5, 128, 9000])
    nq = dev_tensor(gi.make_tensor(51, gi.T_Q, (3, 64, 64), 1.0, "bf16"), "cuda")
    nk = dev_tensor(gi.make_tensor(51, gi.T_K, (3, 8, 64), 1.0, "bf16"), "cuda")
    nv = dev_tensor(gi.make_tensor(51, gi.T_V, (3, 8, 64), 1.0, "bf16"), "cuda")
    rq, rk, rv = (dev_tensor(gi.make_tensor(52, t, (2, h, 64), 1.0, "bf16"), "cuda")
                  for t, h in ((gi.T_Q, 64), (gi.T_K, 8), (gi.T_V, 8)))

    def calls():
        outs = []
        krc, vrc = kr.clone(), vr.clone()
        outs += list(gq.attn_prefill_ring(q, k, v, dev_i32(cu, "cuda"), dev_i32(sl, "cuda"), (krc, vrc), s,
                                          return_lse=True)) + [krc, vrc]
        outs += list(gq.attn_prefill_rope(pq, pk, pv, s, window=128, pairing=1, return_lse=True))
        kc, vc = dev_tensor(d.k, "cuda"), dev_tensor(d.v, "cuda")
        outs += list(gq.attn_decode_step(nq, nk, nv, dev_i32(d.seqlens, "cuda"), (kc, vc), s, window=128,
                                         return_lse=True)) + [kc, vc]
        pkc, pvc = dev_tensor(r.k, "cuda"), dev_tensor(r.v, "cuda")
        outs += list(gq.attn_decode_step(rq, rk, rv, dev_i32(r.seqlens_k, "cuda"), (pkc, pvc), s, window=0,
                                         block_table=dev_i32(r.block_table, "cuda"), return_lse=True)) + [pkc, pvc]
        rkc, rvc = dev_tensor(ring.k_ring, "cuda"), dev_tensor(ring.v_ring, "cuda")
        outs += list(gq.attn_decode_step(nq, nk, nv, dev_i32(ring.seqlens, "cuda"), (rkc, rvc), s, ring=True,
                                         return_lse=True)) + [rkc, rvc]
        torch.cuda.synchronize()
        return outs

    use("debug")
    say("fused entry points, valid metadata, debug build")
    gq.debug_flags(reset=True)
    got = calls()
    flags = gq.debug_flags(reset=True)
    say(f"fused entry points: flags {flags}")
    assert flags == 0
    use("release")
    want = calls()
    for i, (a, b) in enumerate(zip(got, want)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), i


def test_ring_prefill_more_queries_than_positions(use):
    """A chunk longer than its sequence's position count (seqlens below q_len) is metadata out
    of range: recorded as GQA_DBG_Q_LEN, the writes stay inside the output, and the other
    sequences get the rows of a call with all metadata valid."""
    q, k, v, kr, vr, cu, sl, s = _ring_chunks()
    bad = sl.copy()
    bad[1] = 30  # 78 new rows but 30 positions
    T = q.shape[0]
    use("release")
    ok = gq.attn_prefill_ring(q, k, v, dev_i32(cu, "cuda"), dev_i32(sl, "cuda"), (kr.clone(), vr.clone()), s,
                              append=False)
    for which in ("debug", "release"):
        use(which)
        say(f"ring prefill, seqlens below q_len, {which} build")
        if which == "debug":
            gq.debug_flags(reset=True)
        big, out = guarded(T, 64, 64)
        gq.attn_prefill_ring(q, k, v, dev_i32(cu, "cuda"), dev_i32(bad, "cuda"), (kr.clone(), vr.clone()), s,
                             append=False, out=out)
        torch.cuda.synchronize()
        assert_guard_intact(big, T, f"ring prefill ({which})")
        if which == "debug":
            assert gq.debug_flags(reset=True) & gq.GQA_DBG_Q_LEN
        for b in (0, 2, 3):
            r0, r1 = int(cu[b]), int(cu[b + 1])
            assert torch.equal(out[r0:r1].view(torch.int16), ok[r0:r1].view(torch.int16)), (which, b)
