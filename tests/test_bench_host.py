"""Host logic of bench.py on the CPU: the algorithmic work counts behind every
roofline fraction, checked against the oracle's visibility mask counted pair by
pair, and the rocprofv3 summarizers on small synthetic counter files."""
import csv
import json
import os

import numpy as np
import pytest

import bench
import oracle


def _pairs_by_mask(q_pos, n_keys, window, sink_tokens=0):
    return int(oracle.visible_mask(np.asarray(q_pos), np.arange(n_keys), window, sink_tokens).sum())


@pytest.mark.parametrize("S,W", [(1, 0), (7, 0), (300, 0), (300, 1), (300, 64), (257, 128), (100, 500)])
def test_prefill_pairs_match_mask(S, W):
    D, Hq, Hkv = 64, 8, 2
    flop, byts = bench.prefill_work(2, S, Hq, Hkv, D, W)
    assert flop == 4 * D * Hq * 2 * _pairs_by_mask(np.arange(S), S, W)
    assert byts == 2 * (2 * 2 * S * Hq * D + 2 * 2 * S * Hkv * D)


@pytest.mark.parametrize("S,W,n", [(300, 64, 4), (300, 1, 3), (50, 128, 4), (1000, 128, 100)])
def test_sink_token_pairs_match_mask(S, W, n):
    flop, _ = bench.prefill_work_sink_tokens(1, S, 8, 2, 64, W, n)
    assert flop == 4 * 64 * 8 * _pairs_by_mask(np.arange(S), S, W, n)


def test_decode_and_varlen_counts_match_mask():
    lens = [1, 5, 128, 129, 1000]
    for W, n_sink in ((0, 0), (128, 0), (128, 4), (7, 2)):
        flop, byts = bench.decode_work(lens, 8, 2, 64, W, n_sink=n_sink)
        keys = [_pairs_by_mask([L - 1], L, W, n_sink) for L in lens]
        assert flop == 4 * 64 * 8 * sum(keys)
        assert byts == 2 * (2 * sum(keys) * 2 * 64 + 2 * len(lens) * 8 * 64)
    kv, ql = [300, 40, 1, 513], [17, 40, 1, 0]
    for W in (0, 16, 128):
        flop, _ = bench.varlen_work(kv, ql, 8, 2, 64, W)
        pairs = sum(_pairs_by_mask(np.arange(L - n, L), L, W) for L, n in zip(kv, ql) if n)
        assert flop == 4 * 64 * 8 * pairs


def _write_counter_csv(path, dispatches):
    """dispatches: list of (name, grid, wg, ns, {counter: value})."""
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        t = 1000
        for i, (name, grid, wg, ns, ctr) in enumerate(dispatches, 1):
            for cn, cv in ctr.items():
                w.writerow([i, i, "Agent 1", 1, 1, 1, grid, i, name, wg, 0, 0, 8, 0, 32, cn, cv, t, t + ns])
            t += ns + 100


def test_summarize_units_on_synthetic_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    d = tmp_path / "units_x"
    d.mkdir()
    # per XCD 2e5 GUI-active cycles over 100 us: a 2 GHz clock; 8 XCDs summed in the file
    base = {"GRBM_GUI_ACTIVE": 8 * 2e5, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e6 / 512 * 3, "SQ_VALU_MFMA_BUSY_CYCLES":
            0.25 * 2e5 * 1024, "SQ_ACTIVE_INST_VALU": 0.5 * 2e5 * 256, "SQ_INSTS_VALU_TRANS_F32": 1000,
            "SQ_LDS_BANK_CONFLICT": 10, "SQ_LDS_IDX_ACTIVE": 110, "SQ_ACTIVE_INST_LDS": 0.1 * 2e5 * 256}
    calib = {k: 1.0 for k in base}
    lib = "void gqa::(anonymous namespace)::prefill_bf16_kernel<0, false, false, 0>(gqa::PrefillArgs)"
    _write_counter_csv(d / "run_counter_collection.csv",
                       [(lib, 65536, 256, 100000, base),  # before the calibration copy: not counted
                        ("__amd_rocclr_copyBuffer", 131072, 256, 5000, calib)]
                       + [(lib, 65536, 256, 100000, base)] * 3)
    with open(d / "stage.json", "w") as f:
        json.dump({"stages": [{"name": "prefill_dense", "calls": 3, "flop": 1e6, "bytes": 1, "exp": 64000}]}, f)
    bench.summarize_units([str(d)])
    text = (tmp_path / "units_counters.md").read_text()
    row = [ln for ln in text.splitlines() if ln.startswith("| prefill_dense | 100.0")]
    assert row, text
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # us, MFMA ratio 3, exp ratio 1, matrix 25 %, vector 50 %, LDS 10 %, conflicts 0.1, clock 2 GHz
    assert cells[1:] == ["100.0", "3.00", "1.00", "25.0 %", "50.0 %", "10.0 %", "0.10", "2.00"]


def test_summarize_units_rejects_uneven_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    d = tmp_path / "u"
    d.mkdir()
    c = {"GRBM_GUI_ACTIVE": 8.0}
    lib = "gqa::(anonymous namespace)::decode_combine_kernel(gqa::DecodeArgs)"
    _write_counter_csv(d / "run_counter_collection.csv", [("__amd_rocclr_copyBuffer", 1, 1, 10, c)] + [(lib, 1, 1, 10, c)] * 2)
    with open(d / "stage.json", "w") as f:
        json.dump({"stages": [{"name": "decode_dense", "calls": 3, "flop": 1, "bytes": 1, "exp": 1}]}, f)
    with pytest.raises(SystemExit):
        bench.summarize_units([str(d)])


def test_bench_refuses_more_than_one_gpu(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
