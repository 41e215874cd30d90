"""Benchmark of the attention hot path on one MI355X; prints ONE JSON line.

A step is one pass over every stage of the path, on seeded synthetic inputs
already resident in HBM:
  1. layer-shaped prefill  B1 S4096, 64 query / 8 KV heads, D64, bf16 -- one
     dense layer, one 128-token sliding-window layer, and one windowed layer
     that keeps 4 start-of-sequence sink tokens visible;
  2. batched decode        B64, cache 8192, same heads -- dense, window 128,
     window 128 with 4 sink tokens, and the windowed layer's whole decode step
     (rotary encoding of the new token, KV append, attention) in one launch;
  3. ragged + paged        16 sequences, lengths U{128..8192}, 512-token
     prefill chunks and single-token decode steps, 16-token pages under a
     permuted block table -- dense, then window 128; then the windowed layer
     of the same batch over 128-slot rings (each chunk attends over its ring
     plus its own rows, then joins the ring);
  4. ring cache of a windowed layer (128 slots per sequence): append of one
     new token per sequence (B64), then decode from the rings at position 8191
     for B64 and for B4096 (the B4096 rings hold as many bytes as the dense
     B64 x 8192 cache);
  5. rotary encoding of new rows fused with their KV-cache append: the 4096
     rows of the layer-shaped prefill (queries and keys, and keys only, for
     the prefill that rotates its queries as it loads them: "prefill_rope_*"
     in stage 1), and a decode step of 64 sequences;
  6. backward of the layer-shaped prefill (dq, dk, dv, dsinks from dL/dout,
     the forward's output and log-sum-exp), dense and window 128: algorithmic
     work 10*D*Hq per visible pair (the five matrix products S, dP, dV, dK, dQ);
  7. long context (the 131 072-token context of the model card): prefill
     S32768 and decode B8 x 131072, dense and window 128 ("long_*" parts;
     --skip-long leaves them out).
`value` is the prefill throughput of the layer pair (1), in algorithmic
TFLOP/s (4*D*Hq per visible query-key pair), timed with HIP events on the
stream the kernels run on; every stage's own time, TFLOP/s, GB/s and roofline
fraction is reported under "parts".  "roofline" describes the dominant kernel
(dense prefill, MFMA-bound); "roofline_decode" the HBM-bound dense decode.
Each part also carries two other timings of the same stage, never used for
`value`: cold (each call after a 512 MiB read pass that evicts the last-level
cache and leaves it clean; median) and back to back (the stage alone, called `steps` times in a
row, median; a dense MFMA kernel then runs at the lower clock its own power
draw settles at, where inside the step it starts from the clock the HBM-bound
stages left).  A part's `roofline_frac` is quoted on the cold median for
HBM-bound stages (a warm stage's inputs may still sit in the 256 MiB cache)
and on the in-step mean for MFMA-bound ones; `roofline_frac_warm` and
`roofline_frac_cold` are both kept beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
METRIC = "prefill attn TFLOP/s + decode KV GB/s, % of MI355X roofline, dense vs SWA-128"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "attention_gqa_causal_amd", "csrc")


# ----------------------------------------------------------------------------- algorithmic work

def visible_pairs(q_pos_last, n_q, window):
    """Number of (query, key) pairs visible for n_q queries at positions q_pos_last-n_q+1 .. q_pos_last."""
    tot = 0
    p0 = q_pos_last - n_q + 1
    # sum over p of min(p + 1, W) (or p + 1 when dense)
    if window <= 0:
        return (p0 + 1 + q_pos_last + 1) * n_q // 2
    for p in range(p0, q_pos_last + 1):
        tot += min(p + 1, window)
    return tot


def prefill_work(B, S, Hq, Hkv, D, window, elt=2):
    pairs = B * visible_pairs(S - 1, S, window)
    flop = 4 * D * Hq * pairs
    byts = elt * (2 * B * S * Hq * D + 2 * B * S * Hkv * D)
    return flop, byts


def prefill_work_sink_tokens(B, S, Hq, Hkv, D, window, n_sink, elt=2):
    """Work of a windowed prefill whose first n_sink positions stay visible."""
    import numpy as np

    p = np.arange(S, dtype=np.int64)
    keys = np.minimum(window, p + 1) + np.minimum(n_sink, np.maximum(0, p - window + 1))
    flop = 4 * D * Hq * B * int(keys.sum())
    byts = elt * (2 * B * S * Hq * D + 2 * B * S * Hkv * D)
    return flop, byts


def decode_work(seqlens, Hq, Hkv, D, window, elt=2, n_sink=0):
    n_read = [(min(L, window) + min(n_sink, max(0, L - window))) if window > 0 else L for L in seqlens]
    flop = 4 * D * Hq * sum(n_read)
    byts = elt * (2 * sum(n_read) * Hkv * D + 2 * len(seqlens) * Hq * D)
    return flop, byts


def varlen_work(kv_lens, q_lens, Hq, Hkv, D, window, elt=2):
    pairs = 0
    rows = 0
    for L, n in zip(kv_lens, q_lens):
        L, n = int(L), int(n)
        if n == 0:
            continue
        pairs += visible_pairs(L - 1, n, window)
        first = L - n
        lo = max(0, first - window + 1) if window > 0 else 0
        rows += L - lo
    flop = 4 * D * Hq * pairs
    byts = elt * (2 * sum(int(n) for n in q_lens) * Hq * D + 2 * rows * Hkv * D)
    return flop, byts


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ["prefill_bf16.hip", "common.h", "kernels.h"],
    "decode": ["decode_bf16.hip", "common.h", "kernels.h"],
}


def load_traffic(kind, launches_per_call=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the kernel source as it is now; None otherwise."""
    path = os.path.join(PROFILES, f"traffic_{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kind]):
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- HBM traffic from counters

COPY_BYTES = 256 << 20
FLUSH_BYTES = 512 << 20  # twice the MI355X last-level cache (256 MiB MALL)


def _read_counter_csv(d, counter):
    """Per-dispatch values of one counter: list of (kernel name, value in KiB)."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def summarize_counters(fetch_dir, write_dir):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the prefill and decode kernels,
    scaled by what the same counters read for a plain copy of COPY_BYTES."""
    import statistics

    fetch = _read_counter_csv(fetch_dir, "FETCH_SIZE")
    write = _read_counter_csv(write_dir, "WRITE_SIZE")

    def pick(rows, key):
        vals = [v for n, v in rows if key in n]
        return statistics.median(vals) if vals else None

    def pick_copy(rows):
        # the three largest copy dispatches are the timed 256 MiB copies (smaller ones are uploads)
        vals = sorted(v for n, v in rows if "copyBuffer" in n or "copy_kernel" in n)[-3:]
        return statistics.median(vals)

    f_copy, w_copy = pick_copy(fetch), pick_copy(write)
    f_scale = (f_copy * 1024.0) / COPY_BYTES  # counter bytes per true byte read
    w_scale = (w_copy * 1024.0) / COPY_BYTES
    res = {}
    # the dense B1 S4096 prefill: one job per workgroup, batched keys, no sink tokens, queries already rotated
    for kind, key, work in (("prefill", "prefill_bf16_kernel<0, false, false, 0, false>", prefill_work(1, 4096, 64, 8, 64, 0)),
                            ("decode", "decode_rows_kernel", decode_work([8192] * 64, 64, 8, 64, 0))):
        fk, wk = pick(fetch, key), pick(write, key)
        rd = fk * 1024.0 / f_scale
        wr = wk * 1024.0 / w_scale
        rec = {
            "kernel": key,
            "workload": "dense prefill B1 S4096 64/8 heads" if kind == "prefill" else "dense decode B64 x 8192 64/8 heads",
            "fetch_kib_per_dispatch": fk,
            "write_kib_per_dispatch": wk,
            "copy_fetch_kib": f_copy,
            "copy_write_kib": w_copy,
            "copy_bytes": COPY_BYTES,
            "fetch_scale": f_scale,
            "write_scale": w_scale,
            "hbm_read_bytes_per_launch": rd,
            "hbm_write_bytes_per_launch": wr,
            "hbm_bytes_per_launch": rd + wr,
            "algorithmic_bytes_per_launch": work[1],
            "source_sha256_16": source_hash(KERNEL_SOURCES[kind]),
        }
        res[kind] = rec
        with open(os.path.join(PROFILES, f"traffic_{kind}.json"), "w") as f:
            json.dump(rec, f, indent=1)
    lines = ["# HBM traffic per launch from rocprofv3 counters", "",
             "Commands (repository root, one MI355X; each pass a run of its own):", "",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python3 bench.py --counters",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python3 bench.py --counters",
             "    python3 bench.py --summarize-counters gpurun_out/pmc_fetch gpurun_out/pmc_write", "",
             f"Calibration: a plain device copy of {COPY_BYTES >> 20} MiB reads FETCH_SIZE = {f_copy:.0f} KiB and "
             f"WRITE_SIZE = {w_copy:.0f} KiB, i.e. {f_scale:.3f} and {w_scale:.3f} counter bytes per true byte; "
             "kernel counters are divided by these factors.", "",
             "| kernel | workload | FETCH KiB | WRITE KiB | HBM read MB | HBM write MB | algorithmic MB | traffic / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    for kind, r in res.items():
        lines.append(f"| `{r['kernel']}` | {r['workload']} | {r['fetch_kib_per_dispatch']:.0f} | "
                     f"{r['write_kib_per_dispatch']:.0f} | {r['hbm_read_bytes_per_launch'] / 1e6:.1f} | "
                     f"{r['hbm_write_bytes_per_launch'] / 1e6:.1f} | {r['algorithmic_bytes_per_launch'] / 1e6:.1f} | "
                     f"{r['hbm_bytes_per_launch'] / r['algorithmic_bytes_per_launch']:.2f} |")
    with open(os.path.join(PROFILES, "hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _short_kernel_name(n):
    """Kernel name without namespaces and argument lists."""
    import re

    if n.startswith("_Z"):  # mangled: keep the identifier and a rough template hint
        m = re.search(r"N_1\d+(\w+?)(I|E)", n)
        base = m.group(1) if m else n
        base = re.sub(r"^\d+", "", base)
        tmpl = re.search(r"I(.*)EEvNS", n)
        return base + (f"<{tmpl.group(1)}>" if tmpl else "")
    n = n.replace("void ", "").replace("gqa::(anonymous namespace)::", "")
    return n.split("(")[0]


def summarize_trace(trace_dir, out_md=None):
    """Kernel-trace summary of one bench run: rocprofv3's per-kernel statistics, and
    per-dispatch medians grouped by (kernel, grid size), which tells the stages of
    one kernel apart."""
    import csv
    import glob
    import statistics

    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel_stats.csv / kernel_trace.csv under {trace_dir}")
    lines = ["# Kernel trace: one bench step (all stages)", "",
             "Command (repository root, one MI355X):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o run -- "
             "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline",
             "    python3 bench.py --summarize-trace gpurun_out/prof_trace", "",
             "Every stage runs 35 times: 3 warm-up, 10 in the step loop, 10 cold (each after a 512 MiB read pass, the "
             "`reduce_kernel` rows), 2 + 10 back to back. rocprofv3 `--stats` summary (all stages of one kernel "
             "pooled):", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    with open(stats[0]) as f:
        for r in csv.DictReader(f):
            lines.append(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                         f"{float(r['Percentage']):.1f} |")
    groups = {}
    with open(trace[0]) as f:
        for r in csv.DictReader(f):
            key = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    # stages that launch one kernel on the same grid (dense and windowed layers)
    # differ in duration: split such a group at its largest gap
    rows = []
    for (name, wgs), v in groups.items():
        v = sorted(v)
        parts = [v]
        if len(v) >= 4 and v[-1] > 2 * v[0]:
            gaps = [(v[i + 1] / max(v[i], 1e-9), i) for i in range(len(v) - 1)]
            _, cut = max(gaps)
            parts = [v[:cut + 1], v[cut + 1:]]
        for part in parts:
            rows.append((name, wgs, len(part), statistics.median(part)))
    lines += ["", "Per-dispatch durations by (kernel, workgroups), median over the run (a group whose durations "
              "fall into two clusters, e.g. the dense and the windowed layer on one grid, is shown as two rows):", "",
              "| kernel | workgroups | dispatches | median us |", "|---|---|---|---|"]
    for name, wgs, n, med in sorted(rows, key=lambda r: -r[3] * r[2]):
        lines.append(f"| `{name}` | {wgs} | {n} | {med:.1f} |")
    text = "\n".join(lines) + "\n"
    with open(out_md or os.path.join(PROFILES, "kernel_trace_bench_step.md"), "w") as f:
        f.write(text)
    print(text)


UNIT_COUNTERS = ("GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU "
                 "SQ_INSTS_VALU_TRANS_F32 SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS")


def _read_dispatches(d):
    """Dispatches of one rocprofv3 --pmc run in order: dicts with name, workgroups, duration (ns) and the counter
    values (rocprofv3's csv sums each counter over all its hardware instances: SEs, XCDs)."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    disp = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            i = int(r["Dispatch_Id"])
            e = disp.setdefault(i, {"name": r["Kernel_Name"],
                                    "wgs": int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])),
                                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agent = {"xcc": 8, "simd": 1024, "cu": 256, "clk_mhz": 2400}
    info = glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True)
    if info:
        with open(info[0]) as f:
            for r in csv.DictReader(f):
                if r.get("Agent_Type") == "GPU":
                    agent = {"xcc": int(r["Num_Xcc"]), "simd": int(r["Simd_Count"]), "cu": int(r["Cu_Count"]),
                             "clk_mhz": int(r["Max_Engine_Clk_Fcompute"])}
    return [disp[i] for i in sorted(disp)], agent


def summarize_units(dirs):
    """Execution-unit counters of single stages (one rocprofv3 --pmc run per stage, `bench.py --counters --parts
    STAGE --manifest DIR/stage.json`): executed matrix-core FLOP and exp instructions against the algorithmic
    counts, matrix-unit and vector-unit busy fractions, LDS bank conflicts.  The busy fractions follow rocprofv3's
    own derived metrics (MfmaUtil, VALUBusy, LdsBankConflict) with GRBM_GUI_ACTIVE per XCD as the time base."""
    import statistics

    rows, krows, agent = [], [], None
    for d in dirs:
        with open(os.path.join(d, "stage.json")) as f:
            st = json.load(f)["stages"][0]
        disp, agent = _read_dispatches(d)
        last_copy = max(i for i, e in enumerate(disp) if "copyBuffer" in e["name"] or "copy_kernel" in e["name"])
        mine = [e for e in disp[last_copy + 1:] if "gqa::" in e["name"]]
        if not mine or len(mine) % st["calls"]:
            raise SystemExit(f"{d}: {len(mine)} library dispatches for {st['calls']} calls")
        nx, ns, nc = agent["xcc"], agent["simd"], agent["cu"]
        calls = st["calls"]
        # per (kernel, grid): the median dispatch of each counter (the first dispatch of a run can carry
        # collection set-up in its GUI-active count), times the group's dispatches per call
        groups = {}
        for e in mine:
            groups.setdefault((_short_kernel_name(e["name"]), e["wgs"]), []).append(e)
        names_c = sorted({c for e in mine for c in e["c"]})
        med = {}
        for key, es in groups.items():
            m = {c: statistics.median(e["c"].get(c, 0.0) for e in es) for c in names_c}
            m["ns"] = statistics.median(e["ns"] for e in es)
            med[key] = (m, len(es) / calls)

        def per_call(c):
            return sum(m[c] * k for m, k in med.values())

        g = per_call("GRBM_GUI_ACTIVE") / nx  # GUI-active cycles of one XCD per call
        conf, idx = per_call("SQ_LDS_BANK_CONFLICT"), per_call("SQ_LDS_IDX_ACTIVE")
        rows.append({
            "stage": st["name"], "us": per_call("ns") / 1e3,
            "clk": g / (per_call("ns") * 1e-9) / 1e9,
            "mfma_ratio": per_call("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / st["flop"] if st["flop"] else None,
            "exp_ratio": per_call("SQ_INSTS_VALU_TRANS_F32") * 64 / st["exp"] if st.get("exp") else None,
            "mfma_busy": per_call("SQ_VALU_MFMA_BUSY_CYCLES") / (g * ns),
            "valu_busy": per_call("SQ_ACTIVE_INST_VALU") / (g * nc),
            "lds_busy": per_call("SQ_ACTIVE_INST_LDS") / (g * nc),
            "lds_conf": conf / (idx - conf) if idx > conf else 0.0,
        })
        for (kn, wgs), (m, _) in med.items():
            gk = m["GRBM_GUI_ACTIVE"] / nx
            ck, ik = m["SQ_LDS_BANK_CONFLICT"], m["SQ_LDS_IDX_ACTIVE"]
            krows.append((st["name"], kn, wgs, m["ns"] / 1e3, m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9,
                          m["SQ_INSTS_VALU_TRANS_F32"] * 64 / 1e6, m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gk * ns),
                          m["SQ_ACTIVE_INST_VALU"] / (gk * nc), ck / (ik - ck) if ik > ck else 0.0))

    def pct(x):
        return "–" if x is None else f"{100 * x:.1f} %"

    def rat(x):
        return "–" if x is None else f"{x:.2f}"

    lines = ["# Execution-unit counters per stage", "",
             "Commands (repository root, one MI355X; one rocprofv3 run per stage, 3 calls each after a 256 MiB "
             "calibration copy):", "",
             "    R=$PWD; cd /tmp && export TMPDIR=/tmp",
             "    for s in " + " ".join(r["stage"] for r in rows) + "; do",
             f"      rocprofv3 --pmc {UNIT_COUNTERS} --output-format csv -d $R/gpurun_out/units_$s -o run -- \\",
             "        python3 $R/bench.py --counters --parts $s --manifest $R/gpurun_out/units_$s/stage.json",
             "    done",
             "    python3 bench.py --summarize-units " + " ".join(f"gpurun_out/units_{r['stage']}" for r in rows), "",
             f"Device: {agent['xcc']} XCDs, {agent['cu']} CUs, {agent['simd']} SIMDs, rated engine clock "
             f"{agent['clk_mhz']} MHz.", "",
             "Definitions (per call: for each kernel of the call, the median over its dispatches of each counter, "
             "summed over the call's kernels):", "",
             "* MFMA FLOP ratio = 512 · `SQ_INSTS_VALU_MFMA_MOPS_BF16` ÷ algorithmic FLOP (visible pairs only); above 1 "
             "means masked or padded matrix work.",
             "* exp ratio = 64 · `SQ_INSTS_VALU_TRANS_F32` ÷ algorithmic exponentials (one per visible pair and query "
             "head; for the backward, one pass over the probabilities). Counts every transcendental instruction of "
             "a wave, all 64 lanes, so it is an upper bound on exponentials evaluated.",
             "* matrix busy = `SQ_VALU_MFMA_BUSY_CYCLES` ÷ (GRBM cycles per XCD × SIMDs) (rocprofv3's MfmaUtil).",
             "* vector busy = `SQ_ACTIVE_INST_VALU` ÷ (GRBM cycles per XCD × CUs) (rocprofv3's VALUBusy); LDS busy "
             "likewise with `SQ_ACTIVE_INST_LDS`.",
             "* LDS conflicts = `SQ_LDS_BANK_CONFLICT` ÷ (`SQ_LDS_IDX_ACTIVE` − `SQ_LDS_BANK_CONFLICT`), conflict "
             "cycles per access cycle (rocprofv3's LdsBankConflict).",
             "* GRBM clock = `GRBM_GUI_ACTIVE` per XCD ÷ kernel time. The counter window is a little longer than "
             "the kernel (start and stop of collection), so this overstates the clock most for short kernels.", "",
             "| stage | us / call (profiled) | MFMA FLOP ratio | exp ratio | matrix busy | vector busy | LDS busy | "
             "LDS conflicts | GRBM clock GHz |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['stage']} | {r['us']:.1f} | {rat(r['mfma_ratio'])} | {rat(r['exp_ratio'])} | "
                     f"{pct(r['mfma_busy'])} | {pct(r['valu_busy'])} | {pct(r['lds_busy'])} | "
                     f"{rat(r['lds_conf'])} | {r['clk']:.2f} |")
    lines += ["", "Per kernel (median dispatch):", "",
              "| stage | kernel | workgroups | us | MFMA GFLOP | exp lanes (M) | matrix busy | vector busy | "
              "LDS conflicts |", "|---|---|---|---|---|---|---|---|---|"]
    for s_, kn, wgs, us, gf, ex, mb, vb, lc in krows:
        lines.append(f"| {s_} | `{kn}` | {wgs} | {us:.1f} | {gf:.2f} | {ex:.1f} | {pct(mb)} | {pct(vb)} | "
                     f"{lc:.2f} |")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "units_counters.md"), "w") as f:
        f.write(text)
    print(text)


# ----------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(seconds: float):
    """Time the fp64 oracle on a bounded row sample of the dense layer-shaped prefill."""
    import numpy as np

    import gqa_inputs as gi
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    p = gi.c2_layer()
    q, k, v = p.q.f64, p.k.f64, p.v.f64
    S, Hq, D = 4096, 64, 64
    rng = np.random.default_rng(0)
    done_rows = 0
    flop = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        rows = np.sort(rng.choice(S, size=16, replace=False))
        oracle.prefill_rows_ref(q, k, v, p.sinks, 0, p.scale, rows=rows)
        done_rows += len(rows)
        flop += 4 * D * Hq * int((rows + 1).sum())
    dt = time.perf_counter() - t0
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"dense layer-shaped prefill (B1 S4096 64/8 heads), {done_rows} query rows drawn uniformly, "
                  f"all 64 heads, fp64 NumPy oracle, {dt:.1f} s",
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


# ----------------------------------------------------------------------------- stages

def add_prefill(stages, gq, p, up, f32, dev):
    import torch

    B, S, Hq, Hkv, D = p.dims
    pq, pk, pv, ps = up(p.q), up(p.k), up(p.v), f32(p.sinks)
    pout = torch.empty_like(pq)
    for name, W in (("prefill_dense", 0), ("prefill_swa128", 128)):
        fl, by = prefill_work(B, S, Hq, Hkv, D, W)
        stages[name] = dict(fn=(lambda W=W: gq.attn_prefill(pq, pk, pv, ps, window=W, out=pout)), flop=fl, bytes=by,
                            exp=fl // (4 * D), bound="mfma" if W == 0 else "hbm")
    # the same layers with the queries arriving unrotated: the kernel rotates them as it loads them (with the
    # keys-only rotary append below, this replaces the rotary append of all rows + the prefill)
    for name, W in (("prefill_rope_dense", 0), ("prefill_rope_swa128", 128)):
        fl, by = prefill_work(B, S, Hq, Hkv, D, W)
        stages[name] = dict(fn=(lambda W=W: gq.attn_prefill_rope(pq, pk, pv, ps, window=W, out=pout)), flop=fl,
                            bytes=by, exp=fl // (4 * D), bound="mfma" if W == 0 else "hbm")
    # windowed layer with 4 start-of-sequence sink tokens kept visible
    fl, by = prefill_work_sink_tokens(B, S, Hq, Hkv, D, 128, 4)
    stages["prefill_swa128_sink4"] = dict(
        fn=(lambda: gq.attn_prefill(pq, pk, pv, ps, window=128, sink_tokens=4, out=pout)), flop=fl, bytes=by,
        exp=fl // (4 * D), bound="hbm")


def add_decode(stages, gq, d, up, i32, f32, dev):
    import torch

    Hq, Hkv, D = d.q.shape[1], d.k.shape[2], d.q.shape[2]
    dq, dk, dv, dsl, ds = up(d.q), up(d.k), up(d.v), i32(d.seqlens), f32(d.sinks)
    Bd, Ld = d.k.shape[0], d.k.shape[1]
    for name, W in (("decode_dense", 0), ("decode_swa128", 128)):
        fl, by = decode_work([int(x) for x in d.seqlens], Hq, Hkv, D, W)
        nbytes = gq.decode_workspace_size(Bd, Ld, Hq, Hkv, D, W)
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        stages[name] = dict(fn=(lambda W=W, ws=ws: gq.attn_decode(dq, (dk, dv), dsl, ds, window=W, workspace=ws)),
                            flop=fl, bytes=by, exp=fl // (4 * D), bound="hbm")
    # the windowed layer's whole decode step in one launch: rotate the new token's query and key, append the
    # key and value at the last position, attend over the last 128 (the alternative is rope_append + decode)
    import gqa_inputs as gi
    sq = up(gi.make_tensor(9, gi.T_Q, (Bd, Hq, D), 1.0, "bf16"))
    sk = up(gi.make_tensor(9, gi.T_K, (Bd, Hkv, D), 1.0, "bf16"))
    sv = up(gi.make_tensor(9, gi.T_V, (Bd, Hkv, D), 1.0, "bf16"))
    sout = torch.empty_like(sq)
    fl, by = decode_work([int(x) for x in d.seqlens], Hq, Hkv, D, 128)
    by += 2 * Bd * Hkv * D * 2 * 2  # the new key and value rows: read, then written to the cache
    stages["decode_step_swa128"] = dict(
        fn=(lambda: gq.attn_decode_step(sq, sk, sv, dsl, (dk, dv), ds, window=128, out=sout)),
        flop=fl, bytes=by, exp=fl // (4 * D), bound="hbm")
    fl, by = decode_work([int(x) for x in d.seqlens], Hq, Hkv, D, 128, n_sink=4)
    nbytes = gq.decode_workspace_size(Bd, Ld, Hq, Hkv, D, 128, sink_tokens=4)
    ws4 = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    stages["decode_swa128_sink4"] = dict(
        fn=(lambda: gq.attn_decode(dq, (dk, dv), dsl, ds, window=128, sink_tokens=4, workspace=ws4)),
        flop=fl, bytes=by, exp=fl // (4 * D), bound="hbm")


def add_varlen(stages, gq, r, up, i32, f32, dev):
    import torch

    Hq, Hkv, D = r.q.shape[1], r.k.shape[2], r.q.shape[2]
    rq, rk, rv, rs = up(r.q), up(r.k), up(r.v), f32(r.sinks)
    rbt, rcu, rsl = i32(r.block_table), i32(r.cu_seqlens_q), i32(r.seqlens_k)
    nseq = len(r.seqlens_k)
    for name, W in (("varlen_dense", 0), ("varlen_swa128", 128)):
        fl, by = varlen_work(r.seqlens_k, r.q_lens, Hq, Hkv, D, W)
        nbytes = gq.varlen_workspace_size(nseq, r.max_q_len, r.max_kv_len, Hq, Hkv, D, W)
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        stages[name] = dict(fn=(lambda W=W, ws=ws: gq.attn_varlen_paged(
            rq, (rk, rv), rbt, rcu, rsl, rs, window=W, max_q_len=r.max_q_len, max_kv_len=r.max_kv_len,
            workspace=ws)), flop=fl, bytes=by, exp=fl // (4 * D), bound="mfma" if W == 0 else "hbm")
    # the windowed layer of the same batch with a 128-slot ring per sequence instead of pages: each chunk
    # (or decode row) attends over its ring plus its own rows, then joins the ring
    import gqa_inputs as gi
    W = 128
    Tq = r.q.shape[0]
    kr = up(gi.make_tensor(69, gi.T_K, (nseq, W, Hkv, D), 1.0, "bf16"))
    vr = up(gi.make_tensor(69, gi.T_V, (nseq, W, Hkv, D), 1.0, "bf16"))
    kn = up(gi.make_tensor(70, gi.T_K, (Tq, Hkv, D), 1.0, "bf16"))
    vn = up(gi.make_tensor(70, gi.T_V, (Tq, Hkv, D), 1.0, "bf16"))
    rout = torch.empty_like(rq)
    fl, by = varlen_work(r.seqlens_k, r.q_lens, Hq, Hkv, D, W)
    by += 2 * 2 * sum(min(int(n), W) for n in r.q_lens) * Hkv * D  # the append: rows written to the rings
    stages["varlen_ring_swa128"] = dict(
        fn=(lambda: gq.attn_prefill_ring(rq, kn, vn, rcu, rsl, (kr, vr), rs, max_q_len=r.max_q_len, out=rout)),
        flop=fl, bytes=by, exp=fl // (4 * D), bound="hbm")


def add_ring(stages, gq, up, i32, f32, dev):
    import torch

    import gqa_inputs as gi

    for B in (64, 4096):
        r = gi.c6_ring(B)
        Hq, Hkv, D = r.q.shape[1], r.k_ring.shape[2], r.q.shape[2]
        rq, rk, rv, rsl, rs = up(r.q), up(r.k_ring), up(r.v_ring), i32(r.seqlens), f32(r.sinks)
        n_read = [min(int(L), r.W) for L in r.seqlens]
        fl, by = decode_work(n_read, Hq, Hkv, D, 0)
        nbytes = gq.decode_workspace_size(B, r.W, Hq, Hkv, D, 0)
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        stages[f"ring_decode_w128_b{B}"] = dict(
            fn=(lambda rq=rq, rk=rk, rv=rv, rsl=rsl, rs=rs, ws=ws: gq.attn_decode_ring(rq, (rk, rv), rsl, rs,
                                                                                      workspace=ws)),
            flop=fl, bytes=by, exp=fl // (4 * D), bound="hbm")
        if B == 64:
            kn = up(gi.make_tensor(68, gi.T_K, (B, Hkv, D), 1.0, "bf16"))
            vn = up(gi.make_tensor(68, gi.T_V, (B, Hkv, D), 1.0, "bf16"))
            row = Hkv * D * 2
            stages["ring_append_b64"] = dict(
                fn=(lambda kn=kn, vn=vn, rk=rk, rv=rv, rsl=rsl: gq.kv_ring_append(kn, vn, (rk, rv), rsl)),
                flop=0, bytes=4 * B * row, bound="hbm")


def add_backward(stages, gq, p, up, f32, dev):
    import torch

    import gqa_inputs as gi

    B, S, Hq, D = p.q.shape
    Hkv = p.k.shape[2]
    q, k, v = up(p.q), up(p.k), up(p.v)
    sinks = f32(p.sinks)
    dout = up(gi.make_tensor(2, gi.T_DOUT, p.q.shape, 1.0, "bf16"))
    ws = torch.empty((gq.backward_workspace_size(B, S, Hq, Hkv, D),), dtype=torch.uint8, device=dev)
    for name, W in (("backward_dense", 0), ("backward_swa128", 128)):
        out, lse = gq.attn_prefill(q, k, v, sinks, window=W, return_lse=True)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty((Hq,), dtype=torch.float32, device=dev))
        flop, _ = prefill_work(B, S, Hq, Hkv, D, W)
        # reads q, k, v, out, dout, lse; writes dq, dk, dv
        byts = 2 * (3 * B * S * Hq * D + 4 * B * S * Hkv * D) + 4 * B * Hq * S
        stages[name] = dict(
            fn=(lambda out=out, lse=lse, grads=grads, W=W: gq.attn_prefill_backward(
                q, k, v, sinks, out, lse, dout, window=W, workspace=ws, grads=grads)),
            flop=flop * 10 // 4, bytes=byts, exp=flop // (4 * D), bound="mfma" if W == 0 else "hbm")


def add_rope(stages, gq, up, i32, dev):
    import torch

    import gqa_inputs as gi

    # the layer-shaped prefill's 4096 new rows, rotated and appended to a contiguous cache
    S, Hq, Hkv, D = 4096, 64, 8, 64
    q = up(gi.make_tensor(7, gi.T_Q, (S, Hq, D), 1.0, "bf16"))
    k = up(gi.make_tensor(7, gi.T_K, (S, Hkv, D), 1.0, "bf16"))
    v = up(gi.make_tensor(7, gi.T_V, (S, Hkv, D), 1.0, "bf16"))
    kc = torch.zeros((1, S, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    qo = torch.empty_like(q)
    sl = i32([S])
    cu = i32([0, S])
    by = 2 * 2 * (S * Hq * D + 2 * S * Hkv * D)
    stages["rope_append_s4096"] = dict(
        fn=(lambda: gq.rope_append(q, k, v, sl, (kc, vc), q_out=qo, cu_seqlens_q=cu)),
        flop=0, bytes=by, bound="hbm")
    # keys only (the prefill rotates its queries itself)
    stages["rope_k_append_s4096"] = dict(
        fn=(lambda: gq.rope_append(None, k, v, sl, (kc, vc), cu_seqlens_q=cu)),
        flop=0, bytes=2 * 2 * 2 * S * Hkv * D, bound="hbm")
    # one decode step of 64 sequences
    B = 64
    qd = up(gi.make_tensor(8, gi.T_Q, (B, Hq, D), 1.0, "bf16"))
    kd = up(gi.make_tensor(8, gi.T_K, (B, Hkv, D), 1.0, "bf16"))
    vd = up(gi.make_tensor(8, gi.T_V, (B, Hkv, D), 1.0, "bf16"))
    kcd = torch.zeros((B, 1024, Hkv, D), dtype=torch.bfloat16, device=dev)
    vcd = torch.zeros_like(kcd)
    qod = torch.empty_like(qd)
    sld = i32([1000] * B)
    byd = 2 * 2 * (B * Hq * D + 2 * B * Hkv * D)
    stages["rope_append_decode_b64"] = dict(
        fn=(lambda: gq.rope_append(qd, kd, vd, sld, (kcd, vcd), q_out=qod)),
        flop=0, bytes=byd, bound="hbm")


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--parts", default="all", help="comma list of stages to run (profiling aid)")
    ap.add_argument("--skip-long", action="store_true",
                    help="leave out the long-context workloads (prefill S32768, decode B8 x 131072)")
    ap.add_argument("--counters", action="store_true",
                    help="run only a plain 256 MiB device copy, then each selected stage (--parts; default the "
                         "dense prefill and the dense decode) 3 times, for rocprofv3 --pmc runs")
    ap.add_argument("--manifest", metavar="PATH",
                    help="with --counters: write the selected stages and their algorithmic work as JSON to PATH")
    ap.add_argument("--summarize-units", nargs="+", metavar="DIR",
                    help="turn per-stage rocprofv3 --pmc runs of the execution-unit counters (each DIR holds one "
                         "run and its --manifest stage.json) into profiles/units_counters.md")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats run into profiles/kernel_trace_bench_step.md")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two counter runs into profiles/traffic_*.json and profiles/hbm_traffic.md")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_units:
        summarize_units(args.summarize_units)
        return
    if args.counters and args.parts == "all":
        args.parts = "prefill_dense,decode_dense"

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the attention path is not sharded across GPUs in this library)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_gqa_causal_amd as gq
    import gqa_inputs as gi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    gq.lib()

    def up(t):
        return gi.to_torch(t, dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    stages = {}
    want = None if args.parts == "all" else set(args.parts.split(","))

    def wanted(prefix):
        return want is None or any(w.startswith(prefix) for w in want)

    # 1. layer-shaped prefill
    if wanted("prefill"):
        add_prefill(stages, gq, gi.c2_layer(), up, f32, dev)
    # 2. batched decode
    if wanted("decode"):
        add_decode(stages, gq, gi.c3_decode(), up, i32, f32, dev)
    # 3. ragged + paged
    if wanted("varlen"):
        add_varlen(stages, gq, gi.c5_ragged(), up, i32, f32, dev)
    # 4. ring cache of a windowed layer
    if wanted("ring"):
        add_ring(stages, gq, up, i32, f32, dev)
    # 5. rotary encoding fused with the KV append
    if wanted("rope"):
        add_rope(stages, gq, up, i32, dev)
    # 6. backward of the layer-shaped prefill
    if wanted("backward"):
        add_backward(stages, gq, gi.c2_layer(), up, f32, dev)
    if not args.skip_long and wanted("long"):
        long_stages = {}
        add_prefill(long_stages, gq, gi.c4_prefill(), up, f32, dev)
        add_decode(long_stages, gq, gi.c4_decode(), up, i32, f32, dev)
        for k_, v_ in long_stages.items():
            stages["long_" + k_] = v_
    if want is not None:
        stages = {k: v for k, v in stages.items() if k in want}
    names = list(stages)

    if args.counters:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        # every library dispatch after the last calibration copy belongs to these calls, in this order
        for n in names:
            for _ in range(3):
                stages[n]["fn"]()
            torch.cuda.synchronize()
        if args.manifest:
            os.makedirs(os.path.dirname(os.path.abspath(args.manifest)), exist_ok=True)
            with open(args.manifest, "w") as f:
                json.dump({"stages": [{"name": n, "calls": 3, "flop": stages[n]["flop"], "bytes": stages[n]["bytes"],
                                       "exp": stages[n].get("exp")} for n in names]}, f, indent=1)
        print("counter workload done", flush=True)
        return

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for n in names:
            stages[n]["fn"]()
    torch.cuda.synchronize()

    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
          for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for n in names:
            a, b = ev[n][i]
            a.record()
            stages[n]["fn"]()
            b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # cold cache: before each call a 512 MiB read pass evicts the 256 MiB last-level cache (and the L2s),
    # so the call's inputs come from HBM; reported beside the warm numbers, never as `value`.  A read pass
    # leaves clean lines behind: after a write pass the timed call would also pay the write-back of 256 MiB
    # of someone else's dirty lines (measured: +3.4 us on the window-128 prefill)
    # (fp32 zeros summed in fp32: one read pass, no conversion copy)
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    cold = {n: [] for n in names}
    for i in range(args.steps):
        for n in names:
            torch.sum(flush, dim=0, out=flush_sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            stages[n]["fn"]()
            b.record()
            cold[n].append((a, b))
    torch.cuda.synchronize()
    del flush

    # back to back: the same stage called `steps` times in a row.  In the step loop above each stage runs between
    # other stages, and a compute-bound kernel then finds the clock that the HBM-bound stages left it; called back
    # to back it runs at the clock its own power draw settles at (lower for dense MFMA work)
    # (events around each call, median: a stage shorter than its host-side launch cost would otherwise be timed
    # at the launch rate)
    b2b = {}
    for n in names:
        for _ in range(2):
            stages[n]["fn"]()
        evs = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            stages[n]["fn"]()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        b2b[n] = sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2]

    parts = {}
    for n in names:
        ms = sorted(a.elapsed_time(b) for a, b in ev[n])
        avg = sum(ms) / len(ms)
        st = stages[n]
        t = avg / 1e3
        ms_cold = sorted(a.elapsed_time(b) for a, b in cold[n])[len(cold[n]) // 2]
        t_roof = max(st["flop"] / (PEAK_BF16_TFLOPS * 1e12), st["bytes"] / (PEAK_HBM_GBPS * 1e9))
        frac_warm = round(t_roof / t, 4)
        frac_cold = round(t_roof / (ms_cold / 1e3), 4)
        parts[n] = {
            "ms": round(avg, 5),
            "ms_median": round(ms[len(ms) // 2], 5),
            "tflops": round(st["flop"] / t / 1e12, 3),
            "gbps": round(st["bytes"] / t / 1e9, 2),
            "bound": st["bound"],
            "roofline_frac": frac_cold if st["bound"] == "hbm" else frac_warm,
            "roofline_frac_basis": "cold median" if st["bound"] == "hbm" else "in-step mean",
            "roofline_frac_warm": frac_warm,
            "ms_cold_median": round(ms_cold, 5),
            "roofline_frac_cold": frac_cold,
            "ms_back_to_back_median": round(b2b[n], 5),
            "roofline_frac_back_to_back": round(t_roof / (b2b[n] / 1e3), 4),
            "alg_flop": st["flop"],
            "alg_bytes": st["bytes"],
        }

    out = {
        "metric": METRIC,
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "layer-shaped prefill B1 S4096 Hq64 Hkv8 D64 bf16, dense layer then 128-token sliding-window "
                        "layer (value); each step also runs batched decode B64 cache 8192 (dense, window 128) and "
                        "ragged+paged 16 sequences (dense, window 128; the windowed layer also over 128-slot rings), and a "
                        "windowed layer's 128-slot ring cache (append B64; decode B64 and B4096), the rotary encoding + KV append of the prefill rows and of a decode step, "
                        "the backward of the layer-shaped prefill (dense, window 128), and the long-context prefill "
                        "S32768 and decode B8 x 131072 (dense, window 128)",
            "global_batch": 1,
            "seq_len": 4096,
            "parallelism": "single GPU",
        },
        "parts": parts,
    }
    if "prefill_dense" in parts and "prefill_swa128" in parts:
        tot_f = stages["prefill_dense"]["flop"] + stages["prefill_swa128"]["flop"]
        tot_t = (parts["prefill_dense"]["ms"] + parts["prefill_swa128"]["ms"]) / 1e3
        out["value"] = round(tot_f / tot_t / 1e12, 3)
    if "prefill_dense" in parts:
        pd = parts["prefill_dense"]
        out["roofline"] = {
            "bound": "mfma",
            "achieved": pd["tflops"],
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pd["tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic("prefill"),
            "kernel": "prefill_bf16_kernel (dense, B1 S4096)",
        }
    if "decode_dense" in parts:
        dd = parts["decode_dense"]
        out["roofline_decode"] = {
            "bound": "hbm",
            "achieved": dd["gbps"],
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dd["gbps"] / PEAK_HBM_GBPS, 4),
            "traffic": load_traffic("decode"),
            "kernel": "decode_rows_kernel (dense, B64 x 8192, whole 1 KB K/V rows)",
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
