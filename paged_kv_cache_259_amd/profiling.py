"""Summaries of rocprofv3 runs of bench.py (reads the result databases; no GPU).

    python -m paged_kv_cache_259_amd.profiling trace DIR
        per-kernel call count and durations from a ``--kernel-trace`` run.
    python -m paged_kv_cache_259_amd.profiling counters FETCH_DIR WRITE_DIR --workload W --calibrate-copy N
        HBM bytes per timed call from a ``--pmc FETCH_SIZE`` run and a
        ``--pmc WRITE_SIZE`` run of ``bench.py --calibrate-copy N``.  The runs'
        one copy_blocks call over N block pairs is a plain copy of known size
        (N blocks read and N written in each pool); the counters' reading on it
        gives the factor that turns each counter into bytes.  Writes the entry
        for W into profiles/attention_traffic.json, keyed by the hash of the
        attention kernels' sources, so bench.py reports it only while the
        kernels are unchanged.  The timed call of a decode workload is decode
        with append (the attn_*_append_kernel launch, plus the split-context
        reduce when planned; for the shared-prefix workload the shared-block
        decode with append); the other decode kernels of the same run are
        listed but not counted.  For a prefill workload it is the prefill kernel.
    python -m paged_kv_cache_259_amd.profiling sq DIR [DIR ...] --workload W
        shader-sequencer counters of the timed call's kernels from one or more
        ``--pmc`` runs of ``bench.py --workload W`` (counter sets PASS_A and
        PASS_B below, one run each: a pass holds at most 8 SQ counters), averaged
        per dispatch, with the ratios that say where the waves' time goes.
"""

import argparse
import collections
import glob
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _db(d):
    found = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not found:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(found[0])


def _short(name):
    s = name.replace("(anonymous namespace)::", "").split("(")[0]
    for p in ("void ", "pkv::"):
        s = s.replace(p, "")
    return s


def trace(d, out=sys.stdout):
    """Calls, mean, median, min and max duration per kernel (warm-up calls included, so the
    median is the figure to set beside a bench line's steady-state mean)."""
    c = _db(d)
    durs = collections.defaultdict(list)
    for name, dur in c.execute("select name, duration from kernels").fetchall():
        durs[name].append(dur)
    tot = sum(sum(v) for v in durs.values()) or 1
    print(f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total%':>7s}",
          file=out)
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1]))[:12]:
        v = sorted(v)
        med = v[len(v) // 2] if len(v) % 2 else (v[len(v) // 2 - 1] + v[len(v) // 2]) / 2
        print(f"{_short(name)[:64]:64s} {len(v):6d} {sum(v) / len(v) / 1e3:9.2f} {med / 1e3:9.2f} "
              f"{v[0] / 1e3:9.2f} {v[-1] / 1e3:9.2f} {100 * sum(v) / tot:7.2f}", file=out)


def _counter(d, counter):
    c = _db(d)
    rows = c.execute("select kernel_name, grid_size, counter_name, value from counters_collection").fetchall()
    agg = collections.defaultdict(list)
    for k, g, n, v in rows:
        if n == counter and "pkv" in k:
            agg[(_short(k), g)].append(v)
    return {k: sum(v) / len(v) for k, v in agg.items()}


def _in_timed_call(kernel, workload):
    """Kernels of the call bench.py times: decode with append (+ its reduce), the
    shared-block decode with append (shared-prefix workload) or prefill."""
    if kernel.startswith("prefill_"):
        return True
    if workload.startswith("shared_prefix"):
        return kernel.startswith("attn_shared_append")
    return "_append_" in kernel or kernel.startswith(("attn_reduce", "attn_slice_finish"))


COPY_CHUNKS_PER_WG = 1024   # kCopyChunksPerWg: 16-byte chunks per copy_blocks workgroup and tensor


def counters(fetch_dir, write_dir, workload, n_pairs, out=sys.stdout):
    sys.path.insert(0, ROOT)
    import bench
    from paged_kv_cache_259_amd import synth
    w = synth.WORKLOADS[workload]
    elt = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[getattr(w, "kv_dtype", None) or w.dtype]
    block_bytes = w.num_kv_heads * w.block_size * w.head_dim * elt
    f = _counter(fetch_dir, "FETCH_SIZE")
    wr = _counter(write_dir, "WRITE_SIZE")
    # the calibration copy is the device-to-device copy_blocks dispatch whose grid is n_pairs x
    # (workgroups per block, COPY_CHUNKS_PER_WG 16-byte chunks each); other copy_blocks dispatches
    # (copy-on-write pairs, swaps) have other grids
    grid = n_pairs * ((block_bytes // 16 + COPY_CHUNKS_PER_WG - 1) // COPY_CHUNKS_PER_WG) * 256
    cal = next((k for k in f if k[0].startswith("copy_blocks_kernel") and k[1] == grid and k in wr), None)
    if cal is None:
        raise SystemExit(f"no copy_blocks dispatch with grid {grid} (the calibration copy) in the counter runs")
    copy_bytes = 2 * n_pairs * block_bytes          # K and V pools, each read once and written once
    fs, ws = copy_bytes / (f[cal] * 1024), copy_bytes / (wr[cal] * 1024)
    print(f"calibration: copy_blocks of {n_pairs} block pairs ({copy_bytes / 1e9:.3f} GB read, same written): "
          f"FETCH_SIZE {f[cal]:.1f} KiB (scale {fs:.4f}), WRITE_SIZE {wr[cal]:.1f} KiB (scale {ws:.4f})", file=out)
    total_r = total_w = 0.0
    for k in sorted(k for k in f if k[0].startswith(("attn_", "prefill_"))):
        rb, wb = f[k] * 1024 * fs, wr.get(k, 0.0) * 1024 * ws
        counted = _in_timed_call(k[0], workload)
        if counted:
            total_r += rb
            total_w += wb
        print(f"{k[0][:58]:58s} grid {k[1]:8d}  FETCH_SIZE {f[k]:12.1f} KiB -> {rb / 1e6:9.2f} MB read;  "
              f"WRITE_SIZE {wr.get(k, 0.0):10.1f} KiB -> {wb / 1e6:7.2f} MB written"
              f"{'' if counted else '  (not the timed call)'}", file=out)
    print(f"timed call total: {total_r / 1e6:.2f} MB read + {total_w / 1e6:.2f} MB written = "
          f"{(total_r + total_w) / 1e6:.2f} MB", file=out)
    path = os.path.join(ROOT, "profiles", "attention_traffic.json")
    table = {}
    if os.path.exists(path):
        with open(path) as fh:
            table = json.load(fh)
    table[workload] = {"kernel_source_hash": bench.kernel_source_hash(workload), "bytes_per_call": int(total_r + total_w),
                       "read_bytes": int(total_r), "write_bytes": int(total_w),
                       "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
                       "summary": f"profiles/{'paged_prefill_attention' if workload.startswith('prefill') else 'paged_attention_decode'}_{workload}.md"}
    with open(path, "w") as fh:
        json.dump(table, fh, indent=1)
        fh.write("\n")


# Counter sets of the two --pmc passes (8 SQ counters each, plus GRBM_GUI_ACTIVE).
# MfmaUtil, OccupancyPercent, VALUBusy, LdsBankConflict and LdsUtil are rocprofv3's
# derived metrics: MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) /
# (max(GRBM_GUI_ACTIVE) * SIMDs); OccupancyPercent = 400 * sum(SQ_WAVE_CYCLES) /
# max(GRBM_GUI_ACTIVE) / CUs / 32; VALUBusy = 100 * sum(SQ_ACTIVE_INST_VALU) / CUs /
# max(GRBM_GUI_ACTIVE); LdsBankConflict = conflict cycles / (LDS indexed cycles -
# conflict cycles); LdsUtil = 100 * sum(SQ_LDS_IDX_ACTIVE) / (max(GRBM_GUI_ACTIVE) * CUs).
PASS_A = ("GRBM_GUI_ACTIVE MfmaUtil OccupancyPercent VALUBusy SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
          "SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA")
PASS_B = ("GRBM_GUI_ACTIVE LdsBankConflict LdsUtil SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS "
          "SQ_INSTS_LDS SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_FLAT SQ_INSTS_SALU")


def _all_counters(dirs):
    """{(kernel, grid): {counter: mean value per dispatch}} over the runs in ``dirs``."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for k, g, n, v in _db(d).execute("select kernel_name, grid_size, counter_name, value "
                                         "from counters_collection").fetchall():
            if "pkv" in k:
                agg[(_short(k), g)][n].append(v)
    return {key: {n: sum(v) / len(v) for n, v in cs.items()} for key, cs in agg.items()}


def sq(dirs, workload, out=sys.stdout):
    table = _all_counters(dirs)
    keys = sorted(k for k in table if k[0].startswith(("attn_", "prefill_")) and _in_timed_call(k[0], workload))
    if not keys:
        raise SystemExit(f"no timed-call kernel of {workload} in {dirs}")

    def ratio(c, a, b):
        return c[a] / c[b] if a in c and b in c and c[b] else float("nan")

    rows = []
    for k in keys:
        c = table[k]
        waves = c.get("SQ_WAVES", float("nan"))
        rows.append((f"{k[0][:52]} grid {k[1]}", [
            ("GRBM_GUI_ACTIVE cycles", c.get("GRBM_GUI_ACTIVE")),
            ("waves", waves),
            ("MfmaUtil %", c.get("MfmaUtil")),
            ("VALUBusy %", c.get("VALUBusy")),
            ("OccupancyPercent %", c.get("OccupancyPercent")),
            ("mean resident waves per CU", c["OccupancyPercent"] * 32 / 100 if "OccupancyPercent" in c else None),
            ("SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES", ratio(c, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
            ("SQ_WAIT_ANY / SQ_WAVE_CYCLES", ratio(c, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
            ("SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES", ratio(c, "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")),
            ("SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES", ratio(c, "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES")),
            ("SQ_ACTIVE_INST_FLAT / SQ_WAVE_CYCLES", ratio(c, "SQ_ACTIVE_INST_FLAT", "SQ_WAVE_CYCLES")),
            ("LdsBankConflict (conflict / conflict-free LDS cycles)", c.get("LdsBankConflict")),
            ("LdsUtil %", c.get("LdsUtil")),
            ("MFMA instructions per wave", c.get("SQ_INSTS_MFMA", float("nan")) / waves),
            ("VALU instructions per wave", c.get("SQ_INSTS_VALU", float("nan")) / waves),
            ("LDS instructions per wave", c.get("SQ_INSTS_LDS", float("nan")) / waves),
            ("VMEM read instructions per wave", c.get("SQ_INSTS_VMEM_RD", float("nan")) / waves),
            ("SALU instructions per wave", c.get("SQ_INSTS_SALU", float("nan")) / waves),
        ]))
    print(f"| {workload} | " + " | ".join(name for name, _ in rows) + " |", file=out)
    print("|---|" + "---:|" * len(rows), file=out)
    for i, (label, _) in enumerate(rows[0][1]):
        cells = []
        for _, vals in rows:
            v = vals[i][1]
            cells.append("n/a" if v is None or v != v else (f"{v:.0f}" if abs(v) >= 1000 else f"{v:.3g}"))
        print(f"| {label} | " + " | ".join(cells) + " |", file=out)
    print("\nraw means per dispatch (sums over shader engines / SIMDs, as rocprofv3 reports them):", file=out)
    for k in keys:
        print(f"  {k[0][:52]} grid {k[1]}: " + ", ".join(f"{n}={v:.0f}" for n, v in sorted(table[k].items())
                                                         if n.startswith(("SQ_", "GRBM_"))), file=out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--workload", required=True)
    c.add_argument("--calibrate-copy", type=int, required=True)
    q = sub.add_parser("sq")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--workload", required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        trace(a.dir)
    elif a.cmd == "sq":
        sq(a.dirs, a.workload)
    else:
        counters(a.fetch_dir, a.write_dir, a.workload, a.calibrate_copy)


if __name__ == "__main__":
    main()
