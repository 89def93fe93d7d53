"""Host checks of the rocprofv3 summaries (paged_kv_cache_259_amd/profiling.py) on
small databases with the columns rocprofv3 writes; no GPU."""

import io
import os
import sqlite3

import pytest

from paged_kv_cache_259_amd import profiling


def _make_db(path, kernels=(), counters=()):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, duration integer)")
    c.execute("create table counters_collection (kernel_name text, grid_size integer, counter_name text, value real)")
    c.executemany("insert into kernels values (?, ?)", kernels)
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    c.commit()
    c.close()


APPEND = "void pkv::attn_mfma_append_kernel<pkv::BF16, 128>(pkv::AttnParams)"
OTHER = "void pkv::attn_mfma_kernel<pkv::BF16, 128>(pkv::AttnParams)"


def test_trace_groups_by_kernel(tmp_path):
    _make_db(str(tmp_path / "t" / "run_results.db"),
             kernels=[(APPEND, 1000), (APPEND, 3000), (OTHER, 500)])
    out = io.StringIO()
    profiling.trace(str(tmp_path / "t"), out)
    lines = out.getvalue().splitlines()
    assert lines[1].startswith("attn_mfma_append_kernel")
    assert lines[1].split()[-6:-2] == ["2", "2.00", "2.00", "1.00"]     # calls, mean, median, min (microseconds)


def test_sq_averages_per_dispatch_and_forms_ratios(tmp_path):
    a = [(APPEND, 4096, n, v) for n, v in [
        ("SQ_WAVES", 1000), ("SQ_WAVE_CYCLES", 400), ("SQ_WAIT_INST_ANY", 100), ("SQ_INSTS_MFMA", 8000),
        ("MfmaUtil", 10.0), ("OccupancyPercent", 25.0)]]
    a += [(APPEND, 4096, "SQ_WAIT_INST_ANY", 300)]          # a second dispatch: mean 200
    a += [(OTHER, 4096, "SQ_WAVES", 7)]                     # not the timed call: left out
    b = [(APPEND, 4096, n, v) for n, v in [("SQ_INSTS_LDS", 3000), ("SQ_ACTIVE_INST_LDS", 40), ("LdsBankConflict", 0.5)]]
    _make_db(str(tmp_path / "a" / "x" / "run_results.db"), counters=a)
    _make_db(str(tmp_path / "b" / "run_results.db"), counters=b)
    out = io.StringIO()
    profiling.sq([str(tmp_path / "a"), str(tmp_path / "b")], "gqa_bf16", out)
    rows = {l.split("|")[1].strip(): l.split("|")[2].strip() for l in out.getvalue().splitlines() if l.startswith("| ")}
    assert "attn_mfma_append_kernel" in out.getvalue().splitlines()[0]
    assert "attn_mfma_kernel" not in out.getvalue().splitlines()[0]
    assert rows["SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES"] == "0.5"
    assert rows["mean resident waves per CU"] == "8"
    assert rows["MFMA instructions per wave"] == "8"
    assert rows["LDS instructions per wave"] == "3"
    assert rows["SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES"] == "0.1"
    assert rows["LdsBankConflict (conflict / conflict-free LDS cycles)"] == "0.5"
    assert rows["VALU instructions per wave"] == "n/a"


def test_sq_passes_fit_the_hardware_limits():
    # one --pmc pass holds at most 8 SQ counters (derived metrics count their inputs)
    inputs = {"MfmaUtil": ["SQ_VALU_MFMA_BUSY_CYCLES"], "OccupancyPercent": ["SQ_WAVE_CYCLES"],
              "VALUBusy": ["SQ_ACTIVE_INST_VALU"], "LdsBankConflict": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"],
              "LdsUtil": ["SQ_LDS_IDX_ACTIVE"]}
    for p in (profiling.PASS_A, profiling.PASS_B):
        sq = set()
        for c in p.split():
            sq.update(x for x in inputs.get(c, [c]) if x.startswith("SQ_"))
        assert len(sq) <= 8, (p, sorted(sq))


def test_sq_without_timed_kernels_fails(tmp_path):
    _make_db(str(tmp_path / "a" / "run_results.db"), counters=[(OTHER, 64, "SQ_WAVES", 1)])
    with pytest.raises(SystemExit):
        profiling.sq([str(tmp_path / "a")], "gqa_bf16", io.StringIO())


def test_short_names():
    assert profiling._short("void (anonymous namespace)::stream_read_kernel(uint4 const*, unsigned long)") == \
        "stream_read_kernel"
    assert profiling._short("void pkv::attn_mfma_append_kernel<pkv::BF16, pkv::BF16, 128, 2, true>(pkv::AttnParams)") \
        == "attn_mfma_append_kernel<BF16, BF16, 128, 2, true>"


def test_counters_calibrate_on_the_device_copy(tmp_path, monkeypatch):
    """The calibration copy is the copy_blocks dispatch with n_pairs x (workgroups per block) x 256
    threads; FETCH_SIZE / WRITE_SIZE of the attention kernel are scaled by what the counters read on
    it against its known bytes.  The grid formula follows the library's chunks per workgroup."""
    import re
    hdr = open(os.path.join(profiling.ROOT, "paged_kv_cache_259_amd", "csrc", "pkv_internal.h")).read()
    assert int(re.search(r"#define PKV_COPY_CHUNKS_PER_WG (\d+)", hdr).group(1)) == profiling.COPY_CHUNKS_PER_WG
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))         # the traffic table goes under tmp_path
    os.makedirs(tmp_path / "profiles")
    n = 64
    block_bytes = 8 * 16 * 128 * 2                                 # the GQA bf16 pool's block
    grid = n * (block_bytes // 16 // profiling.COPY_CHUNKS_PER_WG) * 256
    copy = "void pkv::copy_blocks_kernel<4, true>(pkv::CopyParams)"
    kib = 2 * n * block_bytes / 1024
    _make_db(str(tmp_path / "f" / "run_results.db"),
             counters=[(copy, grid, "FETCH_SIZE", kib / 2), (copy, 999, "FETCH_SIZE", 1.0), (APPEND, 4096, "FETCH_SIZE", 100.0)])
    _make_db(str(tmp_path / "w" / "run_results.db"),
             counters=[(copy, grid, "WRITE_SIZE", kib), (APPEND, 4096, "WRITE_SIZE", 10.0)])
    out = io.StringIO()
    profiling.counters(str(tmp_path / "f"), str(tmp_path / "w"), "gqa_bf16", n, out)
    text = out.getvalue()
    assert "scale 2.0000" in text and "scale 1.0000" in text
    assert "timed call total: 0.20 MB read + 0.01 MB written" in text
