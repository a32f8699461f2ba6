"""CPU tests of bench.py's rocprofv3 summary modes (--pmc-summary,
--activity-summary, --trace-summary) on small synthetic result databases with
the tables and columns rocprofv3 writes.  They check the counter scaling by
the calibration dispatches, the split of a kernel's dispatches into per-
workload runs, and the activity formulas, writing into a temporary profiles
directory."""

import argparse
import json
import os
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _db(path, dispatches):
    """dispatches: list of (kernel name, {counter: value}, start_ns, end_ns)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real, start integer, end integer)")
    con.execute("create table kernels (name text, start integer, end integer)")
    for i, (name, counters, start, end) in enumerate(dispatches):
        con.execute("insert into kernels values (?, ?, ?)", (name, start, end))
        for c, v in counters.items():
            con.execute("insert into counters_collection values (?, ?, ?, ?, ?, ?)", (i + 1, name, c, v, start, end))
    con.commit()
    con.close()


def _full(name):
    return f"void {name}(lazyattn::Args)"


STEPS, WARMUP = 2, 1


def _shapes_dispatches(counter, value_of):
    """The --shapes dispatch sequence: calibration first, then each kernel's
    runs of WARMUP + STEPS dispatches (interleaved with an append kernel)."""
    out = [(_full("at::native::vectorized_elementwise_kernel<8, at::native::FillFunctor<short>>"),
            {counter: 1048576.0 if counter == "WRITE_SIZE" else 0.0}, 0, 10),
           ("__amd_rocclr_copyBuffer", {counter: 524288.0 if counter == "FETCH_SIZE" else 1048576.0}, 20, 30)]
    t = 100
    for kernel, names in bench.SHAPES_DISPATCH_ORDER.items():
        for w, name in enumerate(names):
            out.append((_full("lazyattn::append_kernel"), {counter: 7.0}, t, t + 5))
            t += 10
            for k in range(WARMUP + STEPS):
                out.append((_full(kernel), {counter: value_of(name, k)}, t, t + 1000 + 10 * k))
                t += 2000
    return out


def test_pmc_summary_scales_and_groups(tmp_path, monkeypatch):
    fetch = lambda name, k: 1000.0 * (1 + len(name)) + (99999.0 if k < WARMUP else 0.0)  # noqa: E731
    write = lambda name, k: 10.0 * len(name)  # noqa: E731
    fd, wd, td = (str(tmp_path / x) for x in ("fetch", "write", "trace"))
    _db(os.path.join(fd, "run_results.db"), _shapes_dispatches("FETCH_SIZE", fetch))
    _db(os.path.join(wd, "run_results.db"), _shapes_dispatches("WRITE_SIZE", write))
    _db(os.path.join(td, "run_results.db"), _shapes_dispatches("NONE", lambda n, k: 0.0))
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    bench.pmc_summary_main(argparse.Namespace(pmc_summary=(fd, wd, td), steps=STEPS, warmup=WARMUP))
    for kernel, names in bench.SHAPES_DISPATCH_ORDER.items():
        for name in names:
            rec = json.loads((prof / f"{bench.PROFILE_STEMS[name]}_pmc.json").read_text())
            # copy of 1 GiB read as 0.5 GiB -> factor 2; fill of 1 GiB read as 1 GiB -> factor 1
            assert rec["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
            assert rec["copy_calibration"]["write_scale"] == pytest.approx(1.0)
            assert rec["fetch_kib_per_dispatch"] == pytest.approx(fetch(name, WARMUP))   # warm-up dropped
            assert rec["traffic_bytes_per_launch"] == round(fetch(name, WARMUP) * 1024 * 2 + write(name, 0) * 1024)
            assert rec["dispatches"] == STEPS
            assert rec["kernel"] == kernel.replace("lazyattn::", "")
            assert rec["trace_avg_duration_us"] == pytest.approx((1000 + 10 * 1 + 1000 + 10 * 2) / 2 / 1000.0,
                                                                 abs=0.06)
            assert rec["source_hash"] == bench.source_hash(rec["source_files"])
    md = (prof / "decode_shapes_kernel_trace.md").read_text()
    assert "decode_mma16_kernel<4, 0> | zipf_reuse_decode" in md


def test_activity_summary_formulas(tmp_path, monkeypatch):
    cyc = 2_000_000                      # GPU cycles per dispatch
    t_ns = 1_000_000                     # 1 ms -> 2 GHz
    counters = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * cyc * 1024,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e12 / 512, "SQ_ACTIVE_INST_VALU": 0.3 * cyc * 256,
                "SQ_VALU_MFMA_COEXEC_CYCLES": 0.05 * cyc * 1024, "SQ_LDS_IDX_ACTIVE": 0.25 * cyc * 256,
                "SQ_LDS_BANK_CONFLICT": 0.1 * 0.25 * cyc * 256, "SQ_BUSY_CU_CYCLES": 1.0}
    kernel = "lazyattn::prefill_kernel<128, 4, 0, false>"
    disp = []
    t = 0
    for _ in range(2 * (WARMUP + STEPS)):   # the 8B prefill, then the 8-bit one
        disp.append((_full(kernel), counters, t, t + t_ns))
        t += 2 * t_ns
    d = str(tmp_path / "act")
    _db(os.path.join(d, "run_results.db"), disp)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    bench.activity_summary_main(argparse.Namespace(activity_summary=d, steps=STEPS, warmup=WARMUP))
    md = (prof / "decode_prefill_shapes_activity.md").read_text()
    row = next(line for line in md.splitlines() if line.startswith("prefill_kernel<128, 4, 0, false> | llama8b_prefill |"))
    cells = [c.strip() for c in row.split("|")]
    assert cells[2] == "1000.0"          # us
    assert cells[3] == "2.000"           # GHz
    assert cells[4] == "40.0 %"          # MFMA util
    assert cells[5] == "1000.0"          # TFLOP/s counted
    assert cells[7] == "30.0 %"          # VALU busy
    assert cells[8] == "5.0 %"           # co-issue
    assert cells[9] == "25.0 %"          # LDS util
    assert cells[10] == "10.0 %"         # conflict cycles


def test_trace_summary(tmp_path, monkeypatch):
    disp = [(_full("lazyattn::decode_mma16_kernel<4, 0>"), {}, 0, 360_000),
            (_full("lazyattn::decode_mma16_kernel<4, 0>"), {}, 400_000, 762_000),
            (_full("lazyattn::prefill_kernel<128, 4, 0, false>"), {}, 800_000, 1_800_000)]
    d = str(tmp_path / "tr")
    _db(os.path.join(d, "run_results.db"), disp)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    bench.trace_summary_main(argparse.Namespace(trace_summary=d, steps=2, warmup=0))
    md = (prof / "decode_prefill_llama8b_kernel_trace.md").read_text()
    assert "lazyattn::decode_mma16_kernel<4, 0> | 2 | 361.0 | 361.0 | 722.0 |" in md
    assert "lazyattn::prefill_kernel<128, 4, 0, false> | 1 | 1000.0 |" in md
