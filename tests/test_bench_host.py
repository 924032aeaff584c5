"""Host-side tests of bench.py: the one-GPU refusal and the profile summaries it reports from.

The summaries read rocprofv3 result databases (sqlite); these tests build tiny databases with the
same tables, so the arithmetic behind the committed profiles (per-kernel averages, the copy
calibration of the byte counters, the source check of the traffic record) is checked without a GPU.
"""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _kernels_db(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer, grid_x integer, workgroup_x integer, "
                "vgpr_count integer, accum_vgpr_count integer, scratch_size integer, lds_size integer)")
    con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_trace_summary_averages_per_kernel(tmp_path, capsys):
    a = ("void ba::fwd_kernel<128>(ba::FwdArgs)", 256, 256, 128, 0, 16, 65536)
    b = ("merge", 1024, 256, 12, 0, 0, 0)
    _kernels_db(str(tmp_path / "run" / "x_results.db"),
                [(a[0], 1000, *a[1:]), (a[0], 2000, *a[1:]), (b[0], 500, *b[1:])])
    _kernels_db(str(tmp_path / "run2" / "y_results.db"), [(a[0], 3000, *a[1:])])
    bench.trace_summary(str(tmp_path))
    lines = capsys.readouterr().out.strip().splitlines()
    assert len(lines) == 2
    # sorted by total time; durations are nanoseconds, the summary prints microseconds
    assert lines[0].split()[:5] == ["3", "calls", "avg", "2.000", "us"] and "fwd_kernel<128>" in lines[0]
    assert "lds 65536" in lines[0] and "scratch 16" in lines[0]
    assert lines[1].split()[:4] == ["1", "calls", "avg", "0.500"]


def _counters_db(path, rows, duration_ns=1000):
    """rocprofv3's counters_collection table, each dispatch lasting duration_ns."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real, duration integer)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)",
                    [(*r, duration_ns) for r in rows])
    con.commit()
    con.close()


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    k = "ba::fwd_kernel<128>(ba::FwdArgs)"
    # two dispatches; each counter arrives split over several rows (per XCD), summed per dispatch
    _counters_db(str(tmp_path / "f" / "a_results.db"),
                 [(1, k, "FETCH_SIZE", 60.0), (1, k, "FETCH_SIZE", 40.0), (2, k, "FETCH_SIZE", 300.0),
                  (3, "other", "FETCH_SIZE", 1e9)])
    _counters_db(str(tmp_path / "w" / "a_results.db"), [(1, k, "WRITE_SIZE", 50.0), (2, k, "WRITE_SIZE", 50.0)])
    # the 1 GiB copy: the fetch counter reports half the bytes, the write counter all of them
    _counters_db(str(tmp_path / "cf" / "a_results.db"), [(1, "copy", "FETCH_SIZE", 524288.0), (2, "fill", "FETCH_SIZE", 8.0)])
    _counters_db(str(tmp_path / "cw" / "a_results.db"), [(1, "copy", "WRITE_SIZE", 1048576.0)])
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    bench.traffic_summary("fwd", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    out = str(tmp_path / "fwd_kernel_d128_traffic.json")
    rec = json.load(open(out))
    assert rec["copy_calibration"]["fetch_scale"] == 2.0 and rec["copy_calibration"]["write_scale"] == 1.0
    per = rec["per_kernel"]["fwd_kernel<128>"]
    assert per["fetch_size_kib_per_dispatch"] == [100.0, 300.0]
    assert rec["hbm_fetch_bytes_per_launch"] == 200 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 50 * 1024
    # the bench line reports the record only while the kernel source is the one it was taken on
    wl = "llama2_7b_s32k_ring8"
    assert rec["workload"].split(" ")[0] == wl
    assert bench._traffic("fwd_kernel_d128", bench.FWD_SRC, wl) == rec["hbm_bytes_per_launch"]
    # ... and only on the workload it was taken on
    assert bench._traffic("fwd_kernel_d128", bench.FWD_SRC, "gqa_llama3_8b_s128k_ring16") is None
    rec["kernel_source_sha"] = "0" * 16
    json.dump(rec, open(str(tmp_path / "fwd_kernel_d128_traffic.json"), "w"))
    assert bench._traffic("fwd_kernel_d128", bench.FWD_SRC, wl) is None
    assert bench._traffic("no_such_kernel", bench.FWD_SRC, wl) is None


def test_backward_traffic_is_summed_per_call(tmp_path, monkeypatch):
    """Target bwd: one blockattn_bwd call launches a dK/dV and a dQ kernel (and delta on the first
    call); bytes per call = all their bytes over the number of calls (dQ launches)."""
    kv, dq, de = ("void ba::bwd_dkdv_kernel<128>(ba::BwdArgs)", "void ba::bwd_dq_kernel<128>(ba::BwdArgs)",
                  "void ba::bwd_delta_kernel<128>(ba::BwdArgs, long)")
    _counters_db(str(tmp_path / "f" / "a_results.db"),
                 [(1, de, "FETCH_SIZE", 10.0), (2, kv, "FETCH_SIZE", 100.0), (3, dq, "FETCH_SIZE", 50.0),
                  (4, kv, "FETCH_SIZE", 100.0), (5, dq, "FETCH_SIZE", 50.0),
                  (6, "void ba::fwd_kernel<128>(ba::FwdArgs)", "FETCH_SIZE", 1e6)])
    _counters_db(str(tmp_path / "w" / "a_results.db"),
                 [(1, de, "WRITE_SIZE", 1.0), (2, kv, "WRITE_SIZE", 20.0), (3, dq, "WRITE_SIZE", 30.0),
                  (4, kv, "WRITE_SIZE", 20.0), (5, dq, "WRITE_SIZE", 30.0)])
    _counters_db(str(tmp_path / "cf" / "a_results.db"), [(1, "copy", "FETCH_SIZE", 1048576.0)])
    _counters_db(str(tmp_path / "cw" / "a_results.db"), [(1, "copy", "WRITE_SIZE", 1048576.0)])
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    bench.traffic_summary("bwd", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    rec = json.load(open(str(tmp_path / "bwd_kernels_d128_traffic.json")))
    assert rec["hbm_fetch_bytes_per_call"] == (10 + 200 + 100) * 1024 // 2
    assert rec["hbm_write_bytes_per_call"] == (1 + 40 + 60) * 1024 // 2
    assert rec["per_kernel"]["bwd_dkdv_kernel<128>"]["dispatches"] == 2
    wl = "llama2_13b_s64k_ring8_train"
    assert bench._traffic("bwd_kernels_d128", bench.BWD_SRC, wl, field="hbm_bytes_per_call") == rec["hbm_bytes_per_call"]


def test_backward_algorithmic_bytes_small_case():
    """bwd_algorithmic_bytes against a hand count: S=4, 2 chunks of 2, one head, D=8."""
    from workloads.configs import Workload
    w = Workload("t", 1, 1, 1, 4, 8, n_chunks=2, backward=True)
    # chunk 0: 4 rows x (8*(2+2) + 8 + 8*8) = 4 * 104; K, V read and dK, dV written: 2 keys x 8 x 2 B x 4
    # chunk 1: 2 rows x 104 + 2 x 8 x 2 x 4; once: delta 4 x (8*2*2 + 4), final dQ 4 x 8 x 2
    want = (4 * 104 + 128 + 2 * 104 + 128 + 4 * 36 + 64) / 2
    assert bench.bwd_algorithmic_bytes(w) == want


def test_missing_profile_directory_is_reported(tmp_path):
    with pytest.raises(SystemExit, match="no rocprofv3"):
        bench.trace_summary(str(tmp_path))


def test_counter_record_is_reported_only_when_current(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    rec = {"workload": "llama2_7b_s32k_ring8", "kernel_source_sha": bench._src_sha(bench.FWD_SRC),
           "mfma_busy": 0.5, "valu_busy_est": 0.2, "valu_per_mfma": 5.0, "trans_per_mfma": 1.0,
           "lds_per_mfma": 1.5, "wave_waiting": 0.3}
    json.dump(rec, open(str(tmp_path / "fwd_kernel_d128_counters.json"), "w"))
    got = bench._counters("fwd_kernel_d128", bench.FWD_SRC, "llama2_7b_s32k_ring8")
    assert got == {k: rec[k] for k in got} and set(got) >= {"mfma_busy", "valu_busy_est"}
    assert bench._counters("fwd_kernel_d128", bench.FWD_SRC, "gqa_llama3_8b_s128k_ring16") is None
    rec["kernel_source_sha"] = "f" * 16
    json.dump(rec, open(str(tmp_path / "fwd_kernel_d128_counters.json"), "w"))
    assert bench._counters("fwd_kernel_d128", bench.FWD_SRC, "llama2_7b_s32k_ring8") is None


def test_counter_summary_of_another_kernel_prints_only(tmp_path, capsys):
    rows = []
    for disp, name in ((1, "void ba::bwd_dkdv_kernel<128>(ba::BwdArgs)"), (2, "void ba::fwd_kernel<128>(ba::FwdArgs)")):
        for cname, val in (("GRBM_GUI_ACTIVE", 8000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0),
                           ("SQ_INSTS_MFMA", 100.0), ("SQ_INSTS_VALU", 600.0), ("SQ_INSTS_VALU_TRANS_F32", 50.0),
                           ("SQ_INSTS_LDS", 190.0), ("SQ_WAIT_ANY", 40.0), ("SQ_WAVE_CYCLES", 100.0)):
            rows.append((disp, name, cname, val))
    _counters_db(str(tmp_path / "p" / "a_results.db"), rows)
    out = str(tmp_path / "rec.json")
    bench.counter_summary(str(tmp_path / "p"), out, kernel="bwd_dkdv_kernel<128>")
    text = capsys.readouterr().out
    assert "1 dispatches of bwd_dkdv_kernel<128>" in text
    # 500 busy cycles per SIMD over 1000 cycles; 1.9 LDS instructions per MFMA
    assert "mfma_busy          0.500" in text and "lds_per_mfma       1.900" in text
    # 8000 GRBM counts over 8 XCDs = 1000 cycles in the dispatch's 1000 ns: 1 GHz
    assert "engine_clock_ghz    1.000" in text
    assert not os.path.exists(out)  # the summary record is the forward's only


def test_step_counts_are_checked():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--steps" in r.stderr and r.stdout == ""


def test_counter_table_normalises_per_cu_cycle(tmp_path, capsys):
    k = "void ba::fwd_kernel<128>(ba::FwdArgs)"
    # one dispatch of 1000 cycles on each of the 8 XCDs: 256 CUs x 1000 CU-cycles
    rows = [(1, k, "GRBM_GUI_ACTIVE", 8000.0), (1, k, "SQ_LDS_IDX_ACTIVE", 64000.0),
            (1, k, "SQ_INSTS_LDS_LOAD_BANDWIDTH", 256000.0), (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0),
            (1, k, "SQ_VALU_MFMA_COEXEC_CYCLES", 102400.0), (2, "other", "SQ_LDS_IDX_ACTIVE", 1e9)]
    _counters_db(str(tmp_path / "p" / "a_results.db"), rows)
    bench.counter_table(str(tmp_path / "p"), "fwd_kernel<128>")
    out = capsys.readouterr().out
    assert "1 dispatches of fwd_kernel<128>" in out
    assert "LDS busy 0.250 of cycles; LDS loads 64.0 B per CU-cycle" in out
    assert "MFMA busy 0.500 of SIMD-cycles" in out and "in 0.100 of SIMD-cycles" in out


def test_ring_step_table_splits_the_causal_pairs():
    """The per-position pair counts of a causal ring add up to the workload's allowed pairs, so a
    ring whose launches each take their pair share of the one-call time reads 1.0 everywhere."""
    from workloads import chunk_order, get
    w = get("llama2_7b_s32k_ring8")
    order = chunk_order(w.n_chunks, seed=w.seed)
    one_shot_ms = 8.0
    # launch times exactly proportional to each chunk's pairs, two timed steps
    L = w.chunk_len
    pairs = [L * (L + 1) // 2 + (w.seqlen - (c + 1) * L) * L for c in order]
    assert sum(pairs) == w.allowed_pairs_per_head()
    ms = [one_shot_ms * p / w.allowed_pairs_per_head() for p in pairs]
    rows = bench.ring_step_table(w, ms + ms, order, one_shot_ms)
    assert [r["chunk"] for r in rows] == order
    assert all(abs(r["over_share"] - 1.0) < 1e-3 for r in rows)
    flop = sum(r["tflops"] * r["ms"] * 1e9 for r in rows)
    assert abs(flop / w.fwd_flop() - 1.0) < 1e-3
