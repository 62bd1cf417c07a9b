"""The rocprofv3 summaries behind the committed profiles (host logic only).

Each test writes a small SQLite file with the tables/views of a rocprofv3
results database that the summary tool reads, with counter values chosen so
the expected figures follow by hand: the copy calibration, the warm-up drop,
the pairing of a split-K launch's two kernels, the MFMA busy share and the
SQ wait shares.
"""
import json
import sqlite3

import pytest

from sparse_kv_refresh_amd import rocprof_summary as R

UP = "void wamc::gemm_bf16_sk_kernel<2, 128, 128, 64, 2, 2, 2>(wamc::GemmArgs)"
DOWN = "void wamc::gemm_bf16_sk_kernel<3, 256, 256, 64, 2, 2, 2>(wamc::GemmArgs)"
DOWN_RED = "void wamc::gemm_parts_resid_ln_kernel<6, 3, true>(wamc::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _db(path, counters=(), kernels=()):
    """counters: (kernel_name, counter_name, value) in dispatch order;
    kernels: (name, duration_ns) in start order."""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, dispatch_id int)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)",
                    [(k, c, v, i) for i, (k, c, v) in enumerate(counters)])
    con.execute("create table kernels (name text, duration real, start int)")
    con.executemany("insert into kernels values (?, ?, ?)", [(n, d, i) for i, (n, d) in enumerate(kernels)])
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real)")
    con.commit()
    con.close()
    return str(path)


def test_copy_factor_from_the_calibration_copy(tmp_path):
    # a 1 GiB copy that the counter reads as 0.5 GiB -> factor 2
    db = _db(tmp_path / "f.db", [(COPY, "FETCH_SIZE", 4.0), (COPY, "FETCH_SIZE", 524288.0)])
    assert R.copy_factor(R.counters(db, "FETCH_SIZE"), "FETCH_SIZE") == pytest.approx(2.0)


def test_traffic_drops_warmup_and_pairs_the_reduction(tmp_path, capsys):
    # four launches of the down projection (pieces + reduction), the first
    # two warm-up; fetch counts 100 / 10 KiB for the kept pieces / reductions
    fetch = [(COPY, "FETCH_SIZE", 524288.0)]
    write = [(COPY, "WRITE_SIZE", 1048576.0)]
    for i in range(4):
        fetch += [(DOWN, "FETCH_SIZE", 1000.0 if i < 2 else 100.0), (DOWN_RED, "FETCH_SIZE", 500.0 if i < 2 else 10.0)]
        write += [(DOWN, "WRITE_SIZE", 7.0), (DOWN_RED, "WRITE_SIZE", 3.0)]
    f = _db(tmp_path / "f.db", fetch)
    w = _db(tmp_path / "w.db", write)
    out = tmp_path / "t.json"
    R.main(["traffic", f, w, "--kernel", "gemm_down_resid", "--config", "c3_stack", "--skip-first", "2",
            "--out", str(out)])
    rec = json.loads(out.read_text())
    fr, wr = rec["counter_runs"]["fetch"], rec["counter_runs"]["write"]
    assert fr["copy_factor"] == pytest.approx(2.0) and wr["copy_factor"] == pytest.approx(1.0)
    assert fr["launches"] == 2 and fr["kernels_per_launch"] == 2
    assert fr["raw_kib_per_launch"] == pytest.approx(110.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(110.0 * 1024 * 2 + 10.0 * 1024)
    assert rec["source_file"] == "gemm.hip" and rec["source_sha256_16"] == R.source_hash("gemm.hip")
    capsys.readouterr()


def test_mfma_share_over_the_last_chunks(tmp_path):
    # 3 chunks of one MLP-up launch each, the last 2 kept; busy cycles summed
    # over 1024 SIMDs, active cycles summed over 8 XCDs
    rows = []
    for i in range(3):
        rows += [(UP, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0 if i == 0 else 1024 * 250.0),
                 (UP, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 10.0),
                 (UP, "GRBM_GUI_ACTIVE", 8 * 1000.0)]
    rec = R.mfma_summary(_db(tmp_path / "m.db", rows), chunks=3, last=2, simds=1024, xcds=8)
    k = rec["kernels"]["gemm_up_gelu"]
    assert k["launches"] == 2
    assert k["mfma_util"] == pytest.approx(0.25)
    assert k["gpu_active_cycles_per_xcd"] == pytest.approx(1000.0)
    assert k["bf16_mfma_flops"] == pytest.approx(10.0 * 512)


def test_sq_shares_weight_launches_by_wave_cycles(tmp_path):
    rows = []
    for cyc, wait, dep in ((100.0, 50.0, 20.0), (300.0, 30.0, 60.0)):
        rows += [(UP, "SQ_WAVES", 64.0), (UP, "SQ_WAVE_CYCLES", cyc), (UP, "SQ_WAIT_ANY", wait),
                 (UP, "SQ_WAIT_INST_ANY", dep), (UP, "SQ_ACTIVE_INST_VALU", 40.0), (UP, "SQ_ACTIVE_INST_LDS", 4.0)]
    (kn, n, waves, sh, tot), = R.sq_summary(_db(tmp_path / "s.db", rows))
    assert kn == UP and n == 2 and waves == pytest.approx(64.0) and tot == pytest.approx(400.0)
    assert sh["SQ_WAIT_ANY"] == pytest.approx(80.0 / 400.0)
    assert sh["SQ_WAIT_INST_ANY"] == pytest.approx(80.0 / 400.0)
    assert sh["SQ_ACTIVE_INST_VALU"] == pytest.approx(80.0 / 400.0)
    assert sh["SQ_ACTIVE_INST_LDS"] == pytest.approx(8.0 / 400.0)


def test_stats_keep_the_timed_steps(tmp_path):
    # 2 warm-up + 3 timed steps of one kernel: durations 9, 9, then 1, 2, 3 us;
    # a copy launched a number of times that does not divide is kept whole
    ks = [(UP, d * 1e3) for d in (9.0, 9.0, 1.0, 2.0, 3.0)] + [(COPY, 5e3)] * 7
    rows = {n: (c, t, a) for n, c, t, a in R.kernel_stats_timed(_db(tmp_path / "k.db", kernels=ks), 3, 2)}
    assert rows[UP] == (3, pytest.approx(6.0), pytest.approx(2.0))
    assert rows[COPY][0] == 7
