"""Host logic of bench.py (no GPU): the roofline's traffic floor, the rank correlation, the sweep's
variants, the rocprofv3 counter passes' per-block limits and the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_xcd_traffic_floor_closed_form():
    # 4096^3 with 256 x 256 tiles: 256 tiles, 32 per XCD; the squarest block in bytes is 4 x 8 tiles,
    # so each XCD reads 4 row panels of A and 8 column panels of B (256 x 4096 x 2 bytes each) once
    panel = 256 * 4096 * 2
    c_bytes = 4096 * 4096 * 2
    assert bench._xcd_traffic_floor() == 8 * (4 + 8) * panel + c_bytes == 234881024
    # one cache holding everything: each operand panel read once
    assert bench._xcd_traffic_floor(xcds=1) == (16 + 16) * panel + c_bytes


def test_rank_corr_ties_in_index_order():
    assert bench.rank_corr([1, 2, 3, 4], [10, 20, 30, 40]) == pytest.approx(1.0)
    assert bench.rank_corr([1, 2, 3, 4], [4, 3, 2, 1]) == pytest.approx(-1.0)
    # ties take ranks in index order: x ranks 0, 1, 2 against y ranks 2, 1, 0
    assert bench.rank_corr([1, 1, 2], [3, 2, 1]) == pytest.approx(-1.0)


def test_sweep_variants():
    names = [n for n, _, _ in bench.MODES]
    assert len(names) == 12 and len(set(names)) == 12
    for name, mode, _ in bench.MODES:
        assert bool(mode & bench.REMAP) == name.endswith("+remap")
    # the 8192^3 target: row-major (the linear baseline of the gain), then the two orders the
    # workload names, each without and with the remap
    assert [n for n, _, _ in bench.C3_MODES][:6] == ["row", "row+remap", "group_major_g8", "serpentine_s8",
                                                     "group_major_g8+remap", "serpentine_s8+remap"]
    for name, mode, _ in bench.C3_MODES:
        assert bool(mode & bench.REMAP) == ("+remap" in name)


def test_host_cpu_fields():
    h = bench._host_cpu()
    assert h["host_logical_cpus"] >= 1 and 1 <= h["usable_cpus"] <= h["host_logical_cpus"]
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)


# per-pass hardware limits of rocprofv3 on this GPU (a pass asking for more cannot be collected):
# 8 SQ_, 4 TCC_ (FETCH_SIZE takes 3, WRITE_SIZE 2), 4 TCP_, 2 TA_, 2 TD_, 2 GRBM_ counters
_COST = {"FETCH_SIZE": ("TCC_", 3), "WRITE_SIZE": ("TCC_", 2)}
_LIMIT = {"SQ_": 8, "TCC_": 4, "TCP_": 4, "TA_": 2, "TD_": 2, "GRBM_": 2}


@pytest.mark.parametrize("tag,ctrs", list(bench.PMC_PASSES) + list(bench.TARGET_PMC_PASSES))
def test_counter_passes_fit_one_run(tag, ctrs):
    used = {}
    for c in ctrs:
        block, n = _COST.get(c, (next((b for b in _LIMIT if c.startswith(b)), None), 1))
        assert block is not None, (tag, c)
        used[block] = used.get(block, 0) + n
    for block, n in used.items():
        assert n <= _LIMIT[block], (tag, block, n)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_rank_corr_matches_the_oracles_and_the_page():
    # bench.py's own Spearman (no oracle import on its measured path) against the oracle's, on
    # random data with ties, and on the page's printed columns (0.045 / 0.064)
    import numpy as np
    from conftest import golden_lines
    from oracle import l2_model
    rng = np.random.default_rng(3)
    for n in (2, 5, 12, 30):
        for _ in range(20):
            x = rng.integers(0, 6, size=n).tolist()
            y = rng.integers(0, 6, size=n).tolist()
            assert abs(bench.rank_corr(x, y) - l2_model.rank_correlation(x, y)) < 1e-12
    rows = [ln.split() for ln in golden_lines("p1_predicted_l2_hit_rates.txt") if not ln.startswith("spearman")]
    pred = [float(r[3]) for r in rows]
    assert round(bench.rank_corr(pred, [float(r[4]) for r in rows]), 3) == 0.045
    assert round(bench.rank_corr(pred, [float(r[5]) for r in rows]), 3) == 0.064


def test_l2_check_cases_are_the_committed_predictions():
    cases = bench._l2_check_cases()
    assert len(cases) == 23
    assert sum(1 for c in cases if c["kind"] == "fit") == 7
    # the fitted rows are the 8192^3 target's seven static orders, in the same order
    assert [c["name"] for c in cases if c["kind"] == "fit"] == [n for n, _, _ in bench.C3_MODES]
    shapes = bench._l2_check_shapes()
    assert shapes == [(8192, 8192, 8192), (8192, 8192, 16384), (8192, 8192, 4096)]
    # every case runs on a grid the persistent kernel tiles exactly
    for c in cases:
        assert c["M"] % 256 == 0 and c["N"] % 256 == 0 and c["K"] % 32 == 0


def test_ranks_desc_and_line_fit():
    assert bench._ranks_desc([87.5, 65.6, 87.5, 32.3]) == [1, 3, 1, 4]
    fit = bench._line_model_fit({"a": {"hit_pct": 80.0, "fetch_mb": 100.0}, "b": {"hit_pct": 30.0, "fetch_mb": 400.0}},
                                {"a": {"l2_hit_pct": 82.0, "fetch_mb": 110.0}, "b": {"l2_hit_pct": 33.0, "fetch_mb": 380.0}})
    assert fit["spearman_vs_measured_hit"] == 1.0 and fit["max_abs_hit_err_pp"] == 3.0
    assert fit["max_rel_fetch_err"] == round(10 / 110, 4)


def test_counter_rows_clock_and_peak_at_clock(tmp_path):
    # a two-dispatch counter CSV as rocprofv3 writes it: the dispatch duration comes from its
    # timestamps; GRBM_GUI_ACTIVE sums the eight XCDs' busy clocks
    path = tmp_path / "x_counter_collection.csv"
    path.write_text(
        '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n'
        '1,"k1","GRBM_GUI_ACTIVE",1600000,1000,101000\n'
        '1,"k1","SQ_BUSY_CYCLES",5,1000,101000\n'
        '2,"k2","GRBM_GUI_ACTIVE",8,0,4\n')
    rows = bench._pmc_rows(str(path))
    assert [r["kernel"] for r in rows] == ["k1", "k2"]
    assert rows[0]["dur_ns"] == 100000.0 and rows[0]["SQ_BUSY_CYCLES"] == 5.0
    clk = bench.sustained_clock(rows[0]["GRBM_GUI_ACTIVE"], rows[0]["dur_ns"])
    assert clk == pytest.approx(2.0)               # 1.6e6 / 8 XCDs over 100 us
    # 2 * 4096^3 flops in 100 us at 2.0 GHz: 1374.4 TFLOP/s against 2500 * 2.0 / 2.4 = 2083.3
    pct = bench.pct_peak_at_clock(2 * 4096 ** 3, rows[0]["dur_ns"], clk)
    assert pct == pytest.approx(100 * 1374.389534720 / (2500 * 2.0 / 2.4))
    assert bench.pct_peak_at_clock(1.0, 0.0, 2.0) is None and bench.sustained_clock(1.0, 0.0) is None
