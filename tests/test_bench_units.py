"""The benchmark's throughput arithmetic, pinned to the figures the FP8 kernel
write-up prints (demingchina.com/news/60142, section 4.4 table and section 2.2
roofline numbers; golden fixture tests/golden/perf_table.json).  CPU only."""
import json
import os

import pytest

import bench


def test_tflops_formula_reproduces_the_page_table(golden_dir):
    rows = json.load(open(os.path.join(golden_dir, "perf_table.json")))["rows"]
    for r in rows:
        got = bench.gemm_tflops(r["M"], r["N"], r["K"], r["ms"] * 1e-3)
        # the page rounds times to 2 significant digits and TFLOPS to ~3
        assert got == pytest.approx(r["tflops"], rel=0.03), r


def test_roofline_numbers_of_the_page(golden_dir):
    rl = json.load(open(os.path.join(golden_dir, "perf_table.json")))["roofline"]
    n = rl["n"]
    # 2n^3 FLOP over 3n^2 one-byte elements = 2n/3
    assert bench.intensity(n, n, n, 1.0) == pytest.approx(rl["intensity_flop_per_byte"], rel=0.01)
    assert rl["peak_tflops"] / rl["hbm_tb_s"] == pytest.approx(rl["balance_flop_per_byte"], rel=0.01)


def test_gpus_other_than_one_are_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "8"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
