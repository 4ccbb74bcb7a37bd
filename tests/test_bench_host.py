"""Host-side checks of bench.py's bookkeeping (no GPU).

* The per-call algorithmic bytes and flops that the call rooflines divide by
  agree with the figures derived independently from the workload shapes:
  13.01 / 129.4 / 16.32 / 18.96 GB and 0.673 / 6.84 / 1.68 / 43.05 TFLOP per
  call for the LingBot batch-1, V2-shaped, E4M3-weight and batch-64
  workloads (weights streamed once per Euler step, the prefix K/V read once
  per step, modulation and time-MLP weights once per call).
* The kernel-name patterns by which the counter summaries pick a layer's
  kernel families out of a rocprofv3 trace match the kernels in the
  committed batch-1 kernel statistics, and the committed traffic summary
  holds a figure for every family.
* The report-line check that bench.py runs on its own JSON line accepts a
  well-formed line and names each kind of defect (missing keys, wrong
  types, a roofline fraction that is not achieved / peak, a value that does
  not follow from the time per step).
"""
import csv
import os

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cfg_id, gbytes, tflop", [(2, 13.01, 0.673), (3, 129.4, 6.84), (4, 16.32, 1.68),
                                                    (5, 18.96, 43.05)])
def test_call_work_matches_the_workload_figures(cfg_id, gbytes, tflop):
    by, fl = bench.call_work(synth.config(cfg_id))
    assert by / 1e9 == pytest.approx(gbytes, rel=2e-3)
    assert fl / 1e12 == pytest.approx(tflop, rel=2e-3)


def _profiled_kernel_names():
    path = os.path.join(ROOT, "profiles", "denoise_loop_lingbot_b1_kernel_stats.txt")
    with open(path) as fh:
        rows = [line for line in fh if not line.startswith("#")]
    return [r["Name"] for r in csv.DictReader(rows)]


def test_counter_kernel_patterns_match_the_profiled_kernels():
    names = _profiled_kernel_names()
    assert names, "no kernels in the committed batch-1 kernel statistics"
    for fam, (pattern, which, per_layer) in bench.TRAFFIC_KERNELS.items():
        assert any(pattern in n for n in names), (fam, pattern)
        assert 0 <= which < per_layer


def test_traffic_summary_has_every_family():
    with open(bench.TRAFFIC_SUMMARY) as fh:
        text = fh.read()
    assert "source_sha256_16:" in text
    for fam in bench.TRAFFIC_KERNELS:
        assert f"traffic_bytes_per_launch.{fam}:" in text, fam


def _good_line():
    # the shape of a report line (figures of a batch-1 call of 13.04 ms)
    return {"metric": bench.METRIC, "value": 766.98, "unit": "denoise_steps/s", "n_gpus": 1, "steps": 30,
            "warmup": 5, "ms_per_step": 13.0381, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "lingbot_b1", "batch": 1, "euler_steps": 10},
            "roofline": {"bound": "hbm", "achieved": 1888.29, "peak": 8000.0, "unit": "GB/s", "frac": 0.236,
                         "traffic": 18314000},
            "cpu_baseline": {"value": 7.84, "unit": "denoise_steps/s", "cores": 16, "kind": "oracle",
                             "sample": "17 Euler steps"}}


def test_report_line_check_accepts_a_well_formed_line():
    assert bench.check_line(_good_line()) == []


@pytest.mark.parametrize("edit, expect", [
    (lambda d: d.pop("roofline"), "missing roofline"),
    (lambda d: d.pop("vs_baseline"), "missing vs_baseline"),
    (lambda d: d.update(n_gpus=True), "n_gpus has type bool"),
    (lambda d: d.update(scaling="linear"), "scaling"),
    (lambda d: d["config"].pop("workload"), "workload"),
    (lambda d: d["roofline"].pop("traffic"), "traffic"),
    (lambda d: d["roofline"].update(frac=0.5), "achieved / peak"),
    (lambda d: d["roofline"].update(bound="latency"), "bound"),
    (lambda d: d["cpu_baseline"].pop("cores"), "cores"),
    (lambda d: d.update(value=700.0), "ms_per_step"),
])
def test_report_line_check_names_each_problem(edit, expect):
    d = _good_line()
    edit(d)
    problems = bench.check_line(d)
    assert any(expect in p for p in problems), problems
