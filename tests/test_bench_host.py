"""Host-side pieces of bench.py: the FLOP count behind the metric, the clock sampler's parser, the
counter-CSV reader and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from exact_io_aware_21_amd import inputs


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 1), ("window", 7),
                                         ("window", 500), ("document", 0)])
def test_allowed_pairs_matches_brute_force(mask, window):
    """The closed-form pair count (the numerator of the metric) equals the count of the oracle's
    allowed() over every (query, key) pair."""
    extra = {"doc_len_range": (1, 40)} if mask == "document" else {}
    w = inputs.Workload("t", B=2, H=3, N=131, d=64, mask=mask, window=window, seed=5, **extra)
    offs = inputs.make_inputs(w)["doc_offsets"] if mask == "document" else None
    rows = np.arange(w.N)
    brute = 0
    for b in range(w.B):
        ok = oracle.allowed(rows, rows, w.N, mask, window, None if offs is None else offs[b])
        brute += int(ok.sum()) * w.H
    assert bench.allowed_pairs(w, offs) == brute


def test_sclk_parser(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\n1: 2057Mhz *\n2: 2400Mhz\n")
    assert bench.SclkSampler._read(str(p)) == 2057.0
    p.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.SclkSampler._read(str(p)) is None
    assert bench.SclkSampler._read(str(tmp_path / "missing")) is None


def test_pmc_average(tmp_path):
    p = tmp_path / "c.csv"
    p.write_text("Kernel_Name,Counter_Name,Counter_Value\n"
                 "copy_kernel(float4 const*),FETCH_SIZE,100\n"
                 "copy_kernel(float4 const*),FETCH_SIZE,300\n"
                 "other,FETCH_SIZE,7\n"
                 "copy_kernel(float4 const*),WRITE_SIZE,5\n")
    assert bench._pmc_avg(str(p), "FETCH_SIZE", "copy_kernel") == 200.0
    with pytest.raises(SystemExit):
        bench._pmc_avg(str(p), "FETCH_SIZE", "fwd_kernel")


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_clock_scaled_peak_never_above_one():
    """A fraction of the clock-scaled peak above 1 cannot be a measurement (the sampled clock
    lagged the hardware): it is withheld, with a note, instead of being printed."""
    rec = bench.clock_scaled_peak({"median": 800.0}, 2500.0, 1100.0)
    assert rec["frac_of_that_peak"] is None and "note" in rec
    rec = bench.clock_scaled_peak({"median": 1800.0}, 2500.0, 1100.0)
    assert rec["frac_of_that_peak"] == round(1100.0 / (2500.0 * 1800.0 / 2400.0), 4) <= 1.0
    assert bench.clock_scaled_peak(None, 2500.0, 1.0) is None


def test_clock_sampler_drops_samples_before_start():
    s = bench.SclkSampler(period_s=0.001, started=lambda: False)
    s.path = __file__  # any readable file: no '*' line, so nothing is parsed
    s.samples.clear()
    assert s.summary() is None


def test_clock_sampler_skips_short_steps():
    s = bench.SclkSampler(step_ms=0.05)
    assert s.path is None
    with s:
        pass
    rec = s.summary()
    assert "skipped" in rec
    assert bench.clock_scaled_peak(rec, 2500.0, 1.0) == rec
    assert not bench.SclkSampler(step_ms=5.0).skipped
    assert not bench.SclkSampler().skipped
