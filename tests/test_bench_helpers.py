"""Host-side helpers of bench.py: the shader-clock sampler reads the current level of a
sysfs pp_dpm_sclk file in either of its formats and summarises the samples."""

import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))

import bench  # noqa: E402


def _sampler(tmp_path, text):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    s = bench.SclkSampler.__new__(bench.SclkSampler)
    s.path, s.samples = str(p), []
    return s


def test_current_level_line(tmp_path):
    # the current clock as its own "S:" line (as on MI355X), or a marked DPM level
    assert _sampler(tmp_path, "S: 1652Mhz *\n0: 500Mhz\n1: 2400Mhz\n")._read() == 1652.0
    assert _sampler(tmp_path, "0: 500Mhz\n1: 2400Mhz *\n")._read() == 2400.0
    assert _sampler(tmp_path, "0: 500Mhz\n1: 2400Mhz\n")._read() is None


def test_stats(tmp_path):
    s = _sampler(tmp_path, "S: 1600Mhz *\n")
    assert s.stats() is None
    s.samples = [1400.0, 1600.0, 1500.0]
    st = s.stats()
    assert (st["median"], st["min"], st["max"], st["samples"]) == (1500.0, 1400.0, 1600.0, 3)
    assert str(tmp_path) in st["source"]
