"""The benchmark's algorithmic pair counts (the numerators of its TFLOP/s
figures) agree with the oracle's allowed-pair definitions."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("N,W,stride", [(100, 7, 0), (300, 64, 16), (257, 1, 0), (64, 100, 5)])
def test_causal_pairs(N, W, stride):
    assert bench.allowed_pairs(N, W, stride) == oracle.allowed_pair_count(N, W, stride)


@pytest.mark.parametrize("N,left,right", [(50, 3, 7), (40, 0, 0), (33, 40, 2)])
def test_two_sided_pairs(N, left, right):
    assert bench.two_sided_pairs(N, left, right) == int(oracle.allowed_mask_two_sided(N, left, right).sum())


@pytest.mark.parametrize("N,W,g", [(60, 5, [0, 7, 30, 59]), (100, 10, list(range(0, 100, 9))), (20, 3, [])])
def test_global_pairs(N, W, g):
    assert bench.global_pairs(N, W, g) == int(oracle.allowed_mask_global(N, W, g).sum())


def test_gpu_count_above_one_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_labels_follow_the_routing_rule():
    from sparse_causal_attention_band_amd import inputs
    assert bench.band_kernel_name(inputs.MISTRAL) == "band8_kernel<d=128, band>"
    assert bench.band_kernel_name(inputs.GEMMA) == "band8_kernel<d=128, band>"
    assert bench.band_kernel_name(inputs.STRIDED) == "band_fwd_kernel<bf16, d=64, strided, key split>"


class _FakeSmi:
    """Stand-in for the management library: a metrics table that shows the
    idle clocks until `switch` seconds after the first read, then loaded ones."""

    def __init__(self, switch):
        import time
        self.t0, self.switch, self.time = None, switch, time

    def amdsmi_init(self):
        pass

    def amdsmi_shut_down(self):
        pass

    def amdsmi_get_processor_handles(self):
        return [0]

    def amdsmi_get_gpu_metrics_info(self, h):
        now = self.time.perf_counter()
        if self.t0 is None:
            self.t0 = now
        if now - self.t0 < self.switch:
            return {"current_gfxclks": [100] * 8}
        # eight XCDs and an unused slot (65535), which the reading drops
        return {"current_gfxclks": [1800, 1900, 1850, 1850, 1850, 1800, 1900, 1850, 65535]}


class _FakeTorch:
    class cuda:
        @staticmethod
        def synchronize():
            pass


def test_smi_clock_keeps_only_refreshed_samples(monkeypatch):
    """The clock is the median over kept samples of the mean over the XCDs
    (unused slots dropped), and only samples from 1.2 s on that differ from
    the idle table count."""
    import sys
    import time
    monkeypatch.setitem(sys.modules, "amdsmi", _FakeSmi(switch=0.5))
    got = bench.smi_clock_under_load(lambda: time.sleep(0.001), _FakeTorch, 1.0, seconds=1.6)
    assert got["sclk_mhz"] == 1850.0 and got["samples"] > 0 and len(got["xcd_mhz"]) == 8


def test_smi_clock_reports_a_table_that_never_refreshed(monkeypatch):
    import sys
    import time
    monkeypatch.setitem(sys.modules, "amdsmi", _FakeSmi(switch=100.0))
    got = bench.smi_clock_under_load(lambda: time.sleep(0.001), _FakeTorch, 1.0, seconds=1.4)
    assert "sclk_mhz" not in got and "did not refresh" in got["error"]
