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
