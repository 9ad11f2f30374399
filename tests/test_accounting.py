"""CPU tests of the workload definitions and the work/traffic accounting."""
import numpy as np
import pytest
import torch

from bruteforce import visible_mask
from parallax_local_linear_amd import accounting, workloads


@pytest.mark.parametrize("L,window,n_sink", [
    (1, 0, 0), (7, 0, 0), (50, 1, 0), (50, 5, 0), (50, 5, 3), (50, 49, 4), (50, 50, 4),
    (50, 80, 2), (40, 3, 40), (33, 7, 60)])
def test_visible_pairs_matches_mask_count(L, window, n_sink):
    assert accounting.visible_pairs(L, window, n_sink) == int(visible_mask(L, window, n_sink).sum())


def test_local_workload_pair_count():
    # 128-key window + 4 sinks over 16384 positions
    assert accounting.visible_pairs(16384, 128, 4) == 2154042


def test_headline_flops():
    cfg = workloads.PREFILL_17B
    assert accounting.prefill_flops(cfg) == 8 * 128 * 2 * 16 * 8192 * 8193 // 2


def test_inputs_are_seeded_and_shaped():
    cfg = workloads.TINY
    a = workloads.prefill_inputs(cfg, dtype=torch.float32)
    b = workloads.prefill_inputs(cfg, dtype=torch.float32)
    for x, y in zip(a, b):
        assert x.shape == (1, 2, 256, 64)
        assert torch.equal(x, y)
    assert not torch.equal(a[0], a[1])
    q, k, v, r = workloads.prefill_inputs(workloads.Prefill("t", 2, 1, 1, 64, 64, 64 ** -0.25),
                                          dtype=torch.float32)
    assert abs(float(q.std()) - 64 ** -0.25) < 0.05
    assert np.isfinite(q.numpy()).all()
