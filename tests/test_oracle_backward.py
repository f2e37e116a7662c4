"""CPU: the oracle's backward direction against its pins (tests/pins.py):
torch autograd through the method's definition, finite differences,
identities."""
import pytest

import synthetic
from tests import pins


@pytest.mark.parametrize("wl,gamma_beta", [
    (synthetic.WORKLOADS["tiny"], False),
    (synthetic.Workload("gb", 24, 64, 3, 20, 5, "f32", "random"), True),      # heads, random BN, gamma, beta
    (synthetic.Workload("bf", 16, 64, 2, 16, 8, "bf16", "unit"), False),      # bf16 table
    (synthetic.Workload("e4", 16, 128, 2, 24, 6, "e4m3", "random"), True),   # E4M3 table + row scales
    (synthetic.Workload("kn", 8, 32, 1, 6, 6, "f32", "random"), False),       # k = n_keys
    (synthetic.Workload("k1", 12, 32, 2, 10, 1, "f32", "random"), True),      # k = 1: softmax is constant
])
def test_backward_matches_autograd(wl, gamma_beta):
    g = pins.pin_backward_autograd(wl, gamma_beta=gamma_beta)
    if wl.k == 1:
        # one winner per head: w = 1 has no gradient, so nothing flows to the scores
        assert not g["dsub"].any() and not g["dwq"].any() and not g["dx"].any()


def test_backward_mid_sample_matches_autograd():
    wl = synthetic.WORKLOADS["mid"].with_(B=48)
    pins.pin_backward_autograd(wl)


def test_backward_finite_differences():
    pins.pin_backward_finite_differences()


def test_backward_identities():
    pins.pin_backward_identities()


def test_backward_thread_count_does_not_change_bits():
    import numpy as np

    import oracle

    wl = synthetic.Workload("thr", 37, 64, 2, 16, 4, "e4m3", "random")
    params, x, dout = pins.backward_case(wl, 8, gamma_beta=True)
    model = oracle.Model.from_params(params, wl.k, wl.table)
    a = oracle.backward(model, x, dout, nthreads=1)
    b = oracle.backward(model, x, dout, nthreads=7)
    for name in oracle.GRADS:
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("wl", [
    synthetic.Workload("bs1", 24, 64, 3, 20, 5, "f32", "random"),
    synthetic.Workload("bs2", 16, 128, 2, 24, 6, "e4m3", "random"),
    synthetic.Workload("bs3", 2, 32, 1, 8, 4, "bf16", "unit"),     # the smallest batch with a variance
])
def test_batch_stats_match_torch(wl):
    pins.pin_batch_stats_autograd(wl)


def test_batch_stats_finite_differences():
    pins.pin_batch_stats_finite_differences()
