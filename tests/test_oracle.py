"""CPU: the fp64 oracle against its pins (library routines, the flat exact
search, closed forms, special cases) and the input generator's encoders."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import pins
from tests import support


def test_hand_example():
    pins.pin_hand_example()


def test_codecs_all_codes():
    pins.pin_codecs()


def test_flat_search_tiny_all_tokens():
    pins.pin_against_flat_search(synthetic.WORKLOADS["tiny"])


def test_flat_search_mid_sample():
    wl = synthetic.WORKLOADS["mid"]
    pins.pin_against_flat_search(wl, tokens=np.arange(0, wl.B, 16))


def test_flat_search_random_gamma_beta():
    wl = synthetic.Workload("gb", 24, 64, 3, 20, 5, "f32", "random")
    pins.pin_against_flat_search(wl, gamma_beta=True)


@pytest.mark.parametrize("table", ["bf16", "e4m3", "int8", "int4"])
def test_flat_search_quantised_tables(table):
    wl = synthetic.Workload("q", 24, 128, 2, 24, 8, table, "random")
    pins.pin_against_flat_search(wl, seed=2)


def test_select_against_brute_force_grid():
    pins.pin_select()


def test_gather_against_embedding_bag():
    pins.pin_gather()


def test_running_update_against_torch():
    pins.pin_running_update()


def test_integer_ties_every_k():
    pins.pin_integer_ties()


def test_k_equals_1():
    pins.pin_k_equals_1()


def test_k_equals_n_keys():
    wl = synthetic.Workload("kn", 12, 32, 2, 6, 6, "f32", "random")
    pins.pin_against_flat_search(wl, seed=4)


def test_softmax_large_scores():
    pins.pin_softmax_large_scores()


def test_op_counts():
    pins.pin_op_counts()


def test_invariants_mid():
    """Sum of weights is 1, k^2 candidates, distinct in-range indices sorted
    by non-increasing score, non-increasing weights."""
    wl = synthetic.WORKLOADS["mid"]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)[:128]
    r = oracle.run(support.model_for(wl, params), x, want=("idx", "top", "w", "ncand"))
    np.testing.assert_allclose(r["w"].sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (r["ncand"] == wl.k ** 2).all()
    assert ((r["idx"] >= 0) & (r["idx"] < wl.N)).all()
    s = np.sort(r["idx"], -1)
    assert (s[..., 1:] != s[..., :-1]).all()
    assert (np.diff(r["top"], axis=-1) <= 0).all()
    assert (np.diff(r["w"], axis=-1) <= 0).all()


def test_gap_clean_redraws_and_converges():
    wl = synthetic.WORKLOADS["mid"]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)[:256].copy()
    x0 = x.copy()
    attempts = support.gap_clean(wl, params, x)
    gap, tau = support.gaps_and_tau(wl, params, x)
    assert (gap >= tau).all()
    changed = (x != x0).any(1)
    assert (changed == (attempts > 0)).all()


def test_bf16_encoder_matches_torch():
    a = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32) * 3
    a[:4] = [0.0, -0.0, 1e-40, -3.3895314e38]
    got = synthetic.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == ref).all()


def test_e4m3_encoder_is_nearest_code():
    """Each stored code is the nearest E4M3 value to a/scale (ties to even),
    scale = row max / 448."""
    a = np.random.default_rng(1).standard_normal((64, 96)).astype(np.float32)
    codes, scale = synthetic.f32_to_e4m3_rows(a)
    np.testing.assert_allclose(scale, np.abs(a).max(1) / 448.0, rtol=1e-7)
    table = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    finite = ~np.isnan(table)
    y = (a / scale[:, None]).astype(np.float64)
    dist = np.abs(y[..., None] - np.where(finite, table, np.inf)[None, None, :])
    best = dist.min(-1)
    got = np.abs(y - table[codes])
    assert (got <= best + 1e-12).all()
    assert (np.abs(table[codes]) <= 448).all()


@pytest.mark.parametrize("bits,qmax", [(8, 127), (4, 7)])
def test_integer_encoders_are_nearest_codes(bits, qmax):
    """int8 / int4 codes: the nearest integer to a / scale (ties to even) in
    [-qmax, qmax], scale = row max / qmax; int4 codes two per byte."""
    a = np.random.default_rng(2).standard_normal((64, 96)).astype(np.float32)
    a[3] = 0.0  # an all-zero row: scale 1, codes 0
    if bits == 8:
        codes, scale = synthetic.f32_to_int8_rows(a)
        q = codes.astype(np.float64)
    else:
        packed, scale = synthetic.f32_to_int4_rows(a)
        assert packed.shape == (64, 48)
        q = pins.unpack_int4(packed).astype(np.float64)
    amax = np.abs(a).max(1)
    np.testing.assert_allclose(scale, np.where(amax > 0, amax / qmax, 1.0), rtol=1e-7)
    y = (a / scale[:, None]).astype(np.float64)
    assert (np.abs(q) <= qmax).all()
    assert (np.abs(y - q) <= 0.5 + 1e-6).all()
    assert not q[3].any()


def test_generator_is_deterministic_and_seeded():
    wl = synthetic.Workload("g", 4, 64, 2, 64, 4, "bf16", "random")
    p1, p2, p3 = synthetic.make_params(wl, 0), synthetic.make_params(wl, 0), synthetic.make_params(wl, 1)
    for key in p1:
        if p1[key] is None:
            continue
        assert (p1[key] == p2[key]).all()
    assert not (p1["wq"] == p3["wq"]).all()
    assert (synthetic.redraw_row(wl, 0, 3, 1) == synthetic.redraw_row(wl, 0, 3, 1)).all()
    assert not (synthetic.redraw_row(wl, 0, 3, 1) == synthetic.redraw_row(wl, 0, 3, 2)).all()


def test_usage_counts_match_bincount():
    """Slot usage against numpy's bincount, accumulated over two calls."""
    rng = np.random.default_rng(4)
    N = 5000
    a = rng.integers(0, N, 30000).astype(np.int32)
    b = rng.integers(0, 40, 777).astype(np.int32)  # hot rows
    got = oracle.usage(b, N, oracle.usage(a, N))
    ref = np.bincount(np.concatenate([a, b]), minlength=N)
    assert (got == ref).all()
    with pytest.raises(ValueError):
        oracle.usage(np.array([N], np.int32), N)
