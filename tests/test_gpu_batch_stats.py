"""GPU: the lookup and its gradients with training-mode BN (batch
statistics; pkm_forward_batch_stats, pkm_backward_batch_stats) against the
fp64 oracle (pinned to torch's F.batch_norm(training=True) in
tests/pins.py).

Inputs are gap-clean for the batch-statistics lookup (tests/support.py:
re-drawing a token moves every token's statistics, so the whole batch is
measured again after each round).  Statistics: |mean - ref| within 1e-5 of
the column's standard deviation, var within 1e-4 relative (fp32 sums of B
values); the running statistics within 1e-5 of the oracle's update (pinned
to the buffers torch's F.batch_norm(training=True) updates).  Indices, outputs and weights: the lookup's rules and tolerances.
Gradients: each tensor within 1e-4 of its largest entry, dx per token
within 1e-4 of max(the token's largest entry, the batch median of that) --
as for the running-statistics backward.
"""
import numpy as np
import pytest

import oracle
import product_key_memory_amd as pk
import synthetic
from tests import pins, support
from tests.support import say
from tests.test_gpu_backward import compare

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 2e-2, "int8": 2e-2, "int4": 2e-2}


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


def _to(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(support.device())


def run_case(torch, wl, seed, backward=True, running=True, max_batch=None):
    params, x, dout = pins.backward_case(wl, seed, gamma_beta=True)
    print("[cpu] gap-clean draw with batch statistics", wl.name, flush=True)
    mean, var, tau = support.gap_clean_batch_stats(wl, params, x, seed=seed)
    model = support.model_for(wl, params)
    print("[cpu] oracle lookup", flush=True)
    ref = oracle.run_batch_stats(model, x, mean, var, want=("out", "idx", "top", "w"))
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=max_batch or wl.B)
    P = pk.params_to_device(params, wl.table, support.device())
    xt = _to(torch, x)
    rng = np.random.default_rng([seed, 5])
    rm0 = rng.normal(0, 1, (wl.H, wl.D)).astype(np.float32)
    rv0 = rng.uniform(0.5, 2, (wl.H, wl.D)).astype(np.float32)
    run = (_to(torch, rm0), _to(torch, rv0)) if running else None
    say("forward batch stats", wl, "B =", wl.B)
    out, idx, w, bm, bv = mem.forward_batch_stats(P, xt, running=run, momentum=0.1)
    torch.cuda.synchronize()
    out, idx, w, bm, bv = (t.cpu().numpy() for t in (out, idx, w, bm, bv))

    sd = np.sqrt(var)
    assert (np.abs(bm - mean) <= 1e-5 * sd + 1e-6).all(), float(np.abs(bm - mean).max())
    assert (np.abs(bv - var) <= 1e-4 * var + 1e-7).all(), float((np.abs(bv - var) / var).max())
    support.check_indices(idx, ref["idx"], ref["top"], tau)
    tol = TOL[wl.table]
    assert np.abs(support.weights_by_index(idx, w, ref["idx"]) - ref["w"]).max() <= tol
    assert support.rel_rowmax_err(out, ref["out"]).max() <= tol
    if running:
        rm, rv = (t.cpu().numpy() for t in run)
        want_m, want_v = oracle.running_update(rm0, rv0, mean, var, wl.B, 0.1)
        assert np.abs(rm - want_m).max() <= 1e-5 * (np.abs(want_m).max() + 1)
        assert np.abs(rv - want_v).max() <= 1e-5 * np.abs(want_v).max()
    if not backward:
        return
    say("backward batch stats", wl)
    g = mem.backward(P, xt, _to(torch, idx), _to(torch, w), _to(torch, dout), batch_stats=(_to(torch, bm), _to(torch, bv)))
    torch.cuda.synchronize()
    got = {name: t.cpu().numpy() for name, t in g.items()}
    print("[cpu] oracle gradients", flush=True)
    gref = oracle.backward_batch_stats(model, x, dout, mean, var)
    errs = compare(got, gref)
    print(wl.name, {k: f"{v:.2g}" for k, v in errs.items()}, flush=True)


@pytest.mark.parametrize("wl", [
    synthetic.Workload("bn_tiny", 8, 64, 1, 16, 4, "f32", "unit"),
    synthetic.Workload("bn_mid", 512, 256, 4, 64, 16, "f32", "random"),
    synthetic.Workload("bn_bf", 100, 128, 2, 40, 8, "bf16", "random"),     # ragged B
    synthetic.Workload("bn_e4", 64, 192, 3, 24, 6, "e4m3", "random"),      # D = 3 * 64
    synthetic.Workload("bn_small", 4, 64, 1, 12, 3, "f32", "unit"),        # a batch of four
])
def test_batch_stats_forward_and_backward(torch, wl):
    run_case(torch, wl, 1)


def test_batch_stats_without_running_update(torch):
    run_case(torch, synthetic.Workload("bn_norun", 40, 64, 2, 16, 4, "f32", "random"), 2, backward=False,
             running=False)


@pytest.mark.slow
def test_batch_stats_default_shape(torch):
    """The 1M-row bf16 table of the default shape, on a batch of 256."""
    wl = synthetic.WORKLOADS["default"].with_(B=256)
    run_case(torch, wl, 0)


def test_batch_stats_arguments(torch):
    wl = synthetic.Workload("bn_err", 8, 64, 1, 16, 4, "f32", "unit")
    params = synthetic.make_params(wl)
    P = pk.params_to_device(params, wl.table, support.device())
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=4)
    say("batch stats arguments")
    x = torch.zeros((8, wl.D), device=support.device())
    for bad in (x[:1], x[:5]):  # B = 1: no variance; B > max_batch: not one pass
        with pytest.raises(pk.PkmError) as e:
            mem.forward_batch_stats(P, bad.contiguous())
        assert e.value.status == pk.PKM_E_ARG
    with pytest.raises(pk.PkmError):
        mem.forward_batch_stats(P, x[:4].contiguous(), momentum=1.5)
