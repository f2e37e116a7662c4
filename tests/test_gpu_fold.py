"""GPU: the folded lookup (pkm_prepare with PKM_PREPARE_FOLD).

The projection, inference batch-norm and subkeys are linear, so for fixed
statistics the half scores are one contraction of x with a matrix per half
of a head plus a per-key shift, folded once in fp64.  The scores then
differ from the unfolded path's by fp32 rounding, so the checks are against
the fp64 oracle with the lookup's rules, not bit for bit:
- the folded half scores' error is within half the parity margin tau on
  every (token, head) (the same guard the unfolded scoring passes);
- the folded forward matches the oracle on every token of small, chunked
  and full-size workloads (indices exact on gap-clean inputs, weights and
  outputs within the table's tolerance);
- its stages compose to it bit for bit; arrays other than the folded ones,
  pkm_forward_train and n_keys > D take the unfolded path (bit for bit the
  unprepared results).
"""
import numpy as np
import pytest

import oracle
import product_key_memory_amd as pk
import synthetic
from tests import support
from tests.support import say
from tests.test_gpu_forward import _full_size, compare, invariants

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


def _same(a, b):
    import torch

    return all(torch.equal(u, v) for u, v in zip(a, b))


def _score_error_over_tau(wl, params, x, s):
    """max over (token, head) of (max|ds0| + max|ds1|) / tau for GPU half
    scores s [B, H, 2, n] against fp64."""
    r = oracle.run(support.model_for(wl, params), x, kk=min(wl.k + 1, wl.n), want=("qhat", "idx", "top"))
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    tau = support.taus(wl, params, r["qhat"], r["idx"][:, :, wl.k - 1])
    worst = 0.0
    for h in range(wl.H):
        err = 0.0
        for p in range(2):
            ref = r["qhat"][:, h, p * half:(p + 1) * half] @ sub[h, p].T
            err = err + np.abs(s[:, h, p].astype(np.float64) - ref).max(axis=1)
        worst = max(worst, float((err / tau[:, h]).max()))
    return worst


@pytest.mark.parametrize("name", ["tiny", "mid", "default"])
def test_folded_score_error_guard(torch, name):
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl, with_values=False)
    x = synthetic.make_x(wl)[:: max(1, wl.B // 96)][:96].copy()
    say("folded score error guard", name, "tokens", x.shape[0])
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "bf16")
    P = pk.Params(*[support.to_device(params[key]) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")],
                  None)
    xt = support.to_device(x)
    unfolded = mem.half_scores(P, xt).cpu().numpy()
    mem.prepare(P, "fold")
    folded = mem.half_scores(P, xt).cpu().numpy()
    w_fold = _score_error_over_tau(wl, params, x, folded)
    w_plain = _score_error_over_tau(wl, params, x, unfolded)
    print(f"{name}: max full-score error / tau: folded {w_fold:.3f}, unfolded {w_plain:.3f}", flush=True)
    assert w_fold <= 0.5


def test_folded_scores_with_wide_ranges(torch):
    """Token rows scaled by 2^+-30 and random batch-norm statistics: the
    folded scores stay within fp32-level error of fp64 (relative to the
    L1 mass sum |q^_i| |c_i|, as the unfolded scoring is tested)."""
    wl = synthetic.Workload("wide", 64, 256, 3, 200, 8, "f32", "random")
    params = synthetic.make_params(wl, seed=61, with_values=False)
    x = synthetic.make_x(wl, seed=61)
    rng = np.random.default_rng(61)
    x *= np.exp2(rng.integers(-30, 31, size=(wl.B, 1))).astype(np.float32)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32")
    P = pk.Params(*[support.to_device(params[key]) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")],
                  None)
    mem.prepare(P, "fold")
    say("folded scores, wide ranges")
    s = mem.half_scores(P, support.to_device(x)).cpu().numpy().astype(np.float64)
    r = oracle.run(support.model_for(wl, params), x, want=("qhat",))
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    for h in range(wl.H):
        for p in range(2):
            q = r["qhat"][:, h, p * half:(p + 1) * half]
            ref = q @ sub[h, p].T
            mass = np.abs(q) @ np.abs(sub[h, p]).T
            assert (np.abs(s[:, h, p] - ref) <= 2e-6 * mass + 1e-30).all()


CASES = [
    # (B, D, H, n, k, table, bn, max_batch)
    (8, 64, 1, 16, 4, "f32", "unit", 8),
    (1024, 512, 4, 256, 16, "f32", "random", 1024),
    (700, 320, 5, 256, 7, "e4m3", "random", 256),    # three chunks, D = 320
    (300, 1024, 3, 1024, 32, "bf16", "random", 300),  # n_keys = D, fused select-gather
    (4500, 1024, 4, 1024, 32, "bf16", "unit", 4500),  # persistent walk, ragged last row tile
]


def _ids(c):
    return "B{}-D{}-H{}-n{}-k{}-{}-{}-mb{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_folded_forward_against_oracle(torch, case):
    B, D, H, n, k, table, bn, mb = case
    wl = synthetic.Workload("folded", B, D, H, n, k, table, bn)
    params = synthetic.make_params(wl, seed=62)
    x = synthetic.make_x(wl, seed=62)
    _, tau = support.gap_clean(wl, params, x, seed=62, want_tau=True)
    mem = pk.Memory(D, H, n, k, table, max_batch=mb)
    P = pk.params_to_device(params, table, support.device())
    mem.prepare(P, "fold")
    say("folded forward vs oracle", _ids(case))
    out, idx, w = support.gpu_forward(wl, params, x, mem=mem, dev_params=P)
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w, tau=tau)


@pytest.mark.slow
def test_folded_forward_full_default_every_token(torch):
    """The benchmark's configuration: all 4,096 tokens of the default
    workload through the folded forward in one call, against the oracle."""
    wl, params, x, tau, _, _, _ = _full_size("default")
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=wl.B)
    P = pk.params_to_device(params, wl.table, support.device())
    mem.prepare(P, "fold")
    say("folded forward, full default")
    out, idx, w = support.gpu_forward(wl, params, x, mem=mem, dev_params=P)
    invariants(wl, idx, w)
    err = compare(wl, params, x, out, idx, w, tau=tau)
    print(f"folded default: max row error {err.max():.3g}", flush=True)


def test_folded_stages_and_which_path(torch):
    B, D, H, n, k, table = 300, 1024, 3, 1024, 32, "bf16"
    wl = synthetic.Workload("folded", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=63)
    xt = support.to_device(synthetic.make_x(wl, seed=63))
    P = pk.params_to_device(params, table, support.device())
    mem = pk.Memory(D, H, n, k, table, max_batch=B)
    say("folded stages; unfolded paths")
    plain = mem.forward(P, xt)
    plain_train = mem.forward_train(P, xt)
    mem.prepare(P, "fold")
    folded = mem.forward(P, xt)
    out = torch.full_like(folded[0], float("nan"))
    idx = torch.full_like(folded[1], -1)
    w = torch.full_like(folded[2], float("nan"))
    for stage in range(4):
        mem.forward_stage(P, xt, stage, out, idx, w)
    train = mem.forward_train(P, xt)  # needs the projection: not folded
    # other batch-norm arrays (same values, other memory): not the folded ones
    P2 = pk.Params(*[P[name] if name not in ("bn_var",) else P[name].clone()
                     for name in ("wq", "bn_mean", "bn_var", "bn_gamma", "bn_beta", "subkeys", "values",
                                  "value_scale")])
    other = mem.forward(P2, xt)
    torch.cuda.synchronize()
    assert _same((out, idx, w), folded)
    assert _same(train, plain_train)
    assert _same(other, plain)
    assert not torch.equal(folded[0], plain[0])  # the folded scores round differently
    # n_keys > D: folding would add work; the split form is prepared instead
    wl2 = synthetic.Workload("wide_keys", 200, 64, 2, 128, 8, "f32", "random")
    params2 = synthetic.make_params(wl2, seed=64)
    P3 = pk.params_to_device(params2, "f32", support.device())
    x2 = support.to_device(synthetic.make_x(wl2, seed=64))
    mem2 = pk.Memory(wl2.D, wl2.H, wl2.n, wl2.k, "f32", max_batch=wl2.B)
    ref = mem2.forward(P3, x2)
    mem2.prepare(P3, "fold")
    got = mem2.forward(P3, x2)
    torch.cuda.synchronize()
    assert _same(got, ref)


@pytest.mark.slow
def test_folded_forward_large_batch(torch):
    """The large-batch configuration (65,536 tokens in one call) through the
    folded forward, every 4th token against the oracle (the unfolded
    forward is checked on every token elsewhere)."""
    wl, params, x, tau, _, _, _ = _full_size("large_batch")
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=wl.B)
    P = pk.params_to_device(params, wl.table, support.device())
    mem.prepare(P, "fold")
    say("folded forward, large batch")
    out, idx, w = support.gpu_forward(wl, params, x, mem=mem, dev_params=P)
    invariants(wl, idx, w)
    tokens = np.arange(0, wl.B, 4)
    err = compare(wl, params, x, out, idx, w, tokens=tokens, tau=tau[tokens])
    print(f"folded large_batch: max row error {err.max():.3g}", flush=True)
