"""GPU: prepared weights (pkm_prepare).

Preparing converts Wq and the subkeys once into the form the contractions
read (row exponents, fp16 pieces in staging order).  A forward call given
the prepared arrays must produce exactly the bits of the unprepared call --
the pieces are the ones every tile would compute -- on small grids
(128x128 tiles) and persistent ones (256x256), ragged tails, several chunks
and D that is not a power of two.  Calls with other arrays are unaffected;
a re-prepare picks up changed contents; preparing NULL drops the copy.
The lookup itself is checked against the fp64 oracle elsewhere; one case
here checks the prepared forward against it too.
"""
import numpy as np
import pytest

import product_key_memory_amd as pk
import synthetic
from tests import support
from tests.support import say
from tests.test_gpu_forward import compare, invariants

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


CASES = [
    # (B, D, H, n, k, table, max_batch)
    (8, 64, 1, 16, 4, "f32", 8),            # tiny shape
    (1024, 512, 4, 256, 16, "f32", 1024),   # mid: 128x128 tiles
    (300, 1024, 4, 1024, 32, "bf16", 300),  # 128x128 tiles, fused select-gather
    (4500, 1024, 4, 1024, 32, "bf16", 4500),  # persistent 256x256 walk, ragged last row tile
    (700, 320, 5, 1024, 7, "e4m3", 256),    # three chunks, D = 320
    (600, 1024, 2, 2048, 32, "e4m3", 600),  # n_keys 2048
]


def _ids(c):
    return "B{}-D{}-H{}-n{}-k{}-{}-mb{}".format(*c)


def _setup(torch, case, seed):
    B, D, H, n, k, table, mb = case
    wl = synthetic.Workload("prepared", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=seed)
    x = synthetic.make_x(wl, seed=seed)
    P = pk.params_to_device(params, table, support.device())
    mem = pk.Memory(D, H, n, k, table, max_batch=mb)
    return wl, params, x, P, mem, torch.from_numpy(x).to(support.device())


def _same(a, b):
    return all(torch_equal(u, v) for u, v in zip(a, b))


def torch_equal(u, v):
    import torch

    return torch.equal(u, v)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_prepared_forward_is_bitwise_the_forward(torch, case):
    wl, params, x, P, mem, xt = _setup(torch, case, seed=41)
    say("prepared forward", _ids(case))
    ref = mem.forward(P, xt)
    ref_train = mem.forward_train(P, xt)
    mem.prepare(P)
    got = mem.forward(P, xt)
    got_train = mem.forward_train(P, xt)
    torch.cuda.synchronize()
    assert _same(got, ref)
    assert _same(got_train, ref_train)
    if x.shape[0] <= mem.cfg.max_batch:
        out = torch.full_like(ref[0], float("nan"))
        idx = torch.full_like(ref[1], -1)
        w = torch.full_like(ref[2], float("nan"))
        for stage in range(4):
            mem.forward_stage(P, xt, stage, out, idx, w)
        torch.cuda.synchronize()
        assert _same((out, idx, w), ref)


def test_prepared_only_for_the_prepared_arrays(torch):
    import ctypes

    case = CASES[2]
    wl, params, x, P, mem, xt = _setup(torch, case, seed=42)
    params2 = synthetic.make_params(wl, seed=43)
    P2 = pk.params_to_device(params2, wl.table, support.device())
    say("prepared: other arrays, stale copy, failed prepare, re-prepare, drop")
    ref2 = mem.forward(P2, xt)
    ref1 = mem.forward(P, xt)
    mem.prepare(P)
    got2 = mem.forward(P2, xt)  # not the prepared arrays: read as given
    torch.cuda.synchronize()
    assert _same(got2, ref2)
    # contents changed in place without preparing again: the forward still
    # reads the prepared copy (which shows the copy is what it reads)
    P["wq"].mul_(0.5)
    P["subkeys"].mul_(-1.0)
    stale = mem.forward(P, xt)
    mem.prepare(None)
    fresh = mem.forward(P, xt)  # unprepared, new contents
    torch.cuda.synchronize()
    assert _same(stale, ref1)
    assert not torch.equal(fresh[0], ref1[0])
    # a failed prepare leaves nothing prepared
    mem.prepare(P)
    bad = pk._binding.ParamsStruct(*[getattr(P.struct, f) for f, _ in pk._binding.ParamsStruct._fields_])
    bad.wq = None
    assert mem.lib.pkm_prepare(mem._ctx, ctypes.byref(bad), 0, None) == pk.PKM_E_ARG
    P["wq"].mul_(2.0)
    after_fail = mem.forward(P, xt)
    mem.prepare(P)
    again = mem.forward(P, xt)
    mem.prepare(None)
    ref = mem.forward(P, xt)
    torch.cuda.synchronize()
    assert _same(after_fail, ref) and _same(again, ref)


@pytest.mark.parametrize("case", [CASES[1], CASES[4]], ids=_ids)
def test_prepared_forward_against_oracle(torch, case):
    B, D, H, n, k, table, mb = case
    wl = synthetic.Workload("prepared", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=44)
    x = synthetic.make_x(wl, seed=44)
    support.gap_clean(wl, params, x, seed=44)
    P = pk.params_to_device(params, table, support.device())
    mem = pk.Memory(D, H, n, k, table, max_batch=mb)
    mem.prepare(P)
    say("prepared forward vs oracle", _ids(case))
    out, idx, w = mem.forward(P, torch.from_numpy(x).to(support.device()))
    torch.cuda.synchronize()
    out, idx, w = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w)
