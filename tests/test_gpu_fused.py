"""GPU: the fused selection and gather (pkm_select_gather; what pkm_forward
runs after the scoring when n_keys is 1024 or 2048, H k <= 512 and table
rows are longer than 512 bytes; shorter rows take the two kernels).

It must equal pkm_select followed by pkm_gather bit for bit -- the same
selection, and each output column summed by the same rows in the same
order -- for every table format, fused or not.
The whole lookup through it is checked against the fp64 oracle with the
lookup's rules (indices exact, outputs within 1e-4 for fp32 tables and 2e-2
for the others).
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
    # (B, D, H, n, k, table): rows > 512 bytes are fused; <= 512 bytes take the two kernels
    (300, 1024, 4, 1024, 32, "bf16"),   # two 1 KiB slices
    (200, 256, 3, 1024, 20, "bf16"),    # 512-byte rows: not fused
    (150, 1024, 2, 1024, 16, "f32"),    # four slices
    (100, 128, 4, 1024, 32, "f32"),     # 512-byte rows
    (120, 1024, 4, 2048, 32, "e4m3"),   # n_keys 2048, one slice
    (90, 512, 2, 2048, 8, "e4m3"),      # 512-byte rows
    (160, 1024, 4, 1024, 32, "int8"),
    (160, 1024, 4, 1024, 32, "int4"),   # 512-byte rows: not fused
    (64, 2048, 2, 1024, 64, "int4"),    # 1 KiB rows: fused, k = 64
    (70, 320, 5, 1024, 7, "e4m3"),      # D not a power of two, H > 4 waves
]


def _ids(c):
    return "B{}-D{}-H{}-n{}-k{}-{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fused_equals_select_then_gather(torch, case):
    B, D, H, n, k, table = case
    wl = synthetic.Workload("fused", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=21)
    x = synthetic.make_x(wl, seed=21)
    P = pk.params_to_device(params, table, support.device())
    mem = pk.Memory(D, H, n, k, table, max_batch=B)
    say("fused select+gather", _ids(case))
    xt = torch.from_numpy(x).to(support.device())
    s = mem.score(P, mem.query(P, xt))
    idx, w = mem.select(s)
    ref = mem.gather(P, idx, w)
    fi = torch.full_like(idx, -1)
    fw = torch.full_like(w, float("nan"))
    out, _, _ = mem.select_gather(P, s, idx=fi, weights=fw)
    out2, _, _ = mem.select_gather(P, s)  # selection not written out
    torch.cuda.synchronize()
    assert torch.equal(fi, idx) and torch.equal(fw, w)
    assert torch.equal(out, ref) and torch.equal(out2, ref)


@pytest.mark.parametrize("case", CASES[:6], ids=_ids)
def test_fused_forward_against_oracle(torch, case):
    B, D, H, n, k, table = case
    wl = synthetic.Workload("fused", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=22)
    x = synthetic.make_x(wl, seed=22)
    support.gap_clean(wl, params, x, seed=22)
    out, idx, w = support.gpu_forward(wl, params, x)
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w)


def test_unfusable_shape_takes_two_kernels(torch):
    """H k above 512 (16 heads of 64) is not fused; pkm_select_gather then
    runs the two kernels, in chunks of max_batch through the workspace when
    no idx / weights are given."""
    wl = synthetic.Workload("wide", 40, 128, 16, 1024, 64, "bf16", "random")
    params = synthetic.make_params(wl, seed=23)
    x = synthetic.make_x(wl, seed=23)
    P = pk.params_to_device(params, wl.table, support.device())
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=16)
    say("unfused select+gather, 16 heads of 64")
    xt = torch.from_numpy(x).to(support.device())
    s = mem.score(P, mem.query(P, xt))
    idx, w = mem.select(s)
    ref = mem.gather(P, idx, w)
    out, _, _ = mem.select_gather(P, s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[4]], ids=_ids)
def test_forward_stages_compose_to_forward(torch, case):
    """pkm_forward_stage 0, 1, 2, 3 in order give pkm_forward's bits;
    a stage outside 0-3 and a batch above max_batch are refused."""
    B, D, H, n, k, table = case
    wl = synthetic.Workload("stages", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=24)
    x = synthetic.make_x(wl, seed=24)
    P = pk.params_to_device(params, table, support.device())
    mem = pk.Memory(D, H, n, k, table, max_batch=B)
    xt = torch.from_numpy(x).to(support.device())
    say("forward stages", _ids(case))
    ref = mem.forward(P, xt)
    out = torch.full_like(ref[0], float("nan"))
    idx = torch.full_like(ref[1], -1)
    w = torch.full_like(ref[2], float("nan"))
    for stage in range(4):
        mem.forward_stage(P, xt, stage, out, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(idx, ref[1]) and torch.equal(w, ref[2])
    with pytest.raises(pk.PkmError):
        mem.forward_stage(P, xt, 4, out)
    small = pk.Memory(D, H, n, k, table, max_batch=B - 1)
    with pytest.raises(pk.PkmError):
        small.forward_stage(P, xt, 0, out)
