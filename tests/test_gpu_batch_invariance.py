"""GPU: a token's results do not depend on the batch it comes in.

Every contraction sums each output over the same 16-k chunks in the same
order whatever its tile shape (128x128 tiles for small batches, the
persistent 256x256 walk for large ones) and whatever the batch holds, and
the selection and the gather work per token.  So a token looked up alone in
a small batch must give the same bits (out, idx, weights) as in a large
one: checked for the unprepared lookup and both prepared forms, with the
small batch a contiguous run of the large one's tokens and a scattered
set, and with the large batch also split into chunks by max_batch.
"""
import numpy as np
import pytest

import product_key_memory_amd as pk
import synthetic
from tests import support
from tests.support import say

pytestmark = pytest.mark.gpu

# 8,200 tokens give every contraction at least 256 tiles of 256 x 256 (the
# persistent walk); 300 tokens leave each of them below (128 x 128 tiles)
D, H, N_KEYS, K = 512, 4, 512, 32
B_BIG, B_SMALL = 8200, 300


@pytest.fixture(scope="module")
def setup():
    import torch

    support.device()
    pk.load_library()
    wl = synthetic.Workload("invariance", B_BIG, D, H, N_KEYS, K, "bf16", "random")
    params = synthetic.make_params(wl, seed=21)
    x = synthetic.make_x(wl, seed=21)
    P = pk.params_to_device(params, wl.table, support.device())
    return torch, wl, P, x


def _run(torch, mem, P, x):
    xt = support.to_device(x)
    out, idx, w = mem.forward(P, xt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("form", [None, "split", "fold"])
def test_token_results_independent_of_batch(setup, form):
    torch, wl, P, x = setup
    rng = np.random.default_rng(5)
    picks = {
        "run": np.arange(1000, 1000 + B_SMALL),
        "scattered": np.sort(rng.choice(B_BIG, B_SMALL, replace=False)),
    }
    big = pk.Memory(D, H, N_KEYS, K, wl.table, max_batch=B_BIG)
    small = pk.Memory(D, H, N_KEYS, K, wl.table, max_batch=B_SMALL)
    chunked = pk.Memory(D, H, N_KEYS, K, wl.table, max_batch=3000)  # 3000, 3000, 2200 tokens
    for mem in (big, small, chunked):
        if form:
            mem.prepare(P, form)
    say("batch invariance", form, "large batch", B_BIG)
    ref = _run(torch, big, P, x)
    say("batch invariance", form, "large batch in chunks of 3000")
    got = _run(torch, chunked, P, x)
    for name, a, b in zip(("out", "idx", "weights"), ref, got):
        assert np.array_equal(a, b), (form, "chunked", name)
    for label, rows in picks.items():
        say("batch invariance", form, "small batch", label, B_SMALL)
        got = _run(torch, small, P, np.ascontiguousarray(x[rows]))
        for name, a, b in zip(("out", "idx", "weights"), ref, got):
            assert np.array_equal(a[rows], b), (form, label, name)
