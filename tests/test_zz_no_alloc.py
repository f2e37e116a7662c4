"""GPU: pkm_forward_noalloc -- the lookup without a context or any
allocation, its workspace in the library's static scratch array -- against
pkm_forward on the same inputs, through the C ABI.

Two calls in a row per configuration, the second with a smaller batch (the
array keeps the first call's contents; the second must not depend on them).
The default shape's 4096 tokens do not fit one chunk of the array, so its
first call also runs in two chunks.  Indices must be identical (index work
is bit-exact); outputs and weights within the lookup's tolerance (1e-4 for
fp32 tables, 2e-2 otherwise), and they are in fact bitwise equal: the same
kernels sum in the same order whatever the chunk.
"""
import numpy as np
import pytest

import product_key_memory_amd as pk
import synthetic
from tests import support
from tests.support import say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 2e-2, "int8": 2e-2, "int4": 2e-2}


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


def _both(torch, wl, P, mem, cfg, xt, keep_selection=True):
    B = xt.shape[0]
    dev = xt.device
    say("pkm_forward", wl.name, "B =", B)
    ref = mem.forward(P, xt)
    out = torch.full((B, wl.D), float("nan"), device=dev)
    idx = torch.full((B, wl.H, wl.k), -1, dtype=torch.int32, device=dev) if keep_selection else None
    w = torch.full((B, wl.H, wl.k), float("nan"), device=dev) if keep_selection else None
    say("pkm_forward_noalloc", wl.name, "B =", B, "keep_selection =", keep_selection)
    pk.forward_noalloc(cfg, P, xt, out, idx, w)
    torch.cuda.synchronize()
    ref = [t.cpu().numpy() for t in ref]
    got = [out.cpu().numpy(), None if idx is None else idx.cpu().numpy(), None if w is None else w.cpu().numpy()]
    tol = TOL[wl.table]
    assert support.rel_rowmax_err(got[0], ref[0]).max() <= tol
    if keep_selection:
        assert np.array_equal(got[1], ref[1]), "indices differ from pkm_forward"
        assert np.abs(got[2] - ref[2]).max() <= tol
    bitwise = all(np.array_equal(g, r) for g, r in zip(got, ref) if g is not None)
    print(f"{wl.name} B={B}: bitwise equal to pkm_forward: {bitwise}", flush=True)
    assert bitwise


@pytest.mark.parametrize("name,first,second", [
    ("mid", 1024, 333),          # fp32 table, random BN: one chunk, then a ragged smaller one
    ("default", 4096, 1000),     # 1M-row bf16 table: two chunks (2560 + 1536), then one
])
def test_noalloc_matches_forward_two_calls(torch, name, first, second):
    wl = synthetic.WORKLOADS[name].with_(B=first)
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)
    P = pk.params_to_device(params, wl.table, support.device())
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=first)
    cfg = pk.make_config(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=16384)
    xt = torch.from_numpy(x).to(support.device())
    _both(torch, wl, P, mem, cfg, xt)
    _both(torch, wl, P, mem, cfg, xt[:second].contiguous())


def test_noalloc_small_chunks_and_no_selection(torch):
    """A caller's max_batch below the array's capacity sets the chunk (here
    100 tokens of a 777-token batch: eight chunks, the last ragged); idx and
    weights may be NULL (kept in the array); B = 0 enqueues nothing."""
    wl = synthetic.Workload("na", 777, 256, 3, 96, 12, "e4m3", "random")
    params = synthetic.make_params(wl, seed=4)
    x = synthetic.make_x(wl, seed=4)
    P = pk.params_to_device(params, wl.table, support.device())
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=wl.B)
    cfg = pk.make_config(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=100)
    xt = torch.from_numpy(x).to(support.device())
    _both(torch, wl, P, mem, cfg, xt)
    _both(torch, wl, P, mem, cfg, xt[:50].contiguous(), keep_selection=False)
    empty = torch.zeros((0, wl.D), device=support.device())
    pk.forward_noalloc(cfg, P, empty, torch.zeros((0, wl.D), device=support.device()))
    torch.cuda.synchronize()


def test_noalloc_graph_replays(torch):
    """Captured in a HIP graph (what the entry point is for): every replay,
    with other eager calls that reuse the array between replays, gives the
    eager call's bits."""
    wl = synthetic.Workload("nag", 700, 1024, 4, 1024, 32, "bf16", "random")
    params = synthetic.make_params(wl, seed=6)
    x = synthetic.make_x(wl, seed=6)
    dev = support.device()
    P = pk.params_to_device(params, wl.table, dev)
    cfg = pk.make_config(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=256)  # three chunks
    xt = torch.from_numpy(x).to(dev)
    say("no-alloc graph: eager reference")
    ref = [torch.empty((wl.B, wl.D), device=dev), torch.empty((wl.B, wl.H, wl.k), dtype=torch.int32, device=dev),
           torch.empty((wl.B, wl.H, wl.k), device=dev)]
    pk.forward_noalloc(cfg, P, xt, *ref)
    out, idx, w = (torch.empty_like(t) for t in ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        pk.forward_noalloc(cfg, P, xt, out, idx, w, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("no-alloc graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pk.forward_noalloc(cfg, P, xt, out, idx, w)
    torch.cuda.synchronize()
    other = torch.empty((300, wl.D), device=dev)
    for rep in range(3):
        say("no-alloc graph: replay", rep)
        out.fill_(float("nan"))
        idx.fill_(-1)
        w.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(idx, ref[1]) and torch.equal(w, ref[2]), rep
        pk.forward_noalloc(cfg, P, xt[:300].contiguous(), other)  # eager work on the same array
        torch.cuda.synchronize()
