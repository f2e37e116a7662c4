"""GPU: the lookup and its backward captured in a HIP graph.

The compute entry points only launch kernels on the stream they are given
(no allocation, copy or memset), so a caller can capture them.  The graph
below holds a chunked pkm_forward, a clearing of the parameter gradients by
torch fill kernels and pkm_backward; every replay, with other eager work
and synchronisations between replays, must give the same bits as the eager
calls (every kernel sums in a fixed order)."""
import numpy as np
import pytest

import product_key_memory_amd as pk
import synthetic
from tests import support
from tests.support import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


@pytest.mark.parametrize("table,n,D", [("bf16", 64, 256), ("int4", 64, 256),
                                       ("bf16", 1024, 512)])  # the last: fused select-gather
def test_forward_and_backward_graph_replays(torch, table, n, D):
    dev = support.device()
    wl = synthetic.Workload("graph", 300, D, 2, n, 16, table, "random")
    params = synthetic.make_params(wl, 3)
    P = pk.params_to_device(params, wl.table, dev)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=128)  # three chunks
    x = torch.from_numpy(np.ascontiguousarray(synthetic.make_x(wl, 3))).to(dev)
    dout = torch.from_numpy(np.random.default_rng(4).standard_normal((wl.B, wl.D)).astype(np.float32)).to(dev)
    say("graph", table, "eager reference")
    out_e, idx_e, w_e = mem.forward(P, x)
    grads_e = mem.backward(P, x, idx_e, w_e, dout)
    torch.cuda.synchronize()

    out, idx, w = torch.empty_like(out_e), torch.empty_like(idx_e), torch.empty_like(w_e)
    grads = {name: torch.zeros_like(t) for name, t in grads_e.items()}
    ws = torch.empty(mem.backward_workspace_bytes(), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        mem.forward(P, x, out, idx, w)
        mem.backward(P, x, idx, w, dout, grads=grads, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    say("graph", table, "capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mem.forward(P, x, out, idx, w)
        for t in grads.values():
            t.zero_()
        mem.backward(P, x, idx, w, dout, grads=grads, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        say("graph", table, "replay", rep)
        out.fill_(float("nan"))
        idx.fill_(-1)
        w.fill_(float("nan"))
        for t in grads.values():
            t.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e) and torch.equal(idx, idx_e) and torch.equal(w, w_e), rep
        for name, t in grads.items():
            assert torch.equal(t, grads_e[name]), (rep, name)
        mem.forward(P, x)  # other eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("form", ["split", "fold"])
def test_prepare_and_prepared_forward_graph_replays(torch, form):
    """pkm_prepare only launches kernels too: a graph holding the prepare
    and two prepared forwards (three chunks each) replays to the eager
    prepared results, with eager unprepared lookups between replays."""
    dev = support.device()
    wl = synthetic.Workload("graph", 300, 512, 2, 256, 16, "bf16", "random")
    params = synthetic.make_params(wl, 5)
    P = pk.params_to_device(params, wl.table, dev)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=128)
    x = torch.from_numpy(np.ascontiguousarray(synthetic.make_x(wl, 5))).to(dev)
    say("graph prepared", form, "eager reference")
    mem.prepare(P, form)
    ref = mem.forward(P, x)
    mem.prepare(None)
    torch.cuda.synchronize()
    outs = [tuple(torch.empty_like(t) for t in ref) for _ in range(2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mem.prepare(P, form)
        for o in outs:
            mem.forward(P, x, *o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph prepared", form, "capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mem.prepare(P, form)
        for o in outs:
            mem.forward(P, x, *o)
    torch.cuda.synchronize()
    for rep in range(3):
        say("graph prepared", form, "replay", rep)
        for o in outs:
            for t in o:
                t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert all(torch.equal(a, b) for a, b in zip(o, ref)), rep
        mem.prepare(None)
        mem.forward(P, x)  # eager unprepared work between replays
        torch.cuda.synchronize()
        mem.prepare(P, form)  # the host-side record the captured forwards rely on
