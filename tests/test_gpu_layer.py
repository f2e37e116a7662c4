"""GPU: the torch layer (product_key_memory_amd.layer.ProductKeyMemory) over
the C ABI.

The layer only marshals: its forward and its autograd gradients must be
bit for bit what direct calls of the binding give for the same tensors --
pkm_forward (eval, no gradient), pkm_forward_train + pkm_backward_with_q
(eval with gradients), pkm_forward_batch_stats + pkm_backward_batch_stats
(training mode, running statistics moved in place).  One case is also
checked against the fp64 oracle's gradients (oracle.backward), with the
parameters loaded from the synthetic recipe and gap-clean inputs."""
import numpy as np
import pytest

import oracle
import product_key_memory_amd as pk
import synthetic
from tests import pins, support
from tests.support import say

pytestmark = pytest.mark.gpu

# binding gradient name -> layer parameter name
PARAM_OF = {"dwq": "wq", "dbn_gamma": "bn_gamma", "dbn_beta": "bn_beta", "dsubkeys": "subkeys",
            "dvalues": "values"}


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


def make_layer(torch, D, H, n, k, table, seed, **kw):
    dev = support.device()
    layer = pk.ProductKeyMemory(D, H, n, k, value_type=table, device=dev, **kw)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    layer.reset_parameters(generator=g)
    with torch.no_grad():  # running statistics away from (0, 1), gamma and beta away from (1, 0)
        layer.running_mean.normal_(0.0, 0.1, generator=g)
        layer.running_var.uniform_(0.5, 2.0, generator=g)
        layer.bn_gamma.uniform_(0.5, 1.5, generator=g)
        layer.bn_beta.normal_(0.0, 0.1, generator=g)
    return layer


def direct_params(layer):
    return pk.Params(layer.wq.detach(), layer.running_mean, layer.running_var, layer.bn_gamma.detach(),
                     layer.bn_beta.detach(), layer.subkeys.detach(), layer.values.detach(), layer.value_scale)


def inputs(torch, B, D, seed):
    g = torch.Generator(device=support.device())
    g.manual_seed(seed)
    x = torch.randn(B, D, generator=g, device=support.device())
    dout = torch.randn(B, D, generator=g, device=support.device())
    return x, dout


@pytest.mark.parametrize("table", ["f32", "bf16"])
def test_eval_forward_and_gradients_bitwise(torch, table):
    D, H, n, k, B = 256, 2, 64, 8, 300
    layer = make_layer(torch, D, H, n, k, table, seed=11, max_batch=128).eval()  # three chunks
    x, dout = inputs(torch, B, D, 12)
    mem = pk.Memory(D, H, n, k, table, max_batch=128)
    P = direct_params(layer)
    say("layer eval", table, "no grad")
    with torch.no_grad():
        out0 = layer(x)
    ref_out, ref_idx, ref_w = mem.forward(P, x)
    torch.cuda.synchronize()
    assert torch.equal(out0, ref_out)

    say("layer eval", table, "with gradients")
    xg = x.clone().requires_grad_()
    out, idx, w = layer(xg, return_selection=True)
    (out * dout).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(idx, ref_idx) and torch.equal(w, ref_w)
    ref = mem.backward(P, x, ref_idx, ref_w, dout)
    torch.cuda.synchronize()
    assert torch.equal(xg.grad, ref["dx"])
    for gname, pname in PARAM_OF.items():
        got = getattr(layer, pname).grad
        assert torch.equal(got, ref[gname].to(got.dtype)), gname


def test_training_mode_batch_statistics_bitwise(torch):
    D, H, n, k, B = 192, 3, 40, 6, 200
    layer = make_layer(torch, D, H, n, k, "f32", seed=21, momentum=0.25).train()
    x, dout = inputs(torch, B, D, 22)
    mem = pk.Memory(D, H, n, k, "f32", max_batch=B)
    rm, rv = layer.running_mean.clone(), layer.running_var.clone()
    P = direct_params(layer)  # the running statistics are not read in training mode
    say("layer train", "forward + backward")
    xg = x.clone().requires_grad_()
    out, idx, w = layer(xg, return_selection=True)
    (out * dout).sum().backward()
    ref_out, ref_idx, ref_w, mean, var = mem.forward_batch_stats(P, x, running=(rm, rv), momentum=0.25)
    ref = mem.backward(P, x, ref_idx, ref_w, dout, batch_stats=(mean, var))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(idx, ref_idx) and torch.equal(w, ref_w)
    assert torch.equal(layer.running_mean, rm) and torch.equal(layer.running_var, rv)
    assert not torch.equal(rm, torch.zeros_like(rm))  # they moved
    assert torch.equal(xg.grad, ref["dx"])
    for gname, pname in PARAM_OF.items():
        assert torch.equal(getattr(layer, pname).grad, ref[gname]), gname


def test_sparse_value_gradient_and_accumulation(torch):
    D, H, n, k, B = 128, 2, 48, 8, 150
    dense = make_layer(torch, D, H, n, k, "bf16", seed=31).eval()
    sparse = make_layer(torch, D, H, n, k, "bf16", seed=31, sparse_values=True).eval()
    x, dout = inputs(torch, B, D, 32)
    say("layer sparse values")
    for layer in (dense, sparse):
        for _ in range(2):  # two backward passes: autograd adds the second into .grad
            (layer(x) * dout).sum().backward()
    torch.cuda.synchronize()
    g = sparse.values.grad
    assert g.is_sparse
    assert torch.equal(g.coalesce().to_dense(), dense.values.grad)
    assert torch.equal(sparse.wq.grad, dense.wq.grad)
    # a plain optimiser step on the sparse gradient moves only touched rows
    before = sparse.values.detach().clone()
    torch.optim.SGD([sparse.values], lr=0.5).step()
    torch.cuda.synchronize()
    moved = (sparse.values.detach() != before).any(1)
    touched = torch.zeros(n * n, dtype=torch.bool, device=x.device)
    touched[g.coalesce().indices()[0]] = True
    assert not bool((moved & ~touched).any())
    assert bool(moved.any())


def test_leading_dims_and_quantised_table(torch):
    D, H, n, k = 128, 2, 32, 4
    layer = make_layer(torch, D, H, n, k, "e4m3", seed=41).eval()
    g = torch.Generator(device=support.device())
    g.manual_seed(42)
    table = torch.randn(n * n, D, generator=g, device=support.device()).to(torch.float8_e4m3fn)
    scale = torch.rand(n * n, generator=g, device=support.device()) + 0.5
    layer.load_table(table, scale)
    x = torch.randn(3, 50, D, generator=g, device=support.device())
    say("layer e4m3, leading dims")
    xg = x.clone().requires_grad_()
    out = layer(xg)
    assert out.shape == (3, 50, D)
    out.square().sum().backward()
    mem = pk.Memory(D, H, n, k, "e4m3", max_batch=16384)
    ref_out, idx, w = mem.forward(direct_params(layer), x.reshape(-1, D))
    ref = mem.backward(direct_params(layer), x.reshape(-1, D), idx, w, 2 * ref_out,
                       grads={"dx": torch.empty(150, D, device=x.device)})
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(-1, D), ref_out)
    assert torch.equal(xg.grad.reshape(-1, D), ref["dx"])
    assert layer.values.grad is None  # a quantised table is a buffer, not trained


def test_gradients_against_oracle(torch):
    """The layer's autograd gradients on the synthetic recipe's parameters
    (random BN statistics, gamma and beta), gap-clean inputs, against the
    fp64 oracle's gradients: each tensor within 1e-4 of its largest entry."""
    wl = synthetic.Workload("layer", 120, 128, 2, 24, 6, "f32", "random")
    params, x, dout = pins.backward_case(wl, 5, True)
    support.gap_clean(wl, params, x, seed=5)
    dev = support.device()
    layer = pk.ProductKeyMemory(wl.D, wl.H, wl.n, wl.k, value_type="f32", device=dev).eval()
    with torch.no_grad():
        for name, key in (("wq", "wq"), ("running_mean", "mean"), ("running_var", "var"), ("bn_gamma", "gamma"),
                          ("bn_beta", "beta"), ("subkeys", "subkeys"), ("values", "values")):
            getattr(layer, name).copy_(torch.from_numpy(np.ascontiguousarray(params[key], dtype=np.float32)))
    xg = torch.from_numpy(x).to(dev).requires_grad_()
    say("layer vs oracle gradients")
    (layer(xg) * torch.from_numpy(dout).to(dev)).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    got = {"dx": xg.grad, "dwq": layer.wq.grad, "dgamma": layer.bn_gamma.grad, "dbeta": layer.bn_beta.grad,
           "dsub": layer.subkeys.grad, "dval": layer.values.grad}
    for name, t in got.items():
        g, r = t.cpu().numpy().astype(np.float64), ref[name]
        err = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
        assert err <= 1e-4, (name, err)


def test_prepared_weights_follow_the_parameters(torch):
    """prepare_weights=True gives the unprepared layer's bits in eval mode,
    with and without gradients, and stays right after an optimiser step
    (the parameters change in place: the prepared copy is made again)."""
    D, H, n, k, B = 256, 2, 64, 8, 300
    ref_layer = make_layer(torch, D, H, n, k, "bf16", seed=31, max_batch=128).eval()
    layer = make_layer(torch, D, H, n, k, "bf16", seed=31, max_batch=128, prepare_weights=True).eval()
    x, dout = inputs(torch, B, D, 32)
    say("layer prepared weights: eval, no grad")
    with torch.no_grad():
        assert torch.equal(layer(x), ref_layer(x))
    opt = torch.optim.SGD(layer.parameters(), lr=0.5)
    ref_opt = torch.optim.SGD(ref_layer.parameters(), lr=0.5)
    for step in range(2):
        say("layer prepared weights: gradient step", step)
        for lay, o in ((layer, opt), (ref_layer, ref_opt)):
            o.zero_grad()
            (lay(x) * dout).sum().backward()
            o.step()
        torch.cuda.synchronize()
        assert torch.equal(layer.wq, ref_layer.wq) and torch.equal(layer.subkeys, ref_layer.subkeys)
        with torch.no_grad():
            assert torch.equal(layer(x), ref_layer(x))
    # a change the version counters do not see, then an explicit refresh
    layer.wq.data.mul_(0.5)
    ref_layer.wq.data.mul_(0.5)
    layer.refresh_prepared()
    with torch.no_grad():
        assert torch.equal(layer(x), ref_layer(x))


def test_folded_layer_follows_the_parameters(torch):
    """prepare_weights="fold": eval forwards without gradients match the
    oracle (gap-clean inputs), and stay right after the running statistics
    move (a training-mode forward) and after an optimiser step, where the
    folded form is made again: the outputs then equal a fresh folded
    lookup of the new parameters."""
    D, H, n, k, B = 256, 2, 64, 8, 300
    layer = make_layer(torch, D, H, n, k, "f32", seed=41, max_batch=512, prepare_weights="fold").eval()
    _, dout = inputs(torch, B, D, 42)
    wl = synthetic.Workload("layer", B, D, H, n, k, "f32", "random")
    params = {"wq": layer.wq.detach().cpu().numpy(), "mean": layer.running_mean.cpu().numpy(),
              "var": layer.running_var.cpu().numpy(), "gamma": layer.bn_gamma.detach().cpu().numpy(),
              "beta": layer.bn_beta.detach().cpu().numpy(), "subkeys": layer.subkeys.detach().cpu().numpy(),
              "values": layer.values.detach().cpu().numpy(), "scale": None}
    xn = synthetic.make_x(wl, seed=42)
    _, tau = support.gap_clean(wl, params, xn, seed=42, want_tau=True)
    x = support.to_device(xn)
    say("layer folded: eval vs oracle")
    with torch.no_grad():
        out, idx, w = layer(x, return_selection=True)
    torch.cuda.synchronize()
    r = oracle.run(support.model_for(wl, params), xn, want=("out", "idx", "top"))
    support.check_indices(idx.cpu().numpy(), r["idx"], r["top"], tau)
    assert support.rel_rowmax_err(out.cpu().numpy(), r["out"]).max() <= 1e-4

    def fresh(lay):
        mem = pk.Memory(D, H, n, k, "f32", max_batch=512)
        P = direct_params(lay)
        mem.prepare(P, "fold")
        return mem.forward(P, x)[0]

    say("layer folded: after a training-mode forward and an optimiser step")
    layer.train()
    (layer(x) * dout).sum().backward()  # moves the running statistics
    layer.eval()
    with torch.no_grad():
        assert torch.equal(layer(x), fresh(layer))
    torch.optim.SGD(layer.parameters(), lr=0.5).step()
    with torch.no_grad():
        assert torch.equal(layer(x), fresh(layer))
