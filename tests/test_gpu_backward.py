"""GPU: the backward direction (pkm_backward) through the C ABI against the
fp64 oracle's gradients (oracle.backward, pinned in tests/pins.py).

The GPU backward takes the winners of the GPU forward; on gap-clean inputs
they are the oracle's (tests/support.py), so both differentiate the same
function.  Tolerance: every gradient tensor within 1e-4 of its largest
entry (max-norm); the backward is fp32 throughout and every table format is
decoded from the same stored bits on both sides.  dx is also checked per
token, within 1e-4 of max(the token's largest entry, the batch median of
that): where a head's softmax is nearly one-hot, dt_j = w_j (g_j - sum w g)
cancels and the token's gradient can fall far below its rounding scale,
which is set by dout and the value rows and is alike across tokens (seen:
a token with weights 1 - 5e-8 whose dx is 1/1500 of the median).
"""
import numpy as np
import pytest

import oracle
import product_key_memory_amd as pk
import synthetic
from tests import pins, support
from tests.support import say

pytestmark = pytest.mark.gpu

TOL = 1e-4
# oracle name -> binding name
NAMES = {"dx": "dx", "dwq": "dwq", "dgamma": "dbn_gamma", "dbeta": "dbn_beta", "dsub": "dsubkeys",
         "dval": "dvalues"}


@pytest.fixture(scope="module")
def torch():
    import torch as t

    support.device()
    pk.load_library()
    return t


def _to(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(support.device())


def case(wl, seed=0, gamma_beta=False):
    params, x, dout = pins.backward_case(wl, seed, gamma_beta)
    support.gap_clean(wl, params, x, seed=seed)
    return params, x, dout


def gpu_backward(torch, wl, params, x, dout, max_batch=16384, grads=None, mem=None):
    mem = mem or pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=max_batch)
    P = pk.params_to_device(params, wl.table, support.device())
    xt, dt = _to(torch, x), _to(torch, dout)
    say("backward", wl, "B =", x.shape[0], "max_batch =", max_batch)
    _, idx, w = mem.forward(P, xt)
    g = mem.backward(P, xt, idx, w, dt, grads=grads)
    torch.cuda.synchronize()
    return {name: t.cpu().numpy() for name, t in g.items()}, idx.cpu().numpy()


def compare(got, ref, names=NAMES):
    errs = {}
    for oname, gname in names.items():
        if oname not in ref or gname not in got:
            continue
        r, g = ref[oname], got[gname].astype(np.float64)
        scale = max(np.abs(r).max(), 1e-30)
        errs[oname] = float(np.abs(g - r).max() / scale)
        assert errs[oname] <= TOL, (oname, errs[oname])
        if oname == "dx" and r.shape[0]:
            mag = np.abs(r).max(1)
            floor = np.maximum(mag, np.median(mag))
            row = np.abs(g - r).max(1) / np.maximum(floor, 1e-30)
            assert row.max() <= TOL, ("dx per token", float(row.max()), int(row.argmax()))
    return errs


@pytest.mark.parametrize("wl,gamma_beta", [
    (synthetic.WORKLOADS["tiny"], False),
    (synthetic.WORKLOADS["mid"], False),
    (synthetic.Workload("bgb", 100, 128, 3, 20, 5, "f32", "random"), True),   # ragged B, random BN, gamma, beta
    (synthetic.Workload("bbf", 64, 256, 2, 48, 16, "bf16", "unit"), False),  # bf16 table
    (synthetic.Workload("be4", 77, 192, 2, 33, 9, "e4m3", "random"), True),  # E4M3 + row scales, D = 3 * 64
    (synthetic.Workload("bkn", 40, 64, 1, 12, 12, "f32", "random"), False),  # k = n_keys
    (synthetic.Workload("bk1", 50, 64, 2, 30, 1, "bf16", "random"), True),   # k = 1: no gradient to the scores
    (synthetic.Workload("bi8", 60, 128, 2, 24, 8, "int8", "random"), True),  # int8 table + row scales
    (synthetic.Workload("bi4", 60, 192, 2, 24, 8, "int4", "random"), True),  # int4 table
    # 2048 tokens in one chunk: dWq (K = tokens) runs split-K on 256x256 tiles
    (synthetic.Workload("bsk", 2048, 256, 2, 32, 8, "bf16", "random"), True),
])
def test_backward_against_oracle(torch, wl, gamma_beta):
    params, x, dout = case(wl, 2, gamma_beta)
    got, _ = gpu_backward(torch, wl, params, x, dout)
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    errs = compare(got, ref)
    print(wl.name, {k: f"{v:.2g}" for k, v in errs.items()}, flush=True)


def _random_backward_configs(count, seed):
    """Seeded random small configurations (D a multiple of 64, every table
    format, chunked and unchunked), with random BN affine parameters."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        D = int(rng.choice([64, 128, 192, 256]))
        n = int(rng.integers(2, 80))
        k = int(rng.integers(1, min(32, n) + 1))
        H = int(rng.integers(1, 4))
        B = int(rng.integers(2, 300))
        table = str(rng.choice(["f32", "bf16", "e4m3", "int8", "int4"]))
        max_batch = int(rng.choice([B, max(1, B // 2), 64]))
        out.append(dict(B=B, D=D, H=H, n=n, k=k, table=table, max_batch=max_batch, seed=int(200 + i)))
    return out


@pytest.mark.parametrize("cfg", _random_backward_configs(8, 7),
                         ids=lambda c: "B{B}-D{D}-H{H}-n{n}-k{k}-{table}-mb{max_batch}".format(**c))
def test_backward_random_configs(torch, cfg):
    wl = synthetic.Workload("rb", cfg["B"], cfg["D"], cfg["H"], cfg["n"], cfg["k"], cfg["table"], "random")
    params, x, dout = case(wl, cfg["seed"], gamma_beta=True)
    got, _ = gpu_backward(torch, wl, params, x, dout, max_batch=cfg["max_batch"])
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    compare(got, ref)


def test_backward_chunks_accumulate_and_repeat_bitwise(torch):
    """max_batch smaller than B: the chunks add into the parameter gradients;
    a second call adds the same again (to rounding: each chunk's sum is
    added to what the buffer holds, so g + g is not summed as 2 g); two runs
    give the same bits."""
    wl = synthetic.Workload("bch", 150, 128, 2, 24, 6, "bf16", "random")
    params, x, dout = case(wl, 3, True)
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    one, _ = gpu_backward(torch, wl, params, x, dout, max_batch=64)
    compare(one, ref)
    again, _ = gpu_backward(torch, wl, params, x, dout, max_batch=64)
    for name in one:
        assert np.array_equal(one[name], again[name]), name
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=64)
    twice, _ = gpu_backward(torch, wl, params, x, dout, mem=mem)
    grads = {name: _to(torch, t) for name, t in twice.items()}
    P = pk.params_to_device(params, wl.table, support.device())
    xt = _to(torch, x)
    _, idx, w = mem.forward(P, xt)
    mem.backward(P, xt, idx, w, _to(torch, dout), grads=grads)
    torch.cuda.synchronize()
    for name, t in grads.items():
        t = t.cpu().numpy()
        if name == "dx":
            assert np.array_equal(t, twice[name])
        else:
            want = 2 * twice[name].astype(np.float64)
            assert np.abs(t - want).max() <= 1e-6 * max(np.abs(want).max(), 1e-30), name


@pytest.mark.parametrize("wl,max_batch,sample", [
    (synthetic.Workload("bsq", 300, 256, 2, 40, 8, "bf16", "random"), 128, 1),    # chunked: q per chunk
    (synthetic.Workload("bsq3", 200, 192, 3, 30, 6, "e4m3", "random"), 16384, 1),  # half-heads of 96 columns
    (synthetic.WORKLOADS["default"], 4096, 37),                                   # the default shape
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_forward_train_and_backward_with_q(torch, wl, max_batch, sample):
    """pkm_forward_train: out / idx / weights bitwise those of pkm_forward,
    and q the projection before BN (Wq x against fp64, within fp32-level
    rounding, on every `sample`-th token); pkm_backward_with_q on that q:
    every gradient -- the dense and the sparse value gradient too --
    bitwise that of pkm_backward, which computes q again."""
    params, x, dout = case(wl, 7, True)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=max_batch)
    P = pk.params_to_device(params, wl.table, support.device())
    xt, dt = _to(torch, x), _to(torch, dout)
    say("forward_train / backward_with_q", wl, "max_batch =", max_batch)
    out0, idx0, w0 = mem.forward(P, xt)
    out1, idx1, w1, q = mem.forward_train(P, xt)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(idx0, idx1) and torch.equal(w0, w1)
    rows = np.arange(0, wl.B, sample)
    ref_q = np.einsum("bd,hfd->bhf", x[rows].astype(np.float64), params["wq"].astype(np.float64))
    got_q = q.cpu().numpy()[rows].astype(np.float64)
    assert np.abs(got_q - ref_q).max() <= 1e-5 * np.abs(ref_q).max()
    for sparse in (False, True) if wl.B <= max_batch else (False,):  # the sparse form takes one chunk
        g0 = mem.backward(P, xt, idx0, w0, dt, sparse_values=sparse)
        g1 = mem.backward(P, xt, idx1, w1, dt, sparse_values=sparse, q=q)
        torch.cuda.synchronize()
        for name in g0:
            assert torch.equal(g0[name], g1[name]), (sparse, name)
        del g0, g1


def test_backward_subset_of_gradients(torch):
    """Skipped gradients leave no trace; the computed ones are unchanged."""
    wl = synthetic.Workload("bsub", 40, 64, 2, 16, 4, "f32", "random")
    params, x, dout = case(wl, 4, True)
    full, _ = gpu_backward(torch, wl, params, x, dout)
    for subset in (("dvalues",), ("dx",), ("dbn_gamma", "dbn_beta"), ("dsubkeys", "dwq")):
        grads = {name: torch.zeros(full[name].shape, dtype=torch.float32, device=support.device())
                 for name in subset}
        part, _ = gpu_backward(torch, wl, params, x, dout, grads=grads)
        for name in subset:
            assert np.array_equal(part[name], full[name]), (subset, name)


def test_backward_hot_rows(torch):
    """One token repeated 100 times: every selected row occurs 100 * H / H =
    100 times per head set, past the 64-occurrence sort, so the value
    gradient walks its occurrences by repeated minimum search."""
    wl = synthetic.Workload("bhot", 1, 64, 2, 16, 4, "f32", "random")
    params, x1, _ = case(wl, 5, True)
    x = np.repeat(x1, 100, axis=0)
    dout = np.random.default_rng(6).standard_normal(x.shape).astype(np.float32)
    wl = wl.with_(B=100)
    got, idx = gpu_backward(torch, wl, params, x, dout)
    assert np.bincount(idx.ravel()).max() >= 100
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    compare(got, ref)


def _sparse_grads(torch, wl, B, sentinel_rows=-7, sentinel=3.5):
    cap = min(wl.N, B * wl.H * wl.k)
    dev = support.device()
    return {"dvalues_rows": torch.full((cap,), sentinel_rows, dtype=torch.int32, device=dev),
            "dvalues_sparse": torch.full((cap, wl.D), sentinel, dtype=torch.float32, device=dev),
            "dvalues_count": torch.full((1,), -1, dtype=torch.int64, device=dev)}


@pytest.mark.parametrize("name,B,dim,heads,n,k,table,seed,others", [
    ("bsp", 40, 64, 2, 16, 4, "f32", 8, True),      # most rows touched, some more than once
    ("bsp1", 40, 64, 2, 16, 4, "int8", 9, False),   # the value gradient alone
    ("bsp2", 33, 192, 3, 40, 8, "bf16", 10, True),  # ragged: 33 tokens, 1600 rows
    ("bsp3", 100, 64, 2, 16, 4, "f32", 11, True),   # one token repeated: rows past 64 occurrences
])
def test_backward_sparse_values(torch, name, B, dim, heads, n, k, table, seed, others):
    """The sparse value gradient: the distinct rows of idx in increasing
    order, their count, and rows that scattered into zeros equal the dense
    gradient bit for bit (and so the oracle's); entries past the count are
    left as they were; the other gradients are unchanged."""
    wl = synthetic.Workload(name, B, dim, heads, n, k, table, "random")
    params, x, dout = case(wl, seed, True)
    if name == "bsp3":
        x = np.repeat(x[:1], B, axis=0)
    dense, idx = gpu_backward(torch, wl, params, x, dout)
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    compare(dense, ref)
    grads = _sparse_grads(torch, wl, B)
    if others:
        grads.update({nm: torch.zeros(dense[nm].shape, dtype=torch.float32, device=support.device())
                      for nm in ("dx", "dwq", "dbn_gamma", "dbn_beta", "dsubkeys")})
    got, idx2 = gpu_backward(torch, wl, params, x, dout, grads=grads)
    assert np.array_equal(idx, idx2)
    rows = np.unique(idx)
    U = int(got["dvalues_count"][0])
    assert U == rows.size
    assert np.array_equal(got["dvalues_rows"][:U], rows)
    assert (got["dvalues_rows"][U:] == -7).all() and (got["dvalues_sparse"][U:] == 3.5).all()
    assert np.array_equal(got["dvalues_sparse"][:U], dense["dvalues"][rows])
    assert not np.delete(dense["dvalues"], rows, axis=0).any()
    for nm in got:
        if nm in dense:
            assert np.array_equal(got[nm], dense[nm]), nm


@pytest.mark.parametrize("cfg", _random_backward_configs(6, 31),
                         ids=lambda c: "B{B}-D{D}-H{H}-n{n}-k{k}-{table}".format(**c))
def test_backward_sparse_values_random_configs(torch, cfg):
    """Seeded random configurations (one chunk): the sparse value gradient's
    rows are the distinct rows of idx in order, and its values equal the
    dense gradient's rows bit for bit."""
    wl = synthetic.Workload("rbs", cfg["B"], cfg["D"], cfg["H"], cfg["n"], cfg["k"], cfg["table"], "random")
    params, x, dout = case(wl, cfg["seed"], gamma_beta=True)
    dense, idx = gpu_backward(torch, wl, params, x, dout, max_batch=cfg["B"],
                              grads={"dvalues": torch.zeros((wl.N, wl.D), device=support.device())})
    got, idx2 = gpu_backward(torch, wl, params, x, dout, max_batch=cfg["B"], grads=_sparse_grads(torch, wl, wl.B))
    assert np.array_equal(idx, idx2)
    rows = np.unique(idx)
    U = int(got["dvalues_count"][0])
    assert U == rows.size and np.array_equal(got["dvalues_rows"][:U], rows)
    assert np.array_equal(got["dvalues_sparse"][:U], dense["dvalues"][rows])


def test_backward_sparse_values_batch_stats_and_empty(torch):
    """The sparse form under training-mode BN equals the dense one; B = 0
    writes a count of zero."""
    wl = synthetic.Workload("bsps", 48, 128, 2, 20, 6, "bf16", "random")
    params, x, dout = case(wl, 12, True)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=64)
    P = pk.params_to_device(params, wl.table, support.device())
    xt, dt = _to(torch, x), _to(torch, dout)
    say("sparse value gradient, batch statistics", wl)
    _, idx, w, mean, var = mem.forward_batch_stats(P, xt)
    dense = mem.backward(P, xt, idx, w, dt, batch_stats=(mean, var))
    sparse = mem.backward(P, xt, idx, w, dt, batch_stats=(mean, var), sparse_values=True)
    torch.cuda.synchronize()
    assert "dvalues" not in sparse and "dvalues" in dense
    rows = torch.unique(idx.long()).to(torch.int32)
    U = int(sparse["dvalues_count"].item())
    assert U == rows.numel()
    assert torch.equal(sparse["dvalues_rows"][:U], rows)
    assert torch.equal(sparse["dvalues_sparse"][:U], dense["dvalues"][rows.long()])
    for nm in ("dx", "dwq", "dbn_gamma", "dbn_beta", "dsubkeys"):
        assert torch.equal(sparse[nm], dense[nm]), nm
    say("sparse value gradient, B = 0")
    grads = _sparse_grads(torch, wl, 0)
    mem.backward(P, xt[:0], idx[:0], w[:0], dt[:0], grads=grads)
    torch.cuda.synchronize()
    assert int(grads["dvalues_count"].item()) == 0


def test_backward_arguments(torch):
    wl = synthetic.Workload("berr", 4, 64, 1, 16, 4, "f32", "unit")
    params = synthetic.make_params(wl)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=8)
    P = pk.params_to_device(params, wl.table, support.device())
    x = torch.zeros((4, wl.D), device=support.device())
    _, idx, w = mem.forward(P, x)
    say("backward arguments")
    small = torch.empty(mem.backward_workspace_bytes() - 256, dtype=torch.uint8, device=support.device())
    with pytest.raises(pk.PkmError) as e:
        mem.backward(P, x, idx, w, x, workspace=small)
    assert e.value.status == pk.PKM_E_ARG
    with pytest.raises(pk.PkmError):
        mem.backward(P, x, idx, w, x, grads={"dbn_gamma": torch.zeros((1, wl.D), device=support.device())})
    g = mem.backward(P, x[:0], idx[:0], w[:0], x[:0])
    torch.cuda.synchronize()
    assert g["dx"].shape == (0, wl.D)
    # the sparse value gradient: all three members or none, not with the
    # dense one, and one chunk only
    sp = _sparse_grads(torch, wl, 4)
    for bad in ({"dvalues_rows": sp["dvalues_rows"]},
                {**sp, "dvalues": torch.zeros((wl.N, wl.D), device=support.device())}):
        with pytest.raises(pk.PkmError) as e:
            mem.backward(P, x, idx, w, x, grads=bad)
        assert e.value.status == pk.PKM_E_ARG
    x16 = torch.zeros((16, wl.D), device=support.device())
    _, idx16, w16 = mem.forward(P, x16)
    with pytest.raises(pk.PkmError) as e:
        mem.backward(P, x16, idx16, w16, x16, grads=_sparse_grads(torch, wl, 16))
    assert e.value.status == pk.PKM_E_ARG and "max_batch" in pk.last_error()


@pytest.mark.slow
def test_backward_default_shape(torch):
    """The pages' default shape (1M-row bf16 table) on 1024 gap-clean tokens;
    the value gradient is compared on the rows the batch touched and checked
    whole by its column sums (H * sum_b dout_b)."""
    wl = synthetic.WORKLOADS["default"].with_(B=1024)
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)[:1024].copy()
    support.gap_clean(wl, params, x)
    dout = np.random.default_rng(1).standard_normal(x.shape).astype(np.float32)
    got, idx = gpu_backward(torch, wl, params, x, dout, max_batch=512)
    ref = oracle.backward(support.model_for(wl, params), x, dout)
    rows = np.unique(idx)
    touched = dict(got)
    touched["dvalues"] = got["dvalues"][rows]
    reff = dict(ref)
    reff["dval"] = ref["dval"][rows]
    errs = compare(touched, reff)
    untouched = np.ones(wl.N, bool)
    untouched[rows] = False
    assert not got["dvalues"][untouched].any()
    want = wl.H * dout.astype(np.float64).sum(0)
    assert np.abs(got["dvalues"].sum(0, dtype=np.float64) - want).max() <= 1e-4 * np.abs(want).max()
    print("default backward", {k: f"{v:.2g}" for k, v in errs.items()}, flush=True)
    # the sparse value gradient (one chunk of all 1024 tokens): the same
    # touched rows, in order, against the oracle's rows
    sparse = _sparse_grads(torch, wl, x.shape[0])
    got_s, idx_s = gpu_backward(torch, wl, params, x, dout, max_batch=1024, grads=sparse)
    assert np.array_equal(idx_s, idx)
    U = int(got_s["dvalues_count"][0])
    assert U == rows.size and np.array_equal(got_s["dvalues_rows"][:U], rows)
    compare({"dvalues": got_s["dvalues_sparse"][:U]}, {"dval": ref["dval"][rows]})
