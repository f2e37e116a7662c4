"""GPU: the whole lookup through the C ABI against the fp64 oracle.

Index parity rule: identical winner sets for every compared (token, head),
and identical order wherever adjacent fp64 winners are at least tau apart
(tests/support.py).  Output tolerance, per token, max-norm relative:
1e-4 for fp32 tables, 2e-2 for bf16 / E4M3 tables (both sides decode the
same stored bits, so the table format adds no error of its own; the bound
covers fp32 scoring, softmax and accumulation).  Weights: |w - w_ref| within
the same tolerance, matched by index.
"""
import numpy as np
import pytest

import oracle
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


def compare(wl, params, x, out, idx, w, tokens=None, tau=None):
    """Oracle on the listed tokens (all by default) vs the GPU results; tau
    [len(tokens), H] as the gap-clean draw measured it (else measured here)."""
    tokens = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    model = support.model_for(wl, params)
    r = oracle.run(model, x[tokens], want=("out", "idx", "top", "w"))
    if tau is None:
        _, tau = support.gaps_and_tau(wl, params, x[tokens], model)
    support.check_indices(idx[tokens], r["idx"], r["top"], tau)
    tol = TOL[wl.table]
    wm = support.weights_by_index(idx[tokens], w[tokens], r["idx"])
    assert np.abs(wm - r["w"]).max() <= tol
    err = support.rel_rowmax_err(out[tokens], r["out"])
    assert err.max() <= tol, (err.max(), int(err.argmax()))
    return err


def invariants(wl, idx, w):
    """Properties every (token, head) must satisfy whatever the inputs."""
    assert ((idx >= 0) & (idx < wl.N)).all()
    s = np.sort(idx, -1)
    assert (s[..., 1:] != s[..., :-1]).all()
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-5)
    assert (np.diff(w, axis=-1) <= 1e-7).all()


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_forward_small_workloads_every_token(torch, name):
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)
    support.gap_clean(wl, params, x)
    out, idx, w = support.gpu_forward(wl, params, x)
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w)


def test_tiny_product_search_equals_flat_search(torch):
    """The exactness argument on the GPU: Tiny's winners equal the top-k of
    all 256 concatenated keys (brute force, fp64)."""
    from tests import pins

    wl = synthetic.WORKLOADS["tiny"]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)
    support.gap_clean(wl, params, x)
    out, idx, w = support.gpu_forward(wl, params, x)
    f = pins.flat_search(params, x, wl.k)
    assert (np.sort(idx, -1) == np.sort(f["idx"], -1)).all()


@pytest.mark.parametrize("shape", [
    dict(B=1000, D=64, H=2, n=100, k=7, table="f32"),      # ragged tiles, n not a multiple of 64
    dict(B=129, D=128, H=3, n=64, k=64, table="bf16"),     # k = n_keys: every key is a candidate
    dict(B=77, D=192, H=1, n=300, k=1, table="e4m3"),      # k = 1: argmax of each half
    dict(B=64, D=64, H=2, n=2048, k=64, table="bf16"),     # large n with the largest k
    dict(B=48, D=64, H=1, n=4096, k=64, table="int4"),     # the largest n_keys (16.8 M rows) and k
    dict(B=1, D=64, H=1, n=2, k=2, table="f32"),           # smallest memory
    dict(B=300, D=320, H=5, n=33, k=33, table="e4m3"),     # k = n, odd sizes, random BN
    dict(B=200, D=256, H=2, n=50, k=10, table="int8"),     # int8 table + row scales
    dict(B=150, D=192, H=3, n=40, k=16, table="int4"),     # int4 table: a row is D/2 bytes, half-active lanes
])
def test_forward_edge_shapes(torch, shape):
    wl = synthetic.Workload("edge", shape["B"], shape["D"], shape["H"], shape["n"], shape["k"], shape["table"],
                            "random")
    params = synthetic.make_params(wl, seed=3)
    x = synthetic.make_x(wl, seed=3)
    support.gap_clean(wl, params, x, seed=3)
    out, idx, w = support.gpu_forward(wl, params, x)
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w)


def _random_configs(count, seed):
    """Seeded random small configurations over the supported ranges (D a
    multiple of 64, 1 <= k <= min(64, n_keys), every table format, chunked
    and unchunked)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        D = int(rng.choice([64, 128, 192, 256, 320, 512]))
        n = int(rng.integers(2, 260))
        k = int(rng.integers(1, min(64, n) + 1))
        H = int(rng.integers(1, 5))
        B = int(rng.integers(1, 700))
        table = str(rng.choice(["f32", "bf16", "e4m3", "int8", "int4"]))
        max_batch = int(rng.choice([B, max(1, B // 3), 64]))
        out.append(dict(B=B, D=D, H=H, n=n, k=k, table=table, max_batch=max_batch, seed=int(100 + i)))
    return out


@pytest.mark.parametrize("cfg", _random_configs(12, 2026), ids=lambda c: "B{B}-D{D}-H{H}-n{n}-k{k}-{table}-mb{max_batch}".format(**c))
def test_forward_random_configs(torch, cfg):
    """The whole lookup on seeded random configurations against the oracle
    (every token), with the invariants."""
    wl = synthetic.Workload("rand", cfg["B"], cfg["D"], cfg["H"], cfg["n"], cfg["k"], cfg["table"], "random")
    params = synthetic.make_params(wl, seed=cfg["seed"])
    x = synthetic.make_x(wl, seed=cfg["seed"])
    support.gap_clean(wl, params, x, seed=cfg["seed"])
    out, idx, w = support.gpu_forward(wl, params, x, max_batch=cfg["max_batch"])
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w)


def test_forward_random_gamma_beta(torch):
    wl = synthetic.Workload("gb", 200, 256, 2, 128, 16, "f32", "random")
    params = synthetic.make_params(wl, seed=9)
    rng = np.random.default_rng(9)
    params["gamma"] = rng.uniform(0.5, 1.5, params["gamma"].shape).astype(np.float32)
    params["beta"] = rng.normal(0, 0.3, params["beta"].shape).astype(np.float32)
    x = synthetic.make_x(wl, seed=9)
    support.gap_clean(wl, params, x, seed=9)
    out, idx, w = support.gpu_forward(wl, params, x)
    compare(wl, params, x, out, idx, w)


@pytest.mark.parametrize("shape", [
    (1000, 256, 2, 128, 16, "bf16"),
    (333, 1024, 4, 1024, 32, "bf16"),   # the default widths, a ragged batch (fused select-gather)
    (4500, 1024, 4, 1024, 32, "bf16"),  # more tiles than CUs in both contractions (one workgroup per CU walks them)
    (300, 1024, 32, 64, 8, "bf16"),     # a wide projection over few tokens: 256 tiles in 2 rows (plain order)
    (70, 64, 3, 40, 8, "f32"),          # subkey rows of 32 floats: two chunks
    (257, 192, 1, 100, 12, "e4m3"),     # 12- and 6-chunk rows, a ragged 32-row group
    (40, 2048, 1, 64, 4, "bf16"),       # a wide model, few tokens (small tiles)
], ids=lambda s: "B{}-D{}-H{}-n{}-k{}-{}".format(*s))
def test_chunking_stages_and_determinism(torch, shape):
    """Chunked (max_batch < B) and unchunked runs, a second identical run and
    the four single-step calls composed by hand all give bitwise identical
    results (the forward takes the scoring's row exponents from the
    projection's recorded maxima and one pre-pass; the single steps compute
    their own)."""
    B, D, H, n, k, table = shape
    wl = synthetic.Workload("chunk", B, D, H, n, k, table, "random")
    params = synthetic.make_params(wl, seed=5)
    x = synthetic.make_x(wl, seed=5)
    P = pk.params_to_device(params, wl.table, support.device())
    a = support.gpu_forward(wl, params, x, max_batch=16384, dev_params=P)
    b = support.gpu_forward(wl, params, x, max_batch=16384, dev_params=P)
    c = support.gpu_forward(wl, params, x, max_batch=min(96, B - 1), dev_params=P)
    for u, v in zip(a, b):
        assert (u == v).all()
    for u, v in zip(a, c):
        assert (u == v).all()
    say("stages by hand")
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table)
    xt = torch.from_numpy(x).to(support.device())
    q = mem.query(P, xt)
    s = mem.score(P, q)
    idx, w = mem.select(s)
    out = mem.gather(P, idx, w)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == a[1]).all()
    assert (w.cpu().numpy() == a[2]).all()
    assert (out.cpu().numpy() == a[0]).all()


def test_empty_batch_and_argument_errors(torch):
    wl = synthetic.Workload("err", 4, 64, 1, 16, 4, "e4m3", "unit")
    params = synthetic.make_params(wl)
    P = pk.params_to_device(params, wl.table, support.device())
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table)
    say("empty batch")
    x0 = torch.zeros((0, wl.D), device=support.device())
    out, idx, w = mem.forward(P, x0)
    torch.cuda.synchronize()
    assert out.shape == (0, wl.D)
    # misaligned x: rejected on the host by the C ABI, nothing launched
    import ctypes

    xt = torch.zeros((5, wl.D), device=support.device())
    outt = torch.zeros((4, wl.D), device=support.device())
    st = torch.cuda.current_stream().cuda_stream
    rc = mem.lib.pkm_forward(mem._ctx, ctypes.byref(P.struct), 4, ctypes.c_void_p(xt.data_ptr() + 4),
                             ctypes.c_void_p(outt.data_ptr()), None, None, ctypes.c_void_p(st))
    assert rc == pk.PKM_E_ARG and "aligned" in pk.last_error()
    # an E4M3 table without row scales
    bad = pk.Params(*[P[name] for name in ("wq", "bn_mean", "bn_var", "bn_gamma", "bn_beta", "subkeys", "values")],
                    None)
    rc = mem.lib.pkm_forward(mem._ctx, ctypes.byref(bad.struct), 4, ctypes.c_void_p(xt.data_ptr()),
                             ctypes.c_void_p(outt.data_ptr()), None, None, ctypes.c_void_p(st))
    assert rc == pk.PKM_E_ARG and "value_scale" in pk.last_error()
    with pytest.raises(ValueError):
        mem.forward(P, torch.zeros((4, wl.D + 64), device=support.device()))


# Full-size workloads: every token is re-drawn until gap-clean, the GPU
# looks up the whole batch in one call (the configuration the benchmark
# times), and every token is compared with the oracle, in parts of at most
# 8192 tokens per test so that each test stays well inside a minute of
# oracle time.
FULL_PART = 8192
_FULL = {}


def _full_size(name):
    """(wl, params, x, tau, out, idx, w) of a full-size workload, built once
    per workload (the previous one is dropped)."""
    if name not in _FULL:
        _FULL.clear()
        wl = synthetic.WORKLOADS[name]
        print(f"[cpu] {name}: drawing inputs", flush=True)
        params = synthetic.make_params(wl)
        x = synthetic.make_x(wl)
        print(f"[cpu] {name}: gap-clean draw of all {wl.B} tokens", flush=True)
        attempts, tau = support.gap_clean(wl, params, x, want_tau=True)
        print(f"[cpu] {name}: {(attempts > 0).sum()} tokens re-drawn", flush=True)
        out, idx, w = support.gpu_forward(wl, params, x, max_batch=wl.B)
        invariants(wl, idx, w)
        _FULL[name] = (wl, params, x, tau, out, idx, w)
    return _FULL[name]


def _full_size_parts():
    for name in ("default", "default_int8", "default_int4", "large_memory", "large_batch"):
        B = synthetic.WORKLOADS[name].B
        for t0 in range(0, B, FULL_PART):
            yield name, t0, min(B, t0 + FULL_PART)


@pytest.mark.slow
@pytest.mark.parametrize("name,t0,t1", list(_full_size_parts()), ids=lambda v: str(v))
def test_forward_full_size_every_token(torch, name, t0, t1):
    wl, params, x, tau, out, idx, w = _full_size(name)
    tokens = np.arange(t0, t1)
    print(f"[cpu] {name}: oracle on tokens {t0}..{t1 - 1}", flush=True)
    err = compare(wl, params, x, out, idx, w, tokens=tokens, tau=tau[tokens])
    print(f"{name} tokens {t0}..{t1 - 1}: max row error {err.max():.3g}", flush=True)


def test_usage_counts(torch):
    """pkm_usage on the forward's winners equals the oracle's counts; a
    second call adds; rows repeated by identical tokens count each time."""
    wl = synthetic.WORKLOADS["mid"]
    params = synthetic.make_params(wl)
    x = synthetic.make_x(wl)
    x[500:600] = x[7]  # a hot token: its rows occur 101 times per head
    _, idx, _ = support.gpu_forward(wl, params, x)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table)
    say("usage counts")
    it = torch.from_numpy(idx).to(support.device())
    counts = mem.usage(it)
    counts = mem.usage(it, counts)
    torch.cuda.synchronize()
    got = counts.cpu().numpy().astype(np.int64)
    ref = oracle.usage(idx, wl.N, oracle.usage(idx, wl.N)).astype(np.int64)
    assert (got == ref).all()
    assert got.sum() == 2 * idx.size and got.max() >= 2 * 101
