"""GPU: the flat exact search (pkm_flat_search) through the C ABI.

The flat search scores every one of the n^2 concatenated keys with one
D-long fp32 dot product.  By the exactness argument of "Product-Key Memory"
(§Factorising the key space) its top-k is the product search's, so it is
compared with the oracle's product search (pinned on the CPU to the fp64
flat search) under the lookup's index parity rule (tests/support.py: equal
winner sets, equal order wherever adjacent fp64 winners are at least tau
apart), and with the GPU's own product search on the same queries.  Scores:
|top - top_ref| <= 1e-5 * sum_i |q^_i| |key_i| + 1e-7, the scale of fp32
rounding of one D-long dot product.  With integer inputs every score is
exact, so indices, order under ties and scores must match bit for bit.
"""
import numpy as np
import pytest

import oracle
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


def _to(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(support.device())


def _search_params(torch, params):
    """Device parameters with the subkeys only (the flat search reads nothing else)."""
    dev = [_to(torch, params[key]) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")]
    return pk.Params(*dev, None)


def flat_vs_oracle(torch, wl, params, x):
    """Runs the GPU flat search on the oracle's q^ (rounded to fp32) and
    checks it against the oracle's product search and the GPU's."""
    model = support.model_for(wl, params)
    r = oracle.run(model, x, want=("qhat", "idx", "top"))
    _, tau = support.gaps_and_tau(wl, params, x, model)
    q32 = r["qhat"].astype(np.float32)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32", max_batch=max(1, x.shape[0]))
    P = _search_params(torch, params)
    say("flat search", wl, "B =", x.shape[0])
    qd = _to(torch, q32)
    idx, top = mem.flat_search(P, qd)
    # the GPU product search from the same fp32 queries
    scores = mem.score(P, qd)
    pidx, _ = mem.select(scores)
    torch.cuda.synchronize()
    idx, top, pidx = idx.cpu().numpy(), top.cpu().numpy(), pidx.cpu().numpy()

    support.check_indices(idx, r["idx"], r["top"], tau)
    support.check_indices(pidx, r["idx"], r["top"], tau)
    got = support.weights_by_index(idx, top.astype(np.float64), r["idx"])
    mass = np.empty_like(r["top"])
    for b in range(x.shape[0]):
        for h in range(wl.H):
            for j in range(wl.k):
                mass[b, h, j] = support.key_l1_mass(wl, params, r["qhat"][b, h], r["idx"][b, h, j], h)
    err = np.abs(got - r["top"]) / (mass + 1e-300)
    assert (np.abs(got - r["top"]) <= 1e-5 * mass + 1e-7).all(), float(err.max())
    return float(err.max())


@pytest.mark.parametrize("name,tokens", [("tiny", 8), ("mid", 64)])
def test_flat_search_small_workloads(torch, name, tokens):
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl, with_values=False)
    x = synthetic.make_x(wl)[:: max(1, wl.B // tokens)][:tokens].copy()
    support.gap_clean(wl, params, x)
    flat_vs_oracle(torch, wl, params, x)


@pytest.mark.slow
@pytest.mark.parametrize("name,tokens", [("default", 16), ("large_memory", 8)])
def test_flat_search_full_size(torch, name, tokens):
    """N = 1,048,576 and 4,194,304 keys per head: every key scored."""
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl, with_values=False)
    x = synthetic.make_x(wl)[:: wl.B // tokens][:tokens].copy()
    support.gap_clean(wl, params, x)
    err = flat_vs_oracle(torch, wl, params, x)
    print(f"{name}: flat search over {wl.N} keys, max score error {err:.3g} of the L1 mass", flush=True)


@pytest.mark.parametrize("shape", [
    dict(B=5, D=64, H=1, n=16, k=4),       # n^2 = 256: one pass
    dict(B=7, D=128, H=2, n=70, k=9),      # 4900 keys: two segments, short last one
    dict(B=6, D=128, H=2, n=65, k=64),     # 4225 keys (odd): scalar loads, last segment 129
    dict(B=3, D=64, H=1, n=2048, k=64),    # 4M keys: two merge passes
    dict(B=2, D=64, H=1, n=4096, k=32),    # the largest n_keys: 16.7M keys
    dict(B=4, D=64, H=3, n=8, k=8),        # k = n_keys
    dict(B=33, D=192, H=1, n=40, k=1),     # k = 1, one ragged 64-row tile
    dict(B=31, D=64, H=2, n=24, k=8),      # one ragged 32-row tile; n not a multiple of 32
    dict(B=70, D=128, H=2, n=24, k=8),     # two 64-row tiles, the second ragged
    dict(B=64, D=64, H=2, n=16, k=4),      # one full 64-row tile
    dict(B=65, D=64, H=1, n=16, k=4),      # a second 64-row tile holding one row
])
def test_flat_search_edge_shapes(torch, shape):
    wl = synthetic.Workload("flat_edge", shape["B"], shape["D"], shape["H"], shape["n"], shape["k"], "f32", "random")
    params = synthetic.make_params(wl, seed=5, with_values=False)
    x = synthetic.make_x(wl, seed=5)
    support.gap_clean(wl, params, x, seed=5)
    flat_vs_oracle(torch, wl, params, x)


@pytest.mark.parametrize("B,D,H,n,k", [(6, 64, 2, 64, 32), (3, 64, 1, 100, 64), (2, 128, 1, 300, 17),
                                       (40, 64, 1, 48, 16)])
def test_flat_search_exact_ties(torch, B, D, H, n, k):
    """Small integer queries and subkeys: every score is exact in fp32, and
    many keys tie.  The oracle's steps a4-a6 on the exact half scores give
    the canonical answer (score desc, flat index asc)."""
    rng = np.random.default_rng(11)
    q = rng.integers(-3, 4, size=(B, H, D)).astype(np.float32)
    sub = rng.integers(-2, 3, size=(H, 2, n, D // 2)).astype(np.float32)
    half = D // 2
    s = np.stack([np.einsum("bhd,hnd->bhn", q[..., p * half:(p + 1) * half].astype(np.float64),
                            sub[:, p].astype(np.float64)) for p in range(2)], axis=2)
    ref_idx, ref_top, _ = oracle.select(s, k)
    mem = pk.Memory(D, H, n, k, "f32", max_batch=B)
    dummy = np.zeros((H, D), np.float32)
    P = pk.Params(_to(torch, np.zeros((H, D, D), np.float32)), *[_to(torch, dummy) for _ in range(4)],
                  _to(torch, sub), None)
    say("flat search ties", B, D, H, n, k)
    idx, top = mem.flat_search(P, _to(torch, q))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(top.cpu().numpy().astype(np.float64), ref_top)


def threshold_counts(s, k):
    """For exact half scores s [B, H, 2, n]: per row of n^2 keys, how many
    scores are >= theta, the k-th largest maximum over groups of 64
    consecutive flat indices (the flat search keeps those in a list of 512
    and rescans rows with more)."""
    B, H, _, n = s.shape
    N = n * n
    flat = (s[:, :, 0, :, None] + s[:, :, 1, None, :]).reshape(B, H, N)
    G = (N + 63) // 64
    padded = np.full((B, H, G * 64), -np.inf)
    padded[..., :N] = flat
    gmax = padded.reshape(B, H, G, 64).max(-1)
    theta = -np.sort(-gmax, axis=-1)[..., k - 1]
    return (flat >= theta[..., None]).sum(-1)


@pytest.mark.parametrize("B,D,H,n,k,lo,hi,overflow", [
    (3, 64, 2, 128, 64, -1, 2, True),     # heavy ties at theta: rows rescanned
    (2, 64, 1, 67, 64, -1, 2, True),      # 4489 keys (odd: scalar loads), rescanned
    (3, 64, 2, 96, 16, -40, 41, False),   # wide integer range: every row from its list
])
def test_flat_search_threshold_paths(torch, B, D, H, n, k, lo, hi, overflow):
    """Rows of more than 4096 keys are topped through a threshold: the
    scores >= theta go to a list and a row with more than 512 of them is
    scanned in full.  Integer inputs make every score exact, so the test
    knows which rows take which path and the result must match the
    canonical answer bit for bit either way."""
    rng = np.random.default_rng(23)
    q = rng.integers(lo, hi, size=(B, H, D)).astype(np.float32)
    sub = rng.integers(lo, hi, size=(H, 2, n, D // 2)).astype(np.float32)
    half = D // 2
    s = np.stack([np.einsum("bhd,hnd->bhn", q[..., p * half:(p + 1) * half].astype(np.float64),
                            sub[:, p].astype(np.float64)) for p in range(2)], axis=2)
    assert np.abs(s).max() * 2 < 2 ** 24  # every score exact in fp32
    counts = threshold_counts(s, k)
    assert (counts >= k).all()
    assert bool((counts > 512).any()) == overflow, counts
    ref_idx, ref_top, _ = oracle.select(s, k)
    mem = pk.Memory(D, H, n, k, "f32", max_batch=B)
    dummy = np.zeros((H, D), np.float32)
    P = pk.Params(_to(torch, np.zeros((H, D, D), np.float32)), *[_to(torch, dummy) for _ in range(4)],
                  _to(torch, sub), None)
    say("flat search threshold paths", B, D, H, n, k, "list counts", counts.ravel().tolist())
    idx, top = mem.flat_search(P, _to(torch, q))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(top.cpu().numpy().astype(np.float64), ref_top)


def test_flat_search_arguments(torch):
    wl = synthetic.Workload("flat_err", 4, 64, 1, 16, 4, "f32", "unit")
    params = synthetic.make_params(wl, with_values=False)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32")
    P = _search_params(torch, params)
    q = torch.zeros((4, wl.H, wl.D), device=support.device())
    say("flat search arguments")
    small = torch.empty(mem.flat_workspace_bytes(4) - 256, dtype=torch.uint8, device=support.device())
    with pytest.raises(pk.PkmError) as e:
        mem.flat_search(P, q, workspace=small)
    assert e.value.status == pk.PKM_E_ARG
    with pytest.raises(pk.PkmError):
        mem.flat_workspace_bytes(65537)
    idx, top = mem.flat_search(P, torch.zeros((0, wl.H, wl.D), device=support.device()))
    torch.cuda.synchronize()
    assert idx.shape == (0, wl.H, wl.k)
