"""GPU: each kernel of the HIP path against the fp64 oracle, fed identical
inputs, through the C ABI."""
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


def test_e4m3_decode_every_code(torch):
    """All 256 E4M3 codes through the gather (row scale 1, weight 1) equal the
    oracle's decoder exactly (the two NaN codes excepted)."""
    say("gather e4m3 all codes")
    mem = pk.Memory(256, 1, 2, 1, "e4m3")
    values = np.zeros((4, 256), np.uint8)
    values[0] = np.arange(256, dtype=np.uint8)
    values[1] = np.arange(256, dtype=np.uint8)[::-1]
    scale = np.ones(4, np.float32)
    scale[1] = 0.5
    p = {"wq": np.zeros((1, 256, 256), np.float32), "mean": np.zeros((1, 256), np.float32),
         "var": np.ones((1, 256), np.float32), "gamma": np.ones((1, 256), np.float32),
         "beta": np.zeros((1, 256), np.float32), "subkeys": np.zeros((1, 2, 2, 128), np.float32),
         "values": values, "scale": scale}
    P = pk.params_to_device(p, "e4m3", support.device())
    idx = _to(torch, np.array([[0], [1]], np.int32))
    w = _to(torch, np.ones((2, 1), np.float32))
    out = mem.gather(P, idx, w).cpu().numpy()
    ref = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    ok = ~np.isnan(ref)
    assert (out[0][ok] == ref[ok]).all()
    assert (out[1][ok[::-1]] == 0.5 * ref[::-1][ok[::-1]]).all()


@pytest.mark.parametrize("table", ["int8", "int4"])
def test_integer_decode_every_code(torch, table):
    """Every int8 code (and every int4 code in both nibbles of a byte)
    through the gather, row scale 1 then 0.25, equals the oracle's decoder
    times the scale exactly."""
    say("gather", table, "all codes")
    D = 256 if table == "int8" else 512
    mem = pk.Memory(D, 1, 2, 1, table)
    if table == "int8":
        codes = np.arange(-128, 128, dtype=np.int8)
        values = np.zeros((4, D), np.int8)
        values[0], values[1] = codes, codes[::-1]
        ref0 = np.array([oracle.int8_to_f64(int(c)) for c in codes])
        ref1 = ref0[::-1]
    else:
        lo, hi = np.meshgrid(np.arange(16, dtype=np.uint8), np.arange(16, dtype=np.uint8), indexing="ij")
        byte = (lo | (hi << np.uint8(4))).reshape(-1)  # all 256 (low, high) pairs
        values = np.zeros((4, D // 2), np.uint8)
        values[0], values[1] = byte, byte[::-1]
        dec = np.array([oracle.int4_to_f64(c) for c in range(16)])

        def expand(b):
            out = np.empty(2 * b.size)
            out[0::2], out[1::2] = dec[b & 0xF], dec[b >> 4]
            return out

        ref0, ref1 = expand(byte), expand(byte[::-1])
    scale = np.array([1.0, 0.25, 1.0, 1.0], np.float32)
    p = {"wq": np.zeros((1, D, D), np.float32), "mean": np.zeros((1, D), np.float32),
         "var": np.ones((1, D), np.float32), "gamma": np.ones((1, D), np.float32),
         "beta": np.zeros((1, D), np.float32), "subkeys": np.zeros((1, 2, 2, D // 2), np.float32),
         "values": values, "scale": scale}
    P = pk.params_to_device(p, table, support.device())
    idx = _to(torch, np.array([[0], [1]], np.int32))
    w = _to(torch, np.ones((2, 1), np.float32))
    out = mem.gather(P, idx, w).cpu().numpy()
    assert (out[0] == ref0).all()
    assert (out[1] == 0.25 * ref1).all()


def test_bf16_decode_every_code(torch):
    """All 65536 bf16 codes (16 rows of 4096) decode exactly; non-finite codes
    are skipped."""
    say("gather bf16 all codes")
    mem = pk.Memory(4096, 1, 4, 1, "bf16")
    values = np.arange(1 << 16, dtype=np.uint16).reshape(16, 4096)
    p = {"wq": np.zeros((1, 4096, 4096), np.float32), "mean": np.zeros((1, 4096), np.float32),
         "var": np.ones((1, 4096), np.float32), "gamma": np.ones((1, 4096), np.float32),
         "beta": np.zeros((1, 4096), np.float32), "subkeys": np.zeros((1, 2, 4, 2048), np.float32),
         "values": values, "scale": None}
    P = pk.params_to_device(p, "bf16", support.device())
    idx = _to(torch, np.arange(16, dtype=np.int32).reshape(16, 1))
    w = _to(torch, np.ones((16, 1), np.float32))
    out = mem.gather(P, idx, w).cpu().numpy().reshape(-1)
    ref = np.array([oracle.bf16_to_f64(c) for c in range(1 << 16)])
    ok = np.isfinite(ref)
    assert (out[ok] == ref[ok]).all()


@pytest.mark.parametrize("table", ["f32", "bf16", "e4m3", "int8", "int4"])
@pytest.mark.parametrize("D,n,B,R", [(64, 16, 5, 4), (512, 64, 33, 16), (1024, 32, 17, 128), (1024, 32, 9, 130),
                                     (192, 8, 7, 1), (2048, 16, 3, 67),
                                     # rows of two column slices, the second one partial (fp32 at 384, bf16 at
                                     # 768) or full (int4 at 4096): one wave reads them whole
                                     (384, 16, 9, 33), (768, 32, 11, 20), (4096, 8, 3, 9)])
def test_gather_parity(torch, table, D, n, B, R):
    """Gather fed the same rows and fp32 weights as the oracle.  Both decode
    the same stored bits exactly; the only difference is fp32 vs fp64
    accumulation over R rows, bounded here by 1e-5 of the row max."""
    wl = synthetic.Workload("g", B, D, 1, n, 1, table, "unit")
    values, scale = synthetic.make_values(wl, seed=7)
    rows, w = synthetic.uniform_rows(wl, 7, B, R)
    say("gather", table, "D", D, "n", n, "B", B, "R", R)
    mem = pk.Memory(D, 1, n, 1, table)
    p = {"wq": np.zeros((1, D, D), np.float32), "mean": np.zeros((1, D), np.float32),
         "var": np.ones((1, D), np.float32), "gamma": np.ones((1, D), np.float32),
         "beta": np.zeros((1, D), np.float32), "subkeys": np.zeros((1, 2, n, D // 2), np.float32),
         "values": values, "scale": scale}
    P = pk.params_to_device(p, table, support.device())
    out = mem.gather(P, _to(torch, rows), _to(torch, w)).cpu().numpy()
    model = oracle.Model.from_params(p, 1, table)
    ref = oracle.gather(model, rows, w.astype(np.float64))
    err = support.rel_rowmax_err(out, ref)
    assert err.max() <= 1e-5, err.max()


@pytest.mark.parametrize("n,k", [(16, 4), (256, 16), (1024, 32), (2048, 32), (100, 7), (64, 64), (4096, 64),
                                 (1024, 1), (1024, 33), (2, 2), (300, 64)])
@pytest.mark.parametrize("spread", [1 << 20, 64, 3])
def test_select_parity_exact(torch, n, k, spread):
    """Select fed the same half scores as the oracle.  Scores are multiples
    of 2^-10 below 2^13, so the fp32 candidate sums are exact and both sides
    rank identical numbers: winners and their order must match bit for bit,
    ties included (spread 3 makes nearly every score a tie, which drives the
    bisection path).  Weights: fp32 exp/sum vs fp64, within 1e-6."""
    B, H = 37, 3
    rng = np.random.default_rng([n, k, spread])
    s = (rng.integers(-spread, spread + 1, size=(B, H, 2, n)) % 8192).astype(np.float64)
    s = np.where(rng.random(s.shape) < 0.5, -s, s) / 1024.0
    scores = s.astype(np.float32)
    assert (scores.astype(np.float64) == s).all()
    say("select n", n, "k", k, "spread", spread)
    mem = pk.Memory(64, H, n, k, "f32")
    idx, w = mem.select(_to(torch, scores))
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    ref_idx, ref_top, ref_w = oracle.select(s, k)
    assert (idx == ref_idx).all(), np.argwhere(idx != ref_idx)[:5]
    assert np.abs(w - ref_w).max() <= 1e-6


def test_select_random_scores_sets(torch):
    """Continuous random scores at the default shape: winner sets equal the
    oracle's wherever its k | k+1 gap clears fp32 rounding of the sums."""
    B, H, n, k = 256, 4, 1024, 32
    s = np.random.default_rng(11).standard_normal((B, H, 2, n)).astype(np.float32) * 20
    say("select random n", n, "k", k)
    mem = pk.Memory(64, H, n, k, "f32")
    idx, w = mem.select(_to(torch, s))
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    ref_idx, ref_top, ref_w = oracle.select(s.astype(np.float64), k + 1)
    gap = ref_top[..., k - 1] - ref_top[..., k]
    tau = 1e-5 * np.abs(ref_top[..., 0]) + 1e-6
    clean = gap >= tau
    assert clean.mean() > 0.95
    support.check_indices(idx[clean][:, None], ref_idx[..., :k][clean][:, None], ref_top[..., :k][clean][:, None],
                          tau[clean][:, None])
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_query_and_score_parity(torch, name):
    """Projection + BN and the subkey scores against fp64, element by element:
    |error| <= 1e-5 of the dot product's L1 mass (sum |a_i b_i|), the scale
    of fp32 rounding of a sum of products."""
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl, with_values=False)
    params["values"] = np.zeros((wl.N, wl.D), np.float32)
    params["scale"] = None
    x = synthetic.make_x(wl)[:256]
    B = x.shape[0]
    r = oracle.run(support.model_for(wl, params), x, want=("qhat",))
    say("query/score", name)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32")
    P = pk.params_to_device(params, "f32", support.device())
    qhat = mem.query(P, _to(torch, x)).cpu().numpy().astype(np.float64)
    inv = 1.0 / np.sqrt(params["var"].astype(np.float64) + 1e-5) * np.abs(params["gamma"])
    mass = np.einsum("hfd,bd->bhf", np.abs(params["wq"]).astype(np.float64), np.abs(x).astype(np.float64)) * inv
    assert (np.abs(qhat - r["qhat"]) <= 1e-5 * mass + 1e-7).all()
    # scores from the oracle's q^ rounded to fp32 (so only the scoring differs)
    q32 = r["qhat"].astype(np.float32)
    scores = mem.score(P, _to(torch, q32)).cpu().numpy().astype(np.float64)
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    for h in range(wl.H):
        for p in range(2):
            qp = q32[:, h, p * half:(p + 1) * half].astype(np.float64)
            ref = qp @ sub[h, p].T
            m = np.abs(qp) @ np.abs(sub[h, p]).T
            assert (np.abs(scores[:, h, p] - ref) <= 1e-5 * m + 1e-7).all()


def test_query_and_score_persistent_ragged(torch):
    """More 256x256 tiles than CUs (4,389 tokens: 288 projection tiles and
    576 scoring tiles over 256 workgroups, the last tile row ragged) take
    the path where each workgroup walks several tiles.  Sampled tokens,
    including every row of the ragged tile, against fp64 as above."""
    wl = synthetic.Workload("persist", 4389, 1024, 4, 1024, 32, "f32", "random")
    params = synthetic.make_params(wl, with_values=False, seed=3)
    params["values"] = np.zeros((1, wl.D), np.float32)
    params["scale"] = None
    x = synthetic.make_x(wl, seed=3)
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32", max_batch=wl.B)
    dev = [_to(torch, params[key]) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")]
    P = pk.Params(*dev, None)
    say("persistent query/score", wl.B, "tokens")
    qhat = mem.query(P, _to(torch, x)).cpu().numpy()
    tokens = np.array(sorted(set(range(0, wl.B, 97)) | set(range(4352, wl.B)) | {255, 256, 4095, 4096}))
    w64 = params["wq"].astype(np.float64)
    xs = x[tokens].astype(np.float64)
    inv = params["gamma"].astype(np.float64) / np.sqrt(params["var"].astype(np.float64) + 1e-5)
    ref = (np.einsum("hfd,bd->bhf", w64, xs) - params["mean"]) * inv + params["beta"]
    mass = np.einsum("hfd,bd->bhf", np.abs(w64), np.abs(xs)) * np.abs(inv)
    assert (np.abs(qhat[tokens] - ref) <= 1e-5 * mass + 1e-7).all()
    scores = mem.score(P, _to(torch, qhat)).cpu().numpy()[tokens].astype(np.float64)
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    for h in range(wl.H):
        for p in range(2):
            qp = qhat[tokens, h, p * half:(p + 1) * half].astype(np.float64)
            r = qp @ sub[h, p].T
            m = np.abs(qp) @ np.abs(sub[h, p]).T
            assert (np.abs(scores[:, h, p] - r) <= 1e-5 * m + 1e-7).all()


def test_query_and_score_wide_range(torch):
    """The contractions scale every operand row by a power of two before
    splitting it into fp16 pieces, so rows of any size keep fp32 accuracy:
    token rows multiplied by 2^-30 .. 2^30, projection rows by 2^-20 ..
    2^20 and subkey rows by 2^-25 .. 2^25 (far outside fp16's range either
    way), checked element by element against fp64 as above (1e-5 of the L1
    mass)."""
    wl = synthetic.Workload("range", 96, 128, 2, 64, 8, "f32", "random")
    params = synthetic.make_params(wl, with_values=False, seed=7)
    params["values"] = np.zeros((wl.N, wl.D), np.float32)
    params["scale"] = None
    rng = np.random.default_rng(7)
    x = synthetic.make_x(wl, seed=7) * np.exp2(rng.integers(-30, 31, (wl.B, 1))).astype(np.float32)
    params["wq"] = params["wq"] * np.exp2(rng.integers(-20, 21, (wl.H, wl.D, 1))).astype(np.float32)
    params["subkeys"] = params["subkeys"] * np.exp2(rng.integers(-25, 26, (wl.H, 2, wl.n, 1))).astype(np.float32)
    x[5] = 0.0  # a row of zeros
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "f32")
    P = pk.params_to_device(params, "f32", support.device())
    say("wide-range query/score")
    qhat = mem.query(P, _to(torch, x)).cpu().numpy().astype(np.float64)
    w64 = params["wq"].astype(np.float64)
    inv = params["gamma"].astype(np.float64) / np.sqrt(params["var"].astype(np.float64) + 1e-5)
    q = np.einsum("hfd,bd->bhf", w64, x.astype(np.float64))
    ref = (q - params["mean"]) * inv + params["beta"]
    mass = np.einsum("hfd,bd->bhf", np.abs(w64), np.abs(x).astype(np.float64)) * np.abs(inv)
    assert np.isfinite(qhat).all()
    assert (np.abs(qhat - ref) <= 1e-5 * mass + 1e-6 * np.abs(ref) + 1e-30).all()
    q32 = (qhat * np.exp2(rng.integers(-30, 31, (wl.B, 1, 1)))).astype(np.float32)
    scores = mem.score(P, _to(torch, q32)).cpu().numpy().astype(np.float64)
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    for h in range(wl.H):
        for p in range(2):
            qp = q32[:, h, p * half:(p + 1) * half].astype(np.float64)
            r = qp @ sub[h, p].T
            m = np.abs(qp) @ np.abs(sub[h, p]).T
            assert np.isfinite(scores[:, h, p]).all()
            assert (np.abs(scores[:, h, p] - r) <= 1e-5 * m + 1e-30).all()


@pytest.mark.parametrize("name", ["mid", "default", "large_memory"])
def test_score_error_guard(torch, name):
    """The index-parity rule needs tau to exceed twice the largest full-score
    error of the fp32 path (a gap above 2 * (e0 + e1) keeps the winner set).
    Measured here on the GPU's own projection + scoring of sampled tokens
    against fp64: for every (token, head), max|ds0| + max|ds1| <= tau / 2."""
    wl = synthetic.WORKLOADS[name]
    params = synthetic.make_params(wl, with_values=False)
    x = synthetic.make_x(wl)[:: max(1, wl.B // 96)][:96].copy()
    say("score error guard", name, "tokens", x.shape[0])
    mem = pk.Memory(wl.D, wl.H, wl.n, wl.k, "bf16")
    # query and score read only Wq, the BN arrays and the subkeys
    P = pk.Params(*[_to(torch, params[key]) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")], None)
    q = mem.query(P, _to(torch, x))
    s = mem.score(P, q).cpu().numpy().astype(np.float64)
    r = oracle.run(support.model_for(wl, params), x, kk=wl.k + 1, want=("qhat", "idx", "top"))
    half = wl.D // 2
    sub = params["subkeys"].astype(np.float64)
    worst = 0.0
    for h in range(wl.H):
        e = []
        for p in range(2):
            ref = r["qhat"][:, h, p * half:(p + 1) * half] @ sub[h, p].T
            e.append(np.abs(s[:, h, p] - ref).max(axis=1))
        err_full = e[0] + e[1]
        for b in range(x.shape[0]):
            tau = max(support.TAU_ABS, support.TAU_REL * support.key_l1_mass(wl, params, r["qhat"][b, h],
                                                                           r["idx"][b, h, wl.k - 1], h))
            worst = max(worst, err_full[b] / tau)
    print(f"{name}: max over (token, head) of full-score error / tau = {worst:.3f}", flush=True)
    assert worst <= 0.5
