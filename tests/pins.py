"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (the default
build, or a variant passed as ``lib``) disagrees with:
  - library routines that define a step: torch's Linear, BatchNorm1d
    (inference), softmax and embedding_bag(mode="sum", per_sample_weights),
    the bf16 / float8_e4m3fn / int8 casts, and an arithmetic-shift decode of
    two's complement nibbles for int4;
  - the flat exact search the "Product-Key Memory" page contrasts the method
    with (§Factorising the key space): every one of the N = n_keys^2
    concatenated keys (c0_a, c1_b) is scored with one full-length dot product
    and the best k kept -- the page's exactness argument says the product
    search must return the same winners;
  - hand-worked closed forms (tests/golden/hand_example.json) and the page's
    operation counts (tests/golden/op_counts.json);
  - special cases: k = n_keys (every key is a candidate), k = 1 (argmax of
    each half), exact integer ties (lower index wins).
The stand-alone steps are pinned on their own:
  - select (steps 4-6 from given half scores) against a brute force over
    the whole n x n grid of half-score sums (the score of key (a, b) is
    s0[a] + s1[b], §Factorising the key space), ranked by (score desc,
    flat index asc), and torch's softmax; and bit for bit against run() on
    the oracle's own half scores;
  - gather (step 7) against torch's embedding_bag(mode="sum",
    per_sample_weights) on every table format, into a garbage-filled output;
  - the running-statistics update against the buffers torch's
    F.batch_norm(training=True, momentum=m) updates in place.
The backward direction (gradients of sum(dout * out)) is pinned to:
  - torch autograd in fp64 through the method written from its definition,
    per head and summed over heads: Linear, BatchNorm1d, the score of
    every one of the n^2 concatenated keys, the best k of them, softmax,
    and the weighted sum of their value rows;
  - central finite differences of the oracle's own forward output, with
    steps that are exact in fp32 and small enough not to change the winners;
  - identities: the value gradient sums to H * sum_b dout_b (each head's
    weights sum to 1); each subkey set's gradient sums to zero over its rows
    (the softmax Jacobian's rows sum to zero); zero dout gives zero gradients.
"""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def unpack_int4(packed):
    """[rows, D/2] bytes -> [rows, D] int8: each nibble sign-extended by an
    arithmetic right shift of the byte that holds it in its high half."""
    b = np.ascontiguousarray(packed, dtype=np.uint8)
    low = (b << np.uint8(4)).view(np.int8) >> 4
    high = b.view(np.int8) >> 4
    out = np.empty((b.shape[0], 2 * b.shape[1]), np.int8)
    out[:, 0::2], out[:, 1::2] = low, high
    return out


def dequant_table(values, scale, table):
    """fp64 copy of a stored table, decoded by torch's own casts (int4:
    unpack_int4)."""
    if table == "f32":
        return torch.from_numpy(values).double()
    if table == "bf16":
        return torch.from_numpy(values.view(np.int16)).view(torch.bfloat16).double()
    if table == "int8":
        return torch.from_numpy(values.view(np.int8)).double() * torch.from_numpy(scale).double()[:, None]
    if table == "int4":
        return torch.from_numpy(unpack_int4(values)).double() * torch.from_numpy(scale).double()[:, None]
    v = torch.from_numpy(values).view(torch.float8_e4m3fn).double()
    return v * torch.from_numpy(scale).double()[:, None]


def flat_search(params, x, k, eps=1e-5, table="f32", with_values=True):
    """The flat exact search, written with torch CPU library routines in fp64.

    Returns idx [B,H,k] (score desc, flat asc), top [B,H,k], w [B,H,k],
    qhat [B,H,D] and (if with_values) out [B,D]."""
    wq = torch.from_numpy(params["wq"]).double()
    H, D, _ = wq.shape
    sub = torch.from_numpy(params["subkeys"]).double()
    n = sub.shape[2]
    xt = torch.from_numpy(np.ascontiguousarray(x)).double()
    B = xt.shape[0]
    vals = dequant_table(params["values"], params.get("scale"), table) if with_values else None
    out = torch.zeros(B, D, dtype=torch.float64)
    idx = torch.empty(B, H, k, dtype=torch.int64)
    top = torch.empty(B, H, k, dtype=torch.float64)
    w = torch.empty(B, H, k, dtype=torch.float64)
    qhat = torch.empty(B, H, D, dtype=torch.float64)
    for h in range(H):
        q = F.linear(xt, wq[h])
        qh = F.batch_norm(q, torch.from_numpy(params["mean"][h]).double(), torch.from_numpy(params["var"][h]).double(),
                          torch.from_numpy(params["gamma"][h]).double(), torch.from_numpy(params["beta"][h]).double(),
                          training=False, eps=eps)
        qhat[:, h] = qh
        # key a*n + b is the concatenation (c0_a, c1_b); scored in chunks of a
        scores = torch.empty(B, n * n, dtype=torch.float64)
        step = max(1, (1 << 22) // (n * D))
        for a0 in range(0, n, step):
            a1 = min(n, a0 + step)
            keys = torch.cat([sub[h, 0, a0:a1].repeat_interleave(n, 0), sub[h, 1].repeat(a1 - a0, 1)], dim=1)
            scores[:, a0 * n:a1 * n] = qh @ keys.T
        order = torch.sort(scores, dim=1, descending=True, stable=True).indices[:, :k]
        t = torch.gather(scores, 1, order)
        idx[:, h], top[:, h] = order, t
        w[:, h] = torch.softmax(t, dim=-1)
        if with_values:
            out += F.embedding_bag(order, vals, per_sample_weights=w[:, h], mode="sum")
    res = {"idx": idx.numpy().astype(np.int32), "top": top.numpy(), "w": w.numpy(), "qhat": qhat.numpy()}
    if with_values:
        res["out"] = out.numpy()
    return res


def _model(params, k, table, eps=1e-5):
    return oracle.Model.from_params(params, k, table, eps)


def _assert_same_winners(got, ref, top_ref, tol_gap=1e-9):
    """Same sets; same order wherever neighbours differ by more than rounding."""
    assert (np.sort(got, -1) == np.sort(ref, -1)).all(), "winner sets differ"
    gaps = top_ref[..., :-1] - top_ref[..., 1:]
    pinned = np.concatenate([gaps > tol_gap, np.ones(gaps.shape[:-1] + (1,), bool)], -1)
    pinned &= np.concatenate([np.ones(gaps.shape[:-1] + (1,), bool), gaps > tol_gap], -1)
    assert (got[pinned] == ref[pinned]).all(), "winner order differs"


def pin_against_flat_search(wl, seed=0, tokens=None, gamma_beta=False, lib=None, rtol=1e-10):
    """Oracle == flat exact search with library routines, on one workload."""
    params = synthetic.make_params(wl, seed)
    if gamma_beta:
        rng = np.random.default_rng([seed, 1234])
        params["gamma"] = rng.uniform(0.5, 1.5, params["gamma"].shape).astype(np.float32)
        params["beta"] = rng.normal(0, 0.3, params["beta"].shape).astype(np.float32)
    x = synthetic.make_x(wl, seed)
    if tokens is not None:
        x = x[tokens]
    r = oracle.run(_model(params, wl.k, wl.table), x, want=("out", "idx", "top", "w", "qhat", "ncand"), lib=lib)
    f = flat_search(params, x, wl.k, table=wl.table)
    np.testing.assert_allclose(r["qhat"], f["qhat"], rtol=1e-12, atol=1e-12)
    _assert_same_winners(r["idx"], f["idx"], f["top"])
    np.testing.assert_allclose(r["top"], f["top"], rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(r["w"], f["w"], rtol=rtol, atol=1e-12)
    np.testing.assert_allclose(r["out"], f["out"], rtol=rtol, atol=1e-10)
    assert (r["ncand"] == wl.k * wl.k).all()
    return r


def pin_hand_example(lib=None):
    """The worked example of tests/golden/hand_example.json."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    inp = g["inputs"]
    D, n = inp["D"], inp["n"]
    values = np.array([[r, 1.0, -r, r / 2.0] for r in range(n * n)], np.float32)
    params = {key: np.array(inp[key], np.float32) for key in ("wq", "mean", "var", "gamma", "beta", "subkeys")}
    params["values"], params["scale"] = values, None
    x = np.array(inp["x"], np.float32)
    e = g["expected"]
    r2 = oracle.run(_model(params, 2, "f32", inp["eps"]), x, want=("out", "idx", "top", "w", "ncand"), lib=lib)
    assert r2["idx"][0, 0].tolist() == e["k2"]["idx"]
    np.testing.assert_allclose(r2["top"][0, 0], e["k2"]["top"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r2["w"][0, 0], e["k2"]["w"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r2["out"][0], e["k2"]["out"], rtol=0, atol=1e-14)
    assert r2["ncand"][0, 0] == 4
    r3 = oracle.run(_model(params, 3, "f32", inp["eps"]), x, want=("out", "idx", "top", "w", "ncand"), lib=lib)
    a = 1.0 / (2.0 + math.exp(-1.0))
    c = math.exp(-1.0) / (2.0 + math.exp(-1.0))
    assert r3["idx"][0, 0].tolist() == e["k3"]["idx"]
    np.testing.assert_allclose(r3["top"][0, 0], e["k3"]["top"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r3["w"][0, 0], [a, a, c], rtol=1e-15, atol=0)
    np.testing.assert_allclose(r3["out"][0], [13 * a, 1.0, -13 * a, 6.5 * a], rtol=1e-14, atol=1e-15)
    assert r3["ncand"][0, 0] == 9


def integer_tie_params(H=2, D=8, n=6, seed=5):
    """Small integer-valued inputs with duplicated subkeys.  Every score is
    an exact small integer, so ties are exact whatever the summation order."""
    rng = np.random.default_rng(seed)
    half = D // 2
    sub = rng.integers(-2, 3, size=(H, 2, n, half)).astype(np.float32)
    sub[:, 0, n - 1] = sub[:, 0, 1]  # duplicate subkeys -> exact ties
    sub[:, 1, 3] = sub[:, 1, 0]
    sub[:, 1, n - 1] = sub[:, 1, 2]
    p = {
        "wq": np.stack([np.eye(D, dtype=np.float32)] * H),
        "mean": np.zeros((H, D), np.float32),
        "var": np.full((H, D), 0.75, np.float32),  # var + eps = 1 exactly (eps = 0.25)
        "gamma": np.ones((H, D), np.float32),
        "beta": np.zeros((H, D), np.float32),
        "subkeys": sub,
        "values": rng.standard_normal((n * n, D)).astype(np.float32),
        "scale": None,
    }
    x = rng.integers(-2, 3, size=(16, D)).astype(np.float32)
    return p, x


def pin_integer_ties(lib=None):
    """Exact ties: the lowest index must win, in both halves and in the grid,
    for every k from 1 to n_keys."""
    p, x = integer_tie_params()
    n = p["subkeys"].shape[2]
    for k in range(1, n + 1):
        r = oracle.run(_model(p, k, "f32", 0.25), x, want=("idx", "top", "w", "out"), lib=lib)
        f = flat_search(p, x, k, eps=0.25)
        assert (r["idx"] == f["idx"]).all(), f"tie order differs at k={k}"
        np.testing.assert_array_equal(r["top"], f["top"])
        np.testing.assert_allclose(r["w"], f["w"], rtol=1e-14)
        np.testing.assert_allclose(r["out"], f["out"], rtol=1e-12, atol=1e-12)


def pin_k_equals_1(lib=None):
    """k = 1: the winner is (argmax of half 0, argmax of half 1), weight 1."""
    wl = synthetic.Workload("k1", 32, 32, 2, 12, 1, "f32", "random")
    params = synthetic.make_params(wl, 3)
    x = synthetic.make_x(wl, 3)
    r = oracle.run(_model(params, 1, "f32"), x, want=("idx", "w", "out", "qhat"), lib=lib)
    f = flat_search(params, x, 1)
    half = wl.D // 2
    for h in range(wl.H):
        s0 = f["qhat"][:, h, :half] @ params["subkeys"][h, 0].astype(np.float64).T
        s1 = f["qhat"][:, h, half:] @ params["subkeys"][h, 1].astype(np.float64).T
        assert (r["idx"][:, h, 0] == s0.argmax(1) * wl.n + s1.argmax(1)).all()
    assert (r["w"] == 1.0).all()
    np.testing.assert_allclose(r["out"], f["out"], rtol=1e-12, atol=1e-12)


def pin_codecs(lib=None):
    """Decoders vs torch's casts on every bf16 and E4M3 code."""
    b = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(v, lib) for v in b])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert (got[ok] == ref[ok]).all(), "bf16 decoder differs from torch"
    e = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(e).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_to_f64(v, lib) for v in e])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert (got[ok] == ref[ok]).all(), "E4M3 decoder differs from torch"
    # format landmarks: largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9
    assert oracle.e4m3_to_f64(0x7E, lib) == 448.0
    assert oracle.e4m3_to_f64(0x08, lib) == 2.0 ** -6
    assert oracle.e4m3_to_f64(0x01, lib) == 2.0 ** -9
    assert oracle.e4m3_to_f64(0xB8, lib) == -1.0
    codes = np.arange(-128, 128, dtype=np.int8)
    ref = torch.from_numpy(codes).double().numpy()
    assert (np.array([oracle.int8_to_f64(int(c), lib) for c in codes]) == ref).all(), "int8 decoder"
    nib = np.arange(16, dtype=np.uint8)
    ref = unpack_int4(nib[:, None])[:, 0].astype(np.float64)  # each code in a low nibble
    assert (np.array([oracle.int4_to_f64(int(c), lib) for c in nib]) == ref).all(), "int4 decoder"
    assert oracle.int4_to_f64(0x8, lib) == -8.0 and oracle.int4_to_f64(0x7, lib) == 7.0


def pin_softmax_large_scores(lib=None):
    """Scores in the thousands: the max-subtracted softmax stays finite and
    matches torch.softmax."""
    wl = synthetic.Workload("big", 8, 32, 1, 8, 4, "f32", "unit")
    params = synthetic.make_params(wl, 1)
    params["subkeys"] = params["subkeys"] * np.float32(400.0)
    x = synthetic.make_x(wl, 1)
    r = oracle.run(_model(params, wl.k, "f32"), x, want=("w", "top", "out"), lib=lib)
    assert np.isfinite(r["w"]).all() and np.isfinite(r["out"]).all()
    assert r["top"].max() > 1000.0
    f = flat_search(params, x, wl.k)
    np.testing.assert_allclose(r["w"], f["w"], rtol=1e-9, atol=1e-300)


def pin_op_counts(lib=None):
    """The page's counts at n_keys = 1024, k = 32: 2048 subkey scores (two
    halves of 1024) and 1024 candidates."""
    g = json.load(open(os.path.join(GOLDEN, "op_counts.json")))
    n, k = g["n_keys"], g["k"]
    wl = synthetic.Workload("counts", 2, 8, 1, n, k, "f32", "unit")
    params = synthetic.make_params(wl, 0, with_values=False)
    params["values"] = np.zeros((n * n, wl.D), np.float32)
    r = oracle.run(_model(params, k, "f32"), synthetic.make_x(wl, 0), want=("ncand", "idx"), lib=lib)
    assert 2 * n == g["subkey_scores"]
    assert (r["ncand"] == g["candidates"]).all()
    assert r["idx"].shape[-1] == k


def _brute_force_select(s, k):
    """Top-k of the full n x n grid of half-score sums for one (token,
    head): s [2, n] fp64.  Returns flat indices, scores, softmax weights."""
    n = s.shape[1]
    grid = (s[0][:, None] + s[1][None, :]).reshape(-1)  # cell a*n + b holds s0[a] + s1[b]
    flat = np.arange(n * n)
    order = np.lexsort((flat, -grid))[:k]  # score desc, then flat index asc
    top = grid[order]
    return order.astype(np.int32), top, torch.softmax(torch.from_numpy(top), -1).numpy()


def pin_select(lib=None):
    """select() against the brute force over the whole grid: random fp64
    scores (every k up to n at a small n, and a larger n), exact integer
    ties; then bit for bit against run() on the oracle's own half scores."""
    rng = np.random.default_rng(21)
    cases = [(rng.standard_normal((30, 2, 9)), k) for k in range(1, 10)]
    cases.append((rng.standard_normal((25, 2, 70)) * 3.0, 16))
    cases.append((rng.integers(-2, 3, (40, 2, 12)).astype(np.float64), 5))  # heavy exact ties
    cases.append((rng.integers(-1, 2, (20, 2, 6)).astype(np.float64), 6))
    for s, k in cases:
        idx, top, w = oracle.select(s, k, lib=lib)
        for p in range(s.shape[0]):
            ri, rt, rw = _brute_force_select(s[p], k)
            assert (idx[p] == ri).all(), f"select winners differ (k={k}, row {p})"
            assert (top[p] == rt).all(), "select scores differ"
            np.testing.assert_allclose(w[p], rw, rtol=1e-13, atol=1e-300)
    # the same function on the scores the lookup ranks: bit for bit
    wl = synthetic.Workload("sel", 20, 64, 3, 24, 7, "f32", "random")
    params = synthetic.make_params(wl, 11, with_values=False)
    model = _model(params, wl.k, wl.table)
    x = synthetic.make_x(wl, 11)
    sc = oracle.scores(model, x, lib=lib)
    idx, top, w = oracle.select(sc, wl.k, lib=lib)
    r = oracle.run(model, x, want=("idx", "top", "w"), lib=lib)
    assert (idx == r["idx"]).all() and (top == r["top"]).all() and (w == r["w"]).all(), "select differs from run"
    # half scores against library products of the oracle's own q^
    qh = oracle.run(model, x, want=("qhat",), lib=lib)["qhat"]
    half = wl.D // 2
    for h in range(wl.H):
        for p in range(2):
            ref = qh[:, h, p * half:(p + 1) * half] @ params["subkeys"][h, p].astype(np.float64).T
            np.testing.assert_allclose(sc[:, h, p], ref, rtol=1e-12, atol=1e-12)


def pin_gather(lib=None):
    """gather() against torch's embedding_bag(mode="sum",
    per_sample_weights) in fp64 on every table format: repeated rows inside
    and across bags, one-row bags, an output buffer full of garbage (every
    entry must be overwritten), and an empty batch."""
    rng = np.random.default_rng(31)
    for t, table in enumerate(("f32", "bf16", "e4m3", "int8", "int4")):
        wl = synthetic.Workload("gat", 1, 64, 1, 8, 2, table, "unit")
        params = synthetic.make_params(wl, 40 + t)
        model = _model(params, wl.k, table)
        vals = dequant_table(params["values"], params.get("scale"), table)
        for B, R in ((17, 9), (5, 1), (0, 4)):
            rows = rng.integers(0, wl.N, (B, R)).astype(np.int32)
            if B and R > 2:
                rows[0, 1] = rows[0, 0]  # a repeat inside a bag
                rows[1, :] = rows[0, 0]  # a bag of one row R times
            w = rng.standard_normal((B, R))
            out = np.full((B, wl.D), np.nan)
            got = oracle.gather(model, rows, w, out=out, lib=lib)
            ref = F.embedding_bag(torch.from_numpy(rows.astype(np.int64)), vals, mode="sum",
                                  per_sample_weights=torch.from_numpy(w)).numpy()
            assert got.shape == (B, wl.D)
            np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def pin_running_update(lib=None):
    """The running statistics after a training-mode batch: the oracle's
    update (from the oracle's own batch statistics, or from given ones)
    against the buffers torch's F.batch_norm(training=True, momentum=m)
    updates in place, for several batch sizes and momenta."""
    rng = np.random.default_rng(51)
    for B, m in ((2, 0.1), (7, 0.37), (100, 0.1), (33, 0.0), (5, 1.0)):
        q = rng.standard_normal((B, 48)) * rng.uniform(0.2, 3.0, 48) + rng.normal(0, 2, 48)
        rm0, rv0 = rng.normal(0, 1, 48), rng.uniform(0.5, 2.0, 48)
        trm, trv = torch.from_numpy(rm0.copy()), torch.from_numpy(rv0.copy())
        F.batch_norm(torch.from_numpy(q), trm, trv, training=True, momentum=m)
        rm, rv = oracle.running_update(rm0, rv0, q.mean(0), q.var(0), B, m, lib=lib)
        np.testing.assert_allclose(rm, trm.numpy(), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(rv, trv.numpy(), rtol=1e-14, atol=1e-15)
    # chained with the oracle's batch statistics of a lookup's queries
    wl = synthetic.Workload("run", 12, 32, 2, 8, 3, "f32", "random")
    params = synthetic.make_params(wl, 52, with_values=False)
    model = _model(params, wl.k, wl.table)
    x = synthetic.make_x(wl, 52)
    mean, var = oracle.batch_stats(model, x, lib=lib)
    rm0 = rng.normal(0, 1, (wl.H, wl.D))
    rv0 = rng.uniform(0.5, 2.0, (wl.H, wl.D))
    rm, rv = oracle.running_update(rm0, rv0, mean, var, wl.B, 0.1, lib=lib)
    xt = torch.from_numpy(x).double()
    for h in range(wl.H):
        trm, trv = torch.from_numpy(rm0[h].copy()), torch.from_numpy(rv0[h].copy())
        F.batch_norm(F.linear(xt, torch.from_numpy(params["wq"][h]).double()), trm, trv, training=True, momentum=0.1)
        np.testing.assert_allclose(rm[h], trm.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rv[h], trv.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ backward

def module_autograd(params, x, dout, k, table="f32", eps=1e-5, training=False):
    """Gradients of sum(dout * out) by torch autograd in fp64 through the
    method written from its definition, per head and summed over heads:
    q^ = BatchNorm1d(Linear(x)); every key (a, b) is the concatenation
    [c0_a; c1_b] ("Product-Key Memory", §Factorising the key space) and
    gets the score q^ . key; the best k scores of all n^2 keys (score desc,
    flat index a*n + b asc) are the winners; their softmax weights the sum
    of their value rows.  Gradients reach the subkeys through the keys they
    form.  With training=True BatchNorm1d normalises with the batch's
    statistics (and the result holds "out", "mean" and "var" too)."""
    leaf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).double().requires_grad_()  # noqa: E731
    wq, gamma, beta, sub = leaf(params["wq"]), leaf(params["gamma"]), leaf(params["beta"]), leaf(params["subkeys"])
    vals = dequant_table(params["values"], params.get("scale"), table).clone().requires_grad_()
    xt = leaf(x)
    mean = torch.from_numpy(params["mean"]).double()
    var = torch.from_numpy(params["var"]).double()
    H, D, _ = wq.shape
    n = sub.shape[2]
    out = torch.zeros(x.shape[0], D, dtype=torch.float64)
    stats = ([], [])
    for h in range(H):
        q = F.linear(xt, wq[h])
        if training:
            stats[0].append(q.detach().mean(0))
            stats[1].append(q.detach().var(0, unbiased=False))
            qh = F.batch_norm(q, None, None, gamma[h], beta[h], training=True, eps=eps)
        else:
            qh = F.batch_norm(q, mean[h], var[h], gamma[h], beta[h], training=False, eps=eps)
        first = torch.arange(n).repeat_interleave(n)  # key a*n + b = [c0_a; c1_b]
        second = torch.arange(n).repeat(n)
        keys = torch.cat([sub[h, 0][first], sub[h, 1][second]], dim=1)
        scores = qh @ keys.T
        win = torch.sort(scores.detach(), dim=1, descending=True, stable=True).indices[:, :k]
        w = torch.softmax(scores.gather(1, win), dim=-1)
        out = out + (w[:, :, None] * vals[win]).sum(dim=1)
    (out * torch.from_numpy(dout).double()).sum().backward()
    res = {"dx": xt.grad.numpy(), "dwq": wq.grad.numpy(), "dgamma": gamma.grad.numpy(),
           "dbeta": beta.grad.numpy(), "dsub": sub.grad.numpy(), "dval": vals.grad.numpy()}
    if training:
        res.update(out=out.detach().numpy(), mean=torch.stack(stats[0]).numpy(), var=torch.stack(stats[1]).numpy())
    return res


def backward_case(wl, seed=0, gamma_beta=False):
    params = synthetic.make_params(wl, seed)
    if gamma_beta:
        rng = np.random.default_rng([seed, 1234])
        params["gamma"] = rng.uniform(0.5, 1.5, params["gamma"].shape).astype(np.float32)
        params["beta"] = rng.normal(0, 0.3, params["beta"].shape).astype(np.float32)
    x = synthetic.make_x(wl, seed)
    dout = np.random.default_rng([seed, 77]).standard_normal(x.shape).astype(np.float32)
    return params, x, dout


def pin_backward_autograd(wl, seed=0, gamma_beta=False, lib=None):
    """Oracle gradients == torch autograd through the method's definition."""
    params, x, dout = backward_case(wl, seed, gamma_beta)
    g = oracle.backward(_model(params, wl.k, wl.table), x, dout, lib=lib)
    ref = module_autograd(params, x, dout, wl.k, wl.table)
    for name in oracle.GRADS:
        scale = max(np.abs(ref[name]).max(), 1e-300)
        err = np.abs(g[name] - ref[name]).max() / scale
        assert err <= 1e-10, f"{name}: max error {err:.3g} of its largest entry"
    return g


def _loss(params, x, dout, k, table, lib, eps=1e-5):
    r = oracle.run(_model(params, k, table, eps), x, want=("out", "idx"), lib=lib)
    return float((r["out"] * dout.astype(np.float64)).sum()), r["idx"]


def pin_backward_finite_differences(lib=None, coords=10):
    """Central differences of the oracle's forward loss against its
    gradients, on a small fp32 workload with random gamma / beta.  Steps are
    powers of two, so theta +- step is exact in fp32; a coordinate whose
    step changes the winners is skipped (at most a fifth of them)."""
    wl = synthetic.Workload("fd", 6, 16, 2, 8, 3, "f32", "random")
    params, x, dout = backward_case(wl, 4, gamma_beta=True)
    g = oracle.backward(_model(params, wl.k, wl.table), x, dout, lib=lib)
    _, idx0 = _loss(params, x, dout, wl.k, wl.table, lib)
    rng = np.random.default_rng(9)
    targets = {"dx": ("x", None), "dwq": ("wq", None), "dgamma": ("gamma", None), "dbeta": ("beta", None),
               "dsub": ("subkeys", None), "dval": ("values", None)}
    checked = skipped = 0
    for gname, (pname, _) in targets.items():
        grad = g[gname]
        flat = grad.reshape(-1)
        # the largest gradients and a few random coordinates (zero ones too)
        pick = list(np.argsort(-np.abs(flat))[:coords // 2]) + list(rng.integers(0, flat.size, coords // 2))
        for c in pick:
            arr = x if pname == "x" else params[pname]
            base = arr.reshape(-1)[c]
            step = np.float32(2.0 ** -14)
            hi, lo = np.float32(base + step), np.float32(base - step)
            assert hi - base == step and base - lo == step
            def loss_at(v):
                saved = arr.reshape(-1)[c]
                arr.reshape(-1)[c] = v
                try:
                    return _loss(params, x, dout, wl.k, wl.table, lib)
                finally:
                    arr.reshape(-1)[c] = saved
            lp, ip = loss_at(hi)
            lm, im = loss_at(lo)
            if not (np.array_equal(ip, idx0) and np.array_equal(im, idx0)):
                skipped += 1
                continue
            fd = (lp - lm) / (2.0 * float(step))
            assert abs(fd - flat[c]) <= 1e-6 + 1e-5 * abs(flat[c]), f"{gname}[{c}]: fd {fd} vs {flat[c]}"
            checked += 1
    assert skipped * 5 <= checked + skipped, f"{skipped} of {checked + skipped} coordinates changed the winners"


def pin_backward_identities(lib=None):
    """Sum of the value gradient, zero-sum subkey gradients, zero dout."""
    wl = synthetic.Workload("ident", 40, 32, 3, 12, 5, "bf16", "random")
    params, x, dout = backward_case(wl, 6, gamma_beta=True)
    model = _model(params, wl.k, wl.table)
    g = oracle.backward(model, x, dout, lib=lib)
    want = wl.H * dout.astype(np.float64).sum(0)
    np.testing.assert_allclose(g["dval"].sum(0), want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    sums = g["dsub"].sum(axis=2)  # over the subkeys of each (head, half)
    assert np.abs(sums).max() <= 1e-12 * max(np.abs(g["dsub"]).max(), 1e-300)
    z = oracle.backward(model, x, np.zeros_like(dout), lib=lib)
    for name in oracle.GRADS:
        assert not z[name].any(), name



def pin_batch_stats_autograd(wl, seed=0, lib=None):
    """Batch-statistics BN: the oracle's statistics, forward output and
    gradients == torch (F.batch_norm(training=True)) in fp64 through the
    method's definition."""
    params, x, dout = backward_case(wl, seed, gamma_beta=True)
    model = _model(params, wl.k, wl.table)
    mean, var = oracle.batch_stats(model, x, lib=lib)
    ref = module_autograd(params, x, dout, wl.k, wl.table, training=True)
    np.testing.assert_allclose(mean, ref["mean"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(var, ref["var"], rtol=1e-12, atol=1e-12)
    r = oracle.run_batch_stats(model, x, mean, var, lib=lib)
    np.testing.assert_allclose(r["out"], ref["out"], rtol=1e-10, atol=1e-12)
    g = oracle.backward_batch_stats(model, x, dout, mean, var, lib=lib)
    for name in oracle.GRADS:
        scale = max(np.abs(ref[name]).max(), 1e-300)
        err = np.abs(g[name] - ref[name]).max() / scale
        assert err <= 1e-10, f"{name}: max error {err:.3g} of its largest entry"
    return g


def pin_batch_stats_finite_differences(lib=None, coords=8):
    """Central differences of the batch-statistics loss (statistics
    recomputed at every step) against the batch-statistics gradients."""
    wl = synthetic.Workload("fdb", 6, 16, 2, 8, 3, "f32", "unit")
    params, x, dout = backward_case(wl, 7, gamma_beta=True)

    def loss():
        model = _model(params, wl.k, wl.table)
        mean, var = oracle.batch_stats(model, x, lib=lib)
        r = oracle.run_batch_stats(model, x, mean, var, want=("out", "idx"), lib=lib)
        return float((r["out"] * dout.astype(np.float64)).sum()), r["idx"]

    model = _model(params, wl.k, wl.table)
    mean, var = oracle.batch_stats(model, x, lib=lib)
    g = oracle.backward_batch_stats(model, x, dout, mean, var, lib=lib)
    _, idx0 = loss()
    rng = np.random.default_rng(13)
    checked = skipped = 0
    for gname, arr in (("dx", x), ("dwq", params["wq"]), ("dgamma", params["gamma"]), ("dbeta", params["beta"]),
                       ("dsub", params["subkeys"])):
        flat = g[gname].reshape(-1)
        for c in list(np.argsort(-np.abs(flat))[:coords // 2]) + list(rng.integers(0, flat.size, coords // 2)):
            base = arr.reshape(-1)[c]
            step = np.float32(2.0 ** -14)
            vals = []
            for v in (np.float32(base + step), np.float32(base - step)):
                arr.reshape(-1)[c] = v
                vals.append(loss())
            arr.reshape(-1)[c] = base
            if not (np.array_equal(vals[0][1], idx0) and np.array_equal(vals[1][1], idx0)):
                skipped += 1
                continue
            fd = (vals[0][0] - vals[1][0]) / (2.0 * float(step))
            assert abs(fd - flat[c]) <= 1e-6 + 1e-5 * abs(flat[c]), f"{gname}[{c}]: fd {fd} vs {flat[c]}"
            checked += 1
    assert skipped * 5 <= checked + skipped