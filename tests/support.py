"""Shared helpers for the tests: gap-clean inputs and comparison rules.

Index parity between the fp64 oracle and an fp32 GPU path is only meaningful
when no score near the k | k+1 boundary is closer than the fp32 error.  For
each (token, head) the gap between the k-th and (k+1)-th best full scores
(the oracle's product search at depth k+1, which is the exact top-(k+1) by the
exactness argument of "Product-Key Memory", §Factorising the key space) must
be at least

    tau = max(TAU_ABS, TAU_REL * sum_i |q^_i| * |key_i|)

where key is the concatenated key of the k-th winner: the fp32 rounding error
of a dot product is proportional to that L1 mass, not to the score itself.
Tokens that fail are re-drawn from their own seeded stream.
"""
import numpy as np

import oracle
import synthetic

TAU_ABS = 1e-6
TAU_REL = 1e-6


def model_for(wl, params, eps=1e-5):
    return oracle.Model.from_params(params, wl.k, wl.table, eps)


def key_l1_mass(wl, params, qhat, flat, h):
    """sum_i |q^_i| |key_i| for the concatenated key of flat row `flat`."""
    half, n = wl.D // 2, wl.n
    a, b = int(flat) // n, int(flat) % n
    c0 = params["subkeys"][h, 0, a].astype(np.float64)
    c1 = params["subkeys"][h, 1, b].astype(np.float64)
    return float(np.abs(qhat[:half]) @ np.abs(c0) + np.abs(qhat[half:]) @ np.abs(c1))


def taus(wl, params, qhat, flat):
    """tau for every (token, head) from q^ [B, H, D] and the flat row of
    its k-th winner [B, H] (vectorised key_l1_mass)."""
    half, n = wl.D // 2, wl.n
    flat = np.asarray(flat, np.int64)
    heads = np.arange(wl.H)[None, :]
    c0 = np.abs(params["subkeys"][heads, 0, flat // n]).astype(np.float64)  # [B, H, D/2]
    c1 = np.abs(params["subkeys"][heads, 1, flat % n]).astype(np.float64)
    q = np.abs(qhat)
    mass = np.einsum("bhd,bhd->bh", q[..., :half], c0) + np.einsum("bhd,bhd->bh", q[..., half:], c1)
    return np.maximum(TAU_ABS, TAU_REL * mass)


def gaps_and_tau(wl, params, x, model=None):
    """Per (token, head): fp64 gap between the k-th and (k+1)-th full scores,
    and the tau it must clear.  Both [B, H]."""
    k = wl.k
    if k + 1 <= wl.n:
        model = model or model_for(wl, params)
        r = oracle.run(model, x, kk=k + 1, want=("top", "idx", "qhat"))
    else:
        # k = n_keys: a half has no (k+1)-th subkey, so take the exact
        # top-(k+1) from the flat search over all n_keys^2 keys instead
        from tests import pins

        r = pins.flat_search(params, x, k + 1, with_values=False)
    gap = r["top"][:, :, k - 1] - r["top"][:, :, k]
    return gap, taus(wl, params, r["qhat"], r["idx"][:, :, k - 1])


def gap_clean(wl, params, x, tokens=None, seed=0, max_attempts=60, want_tau=False, chunk=4096):
    """Re-draw rows of x (in place) until every listed token clears tau on
    every head.  Returns the per-token attempt counts (and, with want_tau,
    the tau [B, H] of the final draw for the listed tokens; NaN elsewhere).
    The oracle runs over at most `chunk` tokens at a time."""
    model = model_for(wl, params)
    todo = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    attempts = np.zeros(x.shape[0], dtype=np.int64)
    tau_all = np.full((x.shape[0], wl.H), np.nan)
    if wl.k >= wl.N:  # no (k+1)-th key: every key is a winner
        tau_all[todo] = TAU_ABS
        return (attempts, tau_all) if want_tau else attempts
    for _ in range(max_attempts):
        bad = []
        for c0 in range(0, todo.size, chunk):
            part = todo[c0:c0 + chunk]
            gap, tau = gaps_and_tau(wl, params, x[part], model)
            tau_all[part] = tau
            bad.append(part[(gap < tau).any(axis=1)])
        bad = np.concatenate(bad) if bad else todo[:0]
        if bad.size == 0:
            return (attempts, tau_all) if want_tau else attempts
        for b in bad:
            attempts[b] += 1
            x[b] = synthetic.redraw_row(wl, seed, b, attempts[b])
        todo = bad
    raise RuntimeError("gap-clean draw did not converge")


def gap_clean_batch_stats(wl, params, x, seed=0, max_rounds=60):
    """gap_clean for the lookup with batch statistics: re-drawing a token
    moves every token's statistics, so the gaps of the whole batch are
    measured again after each round of re-draws.  Returns (mean, var) of
    the final batch (fp64 [H,D]) and the tau of every (token, head)."""
    model = model_for(wl, params)
    attempts = np.zeros(x.shape[0], dtype=np.int64)
    k = wl.k
    for _ in range(max_rounds):
        mean, var = oracle.batch_stats(model, x)
        r = oracle.run_batch_stats(model, x, mean, var, kk=k + 1, want=("top", "idx", "qhat"))
        gap = r["top"][:, :, k - 1] - r["top"][:, :, k]
        tau = taus(wl, params, r["qhat"], r["idx"][:, :, k - 1])
        bad = np.nonzero((gap < tau).any(axis=1))[0]
        if bad.size == 0:
            return mean, var, tau
        for b in bad:
            attempts[b] += 1
            x[b] = synthetic.redraw_row(wl, seed, b, attempts[b])
    raise RuntimeError("gap-clean draw with batch statistics did not converge")


def rel_rowmax_err(got, ref):
    """Per row: max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-300)


def check_indices(idx, ref_idx, ref_top, tau):
    """Index parity: identical winner sets per (token, head); the order must
    agree wherever adjacent fp64 winners are at least tau apart (inside a
    run of nearer scores the order is not pinned).  idx/ref_idx [B,H,k],
    ref_top [B,H,k] fp64, tau [B,H] or a scalar."""
    idx = np.asarray(idx)
    ref_idx = np.asarray(ref_idx)
    assert idx.shape == ref_idx.shape
    same_set = (np.sort(idx, -1) == np.sort(ref_idx, -1)).all(-1)
    bad = np.argwhere(~same_set)
    assert bad.size == 0, f"winner sets differ at (token, head) {bad[:5].tolist()}"
    tau = np.broadcast_to(np.asarray(tau, np.float64), ref_top.shape[:-1])[..., None]
    # a gap of at least tau between reference positions p-1 and p starts a new
    # block; blocks must appear in the same order, members in any order
    gaps = ref_top[..., :-1] - ref_top[..., 1:]
    cut = np.concatenate([np.ones(gaps.shape[:-1] + (1,), bool), gaps >= tau], axis=-1)
    block = np.cumsum(cut, axis=-1)
    B, H, _ = idx.shape
    for b in range(B):
        for h in range(H):
            pos = {int(v): i for i, v in enumerate(ref_idx[b, h])}
            got_blocks = np.array([block[b, h, pos[int(v)]] for v in idx[b, h]])
            assert (got_blocks == block[b, h]).all(), f"order differs at token {b} head {h}"


# ------------------------------------------------------------------ GPU side

def device():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def say(*args):
    """Names the case about to touch the GPU (flushed, so a lost box still
    tells which case was running)."""
    print("[gpu]", *args, flush=True)


def gpu_forward(wl, params, x, max_batch=16384, mem=None, dev_params=None):
    """Runs the whole lookup on the GPU; returns numpy (out, idx, w)."""
    import torch

    import product_key_memory_amd as pk

    say("forward", wl, "B =", x.shape[0], "max_batch =", max_batch)
    mem = mem or pk.Memory(wl.D, wl.H, wl.n, wl.k, wl.table, max_batch=max_batch)
    P = dev_params or pk.params_to_device(params, wl.table, device())
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(device())
    out, idx, w = mem.forward(P, xt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def weights_by_index(idx, w, ref_idx):
    """Reorders w [B,H,k] so that entry j belongs to ref_idx[..., j] (the
    winner sets are already known to be equal)."""
    order = np.argsort(idx, -1)
    ref_order = np.argsort(ref_idx, -1)
    sorted_w = np.take_along_axis(w, order, -1)
    inv = np.argsort(ref_order, -1)
    return np.take_along_axis(sorted_w, inv, -1)


def to_device(a):
    """A numpy array as a contiguous tensor on the GPU."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device())
