"""Seeded synthetic inputs for the product-key memory lookup.

This module only draws random numbers and encodes the value table into its
storage format.  It holds none of the lookup's arithmetic; the oracle and the
HIP library both take what it produces as plain inputs.

Workloads (B tokens, model width D, H heads, n subkeys per half so the table
has N = n*n rows, k winners per head):

  tiny          B=8      D=64   H=1 n=16   k=4   fp32 table, unit BN
  mid           B=1024   D=512  H=4 n=256  k=16  fp32 table, random BN stats
  default       B=4096   D=1024 H=4 n=1024 k=32  bf16 table (the "Product-Key
                                                 Memory" module's defaults)
  large_batch   B=65536  D=1024 H=4 n=1024 k=32  bf16 table
  large_memory  B=16384  D=1024 H=4 n=2048 k=32  E4M3 table + fp32 row scale
  default_int8 / default_int4: the default shape with an int8 / int4 table
                + fp32 row scale

Distributions (second argument of N is the variance):
  x ~ N(0,1); Wq[h] ~ N(0,1/D); subkeys ~ N(0,1); values ~ N(0,1/sqrt(D));
  BN running stats: mean 0, var 1 (unit) or mean ~ N(0,0.1), var ~ U(0.5,2)
  (random); gamma 1, beta 0.

Every array is drawn from its own numpy PCG64 stream keyed by (seed, tag[,
chunk]), so the bits do not depend on thread count or on which arrays are
drawn first.  Row b of x can be re-drawn from a per-token stream keyed by
(seed, b, attempt).
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np

_TAG_X, _TAG_WQ, _TAG_MEAN, _TAG_VAR, _TAG_SUB, _TAG_VAL, _TAG_XROW = 1, 2, 3, 4, 5, 6, 7
_CHUNK_ROWS = 16384  # value-table rows per independent stream


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    D: int
    H: int
    n: int
    k: int
    table: str  # "f32" | "bf16" | "e4m3" | "int8" | "int4"
    bn: str  # "unit" | "random"

    @property
    def N(self):
        return self.n * self.n

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 8, 64, 1, 16, 4, "f32", "unit"),
        Workload("mid", 1024, 512, 4, 256, 16, "f32", "random"),
        Workload("default", 4096, 1024, 4, 1024, 32, "bf16", "unit"),
        Workload("large_batch", 65536, 1024, 4, 1024, 32, "bf16", "unit"),
        Workload("large_memory", 16384, 1024, 4, 2048, 32, "e4m3", "unit"),
        # the default shape with the lower-precision tables
        Workload("default_int8", 4096, 1024, 4, 1024, 32, "int8", "unit"),
        Workload("default_int4", 4096, 1024, 4, 1024, 32, "int4", "unit"),
    ]
}


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _normal(key, shape, std):
    out = np.random.default_rng(key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def f32_to_bf16_bits(a):
    """Round-to-nearest-even fp32 -> bf16 (finite inputs), as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_e4m3_rows(a):
    """Per-row scaled OCP E4M3 (E4M3FN) encoding of a [rows, D] fp32 block.

    scale_r = max|a_r| / 448 (1 for an all-zero row); codes are a_r / scale_r
    rounded to nearest even and saturated to +-448.  Returns (uint8 codes,
    float32 scales)."""
    import torch  # CPU cast only

    a = np.ascontiguousarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(a / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def f32_to_int8_rows(a):
    """Per-row symmetric int8: scale_r = max|a_r| / 127 (1 for an all-zero
    row), codes a_r / scale_r rounded to nearest even, in [-127, 127].
    Returns (int8 codes, float32 scales)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(a / scale[:, None]), -127, 127).astype(np.int8)
    return q, scale


def f32_to_int4_rows(a):
    """Per-row symmetric int4: scale_r = max|a_r| / 7, codes in [-7, 7]
    rounded to nearest even, two per byte (even element in the low nibble).
    Returns (uint8 [rows, D/2], float32 scales)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(a / scale[:, None]), -7, 7).astype(np.int8).view(np.uint8) & np.uint8(0xF)
    return (q[:, 0::2] | (q[:, 1::2] << np.uint8(4))).astype(np.uint8), scale


SCALED_TABLES = ("e4m3", "int8", "int4")  # tables stored with a per-row fp32 scale


def table_shape(wl):
    return (wl.N, wl.D // 2) if wl.table == "int4" else (wl.N, wl.D)


def make_values(wl, seed=0):
    """Value table [N, D] in the workload's storage format (+ row scales);
    int4 tables are [N, D/2] bytes."""
    N, D = wl.N, wl.D
    std = float(D) ** -0.25
    dtype = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "int8": np.int8, "int4": np.uint8}[wl.table]
    values = np.empty(table_shape(wl), dtype=dtype)
    scale = np.empty((N,), dtype=np.float32) if wl.table in SCALED_TABLES else None
    nchunks = (N + _CHUNK_ROWS - 1) // _CHUNK_ROWS

    def fill(c):
        r0, r1 = c * _CHUNK_ROWS, min(N, (c + 1) * _CHUNK_ROWS)
        v = _normal([seed, _TAG_VAL, c], (r1 - r0, D), std)
        if wl.table == "f32":
            values[r0:r1] = v
        elif wl.table == "bf16":
            values[r0:r1] = f32_to_bf16_bits(v)
        elif wl.table == "int8":
            values[r0:r1], scale[r0:r1] = f32_to_int8_rows(v)
        elif wl.table == "int4":
            values[r0:r1], scale[r0:r1] = f32_to_int4_rows(v)
        else:
            values[r0:r1], scale[r0:r1] = f32_to_e4m3_rows(v)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return values, scale


def make_params(wl, seed=0, with_values=True):
    """All parameters of the lookup as numpy arrays (host memory)."""
    H, D, n = wl.H, wl.D, wl.n
    p = {
        "wq": _normal([seed, _TAG_WQ], (H, D, D), 1.0 / np.sqrt(D)),
        "subkeys": _normal([seed, _TAG_SUB], (H, 2, n, D // 2), 1.0),
        "gamma": np.ones((H, D), np.float32),
        "beta": np.zeros((H, D), np.float32),
    }
    if wl.bn == "unit":
        p["mean"] = np.zeros((H, D), np.float32)
        p["var"] = np.ones((H, D), np.float32)
    else:
        p["mean"] = _normal([seed, _TAG_MEAN], (H, D), np.sqrt(0.1))
        p["var"] = np.random.default_rng([seed, _TAG_VAR]).uniform(0.5, 2.0, (H, D)).astype(np.float32)
    if with_values:
        p["values"], p["scale"] = make_values(wl, seed)
    return p


def make_x(wl, seed=0, B=None):
    """Tokens x [B, D] ~ N(0, 1)."""
    B = wl.B if B is None else B
    return _normal([seed, _TAG_X], (B, wl.D), 1.0)


def redraw_row(wl, seed, b, attempt):
    """A fresh draw of token row b from its own stream (seed, b, attempt)."""
    return _normal([seed, _TAG_XROW, int(b), int(attempt)], (wl.D,), 1.0)


def uniform_rows(wl, seed, B, rows_per_token):
    """Uniformly random table rows [B, rows_per_token] (int32) and positive
    weights [B, rows_per_token] (fp32, each token's weights sum to 1), for
    driving the gather on its own with no pipeline locality."""
    rng = np.random.default_rng([seed, 99])
    idx = rng.integers(0, wl.N, size=(B, rows_per_token), dtype=np.int64).astype(np.int32)
    w = rng.random((B, rows_per_token), dtype=np.float32) + np.float32(0.01)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)
