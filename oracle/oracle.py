"""ctypes front end of ``pkm_oracle.c`` (the plain fp64 CPU oracle).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The arithmetic lives in
``pkm_oracle.c``; this file only marshals numpy arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

VALUE_TYPES = {"f32": 0, "bf16": 1, "e4m3": 2, "int8": 3, "int4": 4}
SCALED = ("e4m3", "int8", "int4")  # tables with a per-row fp32 scale


def lib_path():
    return _LIB


def build():
    """Compile the oracle with gcc: -O2, no -ffast-math, so every fp64 sum
    keeps the order written in the source."""
    tmp = f"{_LIB}.{os.getpid()}.tmp"  # parallel test workers may build at once
    compile_source(_SRC, tmp)
    os.replace(tmp, _LIB)
    global _lib
    _lib = None
    return _LIB


class _Model(ctypes.Structure):
    _fields_ = [
        ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
        ("value_type", ctypes.c_int32), ("pad_", ctypes.c_int32), ("eps", ctypes.c_double),
        ("wq", ctypes.c_void_p), ("mean", ctypes.c_void_p), ("var", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("subkeys", ctypes.c_void_p),
        ("values", ctypes.c_void_p), ("scale", ctypes.c_void_p),
    ]


_lib = None


def load_library(path):
    """Open a compiled oracle (the default one, or a variant built from an
    edited copy of the source by the tests that check the pins)."""
    lib = ctypes.CDLL(path)
    lib.pkmo_run.restype = ctypes.c_int
    lib.pkmo_run.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, ctypes.c_void_p, ctypes.c_int] + \
        [ctypes.c_void_p] * 6 + [ctypes.c_int]
    lib.pkmo_bf16_to_f64.restype = ctypes.c_double
    lib.pkmo_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.pkmo_e4m3_to_f64.restype = ctypes.c_double
    lib.pkmo_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.pkmo_int8_to_f64.restype = ctypes.c_double
    lib.pkmo_int8_to_f64.argtypes = [ctypes.c_int8]
    lib.pkmo_int4_to_f64.restype = ctypes.c_double
    lib.pkmo_int4_to_f64.argtypes = [ctypes.c_uint8]
    lib.pkmo_usage.restype = ctypes.c_int
    lib.pkmo_usage.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.pkmo_scores.restype = ctypes.c_int
    lib.pkmo_scores.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.pkmo_running_update.restype = ctypes.c_int
    lib.pkmo_running_update.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_double] + [ctypes.c_void_p] * 4
    lib.pkmo_select.restype = ctypes.c_int
    lib.pkmo_select.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    lib.pkmo_gather.restype = ctypes.c_int
    lib.pkmo_gather.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 3
    lib.pkmo_backward.restype = ctypes.c_int
    lib.pkmo_backward.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64] + [ctypes.c_void_p] * 8 + [ctypes.c_int]
    lib.pkmo_batch_stats.restype = ctypes.c_int
    lib.pkmo_batch_stats.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64] + [ctypes.c_void_p] * 3
    lib.pkmo_run_batch_stats.restype = ctypes.c_int
    lib.pkmo_run_batch_stats.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64, ctypes.c_void_p, ctypes.c_int] + \
        [ctypes.c_void_p] * 7
    lib.pkmo_backward_batch_stats.restype = ctypes.c_int
    lib.pkmo_backward_batch_stats.argtypes = [ctypes.POINTER(_Model), ctypes.c_int64] + [ctypes.c_void_p] * 10
    return lib


def compile_source(src, out):
    """gcc -O2 (no -ffast-math: every fp64 sum keeps its source order)."""
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread", src, "-o", out, "-lm"])
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


class Model:
    """The lookup's parameters as the oracle reads them (numpy, host memory).

    wq [H,D,D] f32 (row f = output feature f), mean/var/gamma/beta [H,D] f32,
    subkeys [H,2,n,D/2] f32, values [n*n,D] as f32 / uint16 (bf16 bits) /
    uint8 (E4M3 bits) / int8 codes, or [n*n,D/2] uint8 of packed int4 codes
    (even element in the low nibble); scale [n*n] f32 for E4M3, int8 and
    int4 tables.  values may be None when only the selection (idx, top, w,
    qhat) is wanted.
    """

    def __init__(self, wq, mean, var, gamma, beta, subkeys, values, scale, k, table, eps=1e-5):
        H, D, D2 = wq.shape
        assert D == D2 and D % 2 == 0
        n = subkeys.shape[2]
        assert subkeys.shape == (H, 2, n, D // 2)
        self.H, self.D, self.n, self.k, self.table, self.eps = H, D, n, int(k), table, float(eps)
        vt = np.dtype({"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "int8": np.int8, "int4": np.uint8}[table])
        self._keep = [
            _c(wq, np.float32), _c(mean, np.float32), _c(var, np.float32), _c(gamma, np.float32),
            _c(beta, np.float32), _c(subkeys, np.float32), None if values is None else _c(values, vt),
            None if scale is None else _c(scale, np.float32),
        ]
        self.has_values = values is not None
        assert not self.has_values or self._keep[6].shape == (n * n, D // 2 if table == "int4" else D)
        if table in SCALED and self.has_values:
            assert self._keep[7] is not None and self._keep[7].shape == (n * n,)
        k_ = self._keep
        self._s = _Model(D, H, n, int(k), VALUE_TYPES[table], 0, float(eps), *[_ptr(a) for a in k_])

    @classmethod
    def from_params(cls, p, k, table, eps=1e-5):
        return cls(p["wq"], p["mean"], p["var"], p["gamma"], p["beta"], p["subkeys"], p.get("values"),
                   p.get("scale"), k, table, eps)


def run(model, x, kk=None, want=("out", "idx", "top", "w"), nthreads=None, lib=None):
    """Run the oracle over every row of x [B,D] (f32).

    kk is the search depth (default: the model's k).  Returns a dict with the
    requested arrays among out [B,D] f64, idx [B,H,kk] i32, top [B,H,kk] f64,
    w [B,H,kk] f64, qhat [B,H,D] f64, ncand [B,H] i32.
    """
    lib = lib or _load()
    x = _c(x, np.float32)
    B = x.shape[0]
    assert x.shape == (B, model.D)
    kk = model.k if kk is None else int(kk)
    if "out" in want and not model.has_values:
        raise ValueError("the model holds no value table")
    H, D = model.H, model.D
    shapes = {"out": ((B, D), np.float64), "idx": ((B, H, kk), np.int32), "top": ((B, H, kk), np.float64),
              "w": ((B, H, kk), np.float64), "qhat": ((B, H, D), np.float64), "ncand": ((B, H), np.int32)}
    res = {name: np.empty(*shapes[name]) for name in want}
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = lib.pkmo_run(ctypes.byref(model._s), B, _ptr(x), kk, *[_ptr(res.get(nm)) for nm in
                      ("out", "idx", "top", "w", "qhat", "ncand")], int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return res


def bf16_to_f64(bits, lib=None):
    return (lib or _load()).pkmo_bf16_to_f64(int(bits))


def e4m3_to_f64(bits, lib=None):
    return (lib or _load()).pkmo_e4m3_to_f64(int(bits))


def int8_to_f64(code, lib=None):
    return (lib or _load()).pkmo_int8_to_f64(int(code))


def int4_to_f64(nibble, lib=None):
    return (lib or _load()).pkmo_int4_to_f64(int(nibble))


def scores(model, x, lib=None):
    """Steps 1-3: the half scores [B, H, 2, n] (fp64) of every token of
    x [B, D] (f32), the numbers run() ranks."""
    lib = lib or _load()
    x = _c(x, np.float32)
    B = x.shape[0]
    assert x.shape == (B, model.D)
    s = np.empty((B, model.H, 2, model.n), np.float64)
    if lib.pkmo_scores(ctypes.byref(model._s), B, _ptr(x), _ptr(s)) != 0:
        raise ValueError("oracle rejected its arguments")
    return s


def select(scores, k, lib=None):
    """Steps 4-6 from given half scores [..., 2, n] (any float dtype, read
    as fp64).  Returns idx, top, w, each [..., k]."""
    lib = lib or _load()
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    lead, n = scores.shape[:-2], scores.shape[-1]
    assert scores.shape[-2] == 2
    P = int(np.prod(lead)) if lead else 1
    idx = np.empty(lead + (k,), np.int32)
    top = np.empty(lead + (k,), np.float64)
    w = np.empty(lead + (k,), np.float64)
    if lib.pkmo_select(P, n, int(k), _ptr(scores), _ptr(idx), _ptr(top), _ptr(w)) != 0:
        raise ValueError("oracle rejected its arguments")
    return idx, top, w


def gather(model, rows, w, out=None, lib=None):
    """Step 7 from given rows [B, R] (int32) and weights [B, R] (read as
    fp64).  Returns out [B, D] fp64 (overwritten when given)."""
    lib = lib or _load()
    rows = _c(np.asarray(rows, np.int32), np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    B, R = rows.shape
    assert w.shape == (B, R)
    if B and (rows.min() < 0 or rows.max() >= model.n * model.n):
        raise ValueError("row index out of range")
    if out is None:
        out = np.empty((B, model.D), np.float64)
    assert out.dtype == np.float64 and out.shape == (B, model.D) and out.flags.c_contiguous
    if lib.pkmo_gather(ctypes.byref(model._s), B, R, _ptr(rows), _ptr(w), _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


GRADS = ("dx", "dwq", "dgamma", "dbeta", "dsub", "dval")


def backward(model, x, dout, want=GRADS, nthreads=None, lib=None):
    """Gradients of sum(dout * out) for x [B,D] (f32) and dout [B,D] (f32):
    dx [B,D], dwq [H,D,D], dgamma / dbeta [H,D], dsub [H,2,n,D/2] and dval
    [n*n,D] (w.r.t. the dequantised value rows), all fp64, the requested
    ones only.  The model must hold its value table."""
    lib = lib or _load()
    if not model.has_values:
        raise ValueError("the backward reads the value table")
    x = _c(x, np.float32)
    dout = _c(dout, np.float32)
    B = x.shape[0]
    assert x.shape == (B, model.D) and dout.shape == (B, model.D)
    H, D, n = model.H, model.D, model.n
    shapes = {"dx": (B, D), "dwq": (H, D, D), "dgamma": (H, D), "dbeta": (H, D), "dsub": (H, 2, n, D // 2),
              "dval": (n * n, D)}
    res = {name: np.empty(shapes[name]) for name in want}
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = lib.pkmo_backward(ctypes.byref(model._s), B, _ptr(x), _ptr(dout), *[_ptr(res.get(nm)) for nm in GRADS],
                           int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments" if rc == -1 else "oracle ran out of memory")
    return res


def batch_stats(model, x, lib=None):
    """Training-mode BN statistics of the batch x [B,D]: mean, biased var,
    each [H,D] fp64."""
    lib = lib or _load()
    x = _c(x, np.float32)
    mean = np.empty((model.H, model.D))
    var = np.empty((model.H, model.D))
    if lib.pkmo_batch_stats(ctypes.byref(model._s), x.shape[0], _ptr(x), _ptr(mean), _ptr(var)) != 0:
        raise ValueError("oracle rejected its arguments")
    return mean, var


def run_batch_stats(model, x, mean, var, kk=None, want=("out", "idx", "top", "w"), lib=None):
    """The lookup normalising with the given fp64 statistics [H,D], at
    search depth kk (default k).  out [B,D], idx / top / w [B,H,kk],
    qhat [B,H,D] as requested."""
    lib = lib or _load()
    x = _c(x, np.float32)
    B, H = x.shape[0], model.H
    kk = model.k if kk is None else int(kk)
    if "out" in want and not model.has_values:
        raise ValueError("the model holds no value table")
    shapes = {"out": ((B, model.D), np.float64), "idx": ((B, H, kk), np.int32), "top": ((B, H, kk), np.float64),
              "w": ((B, H, kk), np.float64), "qhat": ((B, H, model.D), np.float64)}
    res = {name: np.empty(*shapes[name]) for name in want}
    mean, var = _c(mean, np.float64), _c(var, np.float64)
    rc = lib.pkmo_run_batch_stats(ctypes.byref(model._s), B, _ptr(x), kk, _ptr(mean), _ptr(var),
                                  *[_ptr(res.get(nm)) for nm in ("out", "idx", "top", "w", "qhat")])
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return res


def backward_batch_stats(model, x, dout, mean, var, want=GRADS, lib=None):
    """Gradients of sum(dout * out) for the lookup with batch statistics
    (mean, var [H,D] fp64 of this batch): as backward()."""
    lib = lib or _load()
    if not model.has_values:
        raise ValueError("the backward reads the value table")
    x, dout = _c(x, np.float32), _c(dout, np.float32)
    B = x.shape[0]
    H, D, n = model.H, model.D, model.n
    shapes = {"dx": (B, D), "dwq": (H, D, D), "dgamma": (H, D), "dbeta": (H, D), "dsub": (H, 2, n, D // 2),
              "dval": (n * n, D)}
    res = {name: np.empty(shapes[name]) for name in want}
    mean, var = _c(mean, np.float64), _c(var, np.float64)
    rc = lib.pkmo_backward_batch_stats(ctypes.byref(model._s), B, _ptr(x), _ptr(dout), _ptr(mean), _ptr(var),
                                       *[_ptr(res.get(nm)) for nm in GRADS])
    if rc != 0:
        raise ValueError("oracle rejected its arguments" if rc == -1 else "oracle ran out of memory")
    return res


def running_update(rmean, rvar, mean, var, B, momentum=0.1, lib=None):
    """BatchNorm's running statistics after a batch of B tokens with
    statistics mean / var (biased): returns the updated (rmean, rvar), fp64
    copies of the given arrays."""
    lib = lib or _load()
    rm = np.array(rmean, np.float64, copy=True, order="C")
    rv = np.array(rvar, np.float64, copy=True, order="C")
    mean, var = _c(np.asarray(mean, np.float64), np.float64), _c(np.asarray(var, np.float64), np.float64)
    assert rm.shape == rv.shape == mean.shape == var.shape
    if lib.pkmo_running_update(rm.size, int(B), float(momentum), _ptr(mean), _ptr(var), _ptr(rm), _ptr(rv)) != 0:
        raise ValueError("oracle rejected its arguments")
    return rm, rv


def usage(rows, N, counts=None, lib=None):
    """Slot usage: counts [N] uint32 (+= when given) of the rows in rows."""
    lib = lib or _load()
    rows = _c(np.asarray(rows, np.int32).reshape(-1), np.int32)
    counts = np.zeros(N, np.uint32) if counts is None else counts
    assert counts.dtype == np.uint32 and counts.shape == (N,) and counts.flags.c_contiguous
    if lib.pkmo_usage(rows.size, _ptr(rows), N, _ptr(counts)) != 0:
        raise ValueError("oracle rejected its arguments")
    return counts