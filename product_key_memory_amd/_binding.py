"""ctypes binding of libpkm.so (the C ABI declared in include/pkm.h).

Argument marshalling only: torch tensors supply device memory and the current
stream, every step of the lookup runs in the library's HIP kernels.  There is
no fallback: if libpkm.so is missing or cannot be loaded, every call raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpkm.so")

PKM_OK, PKM_E_ARG, PKM_E_UNSUPPORTED, PKM_E_NOMEM, PKM_E_DEVICE = range(5)
VALUE_TYPES = {"f32": 0, "bf16": 1, "e4m3": 2, "int8": 3, "int4": 4}
SCALED = ("e4m3", "int8", "int4")  # tables with a per-row fp32 scale

# Every symbol include/pkm.h declares.
EXPORTS = (
    "pkm_config_check", "pkm_workspace_bytes", "pkm_create", "pkm_destroy", "pkm_forward", "pkm_query",
    "pkm_score", "pkm_select", "pkm_gather", "pkm_flat_workspace_bytes", "pkm_flat_search",
    "pkm_backward_workspace_bytes", "pkm_backward", "pkm_forward_batch_stats", "pkm_backward_batch_stats",
    "pkm_usage", "pkm_status_str", "pkm_last_error", "pkm_forward_noalloc", "pkm_select_gather",
    "pkm_forward_stage", "pkm_forward_train", "pkm_backward_with_q", "pkm_prepare", "pkm_half_scores",
)
PREPARE_FORMS = {"split": 0, "fold": 1}


class PkmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("dim", ctypes.c_int32), ("heads", ctypes.c_int32), ("n_keys", ctypes.c_int32), ("k", ctypes.c_int32),
        ("value_type", ctypes.c_int32), ("bn_eps", ctypes.c_float), ("max_batch", ctypes.c_int64),
    ]


class ParamsStruct(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("wq", "bn_mean", "bn_var", "bn_gamma", "bn_beta", "subkeys", "values", "value_scale")]


_lib = None


def load_library(path=LIB_PATH):
    """Load libpkm.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m product_key_memory_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    cfg_p = ctypes.POINTER(Config)
    par_p = ctypes.POINTER(ParamsStruct)
    sigs = {
        "pkm_config_check": (ctypes.c_int, [cfg_p]),
        "pkm_workspace_bytes": (ctypes.c_int, [cfg_p, ctypes.POINTER(ctypes.c_size_t)]),
        "pkm_create": (ctypes.c_int, [cfg_p, ctypes.POINTER(vp)]),
        "pkm_destroy": (None, [vp]),
        "pkm_forward": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp]),
        "pkm_forward_noalloc": (ctypes.c_int, [cfg_p, par_p, i64, vp, vp, vp, vp, vp]),
        "pkm_forward_stage": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, ctypes.c_int, vp]),
        "pkm_query": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp]),
        "pkm_score": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp]),
        "pkm_select": (ctypes.c_int, [vp, i64, vp, vp, vp, vp]),
        "pkm_gather": (ctypes.c_int, [vp, par_p, i64, i32, vp, vp, vp, vp]),
        "pkm_select_gather": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp]),
        "pkm_flat_workspace_bytes": (ctypes.c_int, [cfg_p, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "pkm_flat_search": (ctypes.c_int, [vp, par_p, i64, vp, vp, ctypes.c_size_t, vp, vp, vp]),
        "pkm_backward_workspace_bytes": (ctypes.c_int, [cfg_p, ctypes.POINTER(ctypes.c_size_t)]),
        "pkm_usage": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
        "pkm_forward_batch_stats": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp]),
        "pkm_backward_batch_stats": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp, vp,
                                                    ctypes.POINTER(GradsStruct), vp, ctypes.c_size_t, vp]),
        "pkm_backward": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, ctypes.POINTER(GradsStruct), vp,
                                        ctypes.c_size_t, vp]),
        "pkm_forward_train": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp, vp]),
        "pkm_prepare": (ctypes.c_int, [vp, par_p, ctypes.c_int, vp]),
        "pkm_half_scores": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp]),
        "pkm_backward_with_q": (ctypes.c_int, [vp, par_p, i64, vp, vp, vp, vp, vp, ctypes.POINTER(GradsStruct), vp,
                                               ctypes.c_size_t, vp]),
        "pkm_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "pkm_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status):
    return load_library().pkm_status_str(int(status)).decode()


def last_error():
    return load_library().pkm_last_error().decode()


def _check(status):
    if status != PKM_OK:
        raise PkmError(status, last_error())


def make_config(dim, heads, n_keys, k, value_type="bf16", bn_eps=1e-5, max_batch=16384):
    vt = VALUE_TYPES[value_type] if isinstance(value_type, str) else int(value_type)
    return Config(int(dim), int(heads), int(n_keys), int(k), vt, float(bn_eps), int(max_batch))


def config_check(cfg):
    """PKM status code for a Config (touches no device)."""
    return load_library().pkm_config_check(ctypes.byref(cfg))


def workspace_bytes(cfg):
    out = ctypes.c_size_t(0)
    _check(load_library().pkm_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def _torch():
    import torch

    return torch


def _stream_handle(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Accepted storage dtypes of the value table (bit patterns are what matter).
_DT = {"f32": ("float32",), "bf16": ("bfloat16", "int16", "uint16"), "e4m3": ("float8_e4m3fn", "uint8", "int8"),
       "int8": ("int8", "uint8"), "int4": ("uint8", "int8")}


def _expect(t, name, shape, dtype, device=None):
    """Shape / dtype / contiguity / device check of one tensor argument."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    dtypes = (dtype,) if isinstance(dtype, str) else dtype
    if str(t.dtype) not in ["torch." + d for d in dtypes]:
        raise ValueError(f"{name}: expected one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on {device or 'the GPU'}, got {t.device}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


GRAD_NAMES = ("dx", "dwq", "dbn_gamma", "dbn_beta", "dsubkeys", "dvalues", "dvalues_rows", "dvalues_sparse",
              "dvalues_count")
SPARSE_VALUE_GRADS = ("dvalues_rows", "dvalues_sparse", "dvalues_count")


class GradsStruct(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in GRAD_NAMES]


class Params:
    """Device tensors of one lookup's parameters (kept alive by this object).

    wq [H,D,D] f32; bn_mean/bn_var/bn_gamma/bn_beta [H,D] f32;
    subkeys [H,2,n,D/2] f32; values [N,D] float32 / bfloat16 / float8_e4m3fn
    (or an integer type of the same width holding the bits); value_scale [N]
    f32 for E4M3 tables (else None)."""

    def __init__(self, wq, bn_mean, bn_var, bn_gamma, bn_beta, subkeys, values, value_scale=None):
        self.tensors = dict(wq=wq, bn_mean=bn_mean, bn_var=bn_var, bn_gamma=bn_gamma, bn_beta=bn_beta,
                            subkeys=subkeys, values=values, value_scale=value_scale)
        self.struct = ParamsStruct(*[None if t is None else t.data_ptr() for t in self.tensors.values()])

    def __getitem__(self, name):
        return self.tensors[name]


def forward_noalloc(cfg, params, x, out, idx=None, weights=None, stream=None):
    """The whole lookup through pkm_forward_noalloc: no context, and nothing
    allocated by the library or here -- out (and idx / weights, if wanted)
    are the caller's tensors.  cfg: a Config (its max_batch caps the chunk).
    Calls on one GPU share the library's scratch array: do not overlap them."""
    B = x.shape[0]
    H, D, k = cfg.heads, cfg.dim, cfg.k
    dev = params["wq"].device
    _expect(x, "x", (B, D), "float32", dev)
    _expect(out, "out", (B, D), "float32", dev)
    for t, name, dt in ((idx, "idx", "int32"), (weights, "weights", "float32")):
        if t is not None:
            _expect(t, name, (B, H, k), dt, dev)
    _check(load_library().pkm_forward_noalloc(ctypes.byref(cfg), ctypes.byref(params.struct), B, _ptr(x), _ptr(out),
                                              _ptr(idx), _ptr(weights), _stream_handle(stream)))
    return out, idx, weights


class Memory:
    """A library context for one (D, H, n_keys, k, table type) on the current
    device.  Calls enqueue on the given stream (default: torch's current
    stream) and return without synchronising."""

    def __init__(self, dim, heads, n_keys, k, value_type="bf16", bn_eps=1e-5, max_batch=16384):
        self.lib = load_library()
        self.cfg = make_config(dim, heads, n_keys, k, value_type, bn_eps, max_batch)
        self.dim, self.heads, self.n_keys, self.k = int(dim), int(heads), int(n_keys), int(k)
        self.value_type = value_type
        handle = ctypes.c_void_p()
        _check(self.lib.pkm_create(ctypes.byref(self.cfg), ctypes.byref(handle)))
        self._ctx = handle

    def close(self):
        if getattr(self, "_ctx", None):
            self.lib.pkm_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ------------------------------------------------------------- helpers
    def _new(self, shape, dtype, like):
        torch = _torch()
        return torch.empty(shape, dtype=dtype, device=like.device)

    def check_params(self, params, parts=("query", "subkeys", "values")):
        """Checks params against this context's shapes before any launch."""
        D, H, n = self.dim, self.heads, self.n_keys
        t = params.tensors
        dev = t["wq"].device if t.get("wq") is not None else None
        if "query" in parts or "query_affine" in parts:
            # query_affine: batch statistics replace the running mean / var
            _expect(t["wq"], "wq", (H, D, D), "float32")
            names = ("bn_gamma", "bn_beta") if "query_affine" in parts else ("bn_mean", "bn_var", "bn_gamma", "bn_beta")
            for name in names:
                _expect(t[name], name, (H, D), "float32", dev)
        if "subkeys" in parts:
            _expect(t["subkeys"], "subkeys", (H, 2, n, D // 2), "float32", dev)
        if "values" in parts:
            vt = self.value_type
            _expect(t["values"], "values", (n * n, D // 2 if vt == "int4" else D), _DT[vt], dev)
            if vt in SCALED:
                _expect(t["value_scale"], "value_scale", (n * n,), "float32", t["values"].device)

    def prepare(self, params, form="split", stream=None):
        """pkm_prepare: keep the parameters that are the same for every call
        in the form the contractions read, for forward calls with these same
        arrays (their contents must not change until prepare is called
        again).  form "split": Wq and the subkeys as fp16 pieces (bit for bit
        the unprepared results); "fold": projection, batch-norm and subkeys
        folded into one matrix per half of a head (n_keys <= D; fp32-accurate,
        not bitwise).  None drops the prepared form."""
        if params is None:
            _check(self.lib.pkm_prepare(self._ctx, None, 0, _stream_handle(stream)))
            return
        self.check_params(params, parts=("query", "subkeys"))
        _check(self.lib.pkm_prepare(self._ctx, ctypes.byref(params.struct), PREPARE_FORMS[form],
                                    _stream_handle(stream)))

    def half_scores(self, params, x, scores=None, stream=None):
        """pkm_half_scores: steps a1-a3 from x, scores [B, H, 2, n] f32 (through
        the folded form when one was prepared for these arrays)."""
        torch = _torch()
        B = x.shape[0]
        self.check_params(params, ("query", "subkeys"))
        _expect(x, "x", (B, self.dim), "float32", params["wq"].device)
        shape = (B, self.heads, 2, self.n_keys)
        scores = self._new(shape, torch.float32, x) if scores is None else scores
        _expect(scores, "scores", shape, "float32", x.device)
        _check(self.lib.pkm_half_scores(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(scores),
                                        _stream_handle(stream)))
        return scores

    def forward(self, params, x, out=None, idx=None, weights=None, stream=None, keep_selection=True):
        """The whole lookup.  Returns (out [B,D] f32, idx [B,H,k] i32,
        weights [B,H,k] f32); idx/weights are None when keep_selection is
        False and none were given."""
        torch = _torch()
        B = x.shape[0]
        self.check_params(params)
        _expect(x, "x", (B, self.dim), "float32", params["wq"].device)
        out = self._new((B, self.dim), torch.float32, x) if out is None else out
        _expect(out, "out", (B, self.dim), "float32", x.device)
        if keep_selection:
            idx = self._new((B, self.heads, self.k), torch.int32, x) if idx is None else idx
            weights = self._new((B, self.heads, self.k), torch.float32, x) if weights is None else weights
        for t, name, dt in ((idx, "idx", "int32"), (weights, "weights", "float32")):
            if t is not None:
                _expect(t, name, (B, self.heads, self.k), dt, x.device)
        _check(self.lib.pkm_forward(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(out), _ptr(idx),
                                    _ptr(weights), _stream_handle(stream)))
        return out, idx, weights

    def forward_train(self, params, x, out=None, idx=None, weights=None, q=None, stream=None):
        """forward() that also writes the projection before BN, q [B,H,D]
        f32, for backward(..., q=q).  Returns (out, idx, weights, q)."""
        torch = _torch()
        B = x.shape[0]
        self.check_params(params)
        _expect(x, "x", (B, self.dim), "float32", params["wq"].device)
        out = self._new((B, self.dim), torch.float32, x) if out is None else out
        idx = self._new((B, self.heads, self.k), torch.int32, x) if idx is None else idx
        weights = self._new((B, self.heads, self.k), torch.float32, x) if weights is None else weights
        q = self._new((B, self.heads, self.dim), torch.float32, x) if q is None else q
        _expect(out, "out", (B, self.dim), "float32", x.device)
        _expect(idx, "idx", (B, self.heads, self.k), "int32", x.device)
        _expect(weights, "weights", (B, self.heads, self.k), "float32", x.device)
        _expect(q, "q", (B, self.heads, self.dim), "float32", x.device)
        _check(self.lib.pkm_forward_train(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(out), _ptr(idx),
                                          _ptr(weights), _ptr(q), _stream_handle(stream)))
        return out, idx, weights, q

    def forward_stage(self, params, x, stage, out, idx=None, weights=None, stream=None):
        """One stage (0-3) of the forward's launches for B <= max_batch
        tokens; stages 0..3 in order equal forward().  out / idx / weights
        as forward() takes them (the caller's tensors)."""
        B = x.shape[0]
        self.check_params(params)
        _expect(x, "x", (B, self.dim), "float32", params["wq"].device)
        _expect(out, "out", (B, self.dim), "float32", x.device)
        for t, name, dt in ((idx, "idx", "int32"), (weights, "weights", "float32")):
            if t is not None:
                _expect(t, name, (B, self.heads, self.k), dt, x.device)
        _check(self.lib.pkm_forward_stage(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(out), _ptr(idx),
                                          _ptr(weights), int(stage), _stream_handle(stream)))
        return out

    def query(self, params, x, qhat=None, stream=None):
        torch = _torch()
        self.check_params(params, ("query",))
        _expect(x, "x", (x.shape[0], self.dim), "float32", params["wq"].device)
        qhat = self._new((x.shape[0], self.heads, self.dim), torch.float32, x) if qhat is None else qhat
        _expect(qhat, "qhat", (x.shape[0], self.heads, self.dim), "float32", x.device)
        _check(self.lib.pkm_query(self._ctx, ctypes.byref(params.struct), x.shape[0], _ptr(x), _ptr(qhat),
                                  _stream_handle(stream)))
        return qhat

    def score(self, params, qhat, scores=None, stream=None):
        torch = _torch()
        B = qhat.shape[0]
        self.check_params(params, ("subkeys",))
        _expect(qhat, "qhat", (B, self.heads, self.dim), "float32", params["subkeys"].device)
        scores = self._new((B, self.heads, 2, self.n_keys), torch.float32, qhat) if scores is None else scores
        _expect(scores, "scores", (B, self.heads, 2, self.n_keys), "float32", qhat.device)
        _check(self.lib.pkm_score(self._ctx, ctypes.byref(params.struct), B, _ptr(qhat), _ptr(scores),
                                  _stream_handle(stream)))
        return scores

    def select(self, scores, idx=None, weights=None, stream=None):
        torch = _torch()
        B = scores.shape[0]
        _expect(scores, "scores", (B, self.heads, 2, self.n_keys), "float32")
        idx = self._new((B, self.heads, self.k), torch.int32, scores) if idx is None else idx
        weights = self._new((B, self.heads, self.k), torch.float32, scores) if weights is None else weights
        _expect(idx, "idx", (B, self.heads, self.k), "int32", scores.device)
        _expect(weights, "weights", (B, self.heads, self.k), "float32", scores.device)
        _check(self.lib.pkm_select(self._ctx, B, _ptr(scores), _ptr(idx), _ptr(weights), _stream_handle(stream)))
        return idx, weights

    def gather(self, params, idx, weights, out=None, stream=None):
        """idx / weights [B, R] (or [B, H, k]); out [B, D] f32."""
        torch = _torch()
        B = idx.shape[0]
        R = idx.numel() // max(B, 1)
        self.check_params(params, ("values",))
        _expect(idx, "idx", tuple(idx.shape), "int32", params["values"].device)
        _expect(weights, "weights", tuple(idx.shape), "float32", idx.device)
        if B and idx.numel() != B * R:
            raise ValueError("idx must hold the same number of rows for every token")
        out = self._new((B, self.dim), torch.float32, idx) if out is None else out
        _expect(out, "out", (B, self.dim), "float32", idx.device)
        _check(self.lib.pkm_gather(self._ctx, ctypes.byref(params.struct), B, R, _ptr(idx), _ptr(weights),
                                   _ptr(out), _stream_handle(stream)))
        return out

    def select_gather(self, params, scores, out=None, idx=None, weights=None, stream=None):
        """a4-a7 from scores [B, H, 2, n]: returns (out [B, D] f32, idx,
        weights); idx / weights ([B, H, k]) are filled when given (both or
        neither), else None."""
        torch = _torch()
        B = scores.shape[0]
        self.check_params(params, ("values",))
        _expect(scores, "scores", (B, self.heads, 2, self.n_keys), "float32", params["values"].device)
        out = self._new((B, self.dim), torch.float32, scores) if out is None else out
        _expect(out, "out", (B, self.dim), "float32", scores.device)
        if (idx is None) != (weights is None):
            raise ValueError("idx and weights go together")
        if idx is not None:
            _expect(idx, "idx", (B, self.heads, self.k), "int32", scores.device)
            _expect(weights, "weights", (B, self.heads, self.k), "float32", scores.device)
        _check(self.lib.pkm_select_gather(self._ctx, ctypes.byref(params.struct), B, _ptr(scores), _ptr(idx),
                                          _ptr(weights), _ptr(out), _stream_handle(stream)))
        return out, idx, weights

    def usage(self, idx, counts=None, stream=None):
        """Slot usage: counts [n_keys^2] uint32 (int32 accepted) += how often
        each row occurs in idx [B, ...] (int32).  counts None: fresh zeros."""
        torch = _torch()
        B = idx.shape[0]
        R = idx.numel() // max(B, 1)
        N = self.n_keys * self.n_keys
        _expect(idx, "idx", tuple(idx.shape), "int32")
        if counts is None:
            counts = torch.zeros(N, dtype=torch.int32, device=idx.device)
        _expect(counts, "counts", (N,), ("int32", "uint32"), idx.device)
        _check(self.lib.pkm_usage(self._ctx, B, max(R, 1), _ptr(idx), _ptr(counts), _stream_handle(stream)))
        return counts

    def backward_workspace_bytes(self):
        n = ctypes.c_size_t()
        _check(self.lib.pkm_backward_workspace_bytes(ctypes.byref(self.cfg), ctypes.byref(n)))
        return n.value

    def forward_batch_stats(self, params, x, out=None, idx=None, weights=None, running=None, momentum=0.1,
                            stream=None):
        """The lookup with training-mode BN (statistics of this batch).
        running: (mean, var) [H, D] f32 tensors updated in place, or None.
        Returns (out, idx, weights, batch_mean, batch_var)."""
        torch = _torch()
        B = x.shape[0]
        H, D, k = self.heads, self.dim, self.k
        self.check_params(params, ("query_affine", "subkeys", "values"))
        dev = params["subkeys"].device
        _expect(x, "x", (B, D), "float32", dev)
        out = self._new((B, D), torch.float32, x) if out is None else out
        idx = self._new((B, H, k), torch.int32, x) if idx is None else idx
        weights = self._new((B, H, k), torch.float32, x) if weights is None else weights
        mean = self._new((H, D), torch.float32, x)
        var = self._new((H, D), torch.float32, x)
        _expect(out, "out", (B, D), "float32", dev)
        _expect(idx, "idx", (B, H, k), "int32", dev)
        _expect(weights, "weights", (B, H, k), "float32", dev)
        rm, rv = running if running is not None else (None, None)
        for t, name in ((rm, "running_mean"), (rv, "running_var")):
            if t is not None:
                _expect(t, name, (H, D), "float32", dev)
        _check(self.lib.pkm_forward_batch_stats(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(out),
                                                _ptr(idx), _ptr(weights), _ptr(mean), _ptr(var), _ptr(rm), _ptr(rv),
                                                float(momentum), _stream_handle(stream)))
        return out, idx, weights, mean, var

    def backward(self, params, x, idx, weights, dout, grads=None, workspace=None, stream=None, batch_stats=None,
                 sparse_values=False, q=None):
        """Gradients of a loss given dout = dL/dout [B, D] for the winners
        (idx, weights) a forward call returned.  grads: dict name -> tensor
        (parameter gradients are added to, dx is overwritten; a missing name
        is skipped), or None for freshly zeroed buffers of every gradient.
        sparse_values: with grads None, the value gradient in its sparse
        form instead of dvalues -- dvalues_rows [cap] int32, dvalues_sparse
        [cap, D] f32 and dvalues_count [1] int64 with cap = min(n^2, B*H*k);
        the first dvalues_count entries hold the touched rows in increasing
        order and their gradients.  batch_stats: (mean, var) from
        forward_batch_stats for the training-mode BN backward, or None
        (running statistics).  q: the projection before BN from
        forward_train, used instead of computing it again (running
        statistics only).  Returns the dict."""
        torch = _torch()
        B = x.shape[0]
        D, H, n, k = self.dim, self.heads, self.n_keys, self.k
        self.check_params(params, ("query_affine" if batch_stats is not None else "query", "subkeys", "values"))
        dev = params["wq"].device
        _expect(x, "x", (B, D), "float32", dev)
        _expect(dout, "dout", (B, D), "float32", dev)
        _expect(idx, "idx", (B, H, k), "int32", dev)
        _expect(weights, "weights", (B, H, k), "float32", dev)
        cap = min(n * n, B * H * k)
        shapes = {"dx": (B, D), "dwq": (H, D, D), "dbn_gamma": (H, D), "dbn_beta": (H, D),
                  "dsubkeys": (H, 2, n, D // 2), "dvalues": (n * n, D), "dvalues_rows": (cap,),
                  "dvalues_sparse": (cap, D), "dvalues_count": (1,)}
        dtypes = {"dvalues_rows": "int32", "dvalues_count": "int64"}
        if grads is None:
            skip = ("dvalues",) if sparse_values else SPARSE_VALUE_GRADS
            grads = {name: torch.zeros(shape, dtype=getattr(torch, dtypes.get(name, "float32")), device=dev)
                     for name, shape in shapes.items() if name not in skip}
        for name, t in grads.items():
            if name not in shapes:
                raise ValueError(f"unknown gradient {name}")
            _expect(t, name, shapes[name], dtypes.get(name, "float32"), dev)
        need = self.backward_workspace_bytes()
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _expect(workspace, "workspace", (workspace.numel(),), "uint8", dev)
        gs = GradsStruct(*[None if grads.get(nm) is None else grads[nm].data_ptr() for nm in GRAD_NAMES])
        if q is not None:
            if batch_stats is not None:
                raise ValueError("q (from forward_train) goes with running statistics only")
            _expect(q, "q", (B, H, D), "float32", dev)
            _check(self.lib.pkm_backward_with_q(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(q),
                                                _ptr(idx), _ptr(weights), _ptr(dout), ctypes.byref(gs),
                                                _ptr(workspace), workspace.numel(), _stream_handle(stream)))
        elif batch_stats is None:
            _check(self.lib.pkm_backward(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(idx),
                                         _ptr(weights), _ptr(dout), ctypes.byref(gs), _ptr(workspace),
                                         workspace.numel(), _stream_handle(stream)))
        else:
            mean, var = batch_stats
            _expect(mean, "batch_mean", (H, D), "float32", dev)
            _expect(var, "batch_var", (H, D), "float32", dev)
            _check(self.lib.pkm_backward_batch_stats(self._ctx, ctypes.byref(params.struct), B, _ptr(x), _ptr(idx),
                                                     _ptr(weights), _ptr(dout), _ptr(mean), _ptr(var),
                                                     ctypes.byref(gs), _ptr(workspace), workspace.numel(),
                                                     _stream_handle(stream)))
        return grads

    def flat_workspace_bytes(self, B):
        n = ctypes.c_size_t()
        _check(self.lib.pkm_flat_workspace_bytes(ctypes.byref(self.cfg), int(B), ctypes.byref(n)))
        return n.value

    def flat_search(self, params, qhat, idx=None, top=None, workspace=None, stream=None):
        """Brute-force top-k over all n_keys^2 concatenated keys from qhat
        [B, H, D]: (idx [B, H, k] int32, top [B, H, k] f32).  workspace: a
        uint8 device tensor of at least flat_workspace_bytes(B) bytes, or
        None to allocate one."""
        torch = _torch()
        B = qhat.shape[0]
        self.check_params(params, ("subkeys",))
        _expect(qhat, "qhat", (B, self.heads, self.dim), "float32", params["subkeys"].device)
        need = self.flat_workspace_bytes(B)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qhat.device)
        _expect(workspace, "workspace", (workspace.numel(),), "uint8", qhat.device)
        idx = self._new((B, self.heads, self.k), torch.int32, qhat) if idx is None else idx
        top = self._new((B, self.heads, self.k), torch.float32, qhat) if top is None else top
        _expect(idx, "idx", (B, self.heads, self.k), "int32", qhat.device)
        _expect(top, "top", (B, self.heads, self.k), "float32", qhat.device)
        _check(self.lib.pkm_flat_search(self._ctx, ctypes.byref(params.struct), B, _ptr(qhat), _ptr(workspace),
                                        workspace.numel(), _ptr(idx), _ptr(top), _stream_handle(stream)))
        return idx, top
