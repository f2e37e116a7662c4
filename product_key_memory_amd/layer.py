"""A torch.nn.Module and autograd function over the library's lookup.

The product-key memory layer ("Product-Key Memory", §Factorising the key
space; batch normalisation of the query as in §Keeping the memory in use)
with its parameters held as torch tensors, so that a torch training loop can
use it: the forward and backward both run in libpkm.so's kernels (through
Memory.forward / forward_train / forward_batch_stats and Memory.backward);
this module only allocates the gradient buffers and hands them to autograd.

- Training mode (module.train()): batch-norm with the batch's statistics,
  the running mean and variance updated in place (BatchNorm1d's rule with
  `momentum`); the backward is the coupled batch-norm backward.  Needs
  2 <= tokens <= max_batch.
- Eval mode: batch-norm with the running statistics; with gradients wanted,
  the forward keeps the projection before batch-norm so that the backward
  need not compute it again.
- The value table trains when it is fp32 or bf16 (its gradient is taken in
  fp32 and cast to the table's type by autograd).  With
  sparse_values=True the table's gradient is a sparse COO tensor of the
  touched rows only (the rows some winner selected; the others get no
  gradient), for optimisers that take sparse gradients.  E4M3, int8 and
  int4 tables (with their row scales) are buffers: looked up, not trained.

- prepare_weights=True (or "split"): the library keeps wq and the subkeys
  in the form its contractions read (pkm_prepare), so each eval-mode
  forward skips converting them; same results bit for bit.
  prepare_weights="fold": eval-mode forwards without gradients run the
  folded lookup (projection, batch-norm with the running statistics and
  subkeys folded into one key matrix per half of a head; n_keys <= dim),
  fp32-accurate rather than bitwise.  Either copy is made again whenever a
  parameter it was made from has changed in place since (torch's version
  counters: optimiser steps, load_state_dict, copy_ under no_grad; a
  training-mode forward, which moves the running statistics).  Changes that
  bypass the counters (writing through .data) need refresh_prepared().

There is no CPU path: the module lives on a GPU, and every call raises if
libpkm.so cannot be loaded.  Calls of one module must not overlap on
different streams (they share the backward's workspace).
"""
import math

import torch

from ._binding import SCALED, Memory, Params

_TABLE_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn, "int8": torch.int8,
                 "int4": torch.uint8}


class _Lookup(torch.autograd.Function):
    """out = lookup(x) with gradients for x, Wq, gamma, beta, the subkeys and
    (trainable tables) the values."""

    @staticmethod
    def forward(ctx, layer, x, wq, bn_gamma, bn_beta, subkeys, values):
        mem, P = layer._memory(), layer._params()
        if layer.training:
            out, idx, w, mean, var = mem.forward_batch_stats(
                P, x, running=(layer.running_mean, layer.running_var), momentum=layer.momentum)
            layer._prep_key = None  # the running statistics moved (behind torch's counters)
            ctx.save_for_backward(x, idx, w, mean, var)
        else:
            layer._sync_prepared(P)
            out, idx, w, q = mem.forward_train(P, x)
            ctx.save_for_backward(x, idx, w, q)
        ctx.layer, ctx.batch_stats = layer, layer.training
        ctx.mark_non_differentiable(idx, w)
        return out, idx, w

    @staticmethod
    def backward(ctx, dout, _didx, _dw):
        layer = ctx.layer
        mem, P = layer._memory(), layer._params()
        x = ctx.saved_tensors[0]
        B, D, H, n = x.shape[0], layer.dim, layer.heads, layer.n_keys
        need = ctx.needs_input_grad  # (layer, x, wq, gamma, beta, subkeys, values)
        dev = x.device
        zeros = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)  # noqa: E731
        grads = {}
        if need[1]:
            grads["dx"] = torch.empty((B, D), dtype=torch.float32, device=dev)  # overwritten
        if need[2]:
            grads["dwq"] = zeros(H, D, D)  # the library adds into these
        if need[3] or need[4]:
            grads["dbn_gamma"], grads["dbn_beta"] = zeros(H, D), zeros(H, D)
        if need[5]:
            grads["dsubkeys"] = zeros(H, 2, n, D // 2)
        sparse = need[6] and layer.sparse_values
        if need[6]:
            if sparse:
                cap = min(n * n, B * H * layer.k)
                grads["dvalues_rows"] = torch.empty(cap, dtype=torch.int32, device=dev)
                grads["dvalues_sparse"] = torch.empty((cap, D), dtype=torch.float32, device=dev)
                grads["dvalues_count"] = torch.zeros(1, dtype=torch.int64, device=dev)
            else:
                grads["dvalues"] = zeros(n * n, D)
        if grads:
            dout = dout.contiguous().float()
            if ctx.batch_stats:
                _, idx, w, mean, var = ctx.saved_tensors
                mem.backward(P, x, idx, w, dout, grads, workspace=layer._workspace(), batch_stats=(mean, var))
            else:
                _, idx, w, q = ctx.saved_tensors
                mem.backward(P, x, idx, w, dout, grads, workspace=layer._workspace(), q=q)
        dval = None
        if need[6]:
            if sparse:
                U = int(grads["dvalues_count"].item())
                rows = grads["dvalues_rows"][:U].long().unsqueeze(0)
                dval = torch.sparse_coo_tensor(rows, grads["dvalues_sparse"][:U], (n * n, D), is_coalesced=True)
            else:
                dval = grads["dvalues"]
        return (None, grads.get("dx"), grads.get("dwq"), grads.get("dbn_gamma") if need[3] else None,
                grads.get("dbn_beta") if need[4] else None, grads.get("dsubkeys"), dval)


class ProductKeyMemory(torch.nn.Module):
    """Product-key memory layer: x [..., dim] fp32 -> out [..., dim] fp32,
    the sum over `heads` heads of a softmax-weighted sum of the k value rows
    whose product keys score best against the head's batch-normalised
    query.

    Parameters (shapes of include/pkm.h): wq [heads, dim, dim] (row f of
    wq[h] is output feature f), bn_gamma / bn_beta [heads, dim], subkeys
    [heads, 2, n_keys, dim/2], values [n_keys^2, dim] (a Parameter for fp32
    and bf16 tables, else a buffer; int4 tables hold [n_keys^2, dim/2]
    bytes, two codes per byte) and, for the E4M3 / int8 / int4 tables, the
    row scales value_scale [n_keys^2] (a buffer).  Buffers running_mean,
    running_var [heads, dim].

    Initialisation (this module's own choice; the pages fix none): wq
    ~ N(0, 1/dim), gamma = 1, beta = 0, running statistics 0 and 1,
    subkeys ~ N(0, 1), fp32 / bf16 values ~ N(0, 1/dim); the quantised
    tables start at zero (load them with load_table).

    forward(x) returns out; forward(x, return_selection=True) also returns
    the winners idx [..., heads, k] int32 and their weights [..., heads, k].
    """

    def __init__(self, dim, heads=4, n_keys=1024, k=32, value_type="bf16", bn_eps=1e-5, momentum=0.1,
                 max_batch=16384, sparse_values=False, prepare_weights=False, device="cuda"):
        super().__init__()
        device = torch.device(device)
        if device.type != "cuda":
            raise ValueError(f"ProductKeyMemory runs on a GPU (got device {device}); there is no CPU path")
        if value_type not in _TABLE_DTYPES:
            raise ValueError(f"value_type must be one of {sorted(_TABLE_DTYPES)}")
        self.dim, self.heads, self.n_keys, self.k = int(dim), int(heads), int(n_keys), int(k)
        self.value_type, self.bn_eps, self.momentum = value_type, float(bn_eps), float(momentum)
        self.max_batch, self.sparse_values = int(max_batch), bool(sparse_values)
        if prepare_weights not in (False, True, "split", "fold"):
            raise ValueError('prepare_weights must be False, True, "split" or "fold"')
        self.prepare_weights = "split" if prepare_weights is True else prepare_weights
        self._prep_key = None
        D, H, n = self.dim, self.heads, self.n_keys
        f32 = dict(dtype=torch.float32, device=device)
        self.wq = torch.nn.Parameter(torch.empty(H, D, D, **f32))
        self.bn_gamma = torch.nn.Parameter(torch.empty(H, D, **f32))
        self.bn_beta = torch.nn.Parameter(torch.empty(H, D, **f32))
        self.subkeys = torch.nn.Parameter(torch.empty(H, 2, n, D // 2, **f32))
        self.register_buffer("running_mean", torch.zeros(H, D, **f32))
        self.register_buffer("running_var", torch.ones(H, D, **f32))
        vshape = (n * n, D // 2 if value_type == "int4" else D)
        values = torch.empty(vshape, dtype=_TABLE_DTYPES[value_type], device=device)
        if value_type in ("f32", "bf16"):
            self.values = torch.nn.Parameter(values)
            self.value_scale = None
        else:
            self.register_buffer("values", values)
            self.register_buffer("value_scale", torch.ones(n * n, **f32))
        self._mem = self._ws = None
        self._mem_device = None
        self.reset_parameters()

    @torch.no_grad()
    def reset_parameters(self, generator=None):
        """Re-draws the parameters (generator: a torch.Generator on the
        module's device, or None) and resets the running statistics."""
        D = self.dim
        self.wq.normal_(0.0, 1.0 / math.sqrt(D), generator=generator)
        self.bn_gamma.fill_(1.0)
        self.bn_beta.zero_()
        self.running_mean.zero_()
        self.running_var.fill_(1.0)
        self.subkeys.normal_(0.0, 1.0, generator=generator)
        if self.value_type in ("f32", "bf16"):
            self.values.normal_(0.0, 1.0 / math.sqrt(D), generator=generator)
        else:
            self.values.zero_()

    @torch.no_grad()
    def load_table(self, values, value_scale=None):
        """Copies a table (and, for the scaled types, its row scales) in."""
        self.values.copy_(values)
        if self.value_type in SCALED:
            if value_scale is None:
                raise ValueError(f"a {self.value_type} table needs value_scale")
            self.value_scale.copy_(value_scale)

    # ----------------------------------------------------------- internals
    def _memory(self):
        dev = self.wq.device
        if self._mem is None or self._mem_device != dev:
            with torch.cuda.device(dev):
                self._mem = Memory(self.dim, self.heads, self.n_keys, self.k, self.value_type, self.bn_eps,
                                   self.max_batch)
            self._mem_device, self._ws, self._prep_key = dev, None, None
        return self._mem

    def _sync_prepared(self, P):
        """With prepare_weights: prepares again when an array the prepared
        form was made from changed since the last time (pointer or version
        counter)."""
        if not self.prepare_weights:
            return
        arrays = (self.wq, self.subkeys)
        if self.prepare_weights == "fold":
            arrays += (self.running_mean, self.running_var, self.bn_gamma, self.bn_beta)
        key = tuple((t.data_ptr(), t._version) for t in arrays)
        if key != self._prep_key:
            self._memory().prepare(P, self.prepare_weights)
            self._prep_key = key

    def refresh_prepared(self):
        """Prepares wq and the subkeys again now (after changes that torch's
        version counters do not see, such as writes through .data)."""
        self._prep_key = None
        self._sync_prepared(self._params())

    def _workspace(self):
        if self._ws is None:
            self._ws = torch.empty(max(self._memory().backward_workspace_bytes(), 1), dtype=torch.uint8,
                                   device=self.wq.device)
        return self._ws

    def _params(self):
        t = lambda p: p.detach()  # noqa: E731  (the library reads the storage)
        return Params(t(self.wq), self.running_mean, self.running_var, t(self.bn_gamma), t(self.bn_beta),
                      t(self.subkeys), t(self.values), self.value_scale)

    def forward(self, x, return_selection=False):
        lead = x.shape[:-1]
        if x.shape[-1] != self.dim:
            raise ValueError(f"x: last dimension must be {self.dim}, got {x.shape[-1]}")
        x2 = x.reshape(-1, self.dim)
        if x2.dtype != torch.float32 or not x2.is_contiguous():
            x2 = x2.float().contiguous()
        trainable = (self.wq, self.bn_gamma, self.bn_beta, self.subkeys) + (
            (self.values,) if isinstance(self.values, torch.nn.Parameter) else ())
        if self.training or (torch.is_grad_enabled() and (x2.requires_grad or any(p.requires_grad for p in trainable))):
            values = self.values if isinstance(self.values, torch.nn.Parameter) else self.values.detach()
            out, idx, w = _Lookup.apply(self, x2, self.wq, self.bn_gamma, self.bn_beta, self.subkeys, values)
        else:
            P = self._params()
            self._sync_prepared(P)
            out, idx, w = self._memory().forward(P, x2)
        out = out.reshape(*lead, self.dim)
        if return_selection:
            return out, idx.reshape(*lead, self.heads, self.k), w.reshape(*lead, self.heads, self.k)
        return out

    def extra_repr(self):
        return (f"dim={self.dim}, heads={self.heads}, n_keys={self.n_keys}, k={self.k}, "
                f"value_type={self.value_type}, max_batch={self.max_batch}, sparse_values={self.sparse_values}, "
                f"prepare_weights={self.prepare_weights}")
