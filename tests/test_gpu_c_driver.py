"""GPU: the library called from a plain C program (tests/c_driver): device
buffers from hipMalloc, a stream of its own, no Python or torch in that
process.  The program runs pkm_forward on seeded inputs this test writes to
a file and returns out / idx / weights, which are checked against the fp64
oracle by the rule of the other forward tests (exact winner sets, order
where fp64 gaps are at least tau, tolerance per table format)."""
import os
import subprocess

import numpy as np
import pytest

import synthetic
from product_key_memory_amd import build as pkm_build
from tests import support
from tests.test_gpu_forward import compare, invariants

pytestmark = pytest.mark.gpu

VALUE_TYPE = {"f32": 0, "bf16": 1, "e4m3": 2, "int8": 3, "int4": 4}


PREPARE = {None: 0, "split": 1, "fold": 2}


def write_inputs(path, wl, params, x, max_batch, prepare=None):
    with open(path, "wb") as f:
        f.write(b"PKMIN1\0\0")
        f.write(np.array([wl.D, wl.H, wl.n, wl.k, VALUE_TYPE[wl.table], PREPARE[prepare]], np.int32).tobytes())
        f.write(np.array([x.shape[0], max_batch], np.int64).tobytes())
        for name in ("wq", "mean", "var", "gamma", "beta", "subkeys"):
            f.write(np.ascontiguousarray(params[name], np.float32).tobytes())
        f.write(np.ascontiguousarray(params["values"]).tobytes())
        if params["scale"] is not None:
            f.write(np.ascontiguousarray(params["scale"], np.float32).tobytes())
        f.write(np.ascontiguousarray(x, np.float32).tobytes())


def read_outputs(path, wl, B):
    raw = np.fromfile(path, dtype=np.uint8)
    sel = B * wl.H * wl.k
    assert raw.size == 4 * (B * wl.D + 2 * sel)
    out = raw[:4 * B * wl.D].view(np.float32).reshape(B, wl.D)
    idx = raw[4 * B * wl.D:4 * (B * wl.D + sel)].view(np.int32).reshape(B, wl.H, wl.k)
    w = raw[4 * (B * wl.D + sel):].view(np.float32).reshape(B, wl.H, wl.k)
    return out, idx, w


@pytest.mark.parametrize("shape", [
    dict(B=333, D=256, H=2, n=128, k=16, table="e4m3", bn="random", max_batch=333),
    dict(B=700, D=128, H=3, n=64, k=8, table="bf16", bn="random", max_batch=256),   # three chunks, ragged last
    dict(B=97, D=64, H=1, n=40, k=40, table="f32", bn="unit", max_batch=97),        # k = n_keys
    dict(B=120, D=192, H=2, n=50, k=12, table="int4", bn="random", max_batch=64),
    dict(B=300, D=256, H=2, n=128, k=16, table="bf16", bn="random", max_batch=128, prepare="fold"),
    dict(B=150, D=128, H=2, n=96, k=8, table="e4m3", bn="random", max_batch=150, prepare="split"),
], ids=lambda s: "B{B}-D{D}-H{H}-n{n}-k{k}-{table}-mb{max_batch}".format(**s) + (
    "-" + s["prepare"] if "prepare" in s else ""))
def test_c_program_forward(tmp_path, shape):
    assert os.path.exists(pkm_build.C_DRIVER), "the C test program is not built (run the package build)"
    wl = synthetic.Workload("c_driver", shape["B"], shape["D"], shape["H"], shape["n"], shape["k"], shape["table"],
                            shape["bn"])
    params = synthetic.make_params(wl, seed=11)
    x = synthetic.make_x(wl, seed=11)
    _, tau = support.gap_clean(wl, params, x, seed=11, want_tau=True)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    write_inputs(inp, wl, params, x, shape["max_batch"], shape.get("prepare"))
    support.say(f"C program: {wl.B} tokens, D {wl.D}, H {wl.H}, n {wl.n}, k {wl.k}, {wl.table}")
    r = subprocess.run([pkm_build.C_DRIVER, str(inp), str(outp)], capture_output=True, text=True, timeout=90)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip().endswith(": ok"), r.stdout
    out, idx, w = read_outputs(outp, wl, wl.B)
    invariants(wl, idx, w)
    compare(wl, params, x, out, idx, w, tau=tau)
