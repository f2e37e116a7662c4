"""CPU: the C-ABI library loads, exports every symbol include/pkm.h declares,
and rejects bad configurations and arguments on the host, before any device
work.  Nothing here launches a kernel or touches a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import product_key_memory_amd as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(pk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = pk.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pk.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s(pkm_\w+)", out.stdout))
    assert set(declared_functions()) <= exported


def test_library_has_gfx950_code_object():
    """Each kernel source contributes one gfx950 offload bundle entry."""
    blob = open(pk.LIB_PATH, "rb").read()
    assert blob.count(b"hipv4-amdgcn-amd-amdhsa--gfx950") >= 3


def test_status_strings():
    assert pk.status_str(pk.PKM_OK) == "ok"
    assert "argument" in pk.status_str(pk.PKM_E_ARG)
    assert "unsupported" in pk.status_str(pk.PKM_E_UNSUPPORTED)
    assert pk.status_str(99) == "unknown status"


GOOD = dict(dim=1024, heads=4, n_keys=1024, k=32, value_type="bf16", bn_eps=1e-5, max_batch=16384)


@pytest.mark.parametrize("change,status", [
    ({}, pk.PKM_OK),
    (dict(dim=63), pk.PKM_E_ARG),                  # odd: the query cannot be halved
    (dict(dim=0), pk.PKM_E_ARG),
    (dict(dim=96), pk.PKM_E_UNSUPPORTED),          # even but not a multiple of 64
    (dict(heads=0), pk.PKM_E_ARG),
    (dict(n_keys=1), pk.PKM_E_ARG),
    (dict(n_keys=46341), pk.PKM_E_ARG),            # n^2 >= 2^31
    (dict(n_keys=4097), pk.PKM_E_UNSUPPORTED),
    (dict(k=0), pk.PKM_E_ARG),
    (dict(n_keys=16, k=17), pk.PKM_E_ARG),         # topk needs k <= n_keys
    (dict(k=65), pk.PKM_E_UNSUPPORTED),
    (dict(value_type=5), pk.PKM_E_ARG),            # no such table format
    (dict(value_type="int8"), pk.PKM_OK),
    (dict(value_type="int4"), pk.PKM_OK),
    (dict(bn_eps=0.0), pk.PKM_E_ARG),
    (dict(bn_eps=-1.0), pk.PKM_E_ARG),
    (dict(bn_eps=float("nan")), pk.PKM_E_ARG),
    (dict(max_batch=0), pk.PKM_E_ARG),
    (dict(max_batch=(1 << 30) + 1), pk.PKM_E_ARG),
    (dict(n_keys=4096, k=64, dim=64, heads=1, value_type="e4m3"), pk.PKM_OK),
    (dict(n_keys=16, k=16, dim=64, heads=1, value_type="f32"), pk.PKM_OK),
])
def test_config_check(change, status):
    cfg = pk.make_config(**{**GOOD, **change})
    assert pk.config_check(cfg) == status, pk.last_error()
    if status != pk.PKM_OK:
        assert pk.last_error() != ""


def test_workspace_bytes():
    cfg = pk.make_config(**GOOD)
    mb, H, D, n, k = 16384, 4, 1024, 1024, 32
    stat_part = 2 * (mb // 64) * H * D * 4  # batch statistics: each 64-row chunk's mean and squared deviations
    exps = max(mb + H * D, 2 * H * (mb + n)) * 4  # GEMM row exponents (query or scoring)
    qmax = mb * 2 * H * 4  # largest |q^| per (token, half of a head)
    sub_exp = 2 * H * n * 4  # the subkeys' row exponents
    # prepared weights: Wq's and the subkeys' row exponents, and both split
    # into two fp16 pieces (as many bytes as the fp32 arrays)
    prepared = H * D * 4 + sub_exp + H * D * D * 4 + H * 2 * n * (D // 2) * 4
    # the folded form (n_keys <= D): row exponents, shifts and fp16 pieces of
    # the [2H n, D] folded matrix
    prepared += 2 * H * n * 4 * 2 + 2 * H * n * D * 4
    prepared += mb * D * 4  # a chunk of x as fp16 pieces (folded lookup)
    assert (pk.workspace_bytes(cfg) ==
            4 * mb * H * (D + 2 * n + 2 * k) + stat_part + exps + qmax + sub_exp + prepared)
    with pytest.raises(pk.PkmError):
        pk.workspace_bytes(pk.make_config(**{**GOOD, "k": 0}))


def test_flat_workspace_bytes():
    """Key scores [B, H, n^2] fp32, the merge buffers, the GEMM's row
    exponents (H (B + 2 n) int32), each rounded to 256 bytes.  Rows of at
    most 4096 keys are topped directly: merge buffers for rows of n^2
    scores, ceil(n^2 / 4096) * k packed keys per row and ceil(that / 2048) *
    k.  Longer rows use a threshold: merge buffers for rows of G = ceil(n^2 /
    64) group maxima, then the group maxima [B, H, G] f32, theta's indices
    and scores [B, H, k], the list counts [B, H] u32 and the lists [B, H, 512]
    of packed keys.  Last, the subkeys split into two fp16 pieces (H * 2 sets
    of n rounded up to 32 rows, D/2 values, 4 bytes each)."""
    lib = pk.load_library()

    def rnd(x):
        return (x + 255) // 256 * 256

    for n, k in ((1024, 32), (64, 32), (65, 64), (16, 4)):
        cfg = pk.make_config(**{**GOOD, "n_keys": n, "k": k})
        H, N = 4, n * n
        for B in (1, 16, 100):
            rows = B * H
            G = (N + 63) // 64
            thr = N > 4096
            keys = ((G if thr else N) + 4095) // 4096 * k
            want = (rnd(rows * N * 4) + rnd(rows * keys * 8) + rnd(rows * ((keys + 2047) // 2048) * k * 8)
                    + rnd(H * (B + 2 * n) * 4))
            if thr:
                want += rnd(rows * G * 4) + 2 * rnd(rows * k * 4) + rnd(rows * 4) + rnd(rows * 512 * 8)
            want += rnd(H * 2 * ((n + 31) // 32) * 32 * (1024 // 2) * 4)  # the split subkeys
            got = ctypes.c_size_t()
            assert lib.pkm_flat_workspace_bytes(ctypes.byref(cfg), B, ctypes.byref(got)) == pk.PKM_OK
            assert got.value == want, (n, k, B)
    cfg = pk.make_config(**GOOD)
    got = ctypes.c_size_t()
    assert lib.pkm_flat_workspace_bytes(ctypes.byref(cfg), 65537, ctypes.byref(got)) == pk.PKM_E_ARG
    assert lib.pkm_flat_workspace_bytes(ctypes.byref(cfg), -1, ctypes.byref(got)) == pk.PKM_E_ARG


def test_backward_workspace_bytes():
    """Chunks of max_batch tokens: q, dq^, dq [mb, H*D], dq^T [H*D, mb32],
    x^T [D, mb32], Wq^T, the half-score gradients [2H, n, mb32],
    the BN partial sums, per-row counts / cursors / offsets and the lists,
    then up to four split-K partial products of the dWq / dx GEMMs and the
    GEMMs' row exponents."""
    lib = pk.load_library()
    cfg = pk.make_config(**{**GOOD, "max_batch": 1000})
    mb, mb32, H, D, n, k = 1000, 1024, 4, 1024, 1024, 32
    HD, N = H * D, n * n

    def rnd(x):
        return (x + 255) // 256 * 256

    want = (3 * rnd(mb * HD * 4) + rnd(mb * H * k * 4) + rnd(HD * mb32 * 4) + rnd(D * mb32 * 4)
            + rnd(D * HD * 4) + rnd(2 * HD * 4) + rnd(2 * H * n * mb32 * 4) + 2 * rnd(((mb + 63) // 64) * HD * 4)
            + 3 * rnd(N * 4) + rnd(((N + 4095) // 4096) * 4) + rnd(mb * H * k * 4)
            + rnd(4 * max(HD * D, mb * D) * 4) + rnd(max(mb + HD, H * 2 * D, mb + D) * 4))
    got = ctypes.c_size_t()
    assert lib.pkm_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(got)) == pk.PKM_OK
    assert got.value == want


def test_null_arguments_rejected_before_any_launch():
    lib = pk.load_library()
    null = ctypes.c_void_p()
    params = pk._binding.ParamsStruct()
    assert lib.pkm_forward(null, ctypes.byref(params), 1, null, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_query(null, ctypes.byref(params), 1, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_score(null, ctypes.byref(params), 1, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_select(null, 1, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_select_gather(null, ctypes.byref(params), 1, null, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_forward_stage(null, ctypes.byref(params), 1, null, null, null, null, 0, null) == pk.PKM_E_ARG
    assert lib.pkm_gather(null, ctypes.byref(params), 1, 1, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_flat_search(null, ctypes.byref(params), 1, null, null, 0, null, null, null) == pk.PKM_E_ARG
    grads = pk._binding.GradsStruct()
    assert lib.pkm_backward(null, ctypes.byref(params), 1, null, null, null, null, ctypes.byref(grads), null, 0,
                            null) == pk.PKM_E_ARG
    assert lib.pkm_forward_train(null, ctypes.byref(params), 1, null, null, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_prepare(null, ctypes.byref(params), 0, null) == pk.PKM_E_ARG
    assert lib.pkm_half_scores(null, ctypes.byref(params), 1, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_backward_with_q(null, ctypes.byref(params), 1, null, null, null, null, null, ctypes.byref(grads),
                                   null, 0, null) == pk.PKM_E_ARG
    good = pk.make_config(**GOOD)
    assert lib.pkm_forward_noalloc(None, ctypes.byref(params), 1, null, null, null, null, null) == pk.PKM_E_ARG
    assert lib.pkm_forward_noalloc(ctypes.byref(good), ctypes.byref(params), 1, null, null, null, null,
                                   null) == pk.PKM_E_ARG
    assert lib.pkm_forward_noalloc(ctypes.byref(good), ctypes.byref(params), -1, null, null, null, null,
                                   null) == pk.PKM_E_ARG
    # one token's workspace larger than the library's scratch array
    huge = pk.make_config(**{**GOOD, "dim": 65536, "heads": 512, "n_keys": 4096})
    assert lib.pkm_config_check(ctypes.byref(huge)) == pk.PKM_OK
    assert lib.pkm_forward_noalloc(ctypes.byref(huge), ctypes.byref(params), 1, null, null, null, null,
                                   null) == pk.PKM_E_UNSUPPORTED
    assert "scratch" in pk.last_error()
    assert lib.pkm_create(None, ctypes.byref(ctypes.c_void_p())) == pk.PKM_E_ARG
    assert lib.pkm_create(ctypes.byref(pk.make_config(**GOOD)), None) == pk.PKM_E_ARG
    assert "NULL" in pk.last_error()
    lib.pkm_destroy(null)  # NULL-safe


def test_binding_rejects_host_tensors():
    import torch

    with pytest.raises(ValueError, match="GPU"):
        pk._binding._expect(torch.zeros(4, 4), "x", (4, 4), "float32")
    with pytest.raises(ValueError, match="shape"):
        pk._binding._expect(torch.zeros(4, 4), "x", (4, 5), "float32")
    with pytest.raises(ValueError, match="expected one of"):
        pk._binding._expect(torch.zeros(4, 4, dtype=torch.float64), "x", (4, 4), "float32")


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structures have the header's member names,
    offsets and sizes (a C program built against include/pkm.h prints
    them)."""
    structs = {"pkm_config": pk._binding.Config, "pkm_params": pk._binding.ParamsStruct,
               "pkm_grads": pk._binding.GradsStruct}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "pkm.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(line.split()[:2]): int(line.split()[2]) for line in out if line}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert got[(cname, field)] == getattr(py, field).offset, (cname, field)
    # every member the header declares is in the binding
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for cname, py in structs.items():
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + cname + ";", text).group(1)
        members = re.findall(r"(\w+)\s*;", body)
        assert members == [f for f, _ in py._fields_], cname


def test_c_program_rejects_bad_inputs_without_a_device(tmp_path):
    """The plain-C caller (tests/c_driver) is built and linked, and turns a
    malformed file or an unsupported configuration into an error before
    any device call."""
    import numpy as np

    from product_key_memory_amd import build as pkm_build

    assert os.path.exists(pkm_build.C_DRIVER)
    bad = tmp_path / "bad.bin"
    bad.write_bytes(b"NOTPKM00")
    r = subprocess.run([pkm_build.C_DRIVER, str(bad), str(tmp_path / "o.bin")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "bad magic" in r.stderr
    odd = tmp_path / "odd.bin"   # D = 63 is not a multiple of 64
    odd.write_bytes(b"PKMIN1\0\0" + np.array([63, 1, 16, 4, 0, 0], np.int32).tobytes() +
                    np.array([8, 8], np.int64).tobytes())
    r = subprocess.run([pkm_build.C_DRIVER, str(odd), str(tmp_path / "o.bin")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "config" in r.stderr, r.stderr
