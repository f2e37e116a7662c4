"""MI355X-native (gfx950) product-key memory lookup.

The forward pass of a product-key memory layer -- query projection with
inference batch-norm, per-half subkey scoring, exact per-half top-k, the k^2
candidate top-k, softmax and the weighted gather-sum over the value table --
runs in hand-written HIP kernels behind the C ABI of include/pkm.h
(libpkm.so, built by ``python -m product_key_memory_amd.build``).  This
package is the thin Python binding: torch provides device memory and
streams, nothing else.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, PKM_E_ARG, PKM_E_DEVICE, PKM_E_NOMEM, PKM_E_UNSUPPORTED, PKM_OK, SCALED, VALUE_TYPES, Config,
    Memory, Params, PkmError, config_check, forward_noalloc, last_error, load_library, make_config, status_str,
    workspace_bytes,
)


def params_to_device(p, table, device="cuda"):
    """Copies host (numpy) parameters to device tensors and wraps them.

    p: dict with wq, mean, var, gamma, beta, subkeys, values and (E4M3 tables)
    scale; values hold fp32 numbers, bf16 bits (uint16), E4M3 bits (uint8),
    int8 codes or packed int4 codes ([N, D/2] uint8); E4M3, int8 and int4
    tables carry row scales.
    """
    import numpy as np
    import torch

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    values = p["values"]
    if table == "bf16":
        v = dev(values.view(np.int16)).view(torch.bfloat16)
    elif table == "e4m3":
        v = dev(values.view(np.uint8)).view(torch.float8_e4m3fn)
    elif table == "int8":
        v = dev(values.view(np.int8))
    elif table == "int4":
        v = dev(values.view(np.uint8))  # [N, D/2]: two codes per byte
    else:
        v = dev(values.astype(np.float32, copy=False))
    scale = dev(p["scale"]) if table in SCALED else None
    return Params(dev(p["wq"]), dev(p["mean"]), dev(p["var"]), dev(p["gamma"]), dev(p["beta"]), dev(p["subkeys"]), v,
                  scale)


def __getattr__(name):
    # the torch layer is imported on first use (it imports torch itself)
    if name == "ProductKeyMemory":
        from .layer import ProductKeyMemory

        return ProductKeyMemory
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
