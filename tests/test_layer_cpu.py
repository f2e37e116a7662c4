"""CPU: the torch layer has no CPU path -- it refuses a CPU device -- and
its import needs no GPU."""
import pytest


def test_layer_refuses_cpu():
    import product_key_memory_amd as pk

    with pytest.raises(ValueError, match="no CPU path"):
        pk.ProductKeyMemory(64, 1, 16, 4, value_type="f32", device="cpu")


def test_layer_rejects_unknown_table():
    from product_key_memory_amd.layer import ProductKeyMemory

    with pytest.raises(ValueError, match="value_type"):
        ProductKeyMemory(64, 1, 16, 4, value_type="fp16", device="cuda")
