"""fp64 CPU oracle for the product-key memory lookup: the forward pass and its
gradients.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library.
"""
from .oracle import (Model, run, bf16_to_f64, e4m3_to_f64, int8_to_f64, int4_to_f64, build, lib_path, load_library,  # noqa: F401
                     compile_source, select, gather, backward, GRADS, batch_stats, run_batch_stats,
                     backward_batch_stats, usage, scores, running_update)
