"""MI355X-native chunked prompt prefill: a HIP (gfx950) library with a C ABI.

`prefill` holds the Python face of the C calls; `build` compiles the library.
"""
from ._lib import lib, LIB_PATH, PrefillError, cp_config, cp_layer_weights  # noqa: F401
from .prefill import (PrefillContext, make_config, arena_sizes, validate_config,  # noqa: F401
                      to_device, chunk_check, cp_quantize_q8_0, cp_test_gemm_plan,
                      cp_measure_peaks, cp_plan_chunk, cp_last_logits)
