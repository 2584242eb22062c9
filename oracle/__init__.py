"""CPU oracle for chunked prompt prefill of a decoder transformer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and never consumes anything the library produced.

Pages cited (by title):
  [split-psm]  "completion : allow the prompt to be processed under its own split mode"
  [split-live] "llama : switch the split mode of a live context"
  [overlap]    the llama.cpp "--split-overlap" pull request (AllReduce of one ubatch
               overlapped with the next ubatch)
  [planner]    "refactor: one prefill planner and one pad-trim hook for CLI and server"
  [pipe]       "Prompt chunks sized for a layer split's pipeline (STRATA_PREFILL_PIPE=1, opt-in)"

The pages measure chunked prefill (a prompt read in ubatches/chunks, each chunk
run through every layer and appended to a device cache of type f16 or q8_0)
but never write the per-layer arithmetic down.  The per-layer math here is the
plain standard decoder layer: RMSNorm, q8_0 projections, NeoX RoPE, causal GQA
softmax attention against the cache (append, then attend), output projection,
SwiGLU FFN dense or top-k routed.  Every reading taken where the pages are
silent is listed in the repository's design notes.

Precision: floating-point math is float64 except where the method itself fixes
a float32 step that decides stored bytes or integers (q8_0 encode, RoPE of the
rows written to the cache, f16 cache conversion, router logits that decide the
expert indices).  Those steps are written in float32 with one rounding per
operation, the precision the GPU kernels take the same decisions in.

Parity status of each function (what pins it) is stated in its docstring.
"""
from .q8_0 import (q8_0_encode, q8_0_decode, q8_0_to_bytes, q8_0_from_bytes,
                   q8_0_encode_bytes, q8_0_decode_bytes, QK)
from .layer import (rmsnorm, rope_table, rope_apply_f32, rope_apply, attention, to_f16,
                    swiglu_ffn, router_logits_ordered, moe_route, moe_ffn,
                    cache_encode_rows, cache_decode_rows)
from .prefill import OracleModel, OracleCache, dequant_layer, quantize_layer
from .state import (state_bytes, state_size, parse_state, load_state, row_bytes,
                    STATE_MAGIC, STATE_VERSION)
from .costfit import fit_linear, fit_quadratic
from .planner import pipeline_chunk
from .logits import last_logits

__all__ = [n for n in dir() if not n.startswith("_")]
