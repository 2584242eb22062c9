"""ctypes binding of libchunkprefill.so: argument marshalling only.

Every computation happens in the HIP library; this module turns torch tensors
into device pointers and Python ints into C integers.  torch is imported
first so that the library binds to the HIP runtime torch already loaded (both
carry the soname libamdhip64.so.7), which makes torch streams and device
pointers valid inside the library.  Loading fails loudly when the library is
not built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime before the library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libchunkprefill.so")

CP_OK, CP_E_INVALID, CP_E_CAPACITY, CP_E_STATE, CP_E_DEVICE, CP_E_ARENA = 0, -1, -2, -3, -4, -5
CP_KV_F16, CP_KV_Q8_0 = 0, 1
KV_TYPES = {"f16": CP_KV_F16, "q8_0": CP_KV_Q8_0}

c_i32, c_i64, c_sz, c_vp, c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class cp_config(ctypes.Structure):
    _fields_ = [("n_layer", c_i32), ("d_model", c_i32), ("n_head", c_i32), ("n_kv_head", c_i32),
                ("head_dim", c_i32), ("ffn_dim", c_i32), ("n_expert", c_i32),
                ("n_expert_used", c_i32), ("expert_ffn_dim", c_i32), ("rms_eps", c_f),
                ("rope_theta", c_f), ("kv_type", c_i32), ("n_ctx_max", c_i32),
                ("n_chunk_max", c_i32)]


class cp_layer_weights(ctypes.Structure):
    _fields_ = [("wq", c_vp), ("wk", c_vp), ("wv", c_vp), ("wo", c_vp), ("attn_norm", c_vp),
                ("ffn_norm", c_vp), ("w_gate", c_vp), ("w_up", c_vp), ("w_down", c_vp),
                ("w_router", c_vp)]


# name -> (restype, argtypes)
SIGNATURES = {
    "cp_weights_arena_bytes": (c_sz, [ctypes.POINTER(cp_config)]),
    "cp_kv_bytes": (c_sz, [ctypes.POINTER(cp_config)]),
    "cp_workspace_bytes": (c_sz, [ctypes.POINTER(cp_config)]),
    "cp_validate_config": (ctypes.c_int, [ctypes.POINTER(cp_config)]),
    "cp_config_error": (ctypes.c_char_p, [ctypes.POINTER(cp_config)]),
    "prefill_init": (ctypes.c_int, [ctypes.POINTER(cp_config), ctypes.POINTER(cp_layer_weights),
                                    c_vp, c_vp, c_vp, c_vp, ctypes.POINTER(c_vp)]),
    "prefill_chunk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32]),
    "prefill_chunk_static": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32]),
    "prefill_chunks": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp),
                                      ctypes.POINTER(c_vp)]),
    "prefill_chunk_timed": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, ctypes.POINTER(c_f)]),
    "prefill_chunk_trace": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_vp, c_i64, c_vp, c_i64]),
    "kv_cache_get_state": (ctypes.c_int, [c_vp, c_vp, c_sz, ctypes.POINTER(c_sz)]),
    "kv_cache_set_state": (ctypes.c_int, [c_vp, c_vp, c_sz]),
    "cp_state_check": (ctypes.c_int, [ctypes.POINTER(cp_config), c_vp, c_sz]),
    "cp_state_bytes": (c_sz, [ctypes.POINTER(cp_config), c_i32]),
    "cp_chunk_check": (ctypes.c_int, [ctypes.POINTER(cp_config), c_i32, c_vp, c_vp, c_i32]),
    "kv_cache_truncate": (ctypes.c_int, [c_vp, c_i32]),
    "prefill_n_past": (c_i32, [c_vp]),
    "prefill_last_error": (ctypes.c_char_p, [c_vp]),
    "prefill_free": (None, [c_vp]),
    "cp_kernel_timing": (ctypes.c_int, [c_vp, ctypes.c_char_p]),
    "cp_kernel_times": (ctypes.c_int, [c_vp, ctypes.c_char_p, ctypes.POINTER(c_f),
                                       ctypes.POINTER(c_i32)]),
    "cp_quantize_q8_0": (ctypes.c_int, [c_vp, c_i64, c_i32, c_i64, c_vp, c_vp]),
    "cp_plan_chunk": (c_i32, [c_i32, c_i32, c_i32, ctypes.c_double]),
    "cp_last_logits": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_i32, c_f, c_vp, c_vp]),
    "cp_peak_sink_bytes": (c_sz, []),
    "cp_measure_peaks": (ctypes.c_int, [c_vp, c_sz, c_vp, c_sz, c_vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]),
    "cp_test_kv_layer_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
    "cp_test_rope_kv_append": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                              c_i32, c_i32, c_vp, c_vp, c_vp]),
    "cp_test_rope_kv_append_planes": (ctypes.c_int, [c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                                     c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "cp_test_kv_rows": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "cp_test_router_scratch_bytes": (c_sz, [c_i32, c_i32]),
    "cp_test_router": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                      c_vp, c_vp]),
    "cp_test_gemm_scratch_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
    "cp_test_gemm_plan": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]),
    "cp_test_set_plan_shared": (ctypes.c_int, [c_vp, c_i32]),
    "cp_test_gemm": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                    c_vp]),
    "cp_test_gemm_scratch_bytes_ex": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "cp_test_gemm_ex": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                       c_vp, c_vp]),
    "cp_test_attention_scratch_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
    "cp_test_attention": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_i32, c_i32, c_vp, c_vp, c_vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m chunked_prompt_prefill_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class PrefillError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"chunk_prefill error {code}: {msg}")
        self.code = code


def ptr(t) -> int:
    """Device/host address of a tensor (or None -> NULL)."""
    return None if t is None else t.data_ptr()


def stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream
