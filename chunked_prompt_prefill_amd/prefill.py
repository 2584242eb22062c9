"""Python face of the C ABI: the same calls, with torch tensors for device buffers.

The binding is the library's caller: it allocates the three device arenas with
torch (PyTorch is used for device memory and streams only) and passes raw
pointers.  Nothing here computes any part of the prefill path.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from ._lib import (CP_OK, KV_TYPES, PrefillError, c_vp, cp_config, cp_layer_weights, lib, ptr,
                   stream_ptr)

MATRIX_KEYS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "w_router")


def make_config(model, n_ctx_max: int, n_chunk_max: int) -> cp_config:
    """cp_config from any object with the model's geometry attributes (n_layer, d_model,
    n_head, n_kv_head, head_dim, ffn_dim, n_expert, n_expert_used, expert_ffn_dim,
    rms_eps, rope_theta, kv_type as "f16"/"q8_0")."""
    kv = model.kv_type
    return cp_config(model.n_layer, model.d_model, model.n_head, model.n_kv_head, model.head_dim,
                     model.ffn_dim, model.n_expert, model.n_expert_used, model.expert_ffn_dim,
                     float(model.rms_eps), float(model.rope_theta),
                     KV_TYPES[kv] if isinstance(kv, str) else int(kv), int(n_ctx_max),
                     int(n_chunk_max))


def arena_sizes(cfg: cp_config):
    L = lib()
    return (L.cp_weights_arena_bytes(ctypes.byref(cfg)), L.cp_kv_bytes(ctypes.byref(cfg)),
            L.cp_workspace_bytes(ctypes.byref(cfg)))


def validate_config(cfg: cp_config) -> str:
    """Empty string when valid, else the library's message."""
    L = lib()
    if L.cp_validate_config(ctypes.byref(cfg)) == CP_OK:
        return ""
    return L.cp_config_error(ctypes.byref(cfg)).decode()


def chunk_check(cfg: cp_config, n_past: int, x_in_ptr: int, x_out_ptr: int, n_tokens: int) -> int:
    """The host-side checks prefill_chunk makes for a context of cfg at n_past (status code)."""
    return lib().cp_chunk_check(ctypes.byref(cfg), int(n_past), x_in_ptr, x_out_ptr, int(n_tokens))


def to_device(layer: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    """Copy one layer's interchange bytes / gains to device memory."""
    out = {}
    for k, v in layer.items():
        t = v if isinstance(v, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device)
    return out


class PrefillContext:
    """Owns the arenas of one cp_ctx and forwards every call to the library."""

    def __init__(self, cfg: cp_config, layers: Sequence[Dict[str, torch.Tensor]],
                 device="cuda", stream: Optional[torch.cuda.Stream] = None):
        self.L = lib()
        self.cfg = cfg
        self.device = torch.device(device)
        self.stream = stream
        wb, kb, sb = arena_sizes(cfg)
        if wb == 0:
            raise PrefillError(-1, validate_config(cfg))
        self.warena = torch.empty(wb, dtype=torch.uint8, device=self.device)
        self.kv = torch.empty(kb, dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(sb, dtype=torch.uint8, device=self.device)
        arr = (cp_layer_weights * cfg.n_layer)()
        for i, lw in enumerate(layers):
            arr[i] = cp_layer_weights(*(ptr(lw.get(k)) for k in
                                        ("wq", "wk", "wv", "wo", "attn_norm", "ffn_norm",
                                         "w_gate", "w_up", "w_down", "w_router")))
        self._ctx = ctypes.c_void_p()
        rc = self.L.prefill_init(ctypes.byref(cfg), arr, ptr(self.warena), ptr(self.kv),
                                 ptr(self.ws), stream_ptr(stream), ctypes.byref(self._ctx))
        if rc != CP_OK:
            raise PrefillError(rc, "prefill_init failed")

    # -- calls ---------------------------------------------------------------------------
    def _check(self, rc: int):
        if rc != CP_OK:
            raise PrefillError(rc, self.L.prefill_last_error(self._ctx).decode())

    def _out_like(self, x_in: torch.Tensor, *streams) -> torch.Tensor:
        """An output allocated here for work on the context's own stream(s): torch's caching
        allocator is told those streams use it, so the block is not handed out again
        before their work on it is done (even if the caller drops the tensor at once)."""
        x_out = torch.empty_like(x_in)
        for st in (self.stream,) + streams:
            if st is not None:
                x_out.record_stream(st)
        return x_out

    def _follow_caller(self):
        """With a stream of its own, the context's work starts after the work already
        enqueued on the caller's current stream: the producers of the tensors it is handed,
        and the last users of any block torch's allocator hands out there."""
        if self.stream is not None:
            self.stream.wait_stream(torch.cuda.current_stream(self.device))

    def prefill_chunk(self, x_in: torch.Tensor, x_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        self._follow_caller()
        x_out = self._out_like(x_in) if x_out is None else x_out
        self._check(self.L.prefill_chunk(self._ctx, ptr(x_in), ptr(x_out), x_in.shape[0]))
        return x_out

    def _lanes(self, n_lanes: int):
        """Workspaces and streams of lanes 1 .. n_lanes-1, created on first use and kept (as
        ctypes arrays of their addresses)."""
        if not hasattr(self, "lane_ws"):
            self.lane_ws, self.lane_streams = [], []
        while len(self.lane_ws) < n_lanes - 1:
            self.lane_ws.append(torch.empty_like(self.ws))
            self.lane_streams.append(torch.cuda.Stream(device=self.device))
        k = max(0, n_lanes - 1)
        ws = (c_vp * max(1, k))(*[t.data_ptr() for t in self.lane_ws[:k]])
        st = (c_vp * max(1, k))(*[s.cuda_stream for s in self.lane_streams[:k]])
        return ws, st

    def prefill_chunks(self, x_in: torch.Tensor, x_out: Optional[torch.Tensor] = None, chunk: int = 0,
                       n_lanes: int = 2) -> torch.Tensor:
        """The prompt x_in in chunks of `chunk` tokens (default n_chunk_max), n_lanes chunks in
        flight: lane 0 is the context's stream, the others have streams and workspaces owned
        by this object."""
        self._follow_caller()
        ws, st = self._lanes(n_lanes)
        x_out = self._out_like(x_in, *self.lane_streams[:n_lanes - 1]) if x_out is None else x_out
        self._check(self.L.prefill_chunks(self._ctx, ptr(x_in), ptr(x_out), x_in.shape[0],
                                          chunk or self.cfg.n_chunk_max, n_lanes, ws, st))
        return x_out

    def prefill_chunks_raw(self, x_in_ptr: int, x_out_ptr: int, n: int, chunk: int, n_lanes: int = 2) -> int:
        """prefill_chunks on raw device pointers (lanes as above)."""
        ws, st = self._lanes(n_lanes)
        return self.L.prefill_chunks(self._ctx, x_in_ptr, x_out_ptr, n, chunk, n_lanes, ws, st)

    def prefill_chunk_static(self, x_in: torch.Tensor, x_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """prefill_chunk with the chunk's buffers in the library's static device array."""
        self._follow_caller()
        x_out = self._out_like(x_in) if x_out is None else x_out
        self._check(self.L.prefill_chunk_static(self._ctx, ptr(x_in), ptr(x_out), x_in.shape[0]))
        return x_out

    def prefill_chunk_trace(self, x_in: torch.Tensor, x_out: torch.Tensor, layer_out=None,
                            layer_stride: int = 0, route_idx=None, route_stride: int = 0):
        """layer_out / route_idx: device tensors (or None); strides in elements."""
        self._follow_caller()
        self._check(self.L.prefill_chunk_trace(self._ctx, ptr(x_in), ptr(x_out), x_in.shape[0],
                                               ptr(layer_out), layer_stride, ptr(route_idx),
                                               route_stride))
        return x_out

    def prefill_chunk_raw(self, x_in_ptr: int, x_out_ptr: int, n: int) -> int:
        return self.L.prefill_chunk(self._ctx, x_in_ptr, x_out_ptr, n)

    def prefill_chunk_timed(self, x_in: torch.Tensor, x_out: Optional[torch.Tensor] = None):
        self._follow_caller()
        x_out = self._out_like(x_in) if x_out is None else x_out
        ms = (ctypes.c_float * self.cfg.n_layer)()
        self._check(self.L.prefill_chunk_timed(self._ctx, ptr(x_in), ptr(x_out), x_in.shape[0], ms))
        return x_out, list(ms)

    def kv_cache_get_state(self) -> bytes:
        n = ctypes.c_size_t()
        self._check(self.L.kv_cache_get_state(self._ctx, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value)
        self._check(self.L.kv_cache_get_state(self._ctx, buf, n.value, ctypes.byref(n)))
        return buf.raw[:n.value]

    def kv_cache_set_state(self, blob: bytes) -> int:
        """Returns the library's status code (CP_OK or an error) without raising."""
        return self.L.kv_cache_set_state(self._ctx, blob, len(blob))

    def kv_cache_truncate(self, n_keep: int) -> int:
        return self.L.kv_cache_truncate(self._ctx, n_keep)

    @property
    def n_past(self) -> int:
        return self.L.prefill_n_past(self._ctx)

    def last_error(self) -> str:
        return self.L.prefill_last_error(self._ctx).decode()

    def set_plan_shared(self, shared: bool):
        """GEMM launch plans of later single-chunk calls: those prefill_chunks uses with
        several lanes (True) or the single-lane ones (False, the default)."""
        self._check(self.L.cp_test_set_plan_shared(self._ctx, int(shared)))

    def cp_kernel_timing(self, classes: Optional[str]):
        """None: off; "*": every class; else comma-separated class names."""
        self._check(self.L.cp_kernel_timing(self._ctx, None if classes is None else classes.encode()))

    def cp_kernel_times(self, cls: str):
        ms, n = ctypes.c_float(), ctypes.c_int32()
        self._check(self.L.cp_kernel_times(self._ctx, cls.encode(), ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def close(self):
        if self._ctx:
            self.L.prefill_free(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------- helpers
def cp_quantize_q8_0(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q8_0 interchange bytes of float32 device rows x [..., k] (encode on the GPU)."""
    k = x.shape[-1]
    rows = x.numel() // k
    nb = (k + 31) // 32
    if out is None:
        out = torch.empty(x.shape[:-1] + (nb * 34,), dtype=torch.uint8, device=x.device)
    rc = lib().cp_quantize_q8_0(ptr(x), rows, k, k, ptr(out), stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_quantize_q8_0 failed")
    return out


def cp_last_logits(x_row: torch.Tensor, norm_gain: torch.Tensor, lm_head: torch.Tensor,
                   vocab: int, eps: float, logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Logits of one residual row: RMSNorm then the q8_0 LM head (interchange bytes)."""
    d = x_row.numel()
    if logits is None:
        logits = torch.empty(vocab, dtype=torch.float32, device=x_row.device)
    rc = lib().cp_last_logits(ptr(x_row), ptr(norm_gain), ptr(lm_head), int(vocab), int(d), float(eps),
                              ptr(logits), stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_last_logits failed")
    return logits


def cp_plan_chunk(n_tokens: int, cap: int, stages: int, b_over_a: float) -> int:
    """Pipeline chunk size from the fitted b/a (host code of the library)."""
    c = lib().cp_plan_chunk(int(n_tokens), int(cap), int(stages), float(b_over_a))
    if c < 0:
        raise PrefillError(c, "cp_plan_chunk: invalid arguments")
    return c


def cp_measure_peaks(read_bytes: int = 2 << 30, device="cuda"):
    """(MFMA fp16 TFLOP/s, HBM read GB/s) measured on the device by the library's own
    MFMA-only and streaming-read kernels (the buffers are allocated here)."""
    L = lib()
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=device)
    sink = torch.empty(L.cp_peak_sink_bytes(), dtype=torch.uint8, device=device)
    tf, gb = ctypes.c_double(), ctypes.c_double()
    rc = L.cp_measure_peaks(ptr(buf), read_bytes, ptr(sink), sink.numel(), stream_ptr(),
                            ctypes.byref(tf), ctypes.byref(gb))
    if rc != CP_OK:
        raise PrefillError(rc, "cp_measure_peaks failed")
    return tf.value, gb.value


def cp_test_kv_layer_bytes(n_kv_head, head_dim, n_ctx, kv_type) -> int:
    return lib().cp_test_kv_layer_bytes(n_kv_head, head_dim, n_ctx, kv_type)


def cp_test_rope_kv_append(qkv, cos_t, sin_t, n, start, n_head, n_kv_head, head_dim, kv_type,
                           n_ctx, q_out, kv):
    rc = lib().cp_test_rope_kv_append(ptr(qkv), ptr(cos_t), ptr(sin_t), n, start, n_head,
                                      n_kv_head, head_dim, kv_type, n_ctx, ptr(q_out), ptr(kv),
                                      stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_rope_kv_append failed")


def cp_test_rope_kv_append_planes(partial, splits, cos_t, sin_t, n, start, n_head, n_kv_head,
                                  head_dim, kv_type, n_ctx, q_out, kv):
    """RoPE + K/V append from the QKV GEMM's split planes, as prefill_chunk runs it."""
    work = torch.empty(n * (n_head + 2 * n_kv_head) * head_dim, dtype=torch.float32,
                       device=partial.device)
    rc = lib().cp_test_rope_kv_append_planes(ptr(partial), splits, ptr(cos_t), ptr(sin_t), n, start,
                                             n_head, n_kv_head, head_dim, kv_type, n_ctx,
                                             ptr(q_out), ptr(kv), ptr(work), stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_rope_kv_append_planes failed")


def cp_test_kv_rows(kv, n_tokens, n_kv_head, head_dim, kv_type, n_ctx, out):
    rc = lib().cp_test_kv_rows(ptr(kv), n_tokens, n_kv_head, head_dim, kv_type, n_ctx, ptr(out),
                               stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_kv_rows failed")


def cp_test_router(y, w_router, n, d, n_expert, k, logits, idx, weight):
    L = lib()
    scratch = torch.empty(L.cp_test_router_scratch_bytes(n_expert, d), dtype=torch.uint8,
                          device=y.device)
    rc = L.cp_test_router(ptr(y), ptr(w_router), n, d, n_expert, k, ptr(logits), ptr(idx),
                          ptr(weight), ptr(scratch), stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_router failed")


def cp_test_gemm(A, W, M, N, K, mode, splits, out, row_tile=0):
    """One q8_0 GEMM through the library (row_tile 0: the layer's own launch plan)."""
    L = lib()
    nbytes = L.cp_test_gemm_scratch_bytes_ex(M, N, K, splits, row_tile)
    if nbytes == 0:
        raise PrefillError(-1, "cp_test_gemm: unsupported shape")
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=A.device)
    rc = L.cp_test_gemm_ex(ptr(A), ptr(W), M, N, K, mode, splits, row_tile, ptr(out), ptr(scratch),
                           stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_gemm failed")


def cp_test_gemm_plan(M, N, K, plan=0):
    """(row tile, [(first column, split-K factor), ...]) of the layer's launch plan: plan 0
    on a device of its own, 1 beside other chunks in flight, 2 likewise for a GEMM whose
    split-K sums the next kernel adds (output and down projections)."""
    out = (ctypes.c_int32 * 6)()
    rc = lib().cp_test_gemm_plan(M, N, K, int(plan), out)
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_gemm_plan failed")
    return out[0], [(out[2 + 2 * i], out[3 + 2 * i]) for i in range(out[1])]


def cp_test_attention(q, kv, n, start, n_head, n_kv_head, head_dim, kv_type, n_ctx, kv_splits, out):
    L = lib()
    scratch = torch.empty(L.cp_test_attention_scratch_bytes(n, n_head, head_dim, kv_splits),
                          dtype=torch.uint8, device=q.device)
    rc = L.cp_test_attention(ptr(q), ptr(kv), n, start, n_head, n_kv_head, head_dim, kv_type, n_ctx,
                             kv_splits, ptr(out), ptr(scratch), stream_ptr())
    if rc != CP_OK:
        raise PrefillError(rc, "cp_test_attention failed")
