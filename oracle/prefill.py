"""Chunked prompt prefill through a stack of decoder layers (oracle, test infrastructure only).

Chunked prefill ([overlap], section "How"; [pipe], section "Summary"; [planner],
section "Current Behavior"): the prompt is read in consecutive chunks of C
tokens; each chunk runs through every layer, appending its K/V rows to that
layer's cache before attending, and the next chunk starts at n_past += C.

Two drivers compute the same thing:
  * `prefill(x, chunk)` runs exactly the chunk loop;
  * `prefill_layer_major(x)` runs the whole prompt through layer 0, then layer 1, ...
They agree because every per-row step is row-local and attention of a row only
reads cache rows at or before its own position, which both drivers have
written identically by then.  The layer-major driver bounds memory and time on
large prompts.

Pinned by: chunked == layer-major, and equality across chunk sizes; the
per-layer functions' own pins (see layer.py); the prefix property (outputs of
a prefix do not change when tokens are appended); closed-form stacks: with
W_q = 0 and W_down = 0 every layer is the residual plus the causal prefix mean
of the cached V rows through W_o, evaluated independently in numpy.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .q8_0 import q8_0_decode_bytes, q8_0_from_bytes, q8_0_encode_bytes, QK
from .layer import (rmsnorm, rope_table, rope_apply_f32, attention, swiglu_ffn,
                    router_logits_ordered, moe_route, moe_ffn, cache_encode_rows,
                    cache_decode_rows, to_f16)

MATRIX_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "w_router")


def quantize_layer(fp32_layer: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """float32 tensors -> the layer as handed to both sides: q8_0 interchange bytes
    for every matrix ([..., N][ceil(K/32)*34] uint8), float32 for the norm gains."""
    out = {}
    for name, t in fp32_layer.items():
        out[name] = q8_0_encode_bytes(t) if name in MATRIX_NAMES else np.asarray(t, np.float32)
    return out


def _decode_matrix(b: np.ndarray, K: int, dtype, rows_per_block: int = 1024,
                   f16: bool = False) -> np.ndarray:
    """q8_0_decode_bytes of every row, converted to dtype (f16: each value rounded to
    binary16 first).  Each row decodes on its own, so the rows are split into blocks
    decoded by a thread pool (NumPy releases the GIL in these loops); the values are those
    of one call over the whole matrix."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    flat = b.reshape(-1, b.shape[-1])
    out = np.empty((flat.shape[0], K), dtype=dtype)

    def work(s):
        blk = q8_0_decode_bytes(flat[s:s + rows_per_block], K)
        out[s:s + rows_per_block] = to_f16(blk) if f16 else blk

    starts = range(0, flat.shape[0], rows_per_block)
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(work, starts))
    return out.reshape(b.shape[:-1] + (K,))


def dequant_layer(qlayer: Dict[str, np.ndarray], K_of: Dict[str, int],
                  dtype=np.float64, f16_names=()) -> Dict[str, np.ndarray]:
    """Interchange bytes -> dense matrices (float64 by default); gains passed through.
    Matrices named in f16_names have every value rounded to binary16."""
    out = {}
    for name, t in qlayer.items():
        if name in MATRIX_NAMES:
            out[name] = _decode_matrix(t, K_of[name], dtype, f16=name in f16_names)
        else:
            out[name] = np.asarray(t, dtype=dtype)
    return out


class OracleCache:
    """Per-layer KV cache: the stored form (f16 array or q8_0 (d16, q)) and its values."""

    def __init__(self, n_layer: int, n_ctx: int, n_kv_head: int, head_dim: int, kv_type: str):
        self.n_layer, self.n_ctx, self.n_kv_head, self.head_dim = n_layer, n_ctx, n_kv_head, head_dim
        self.kv_type = kv_type
        self.n_past = 0
        shp = (n_ctx, n_kv_head, head_dim)
        nb = head_dim // QK
        if kv_type == "f16":
            self.k = [np.zeros(shp, np.float16) for _ in range(n_layer)]
            self.v = [np.zeros(shp, np.float16) for _ in range(n_layer)]
        elif kv_type == "q8_0":
            mk = lambda: (np.zeros((n_ctx, n_kv_head, nb), np.float16),
                          np.zeros((n_ctx, n_kv_head, nb, QK), np.int8))
            self.k = [mk() for _ in range(n_layer)]
            self.v = [mk() for _ in range(n_layer)]
        else:
            raise ValueError(kv_type)
        self.kval = [np.zeros(shp, np.float32) for _ in range(n_layer)]
        self.vval = [np.zeros(shp, np.float32) for _ in range(n_layer)]

    def write(self, l: int, start: int, k32: np.ndarray, v32: np.ndarray):
        """Convert rows to the cache type and store them at positions start .. start+n-1."""
        n = k32.shape[0]
        if start + n > self.n_ctx:
            raise ValueError("cache capacity exceeded")
        for store, vals, rows in ((self.k, self.kval, k32), (self.v, self.vval, v32)):
            enc = cache_encode_rows(rows, self.kv_type)
            if self.kv_type == "f16":
                store[l][start:start + n] = enc
            else:
                store[l][0][start:start + n] = enc[0]
                store[l][1][start:start + n] = enc[1]
            vals[l][start:start + n] = cache_decode_rows(enc, self.kv_type)

    def stored(self, l: int, which: str, n_tokens: int):
        s = (self.k if which == "k" else self.v)[l]
        if self.kv_type == "f16":
            return s[:n_tokens]
        return s[0][:n_tokens], s[1][:n_tokens]

    def set_stored(self, l: int, which: str, stored, n_tokens: int):
        store = self.k if which == "k" else self.v
        vals = self.kval if which == "k" else self.vval
        if self.kv_type == "f16":
            store[l][:n_tokens] = stored
        else:
            store[l][0][:n_tokens] = stored[0]
            store[l][1][:n_tokens] = stored[1]
        vals[l][:n_tokens] = cache_decode_rows(stored, self.kv_type)


class OracleModel:
    """A stack of decoder layers given as q8_0 interchange bytes + float32 gains.

    cfg: any object with n_layer, d_model, n_head, n_kv_head, head_dim, ffn_dim,
    n_expert, n_expert_used, expert_ffn_dim, rms_eps, rope_theta, kv_type.
    layers: one dict per layer (see quantize_layer).  Dequantised float64
    weights are kept for at most `keep_layers` layers at a time.

    operands: "exact" (default) evaluates every matrix product on the exact operands in
    float64.  "f16" rounds every operand of a matrix product to binary16 first and then
    accumulates exactly (float64): the normed rows entering the projections, each q8_0
    weight (the binary16 of d*q), q and the cache values entering attention, the
    unnormalised attention weights, the attention output, and the SwiGLU intermediate
    (saturated to +-65504).  It is the arithmetic the library states for its matrix
    products, and it is where a q8_0 cache's codes are decided: a K/V value is encoded from
    the products of those operands.  Everything else (norms, RoPE, cache encode, router,
    softmax normaliser, residual) is the same in both modes.
    """

    def __init__(self, cfg, layers: Sequence[Dict[str, np.ndarray]], keep_layers: int = 64,
                 operands: str = "exact"):
        if operands not in ("exact", "f16"):
            raise ValueError(operands)
        self.cfg = cfg
        self.layers = list(layers)
        self.keep = keep_layers
        self.f16 = operands == "f16"
        self._deq: Dict[int, Dict[str, np.ndarray]] = {}
        self._rope = None
        c = cfg
        self.G = c.n_head // c.n_kv_head
        d, hd = c.d_model, c.head_dim
        self.K_of = {"wq": d, "wk": d, "wv": d, "wo": c.n_head * hd, "w_gate": d, "w_up": d,
                     "w_down": c.expert_ffn_dim if c.n_expert else c.ffn_dim, "w_router": d}

    # -- weights ------------------------------------------------------------------------
    def weights(self, l: int) -> Dict[str, np.ndarray]:
        if l not in self._deq:
            if len(self._deq) >= self.keep:
                self._deq.pop(next(iter(self._deq)))
            f16_names = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down") if self.f16 else ()
            self._deq[l] = dequant_layer(self.layers[l], self.K_of, f16_names=f16_names)
        return self._deq[l]

    def _op(self, a: np.ndarray) -> np.ndarray:
        """A matrix-product operand as this mode takes it."""
        return to_f16(a) if self.f16 else a

    def rope(self, n_pos: int):
        if self._rope is None or self._rope[0].shape[0] < n_pos:
            self._rope = rope_table(n_pos, self.cfg.head_dim, self.cfg.rope_theta)
        return self._rope

    def new_cache(self, n_ctx: int) -> OracleCache:
        c = self.cfg
        return OracleCache(c.n_layer, n_ctx, c.n_kv_head, c.head_dim, c.kv_type)

    # -- one layer ----------------------------------------------------------------------
    def qkv_rows(self, l: int, x: np.ndarray, positions: np.ndarray):
        """RMSNorm -> q/k/v projections -> RoPE (float32) for rows at `positions`.

        Returns (q32 [n][Hq][hd], k32 [n][Hkv][hd], v32 [n][Hkv][hd]) float32: the
        rows as they are decided before the cache conversion.
        """
        c, W = self.cfg, self.weights(l)
        n, hd = x.shape[0], c.head_dim
        y = self._op(rmsnorm(x, W["attn_norm"], c.rms_eps))
        q = (y @ W["wq"].T).astype(np.float32).reshape(n, c.n_head, hd)
        k = (y @ W["wk"].T).astype(np.float32).reshape(n, c.n_kv_head, hd)
        v = (y @ W["wv"].T).astype(np.float32).reshape(n, c.n_kv_head, hd)
        cos, sin = self.rope(int(np.max(positions)) + 1)
        cs, sn = cos[positions], sin[positions]
        return rope_apply_f32(q, cs, sn), rope_apply_f32(k, cs, sn), v

    def kv_rows(self, l: int, x: np.ndarray, positions: np.ndarray):
        """RMSNorm -> k/v projections -> RoPE of k (float32) for rows at `positions`:
        the K/V half of qkv_rows, for rows whose query is not needed."""
        c, W = self.cfg, self.weights(l)
        n, hd = x.shape[0], c.head_dim
        y = self._op(rmsnorm(x, W["attn_norm"], c.rms_eps))
        k = (y @ W["wk"].T).astype(np.float32).reshape(n, c.n_kv_head, hd)
        v = (y @ W["wv"].T).astype(np.float32).reshape(n, c.n_kv_head, hd)
        cos, sin = self.rope(int(np.max(positions)) + 1)
        return rope_apply_f32(k, cos[positions], sin[positions]), v

    def attn_out_rows(self, l: int, x: np.ndarray, q32: np.ndarray, K: np.ndarray, V: np.ndarray,
                      positions: np.ndarray) -> np.ndarray:
        """Attention of rows q32 against cache values K/V, then x + o W_o^T."""
        c, W = self.cfg, self.weights(l)
        if self.f16:
            T = int(np.max(positions)) + 1
            o = to_f16(attention(to_f16(q32), to_f16(K[:T]), to_f16(V[:T]), positions, p_f16=True))
        else:
            o = attention(q32, K, V, positions)
        return np.asarray(x, np.float64) + o.reshape(x.shape[0], -1) @ W["wo"].T

    def ffn_rows(self, l: int, x: np.ndarray, return_routing: bool = False):
        """x + FFN(RMSNorm(x)): dense SwiGLU, or routed experts (the oracle's own top-k)."""
        c, W = self.cfg, self.weights(l)
        y = rmsnorm(x, W["ffn_norm"], c.rms_eps)
        if not c.n_expert:
            out = x + swiglu_ffn(self._op(y), W["w_gate"], W["w_up"], W["w_down"], h_f16=self.f16)
            return (out, None) if return_routing else out
        nb = c.d_model // QK
        d16, q = q8_0_from_bytes(self.layers[l]["w_router"], nb)
        r = router_logits_ordered(y.astype(np.float32), d16, q)
        idx, w = moe_route(r, c.n_expert_used)
        out = x + moe_ffn(self._op(y), idx, w, W["w_gate"], W["w_up"], W["w_down"], h_f16=self.f16)
        return (out, (r, idx, w)) if return_routing else out

    def layer(self, l: int, x: np.ndarray, cache: OracleCache, start: int,
              routing_out: Optional[List] = None) -> np.ndarray:
        """One layer over rows at positions start .. start+n-1 (append, then attend)."""
        n = x.shape[0]
        pos = np.arange(start, start + n)
        q32, k32, v32 = self.qkv_rows(l, x, pos)
        cache.write(l, start, k32, v32)
        x = self.attn_out_rows(l, x, q32, cache.kval[l], cache.vval[l], pos)
        out, routing = self.ffn_rows(l, x, return_routing=True)
        if routing_out is not None:
            routing_out.append(routing)
        return out

    def layer_rows(self, l: int, x: np.ndarray, rows, block: int = 2048):
        """Layer l over the prompt x (row t at position t), evaluated at the rows `rows` only.

        Attention of a row reads only cache rows at or before its own position, so K/V are
        computed and stored (in the cache's type) for every position up to max(rows), while
        q, attention, the output projection and the FFN run for `rows` alone.  This is
        `layer` restricted to those rows; it lets long prompts be checked at sampled rows.
        Returns (outputs [len(rows)][d] float64, the cache holding rows 0 .. max(rows) of
        layer l)."""
        rows = np.asarray(rows, dtype=np.int64)
        T = int(rows.max()) + 1
        cache = self.new_cache(T)
        self.rope(T)    # one table for every position, instead of regrowing it per block
        for r0 in range(0, T, block):
            r1 = min(T, r0 + block)
            k32, v32 = self.kv_rows(l, x[r0:r1], np.arange(r0, r1))
            cache.write(l, r0, k32, v32)
        xr = np.asarray(x[rows], dtype=np.float64)
        q32, _, _ = self.qkv_rows(l, xr, rows)
        h = self.attn_out_rows(l, xr, q32, cache.kval[l], cache.vval[l], rows)
        out, routing = self.ffn_rows(l, h, return_routing=True)
        self.last_routing = routing    # (logits, indices, weights) of the rows, routed layers
        return out, cache

    # -- drivers ------------------------------------------------------------------------
    def forward_chunk(self, x: np.ndarray, cache: OracleCache) -> np.ndarray:
        """All layers for one chunk at positions n_past ..; advances n_past."""
        start = cache.n_past
        h = np.asarray(x, dtype=np.float64)
        for l in range(self.cfg.n_layer):
            h = self.layer(l, h, cache, start)
        cache.n_past = start + x.shape[0]
        return h

    def prefill(self, x: np.ndarray, chunk: int, cache: Optional[OracleCache] = None,
                n_ctx: Optional[int] = None) -> np.ndarray:
        """Chunked driver: the prompt in consecutive chunks of `chunk` tokens."""
        if cache is None:
            cache = self.new_cache(n_ctx or x.shape[0])
        outs = []
        for s in range(0, x.shape[0], chunk):
            outs.append(self.forward_chunk(x[s:s + chunk], cache))
        self.last_cache = cache
        return np.concatenate(outs, axis=0) if outs else np.zeros((0, self.cfg.d_model))

    def prefill_layer_major(self, x: np.ndarray, cache: Optional[OracleCache] = None,
                            n_ctx: Optional[int] = None, layer_outputs: Optional[List] = None,
                            routing_out: Optional[List] = None) -> np.ndarray:
        """Layer-major driver: the whole prompt through layer 0, then layer 1, ...

        layer_outputs collects each layer's output; routing_out collects each routed
        layer's (logits, indices, weights)."""
        if cache is None:
            cache = self.new_cache(n_ctx or x.shape[0])
        start = cache.n_past
        h = np.asarray(x, dtype=np.float64)
        for l in range(self.cfg.n_layer):
            h = self.layer(l, h, cache, start, routing_out)
            if layer_outputs is not None:
                layer_outputs.append(h.copy())
        cache.n_past = start + x.shape[0]
        self.last_cache = cache
        return h
