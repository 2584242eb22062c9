"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module holds the workload shapes and the random-number recipe only. It
contains none of the prefill method's arithmetic (no quantisation, no norm, no
attention): it produces float32 arrays and integer token ids, and both the
oracle and the GPU library consume what it returns.

Value law.  Every weight and every hidden-state input is drawn from N(0, 0.02)
(the law the workloads name).  A Gaussian sampler in NumPy runs at a few
million values per second on slow hosts, far too slow for 5 G-parameter layer
stacks, so draws are made by table lookup: a fixed table of 2**20 standard
normal samples (NumPy PCG64, seed 20261202) is indexed by the top 20 bits of a
splitmix64 hash of (tensor seed, element counter).  The hash is plain integer
arithmetic, so the NumPy path and the torch path (used to fill device memory
directly) return bit-identical float32 values for the same seed and size, on
any device.
"""
from __future__ import annotations

import os
import zlib
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

TABLE_BITS = 20
TABLE_SEED = 20261202
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1

_table_cache: Optional[np.ndarray] = None


def normal_table() -> np.ndarray:
    """The 2**20 standard-normal samples every draw is looked up in (float32)."""
    global _table_cache
    if _table_cache is None:
        g = np.random.Generator(np.random.PCG64(TABLE_SEED))
        _table_cache = g.standard_normal(1 << TABLE_BITS, dtype=np.float32)
        _table_cache.setflags(write=False)
    return _table_cache


def tensor_seed(*parts) -> int:
    """Stable 32-bit seed from a tuple of names/ints (crc32 of their text)."""
    return zlib.crc32("/".join(str(p) for p in parts).encode()) & 0xFFFFFFFF


def _index_np(seed: int, start: int, n: int) -> np.ndarray:
    base = (seed * _GOLDEN) & _MASK64
    z = np.arange(start, start + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z += np.uint64(base)
        z ^= z >> np.uint64(30)
        z *= np.uint64(_M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(_M2)
        z ^= z >> np.uint64(31)
    return (z >> np.uint64(64 - TABLE_BITS)).astype(np.int64)


def normal(seed: int, shape, scale: float = 0.02, block: int = 1 << 20) -> np.ndarray:
    """float32 array of `shape` with N(0, scale) values for `seed` (NumPy).

    Every value depends only on (seed, element index), so the blocks are filled by a
    thread pool (NumPy releases the GIL in these loops) with the same result."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    tab = normal_table()
    out = np.empty(n, dtype=np.float32)
    s32 = np.float32(scale)

    def fill(s):
        m = min(block, n - s)
        np.multiply(tab[_index_np(seed, s, m)], s32, out=out[s:s + m])

    starts = range(0, n, block)
    if len(starts) <= 1:
        for s in starts:
            fill(s)
    else:
        with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, starts))
    return out.reshape(shape)


def normal_torch(seed: int, shape, scale: float = 0.02, device="cpu", block: int = 1 << 24):
    """Same values as `normal`, produced with torch ops on `device` (float32)."""
    import torch

    def s64(v):  # unsigned 64-bit constant as the signed int64 with the same bits
        return v - (1 << 64) if v >= (1 << 63) else v

    n = 1
    for d in shape:
        n *= int(d)
    tab = torch.from_numpy(np.array(normal_table())).to(device)
    out = torch.empty(n, dtype=torch.float32, device=device)
    base = s64((seed * _GOLDEN) & _MASK64)
    for s in range(0, n, block):
        m = min(block, n - s)
        z = torch.arange(s, s + m, dtype=torch.int64, device=device)
        z += base
        z ^= (z >> 30) & ((1 << 34) - 1)
        z *= s64(_M1)
        z ^= (z >> 27) & ((1 << 37) - 1)
        z *= s64(_M2)
        z ^= (z >> 31) & ((1 << 33) - 1)
        idx = (z >> (64 - TABLE_BITS)) & ((1 << TABLE_BITS) - 1)
        out[s:s + m] = tab[idx] * scale
    return out.view(*shape)


# --------------------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    ffn_dim: int                 # dense FFN width (0 for MoE)
    n_expert: int = 0
    n_expert_used: int = 0
    expert_ffn_dim: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    kv_type: str = "f16"         # "f16" or "q8_0"
    n_prompt: int = 0
    chunk: int = 0
    vocab: int = 0               # >0: prompt is token ids into an embedding table
    chunk_sweep: Tuple[int, ...] = ()
    depths: Tuple[int, ...] = ()
    depth_prefill: int = 0

    @property
    def is_moe(self) -> bool:
        return self.n_expert > 0

    @property
    def n_ctx(self) -> int:
        return self.n_prompt + max(self.depths, default=0)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny dense decoder, 512 token ids, chunks of 128
    "tiny_dense": Workload("tiny_dense", 2, 256, 4, 2, 64, 688, kv_type="f16",
                           n_prompt=512, chunk=128, vocab=4096),
    # dense 27B-class share of 16 layers, 17,055-token prompt in 512-token chunks
    "dense27b_f16": Workload("dense27b_f16", 16, 5120, 40, 8, 128, 17408, kv_type="f16",
                             n_prompt=17055, chunk=512),
    # same shapes, q8_0 cache, 58,300-token prompt in 2048-token chunks
    "dense27b_q8": Workload("dense27b_q8", 16, 5120, 40, 8, 128, 17408, kv_type="q8_0",
                            n_prompt=58300, chunk=2048),
    # chunk sweep for the b + aC fit, 4 layers, depth 0 and 16,384
    "dense27b_sweep": Workload("dense27b_sweep", 4, 5120, 40, 8, 128, 17408, kv_type="f16",
                               n_prompt=10041, chunk=512,
                               chunk_sweep=(128, 256, 384, 512, 1024, 2048, 4096, 8192),
                               depths=(0, 16384), depth_prefill=16384),
    # MoE stack, 128 experts top-8, 28,998-token prompt in 3328-token chunks
    "moe_a3b": Workload("moe_a3b", 8, 2048, 32, 4, 128, 0, n_expert=128, n_expert_used=8,
                        expert_ffn_dim=768, kv_type="f16", n_prompt=28998, chunk=3328),
}


def weight_shapes(w: Workload) -> List[Tuple[str, Tuple[int, ...]]]:
    """(name, shape) of every per-layer tensor, in generation order.

    Matrices are [out][in]; the norms are 1-D gains.  Expert tensors carry a
    leading expert dimension.
    """
    d, hd = w.d_model, w.head_dim
    shapes = [
        ("attn_norm", (d,)),
        ("wq", (w.n_head * hd, d)),
        ("wk", (w.n_kv_head * hd, d)),
        ("wv", (w.n_kv_head * hd, d)),
        ("wo", (d, w.n_head * hd)),
        ("ffn_norm", (d,)),
    ]
    if w.is_moe:
        E, Fe = w.n_expert, w.expert_ffn_dim
        shapes += [("w_router", (E, d)), ("w_gate", (E, Fe, d)), ("w_up", (E, Fe, d)),
                   ("w_down", (E, d, Fe))]
    else:
        F = w.ffn_dim
        shapes += [("w_gate", (F, d)), ("w_up", (F, d)), ("w_down", (d, F))]
    return shapes


def layer_weight(w: Workload, layer: int, name: str, shape, gains: str = "ones",
                 backend: str = "numpy", device="cpu"):
    """One per-layer tensor.

    Matrices: N(0, 0.02).  Norm gains: all ones (gains="ones") or 1 + N(0, 0.02)
    (gains="random", used by the tests to exercise the gain multiply).
    """
    seed = tensor_seed(w.d_model, w.n_head, w.n_kv_head, w.head_dim, w.ffn_dim,
                       w.n_expert, w.expert_ffn_dim, layer, name)
    if name.endswith("_norm"):
        if gains == "ones":
            if backend == "numpy":
                return np.ones(shape, dtype=np.float32)
            import torch
            return torch.ones(shape, dtype=torch.float32, device=device)
        if backend == "numpy":
            return (np.float32(1.0) + normal(seed, shape)).astype(np.float32)
        return 1.0 + normal_torch(seed, shape, device=device)
    if backend == "numpy":
        return normal(seed, shape)
    return normal_torch(seed, shape, device=device)


def prompt_inputs(w: Workload, n_tokens: Optional[int] = None, salt: str = "prompt",
                  backend: str = "numpy", device="cpu"):
    """Hidden-state rows x_in [n][d_model] float32 for the prompt.

    With a vocabulary (tiny_dense) the rows are embedding-table rows picked by
    uniform token ids; otherwise they are seeded N(0, 0.02) rows directly.
    """
    n = w.n_prompt if n_tokens is None else n_tokens
    d = w.d_model
    if w.vocab:
        ids = token_ids(w, n, salt)
        table = normal(tensor_seed("embedding", w.vocab, d), (w.vocab, d))
        x = table[ids]
        if backend == "numpy":
            return x
        import torch
        return torch.from_numpy(x).to(device)
    seed = tensor_seed("x", salt, d)
    if backend == "numpy":
        return normal(seed, (n, d))
    return normal_torch(seed, (n, d), device=device)


def token_ids(w: Workload, n: int, salt: str = "prompt") -> np.ndarray:
    """Uniform token ids in [0, vocab) (PCG64, seeded by the salt)."""
    g = np.random.Generator(np.random.PCG64(tensor_seed("ids", salt, w.vocab)))
    return g.integers(0, w.vocab, size=n, dtype=np.int64)


def uniform(seed: int, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Seeded uniform float32 values (PCG64) for test vectors."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.uniform(lo, hi, size=shape).astype(np.float32)
