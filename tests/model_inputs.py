"""Test helper: seeded layer stacks as q8_0 interchange bytes (encoded by the oracle).

Both sides of a parity test receive these same bytes; nothing here comes from
the HIP library.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TINY_DENSE = synth.Workload("tiny_test_dense", 2, 64, 4, 2, 32, 96, kv_type="f16",
                            n_prompt=23, chunk=7)
TINY_MOE = synth.Workload("tiny_test_moe", 2, 64, 4, 2, 32, 0, n_expert=8, n_expert_used=2,
                          expert_ffn_dim=32, kv_type="f16", n_prompt=19, chunk=5)


def fp32_layers(w: synth.Workload, gains: str = "random"):
    return [{name: synth.layer_weight(w, l, name, shp, gains=gains)
             for name, shp in synth.weight_shapes(w)} for l in range(w.n_layer)]


def q8_layers(w: synth.Workload, gains: str = "random"):
    return [oracle.quantize_layer(t) for t in fp32_layers(w, gains)]


def _encode_rows_blocked(t: np.ndarray, rows_per_block: int = 256) -> np.ndarray:
    """oracle.q8_0_encode_bytes over row blocks in a thread pool.  Each row is encoded on
    its own, so the bytes equal one call over the whole tensor; blocking keeps the
    working set in cache, which is what makes full-size layers take seconds."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    flat = t.reshape(-1, t.shape[-1])
    starts = range(0, flat.shape[0], rows_per_block)
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda s: oracle.q8_0_encode_bytes(flat[s:s + rows_per_block]), starts))
    out = np.concatenate(parts, axis=0)
    return out.reshape(t.shape[:-1] + (out.shape[-1],))


def q8_layer_full(w: synth.Workload, l: int, gains: str = "ones"):
    """Layer l of a full-size workload as interchange bytes, encoded by the oracle."""
    out = {}
    for name, shp in synth.weight_shapes(w):
        t = synth.layer_weight(w, l, name, shp, gains=gains)
        out[name] = t if name.endswith("_norm") else _encode_rows_blocked(t)
    return out
