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
