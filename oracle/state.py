"""Layout-independent serialized KV state (oracle, test infrastructure only).

[split-psm] section "What this does" and [split-live] section "What this adds":
the sequence state is written in a layout-independent form, so the same bytes
restore into a cache laid out another way and the continuation is
byte-identical.  The pages do not print the format; this is the one the
library reads and writes (little-endian):

  bytes  0..3   magic "CPKV"
         4..7   u32 version = 1
         8..11  u32 kv_type (0 = f16, 1 = q8_0)
        12..15  u32 n_layer
        16..19  u32 n_kv_head
        20..23  u32 head_dim
        24..27  u32 n_tokens
        28..31  f32 rope_theta
  then for every layer l: K_l, then V_l, each n_tokens x n_kv_head rows in
  token-major order (t, h); an f16 row is head_dim binary16 values, a q8_0 row
  is head_dim/32 blocks of {fp16 d, int8 q[32]} (34 bytes).  K is stored after
  RoPE; positions are implicit (0 .. n_tokens-1).

size = 32 + n_layer * 2 * n_tokens * n_kv_head * row_bytes.
Pinned by: the size formula, a byte round trip, rejection of every mutated
header field.
"""
from __future__ import annotations

import struct

import numpy as np

from .q8_0 import q8_0_to_bytes, q8_0_from_bytes, QK

STATE_MAGIC = b"CPKV"
STATE_VERSION = 1
HEADER = struct.Struct("<4sIIIIIIf")
KV_CODE = {"f16": 0, "q8_0": 1}


def row_bytes(head_dim: int, kv_type: str) -> int:
    return head_dim * 2 if kv_type == "f16" else (head_dim // QK) * (2 + QK)


def state_size(n_layer: int, n_kv_head: int, head_dim: int, n_tokens: int, kv_type: str) -> int:
    return HEADER.size + n_layer * 2 * n_tokens * n_kv_head * row_bytes(head_dim, kv_type)


def _rows_to_bytes(stored, kv_type: str) -> bytes:
    if kv_type == "f16":
        return np.ascontiguousarray(stored, dtype="<f2").tobytes()
    d16, q = stored
    return np.ascontiguousarray(q8_0_to_bytes(d16, q)).tobytes()


def state_bytes(cache, rope_theta: float) -> bytes:
    """Serialize an OracleCache's first n_past tokens."""
    n = cache.n_past
    hdr = HEADER.pack(STATE_MAGIC, STATE_VERSION, KV_CODE[cache.kv_type], cache.n_layer,
                      cache.n_kv_head, cache.head_dim, n, float(rope_theta))
    parts = [hdr]
    for l in range(cache.n_layer):
        parts.append(_rows_to_bytes(cache.stored(l, "k", n), cache.kv_type))
        parts.append(_rows_to_bytes(cache.stored(l, "v", n), cache.kv_type))
    return b"".join(parts)


def parse_state(blob: bytes):
    """Split a blob into (header dict, list of (K_stored, V_stored) per layer)."""
    if len(blob) < HEADER.size:
        raise ValueError("short state")
    magic, ver, kvc, L, H, hd, n, theta = HEADER.unpack_from(blob, 0)
    if magic != STATE_MAGIC or ver != STATE_VERSION or kvc not in (0, 1):
        raise ValueError("bad state header")
    kv_type = "f16" if kvc == 0 else "q8_0"
    if hd % QK or state_size(L, H, hd, n, kv_type) != len(blob):
        raise ValueError("state length mismatch")
    rb = row_bytes(hd, kv_type)
    off = HEADER.size
    layers = []
    for _ in range(L):
        kv = []
        for _w in range(2):
            raw = np.frombuffer(blob, dtype=np.uint8, count=n * H * rb, offset=off)
            off += n * H * rb
            if kv_type == "f16":
                kv.append(raw.view("<f2").reshape(n, H, hd).astype(np.float16))
            else:
                d16, q = q8_0_from_bytes(raw.reshape(n, H, rb), hd // QK)
                kv.append((d16, q))
        layers.append(tuple(kv))
    hdr = dict(kv_type=kv_type, n_layer=L, n_kv_head=H, head_dim=hd, n_tokens=n, rope_theta=theta)
    return hdr, layers


def load_state(cache, blob: bytes):
    """Restore a parsed blob into an OracleCache (header must match the cache)."""
    hdr, layers = parse_state(blob)
    if (hdr["kv_type"], hdr["n_layer"], hdr["n_kv_head"], hdr["head_dim"]) != (
            cache.kv_type, cache.n_layer, cache.n_kv_head, cache.head_dim):
        raise ValueError("state does not match the cache")
    if hdr["n_tokens"] > cache.n_ctx:
        raise ValueError("state longer than the cache")
    for l, (k, v) in enumerate(layers):
        cache.set_stored(l, "k", k, hdr["n_tokens"])
        cache.set_stored(l, "v", v, hdr["n_tokens"])
    cache.n_past = hdr["n_tokens"]
    return hdr
