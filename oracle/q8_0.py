"""q8_0 block quantisation (oracle, test infrastructure only).

The pages name q8_0 as a device-resident cache type ([split-psm], section
"Why": the 58.3k-token prompt is run "with a q8_0 device-resident cache") and
the workloads store weights as q8_0: blocks of 32 int8 values sharing one fp16
scale.  The pages do not spell out the encode rule; this is the plain q8_0
definition:

    amax = max |x_j| over the 32 values of the block
    d    = amax / 127                 (float32, correctly rounded)
    id   = 1 / d  if d != 0 else 0    (float32)
    q_j  = round_half_away_from_zero(x_j * id)     (x_j * id in float32)
    stored scale = fp16(d)  (IEEE round-to-nearest-even, subnormals kept)

    decode: x_hat_j = float32(fp16 d) * q_j       (exact in float32)

q uses the unrounded float32 d.  |q| <= 127 always (-128 never occurs).
Interchange bytes of one block: little-endian fp16 d, then int8 q[32] (34 B).

Pinned by: a scalar pure-Python re-derivation with explicit float32 rounding
per operation (tests), tie vectors (2.5 -> 3, -0.5 -> -1), the all-zero block,
subnormal scales, the round-trip error bound and encode(decode(encode(x))) ==
encode(x).
"""
from __future__ import annotations

import numpy as np

QK = 32
BLOCK_BYTES = 2 + QK


def _round_half_away(v32: np.ndarray) -> np.ndarray:
    # float32 -> float64 is exact and |v| + 0.5 is exact in float64 for |v| < 2**29,
    # so trunc(v + copysign(0.5, v)) rounds half away from zero with no double rounding.
    v = v32.astype(np.float64)
    return np.trunc(v + np.copysign(0.5, v))


def q8_0_encode(x) -> tuple[np.ndarray, np.ndarray]:
    """Encode rows of float32 values into q8_0.

    x: [..., K] (any float; cast to float32 first).  K is zero-padded to a
    multiple of 32 (padding changes neither amax nor any real value's code).
    Returns (d16 [..., K/32] float16, q [..., K/32, 32] int8).
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    Kp = -(-K // QK) * QK
    if Kp != K:
        pad = np.zeros(x.shape[:-1] + (Kp - K,), dtype=np.float32)
        x = np.concatenate([x, pad], axis=-1)
    xb = x.reshape(x.shape[:-1] + (Kp // QK, QK))
    amax = np.max(np.abs(xb), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (xb * inv[..., None]).astype(np.float32)
    q = _round_half_away(v)
    q = np.clip(q, -127, 127).astype(np.int8)
    return d.astype(np.float16), q


def q8_0_decode(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """float32 values [..., K/32 * 32] from (d16 [..., nb], q [..., nb, 32])."""
    v = d16.astype(np.float32)[..., None] * q.astype(np.float32)
    return v.reshape(v.shape[:-2] + (v.shape[-2] * QK,))


def q8_0_to_bytes(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Interchange bytes [..., nb * 34]: per block fp16 d (little-endian) then 32 int8."""
    nb = d16.shape[-1]
    out = np.empty(d16.shape + (BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0:2] = d16.astype("<f2").view(np.uint8).reshape(d16.shape + (2,))
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(d16.shape[:-1] + (nb * BLOCK_BYTES,))


def q8_0_from_bytes(b: np.ndarray, nb: int) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of q8_0_to_bytes: bytes [..., nb*34] -> (d16 [..., nb], q [..., nb, 32])."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    blk = b.reshape(b.shape[:-1] + (nb, BLOCK_BYTES))
    d16 = np.ascontiguousarray(blk[..., 0:2]).view("<f2").reshape(blk.shape[:-1]).astype(np.float16)
    q = np.ascontiguousarray(blk[..., 2:]).view(np.int8)
    return d16, q


def q8_0_encode_bytes(x) -> np.ndarray:
    """float32 [..., K] -> interchange bytes [..., ceil(K/32) * 34]."""
    d16, q = q8_0_encode(x)
    return q8_0_to_bytes(d16, q)


def q8_0_decode_bytes(b: np.ndarray, K: int) -> np.ndarray:
    """Interchange bytes [..., nb*34] -> float32 [..., K] (padding dropped)."""
    nb = -(-K // QK)
    d16, q = q8_0_from_bytes(b, nb)
    return q8_0_decode(d16, q)[..., :K]
