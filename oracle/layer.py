"""Per-layer arithmetic of a decoder layer (oracle, test infrastructure only).

The pages measure prefill of decoder transformers whose per-layer math they do
not print; each function below is the plain textbook definition, float64
unless the step writes stored bytes or decides integers (then float32, one
rounding per operation).  Readings taken where the pages are silent:
  * RMSNorm with the epsilon inside the square root.
  * RoPE in the NeoX "rotate-half" pairing (x_i, x_{i+hd/2}) over the whole head,
    theta**(-2i/hd) frequencies, absolute positions from 0, angles in float64,
    cos/sin rounded to float32.
  * The chunk's own K/V enter attention after the cache conversion ("append,
    then attend"): attention always reads the cache as stored (f16 or q8_0).
  * Causal mask j <= position of the query; GQA head h reads kv head h // G.
  * Routed experts: top-k by router logit (ties to the lower expert index),
    weights = softmax over the k selected logits, contributions summed in rank
    order; no shared expert, no capacity limit.
"""
from __future__ import annotations

import math

import numpy as np

from .q8_0 import q8_0_encode, q8_0_decode, QK


# ---------------------------------------------------------------------------------------
# fp16 operands
# ---------------------------------------------------------------------------------------

F16_MAX = 65504.0


def to_f16(x: np.ndarray, saturate: bool = False) -> np.ndarray:
    """Values rounded to IEEE binary16 (round to nearest, ties to even), returned as
    float64.  saturate: clamp to +-65504 first (the largest finite binary16).

    Used by the oracle's "f16 operands" mode: every matrix-product operand is rounded to
    binary16 and the products are then accumulated exactly (float64), the arithmetic the
    library states for its matrix products.  Pinned by: hand-picked ties and boundaries
    (1 + 2^-11 -> 1, 1 + 3*2^-11 -> 1 + 2^-9, 65519 -> 65504, 65520 -> inf, saturated
    -> 65504), and agreement with the bit patterns of the float16 type.
    """
    x = np.asarray(x, dtype=np.float64)
    if saturate:
        x = np.clip(x, -F16_MAX, F16_MAX)
    return x.astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma over the last axis (float64).

    Pinned by: the closed form on constant rows, unit output RMS for gamma = 1,
    invariance to positive scaling of x.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# ---------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------

def rope_table(n_pos: int, head_dim: int, theta: float, start: int = 0):
    """float32 cos/sin tables [n_pos][head_dim/2] for positions start .. start+n_pos-1.

    omega_i = theta ** (-2 i / head_dim), angle = p * omega_i, all in float64
    (C library pow/cos/sin), then cos and sin rounded to float32.
    Pinned by: position 0 gives cos 1 / sin 0; agreement with an independent
    NumPy float64 evaluation to within one float32 ulp.
    """
    half = head_dim // 2
    omega = [math.pow(float(theta), -2.0 * i / head_dim) for i in range(half)]
    c = np.empty((n_pos, half), dtype=np.float32)
    s = np.empty((n_pos, half), dtype=np.float32)
    for i, w in enumerate(omega):
        ang = [(start + p) * w for p in range(n_pos)]
        c[:, i] = np.array([math.cos(a) for a in ang], dtype=np.float64).astype(np.float32)
        s[:, i] = np.array([math.sin(a) for a in ang], dtype=np.float64).astype(np.float32)
    return c, s


def rope_apply_f32(x: np.ndarray, cos32: np.ndarray, sin32: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE in float32 with one rounding per operation (no fused multiply-add).

    x: [n][heads][hd] float32; cos32/sin32: [n][hd/2] float32 (rows = positions of x).
        out_i        = x_i * c_i - x_{i+hd/2} * s_i
        out_{i+hd/2} = x_{i+hd/2} * c_i + x_i * s_i
    This is the precision the rows written to the cache are decided in.
    Pinned by: position 0 is the identity; agreement with the float64 rotation
    to float32 rounding; the relative-position identity (via rope_apply).
    """
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    c = cos32[:, None, :].astype(np.float32)
    s = sin32[:, None, :].astype(np.float32)
    a, b = x[..., :h], x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = (a * c) - (b * s)
    out[..., h:] = (b * c) + (a * s)
    return out


def rope_apply(x: np.ndarray, positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """float64 rotate-half RoPE with float64 cos/sin (used to pin the rotation itself)."""
    x = np.asarray(x, dtype=np.float64)
    h = head_dim // 2
    i = np.arange(h, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------------------
# KV cache rows
# ---------------------------------------------------------------------------------------

def cache_encode_rows(rows32: np.ndarray, kv_type: str):
    """Convert float32 rows [n][n_kv_head][hd] to the cache's stored form.

    f16: IEEE round-to-nearest-even (subnormals kept) -> float16 array.
    q8_0: one q8_0 block per 32 values of each (token, kv head) row -> (d16, q).
    """
    rows32 = np.asarray(rows32, dtype=np.float32)
    if kv_type == "f16":
        return rows32.astype(np.float16)
    if kv_type == "q8_0":
        return q8_0_encode(rows32)
    raise ValueError(kv_type)


def cache_decode_rows(stored, kv_type: str) -> np.ndarray:
    """Stored cache rows -> float32 values [n][n_kv_head][hd]."""
    if kv_type == "f16":
        return np.asarray(stored).astype(np.float32)
    d16, q = stored
    return q8_0_decode(d16, q)


# ---------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: np.ndarray,
              block: int = 512, p_f16: bool = False) -> np.ndarray:
    """Causal GQA softmax attention (float64).

    q: [n][Hq][hd]; K, V: [T][Hkv][hd] (cache values, position = row index);
    positions: [n] absolute position of each query row.  Query row i of head h
    attends keys j <= positions[i] of kv head h // (Hq/Hkv):
        s_j = q_i . K_j / sqrt(hd),  P = softmax(s) (max subtracted),  o_i = sum_j P_j V_j
    p_f16: the unnormalised weights exp(s_j - max) are rounded to binary16 (the operand of
    the P.V product) and the row is normalised by the sum of the rounded weights.
    Pinned by: brute-force scalar loops on tiny inputs, a single visible key
    returning its value row, causality, duplicated KV heads = multi-head; with p_f16,
    scores at multiples of ln 2 (weights exact powers of two) give the exact result, and
    random scores stay within binary16 rounding of it.
    """
    q = np.asarray(q, dtype=np.float64)
    n, Hq, hd = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    pos = np.asarray(positions, dtype=np.int64)
    out = np.empty((n, Hq, hd), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    T = int(pos.max()) + 1 if n else 0
    K64 = np.asarray(K[:T], dtype=np.float64)
    V64 = np.asarray(V[:T], dtype=np.float64)
    jj = np.arange(T)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        Tb = int(pos[r0:r1].max()) + 1
        mask = jj[None, :Tb] > pos[r0:r1, None]
        for h in range(Hq):
            g = h // G
            s = (q[r0:r1, h, :] @ K64[:Tb, g, :].T) * scale
            s[mask] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            if p_f16:
                p = to_f16(p)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r1, h, :] = p @ V64[:Tb, g, :]
    return out


# ---------------------------------------------------------------------------------------
# FFN
# ---------------------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(y: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
               block: int = 2048, h_f16: bool = False) -> np.ndarray:
    """(silu(y Wg^T) * (y Wu^T)) Wd^T in float64, evaluated in row blocks.

    Wg, Wu: [F][d]; Wd: [d][F].  h_f16: the intermediate h (the down projection's
    operand) is saturated to +-65504 and rounded to binary16.  Pinned by: the closed form
    on a tiny example, silu(0) = 0.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.empty((y.shape[0], Wd.shape[0]), dtype=np.float64)
    for r0 in range(0, y.shape[0], block):
        yb = y[r0:r0 + block]
        h = silu(yb @ Wg.T) * (yb @ Wu.T)
        if h_f16:
            h = to_f16(h, saturate=True)
        out[r0:r0 + block] = h @ Wd.T
    return out


# ---------------------------------------------------------------------------------------
# Routed experts
# ---------------------------------------------------------------------------------------

def router_logits_ordered(y32: np.ndarray, d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Router logits in float32 with a fixed operation order.

    y32: [T][d] float32 (the RMSNorm output); router weights as q8_0
    (d16 [E][d/32], q [E][d/32][32]).  For every (t, e):
        P_b = sum_{j = 0..31, ascending} float(q_{e,b,j}) * y_{t, 32b+j}
        r   = sum_{b ascending} float(d_{e,b}) * P_b
    every product and every sum rounded to float32 separately (no fused
    multiply-add); both sums start from the first term.  This order is what
    makes the selected expert indices reproducible bit for bit.
    Pinned by: a scalar pure-Python evaluation with explicit float32 rounding.
    """
    y32 = np.asarray(y32, dtype=np.float32)
    T = y32.shape[0]
    E, nb = d16.shape
    qf = q.astype(np.float32)
    df = d16.astype(np.float32)
    acc = np.zeros((T, E), dtype=np.float32)
    for b in range(nb):
        P = (y32[:, b * QK][:, None] * qf[None, :, b, 0]).astype(np.float32)
        for j in range(1, QK):
            P = P + (y32[:, b * QK + j][:, None] * qf[None, :, b, j])
        term = (df[None, :, b] * P).astype(np.float32)
        acc = term if b == 0 else (acc + term).astype(np.float32)
    return acc


def moe_route(r32: np.ndarray, k: int):
    """Top-k experts per token and their weights.

    Ranked by logit, descending; equal logits rank the lower expert index first.
    Weights: softmax over the k selected logits (float64).
    Returns (idx [T][k] int32, w [T][k] float64).
    Pinned by: a brute-force full sort per row; a dominant logit gives weight ~1;
    k = 1 gives weight exactly 1.
    """
    r32 = np.asarray(r32, dtype=np.float32)
    order = np.argsort(-r32.astype(np.float64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(r32, idx, axis=1).astype(np.float64)
    sel = sel - sel.max(axis=1, keepdims=True)
    e = np.exp(sel)
    w = e / e.sum(axis=1, keepdims=True)
    return idx, w


def moe_ffn(y: np.ndarray, idx: np.ndarray, w: np.ndarray, Wg: np.ndarray, Wu: np.ndarray,
            Wd: np.ndarray, h_f16: bool = False) -> np.ndarray:
    """sum_{rank 0..k-1} w[t,rank] * FFN_{idx[t,rank]}(y_t), summed in rank order (float64).

    Wg, Wu: [E][Fe][d]; Wd: [E][d][Fe].  Pinned by: E identical experts reduce
    to the dense SwiGLU FFN.
    """
    y = np.asarray(y, dtype=np.float64)
    T, k = idx.shape
    out = np.zeros((T, Wd.shape[1]), dtype=np.float64)
    for rank in range(k):
        contrib = np.zeros_like(out)
        col = idx[:, rank]
        for e in np.unique(col):
            rows = np.nonzero(col == e)[0]
            contrib[rows] = swiglu_ffn(y[rows], Wg[e], Wu[e], Wd[e], h_f16=h_f16)
        out = out + w[:, rank][:, None] * contrib
    return out
