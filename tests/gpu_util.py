"""Helpers for the GPU tests: device checks and running the library on oracle-encoded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_prompt_prefill_amd as cpa  # raises ImportError if the library is not built
    cpa.lib()
    return torch


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def cache_row_bytes(stored, kv_type: str) -> np.ndarray:
    """Serialized row bytes [n][Hkv][row_bytes] of the oracle's stored cache rows."""
    import oracle
    if kv_type == "f16":
        a = np.ascontiguousarray(stored, dtype="<f2")
        return a.view(np.uint8).reshape(a.shape[0], a.shape[1], -1)
    d16, q = stored
    return oracle.q8_0_to_bytes(d16, q)


def run_prefill(torch, w, qlayers, x: np.ndarray, chunk: int, n_ctx: int = None, trace=False):
    """Run the HIP path over the prompt x in chunks; returns (out, ctx[, layer_out, routes])."""
    import chunked_prompt_prefill_amd as cpa
    n = x.shape[0]
    cfg = cpa.make_config(w, n_ctx or n, min(chunk, n_ctx or n))
    dev = [cpa.to_device(l) for l in qlayers]
    ctx = cpa.PrefillContext(cfg, dev)
    del dev
    xin = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.empty_like(xin)
    lo = ro = None
    if trace:
        lo = torch.empty((w.n_layer, n, w.d_model), dtype=torch.float32, device="cuda")
        if w.n_expert:
            ro = torch.empty((w.n_layer, n, w.n_expert_used), dtype=torch.int32, device="cuda")
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        if trace:
            ctx.prefill_chunk_trace(xin[s:e], out[s:e],
                                    None if lo is None else lo[:, s:e], n * w.d_model,
                                    None if ro is None else ro[:, s:e],
                                    n * w.n_expert_used if ro is not None else 0)
        else:
            ctx.prefill_chunk(xin[s:e], out[s:e])
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if trace:
        return (res, ctx, lo.cpu().numpy(), None if ro is None else ro.cpu().numpy())
    return res, ctx


# A GPU expert set may differ from the oracle's only where the oracle's own k-th and
# (k+1)-th router logits are closer than this fraction of max|r| (a near tie that the
# 16-bit-level difference of the router input can flip).
ROUTE_TIE = 1e-3


def routing_agreement(r: np.ndarray, own: np.ndarray, got: np.ndarray, tie: float = ROUTE_TIE):
    """Compare the GPU's expert sets `got` [T][k] with the oracle's `own` for the oracle's
    logits r [T][E].  Asserts that every row whose set differs sits at a near tie of the
    oracle's logits and that the GPU's set is still a top-k set there up to the same margin;
    returns the boolean mask of rows whose sets agree."""
    k = own.shape[1]
    same = np.all(np.sort(own, 1) == np.sort(got, 1), axis=1)
    tol = tie * float(np.max(np.abs(r)))
    if not same.all():
        srt = -np.sort(-np.asarray(r, np.float64), axis=1)
        near = srt[:, k - 1] - srt[:, k] < tol if k < r.shape[1] else np.ones(len(r), bool)
        mask = np.zeros(r.shape, bool)
        np.put_along_axis(mask, got.astype(np.int64), True, axis=1)
        gap = np.where(mask, -np.inf, r).max(axis=1) - np.where(mask, r, np.inf).min(axis=1)
        assert np.all(near[~same]), "an expert set differs away from a near tie"
        assert np.all(gap[~same] <= tol)
    return same
