"""Final hidden states at full depth: every layer of each large workload's share (GPU).

The acceptance of chunked prefill on the planner page is that chunked equals a single
pass on the model's output ("refactor: one prefill planner and one pad-trim hook for CLI
and server", section "Acceptance Criteria").  Here the GPU runs the first chunks of each
workload's prompt through all of its layers at the real shapes and chunk size, and the
oracle runs the same rows layer-major through the same layers.  By causality (a row
attends only to positions at or before its own) the outputs of a prompt prefix are
final, so the prefix's last-layer rows are the prompt's final hidden states there and
are compared element by element: max|delta| / max|ref| <= 1e-2 over the whole prefix.
Every layer's weights are encoded by the oracle; both sides receive the same bytes.
The per-layer errors are logged to show how the error grows with depth.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, need_gpu, rel_err, routing_agreement
from model_inputs import q8_layer_full

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

TOL = 1e-2

_ENCODED = {}


def oracle_layers(w):
    """All layers of w as oracle-encoded interchange bytes (norm gains all ones), kept for
    the module: workloads with the same shapes share their layers."""
    out = []
    for l in range(w.n_layer):
        key = (w.d_model, w.n_head, w.n_kv_head, w.head_dim, w.ffn_dim, w.n_expert,
               w.expert_ffn_dim, l)
        if key not in _ENCODED:
            _ENCODED[key] = q8_layer_full(w, l)
            log(f"  layer {l} encoded by the oracle")
        out.append(_ENCODED[key])
    return out


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


def gpu_prefix(torch, w, layers, x, chunks):
    """The prefix through every layer on the GPU, chunk by chunk (one context per chunk
    size); returns {chunk: (final rows, per-layer rows, per-layer expert indices)}."""
    import chunked_prompt_prefill_amd as cpa
    n = x.shape[0]
    dev = [cpa.to_device(l) for l in layers]
    xd = torch.from_numpy(x).cuda()
    res = {}
    for C in chunks:
        ctx = cpa.PrefillContext(cpa.make_config(w, n, C), dev)
        out = torch.empty_like(xd)
        lo = torch.empty((w.n_layer, n, w.d_model), dtype=torch.float32, device="cuda")
        ro = torch.empty((w.n_layer, n, w.n_expert_used), dtype=torch.int32, device="cuda") \
            if w.n_expert else None
        for s in range(0, n, C):
            e = min(n, s + C)
            ctx.prefill_chunk_trace(xd[s:e], out[s:e], lo[:, s:e], n * w.d_model,
                                    None if ro is None else ro[:, s:e],
                                    n * w.n_expert_used if ro is not None else 0)
        torch.cuda.synchronize()
        assert ctx.n_past == n
        res[C] = (out.cpu().numpy(), lo.cpu().numpy(), None if ro is None else ro.cpu().numpy())
        ctx.close()
        del out, lo, ro
    del dev, xd
    torch.cuda.empty_cache()
    return res


def oracle_run(w, layers, x, operands):
    """The oracle's layer-major driver over x, one layer at a time (progress is logged);
    returns (per-layer outputs, per-layer routing)."""
    m = oracle.OracleModel(w, layers, keep_layers=1, operands=operands)
    ref_lo, routing = [], []
    cache = m.new_cache(x.shape[0])
    ref = np.asarray(x, dtype=np.float64)
    for l in range(w.n_layer):
        ref = m.layer(l, ref, cache, 0, routing if w.n_expert else None)
        ref_lo.append(ref)
        log(f"  oracle ({operands} operands) layer {l} done")
    return ref_lo, routing


def compare(w, name, ref_lo, routing, out, lo, ro):
    """Per-layer and final max|d|/max|ref| of the GPU rows against one oracle run (rows
    whose expert set differs at a near tie left out); returns the final error."""
    agree = np.ones(out.shape[0], bool)
    errs = []
    for l in range(w.n_layer):
        if ro is not None:
            r, own, _ = routing[l]
            same = routing_agreement(r, own, ro[l])
            if not same.all():
                log(f"  {name}, layer {l}: {int((~same).sum())} near-tie expert sets differ")
            agree &= same
        errs.append(rel_err(lo[l][agree], ref_lo[l][agree]))
    log(f"  vs {name}: max rel err per layer " + " ".join(f"{e:.2e}" for e in errs))
    e = rel_err(out[agree], ref_lo[-1][agree])
    log(f"  vs {name}: final hidden states over {int(agree.sum())}/{len(agree)} rows: {e:.3e}")
    return e


def check_full_depth(w, layers, x, gpu):
    """The GPU rows against two oracle runs.  "f16" (every matrix-product operand rounded
    to binary16, exact accumulation: the arithmetic the library states) must agree to
    1e-2.  "exact" (float64 throughout) must agree to 1e-2 with an f16 cache; with a q8_0
    cache, whose codes are decided from those products, the two oracle runs themselves
    drift apart with depth (a 16-bit-level difference moves a value across a code
    boundary, a change of one code step, 1/127 of the block's amax), and the GPU may
    deviate from the exact run by at most twice as much as the f16 run does."""
    log(f"  oracle: {w.n_layer} layers layer-major over {x.shape[0]} rows, both operand modes")
    exact_lo, exact_routing = oracle_run(w, layers, x, "exact")
    f16_lo, f16_routing = oracle_run(w, layers, x, "f16")
    drift = rel_err(f16_lo[-1], exact_lo[-1])
    log(f"  oracle f16 operands vs exact: final {drift:.3e}")
    for C, (out, lo, ro) in gpu.items():
        log(f"  chunk {C}:")
        assert np.array_equal(out, lo[-1])
        e16 = compare(w, "f16-operand oracle", f16_lo, f16_routing, out, lo, ro)
        ex = compare(w, "exact oracle", exact_lo, exact_routing, out, lo, ro)
        assert e16 < TOL
        if w.kv_type == "f16":
            assert ex < TOL
        else:
            assert ex < max(TOL, 2.0 * drift)


def test_dense27b_f16_final_hidden_states(torch):
    """16 layers, f16 cache: the first 1,536 prompt rows in three 512-token chunks."""
    w = synth.WORKLOADS["dense27b_f16"]
    n = 3 * w.chunk
    log(f"{w.name}: {w.n_layer} layers, {n} rows in chunks of {w.chunk}")
    layers = oracle_layers(w)
    x = synth.prompt_inputs(w, n)
    check_full_depth(w, layers, x, gpu_prefix(torch, w, layers, x, [w.chunk]))


def test_dense27b_q8_0_final_hidden_states(torch):
    """16 layers, q8_0 cache: the first 4,096 prompt rows in two 2048-token chunks."""
    w = synth.WORKLOADS["dense27b_q8"]
    n = 2 * w.chunk
    log(f"{w.name}: {w.n_layer} layers, {n} rows in chunks of {w.chunk}")
    layers = oracle_layers(w)
    x = synth.prompt_inputs(w, n)
    check_full_depth(w, layers, x, gpu_prefix(torch, w, layers, x, [w.chunk]))


def test_sweep_shapes_final_hidden_states_at_several_chunk_sizes(torch):
    """The sweep's 4 layers: a 4,096-row prompt read in chunks of 128, 1024 and 4096
    (three launch plans, from the weight-bound end to the largest), one oracle run for
    all three (the result does not depend on the chunk size)."""
    w = synth.WORKLOADS["dense27b_sweep"]
    n = 4096
    log(f"{w.name}: {w.n_layer} layers, {n} rows in chunks of 128, 1024, 4096")
    layers = oracle_layers(w)
    x = synth.prompt_inputs(w, n)
    check_full_depth(w, layers, x, gpu_prefix(torch, w, layers, x, [128, 1024, 4096]))


def test_moe_final_hidden_states(torch):
    """8 routed-expert layers: the first 6,656 prompt rows in two 3328-token chunks."""
    w = synth.WORKLOADS["moe_a3b"]
    n = 2 * w.chunk
    log(f"{w.name}: {w.n_layer} layers, {n} rows in chunks of {w.chunk}")
    layers = oracle_layers(w)
    x = synth.prompt_inputs(w, n)
    check_full_depth(w, layers, x, gpu_prefix(torch, w, layers, x, [w.chunk]))
