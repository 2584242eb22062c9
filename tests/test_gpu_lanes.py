"""prefill_chunks (several chunks in flight on several streams) against prefill_chunk in
turn (GPU).

With several lanes prefill_chunks takes the GEMM launch plans of a shared device; the
reference runs prefill_chunk per chunk under the same plans (cp_test_set_plan_shared).
Both then run the same kernels in the same launch plans on the same rows; only the order
in which chunks and layers overlap differs, and every cross-chunk dependency (a chunk's
layer reads the cache rows the previous chunk wrote at that layer) is ordered by events.
So outputs, n_past and the cache state must be bitwise equal, for dense and routed
layers, both cache types, two to eight lanes, chunk counts that are and are not a
multiple of the lane count, a ragged last chunk, a prompt that starts at a non-zero depth
and one that fits a single chunk.
"""
import pytest

import synth
from gpu_util import log, need_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


def gpu_layers(torch, cpa, w):
    out = []
    for l in range(w.n_layer):
        lw = {}
        for name, shape in synth.weight_shapes(w):
            t = synth.layer_weight(w, l, name, shape, backend="torch", device="cuda", gains="random")
            lw[name] = t if name.endswith("_norm") else cpa.cp_quantize_q8_0(t)
        out.append(lw)
    torch.cuda.synchronize()
    return out


def compare(torch, w, n, chunk, prefix=0, in_place=False, lanes=2):
    import chunked_prompt_prefill_amd as cpa
    layers = gpu_layers(torch, cpa, w)
    chunk = min(chunk, prefix + n)
    cfg = cpa.make_config(w, prefix + n, chunk)
    ref = cpa.PrefillContext(cfg, layers)
    ref.set_plan_shared(lanes > 1)
    lan = cpa.PrefillContext(cfg, layers, stream=torch.cuda.Stream())
    x = torch.from_numpy(synth.prompt_inputs(w, prefix + n)).cuda()
    torch.cuda.synchronize()          # x is read on the contexts' own streams
    if prefix:
        for c in (ref, lan):
            for s in range(0, prefix, chunk):
                c.prefill_chunk(x[s:min(prefix, s + chunk)])
    out_ref = torch.empty_like(x[prefix:])
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        ref.prefill_chunk(x[prefix + s:prefix + e], out_ref[s:e])
    if in_place:
        out = x[prefix:].clone()
        lan.prefill_chunks(out, out, chunk, lanes)
    else:
        out = lan.prefill_chunks(x[prefix:], None, chunk, lanes)
    torch.cuda.synchronize()
    same = torch.equal(out, out_ref)
    log(f"  {w.name} n={n} chunk={chunk} prefix={prefix} in_place={in_place} lanes={lanes}: "
        f"bitwise equal {same}")
    assert same
    assert lan.n_past == ref.n_past == prefix + n
    assert lan.kv_cache_get_state() == ref.kv_cache_get_state()
    ref.close()
    lan.close()
    return out


@pytest.mark.parametrize("kv,lanes", [("f16", 2), ("q8_0", 2), ("f16", 3)])
def test_lanes_equal_sequential_dense(torch, kv, lanes):
    """Two layers of the 27B-class dense shapes: 5 chunks of 512 and a ragged sixth."""
    w = synth.WORKLOADS["dense27b_sweep"].with_(n_layer=2, kv_type=kv)
    compare(torch, w, 5 * 512 + 137, 512, lanes=lanes)


def test_shared_plans_agree_with_single_lane_plans(torch):
    """The shared-device plans (fewer K splits) change only the order of the split-K sums:
    three lanes against prefill_chunk per chunk under the single-lane plans, two layers of
    the dense shapes, to max|d|/max|ref| <= 1e-3."""
    import numpy as np
    w = synth.WORKLOADS["dense27b_sweep"].with_(n_layer=2)
    got = compare(torch, w, 4 * 512, 512, lanes=3).cpu().numpy()
    single = compare(torch, w, 4 * 512, 512, lanes=1).cpu().numpy()
    e = float(np.max(np.abs(got - single)) / np.max(np.abs(single)))
    log(f"  shared against single-lane plans: max rel diff {e:.3e}")
    assert 0 < e <= 1e-3      # (0 would mean the plans did not differ)


def test_lanes_equal_sequential_routed_experts(torch):
    """Two routed-expert layers: 4 chunks of 384 (an even count) after a 100-token prefix."""
    w = synth.WORKLOADS["moe_a3b"].with_(n_layer=2)
    compare(torch, w, 4 * 384, 384, prefix=100)


def test_lanes_small_shapes_in_place_and_single_chunk(torch):
    """The tiny decoder: chunks of 7 (odd count), in place, after a prefix; and a prompt of
    one chunk."""
    w = synth.WORKLOADS["tiny_dense"]
    compare(torch, w.with_(kv_type="q8_0"), 23, 7, prefix=9, in_place=True)
    compare(torch, w, 5, 7)


@pytest.mark.parametrize("lanes,n", [(1, 30), (4, 30), (8, 29), (8, 21)])
def test_lanes_count(torch, lanes, n):
    """The tiny decoder in 4-token chunks after a 5-token prefix: one lane; four lanes over
    eight chunks (a ragged last one); eight lanes over eight chunks and over six."""
    w = synth.WORKLOADS["tiny_dense"]
    compare(torch, w, n, 4, prefix=5, lanes=lanes)


def test_lanes_refuse_before_enqueue(torch):
    """A chunk above n_chunk_max, a prompt past n_ctx_max, a lane count outside 1 .. 8, the
    context's own stream as a lane stream and one stream given to two lanes are refused;
    n_past and the cache are unchanged."""
    import ctypes
    import chunked_prompt_prefill_amd as cpa
    from chunked_prompt_prefill_amd._lib import CP_E_CAPACITY, CP_E_INVALID
    w = synth.WORKLOADS["tiny_dense"]
    layers = gpu_layers(torch, cpa, w)
    ctx = cpa.PrefillContext(cpa.make_config(w, 32, 8), layers)
    x = torch.from_numpy(synth.prompt_inputs(w, 40)).cuda()
    ctx.prefill_chunk(x[:8])
    blob = ctx.kv_cache_get_state()
    out = torch.empty_like(x)
    ws = [torch.empty_like(ctx.ws) for _ in range(8)]
    st = [torch.cuda.Stream() for _ in range(8)]
    L = ctx.L

    def call(n, chunk, lanes, streams):
        arr = ctypes.c_void_p * 8
        return L.prefill_chunks(ctx._ctx, x.data_ptr(), out.data_ptr(), n, chunk, lanes,
                                arr(*[t.data_ptr() for t in ws]), arr(*streams))

    ok = [s.cuda_stream for s in st]
    own = torch.cuda.current_stream().cuda_stream
    assert call(16, 9, 2, ok) == CP_E_CAPACITY
    assert call(25, 8, 2, ok) == CP_E_CAPACITY
    assert call(8, 8, 0, ok) == CP_E_INVALID
    assert call(8, 8, 9, ok) == CP_E_INVALID
    assert call(8, 8, 2, [own] + ok[1:]) == CP_E_INVALID
    assert call(16, 4, 3, [ok[0], ok[0]] + ok[2:]) == CP_E_INVALID
    assert ctx.n_past == 8
    assert ctx.kv_cache_get_state() == blob
    # and it still works afterwards
    assert call(16, 8, 2, ok) == 0
    torch.cuda.synchronize()
    assert ctx.n_past == 24
    assert bool(torch.isfinite(out[:16]).all())
    ctx.close()
