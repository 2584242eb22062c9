"""prefill_chunk_static, the chunk call that allocates nothing, against prefill_chunk (GPU).

Two contexts over the same weights run the same chunks, one through prefill_chunk (its
per-chunk buffers in the context's workspace) and one through prefill_chunk_static (the
same buffers in the library's static device array).  Both enqueue the same kernels in the
same launch plans on identical inputs, so outputs and caches must be bitwise equal.  Two
calls in a row, the second with a smaller chunk, so the second reuses the array with
smaller buffers after the first left its contents there.  A chunk whose buffers exceed the
array is refused before anything is enqueued, and the context stays usable.
"""
import numpy as np
import pytest

import synth
from gpu_util import log, need_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]


@pytest.fixture(scope="module")
def torch():
    return need_gpu()


def gpu_layers(torch, cpa, w):
    """w's layers generated and q8_0-encoded on the GPU (norm gains random)."""
    out = []
    for l in range(w.n_layer):
        lw = {}
        for name, shape in synth.weight_shapes(w):
            t = synth.layer_weight(w, l, name, shape, backend="torch", device="cuda", gains="random")
            lw[name] = t if name.endswith("_norm") else cpa.cp_quantize_q8_0(t)
        out.append(lw)
    torch.cuda.synchronize()
    return out


def run_pair(torch, w, chunks, n_chunk_max, n_ctx):
    """The chunk sizes `chunks` through prefill_chunk and through prefill_chunk_static on two
    fresh contexts; asserts bitwise equal outputs, n_past and cache state after every call."""
    import chunked_prompt_prefill_amd as cpa
    layers = gpu_layers(torch, cpa, w)
    cfg = cpa.make_config(w, n_ctx, n_chunk_max)
    ref_ctx = cpa.PrefillContext(cfg, layers)
    new_ctx = cpa.PrefillContext(cfg, layers)
    n = sum(chunks)
    x = torch.from_numpy(synth.prompt_inputs(w, n)).cuda()
    s = 0
    for C in chunks:
        ref = ref_ctx.prefill_chunk(x[s:s + C])
        got = new_ctx.prefill_chunk_static(x[s:s + C])
        torch.cuda.synchronize()
        assert new_ctx.n_past == ref_ctx.n_past == s + C
        assert bool(torch.isfinite(ref).all())
        same = torch.equal(got, ref)
        diff = float((got - ref).abs().max() / ref.abs().max())
        log(f"  {w.name}: chunk of {C} at depth {s}: bitwise equal {same}, max rel diff {diff:.3e}")
        assert same
        assert new_ctx.kv_cache_get_state() == ref_ctx.kv_cache_get_state()
        s += C
    ref_ctx.close()
    new_ctx.close()
    del layers
    torch.cuda.empty_cache()


def test_static_chunk_equals_prefill_chunk_dense(torch):
    """Two layers of the 27B-class dense shapes (split-K GEMMs, deferred partial sums):
    512 rows, then 200, then decode-sized chunks of 3 and 1 (weight-streaming GEMMs, the
    one-launch RoPE + append)."""
    w = synth.WORKLOADS["dense27b_sweep"].with_(n_layer=2)
    run_pair(torch, w, [512, 200, 3, 1], n_chunk_max=512, n_ctx=1024)


def test_static_chunk_equals_prefill_chunk_q8_0_cache_and_routed_experts(torch):
    """Two routed-expert layers with a q8_0 cache (router, permute, grouped GEMMs, split-KV
    attention at depth): 384 rows, then 97."""
    w = synth.WORKLOADS["moe_a3b"].with_(n_layer=2, kv_type="q8_0")
    run_pair(torch, w, [384, 97], n_chunk_max=512, n_ctx=4096)


def test_static_chunk_refuses_a_chunk_beyond_the_array(torch):
    """A 2048-row chunk of the dense shapes needs more than the 256 MiB array: refused with
    CP_E_CAPACITY, nothing enqueued, n_past unchanged; a 256-row chunk on the same context
    then runs and equals prefill_chunk's."""
    import chunked_prompt_prefill_amd as cpa
    w = synth.WORKLOADS["dense27b_sweep"].with_(n_layer=1)
    layers = gpu_layers(torch, cpa, w)
    cfg = cpa.make_config(w, 4096, 2048)
    ctx = cpa.PrefillContext(cfg, layers)
    ref_ctx = cpa.PrefillContext(cfg, layers)
    x = torch.from_numpy(synth.prompt_inputs(w, 2048)).cuda()
    out = torch.empty_like(x)
    with pytest.raises(cpa.PrefillError) as ei:
        ctx.prefill_chunk_static(x, out)
    from chunked_prompt_prefill_amd._lib import CP_E_CAPACITY
    assert ei.value.code == CP_E_CAPACITY
    assert "static scratch" in str(ei.value)
    assert ctx.n_past == 0
    got = ctx.prefill_chunk_static(x[:256])
    ref = ref_ctx.prefill_chunk(x[:256])
    torch.cuda.synchronize()
    assert ctx.n_past == 256
    assert torch.equal(got, ref)
    ctx.close()
    ref_ctx.close()
