"""A stack of layers as one decode step (stack_decode_paged): each layer has
its own weights and cache over the same sequences and block tables.  The
oracle runs the layers one after another with the activations between them
rounded to bf16 (the layer interface's dtype), and the GPU stack must match
its last output within the bf16 bar; a captured graph of the whole step must
replay bit for bit."""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from harness import compare, gpu_setup, run_oracle
from test_gpu_graph import replay_matches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def stack_inputs(wl, n_layers, ctx, seed):
    """Per layer: inputs sharing the sequences and tables of layer 0, with
    their own weights and cached K/V; x of layer 0 only."""
    base = synth.make_inputs(wl, seed=seed, decode_batch=len(ctx), decode_ctx=ctx)
    shape, b = wl.shape, base.batch
    out = [base]
    for l in range(1, n_layers):
        rng = np.random.default_rng(seed * 100 + l)
        w = synth.make_weights(shape, rng=rng)
        kv = synth.cached_kv(rng, int(b.ctx_len.sum()), shape.n_kv_heads, shape.head_dim,
                             bf16=(wl.kv_dtype == "bf16"))
        out.append(dataclasses.replace(base, weights=w, cache_k=kv["k"], cache_v=kv["v"]))
    return out


@pytest.mark.parametrize("kvd", ["bf16", "u8", "u4"])
def test_stack_decode_matches_chained_oracle(kvd):
    import torch
    import transformer_decoder_layer_amd as tdl
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY, kv_dtype=kvd)
    ctx = [0, 15, 16, 47, 130, 511]
    layers_in = stack_inputs(wl, 3, ctx, seed=41)
    log(f"[stack {kvd}] gpu")
    built = [gpu_setup(inp) for inp in layers_in]
    stack = tdl.Stack([layer for layer, _, _ in built])
    t0 = built[0][2]
    kvs = [kv for _, kv, _ in built]
    max_ctx = int(max(ctx) + 1)
    stack.decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"], max_ctx, kvs)
    torch.cuda.synchronize()
    y = t0["y"].float().cpu().numpy()
    log(f"[stack {kvd}] oracle")
    x = layers_in[0].x
    for l, inp in enumerate(layers_in):
        rows, ref, _ = run_oracle(dataclasses.replace(inp, x=x))
        x = synth.to_bf16_values(np.asarray(ref, np.float64)) if l + 1 < len(layers_in) else ref
    e = compare(y[rows], ref)
    log(f"[stack {kvd}] {e}")
    assert e.ok, str(e)
    # the same step with one layer is layer_decode_paged
    solo = tdl.Stack([built[0][0]])
    y1 = torch.empty_like(t0["y"])
    t0["y"].fill_(float("nan"))
    solo.decode_paged(t0["x"], y1, t0["ctx_len"], t0["table"], max_ctx, kvs[:1])
    built[0][0].decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"], max_ctx, kvs[0])
    torch.cuda.synchronize()
    assert torch.equal(y1, t0["y"])
    stack.close()
    solo.close()


def test_stack_graph_replay():
    import transformer_decoder_layer_amd as tdl
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY)
    ctx = [3, 16, 200, 64]
    layers_in = stack_inputs(wl, 4, ctx, seed=43)
    built = [gpu_setup(inp) for inp in layers_in]
    stack = tdl.Stack([layer for layer, _, _ in built])
    t0 = built[0][2]
    kvs = [kv for _, kv, _ in built]
    log("[stack graph] capture + replays")
    replay_matches(lambda: stack.decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"],
                                              int(max(ctx) + 1), kvs), t0["y"])
    stack.close()


def test_stack_rejects_before_enqueueing():
    # the second layer's max_position is too small for the call: the stack
    # must fail without running the first layer either
    import torch
    import transformer_decoder_layer_amd as tdl
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY)
    ctx = [3, 16]
    layers_in = stack_inputs(wl, 2, ctx, seed=44)
    built = [gpu_setup(layers_in[0]), gpu_setup(layers_in[1], max_position=16)]
    stack = tdl.Stack([layer for layer, _, _ in built])
    t0 = built[0][2]
    kvs = [kv for _, kv, _ in built]
    t0["y"].fill_(7.0)
    with pytest.raises(tdl.TdlError) as e:
        stack.decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"], 17, kvs)
    assert e.value.status == tdl.TDL_E_CAPACITY
    with pytest.raises(tdl.TdlError) as e:   # a missing cache
        stack.decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"], 17, [kvs[0], None])
    assert e.value.status == tdl.TDL_E_INVALID
    with pytest.raises(tdl.TdlError) as e:   # max_ctx_len beyond the table
        stack.decode_paged(t0["x"], t0["y"], t0["ctx_len"], t0["table"], 600, kvs)
    assert e.value.status == tdl.TDL_E_INVALID
    torch.cuda.synchronize()
    assert bool((t0["y"] == 7.0).all())     # nothing ran
    stack.close()
