"""layer_decode_paged_noalloc (the decode step whose partial results live in
the library's static scratch instead of the layer's workspace) against
layer_decode_paged through the C ABI: same kernels, so the outputs must agree
bit for bit, on two calls in a row (the second with a smaller batch and
shorter contexts, reusing the scratch the first left behind), for a bf16 and
a u8 cache and for a layer whose projections split K (partial slices in the
scratch), and against the oracle at the bf16 bar.  A step too large for the
scratch is refused before anything is enqueued."""
import ctypes
import dataclasses

import numpy as np
import pytest

import synth
from harness import compare, gpu_setup, run_oracle

pytestmark = pytest.mark.gpu

TINY_Q3 = dataclasses.replace(synth.TINY, name="tiny-qwen3", qkv_bias=False, qk_norm=True,
                              weight_dtype="bf16", rope_theta=1e6)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def _decode_both(inp, what):
    import torch
    b = inp.batch
    layer, kv, t = gpu_setup(inp)
    max_ctx = int((b.ctx_len + 1).max())
    # the no-alloc step first, on the cache as set up; then the regular step
    # on a fresh copy of the same cache contents (each writes the new token)
    snap = [x.clone() for x in kv.tensors()[:2]]
    y_na = torch.full_like(t["x"], float("nan"))
    layer.decode_paged_noalloc(t["x"], y_na, t["ctx_len"], t["table"], max_ctx, kv)
    torch.cuda.synchronize()
    kt, vt = kv.tensors()[:2]
    k_na, v_na = kt.clone(), vt.clone()
    kt.copy_(snap[0])
    vt.copy_(snap[1])
    layer.decode_paged(t["x"], t["y"], t["ctx_len"], t["table"], max_ctx, kv)
    torch.cuda.synchronize()
    assert torch.equal(y_na, t["y"]), f"{what}: no-alloc output differs from layer_decode_paged"
    assert torch.equal(k_na, kt) and torch.equal(v_na, vt), f"{what}: cache writes differ"
    rows, ref, _ = run_oracle(inp)
    e = compare(y_na.float().cpu().numpy()[rows], ref)
    print(f"[{what}] no-alloc vs oracle: {e}", flush=True)
    assert e.ok, f"{what}: {e}"
    layer.close()
    kv.close()


@pytest.mark.parametrize("kvd", ["bf16", "u8"])
def test_noalloc_matches_decode_paged_two_calls(kvd):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_decode_u8_b128"], shape=TINY_Q3, kv_dtype=kvd)
    big = [1, 15, 16, 17, 64, 300, 777, 2048, 3000, 5]
    small = [0, 33, 129]
    _decode_both(synth.make_inputs(wl, seed=91, decode_batch=len(big), decode_ctx=big,
                                   random_gains=True), f"{kvd} first call, batch {len(big)}")
    _decode_both(synth.make_inputs(wl, seed=92, decode_batch=len(small), decode_ctx=small,
                                   random_gains=True), f"{kvd} second call, batch {len(small)}")


def test_noalloc_split_projections_qwen25_shape():
    # the Qwen2.5-7B shape at batch 64 splits the QKV, output and down
    # projections over K: their partial slices go through the static scratch
    wl = synth.WORKLOADS["qwen25_decode_b64"]
    ctx = [int(c) for c in synth.context_lengths(np.random.default_rng(93), wl)][:64]
    ctx = [min(c, 700) for c in ctx]
    _decode_both(synth.make_inputs(wl, seed=94, decode_ctx=ctx), "qwen2.5 b64 first call")
    _decode_both(synth.make_inputs(wl, seed=95, decode_batch=8, decode_ctx=ctx[:8]),
                 "qwen2.5 b8 second call")


def test_noalloc_refuses_a_step_beyond_the_scratch():
    import torch
    import transformer_decoder_layer_amd as tdl
    shape = synth.QWEN3_8B
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=128, max_seqs=128, max_position=8448),
                      synth.torch_weights(shape, seed=1))
    kv = tdl.KvCache(16, shape.n_kv_heads, shape.head_dim, "u8")
    x = torch.zeros(128, shape.hidden, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ctx = torch.zeros(128, dtype=torch.int32, device="cuda")
    tab = torch.zeros(128, 513, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="static scratch"):
        layer.decode_paged_noalloc(x, y, ctx, tab, 8193, kv)
    layer.close()
    kv.close()
