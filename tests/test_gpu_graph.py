"""The layer's calls captured into a HIP graph (torch.cuda.CUDAGraph around the
C-ABI call) and replayed: every replay, with eager work and synchronisation
in between, must reproduce the eager call's output bit for bit.  The decode
case uses the Qwen2.5-7B shapes, whose decode-sized projections are split
over K with the partial sums reduced inside the RoPE and RMSNorm kernels."""
import dataclasses
import math
import sys

import numpy as np
import pytest

import synth
from harness import compare, gpu_call, gpu_setup, run_oracle

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


def replay_matches(call, y, n_replays=3):
    """Eager call, capture, then replays interleaved with unrelated eager
    work; returns the eager output."""
    import torch
    call()
    torch.cuda.synchronize()
    y_eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(n_replays):
        y.fill_(float("nan"))
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r} differs from the eager call"
    return y_eager


def test_graph_tiny_decode():
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY)
    ctx = [0, 15, 16, 100, 511]
    inp = synth.make_inputs(wl, seed=11, decode_batch=len(ctx), decode_ctx=ctx)
    layer, kv, t = gpu_setup(inp)
    log("[graph tiny decode] capture + replays")
    y = replay_matches(lambda: gpu_call(inp, layer, kv, t), t["y"])
    rows, ref, _ = run_oracle(inp)
    err = compare(y.float().cpu().numpy()[rows], ref)
    log(f"[graph tiny decode] vs oracle: {err}")
    assert err.ok


@pytest.mark.parametrize("kvd,wdt", [("u4", "bf16"), ("bf16", "iq8"), ("u8", "iq8")])
def test_graph_tiny_decode_quantised(kvd, wdt):
    # code caches and per-row int8 weights replay like the bf16 path
    shape = dataclasses.replace(synth.TINY, name=f"tiny-{wdt}", intermediate=704, weight_dtype=wdt)
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=shape, kv_dtype=kvd)
    ctx = [0, 15, 16, 100, 511]
    inp = synth.make_inputs(wl, seed=13, decode_batch=len(ctx), decode_ctx=ctx)
    layer, kv, t = gpu_setup(inp)
    log(f"[graph tiny decode {kvd} {wdt}] capture + replays")
    y = replay_matches(lambda: gpu_call(inp, layer, kv, t), t["y"])
    rows, ref, _ = run_oracle(inp)
    err = compare(y.float().cpu().numpy()[rows], ref)
    log(f"[graph tiny decode {kvd} {wdt}] vs oracle: {err}")
    assert err.ok


def test_graph_a8w8_gemm():
    import torch
    import transformer_decoder_layer_amd as tdl
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    A = torch.randint(-128, 128, (300, 512), generator=g, device="cuda", dtype=torch.int8)
    B = torch.randint(-128, 128, (200, 512), generator=g, device="cuda", dtype=torch.int8)
    sa = torch.rand(300, generator=g, device="cuda")
    sb = torch.rand(200, generator=g, device="cuda")
    out = torch.empty((300, 200), dtype=torch.float32, device="cuda")
    log("[graph a8w8] capture + replays")
    replay_matches(lambda: tdl.gemm_a8w8(A, B, sa, sb, out), out)


def test_graph_tiny_prefill():
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=12, prefill_len=77, spare_blocks=2)
    layer, kv, t = gpu_setup(inp)
    log("[graph tiny prefill] capture + replays")
    y = replay_matches(lambda: gpu_call(inp, layer, kv, t), t["y"])
    rows, ref, _ = run_oracle(inp)
    err = compare(y.float().cpu().numpy()[rows], ref)
    log(f"[graph tiny prefill] vs oracle: {err}")
    assert err.ok


def test_graph_qwen25_decode_split_projections():
    import torch
    import transformer_decoder_layer_amd as tdl
    shape = synth.QWEN25_7B
    B = 16
    rng = np.random.default_rng(5)
    ctx = rng.integers(16, 1024, size=B).astype(np.int32)
    totals = (ctx + 1).tolist()
    nb = int(sum(math.ceil(v / 16) for v in totals))
    tab = torch.from_numpy(synth.random_tables(np.random.default_rng(6), totals, n_blocks=nb)).cuda()
    w = synth.torch_weights(shape, seed=3)
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=B, max_seqs=B, max_position=2048), w)
    kv = tdl.KvCache(nb, shape.n_kv_heads, shape.head_dim, "bf16")
    n_cached = int(ctx.sum())
    ck = synth.torch_normal((n_cached, shape.n_kv_heads, shape.head_dim), seed=7, dtype=torch.bfloat16)
    cv = synth.torch_normal((n_cached, shape.n_kv_heads, shape.head_dim), seed=8, dtype=torch.bfloat16)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
    kv.write(cu, torch.zeros(B, dtype=torch.int32, device="cuda"), tab, ck, cv)
    x = synth.torch_normal((B, shape.hidden), seed=9, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    ctx_d = torch.from_numpy(ctx).cuda()
    log("[graph qwen25 decode b16] capture + replays")
    out = replay_matches(lambda: layer.decode_paged(x, y, ctx_d, tab, int(ctx.max()) + 1, kv), y)
    assert torch.isfinite(out.float()).all()
