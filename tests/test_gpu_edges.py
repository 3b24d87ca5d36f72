"""GPU parity at the edges of the supported shapes and sizes: every
query-group ratio and head dimension the attention kernels are built for,
Q8_0 weights on the decode-sized GEMM, a reduction dimension that ends in a
half 64-k stage, calls exactly at max_tokens / max_position, and mixed steps
with only decode or only prefill rows, Q8_0 layers above 128 rows (expanded
weight copies), and the rejection of misaligned activation pointers.  Same
tolerance as the other layer tests (stage by stage, cache rows checked)."""
import dataclasses

import numpy as np

import pytest

import synth
from harness import gpu_setup
from test_gpu_layer import TINY_Q80, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def _shape(name, hidden, hq, hkv, d, inter, **kw):
    return dataclasses.replace(synth.TINY, name=name, hidden=hidden, n_q_heads=hq, n_kv_heads=hkv,
                               head_dim=d, intermediate=inter, weight_dtype="bf16", rope_theta=1e6, **kw)


# one shape per (head_dim, query heads per KV head) the kernels instantiate
GQA_SHAPES = [
    _shape("mha-d64", 256, 4, 4, 64, 512),                 # 1:1
    _shape("gqa4-d64", 512, 8, 2, 64, 768),                # 4:1
    _shape("gqa8-d128", 1024, 8, 1, 128, 1536),            # 8:1
    _shape("mha-d128", 512, 4, 4, 128, 1024, qk_norm=True, qkv_bias=False),
]


@pytest.mark.parametrize("shape", GQA_SHAPES, ids=lambda s: s.name)
def test_gqa_ratios_prefill_and_decode(shape):
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=21, prefill_len=70, prefill_start=19, spare_blocks=2)
    layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {shape.name}")
    check_cache_rows(inp, kv, cache, [0])
    for kvd in ("bf16", "u8", "u4"):
        wd = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=shape, kv_dtype=kvd)
        ctx = [0, 9, 33, 255, 700]
        inp = synth.make_inputs(wd, seed=22, decode_batch=len(ctx), decode_ctx=ctx)
        layer, kv, t, cache, rows = check_layer(inp, what=f"decode {kvd} {shape.name}")
        check_cache_rows(inp, kv, cache, range(len(ctx)))


def test_q80_decode_stream_gemm():
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=TINY_Q80)
    ctx = [1, 16, 47, 300, 1023, 64, 5]
    inp = synth.make_inputs(wl, seed=23, decode_batch=len(ctx), decode_ctx=ctx)
    layer, kv, t, cache, rows = check_layer(inp, what="decode q80")
    check_cache_rows(inp, kv, cache, range(len(ctx)))


def test_half_stage_reduction_dim():
    # intermediate 736: the down projection's K = 23 steps of 32, so the decode
    # GEMM's last 64-k stage is half empty; the prefill GEMM takes K % 64 != 0
    shape = _shape("k736", 256, 4, 2, 64, 736)
    wd = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=shape)
    ctx = [3, 40, 129, 600, 17, 2]
    inp = synth.make_inputs(wd, seed=24, decode_batch=len(ctx), decode_ctx=ctx)
    check_layer(inp, what="decode k736")
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=25, prefill_len=150, spare_blocks=1)
    check_layer(inp, what="prefill k736")


def test_calls_at_capacity_limits():
    # prefill of exactly max_tokens rows ending exactly at max_position
    T, start = 96, 160
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=26, prefill_len=T, prefill_start=start)
    layer, kv, t, cache, rows = check_layer(inp, what="prefill at max_tokens/max_position",
                                            max_tokens=T, max_position=start + T)
    check_cache_rows(inp, kv, cache, [0])
    # decode tokens landing on the last position, max_position - 1
    wd = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY)
    ctx = [511, 511, 100]
    inp = synth.make_inputs(wd, seed=27, decode_batch=len(ctx), decode_ctx=ctx)
    layer, kv, t, cache, rows = check_layer(inp, what="decode at max_position - 1",
                                            max_tokens=len(ctx), max_position=512)
    check_cache_rows(inp, kv, cache, range(len(ctx)))


@pytest.mark.parametrize("what", ["decode_only", "prefill_only"])
def test_mixed_step_one_sided(what):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q80)
    if what == "decode_only":
        ctx = [0, 31, 200, 513]
        inp = synth.make_inputs(wl, seed=28, prefill_len=0, decode_batch=len(ctx), decode_ctx=ctx)
        rows = range(len(ctx))
    else:
        inp = synth.make_inputs(wl, seed=29, prefill_len=61, prefill_start=35, decode_batch=0)
        rows = [0]
    layer, kv, t, cache, _ = check_layer(inp, what=f"mixed {what}")
    check_cache_rows(inp, kv, cache, rows)


def test_misaligned_activations_rejected():
    # x and y move in 16-byte chunks: a pointer off that grid is an argument
    # error raised before anything is enqueued
    import torch
    import transformer_decoder_layer_amd as tdl
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], kv_dtype="none")
    inp = synth.make_inputs(wl, seed=30, prefill_len=8)
    layer, kv, t = gpu_setup(inp)
    T, H = t["x"].shape
    buf = torch.zeros(T * H + 8, dtype=torch.bfloat16, device="cuda")
    x_off = buf[1:1 + T * H].view(T, H)
    assert x_off.data_ptr() % 16 == 2
    with pytest.raises(tdl.TdlError):
        layer.prefill(x_off, t["y"], 0, None, None)
    y_off = torch.zeros(T * H + 8, dtype=torch.bfloat16, device="cuda")[4:4 + T * H].view(T, H)
    with pytest.raises(tdl.TdlError):
        layer.prefill(t["x"], y_off, 0, None, None)
    torch.cuda.synchronize()


def test_q80_over_128_rows_codes():
    # more than 128 rows: the Q8_0 layer's GEMMs take its packed codes and
    # block scales through the direct-load tiles (no expanded weight copy)
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q80)
    ctx = [5, 130, 301]
    inp = synth.make_inputs(wl, seed=31, prefill_len=200, prefill_start=40, decode_batch=len(ctx),
                            decode_ctx=ctx)
    layer, kv, t, cache, rows = check_layer(inp, what="mixed q80 203 rows")
    check_cache_rows(inp, kv, cache, range(1 + len(ctx)))


def _scaled_kv_inputs(scale, seed):
    # the tiny fp32 layer with Wk and Wv multiplied by `scale`: K / V values
    # of about 16 * 0.02 * scale (xn ~ N(0, 1) over 256 inputs)
    inp = synth.make_inputs(synth.WORKLOADS["tiny_prefill_32"], seed=seed, random_gains=True)
    w = dict(inp.weights)
    for name in ("wk", "wv", "bk", "bv"):
        w[name] = (w[name].astype(np.float64) * scale).astype(np.float32)
    return dataclasses.replace(inp, weights=w)


def test_prefill_attention_near_fp16_limit():
    # prefill attention computes on fp16 copies of K and V: values up to a
    # few 10^4 (max |V| below 65504) keep the bf16 tolerance
    inp = _scaled_kv_inputs(25000.0, 91)
    layer, kv, t, cache, rows = check_layer(inp, what="prefill, |K|, |V| up to ~3e4")
    from harness import run_oracle
    _, (ref, st), _ = run_oracle(inp, want_stages=True)
    vmax = float(np.abs(st["v"]).max())
    print(f"max |V| {vmax:.0f}", flush=True)
    assert 2e4 < vmax < 65504


def test_prefill_attention_beyond_fp16_limit_saturates():
    # beyond 65504 the fp16 copies saturate (documented in include/tdl.h):
    # the output stays finite
    import torch
    from harness import gpu_call, gpu_setup, run_oracle
    inp = _scaled_kv_inputs(100000.0, 92)
    _, (ref, st), _ = run_oracle(inp, want_stages=True)
    assert float(np.abs(st["v"]).max()) > 65504
    layer, kv, t = gpu_setup(inp)
    gpu_call(inp, layer, kv, t)
    torch.cuda.synchronize()
    assert torch.isfinite(t["y"].float()).all()
