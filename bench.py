#!/usr/bin/env python3
"""Benchmark of the decoder layer on one MI355X.

Headline: prompt prefill of the Qwen2.5-7B-shaped layer (hidden 3584, 28 Q /
4 KV heads, head_dim 128, SwiGLU 18944, QKV bias) over 4096 tokens, batch 1,
writing K/V into a bf16 block-paged cache -- one layer_prefill call per step,
inputs resident in HBM.  value = tokens/s.

Also reported (same JSON line): the paged decode step of the same layer (batch
64, contexts U[128, 4096], bf16 cache, random block permutation) in us/step
with its HBM fraction; the dominant kernel's roofline (per-kernel HIP-event
durations recorded by the library on the call's stream over the timed
region); the other configurations (the 512-token prefill, the Qwen3-8B
decode over u8 and u4 caches at batch 128, the Qwen2.5-7B decode with
per-row int8 weights, the Qwen3-8B Q8_0 mixed step, a 28-layer decode
stack), each with
its roofline fraction; and the oracle's CPU throughput on a bounded sample of
the prefill.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_INT8_TOPS = 5000.0   # dense int8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=30)
    ap.add_argument("--prefill-len", type=int, default=4096)
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="prompt tokens the oracle runs for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--rope-unfused", action="store_true",
                    help="the RoPE kernel rotates the prefill queries too (instead of the prefill "
                         "attention kernel as it loads them)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other workloads (512-token prefill, Qwen3 u8 / u4 decode, Q8_0 mixed step, layer stack)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 512 MiB device-to-device copy (a known byte count that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_qwen25_prefill4096_hbm_traffic.txt")
GEMM_SOURCES = ["gemm.hip", "common.h", "kernels.h"]


def measured_traffic():
    """HBM bytes per gate_up launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when the GEMM sources changed since it was taken."""
    import hashlib
    try:
        line = [l for l in open(TRAFFIC_FILE) if l.startswith("TRAFFIC ")][-1]
    except (OSError, IndexError):
        return None
    meta = json.loads(line[len("TRAFFIC "):])
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "transformer_decoder_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != meta.get("kernel_source_sha256"):
        return None
    return meta.get("traffic_bytes_per_launch")


def layer_weight_bytes_q80(s):
    """Bytes a Q8_0 layer keeps for its four projections: one byte per code
    plus a 2-byte scale per 32 codes."""
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    n = (qd + 2 * kd) * s.hidden + s.hidden * qd + 3 * s.intermediate * s.hidden
    return n + n // 32 * 2


def linear_flops_per_token(s):
    D = s.head_dim
    n = (s.n_q_heads + 2 * s.n_kv_heads) * D * s.hidden + s.hidden * s.n_q_heads * D \
        + 2 * s.intermediate * s.hidden + s.hidden * s.intermediate
    return 2 * n


def weight_bytes(s):
    return linear_flops_per_token(s) // 2 * 2   # 2-byte weights


def timed_steps(torch, stream, step_fn, n, flush=None, sink=None):
    """Per-step HIP-event times (ms, sorted) of n calls on `stream`; with
    `flush`, a 1 GiB read evicts L2 and the MALL before each call."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        e0.record(stream)
        step_fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in ev)


def stage_profile(layer, step_fn, n, before=None):
    """ms per launch of each stage over n calls, from the library's HIP events."""
    import torch
    layer.profile_enable(True)
    for _ in range(n):
        if before is not None:
            before()
        step_fn()
    torch.cuda.synchronize()
    prof = layer.profile_read()
    layer.profile_enable(False)
    return {k: round(v[0] / v[1], 4) for k, v in prof.items() if v[1]}


def attention_flops(D, Hq, n_pairs):
    return 4 * D * Hq * n_pairs  # Q.K and P.V: 2 FLOP x D per (query, key) pair and head


def quantised_decode(args, torch, synth, tdl, stream, kvd, flush, sink):
    """Qwen3-8B-shaped decode at batch 128 over a u8 or u4 (per-channel
    asymmetric) cache; contexts and block placement as for the bf16 decode."""
    wl = synth.WORKLOADS[f"qwen3_decode_{kvd}_b128"]
    shape = wl.shape
    Hkv, D, H = shape.n_kv_heads, shape.head_dim, shape.hidden
    B = wl.decode_batch
    ctx = synth.context_lengths(np.random.default_rng(30), wl)
    totals = (ctx + 1).tolist()
    nb = int(sum(math.ceil(t / 16) for t in totals))
    tab_np = synth.random_tables(np.random.default_rng(31), totals, n_blocks=nb)
    tab = torch.from_numpy(tab_np).cuda()
    log(f"qwen3 {kvd} decode: weights, cache of {int(ctx.sum())} tokens")
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=B, max_seqs=B, max_position=8448),
                      synth.torch_weights(shape, seed=32))
    kv = tdl.KvCache(nb, Hkv, D, kvd)
    # per-channel parameters from a sample of the same N(0,1) distribution,
    # then the cached tokens, 16 sequences at a time
    kv.calibrate(synth.torch_normal((1 << 16, Hkv, D), seed=33), synth.torch_normal((1 << 16, Hkv, D), seed=34))
    for s0 in range(0, B, 16):
        c = ctx[s0:s0 + 16]
        n = int(c.sum())
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(c)]).astype(np.int32)).cuda()
        kv.write(cu, torch.zeros(len(c), dtype=torch.int32, device="cuda"), tab[s0:s0 + 16].contiguous(),
                 synth.torch_normal((n, Hkv, D), seed=100 + s0), synth.torch_normal((n, Hkv, D), seed=200 + s0))
    ctx_d = torch.from_numpy(ctx).cuda()
    x = synth.torch_normal((B, H), seed=35, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    max_ctx = int(ctx.max()) + 1
    for _ in range(3):
        layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv)
    times = timed_steps(torch, stream, lambda: layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv),
                        args.decode_steps, flush, sink)
    us = 1e3 * float(np.median(times))
    bits = 8 if kvd == "u8" else 4
    kv_bytes = int(sum(totals)) * Hkv * D * 2 * bits // 8  # K and V codes
    step_bytes = weight_bytes(shape) + kv_bytes + 2 * B * H * 2
    assert torch.isfinite(y.float()).all(), f"non-finite {kvd} decode output"
    res = {f"qwen3_decode_{kvd}_b128": {
        "workload": "qwen3-8b-shaped layer (Q/K RMSNorm) paged decode, batch 128, ctx U[512,8192], "
                    f"{kvd} per-channel asymmetric KV, block 16, random block permutation; L2/MALL flushed between steps",
        "us_per_step": round(us, 2), "algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "stages_ms": stage_profile(layer, lambda: layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv), 5,
                                   lambda: torch.sum(flush, dim=0, out=sink))}}
    log(f"qwen3 {kvd} decode: {us:.1f} us/step")
    layer.close()
    kv.close()
    return res


def other_workloads(args, torch, synth, tdl, stream, layer512):
    """The other configurations of the layer, measured the same way (synthetic
    inputs, resident in HBM): the 512-token prefill of the same Qwen2.5-7B
    layer, the Qwen3-8B decode over a u8 and over a u4 cache (batch 128), the
    Qwen2.5-7B decode with per-row int8 weights (batch 64), the int8 x int8
    GEMM at the gate/up shape, the Qwen3-8B
    Q8_0 mixed step (a 2048-token chunk + 64 decode rows), and a 28-layer
    stack of the Qwen2.5-7B layer decoding batch 64."""
    out = {}
    n_steps = max(5, args.steps)
    # ---- Qwen2.5-7B prefill of 512 tokens
    layer, shape = layer512
    T = 512
    x = synth.torch_normal((T, shape.hidden), seed=21, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    nb = T // 16
    tab = torch.from_numpy(synth.random_tables(np.random.default_rng(22), [T], n_blocks=nb)[0]).cuda()
    kv = tdl.KvCache(nb, shape.n_kv_heads, shape.head_dim, "bf16")
    for _ in range(3):
        layer.prefill(x, y, 0, kv, tab)
    times = timed_steps(torch, stream, lambda: layer.prefill(x, y, 0, kv, tab), n_steps)
    ms = float(np.median(times))
    fl = linear_flops_per_token(shape) * T + attention_flops(shape.head_dim, shape.n_q_heads, T * (T + 1) // 2)
    out["qwen25_prefill_512"] = {
        "workload": "qwen2.5-7b-shaped layer, causal prefill seq 512, batch 1, bf16 paged KV cache written",
        "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
        "stages_ms": stage_profile(layer, lambda: layer.prefill(x, y, 0, kv, tab), 5)}
    log(f"prefill 512: {ms * 1e3:.1f} us/step")
    kv.close()
    del x, y, kv

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    # ---- Qwen3-8B decode, batch 128, ctx U[512, 8192], u8 and u4 caches
    for kvd in ("u8", "u4"):
        out.update(quantised_decode(args, torch, synth, tdl, stream, kvd, flush, sink))

    # ---- Qwen3-8B Q8_0 mixed step: one 2048-token chunk + 64 decode rows at ctx 2048
    wl = synth.WORKLOADS["qwen3_q80_mixed"]
    shape = wl.shape
    Hq, Hkv, D, H = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.hidden
    Tc, B, c0 = wl.prefill_len, wl.decode_batch, wl.ctx_fixed
    totals = [Tc] + [c0 + 1] * B
    nb = int(sum(math.ceil(t / 16) for t in totals))
    tab = torch.from_numpy(synth.random_tables(np.random.default_rng(40), totals, n_blocks=nb)).cuda()
    log("q8_0 mixed: weights, cache")
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=Tc + B, max_seqs=B + 1, max_position=4096),
                      synth.torch_weights(shape, seed=41))
    kv = tdl.KvCache(nb, Hkv, D, "bf16")
    cu = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * c0).cuda()
    kv.write(cu, torch.zeros(B, dtype=torch.int32, device="cuda"), tab[1:].contiguous(),
             synth.torch_normal((B * c0, Hkv, D), seed=42, dtype=torch.bfloat16),
             synth.torch_normal((B * c0, Hkv, D), seed=43, dtype=torch.bfloat16))
    rows = Tc + B
    q_start = torch.from_numpy(np.array([0] + [Tc + i for i in range(B)], np.int32)).cuda()
    q_len = torch.from_numpy(np.array([Tc] + [1] * B, np.int32)).cuda()
    ctx_len = torch.from_numpy(np.array([0] + [c0] * B, np.int32)).cuda()
    x = synth.torch_normal((rows, H), seed=44, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    step = lambda: layer.step(x, y, q_start, q_len, ctx_len, tab, 1, Tc, c0 + 1, kv)
    for _ in range(3):
        step()
    times = timed_steps(torch, stream, step, n_steps)
    ms = float(np.median(times))
    fl = linear_flops_per_token(shape) * rows + attention_flops(D, Hq, Tc * (Tc + 1) // 2 + B * (c0 + 1))
    assert torch.isfinite(y.float()).all(), "non-finite mixed-step output"
    out["qwen3_q80_mixed"] = {
        "workload": "qwen3-8b-shaped layer with Q8_0 weights (codes + fp16 block scales only, 1.0625 "
                    "bytes per weight), mixed step: 2048-token chunked prefill + 64 decode rows at ctx "
                    "2048, bf16 paged KV cache.  The codes enter fp16/bf16 MFMAs exactly and each 32-input "
                    "block's product is scaled in fp32, so the fp16 peak bounds this path; the int8 "
                    "matrix peak is given beside it",
        "ms_per_step": round(ms, 4), "rows_per_s": round(rows / (ms * 1e-3), 1),
        "weight_bytes": int(layer_weight_bytes_q80(shape)),
        "roofline": {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
        "roofline_int8": {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 1), "peak": PEAK_INT8_TOPS,
                          "unit": "TOP/s", "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)},
        "stages_ms": stage_profile(layer, step, 5)}
    log(f"q8_0 mixed: {ms * 1e3:.1f} us/step")
    layer.close()
    kv.close()
    del x, y, kv, tab

    # ---- Qwen2.5-7B decode with weight-only per-row int8 weights: batch,
    # contexts, block placement and cache drawn as for the bf16 decode
    wl = synth.WORKLOADS["qwen25_iq8_decode_b64"]
    shape = wl.shape
    Hkv, D, H = shape.n_kv_heads, shape.head_dim, shape.hidden
    B = wl.decode_batch
    ctx = synth.context_lengths(np.random.default_rng(0), wl)
    totals = (ctx + 1).tolist()
    nb = int(sum(math.ceil(t / 16) for t in totals))
    tab = torch.from_numpy(synth.random_tables(np.random.default_rng(3), totals, n_blocks=nb)).cuda()
    log(f"qwen2.5 iq8 decode: weights, cache of {int(ctx.sum())} tokens")
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=B, max_seqs=B, max_position=4352),
                      synth.torch_weights(shape, seed=7))
    kv = tdl.KvCache(nb, Hkv, D, "bf16")
    n_cached = int(ctx.sum())
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
    kv.write(cu, torch.zeros(B, dtype=torch.int32, device="cuda"), tab,
             synth.torch_normal((n_cached, Hkv, D), seed=4, dtype=torch.bfloat16),
             synth.torch_normal((n_cached, Hkv, D), seed=5, dtype=torch.bfloat16))
    ctx_d = torch.from_numpy(ctx).cuda()
    x = synth.torch_normal((B, H), seed=6, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    max_ctx = int(ctx.max()) + 1
    for _ in range(3):
        layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv)
    times = timed_steps(torch, stream, lambda: layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv),
                        args.decode_steps, flush, sink)
    us = 1e3 * float(np.median(times))
    n_rows = shape.n_q_heads * D + 2 * Hkv * D + H + 2 * shape.intermediate + H
    w_bytes = weight_bytes(shape) // 2 + 5 * n_rows  # 1-byte codes + fp32 scale and int8 zero point per row
    step_bytes = w_bytes + int(sum(totals)) * Hkv * D * 2 * 2 + 2 * B * H * 2
    assert torch.isfinite(y.float()).all(), "non-finite iq8 decode output"
    out["qwen25_iq8_decode_b64"] = {
        "workload": "qwen2.5-7b-shaped layer with weight-only per-row int8 weights (code - zp) * scale, "
                    "paged decode, batch 64, ctx U[128,4096], bf16 KV, block 16, random block permutation; "
                    "L2/MALL flushed between steps",
        "us_per_step": round(us, 2), "algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "stages_ms": stage_profile(layer, lambda: layer.decode_paged(x, y, ctx_d, tab, max_ctx, kv), 5,
                                   lambda: torch.sum(flush, dim=0, out=sink))}
    log(f"qwen2.5 iq8 decode: {us:.1f} us/step")
    layer.close()
    kv.close()
    del x, y, kv, tab, ctx_d

    # ---- int8 x int8 GEMM (activation-quantised), at the gate/up shape of
    # the 4096-token prefill: M 4096, N 2 x 18944, K 3584
    M, N, K = 4096, 37888, 3584
    g = torch.Generator(device="cuda")
    g.manual_seed(80)
    A8 = torch.randint(-128, 128, (M, K), generator=g, device="cuda", dtype=torch.int8)
    B8 = torch.randint(-128, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    sa = torch.rand(M, generator=g, device="cuda") * 0.01 + 1e-4
    sb = torch.rand(N, generator=g, device="cuda") * 0.01 + 1e-4
    o8 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for _ in range(3):
        tdl.gemm_a8w8(A8, B8, sa, sb, o8)
    times = timed_steps(torch, stream, lambda: tdl.gemm_a8w8(A8, B8, sa, sb, o8), n_steps)
    ms = float(np.median(times))
    tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    assert torch.isfinite(o8).all(), "non-finite a8w8 output"
    out["a8w8_gemm_4096x37888x3584"] = {
        "workload": "int8 x int8 GEMM, int32 accumulation, per-row x per-column fp32 dequantising epilogue, "
                    "fp32 output; M 4096, N 37888, K 3584 (the Qwen2.5-7B gate/up shape of the 4096-token prefill)",
        "ms_per_call": round(ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(tops / PEAK_INT8_TOPS, 4)}}
    log(f"a8w8 gemm: {ms * 1e3:.1f} us, {tops:.0f} TOP/s")
    del A8, B8, o8

    # ---- the Qwen2.5-7B layer on the A8W8 path (int8 weights with a scale
    # per output row, every projection's input quantised per row to int8):
    # causal prefill of 4096 tokens into a bf16 paged cache, as the headline
    shape = synth.QWEN25_7B_A8W8
    T, H, D, Hq, Hkv = 4096, shape.hidden, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    log("qwen2.5 a8w8 prefill 4096: weights")
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=T, max_seqs=1, max_position=T),
                      synth.torch_weights(shape, seed=90))
    kv = tdl.KvCache(T // 16, Hkv, D, "bf16")
    table = torch.arange(T // 16, dtype=torch.int32, device="cuda").view(1, -1)
    x = synth.torch_normal((T, H), seed=91, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    step = lambda: layer.prefill(x, y, 0, kv, table)
    for _ in range(3):
        step()
    times = timed_steps(torch, stream, step, n_steps)
    ms = float(np.median(times))
    lin = linear_flops_per_token(shape) * T
    fl = lin + attention_flops(D, Hq, T * (T + 1) // 2)
    assert torch.isfinite(y.float()).all(), "non-finite a8w8 prefill output"
    stages = stage_profile(layer, step, 5)
    gu_ms = stages.get("gate_up", 0.0)
    out["qwen25_a8w8_prefill_4096"] = {
        "workload": "qwen2.5-7b-shaped layer on the A8W8 path (int8 weights, fp32 scale per output row; each "
                    "projection's input rows quantised to int8 with a scale per row; int8 MFMAs with int32 "
                    "sums), causal prefill of 4096 tokens into a bf16 paged cache; attention on fp16 MFMAs",
        "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
        "linear_ops_per_step": lin,
        "gate_up": {"bound": "mfma", "ms_per_launch": gu_ms,
                    "achieved": round(2 * T * 2 * shape.intermediate * H / (gu_ms * 1e-3) / 1e12, 1) if gu_ms else None,
                    "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "note": "quantisation of hn + int8 GEMM + SiLU-gate pass"},
        "stages_ms": stages}
    log(f"qwen2.5 a8w8 prefill: {ms:.3f} ms/step")
    layer.close()
    kv.close()
    del x, y, kv, table

    # ---- a 28-layer stack of Qwen2.5-7B-shaped layers (each with its own
    # weights and bf16 cache), decode batch 64: one token of every sequence
    # through every layer per step, eager and as a replayed HIP graph
    wl = synth.WORKLOADS["qwen25_decode_b64"]
    shape = wl.shape
    Hkv, D, H = shape.n_kv_heads, shape.head_dim, shape.hidden
    B, n_layers = wl.decode_batch, 28
    ctx = synth.context_lengths(np.random.default_rng(50), wl)
    totals = (ctx + 1).tolist()
    nb = int(sum(math.ceil(t / 16) for t in totals))
    tab = torch.from_numpy(synth.random_tables(np.random.default_rng(51), totals, n_blocks=nb)).cuda()
    n_cached = int(ctx.sum())
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    log(f"stack of {n_layers} layers: weights and caches")
    layers, kvs = [], []
    for l in range(n_layers):
        layers.append(tdl.Layer(tdl.make_config(shape, max_tokens=B, max_seqs=B, max_position=4224),
                                synth.torch_weights(shape, seed=500 + l)))
        kv = tdl.KvCache(nb, Hkv, D, "bf16")
        kv.write(cu, zero, tab, synth.torch_normal((n_cached, Hkv, D), seed=600 + l, dtype=torch.bfloat16),
                 synth.torch_normal((n_cached, Hkv, D), seed=700 + l, dtype=torch.bfloat16))
        kvs.append(kv)
    stack = tdl.Stack(layers)
    ctx_d = torch.from_numpy(ctx).cuda()
    x = synth.torch_normal((B, H), seed=52, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    max_ctx = int(ctx.max()) + 1
    step = lambda: stack.decode_paged(x, y, ctx_d, tab, max_ctx, kvs)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    us = 1e3 * float(np.median(timed_steps(torch, stream, step, n_steps, flush, sink)))
    y_eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    us_graph = 1e3 * float(np.median(timed_steps(torch, stream, graph.replay, n_steps, flush, sink)))
    assert torch.equal(y, y_eager), "graph replay of the stack differs from the eager step"
    assert torch.isfinite(y.float()).all(), "non-finite stack output"
    del graph
    step_bytes = n_layers * (weight_bytes(shape) + int(sum(totals)) * Hkv * D * 2 * 2) + 2 * B * H * 2
    out["qwen25_stack28_decode_b64"] = {
        "workload": "28 qwen2.5-7b-shaped layers (own weights and bf16 paged cache each), decode batch 64, "
                    "ctx U[128,4096], random block permutation: one token per sequence through the stack",
        "us_per_step": round(us, 1), "tokens_per_s": round(B / (us * 1e-6), 1),
        "graph_us_per_step": round(us_graph, 1), "algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}}
    log(f"stack of {n_layers}: {us:.1f} us/step eager, {us_graph:.1f} us/step graph")
    stack.close()
    for l in layers:
        l.close()
    for k in kvs:
        k.close()
    del flush
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import transformer_decoder_layer_amd as tdl

    torch.cuda.set_device(0)
    shape = synth.QWEN25_7B
    H, D, Hq, Hkv, I = shape.hidden, shape.head_dim, shape.n_q_heads, shape.n_kv_heads, shape.intermediate
    T = args.prefill_len
    stream = torch.cuda.current_stream()

    log("generating weights")
    w = synth.torch_weights(shape, seed=0)
    cfg = tdl.make_config(shape, max_tokens=T, max_seqs=64, max_position=8192, rope_fused=not args.rope_unfused)
    layer = tdl.Layer(cfg, w)

    # ------------------------------------------------------------ prefill
    x = synth.torch_normal((T, H), seed=1, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    rng = np.random.default_rng(2)
    n_blk = math.ceil(T / 16)
    table = torch.from_numpy(synth.random_tables(rng, [T], n_blocks=n_blk)[0]).cuda()
    kv = tdl.KvCache(n_blk, Hkv, D, "bf16")
    log(f"prefill T={T}: warmup {args.warmup}")
    for _ in range(args.warmup):
        layer.prefill(x, y, 0, kv, table)
    torch.cuda.synchronize()
    log(f"prefill: timing {args.steps} steps")
    # the K timed steps: wall clock between two synchronisations (value,
    # ms_per_step) and a HIP-event pair around each call on its stream
    # (median, p10, p90 of the per-call times)
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in pev:
        e0.record(stream)
        layer.prefill(x, y, 0, kv, table)
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    tok_s = T * args.steps / (t1 - t0)
    pcall = sorted(e0.elapsed_time(e1) for e0, e1 in pev)
    prefill_call_ms = {"median": round(float(np.median(pcall)), 4),
                       "p10": round(pcall[len(pcall) // 10], 4),
                       "p90": round(pcall[(9 * len(pcall)) // 10], 4)}
    log(f"prefill: {ms_step:.4f} ms/step wall, per call {prefill_call_ms}")
    # per-kernel durations from the library's HIP events, in a separate pass
    # of as many calls as the timed steps (the event records are kept out of
    # the timed steps)
    layer.profile_enable(True)
    for _ in range(args.steps):
        layer.prefill(x, y, 0, kv, table)
    torch.cuda.synchronize()
    prof = layer.profile_read()
    layer.profile_enable(False)
    stage_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in prof.items()}
    log("prefill stages (ms/launch): " + ", ".join(f"{k}={v:.3f}" for k, v in stage_ms.items() if v))
    assert torch.isfinite(y.float()).all(), "non-finite prefill output"

    lin_flops = linear_flops_per_token(shape) * T
    attn_flops = 2 * D * Hq * T * (T + 1)
    step_flops = lin_flops + attn_flops
    gu_flops = 2 * T * (2 * I) * H
    gu_ms = stage_ms["gate_up"]
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "gate_up GEMM + SiLU-gate (fp16 operands; with its split-tail reduction)",
                "achieved": round(gu_tflops, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tflops / PEAK_MFMA_TFLOPS, 4), "traffic": measured_traffic(),
                "algorithmic_bytes": 2 * (T * H + 2 * I * H + T * I),
                "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 4)}
    layer_tflops = step_flops / (ms_step * 1e-3) / 1e12
    stage_report = {k: round(v, 4) for k, v in stage_ms.items() if v}

    # ------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        wl = synth.WORKLOADS["qwen25_decode_b64"]
        B = wl.decode_batch
        ctx = synth.context_lengths(np.random.default_rng(0), wl)
        totals = (ctx + 1).tolist()
        nb = int(sum(math.ceil(t / 16) for t in totals))
        tab_np = synth.random_tables(np.random.default_rng(3), totals, n_blocks=nb)
        dkv = tdl.KvCache(nb, Hkv, D, "bf16")
        n_cached = int(ctx.sum())
        log(f"decode: filling cache with {n_cached} tokens")
        ck = synth.torch_normal((n_cached, Hkv, D), seed=4, dtype=torch.bfloat16)
        cv = synth.torch_normal((n_cached, Hkv, D), seed=5, dtype=torch.bfloat16)
        tab = torch.from_numpy(tab_np).cuda()
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
        dkv.write(cu, torch.zeros(B, dtype=torch.int32, device="cuda"), tab, ck, cv)
        del ck, cv
        ctx_d = torch.from_numpy(ctx).cuda()
        xd = synth.torch_normal((B, H), seed=6, dtype=torch.bfloat16)
        yd = torch.empty_like(xd)
        max_ctx = int(ctx.max()) + 1
        # 1 GiB > L2 + MALL, evicted by reading it (a write would leave dirty
        # lines whose write-back then competes with the timed step)
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.empty((), dtype=torch.float32, device="cuda")
        for _ in range(3):
            layer.decode_paged(xd, yd, ctx_d, tab, max_ctx, dkv)
        torch.cuda.synchronize()
        y_eager = yd.clone()

        def timed(step_fn, n):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(n)]
            for e0, e1 in ev:
                torch.sum(flush, dim=0, out=sink)
                e0.record(stream)
                step_fn()
                e1.record(stream)
            torch.cuda.synchronize()
            return sorted(e0.elapsed_time(e1) for e0, e1 in ev)

        times = timed(lambda: layer.decode_paged(xd, yd, ctx_d, tab, max_ctx, dkv), args.decode_steps)
        us = 1e3 * float(np.median(times))
        # the same step captured once into a HIP graph and replayed (what a
        # serving loop does): the launch gaps between the kernels go away
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.decode_paged(xd, yd, ctx_d, tab, max_ctx, dkv)
        torch.cuda.synchronize()
        gtimes = timed(graph.replay, args.decode_steps)
        assert torch.equal(yd, y_eager), "graph replay differs from the eager decode step"
        us_graph = 1e3 * float(np.median(gtimes))
        del graph
        layer.profile_enable(True)
        for _ in range(5):
            torch.sum(flush, dim=0, out=sink)
            layer.decode_paged(xd, yd, ctx_d, tab, max_ctx, dkv)
        torch.cuda.synchronize()
        dprof = layer.profile_read()
        layer.profile_enable(False)
        kv_bytes = int(sum(totals)) * Hkv * D * 2 * 2
        step_bytes = weight_bytes(shape) + kv_bytes + 2 * B * H * 2
        dstage = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in dprof.items()}
        attn_ms = dstage["attn_decode"]
        decode = {"workload": "qwen2.5-7b layer paged decode, batch 64, ctx U[128,4096], bf16 KV, "
                              "block 16, random block permutation; L2/MALL flushed (by a 1 GiB read) between steps",
                  "us_per_step": round(us, 2), "us_p10": round(1e3 * times[len(times) // 10], 2),
                  "us_p90": round(1e3 * times[(9 * len(times)) // 10], 2),
                  "algorithmic_bytes": step_bytes,
                  "hbm_gbs": round(step_bytes / (us * 1e-6) / 1e9, 1),
                  "hbm_frac": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "graph_us_per_step": round(us_graph, 2),
                  "graph_hbm_frac": round(step_bytes / (us_graph * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "attn_kernel": {"bound": "hbm", "avg_launch_ms": round(attn_ms, 4),
                                  "achieved": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(kv_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                  "stages_ms": {k: round(v, 4) for k, v in dstage.items() if v}}
        log(f"decode: {us:.1f} us/step eager, {us_graph:.1f} us/step graph, {decode['hbm_gbs']} GB/s eager")
        assert torch.isfinite(yd.float()).all(), "non-finite decode output"
        del flush

    # ----------------------------------------------- the other workloads
    others = None
    if not args.no_other:
        others = other_workloads(args, torch, synth, tdl, stream, (layer, shape))

    # --------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        n = min(args.cpu_tokens, T)
        log(f"cpu baseline: oracle on {n} prompt tokens")
        wh = {k: v.float().cpu().numpy() for k, v in w.items()}
        W = oracle.expand_weights(shape, wh)
        xh = x[:n].float().cpu().numpy()
        tab_h = table.cpu().numpy()[None, :]
        cache = oracle.PagedCache(n_blk, Hkv, D, "bf16")
        c0 = time.perf_counter()
        oracle.layer_forward(shape, W, xh, [0], [n], [0], tab_h, cache)
        c1 = time.perf_counter()
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        cpu = {"value": round(n / (c1 - c0), 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"float64 numpy oracle, one {n}-token causal prefill of the same layer and "
                         f"weights ({c1 - c0:.1f} s)"}
        log(f"cpu baseline: {cpu['value']} tokens/s on {threads} threads")

    if args.copy_probe:
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 536870912 bytes read and written")

    out = {
        "metric": "layer prefill tokens/s + paged decode us/step; % of MFMA / HBM roofline",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "prefill_call_ms": prefill_call_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA operands, fp32 accumulate; bf16 KV cache",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": f"qwen2.5-7b-shaped decoder layer, causal prefill seq {T}, batch 1, "
                               "QKV bias, bf16 paged KV cache written",
                   "global_batch": 1, "seq_len": T},
        "roofline": roofline,
        "layer_mfma": {"flops_per_step": step_flops, "achieved_tflops": round(layer_tflops, 1),
                       "frac": round(layer_tflops / PEAK_MFMA_TFLOPS, 4)},
        "stages_ms": stage_report,
        "decode": decode,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
