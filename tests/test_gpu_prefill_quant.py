"""Prefill attention over u8 / u4 (per-channel asymmetric) caches and the
paths of the prefill kernel: a prompt from position 0 (the chunk's own keys
through the kernel's fp16 staging copy, which must hold what the cache holds),
a chunk after cached tokens (those gathered from the coded cache and
dequantised), a mixed step, and a step with more prefill sequences than get
a staging copy (the rest read their own chunk back from the cache).  Against
the oracle, which stores every new K/V in the cache's format and reads every
key from the cache ([HET] 2.4 / 2.6: int8 and uint4 KV with per-channel
scales; 2.2 / 4.7: chunked prefill, prefill over a cached prefix)."""
import dataclasses

import numpy as np
import pytest

import synth
from test_gpu_layer import TINY_Q3, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu

TINY_D128 = dataclasses.replace(synth.TINY, name="tiny-d128-q", hidden=512, n_q_heads=7, n_kv_heads=1,
                                head_dim=128, intermediate=1024, weight_dtype="bf16", rope_theta=1e6,
                                qkv_bias=False, qk_norm=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def _calibration(inp, seed, k_std=1.0, v_std=0.35):
    # parameters from a sample of the layer's K / V distribution (unit RMS
    # after the per-head norm; V about 0.3), the same for the GPU and the oracle
    rng = np.random.default_rng(seed)
    s = inp.workload.shape
    k = rng.standard_normal((512, s.n_kv_heads, s.head_dim)).astype(np.float32) * k_std
    v = rng.standard_normal((512, s.n_kv_heads, s.head_dim)).astype(np.float32) * v_std
    return dataclasses.replace(inp, calib_k=k, calib_v=v)


# A new token's code depends on its K / V before quantisation, which the GPU
# computes in fp32 from fp16 operands and the oracle in float64: values within
# about 1e-4 of a rounding boundary may take neighbouring codes (the cache
# check allows one code on under 5% of them).  With every key a new token (a
# prompt from position 0) one such step moves a whole attention row, by one
# quantum -- at u4, a third of a typical value -- so two inputs: the standard
# draws at u8 (quantum about 1% of the range of the values), checked stage by
# stage, and at u4 end to end; and, for both formats, inputs whose K / V the
# two sides compute to within about 1e-7 (x rows with H/256 entries of +-64,
# unit RMSNorm-1 gain: RMSNorm-1 gives +-16 there exactly in fp16), checked
# stage by stage with the chunk's codes bit for bit.

@pytest.mark.parametrize("shape", [TINY_Q3, TINY_D128], ids=lambda s: s.name)
def test_prefill_from_zero_over_u8_cache(shape):
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype="u8")
    for T in (1, 77, 150):
        inp = _calibration(synth.make_inputs(wl, seed=100 + T, prefill_len=T, spare_blocks=2,
                                             random_gains=True), 200 + T)
        layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {T} from 0, u8 {shape.name}")
        check_cache_rows(inp, kv, cache, [0])


@pytest.mark.parametrize("shape", [TINY_Q3, TINY_D128], ids=lambda s: s.name)
def test_prefill_from_zero_over_u4_cache_end_to_end(shape):
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype="u4")
    for T in (1, 77, 150):
        inp = _calibration(synth.make_inputs(wl, seed=110 + T, prefill_len=T, spare_blocks=2,
                                             random_gains=True), 210 + T)
        layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {T} from 0, u4 {shape.name}",
                                                stages=False)
        check_cache_rows(inp, kv, cache, [0])


def _one_hot_rows(inp, seed):
    # H/256 entries of +-64 per row: mean square 16, so RMSNorm-1 (gain 1)
    # gives exactly +-16 there and 0 elsewhere
    rng = np.random.default_rng(seed)
    T, H = inp.x.shape
    n = H // 256
    x = np.zeros((T, H), np.float32)
    for r in range(T):
        cols = rng.choice(H, n, replace=False)
        x[r, cols] = np.where(rng.random(n) < 0.5, -64.0, 64.0)
    w = dict(inp.weights, ln1=np.ones_like(inp.weights["ln1"]))
    return dataclasses.replace(inp, x=x, weights=w)


@pytest.mark.parametrize("kvd", ["u8", "u4"])
@pytest.mark.parametrize("shape", [TINY_Q3, TINY_D128], ids=lambda s: s.name)
def test_prefill_from_zero_coded_cache_exact_codes(kvd, shape):
    import torch
    from harness import unpack_u4
    import oracle
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype=kvd)
    for T in (1, 77, 150):
        inp = synth.make_inputs(wl, seed=120 + T, prefill_len=T, spare_blocks=2, random_gains=True)
        inp = _calibration(_one_hot_rows(inp, 220 + T), 320 + T)
        layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {T} from 0, {kvd} exact {shape.name}")
        kt, vt = kv.tensors()[:2]
        if kvd == "u4":
            kt, vt = map(torch.from_numpy, unpack_u4(kt, vt))
        for p in range(T):
            blk, off = oracle.PagedCache.location(inp.batch.table[0], p)
            assert np.array_equal(kt[blk, :, off, :].cpu().numpy(), cache.k[blk, :, off, :]), (T, p, "K")
            assert np.array_equal(vt[blk, :, :, off].cpu().numpy(), cache.v[blk, :, off, :]), (T, p, "V")


@pytest.mark.parametrize("kvd", ["u8", "u4"])
def test_chunk_after_cached_tokens_coded_cache(kvd):
    # keys 0..P-1 come from the coded cache (the kernel's gather path), the
    # chunk's own from its staging copy; parameters calibrated on the cached
    # tokens
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_Q3, kv_dtype=kvd)
    for P, T in ((83, 37), (16, 100), (200, 64)):
        inp = synth.make_inputs(wl, seed=300 + P, prefill_len=T, prefill_start=P, spare_blocks=1,
                                random_gains=True)
        layer, kv, t, cache, rows = check_layer(inp, what=f"chunk {T} at {P}, {kvd}")
        check_cache_rows(inp, kv, cache, [0])


@pytest.mark.parametrize("kvd", ["u8", "u4"])
def test_mixed_step_coded_cache(kvd):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3, kv_dtype=kvd)
    inp = synth.make_inputs(wl, seed=41, prefill_len=90, decode_batch=5, decode_ctx=[3, 16, 40, 129, 500],
                            random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what=f"mixed {kvd}")
    check_cache_rows(inp, kv, cache, range(6))


@pytest.mark.parametrize("kvd", ["bf16", "u8"])
def test_more_prefill_sequences_than_staged(kvd):
    # 70 prefill sequences (q_len 1..6, some after cached tokens) and 3 decode
    # rows in one step: sequences 64.. read their own chunk back from the cache
    import torch
    import harness
    shape = TINY_Q3
    rng = np.random.default_rng(51)
    n_pre = 70
    q_len = [int(x) for x in rng.integers(1, 7, n_pre)] + [1, 1, 1]
    ctx = [int(x) for x in rng.integers(0, 40, n_pre)] + [5, 70, 300]
    b = synth.make_batch(rng, q_len[:n_pre], ctx[:n_pre], ctx[n_pre:], spare_blocks=2)
    w = synth.make_weights(shape, seed=52, random_gains=True)
    x = synth.make_x(rng, b.n_rows, shape.hidden)
    n_cached = int(b.ctx_len.sum())
    kvv = synth.cached_kv(rng, n_cached, shape.n_kv_heads, shape.head_dim, bf16=(kvd == "bf16"))
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=shape, kv_dtype=kvd,
                             prefill_len=0, decode_batch=3)
    inp = synth.LayerInputs(wl, w, x, b, kvv["k"], kvv["v"])
    layer, kv, t = harness.gpu_setup(inp)
    layer.step(t["x"], t["y"], t["q_start"], t["q_len"], t["ctx_len"], t["table"], n_pre, max(q_len[:n_pre]),
               int((b.ctx_len + b.q_len).max()), kv)
    torch.cuda.synchronize()
    rows, ref, cache = harness.run_oracle(inp)
    e = harness.compare(t["y"].float().cpu().numpy()[rows], ref)
    print(f"[{n_pre} prefill seqs, {kvd}] {e}", flush=True)
    assert e.ok, e


# 1024 rows and more: the RoPE/KV kernel takes four rows per workgroup (the
# loads of all four issued before any is rotated or stored); rows of a group
# may belong to different sequences (the mixed step: the chunk's last rows
# and the first decode rows)
@pytest.mark.parametrize("kvd", ["u8", "u4"])
def test_long_prefill_coded_cache_four_rows_per_workgroup(kvd):
    import torch
    from harness import unpack_u4
    import oracle
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_Q3, kv_dtype=kvd)
    T = 1030
    inp = synth.make_inputs(wl, seed=130, prefill_len=T, spare_blocks=2, random_gains=True)
    inp = _calibration(_one_hot_rows(inp, 230), 330)
    layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {T} from 0, {kvd} exact")
    kt, vt = kv.tensors()[:2]
    if kvd == "u4":
        kt, vt = map(torch.from_numpy, unpack_u4(kt, vt))
    for p in range(T):
        blk, off = oracle.PagedCache.location(inp.batch.table[0], p)
        assert np.array_equal(kt[blk, :, off, :].cpu().numpy(), cache.k[blk, :, off, :]), (p, "K")
        assert np.array_equal(vt[blk, :, :, off].cpu().numpy(), cache.v[blk, :, off, :]), (p, "V")


@pytest.mark.parametrize("kvd", ["bf16", "u8"])
def test_long_mixed_step_four_rows_per_workgroup(kvd):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3, kv_dtype=kvd)
    inp = synth.make_inputs(wl, seed=140, prefill_len=1041, decode_batch=6,
                            decode_ctx=[3, 16, 40, 129, 500, 7], random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what=f"mixed 1041 + 6, {kvd}")
    check_cache_rows(inp, kv, cache, range(7))
