"""rope_fused layers: the prefill rows' queries go from the QKV projection
into the prefill attention kernel, which adds the bias (A8W8 layers), the
Qwen3 Q-norm and RoPE as it loads them ([TFF] 3.7.2 item 4: RoPE applied
while Q is loaded).  Against the oracle, stage by stage (the attention
output checks the fused query path): bf16 prefill with a QKV bias (no cache,
paged, a chunk after cached tokens), a Qwen3-shaped prefill and mixed step
(Q-norm; the decode rows keep the RoPE kernel's q), a u8 cache, Q8_0 and
A8W8 layers, mid-sized layers whose QKV projection is split along K
(their prefill queries take the RoPE kernel's path, which sums the slices in
order and adds the bias), and u4 and per-block-scaled u8 / u4 caches."""
import dataclasses

import pytest

import synth
from test_gpu_a8w8_layer import TINY_A8
from test_gpu_layer import TINY_Q3, TINY_Q80, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.mark.parametrize("T", [1, 45, 150])
def test_fused_prefill_bias(T):
    inp = synth.make_inputs(synth.WORKLOADS["tiny_prefill_32"], seed=120 + T, prefill_len=T, random_gains=True)
    check_layer(inp, what=f"fused prefill {T}, no cache", rope_fused=True)
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=130 + T, prefill_len=T, prefill_start=37, spare_blocks=1,
                            random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what=f"fused chunk {T} at 37", rope_fused=True)
    check_cache_rows(inp, kv, cache, [0])


def test_fused_qwen3_prefill_mixed_u8():
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_Q3, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=140, prefill_len=100, spare_blocks=1, random_gains=True)
    check_layer(inp, what="fused qwen3 prefill 100", rope_fused=True)
    wm = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3, kv_dtype="u8")
    inp = synth.make_inputs(wm, seed=141, prefill_len=70, decode_batch=4, decode_ctx=[3, 16, 40, 129],
                            random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what="fused qwen3 mixed u8", rope_fused=True)
    check_cache_rows(inp, kv, cache, range(5))


def test_fused_q80_and_a8w8():
    wm = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q80)
    inp = synth.make_inputs(wm, seed=142, prefill_len=160, decode_batch=3, decode_ctx=[5, 16, 77],
                            random_gains=True)
    check_layer(inp, what="fused q80 mixed", rope_fused=True)
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_A8, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=143, prefill_len=150, spare_blocks=1, random_gains=True)
    check_layer(inp, what="fused a8w8 prefill 150", rope_fused=True)


# hidden 1024 (8 / 2 heads, QKV bias) and 2048 (16 / 4 heads, Q/K-norm): at
# 150 and 300 rows their QKV projections run as 4, 4 and 5 split-K slices
MID_Q25 = dataclasses.replace(synth.QWEN25_7B, name="mid-qwen2.5", hidden=1024, n_q_heads=8,
                              n_kv_heads=2, intermediate=2816)
MID_Q3 = dataclasses.replace(synth.QWEN3_8B, name="mid-qwen3", hidden=2048, n_q_heads=16,
                             n_kv_heads=4, intermediate=5632)


@pytest.mark.parametrize("shape,T", [(MID_Q25, 150), (MID_Q25, 300), (MID_Q3, 150)])
def test_fused_split_qkv(shape, T):
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=shape, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=150 + T, prefill_len=T, prefill_start=20, spare_blocks=1,
                            random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what=f"fused {shape.name} split QKV, chunk {T} at 20",
                                            rope_fused=True)
    check_cache_rows(inp, kv, cache, [0])


# the fused query path over coded caches: u4, and per-block x per-channel
# u8 / u4 (the chunk's own keys come from the staging copy, which holds the
# block-scaled values; the cached ones are dequantised with their blocks'
# factors).  u4 checks y and the cache (its quantisation noise in o is above
# the stage bar), as the other u4 tests do.
@pytest.mark.parametrize("kvd,bs", [("u4", False), ("u8", True), ("u4", True)])
def test_fused_mixed_step_over_coded_caches(kvd, bs):
    from test_gpu_kv_block_scales import _check_exponents, _narrow_calibration
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3, kv_dtype=kvd)
    inp = synth.make_inputs(wl, seed=170 + 2 * bs + (kvd == "u4"), prefill_len=90, decode_batch=4,
                            decode_ctx=[3, 16, 40, 129], random_gains=True)
    if bs:
        inp = _narrow_calibration(inp, 175)
    what = f"fused mixed {kvd}{' block scales' if bs else ''}"
    layer, kv, t, cache, rows = check_layer(inp, what=what, rope_fused=True, stages=kvd == "u8")
    check_cache_rows(inp, kv, cache, range(5))
    if bs:
        _check_exponents(inp, kv, cache, range(5))


def test_fused_u4_chunk_after_cached_tokens():
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_Q3, kv_dtype="u4")
    inp = synth.make_inputs(wl, seed=178, prefill_len=100, prefill_start=37, spare_blocks=1, random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what="fused u4 chunk 100 at 37", rope_fused=True, stages=False)
    check_cache_rows(inp, kv, cache, [0])
