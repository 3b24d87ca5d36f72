"""Layers on the A8W8 path (int8 activations x int8 weights, [HET] 4.5)
against the oracle's A8W8 projections (oracle.A8W8Weight), stage by stage:
prefill without a cache and into a paged cache, decode, a mixed step, and a
Qwen3-shaped layer over a u8 cache.  Both sides decide the activations'
int8 codes from the values the layer holds (fp16 xn / o / hn, bf16 a), so
they agree up to the codes of values that the GPU computes a rounding step
away from the oracle's."""
import dataclasses

import pytest

import synth
from test_gpu_layer import TINY_Q3, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu

TINY_A8 = dataclasses.replace(synth.TINY, name="tiny-a8w8", weight_dtype="a8w8")
TINY_Q3_A8 = dataclasses.replace(TINY_Q3, name="tiny-qwen3-a8w8", weight_dtype="a8w8")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.mark.parametrize("T", [1, 32, 150])
def test_a8w8_prefill(T):
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_A8, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=80 + T, prefill_len=T, spare_blocks=1, random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what=f"a8w8 prefill {T}")
    check_cache_rows(inp, kv, cache, [0])


def test_a8w8_prefill_no_cache_and_chunk():
    # Without a cache the oracle attends over exact K / V while the GPU holds
    # them in bf16 for the call: o differs by ~2e-3, and each such difference
    # that moves an fp16 value of o across a rounding boundary of its int8
    # code costs a whole step (max |o| / 127) in the output projection, so
    # h - x differs by several times more (~6e-3).  Checked end to end here;
    # the paged cases (K / V rounded to bf16 on both sides) check every stage.
    inp = synth.make_inputs(dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_A8),
                            seed=84, random_gains=True)
    check_layer(inp, what="a8w8 prefill 32, no cache", stages=False)
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_A8, kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=85, prefill_len=40, prefill_start=83, spare_blocks=1, random_gains=True)
    check_layer(inp, what="a8w8 chunk 40 at 83")


def test_a8w8_decode():
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=TINY_A8)
    ctx = [0, 1, 15, 16, 17, 100, 511]
    inp = synth.make_inputs(wl, seed=86, decode_batch=len(ctx), decode_ctx=ctx, random_gains=True)
    layer, kv, t, cache, rows = check_layer(inp, what="a8w8 decode")
    check_cache_rows(inp, kv, cache, range(len(ctx)))


def test_a8w8_mixed_and_qwen3_u8_decode():
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3_A8)
    inp = synth.make_inputs(wl, seed=87, prefill_len=77, decode_batch=4, decode_ctx=[3, 16, 40, 129],
                            random_gains=True)
    check_layer(inp, what="a8w8 mixed")
    wd = dataclasses.replace(synth.WORKLOADS["qwen3_decode_u8_b128"], shape=TINY_Q3_A8)
    ctx = [1, 16, 64, 300]
    inp = synth.make_inputs(wd, seed=88, decode_batch=len(ctx), decode_ctx=ctx, random_gains=True)
    check_layer(inp, what="a8w8 decode u8")
