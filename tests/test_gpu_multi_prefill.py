"""Mixed steps with several prefill chunks of different lengths in one call
(some after cached tokens, one of a single 32-key tile, one of five) next
to decode rows: the per-sequence staging of the chunks' K/V, the prefill
attention's walk over (sequence, query tile) pairs across sequences, the
queries rotated in the attention kernel (rope_fused) for several sequences,
and the RoPE/KV kernel's slot writes for every sequence.  Against the oracle
stage by stage, and every new token's K/V in the cache ([TFF] section
3.6.1: the scheduler's batch of prefill and decode sequences in one
step)."""
import dataclasses

import numpy as np
import pytest

import synth
from test_gpu_layer import TINY_Q3, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def _inputs(shape, kvd, seed):
    rng = np.random.default_rng(seed)
    q_len = [33, 70, 2, 130]     # chunks of 2, 3, 1 and 5 query tiles
    start = [0, 16, 50, 7]       # cached tokens before each chunk
    dctx = [5, 64, 300]          # decode rows
    b = synth.make_batch(rng, q_len, start, dctx, spare_blocks=2)
    w = synth.make_weights(shape, seed=seed + 1, random_gains=True)
    x = synth.make_x(rng, b.n_rows, shape.hidden, bf16=(shape.weight_dtype != "f32"))
    n_cached = int(b.ctx_len.sum())
    kvv = synth.cached_kv(rng, n_cached, shape.n_kv_heads, shape.head_dim, bf16=(kvd == "bf16"))
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=shape, kv_dtype=kvd,
                             prefill_len=0, decode_batch=len(dctx))
    return synth.LayerInputs(wl, w, x, b, kvv["k"], kvv["v"])


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("shape,kvd", [(synth.TINY, "bf16"), (TINY_Q3, "u8")])
def test_several_prefill_chunks_and_decode_rows(shape, kvd, fused):
    inp = _inputs(shape, kvd, seed=61)
    what = f"{shape.name} {kvd}, 4 chunks + 3 decode rows{', fused query RoPE' if fused else ''}"
    layer, kv, t, cache, rows = check_layer(inp, what=what, rope_fused=fused)
    check_cache_rows(inp, kv, cache, range(7))
