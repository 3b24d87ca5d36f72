"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark uses.  Where the oracle would take minutes the
check runs on a sample of rows or sequences (the oracle still writes every
row's K/V into its cache and calibrates u8 / u4 on every cached token)."""
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


def _check(inp, seqs=None, rows_out=None, what=""):
    import torch
    print(f"[{what}] gpu", flush=True)
    layer, kv, t = gpu_setup(inp)
    gpu_call(inp, layer, kv, t)
    torch.cuda.synchronize()
    y = t["y"].float().cpu().numpy()
    print(f"[{what}] oracle", flush=True)
    rows, ref, _ = run_oracle(inp, seqs, rows_out=rows_out)
    e = compare(y[rows], ref)
    print(f"[{what}] {len(rows)} rows: {e}", flush=True)
    assert e.ok, f"{what}: {e}"


def test_tiny_prefill_32_full():
    _check(synth.make_inputs(synth.WORKLOADS["tiny_prefill_32"]), what="tiny prefill 32")


def test_qwen25_prefill_4096_sampled_rows():
    inp = synth.make_inputs(synth.WORKLOADS["qwen25_prefill_4096"])
    rows = [0, 1, 31, 32, 63, 64, 1000, 2047, 2048, 3001, 4064, 4094, 4095]
    _check(inp, [0], rows_out=rows, what="qwen2.5 prefill 4096")


def test_qwen25_decode_b64_full():
    _check(synth.make_inputs(synth.WORKLOADS["qwen25_decode_b64"]), what="qwen2.5 decode b64")


def test_qwen3_decode_u8_b128_sampled_seqs():
    # norm gains N(1, 0.1) (ln1, ln2, q_norm, k_norm) at the full size
    inp = synth.make_inputs(synth.WORKLOADS["qwen3_decode_u8_b128"], random_gains=True)
    ctx = inp.batch.ctx_len
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 0, 17, 64, 101, 127})
    _check(inp, seqs, what="qwen3 u8 decode b128")


def test_qwen3_decode_u4_b128_sampled_seqs():
    inp = synth.make_inputs(synth.WORKLOADS["qwen3_decode_u4_b128"])
    ctx = inp.batch.ctx_len
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 0, 17, 64, 101, 127})
    _check(inp, seqs, what="qwen3 u4 decode b128")


def test_qwen25_iq8_decode_b64_full():
    _check(synth.make_inputs(synth.WORKLOADS["qwen25_iq8_decode_b64"]), what="qwen2.5 iq8 decode b64")


def test_qwen3_q80_mixed_sampled():
    inp = synth.make_inputs(synth.WORKLOADS["qwen3_q80_mixed"])
    # sequence 0 is the 2048-token chunk (rows 0..2047), then 64 decode rows
    rows = [0, 1, 700, 2046, 2047, 2048, 2049, 2100, 2111]
    seqs = [0, 1, 2, 53, 64]
    _check(inp, seqs, rows_out=rows, what="qwen3 q8_0 mixed")


def test_qwen25_decode_b64_longest_partition():
    # one sequence at ctx 4096 (4097 keys = 257 blocks) with 64 x 4 (sequence,
    # KV head) pairs: a single 257-block partition, so one wave walks 65
    # blocks and takes its last block-table entry from the second table load
    wl = synth.WORKLOADS["qwen25_decode_b64"]
    ctx = [int(c) for c in synth.context_lengths(np.random.default_rng(7), wl)]
    ctx[5], ctx[40] = 4096, 4095
    inp = synth.make_inputs(wl, seed=8, decode_ctx=ctx)
    _check(inp, [0, 5, 40, 63], what="qwen2.5 decode b64, ctx 4096")
