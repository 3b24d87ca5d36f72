"""Prefix reuse on the GPU ([HET] 4.7 prefix cache, 4.3 block holders):
sequences whose first blocks are another sequence's blocks, found through the
prefix index, prefill their own chunk at start_pos > 0 and decode over them,
against the oracle computing each sequence from its own logical cache."""
import dataclasses

import numpy as np
import pytest

import synth
from harness import compare, device_weights, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(msg):
    print(msg, flush=True)


def _chain_keys(seed, n):
    # stand-in for a hash chain over the token ids of blocks 0..i
    return [(seed << 32) + i for i in range(n)]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _write(kv, table, start, k, v):
    """Rows k, v [n, Hkv, D] to positions start.. of the sequence with `table`."""
    kv.write(_dev(np.array([0, len(k)], np.int32)), _dev(np.array([start], np.int32)),
             _dev(table[None]), _dev(k), _dev(v))


def test_prefill_chunk_over_shared_prefix():
    import torch
    import transformer_decoder_layer_amd as tdl
    P, T = 96, 40                                # 6 shared full blocks, then B's chunk
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], kv_dtype="bf16")
    inp = synth.make_inputs(wl, seed=31, prefill_len=T, prefill_start=P)
    shape = wl.shape
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=T, max_seqs=2, max_position=1024),
                      device_weights(shape, inp.weights))
    kv = tdl.KvCache(24, shape.n_kv_heads, shape.head_dim, "bf16", seed=5)
    mb = 12
    # sequence A: the P cached tokens, then 24 tokens of its own
    ta = kv.block_table([P + 24], mb)[0]
    rng = np.random.default_rng(32)
    own = rng.standard_normal((2, 24, shape.n_kv_heads, shape.head_dim)).astype(np.float32)
    _write(kv, ta, 0, inp.cache_k, inp.cache_v)
    _write(kv, ta, P, own[0], own[1])
    keys = _chain_keys(7, P // 16)
    kv.prefix_publish(keys, ta[:P // 16])
    # sequence B matches the whole prefix and takes new blocks for its chunk
    m = kv.prefix_match(keys + [12345])
    assert m.tolist() == ta[:P // 16].tolist()
    tb = np.full(mb, -1, np.int32)
    tb[:len(m)] = m
    kv.block_table([P + T], mb, tb[None])
    assert not set(tb[P // 16:(P + T + 15) // 16].tolist()) & set(ta.tolist())
    torch.cuda.synchronize()
    k_before, v_before = [t.clone() for t in kv.tensors()]
    x = torch.from_numpy(inp.x).to(torch.bfloat16).cuda()
    y = torch.full_like(x, float("nan"))
    layer.prefill(x, y, P, kv, _dev(tb))
    torch.cuda.synchronize()
    _, ref, _ = run_oracle(inp)
    e = compare(y.float().cpu().numpy(), ref)
    log(f"[prefix prefill] {e}")
    assert e.ok, e
    # A's blocks (shared and private) are untouched by B's chunk
    k_after, v_after = kv.tensors()
    for blk in map(int, ta[:(P + 24 + 15) // 16]):
        assert torch.equal(k_after[blk], k_before[blk]) and torch.equal(v_after[blk], v_before[blk])
    # holders: A, the index and B on each shared block
    assert [kv.refs(int(b)) for b in m] == [3] * len(m)
    kv.release(ta[:(P + 24 + 15) // 16].tolist())
    assert kv.prefix_evict(100) == 0             # B still holds the prefix
    kv.release(tb[:(P + T + 15) // 16].tolist())
    assert kv.prefix_evict(100) == P // 16 and kv.free_blocks() == 24


@pytest.mark.parametrize("kvd", ["bf16", "u4"])
def test_decode_over_shared_blocks(kvd):
    import torch
    import transformer_decoder_layer_amd as tdl
    P = 96
    ca, cb = 120, 136                            # B = A's first 96 tokens + 40 of its own
    wl = dataclasses.replace(synth.WORKLOADS["qwen25_decode_b64"], shape=synth.TINY, kv_dtype=kvd)
    inp = synth.make_inputs(wl, seed=33, decode_batch=2, decode_ctx=[ca, cb])
    ck, cv = inp.cache_k.copy(), inp.cache_v.copy()
    ck[ca:ca + P], cv[ca:ca + P] = ck[:P], cv[:P]  # B's logical prefix is A's
    inp = dataclasses.replace(inp, cache_k=ck, cache_v=cv)
    shape = wl.shape
    layer = tdl.Layer(tdl.make_config(shape, max_tokens=2, max_seqs=2, max_position=1024),
                      device_weights(shape, inp.weights))
    kv = tdl.KvCache(30, shape.n_kv_heads, shape.head_dim, kvd, seed=9)
    if kvd != "bf16":
        kv.calibrate(_dev(ck), _dev(cv))
    mb = 10
    ta = kv.block_table([ca + 1], mb)[0]         # room for the new token too
    _write(kv, ta, 0, ck[:ca], cv[:ca])
    keys = _chain_keys(11, P // 16)
    kv.prefix_publish(keys, ta[:P // 16])
    tb = np.full(mb, -1, np.int32)
    m = kv.prefix_match(keys)
    tb[:len(m)] = m
    kv.block_table([cb + 1], mb, tb[None])
    _write(kv, tb, P, ck[ca + P:], cv[ca + P:])
    x = torch.from_numpy(inp.x).to(torch.bfloat16).cuda()
    y = torch.full_like(x, float("nan"))
    tables = _dev(np.stack([ta, tb]))
    ctx = _dev(np.array([ca, cb], np.int32))
    layer.decode_paged(x, y, ctx, tables, cb + 1, kv)
    torch.cuda.synchronize()
    _, ref, _ = run_oracle(inp)
    e = compare(y.float().cpu().numpy(), ref)
    log(f"[prefix decode {kvd}] {e}")
    assert e.ok, e
    # A finishes; B decodes on alone over the blocks it still shares with the index
    kv.release(ta[:(ca + 1 + 15) // 16].tolist())
    assert kv.prefix_evict(100) == 0
    y1 = torch.full_like(x[1:], float("nan"))
    layer.decode_paged(x[1:].contiguous(), y1, ctx[1:].contiguous(), tables[1:].contiguous(), cb + 1, kv)
    torch.cuda.synchronize()
    _, ref1, _ = run_oracle(inp, [1])
    e1 = compare(y1.float().cpu().numpy(), ref1)
    log(f"[prefix decode {kvd}, B alone] {e1}")
    assert e1.ok, e1
