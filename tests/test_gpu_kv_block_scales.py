"""Per-block x per-channel KV caches (tdl_kv_config.block_scales) against
the oracle's PagedCache(block_scales=True): the per-block factor exponents
and codes that kv_cache_write stores (bit for bit: both sides quantise the
same float32 inputs), and the layer's prefill, chunked-prefill, decode and
mixed steps over such caches, stage by stage at u8 and end to end at u4
([HET] 2.4: scales managed per channel and per block; 4.3: a block
dequantised with its own scales).  The per-channel parameters come from a
narrower sample than the cached and new K / V, so blocks take factors above
1."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from harness import unpack_u4
from test_gpu_layer import TINY_D128, TINY_Q3, check_cache_rows, check_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_decoder_layer_amd  # noqa: F401  (fails loudly if the library is missing)


def _narrow_calibration(inp, seed, k_std=0.35, v_std=0.12):
    rng = np.random.default_rng(seed)
    s = inp.workload.shape
    k = rng.standard_normal((256, s.n_kv_heads, s.head_dim)).astype(np.float32) * k_std
    v = rng.standard_normal((256, s.n_kv_heads, s.head_dim)).astype(np.float32) * v_std
    return dataclasses.replace(inp, calib_k=k, calib_v=v, block_scales=True)


def _codes(kv, kvd):
    import torch
    kt, vt = kv.tensors()[:2]
    if kvd == "u4":
        kt, vt = map(torch.from_numpy, unpack_u4(kt, vt))
    return kt.cpu().numpy(), vt.cpu().numpy()


@pytest.mark.parametrize("kvd", ["u8", "u4"])
def test_kv_write_exponents_and_codes_bit_exact(kvd):
    import torch
    import transformer_decoder_layer_amd as tdl
    print(f"[kv write block scales {kvd}]", flush=True)
    Hkv, D = 2, 64
    rng = np.random.default_rng(31)
    calib = rng.standard_normal((128, Hkv, D)).astype(np.float32)
    ctx = [20, 16, 37, 5]
    mult = [1.0, 3.0, 10.0, 200.0]  # the last beyond 2^7 times the range: the largest factor, clamped
    ks = [(rng.standard_normal((c, Hkv, D)) * m).astype(np.float32) for c, m in zip(ctx, mult)]
    vs = [(rng.standard_normal((c, Hkv, D)) * m * 0.5).astype(np.float32) for c, m in zip(ctx, mult)]
    n_blocks = 16
    table = synth.random_tables(np.random.default_rng(32), [c + 20 for c in ctx], n_blocks=n_blocks)
    kv = tdl.KvCache(n_blocks, Hkv, D, kvd, block_scales=True)
    kc = torch.from_numpy(calib).cuda()
    kv.calibrate(kc, kc)
    bits = 4 if kvd == "u4" else 8
    params = oracle.kv_calibrate(calib, bits)
    ref = oracle.PagedCache(n_blocks, Hkv, D, kvd, params, params, block_scales=True)
    tab = torch.from_numpy(table).cuda()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)).cuda()
    kv.write(cu, torch.zeros(len(ctx), dtype=torch.int32, device="cuda"), tab,
             torch.from_numpy(np.concatenate(ks)).cuda(), torch.from_numpy(np.concatenate(vs)).cuda())
    for i in range(len(ctx)):
        ref.write_tokens(table[i], 0, ks[i], vs[i])
    # a second call appends 6 tokens to sequences 0 and 2 (mid-block: the
    # factors stay) and 12 to sequence 1 (a new block: its own factor)
    add = [6, 12, 6, 0]
    ks2 = [(rng.standard_normal((a, Hkv, D)) * 4.0).astype(np.float32) for a in add]
    vs2 = [(rng.standard_normal((a, Hkv, D)) * 2.0).astype(np.float32) for a in add]
    cu2 = torch.from_numpy(np.concatenate([[0], np.cumsum(add)]).astype(np.int32)).cuda()
    kv.write(cu2, torch.from_numpy(np.array(ctx, np.int32)).cuda(), tab,
             torch.from_numpy(np.concatenate(ks2)).cuda(), torch.from_numpy(np.concatenate(vs2)).cuda())
    for i in range(len(ctx)):
        ref.write_tokens(table[i], ctx[i], ks2[i], vs2[i])
    torch.cuda.synchronize()
    ex = kv.block_exponents().cpu().numpy()
    used = sorted({int(table[i][p // 16]) for i in range(len(ctx)) for p in range(ctx[i] + add[i])})
    assert ref.ek[used].max() >= 3 and ref.ek[used].max() == oracle.KV_MAX_BLOCK_EXP
    assert np.array_equal(ex[used, :, 0], ref.ek[used]) and np.array_equal(ex[used, :, 1], ref.ev[used])
    kg, vg = _codes(kv, kvd)
    for i in range(len(ctx)):
        for p in range(ctx[i] + add[i]):
            blk, off = oracle.PagedCache.location(table[i], p)
            assert np.array_equal(kg[blk, :, off, :], ref.k[blk, :, off, :]), (i, p, "K")
            assert np.array_equal(vg[blk, :, :, off], ref.v[blk, :, off, :]), (i, p, "V")


def _check_exponents(inp, kv, cache, seqs):
    """Cached tokens' blocks: factor exponents bit for bit (the same float32
    inputs); blocks opened by this call's new tokens (from K / V the two
    sides compute in different precisions): within one."""
    ex = kv.block_exponents().cpu().numpy()
    b = inp.batch
    for i in seqs:
        c, n = int(b.ctx_len[i]), int(b.q_len[i])
        for lb in range((c + n + 15) // 16):
            blk = int(b.table[i][lb])
            d_k = np.abs(ex[blk, :, 0].astype(int) - cache.ek[blk])
            d_v = np.abs(ex[blk, :, 1].astype(int) - cache.ev[blk])
            if 16 * lb < c:
                assert not d_k.any() and not d_v.any(), (i, lb)
            else:
                assert d_k.max() <= 1 and d_v.max() <= 1, (i, lb)


def test_decode_over_block_scaled_u8_cache():
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_decode_u8_b128"], shape=TINY_Q3)
    ctx = [0, 1, 15, 16, 17, 64, 300, 777]
    inp = _narrow_calibration(synth.make_inputs(wl, seed=41, decode_batch=len(ctx), decode_ctx=ctx,
                                                random_gains=True), 42)
    layer, kv, t, cache, rows = check_layer(inp, what="decode u8 block scales")
    assert cache.ek.max() >= 1 and cache.ev.max() >= 1
    check_cache_rows(inp, kv, cache, range(len(ctx)))
    _check_exponents(inp, kv, cache, range(len(ctx)))


@pytest.mark.parametrize("shape", [TINY_Q3, TINY_D128], ids=lambda s: s.name)
def test_decode_over_block_scaled_u4_cache_end_to_end(shape):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_decode_u4_b128"], shape=shape)
    ctx = [0, 1, 15, 16, 17, 64, 300, 777]
    inp = _narrow_calibration(synth.make_inputs(wl, seed=43, decode_batch=len(ctx), decode_ctx=ctx,
                                                random_gains=True), 44)
    layer, kv, t, cache, rows = check_layer(inp, what=f"decode u4 block scales {shape.name}", stages=False)
    check_cache_rows(inp, kv, cache, range(len(ctx)))
    _check_exponents(inp, kv, cache, range(len(ctx)))


@pytest.mark.parametrize("kvd", ["u8", "u4"])
def test_prefill_over_block_scaled_cache(kvd):
    # from position 0 (the chunk's keys through the staging copy, which holds
    # the block-scaled values) and after cached tokens (gathered and
    # dequantised with their blocks' factors)
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_32"], shape=TINY_Q3, kv_dtype=kvd)
    # (1030 and 1100 rows: the RoPE/KV kernel's four rows per workgroup,
    # after the one-row exponent pass)
    for P, T in ((0, 77), (0, 150), (83, 37), (16, 100), (0, 1030), (83, 1100)):
        inp = synth.make_inputs(wl, seed=50 + P + T, prefill_len=T, prefill_start=P, spare_blocks=2,
                                random_gains=True)
        inp = _narrow_calibration(inp, 51 + P + T)
        layer, kv, t, cache, rows = check_layer(inp, what=f"prefill {T} at {P}, {kvd} block scales",
                                                stages=kvd == "u8")
        check_cache_rows(inp, kv, cache, [0])
        _check_exponents(inp, kv, cache, [0])


def test_mixed_step_over_block_scaled_u8_cache():
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_q80_mixed"], shape=TINY_Q3, kv_dtype="u8")
    inp = synth.make_inputs(wl, seed=60, prefill_len=90, decode_batch=5, decode_ctx=[3, 16, 40, 129, 500],
                            random_gains=True)
    inp = _narrow_calibration(inp, 61)
    layer, kv, t, cache, rows = check_layer(inp, what="mixed u8 block scales")
    check_cache_rows(inp, kv, cache, range(6))
    _check_exponents(inp, kv, cache, range(6))
