"""Host-side checks of the C-ABI library, no GPU needed: it loads, exports every
function include/tdl.h declares, and its argument checks and block allocator
behave as documented (nothing here launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "transformer_decoder_layer_amd", "libtdl.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libtdl.so not built")


def header_functions():
    src = open(os.path.join(ROOT, "include", "tdl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+\*?([a-z_0-9]+)\s*\(", src,
                                 flags=re.M)))


def test_exports_every_declared_function():
    import transformer_decoder_layer_amd as tdl
    declared = header_functions()
    assert len(declared) >= 17, declared
    assert sorted(tdl.EXPORTS) == declared
    lib = ctypes.CDLL(LIB)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    import transformer_decoder_layer_amd as tdl
    assert tdl._status_string(0) == b"ok"
    assert tdl._status_string(3) == b"capacity exceeded"


def cfg_ok(tdl, **kw):
    base = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=688, rms_eps=1e-6,
                rope_theta=1e4, qkv_bias=1, qk_norm=0, weight_dtype=tdl.TDL_F32, max_tokens=32,
                max_seqs=1, max_position=64)
    base.update(kw)
    return tdl.LayerConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2), (dict(n_q_heads=6, n_kv_heads=4), 1), (dict(n_q_heads=12, n_kv_heads=4), 2),
    (dict(hidden=200), 2), (dict(intermediate=100), 2), (dict(weight_dtype=3), 1),
    (dict(max_tokens=0), 1), (dict(rope_theta=0.0), 1), (dict(weight_dtype=2, intermediate=688), 1),
    (dict(max_seqs=4096, max_tokens=4096), 2), (dict(max_position=300000), 2),
])
def test_layer_create_rejects_bad_config(kw, status):
    import transformer_decoder_layer_amd as tdl
    cfg = cfg_ok(tdl, **kw)
    w = tdl.LayerWeights()
    h = ctypes.c_void_p()
    st = tdl._layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h))
    assert st == status, tdl._last_error()
    assert not h.value


def test_layer_create_rejects_missing_weights():
    import transformer_decoder_layer_amd as tdl
    cfg = cfg_ok(tdl)
    w = tdl.LayerWeights()
    h = ctypes.c_void_p()
    assert tdl._layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)) == tdl.TDL_E_INVALID
    assert b"NULL" in tdl._last_error()


def test_null_handles_are_invalid():
    import transformer_decoder_layer_amd as tdl
    assert tdl._layer_prefill(None, None, 1, 2, 4, 0, None, None) == tdl.TDL_E_INVALID
    assert tdl._layer_decode(None, None, 1, 2, 4, 3, 5, 1, 16, 6) == tdl.TDL_E_INVALID
    assert tdl._layer_destroy(None) == tdl.TDL_OK
    assert tdl._kv_free(None) == tdl.TDL_OK


def test_stack_argument_checks():
    import transformer_decoder_layer_amd as tdl
    h = ctypes.c_void_p(123)
    assert tdl._stack_create(None, 2, ctypes.byref(h)) == tdl.TDL_E_INVALID
    assert not h.value                           # *out cleared on failure
    null_layers = (ctypes.c_void_p * 2)(None, None)
    assert tdl._stack_create(null_layers, 2, ctypes.byref(h)) == tdl.TDL_E_INVALID
    assert tdl._stack_create(null_layers, 0, ctypes.byref(h)) == tdl.TDL_E_INVALID
    assert tdl._stack_decode(None, None, 1, 2, 4, 3, 5, 1, 16, None) == tdl.TDL_E_INVALID
    assert tdl._stack_destroy(None) == tdl.TDL_OK


def test_kv_cache_bytes():
    import transformer_decoder_layer_amd as tdl
    c = tdl.KvConfig(100, 16, 4, 128, tdl.TDL_BF16, 0)
    assert tdl._kv_bytes(ctypes.byref(c)) == 2 * 100 * 4 * 16 * 128 * 2
    c = tdl.KvConfig(100, 16, 8, 128, tdl.TDL_U8_ASYM, 0)
    assert tdl._kv_bytes(ctypes.byref(c)) == 2 * 100 * 8 * 16 * 128 + 4 * 8 * 128 * 4
    # u4: two codes per byte (half the u8 pool), the same parameter arrays
    c = tdl.KvConfig(100, 16, 8, 128, tdl.TDL_U4_ASYM, 0)
    assert tdl._kv_bytes(ctypes.byref(c)) == 2 * 100 * 8 * 16 * 64 + 4 * 8 * 128 * 4
    assert tdl._kv_bytes(ctypes.byref(tdl.KvConfig(100, 16, 8, 96, tdl.TDL_U4_ASYM, 0))) == 0
    assert tdl._kv_bytes(ctypes.byref(tdl.KvConfig(100, 16, 8, 128, 5, 0))) == 0
    assert tdl._kv_bytes(ctypes.byref(tdl.KvConfig(100, 32, 4, 128, tdl.TDL_BF16, 0))) == 0
    assert tdl._kv_bytes(ctypes.byref(tdl.KvConfig(0, 16, 4, 128, tdl.TDL_BF16, 0))) == 0


def test_kv_cache_view_strides():
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(10, 4, 128)
    v = kv.view()
    assert list(v.k_strides) == [4 * 16 * 128, 16 * 128, 128, 1]
    assert list(v.v_strides) == [4 * 16 * 128, 16 * 128, 1, 16]
    assert v.v_pool - v.k_pool == 10 * 4 * 16 * 128 * 2
    assert v.elem_bytes == 2 and not v.k_scale
    kv.close()
    # u4: byte strides, D/2 bytes per K row and per V channel-pair column
    kv = tdl.KvCache.host_only(10, 4, 128, "u4")
    v = kv.view()
    assert list(v.k_strides) == [4 * 16 * 64, 16 * 64, 64, 1]
    assert list(v.v_strides) == [4 * 16 * 64, 16 * 64, 1, 16]
    assert v.v_pool - v.k_pool == 10 * 4 * 16 * 64
    assert v.elem_bytes == 0 and v.k_scale and v.v_zero_point
    assert v.k_zero_point - v.k_scale == 4 * 128 * 4
    kv.close()


def test_kv_calibrate_rejects_bf16_cache():
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(10, 4, 128)
    assert tdl._kv_calibrate(kv.handle, None, 1 << 20, 1 << 20, 16) == tdl.TDL_E_INVALID
    assert b"TDL_U4_ASYM" in tdl._last_error()
    kv.close()


def test_block_table_identity_order_and_extension():
    # [TFF 3.6.4]: LIFO free list, ceil(n/16) pages per sequence; existing
    # entries are kept when a sequence grows
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(10, 2, 64)
    t = kv.block_table([1, 16, 17], 4)
    assert t.tolist() == [[0, -1, -1, -1], [1, -1, -1, -1], [2, 3, -1, -1]]
    assert kv.free_blocks() == 6
    t = kv.block_table([16, 33, 17], 4, t)     # seq 1 grows past 32 tokens
    assert t.tolist() == [[0, -1, -1, -1], [1, 4, 5, -1], [2, 3, -1, -1]]
    assert kv.free_blocks() == 4
    kv.release([4, 5])
    assert kv.free_blocks() == 6
    t2 = kv.block_table([20], 4)
    assert t2.tolist() == [[5, 4, -1, -1]]    # LIFO: last released comes back first


def test_block_table_all_or_nothing():
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(5, 2, 64)
    t = np.full((2, 4), -1, np.int32)
    with pytest.raises(tdl.TdlError) as e:
        kv.block_table([48, 48], 4, t)          # needs 6 > 5 blocks
    assert e.value.status == tdl.TDL_E_CAPACITY
    assert (t == -1).all() and kv.free_blocks() == 5
    with pytest.raises(tdl.TdlError) as e:
        kv.block_table([80], 4)                 # 5 blocks > max_blocks 4
    assert e.value.status == tdl.TDL_E_INVALID
    assert kv.free_blocks() == 5


def test_block_release_errors():
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(5, 2, 64)
    kv.block_table([32], 2)
    with pytest.raises(tdl.TdlError):
        kv.release([2])                         # never allocated
    with pytest.raises(tdl.TdlError):
        kv.release([0, 0])                      # double release in one call
    with pytest.raises(tdl.TdlError):
        kv.release([7])                         # out of range
    assert kv.free_blocks() == 3
    kv.release([0, 1])
    with pytest.raises(tdl.TdlError):
        kv.release([1])                         # already free
    assert kv.free_blocks() == 5


def test_seeded_free_list_is_a_permutation():
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(300, 2, 64, seed=1234)
    t = kv.block_table([300 * 16], 300)
    assert sorted(t[0].tolist()) == list(range(300))
    assert t[0].tolist() != list(range(300))
    kv2 = tdl.KvCache.host_only(300, 2, 64, seed=1234)
    assert kv2.block_table([300 * 16], 300).tolist() == t.tolist()


def test_kv_alloc_rejects_unaligned_memory_and_bad_block_size():
    import transformer_decoder_layer_amd as tdl
    c = tdl.KvConfig(4, 16, 2, 64, tdl.TDL_BF16, 0)
    h = ctypes.c_void_p()
    assert tdl._kv_alloc(ctypes.byref(c), 0x100010, ctypes.byref(h)) == tdl.TDL_E_INVALID
    c = tdl.KvConfig(4, 32, 2, 64, tdl.TDL_BF16, 0)
    assert tdl._kv_alloc(ctypes.byref(c), 0x100000, ctypes.byref(h)) == tdl.TDL_E_UNSUPPORTED
