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
    (dict(weight_dtype=5, intermediate=688), 1), (dict(weight_dtype=6), 1),
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


def test_layer_create_iq8_needs_scales_and_zero_points():
    # per-row int8 weights: every matrix needs its scale and zero point
    import transformer_decoder_layer_amd as tdl
    cfg = cfg_ok(tdl, weight_dtype=tdl.TDL_I8_ROW, intermediate=704)
    w = tdl.LayerWeights()
    for name in ("ln1", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "ln2", "wg", "wu", "wd"):
        setattr(w, name, 1 << 20)              # never dereferenced: the checks come first
    for m in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        setattr(w, m + "_scale", 1 << 20)
    h = ctypes.c_void_p()
    assert tdl._layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)) == tdl.TDL_E_INVALID
    assert b"_zp" in tdl._last_error() and not h.value


def test_gemm_a8w8_argument_checks():
    import transformer_decoder_layer_amd as tdl
    P = 1 << 20                                  # never dereferenced: the checks come first
    g = tdl._gemm_a8w8
    assert g(None, P, P, P, P, None, P, 0, 8, 16) == tdl.TDL_OK           # empty: nothing to do
    assert g(None, P, P, P, P, None, P, 4, 8, 24) == tdl.TDL_E_INVALID    # K % 16
    assert g(None, P, P, P, P, None, P, 4, 8, 0) == tdl.TDL_E_INVALID
    assert g(None, P, None, P, P, None, P, 4, 8, 16) == tdl.TDL_E_INVALID
    assert g(None, P + 8, P, P, P, None, P, 4, 8, 16) == tdl.TDL_E_INVALID  # alignment
    assert g(None, P, P, P, P, None, P, -1, 8, 16) == tdl.TDL_E_INVALID


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


def test_block_sharing_holders():
    # [HET 4.3]: blocks carry a holder count; a block returns to the free
    # list when its last holder releases it
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(6, 2, 64)
    t = kv.block_table([40], 3)                 # blocks 0, 1, 2
    assert [kv.refs(b) for b in range(6)] == [1, 1, 1, 0, 0, 0]
    kv.share([0, 1, 1])                         # a second sequence takes 0 and 1; 1 twice
    assert [kv.refs(b) for b in range(3)] == [2, 3, 1]
    with pytest.raises(tdl.TdlError):
        kv.share([0, 4])                        # 4 is free: nothing changes
    assert kv.refs(0) == 2 and kv.refs(4) == 0
    with pytest.raises(tdl.TdlError):
        kv.release([2, 2])                      # more often than it is held
    assert kv.refs(2) == 1 and kv.free_blocks() == 3
    kv.release(t[0].tolist())                   # the first sequence lets go
    assert [kv.refs(b) for b in range(3)] == [1, 2, 0] and kv.free_blocks() == 4
    kv.release([1, 1, 0])
    assert kv.free_blocks() == 6 and all(kv.refs(b) == 0 for b in range(6))
    assert kv.refs(6) == -1 and kv.refs(-1) == -1
    # a block table entry that holds a shared block is kept, not reallocated
    t1 = kv.block_table([16], 2)
    kv.share(t1[0, :1].tolist())
    t2 = np.full((1, 2), -1, np.int32)
    t2[0, 0] = t1[0, 0]
    kv.block_table([20], 2, t2)
    assert t2[0, 0] == t1[0, 0] and t2[0, 1] != t1[0, 0] and kv.refs(int(t1[0, 0])) == 2


def test_prefix_index_match_publish_evict():
    # [HET 4.7]: block-aligned longest-prefix matching; a hit gives the
    # caller a hold on the block; idle entries go least recently used first
    import transformer_decoder_layer_amd as tdl
    kv = tdl.KvCache.host_only(10, 2, 64)
    a = kv.block_table([64], 4)[0]              # 4 full blocks of sequence A
    keys = [101, 102, 103, 104]
    kv.prefix_publish(keys, a)
    assert kv.prefix_size() == 4 and all(kv.refs(int(b)) == 2 for b in a)
    # B shares A's first three blocks, then diverges
    m = kv.prefix_match([101, 102, 103, 999, 104])
    assert m.tolist() == a[:3].tolist()
    assert [kv.refs(int(b)) for b in a] == [3, 3, 3, 2]
    assert kv.prefix_match([555, 101]).size == 0  # the prefix ends at the first miss
    # publishing again: same pairs refresh; a known key keeps its block
    kv.prefix_publish(keys[:2], a[:2])
    other = kv.block_table([16], 1)[0]
    kv.prefix_publish([104], other)             # first publisher wins
    assert kv.refs(int(other[0])) == 1 and kv.prefix_match([101, 102, 103, 104])[3] == a[3]
    kv.release(a[:4].tolist())                  # undo that last match
    with pytest.raises(tdl.TdlError):
        kv.prefix_publish([777], a[:1])         # block 0 is indexed under 101
    with pytest.raises(tdl.TdlError):
        kv.prefix_publish([778, 778], [int(other[0]), int(a[3])])  # one key, two blocks
    with pytest.raises(tdl.TdlError):
        kv.prefix_publish([779], [9])           # a free block
    assert kv.prefix_size() == 4
    # A finishes: its blocks stay cached (the index holds them); B still
    # holds the first three, so only block a[3] is idle
    kv.release(a.tolist())
    assert [kv.refs(int(b)) for b in a] == [2, 2, 2, 1]
    free0 = kv.free_blocks()
    assert kv.prefix_evict(10) == 1 and kv.free_blocks() == free0 + 1
    assert kv.prefix_match([104]).size == 0 and kv.prefix_size() == 3
    kv.release(m.tolist())                      # B finishes
    # all idle now; a match refreshes 102, so 101 and 103 go first
    kv.release(kv.prefix_match([101, 102]).tolist())
    kv.prefix_match([102])
    kv.release(a[1:2].tolist())
    assert kv.prefix_evict(2) == 2
    assert kv.prefix_size() == 1 and kv.prefix_match([101]).size == 0
    hit = kv.prefix_match([102])
    assert hit.tolist() == [a[1]]
    kv.release(hit.tolist())
    assert kv.prefix_evict(5) == 1 and kv.prefix_size() == 0
    kv.release(other.tolist())
    assert kv.free_blocks() == 10


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


def test_gemm_a8w8_binding_checks_tensors():
    # the Python wrapper refuses mismatched shapes, dtypes and host tensors
    # before anything reaches the library
    import torch
    import transformer_decoder_layer_amd as tdl
    M, N, K = 4, 8, 32
    a = torch.zeros(M, K, dtype=torch.int8)
    b = torch.zeros(N, K, dtype=torch.int8)
    sa, sb = torch.ones(M), torch.ones(N)
    out = torch.zeros(M, N)
    with pytest.raises(ValueError, match="b: expected"):
        tdl.gemm_a8w8(a, torch.zeros(N, K + 16, dtype=torch.int8), sa, sb, out)
    with pytest.raises(ValueError, match="out: expected"):
        tdl.gemm_a8w8(a, b, sa, sb, torch.zeros(M, N - 1))
    with pytest.raises(ValueError, match="a_scale: expected"):
        tdl.gemm_a8w8(a, b, sa.double(), sb, out)
    with pytest.raises(ValueError, match="c_accum: expected"):
        tdl.gemm_a8w8(a, b, sa, sb, out, c_accum=torch.zeros(M, N))
    with pytest.raises(ValueError, match="contiguous GPU tensor"):
        tdl.gemm_a8w8(a, b, sa, sb, out)


def test_q80_import_gguf_argument_checks():
    # the wrapper refuses mismatched tensors; the C entry point refuses bad
    # sizes, NULLs and misaligned pointers before any HIP call
    import torch
    import transformer_decoder_layer_amd as tdl
    rows, cols = 3, 64
    blocks = torch.zeros(rows * 2 * 34, dtype=torch.uint8)
    codes = torch.zeros(rows, cols, dtype=torch.int8)
    scales = torch.zeros(rows, 2, dtype=torch.float16)
    with pytest.raises(ValueError, match="multiple of 32"):
        tdl.q80_import_gguf(blocks, rows, 48, codes, scales)
    with pytest.raises(ValueError, match="blocks: expected"):
        tdl.q80_import_gguf(blocks[:-1], rows, cols, codes, scales)
    with pytest.raises(ValueError, match="scales: expected"):
        tdl.q80_import_gguf(blocks, rows, cols, codes, scales.float())
    with pytest.raises(ValueError, match="contiguous GPU tensor"):
        tdl.q80_import_gguf(blocks, rows, cols, codes, scales)
    f = tdl._q80_gguf
    assert f(None, None, 1, 48, None, None) == tdl.TDL_E_INVALID
    assert f(None, None, -1, 64, None, None) == tdl.TDL_E_INVALID
    assert f(None, None, 0, 64, None, None) == 0  # no rows: a no-op
    assert f(None, None, 2, 64, None, None) == tdl.TDL_E_INVALID
    assert f(None, 0x1001, 2, 64, 0x2000, 0x3000) == tdl.TDL_E_INVALID  # blocks odd
    assert f(None, 0x1000, 2, 64, 0x2008, 0x3000) == tdl.TDL_E_INVALID  # codes not 16-byte aligned
