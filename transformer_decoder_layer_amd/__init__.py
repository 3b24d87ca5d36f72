"""Python binding of libtdl, the gfx950 Qwen-style GQA decoder layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and streams.  Importing
fails loudly if the library has not been built
(``python transformer_decoder_layer_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtdl.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python transformer_decoder_layer_amd/build.py` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

TDL_OK, TDL_E_INVALID, TDL_E_UNSUPPORTED, TDL_E_CAPACITY, TDL_E_NOMEM, TDL_E_HIP = range(6)
TDL_BF16, TDL_F32, TDL_Q8_0, TDL_U8_ASYM, TDL_U4_ASYM, TDL_I8_ROW, TDL_A8W8 = range(7)
_DTYPES = {"bf16": TDL_BF16, "f32": TDL_F32, "q80": TDL_Q8_0, "u8": TDL_U8_ASYM, "u4": TDL_U4_ASYM,
           "iq8": TDL_I8_ROW, "a8w8": TDL_A8W8}

c_i32, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
P_i32 = ctypes.POINTER(ctypes.c_int32)

EXPORTS = ["layer_create", "layer_destroy", "layer_prefill", "layer_decode_paged",
           "layer_decode_paged_noalloc", "layer_step",
           "layer_workspace_view", "layer_profile_enable", "layer_profile_read", "stack_create",
           "stack_destroy", "stack_decode_paged", "kv_cache_bytes", "kv_cache_alloc", "kv_cache_free",
           "kv_cache_view", "kv_block_table", "kv_block_release", "kv_block_share", "kv_block_refs",
           "kv_free_blocks", "kv_prefix_publish", "kv_prefix_match", "kv_prefix_evict", "kv_prefix_size",
           "kv_cache_calibrate", "kv_cache_write", "gemm_a8w8", "q80_import_gguf", "tdl_status_string",
           "tdl_last_error"]


class LayerConfig(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("intermediate", c_i32), ("rms_eps", c_f32),
                ("rope_theta", c_f32), ("qkv_bias", c_i32), ("qk_norm", c_i32),
                ("weight_dtype", c_i32), ("max_tokens", c_i32), ("max_seqs", c_i32),
                ("max_position", c_i32), ("rope_fused", c_i32)]


_WEIGHT_FIELDS = ["ln1", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "ln2", "wg", "wu", "wd",
                  "q_norm", "k_norm", "wq_scale", "wk_scale", "wv_scale", "wo_scale", "wg_scale",
                  "wu_scale", "wd_scale", "wq_zp", "wk_zp", "wv_zp", "wo_zp", "wg_zp", "wu_zp",
                  "wd_zp"]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in _WEIGHT_FIELDS]


class KvConfig(ctypes.Structure):
    _fields_ = [("n_blocks", c_i32), ("block_size", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("kv_dtype", c_i32), ("free_list_seed", ctypes.c_uint64),
                ("block_scales", c_i32)]


class KvView(ctypes.Structure):
    _fields_ = [("k_pool", c_vp), ("v_pool", c_vp), ("k_strides", ctypes.c_int64 * 4),
                ("v_strides", ctypes.c_int64 * 4), ("elem_bytes", c_i32), ("k_scale", c_vp),
                ("k_zero_point", c_vp), ("v_scale", c_vp), ("v_zero_point", c_vp), ("block_exp", c_vp)]


class Batch(ctypes.Structure):
    _fields_ = [("n_seqs", c_i32), ("n_prefill_seqs", c_i32), ("n_rows", c_i32),
                ("max_q_len", c_i32), ("max_ctx_len", c_i32), ("max_blocks", c_i32),
                ("q_start", c_vp), ("q_len", c_vp), ("ctx_len", c_vp), ("block_tables", c_vp)]


STAGES = ["rmsnorm1", "qkv", "rope_kv", "attn_prefill", "attn_decode", "o_proj", "rmsnorm2",
          "gate_up", "down"]


class Profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(STAGES)), ("launches", ctypes.c_int64 * len(STAGES))]


class WorkspaceView(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ["xn", "qkv", "q", "o", "h", "hn", "a"]]


def _sig(name, restype, *args):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(args)
    return f


_layer_create = _sig("layer_create", c_i32, ctypes.POINTER(LayerConfig), ctypes.POINTER(LayerWeights),
                     c_vp, ctypes.POINTER(c_vp))
_layer_destroy = _sig("layer_destroy", c_i32, c_vp)
_layer_prefill = _sig("layer_prefill", c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp)
_layer_decode = _sig("layer_decode_paged", c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                     c_i32, c_vp)
_layer_decode_na = _sig("layer_decode_paged_noalloc", c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp,
                        c_i32, c_i32, c_vp)
_layer_step = _sig("layer_step", c_i32, c_vp, c_vp, ctypes.POINTER(Batch), c_vp, c_vp, c_vp)
_layer_ws = _sig("layer_workspace_view", c_i32, c_vp, ctypes.POINTER(WorkspaceView))
_layer_prof_enable = _sig("layer_profile_enable", c_i32, c_vp, c_i32)
_layer_prof_read = _sig("layer_profile_read", c_i32, c_vp, ctypes.POINTER(Profile))
_kv_bytes = _sig("kv_cache_bytes", c_sz, ctypes.POINTER(KvConfig))
_kv_alloc = _sig("kv_cache_alloc", c_i32, ctypes.POINTER(KvConfig), c_vp, ctypes.POINTER(c_vp))
_kv_free = _sig("kv_cache_free", c_i32, c_vp)
_kv_view = _sig("kv_cache_view", c_i32, c_vp, ctypes.POINTER(KvView))
_kv_table = _sig("kv_block_table", c_i32, c_vp, c_i32, P_i32, c_i32, P_i32)
_kv_release = _sig("kv_block_release", c_i32, c_vp, P_i32, c_i32)
_kv_free_blocks = _sig("kv_free_blocks", c_i32, c_vp)
_kv_share = _sig("kv_block_share", c_i32, c_vp, P_i32, c_i32)
_kv_refs = _sig("kv_block_refs", c_i32, c_vp, c_i32)
P_u64 = ctypes.POINTER(ctypes.c_uint64)
_kv_publish = _sig("kv_prefix_publish", c_i32, c_vp, P_u64, P_i32, c_i32)
_kv_match = _sig("kv_prefix_match", c_i32, c_vp, P_u64, c_i32, P_i32, P_i32)
_kv_evict = _sig("kv_prefix_evict", c_i32, c_vp, c_i32)
_kv_prefix_size = _sig("kv_prefix_size", c_i32, c_vp)
_gemm_a8w8 = _sig("gemm_a8w8", c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32)
_q80_gguf = _sig("q80_import_gguf", c_i32, c_vp, c_vp, ctypes.c_int64, ctypes.c_int64, c_vp, c_vp)
_kv_calibrate = _sig("kv_cache_calibrate", c_i32, c_vp, c_vp, c_vp, c_vp, ctypes.c_int64)
_kv_write = _sig("kv_cache_write", c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp,
                 c_vp, c_i32)
_stack_create = _sig("stack_create", c_i32, ctypes.POINTER(c_vp), c_i32, ctypes.POINTER(c_vp))
_stack_destroy = _sig("stack_destroy", c_i32, c_vp)
_stack_decode = _sig("stack_decode_paged", c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                     c_i32, ctypes.POINTER(c_vp))
_status_string = _sig("tdl_status_string", ctypes.c_char_p, c_i32)
_last_error = _sig("tdl_last_error", ctypes.c_char_p)


class TdlError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _last_error().decode(errors="replace")
        super().__init__(f"{fn}: {_status_string(status).decode()} ({status}): {msg}")


def _check(fn: str, status: int):
    if status != TDL_OK:
        raise TdlError(fn, status)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(P_i32)


class KvCache:
    """A paged KV cache; its device memory is one torch uint8 tensor."""

    def __init__(self, n_blocks: int, n_kv_heads: int, head_dim: int, dtype: str = "bf16",
                 seed: int = 0, device: str = "cuda", block_size: int = 16, allocate: bool = True,
                 block_scales: bool = False):
        self.cfg = KvConfig(n_blocks, block_size, n_kv_heads, head_dim, _DTYPES[dtype], seed,
                            int(block_scales))
        self.dtype = dtype
        self.block_scales = block_scales
        nbytes = _kv_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            raise TdlError("kv_cache_bytes", TDL_E_INVALID)
        self.nbytes = nbytes
        self.memory = None
        dev_mem = None
        if allocate:
            import torch
            self.memory = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
            dev_mem = (self.memory.data_ptr() + 255) & ~255
        h = c_vp()
        _check("kv_cache_alloc", _kv_alloc(ctypes.byref(self.cfg), dev_mem, ctypes.byref(h)))
        self._h = h

    @classmethod
    def host_only(cls, n_blocks, n_kv_heads, head_dim, dtype="bf16", seed=0, fake_ptr=1 << 20,
                  block_size=16, block_scales=False):
        """A handle over a placeholder device address, for host-side tests of
        the block allocator (the library never dereferences it)."""
        self = cls.__new__(cls)
        self.cfg = KvConfig(n_blocks, block_size, n_kv_heads, head_dim, _DTYPES[dtype], seed,
                            int(block_scales))
        self.dtype = dtype
        self.block_scales = block_scales
        self.memory = None
        self.nbytes = _kv_bytes(ctypes.byref(self.cfg))
        h = c_vp()
        _check("kv_cache_alloc", _kv_alloc(ctypes.byref(self.cfg), fake_ptr, ctypes.byref(h)))
        self._h = h
        return self

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _kv_free(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def block_table(self, n_tokens: Sequence[int], max_blocks: int,
                    table: Optional[np.ndarray] = None) -> np.ndarray:
        n = _host_i32(n_tokens)
        if table is None:
            table = np.full((len(n), max_blocks), -1, np.int32)
        assert table.dtype == np.int32 and table.flags.c_contiguous and table.shape == (len(n), max_blocks)
        _check("kv_block_table", _kv_table(self._h, len(n), _i32p(n), max_blocks, _i32p(table)))
        return table

    def release(self, blocks: Sequence[int]):
        b = _host_i32(blocks)
        _check("kv_block_release", _kv_release(self._h, _i32p(b), len(b)))

    def free_blocks(self) -> int:
        return _kv_free_blocks(self._h)

    def share(self, blocks: Sequence[int]):
        b = _host_i32(blocks)
        _check("kv_block_share", _kv_share(self._h, _i32p(b), len(b)))

    def refs(self, block: int) -> int:
        return _kv_refs(self._h, int(block))

    def prefix_publish(self, keys: Sequence[int], blocks: Sequence[int]):
        k = np.ascontiguousarray(keys, dtype=np.uint64)
        b = _host_i32(blocks)
        assert len(k) == len(b)
        _check("kv_prefix_publish", _kv_publish(self._h, k.ctypes.data_as(P_u64), _i32p(b), len(b)))

    def prefix_match(self, keys: Sequence[int]) -> np.ndarray:
        """Blocks of the longest indexed prefix of ``keys`` (the caller now
        holds each of them once)."""
        k = np.ascontiguousarray(keys, dtype=np.uint64)
        out = np.full(len(k), -1, np.int32)
        m = c_i32(0)
        _check("kv_prefix_match", _kv_match(self._h, k.ctypes.data_as(P_u64), len(k), _i32p(out),
                                            ctypes.byref(m)))
        return out[:m.value]

    def prefix_evict(self, n_blocks: int) -> int:
        return _kv_evict(self._h, int(n_blocks))

    def prefix_size(self) -> int:
        return _kv_prefix_size(self._h)

    def view(self) -> KvView:
        v = KvView()
        _check("kv_cache_view", _kv_view(self._h, ctypes.byref(v)))
        return v

    def tensors(self):
        """torch views (k_pool, v_pool[, k_scale, k_zp, v_scale, v_zp]) of the
        cache memory: k [blocks, Hkv, 16, D], v [blocks, Hkv, D, 16]; u4:
        bytes k [blocks, Hkv, 16, D/2], v [blocks, Hkv, D/2, 16], two codes
        per byte (include/tdl.h gives the nibble order)."""
        import torch
        v = self.view()
        nb, hk, d = self.cfg.n_blocks, self.cfg.n_kv_heads, self.cfg.head_dim
        base = self.memory.data_ptr()
        esz = v.elem_bytes
        if esz == 0:
            d //= 2
        n = nb * hk * 16 * d

        def sl(ptr, count, dt):
            off = ptr - base
            return self.memory[off:off + count * torch.tensor([], dtype=dt).element_size()].view(dt)

        pool_dt = torch.bfloat16 if esz == 2 else torch.uint8
        k = sl(v.k_pool, n, pool_dt).view(nb, hk, 16, d)
        vv = sl(v.v_pool, n, pool_dt).view(nb, hk, d, 16)
        if self.dtype not in ("u8", "u4"):
            return k, vv
        c = hk * self.cfg.head_dim
        return (k, vv, sl(v.k_scale, c, torch.float32), sl(v.k_zero_point, c, torch.int32),
                sl(v.v_scale, c, torch.float32), sl(v.v_zero_point, c, torch.int32))

    def block_exponents(self):
        """torch int8 view [blocks, Hkv, 2] of the per-block factor exponents
        (K, V) of a block_scales cache."""
        import torch
        v = self.view()
        assert self.block_scales and v.block_exp
        nb, hk = self.cfg.n_blocks, self.cfg.n_kv_heads
        off = v.block_exp - self.memory.data_ptr()
        return self.memory[off:off + nb * hk * 2].view(torch.int8).view(nb, hk, 2)

    def calibrate(self, k, v, stream=None):
        _check("kv_cache_calibrate", _kv_calibrate(self._h, _stream(stream), _ptr(k), _ptr(v),
                                                   k.shape[0]))

    def write(self, cu_rows, start_pos, block_tables, k, v, stream=None):
        """cu_rows [n_seqs+1], start_pos [n_seqs], block_tables [n_seqs, max_blocks]:
        device int32 tensors; k, v [rows, Hkv, D] float32 or bfloat16."""
        import torch
        src = TDL_F32 if k.dtype == torch.float32 else TDL_BF16
        _check("kv_cache_write", _kv_write(self._h, _stream(stream), start_pos.shape[0], _ptr(cu_rows),
                                           _ptr(start_pos), _ptr(block_tables), block_tables.shape[1],
                                           src, _ptr(k), _ptr(v), k.shape[0]))


def gemm_a8w8(a, b, a_scale, b_scale, out, c_accum=None, stream=None):
    """out [M, N] float32 = (a [M, K] int8 @ b [N, K]^T int8, in int32) *
    a_scale[m] * b_scale[n]; c_accum [M, N] int32 (optional) gets the sums.
    Raises ValueError before the call when a tensor's shape, dtype, layout or
    device does not match what the kernel reads and writes."""
    import torch
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    want = [("a", a, (M, K), torch.int8), ("b", b, (N, K), torch.int8),
            ("a_scale", a_scale, (M,), torch.float32), ("b_scale", b_scale, (N,), torch.float32),
            ("out", out, (M, N), torch.float32)]
    if c_accum is not None:
        want.append(("c_accum", c_accum, (M, N), torch.int32))
    for name, t, shp, dt in want:
        if tuple(t.shape) != shp or t.dtype != dt:
            raise ValueError(f"{name}: expected {dt} {shp}, got {t.dtype} {tuple(t.shape)}")
    for name, t, _, _ in want:
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _check("gemm_a8w8", _gemm_a8w8(_stream(stream), _ptr(a), _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                   _ptr(c_accum), _ptr(out), M, N, K))


def q80_import_gguf(blocks, rows: int, cols: int, codes, scales, stream=None):
    """GGUF Q8_0 tensor data (blocks: uint8 [rows * cols/32 * 34], on the GPU)
    -> codes int8 [rows, cols] and scales float16 [rows, cols/32], the arrays
    a TDL_Q8_0 layer takes.  Raises ValueError before the call when a tensor's
    shape, dtype, layout or device does not match."""
    import torch
    if cols <= 0 or cols % 32 != 0 or rows < 0:
        raise ValueError("rows >= 0 and a positive multiple of 32 columns required")
    want = [("blocks", blocks, (rows * (cols // 32) * 34,), torch.uint8),
            ("codes", codes, (rows, cols), torch.int8), ("scales", scales, (rows, cols // 32), torch.float16)]
    for name, t, shp, dt in want:
        if tuple(t.shape) != shp or t.dtype != dt:
            raise ValueError(f"{name}: expected {dt} {shp}, got {t.dtype} {tuple(t.shape)}")
    for name, t, _, _ in want:
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _check("q80_import_gguf", _q80_gguf(_stream(stream), _ptr(blocks), rows, cols, _ptr(codes), _ptr(scales)))


def make_config(shape, max_tokens: int, max_seqs: int = 1, max_position: int = 8192,
                rope_fused: bool = False) -> LayerConfig:
    """LayerConfig from any object with the layer-shape attributes (hidden,
    n_q_heads, n_kv_heads, head_dim, intermediate, rms_eps, rope_theta,
    qkv_bias, qk_norm, weight_dtype in {"f32", "bf16", "q80", "iq8", "a8w8"})."""
    return LayerConfig(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                       shape.intermediate, shape.rms_eps, shape.rope_theta, int(shape.qkv_bias),
                       int(shape.qk_norm), _DTYPES[shape.weight_dtype], max_tokens, max_seqs,
                       max_position, int(rope_fused))


class Layer:
    """One decoder layer.  ``weights`` maps names (ln1, wq, bq, ...) to device
    tensors in PyTorch Linear layout; see include/tdl.h for dtypes."""

    def __init__(self, cfg: LayerConfig, weights: Dict[str, "object"], stream=None):
        w = LayerWeights()
        for name in _WEIGHT_FIELDS:
            t = weights.get(name)
            if t is not None:
                setattr(w, name, t.data_ptr())
        self.cfg = cfg
        h = c_vp()
        _check("layer_create", _layer_create(ctypes.byref(cfg), ctypes.byref(w), _stream(stream),
                                             ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _layer_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, x, y, start_pos: int = 0, kv: Optional[KvCache] = None, block_table=None,
                stream=None):
        _check("layer_prefill", _layer_prefill(self._h, _stream(stream), _ptr(x), _ptr(y), x.shape[0],
                                               start_pos, kv.handle if kv else None,
                                               _ptr(block_table)))

    def decode_paged(self, x, y, ctx_lens, block_tables, max_ctx_len: int, kv: KvCache, stream=None):
        _check("layer_decode_paged", _layer_decode(self._h, _stream(stream), _ptr(x), _ptr(y),
                                                   x.shape[0], _ptr(ctx_lens), _ptr(block_tables),
                                                   block_tables.shape[1], max_ctx_len, kv.handle))

    def decode_paged_noalloc(self, x, y, ctx_lens, block_tables, max_ctx_len: int, kv: KvCache,
                             stream=None):
        """decode_paged with its partial results in the library's static
        scratch (layer_decode_paged_noalloc: no device allocation)."""
        _check("layer_decode_paged_noalloc",
               _layer_decode_na(self._h, _stream(stream), _ptr(x), _ptr(y), x.shape[0], _ptr(ctx_lens),
                                _ptr(block_tables), block_tables.shape[1], max_ctx_len, kv.handle))

    def step(self, x, y, q_start, q_len, ctx_len, block_tables, n_prefill_seqs: int, max_q_len: int,
             max_ctx_len: int, kv: KvCache, stream=None):
        b = Batch(q_len.shape[0], n_prefill_seqs, x.shape[0], max_q_len, max_ctx_len,
                  block_tables.shape[1], _ptr(q_start), _ptr(q_len), _ptr(ctx_len), _ptr(block_tables))
        _check("layer_step", _layer_step(self._h, _stream(stream), ctypes.byref(b), _ptr(x), _ptr(y),
                                         kv.handle))

    def profile_enable(self, enable: bool = True):
        _check("layer_profile_enable", _layer_prof_enable(self._h, int(enable)))

    def profile_read(self) -> Dict[str, tuple]:
        # {stage: (total_ms, launches)} since the last profile_enable
        p = Profile()
        _check("layer_profile_read", _layer_prof_read(self._h, ctypes.byref(p)))
        return {name: (p.ms[i], p.launches[i]) for i, name in enumerate(STAGES)}

    def workspace(self) -> WorkspaceView:
        v = WorkspaceView()
        _check("layer_workspace_view", _layer_ws(self._h, ctypes.byref(v)))
        return v


class Stack:
    """Layers applied in order as one decode step (stack_decode_paged).  The
    layers (and their caches) must outlive the stack."""

    def __init__(self, layers: List[Layer]):
        hs = (c_vp * len(layers))(*[l._h.value for l in layers])
        h = c_vp()
        _check("stack_create", _stack_create(hs, len(layers), ctypes.byref(h)))
        self._h = h
        self.layers = list(layers)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _stack_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode_paged(self, x, y, ctx_lens, block_tables, max_ctx_len: int, kvs: List[KvCache],
                     stream=None):
        ks = (c_vp * len(kvs))(*[k.handle.value if k is not None else None for k in kvs])
        _check("stack_decode_paged", _stack_decode(self._h, _stream(stream), _ptr(x), _ptr(y), x.shape[0],
                                                   _ptr(ctx_lens), _ptr(block_tables),
                                                   block_tables.shape[1], max_ctx_len, ks))


def device_tensor(ptr: int, shape, dtype):
    """A torch tensor aliasing library-owned device memory at ``ptr`` (for
    reading intermediate buffers in tests)."""
    import torch
    typestr = {torch.float32: "<f4", torch.bfloat16: "<i2", torch.float16: "<f2", torch.int32: "<i4",
               torch.uint8: "|u1"}[dtype]

    class _Cai:
        __cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (ptr, False),
                                    "version": 2, "strides": None}

    t = torch.as_tensor(_Cai(), device="cuda")
    return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t
