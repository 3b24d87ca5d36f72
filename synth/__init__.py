"""Seeded synthetic inputs for the decoder layer.

This module only draws numbers: layer shapes, weights, activations, context
lengths, block tables and cached K/V.  It holds none of the layer's
arithmetic, so both the oracle and the HIP path may take their inputs from it.

Value distributions follow the workloads the pages describe (a Qwen2.5-7B
layer: hidden 3584, 28 Q / 4 KV heads, head_dim 128 -- "从零实现 C++ LLM 推理
引擎：加载 Qwen2.5-7B 并跑通单层 Forward Pass", section "运行结果"; Qwen3-8B Q8_0
-- "TFFInfer 推理框架项目解析", section 1.1; 16-token KV blocks -- the devpress
"C++ 原生异构推理引擎" article, section 4.3):

* linear weights and QKV biases ~ N(0, 0.02); norm gains 1.0;
* activations and cached K/V ~ N(0, 1);
* bf16 values are fp32 draws rounded to nearest-even bf16 (torch's cast);
* Q8_0 codes uniform integers in [-127, 127], scales |N(0, 0.002)| as fp16;
* block tables: a seeded random permutation of the physical blocks.

Generation order is fixed per workload so every array is reproducible from the
seed alone.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rms_eps: float
    rope_theta: float
    qkv_bias: bool
    qk_norm: bool
    weight_dtype: str  # "f32" | "bf16" | "q80" | "iq8" | "a8w8"

    @property
    def n_rep(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


TINY = LayerShape("tiny", 256, 4, 2, 64, 688, 1e-6, 1e4, True, False, "f32")
QWEN25_7B = LayerShape("qwen2.5-7b", 3584, 28, 4, 128, 18944, 1e-6, 1e6, True, False, "bf16")
QWEN3_8B = LayerShape("qwen3-8b", 4096, 32, 8, 128, 12288, 1e-6, 1e6, False, True, "bf16")
QWEN3_8B_Q80 = dataclasses.replace(QWEN3_8B, name="qwen3-8b-q8_0", weight_dtype="q80")
QWEN25_7B_IQ8 = dataclasses.replace(QWEN25_7B, name="qwen2.5-7b-iq8", weight_dtype="iq8")
QWEN25_7B_A8W8 = dataclasses.replace(QWEN25_7B, name="qwen2.5-7b-a8w8", weight_dtype="a8w8")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One batch of work for one layer call."""
    name: str
    shape: LayerShape
    kind: str                    # "prefill" | "decode" | "mixed"
    prefill_len: int = 0         # new tokens of the (single) prefill chunk
    decode_batch: int = 0        # decode sequences, one new token each
    ctx_lo: int = 0              # decode context lengths ~ U[ctx_lo, ctx_hi]
    ctx_hi: int = 0
    ctx_fixed: int = 0           # if > 0, every decode sequence has this context
    kv_dtype: str = "none"       # "none" | "bf16" | "u8" | "u4"


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_prefill_32", TINY, "prefill", prefill_len=32),
    Workload("qwen25_prefill_512", QWEN25_7B, "prefill", prefill_len=512, kv_dtype="bf16"),
    Workload("qwen25_prefill_4096", QWEN25_7B, "prefill", prefill_len=4096, kv_dtype="bf16"),
    Workload("qwen25_decode_b64", QWEN25_7B, "decode", decode_batch=64, ctx_lo=128, ctx_hi=4096,
             kv_dtype="bf16"),
    Workload("qwen3_decode_u8_b128", QWEN3_8B, "decode", decode_batch=128, ctx_lo=512, ctx_hi=8192,
             kv_dtype="u8"),
    Workload("qwen3_decode_u4_b128", QWEN3_8B, "decode", decode_batch=128, ctx_lo=512, ctx_hi=8192,
             kv_dtype="u4"),
    Workload("qwen25_iq8_decode_b64", QWEN25_7B_IQ8, "decode", decode_batch=64, ctx_lo=128,
             ctx_hi=4096, kv_dtype="bf16"),
    Workload("qwen3_q80_mixed", QWEN3_8B_Q80, "mixed", prefill_len=2048, decode_batch=64,
             ctx_fixed=2048, kv_dtype="bf16"),
]}


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """fp32 draws -> the nearest-even bf16 values, returned as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def _normal(rng, shape, std=1.0):
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def make_weights(shape: LayerShape, seed: int = 0, random_gains: bool = False,
                 rng: Optional[np.random.Generator] = None) -> Dict[str, np.ndarray]:
    """Weights in PyTorch Linear layout [out, in].

    f32/bf16 layers: float32 arrays (bf16-valued for "bf16").  Q8_0 layers:
    ``w*`` are int8 codes [out, in] and ``w*_scale`` float16 [out, in/32].
    ``random_gains`` draws norm gains from N(1, 0.1) so tests can tell a
    dropped gain multiply from a kept one.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    H, D, I = shape.hidden, shape.head_dim, shape.intermediate
    nq, nkv = shape.n_q_heads * D, shape.n_kv_heads * D
    dims = {"wq": (nq, H), "wk": (nkv, H), "wv": (nkv, H), "wo": (H, nq),
            "wg": (I, H), "wu": (I, H), "wd": (H, I)}

    def gain(n):
        if random_gains:
            return (1.0 + _normal(rng, (n,), 0.1)).astype(np.float32)
        return np.ones(n, np.float32)

    def linear(name):
        out, inp = dims[name]
        if shape.weight_dtype == "q80":
            assert inp % 32 == 0
            codes = rng.integers(-127, 128, size=(out, inp), dtype=np.int8)
            scales = np.abs(_normal(rng, (out, inp // 32), 0.002)).astype(np.float16)
            return {name: codes, name + "_scale": scales}
        if shape.weight_dtype == "a8w8":
            # int8 codes and a float32 scale per output row (symmetric);
            # code * scale has a spread like N(0, 0.02)
            codes = rng.integers(-127, 128, size=(out, inp), dtype=np.int8)
            scales = (np.abs(_normal(rng, (out,), 2.7e-4)) + 1e-5).astype(np.float32)
            return {name: codes, name + "_scale": scales}
        if shape.weight_dtype == "iq8":
            # int8 codes, an int8 zero point and a float32 scale per output
            # row; (code - zp) * scale has a spread like N(0, 0.02)
            codes = rng.integers(-128, 128, size=(out, inp), dtype=np.int8)
            zp = rng.integers(-20, 21, size=out, dtype=np.int8)
            scales = (np.abs(_normal(rng, (out,), 2.7e-4)) + 1e-5).astype(np.float32)
            return {name: codes, name + "_scale": scales, name + "_zp": zp}
        w = _normal(rng, (out, inp), 0.02)
        if shape.weight_dtype == "bf16":
            w = to_bf16_values(w)
        return {name: w}

    def bias(n):
        b = _normal(rng, (n,), 0.02)
        return to_bf16_values(b) if shape.weight_dtype != "f32" else b

    w: Dict[str, np.ndarray] = {}
    w["ln1"] = gain(H)
    w.update(linear("wq"))
    if shape.qkv_bias:
        w["bq"] = bias(nq)
    w.update(linear("wk"))
    if shape.qkv_bias:
        w["bk"] = bias(nkv)
    w.update(linear("wv"))
    if shape.qkv_bias:
        w["bv"] = bias(nkv)
    w.update(linear("wo"))
    w["ln2"] = gain(H)
    w.update(linear("wg"))
    w.update(linear("wu"))
    w.update(linear("wd"))
    if shape.qk_norm:
        w["q_norm"] = gain(D)
        w["k_norm"] = gain(D)
    return w


def gguf_q80_bytes(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Serialises Q8_0 codes [rows, cols] int8 and scales [rows, cols/32]
    float16 as GGUF-style interleaved blocks (uint8 [rows * cols/32 * 34]):
    per block the scale's two little-endian bytes, then its 32 codes.  An
    input generator for the import path (no arithmetic of the layer)."""
    rows, cols = codes.shape
    nb = cols // 32
    blk = np.empty((rows, nb, 34), np.uint8)
    blk[:, :, 0:2] = np.ascontiguousarray(scales.astype("<f2")).view(np.uint8).reshape(rows, nb, 2)
    blk[:, :, 2:] = codes.reshape(rows, nb, 32).view(np.uint8)
    return blk.reshape(-1)


def make_x(rng: np.random.Generator, n_rows: int, hidden: int, bf16: bool = True) -> np.ndarray:
    x = _normal(rng, (n_rows, hidden))
    return to_bf16_values(x) if bf16 else x


def random_tables(rng: np.random.Generator, n_tokens: List[int], n_blocks: Optional[int] = None,
                  max_blocks: Optional[int] = None) -> np.ndarray:
    """Block tables [n_seqs, max_blocks] int32 whose used entries are a random
    permutation of the physical blocks 0..n_blocks-1; unused entries are -1."""
    need = [int(math.ceil(n / BLOCK_SIZE)) for n in n_tokens]
    total = sum(need)
    n_blocks = total if n_blocks is None else n_blocks
    assert n_blocks >= total
    max_blocks = max(need + [1]) if max_blocks is None else max_blocks
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((len(n_tokens), max_blocks), -1, np.int32)
    pos = 0
    for i, nb in enumerate(need):
        table[i, :nb] = perm[pos:pos + nb]
        pos += nb
    return table


def context_lengths(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    if wl.ctx_fixed:
        return np.full(wl.decode_batch, wl.ctx_fixed, np.int32)
    return rng.integers(wl.ctx_lo, wl.ctx_hi + 1, wl.decode_batch).astype(np.int32)


def cached_kv(rng: np.random.Generator, n_tokens: int, n_kv_heads: int, head_dim: int,
              bf16: bool) -> Dict[str, np.ndarray]:
    """Cached keys and values [n_tokens, n_kv_heads, head_dim], N(0,1)."""
    k = _normal(rng, (n_tokens, n_kv_heads, head_dim))
    v = _normal(rng, (n_tokens, n_kv_heads, head_dim))
    if bf16:
        k, v = to_bf16_values(k), to_bf16_values(v)
    return {"k": k, "v": v}


@dataclasses.dataclass
class Batch:
    """Sequences of one layer call.  Sequence i owns rows
    [q_start[i], q_start[i]+q_len[i]) of x; its new tokens sit at positions
    ctx_len[i] .. ctx_len[i]+q_len[i]-1; its blocks are table[i]."""
    q_start: np.ndarray
    q_len: np.ndarray
    ctx_len: np.ndarray
    table: np.ndarray          # [n_seqs, max_blocks] int32, -1 = unused
    n_blocks: int              # physical blocks in the pool

    @property
    def n_seqs(self) -> int:
        return int(len(self.q_len))

    @property
    def n_rows(self) -> int:
        return int(self.q_len.sum())


def make_batch(rng: np.random.Generator, prefill_lens: List[int], prefill_start: List[int],
               decode_ctx: List[int], spare_blocks: int = 0) -> Batch:
    """Prefill sequences first, then decode sequences (one new token each)."""
    q_len = [int(t) for t in prefill_lens] + [1] * len(decode_ctx)
    ctx = [int(s) for s in prefill_start] + [int(c) for c in decode_ctx]
    q_start = np.concatenate([[0], np.cumsum(q_len)[:-1]]).astype(np.int32)
    totals = [c + q for c, q in zip(ctx, q_len)]
    need = sum(int(math.ceil(t / BLOCK_SIZE)) for t in totals)
    table = random_tables(rng, totals, n_blocks=need + spare_blocks)
    return Batch(q_start, np.array(q_len, np.int32), np.array(ctx, np.int32), table,
                 need + spare_blocks)


@dataclasses.dataclass
class LayerInputs:
    workload: Workload
    weights: Dict[str, np.ndarray]
    x: np.ndarray                  # [n_rows, hidden] float32 (bf16-valued unless tiny f32)
    batch: Batch
    cache_k: Optional[np.ndarray]  # [n_cached, Hkv, D] float32, tokens in (seq, pos) order
    cache_v: Optional[np.ndarray]
    # u8 / u4 caches: rows [n, Hkv, D] the per-channel parameters are
    # calibrated on; None: the cached tokens
    calib_k: Optional[np.ndarray] = None
    calib_v: Optional[np.ndarray] = None
    # u8 / u4 caches: per-block x per-channel factors (tdl_kv_config.block_scales)
    block_scales: bool = False


def make_inputs(wl: Workload, seed: int = 0, shape: Optional[LayerShape] = None,
                prefill_len: Optional[int] = None, decode_batch: Optional[int] = None,
                decode_ctx: Optional[List[int]] = None, prefill_start: int = 0,
                random_gains: bool = False, spare_blocks: int = 0) -> LayerInputs:
    """All inputs of one workload call, in one fixed generation order:
    weights, x, context lengths, block permutation, cached K, cached V.

    The keyword overrides shrink a workload (fewer rows, shorter contexts)
    while keeping its value distributions."""
    shape = shape or wl.shape
    rng = np.random.default_rng(seed)
    weights = make_weights(shape, rng=rng, random_gains=random_gains)
    T = wl.prefill_len if prefill_len is None else prefill_len
    B = wl.decode_batch if decode_batch is None else decode_batch
    if wl.kind == "prefill":
        B = 0
    if wl.kind == "decode":
        T = 0
    n_rows = T + B
    x = make_x(rng, n_rows, shape.hidden, bf16=(shape.weight_dtype != "f32"))
    if decode_ctx is not None:
        ctx = np.asarray(decode_ctx, np.int32)
        assert len(ctx) == B
    elif B:
        ctx = context_lengths(rng, dataclasses.replace(wl, decode_batch=B))
    else:
        ctx = np.zeros(0, np.int32)
    pre = [T] if T else []
    pre_start = [prefill_start] if T else []
    batch = make_batch(rng, pre, pre_start, list(ctx), spare_blocks=spare_blocks)
    n_cached = int(batch.ctx_len.sum())
    cache_k = cache_v = None
    if wl.kv_dtype != "none" and n_cached:
        kv = cached_kv(rng, n_cached, shape.n_kv_heads, shape.head_dim,
                       bf16=(wl.kv_dtype == "bf16"))
        cache_k, cache_v = kv["k"], kv["v"]
    return LayerInputs(wl, weights, x, batch, cache_k, cache_v)


# ------------------------------------------------------------------------
# Device-side generation for benchmarks: the same distributions drawn with
# torch's generator on the GPU (fast for ~10^8 values; not bitwise equal to
# the numpy draws above).
# ------------------------------------------------------------------------

def torch_weights(shape: LayerShape, seed: int = 0, device: str = "cuda"):
    """Weights as device tensors in the dtypes the C ABI takes: linear weights
    bf16 (or Q8_0 int8 codes + fp16 scales, or per-row int8 codes + fp32
    scale + int8 zero point, or A8W8 int8 codes + fp32 scale per row),
    biases and gains float32."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    H, D, I = shape.hidden, shape.head_dim, shape.intermediate
    nq, nkv = shape.n_q_heads * D, shape.n_kv_heads * D
    dims = {"wq": (nq, H), "wk": (nkv, H), "wv": (nkv, H), "wo": (H, nq),
            "wg": (I, H), "wu": (I, H), "wd": (H, I)}
    w = {"ln1": torch.ones(H, device=device), "ln2": torch.ones(H, device=device)}
    for name, (o, i) in dims.items():
        if shape.weight_dtype == "q80":
            w[name] = torch.randint(-127, 128, (o, i), generator=g, device=device, dtype=torch.int8)
            w[name + "_scale"] = (torch.randn(o, i // 32, generator=g, device=device).abs() * 0.002).half()
        elif shape.weight_dtype == "a8w8":
            w[name] = torch.randint(-127, 128, (o, i), generator=g, device=device, dtype=torch.int8)
            w[name + "_scale"] = torch.randn(o, generator=g, device=device).abs() * 2.7e-4 + 1e-5
        elif shape.weight_dtype == "iq8":
            w[name] = torch.randint(-128, 128, (o, i), generator=g, device=device, dtype=torch.int8)
            w[name + "_zp"] = torch.randint(-20, 21, (o,), generator=g, device=device, dtype=torch.int8)
            w[name + "_scale"] = torch.randn(o, generator=g, device=device).abs() * 2.7e-4 + 1e-5
        else:
            w[name] = (torch.randn(o, i, generator=g, device=device) * 0.02).to(torch.bfloat16)
    if shape.qkv_bias:
        for name, n in (("bq", nq), ("bk", nkv), ("bv", nkv)):
            w[name] = (torch.randn(n, generator=g, device=device) * 0.02).to(torch.bfloat16).float()
    if shape.qk_norm:
        w["q_norm"] = torch.ones(D, device=device)
        w["k_norm"] = torch.ones(D, device=device)
    return w


def torch_normal(shape, seed: int, dtype=None, device: str = "cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device)
    return t.to(dtype) if dtype is not None else t
