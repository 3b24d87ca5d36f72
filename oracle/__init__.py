"""Oracle for one Qwen-style GQA decoder layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the layer computes.  Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the product (the HIP library and its Python binding) never does.  It shares no
code with the HIP path; both take their inputs from ``synth``.

Page abbreviations used in the citations below (the four source pages):

* [QWEN] "从零实现 C++ LLM 推理引擎：加载 Qwen2.5-7B 并跑通单层 Forward Pass"
* [TFF]  "十年 C++ 后端 GAP 六个月，写了一个近 3 万行的LLM-TFFInfer推理框架项目解析"
* [HET]  the devpress article on a C++-native heterogeneous inference engine
         ("为什么要做一套 C++ 原生的异构推理引擎")

Every step is written from the definition it cites.  Where the pages are
silent or garbled the plainest reading is taken and named in the docstring.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
  round_bf16, rms_norm, rope_neox, linear (+ A8W8Weight, quantize_rows_int8), silu, q80_expand,
  q80_from_gguf, iq8_expand, a8w8_gemm, kv_levels,
  kv_calibrate, kv_quantize, kv_dequantize, kv_block_exponent, kv_quantize_block,
  attention, attention_online, PagedCache (per-channel and per-block x per-channel),
  layer_forward -- all pinned (worked examples, closed forms, brute force,
  special cases).  The pages' own printed layer output (Qwen2.5-7B-Instruct
  weights, [QWEN] section "运行结果") cannot be reproduced without those
  weights: that end-to-end value is parity unpinned.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round real values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent
    range.  For a value m * 2**e with m in [0.5, 1) (``np.frexp``), the bf16
    quantum is 2**(e-8); below the normal range (|x| < 2**-126) it is fixed at
    2**-133.  ``np.rint`` rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum_exp = np.maximum(e - 8, -133)
    q = np.ldexp(np.ones_like(x), quantum_exp)
    out = np.rint(x / q) * q
    assert np.all(np.isfinite(out[np.isfinite(x)])) and np.all(np.abs(out) < 3.4e38), \
        "value outside bf16 range"
    return out


def q80_expand(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q8_0 weights to real values: blocks of 32 int8 codes along the input
    (K) dimension of each output row share one fp16 scale,
    W[n, k] = scale[n, k // 32] * code[n, k].

    The format is named on [TFF] section 1.1 (Qwen3-8B Q8_0) and its
    block-strided rows on [TFF] section 3.4 (Tensor block size); the 32-code +
    fp16 block is the Q8_0 definition.  The product of an 11-bit significand
    and a 7-bit integer is exact in float64.
    """
    n, k = codes.shape
    assert k % 32 == 0 and scales.shape == (n, k // 32)
    s = np.repeat(scales.astype(np.float64), 32, axis=1)
    return s * codes.astype(np.float64)


def q80_from_gguf(raw, rows: int, cols: int):
    """GGUF's interleaved Q8_0 tensor data to split arrays (int8 codes [rows,
    cols], fp16 scales [rows, cols/32]).

    [TFF] section 1.1 loads Qwen3-8B as a Q8_0 GGUF file; section 3.4's
    block-aware strides store a row of `cols` values as cols/32 consecutive
    blocks.  Reading of the block itself (the pages name it only): 34 bytes,
    the scale as a little-endian IEEE binary16 first, then the 32 int8 codes
    of columns 32b .. 32b+31 in order.  Parsed here one block at a time with
    the struct module, independent of numpy's views.
    """
    import struct
    raw = bytes(np.asarray(raw, np.uint8).tobytes()) if not isinstance(raw, (bytes, bytearray)) else bytes(raw)
    assert cols % 32 == 0 and len(raw) == rows * (cols // 32) * 34
    codes = np.empty((rows, cols), np.int8)
    scales = np.empty((rows, cols // 32), np.float16)
    for r in range(rows):
        for b in range(cols // 32):
            off = (r * (cols // 32) + b) * 34
            (d,) = struct.unpack_from("<e", raw, off)
            scales[r, b] = d
            codes[r, 32 * b:32 * b + 32] = struct.unpack_from("<32b", raw, off + 2)
    return codes, scales


# --------------------------------------------------------------------------
# Layer building blocks
# --------------------------------------------------------------------------

def rms_norm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * g / sqrt(mean(x**2) + eps).

    [QWEN] section "2. 自定义 CUDA Kernels" (the rms_norm kernel: one row, sum of
    squares divided by the row length, eps inside the reciprocal square root,
    then times the weight).  The page's snippet is garbled (no row offset on
    the output); the reading is the textbook RMSNorm: mean over the full row
    length H (not H-1), eps added before the square root.
    """
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def rope_neox(x, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, half-split ("NeoX") pairing.

    x has shape [..., D]; ``pos`` broadcasts against x[..., 0].  For
    i < D/2 the pair (x_i, x_{i+D/2}) is rotated by a = pos * theta**(-2i/D):
    (x_i cos a - x_{i+D/2} sin a,  x_i sin a + x_{i+D/2} cos a).

    [TFF] section 3.7.2 item 4 rotates pairs by a cos/sin table; [QWEN]
    section "2. 自定义 CUDA Kernels" applies RoPE to Q and K heads.  Neither
    fixes the pairing: the half-split pairing is the reading taken because the
    layer is Qwen-style.  Positions are absolute and 0-based; the frequency
    scale is 1.  Angles are formed in float64.
    """
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / D)
    a = np.asarray(pos, np.float64)[..., None] * inv_freq
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_interleaved(x, pos, theta: float) -> np.ndarray:
    """Adjacent-pair variant ((x_{2i}, x_{2i+1}) as one complex number), as
    [TFF] section 3.7.2 item 4 draws it.  Kept only so tests can tell the two
    pairings apart; the layer uses ``rope_neox``."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    a = np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * i / D)
    c, s = np.cos(a), np.sin(a)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


class A8W8Weight:
    """A projection on the A8W8 path ([HET] section 4.5): int8 weight codes
    [N, K] (Linear layout) and a float32 scale per output row (the listing's
    b_scale[n]; no zero point).  ``act`` is the type ("f16" or "bf16") in
    which the layer holds the activation this projection multiplies: the
    activation's int8 codes are decided from those values
    (quantize_rows_int8)."""

    def __init__(self, codes, scale, act: str):
        assert codes.dtype == np.int8 and act in ("f16", "bf16")
        self.codes = codes
        self.scale = np.asarray(scale, np.float32)
        self.act = act


def quantize_rows_int8(x, act: str):
    """Per-row symmetric int8 activation quantisation for the A8W8 path.

    [HET] section 4.5 stores activations as int8 with a scale per row
    (a_scale[m]) but does not say how the scale is chosen.  Reading taken:
    the row as the layer holds it (rounded to fp16 or bf16, ``act``), s =
    max|x| / 127 in float32 (1 for an all-zero row), codes round-half-even(x
    / s) in float32, clipped to [-127, 127].  Returns (codes int8, s float32).
    """
    x = np.asarray(x, np.float64)
    xs = (x.astype(np.float16) if act == "f16" else round_bf16(x)).astype(np.float32)
    s = (np.abs(xs).max(axis=-1) / np.float32(127)).astype(np.float32)
    s = np.where(s == 0, np.float32(1), s).astype(np.float32)
    q = np.rint(xs / s[..., None]).astype(np.int64)  # float32 divide
    return np.clip(q, -127, 127).astype(np.int8), s


def linear(x, w, b=None) -> np.ndarray:
    """Y = X W^T (+ b) with W in [out, in] row-major layout.

    [QWEN] section "4. cuBLAS Row-Major 陷阱": out[M,N] = input[M,K] @ W[N,K]^T.
    An A8W8Weight multiplies the int8 codes of X (quantize_rows_int8) with its
    own in int8 and dequantises with both scales (a8w8_gemm).
    """
    if isinstance(w, A8W8Weight):
        x2 = np.asarray(x, np.float64).reshape(-1, np.shape(x)[-1])
        codes, s = quantize_rows_int8(x2, w.act)
        _, y = a8w8_gemm(codes, w.codes, s, w.scale)
        y = y.reshape(np.shape(x)[:-1] + (w.codes.shape[0],))
        return y + np.asarray(b, np.float64) if b is not None else y
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        y = y + np.asarray(b, np.float64)
    return y


def silu(z) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gate, up) -> np.ndarray:
    """SwiGLU combination silu(gate) * up ([TFF] section 3.7.1 operator list
    "Unary (SwiGLU)"; [QWEN] architecture overview "SwiGLU MLP").  The gate
    branch is the one that goes through SiLU."""
    return silu(gate) * np.asarray(up, np.float64)


def iq8_expand(codes: np.ndarray, scale: np.ndarray, zero_point: np.ndarray) -> np.ndarray:
    """Weight-only int8 with one (scale, zero point) per output channel to
    real values: W[n, k] = (code[n, k] - zero_point[n]) * scale[n] ([HET]
    section 4.4, the per-channel GEMV that dequantises in registers; its
    listing takes int8 codes, an int8 zero point and a float scale per row n
    of the [N, K] matrix).  Exact in float64 (a 9-bit integer times a float32).
    """
    n, k = codes.shape
    assert codes.dtype == np.int8 and scale.shape == (n,) and zero_point.shape == (n,)
    q = codes.astype(np.float64) - zero_point.astype(np.float64)[:, None]
    return q * scale.astype(np.float32).astype(np.float64)[:, None]


def a8w8_gemm(a_codes: np.ndarray, b_codes: np.ndarray, a_scale: np.ndarray, b_scale: np.ndarray):
    """int8 x int8 GEMM with a dequantising epilogue ([HET] section 4.5):
    C[m, n] = sum_k A[m, k] * B[n, k] accumulated exactly (the s8s8s32 MMA),
    then out[m, n] = C[m, n] * a_scale[m] * b_scale[n].  A [M, K] and B [N, K]
    are int8 (B in Linear layout, like every weight here); the scales are
    float32.  Returns (C as int64, out in float64)."""
    assert a_codes.dtype == np.int8 and b_codes.dtype == np.int8
    M, K = a_codes.shape
    N, K2 = b_codes.shape
    assert K == K2 and a_scale.shape == (M,) and b_scale.shape == (N,)
    C = a_codes.astype(np.int64) @ b_codes.astype(np.int64).T
    out = (C.astype(np.float64) * a_scale.astype(np.float32).astype(np.float64)[:, None]
           * b_scale.astype(np.float32).astype(np.float64)[None, :])
    return C, out


# --------------------------------------------------------------------------
# int8 / uint4 asymmetric per-channel KV quantisation
# --------------------------------------------------------------------------

def kv_levels(n_bits: int) -> int:
    """Largest code of an n-bit cache: 255 for int8 ([HET] section 2.6),
    15 for uint4.  The pages list uint4 KV caches ([HET] sections 2.4, 2.6)
    but give the formula only for 8 bits; the reading taken is the same
    asymmetric formula with 2^4 - 1 in place of 255."""
    assert n_bits in (8, 4)
    return (1 << n_bits) - 1


def kv_calibrate(values: np.ndarray, n_bits: int = 8):
    """Per-channel asymmetric parameters from [HET] section 2.6 (量化公式):
    scale_c = (max_c - min_c) / L, zero_point_c = round(-min_c / scale_c),
    with L = 2^n_bits - 1 (255 for the page's int8, 15 for uint4).

    ``values`` is [n_tokens, n_kv_heads, head_dim] float32; a channel is one
    (kv_head, d) pair, reduced over all tokens.  Reading taken: the arithmetic
    is IEEE float32 (the precision the kernel quantises in); round() is
    round-half-to-even; zero_point stays an unclamped int32; a flat channel
    (max == min) gets scale 1.
    """
    v = np.asarray(values, np.float32)
    assert v.ndim == 3 and v.shape[0] > 0
    mx = v.max(axis=0)
    mn = v.min(axis=0)
    scale = (mx - mn) / np.float32(kv_levels(n_bits))
    scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    zp = np.rint(-mn / scale).astype(np.int32)
    return scale, zp


def kv_quantize(x, scale, zp, n_bits: int = 8) -> np.ndarray:
    """Q_c = clamp(round(x / scale_c) + zero_point_c, 0, L) ([HET] section
    2.6, L = 2^n_bits - 1), in float32 with a correctly rounded divide and
    round-half-to-even; stored one code per uint8 element (the page calls
    the 8-bit codes int8 but clamps them to 0..255)."""
    x32 = np.asarray(x, np.float32)
    q = np.rint(x32 / scale).astype(np.int64) + zp.astype(np.int64)
    return np.clip(q, 0, kv_levels(n_bits)).astype(np.uint8)


def kv_dequantize(codes, scale, zp, e=0) -> np.ndarray:
    """x ~ (Q_c - zero_point_c) * scale_c ([HET] section 2.6), times 2^e for
    a block with a per-block factor (kv_block_exponent)."""
    return (np.asarray(codes, np.float64) - zp.astype(np.float64)) * scale.astype(np.float64) * 2.0 ** e


KV_MAX_BLOCK_EXP = 7


def kv_block_exponent(x, scale, zp, n_bits: int = 8) -> int:
    """Per-block factor of a block's per-channel parameters, 2^e.

    [HET] section 2.4 pairs the int8 / uint4 KV cache with scales managed per
    channel and per block, and the paged kernel of section 4.3 dequantises a
    block with its own scales[b].  Reading taken: a block keeps the pool's
    per-channel (scale_c, zero_point_c) and multiplies the scale by a
    power of two 2^e of its own (per KV head, separately for K and V), e the
    smallest integer in [0, KV_MAX_BLOCK_EXP] for which no value x of the
    block (x: [n, D] for one head) clamps: zero_point_c + round(q * 2^-e) is
    in [0, L] with q = x / scale_c (float32, correctly rounded, then scaled
    exactly by the power of two; round half to even).  e = 0 keeps the
    per-channel quantiser exactly; a larger e widens the block's range around
    the zero point for values beyond the calibrated one.  If no e in the
    range fits, e = KV_MAX_BLOCK_EXP (the rest clamps).
    """
    L = (1 << n_bits) - 1
    q = (np.asarray(x, np.float32) / np.asarray(scale, np.float32)).astype(np.float32)
    zp = np.asarray(zp, np.int64)
    for e in range(KV_MAX_BLOCK_EXP + 1):
        r = np.rint(q.astype(np.float64) * 2.0 ** -e).astype(np.int64) + zp
        if np.all((r >= 0) & (r <= L)):
            return e
    return KV_MAX_BLOCK_EXP


def kv_quantize_block(x, scale, zp, e: int, n_bits: int = 8) -> np.ndarray:
    """Codes of values x in a block with factor 2^e: clamp(zero_point_c +
    round(q * 2^-e), 0, L), q = x / scale_c in float32 (kv_block_exponent);
    e = 0 is kv_quantize."""
    L = (1 << n_bits) - 1
    q = (np.asarray(x, np.float32) / np.asarray(scale, np.float32)).astype(np.float32)
    r = np.rint(q.astype(np.float64) * 2.0 ** -e).astype(np.int64) + np.asarray(zp, np.int64)
    return np.clip(r, 0, L).astype(np.uint8)


# --------------------------------------------------------------------------
# Paged KV cache
# --------------------------------------------------------------------------

class PagedCache:
    """Logical model of the block-paged KV cache.

    Physical storage is a pool of fixed-size blocks; a sequence's block table
    maps logical block t // B to a physical block, and token t lives at
    offset t % B of it ([TFF] section 3.6.4, get_location; [HET] section 4.3
    with 16-token blocks).  ``dtype`` is "bf16" (values rounded to bf16 when
    written), "u8" or "u4" (8- or 4-bit codes + per-channel scale/zero point,
    one code per element here).  Keys/values are held per (block, kv_head,
    offset, d); the physical byte layout of the GPU pool is not modelled here.
    """

    def __init__(self, n_blocks: int, n_kv_heads: int, head_dim: int, dtype: str,
                 k_params=None, v_params=None, block_scales: bool = False):
        assert dtype in ("bf16", "u8", "u4")
        assert not block_scales or dtype != "bf16"
        self.dtype = dtype
        self.block_scales = block_scales
        # per (block, kv head) exponents of K and V (kv_block_exponent); 0
        # for every block until a call writes its first slot
        self.ek = np.zeros((n_blocks, n_kv_heads), np.int64)
        self.ev = np.zeros((n_blocks, n_kv_heads), np.int64)
        self.n_bits = 4 if dtype == "u4" else 8
        self.n_blocks, self.n_kv_heads, self.head_dim = n_blocks, n_kv_heads, head_dim
        shape = (n_blocks, n_kv_heads, BLOCK_SIZE, head_dim)
        if dtype == "bf16":
            self.k = np.full(shape, np.nan)
            self.v = np.full(shape, np.nan)
        else:
            assert k_params is not None and v_params is not None
            self.k_scale, self.k_zp = k_params
            self.v_scale, self.v_zp = v_params
            self.k = np.zeros(shape, np.uint8)
            self.v = np.zeros(shape, np.uint8)
            self.written = np.zeros(shape[:1] + shape[2:3], bool)

    @staticmethod
    def location(table_row: np.ndarray, t: int):
        """(physical block, offset) of token t ([TFF] section 3.6.4)."""
        blk = int(table_row[t // BLOCK_SIZE])
        assert blk >= 0, "token beyond the sequence's allocated blocks"
        return blk, t % BLOCK_SIZE

    def write(self, table_row, t: int, k, v):
        """Store token t's K and V ([n_kv_heads, head_dim] real values),
        rounded to the cache dtype (with block scales: the block's current
        factor)."""
        blk, off = self.location(table_row, t)
        if self.dtype == "bf16":
            self.k[blk, :, off, :] = round_bf16(k)
            self.v[blk, :, off, :] = round_bf16(v)
        elif self.block_scales:
            for g in range(self.n_kv_heads):
                self.k[blk, g, off, :] = kv_quantize_block(k[g], self.k_scale[g], self.k_zp[g],
                                                           int(self.ek[blk, g]), self.n_bits)
                self.v[blk, g, off, :] = kv_quantize_block(v[g], self.v_scale[g], self.v_zp[g],
                                                           int(self.ev[blk, g]), self.n_bits)
            self.written[blk, off] = True
        else:
            self.k[blk, :, off, :] = kv_quantize(k, self.k_scale, self.k_zp, self.n_bits)
            self.v[blk, :, off, :] = kv_quantize(v, self.v_scale, self.v_zp, self.n_bits)
            self.written[blk, off] = True

    def write_tokens(self, table_row, start: int, ks, vs):
        """One call's new tokens of one sequence: positions start ..
        start+n-1 get ks[i], vs[i] ([n, n_kv_heads, head_dim]).  With block
        scales, a block whose first slot this call writes takes its factor
        from the tokens this call writes into it (kv_block_exponent, per KV
        head, K and V separately) before they are stored; tokens written into
        a block by a later call use the factor it has."""
        n = len(ks)
        if self.block_scales and n:
            for bs in range((start + BLOCK_SIZE - 1) // BLOCK_SIZE * BLOCK_SIZE, start + n, BLOCK_SIZE):
                blk, _ = self.location(table_row, bs)
                sl = slice(bs - start, min(bs + BLOCK_SIZE, start + n) - start)
                for g in range(self.n_kv_heads):
                    self.ek[blk, g] = kv_block_exponent(np.asarray(ks)[sl, g], self.k_scale[g], self.k_zp[g],
                                                        self.n_bits)
                    self.ev[blk, g] = kv_block_exponent(np.asarray(vs)[sl, g], self.v_scale[g], self.v_zp[g],
                                                        self.n_bits)
        for i in range(n):
            self.write(table_row, start + i, ks[i], vs[i])

    def read(self, table_row, n_tokens: int):
        """Keys and values of tokens 0..n_tokens-1, [n_tokens, n_kv_heads, D],
        as real numbers (codes dequantised)."""
        K = np.empty((n_tokens, self.n_kv_heads, self.head_dim))
        V = np.empty_like(K)
        for t in range(n_tokens):
            blk, off = self.location(table_row, t)
            if self.dtype == "bf16":
                K[t], V[t] = self.k[blk, :, off, :], self.v[blk, :, off, :]
            else:
                assert self.written[blk, off], "reading a slot never written"
                ek = self.ek[blk][:, None] if self.block_scales else 0
                ev = self.ev[blk][:, None] if self.block_scales else 0
                K[t] = kv_dequantize(self.k[blk, :, off, :], self.k_scale, self.k_zp, ek)
                V[t] = kv_dequantize(self.v[blk, :, off, :], self.v_scale, self.v_zp, ev)
        assert np.all(np.isfinite(K)) and np.all(np.isfinite(V)), "reading a slot never written"
        return K, V


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attention(q, q_pos, K, V) -> np.ndarray:
    """Causal grouped-query attention, exact two-pass softmax.

    q: [Tq, Hq, D] queries at absolute positions q_pos [Tq];
    K, V: [Tk, Hkv, D], key j sitting at position j.
    Query head h reads KV head h // (Hq / Hkv) -- consecutive query heads
    share a KV head ([QWEN] section "3. GQA": 28 Q heads share 4 KV heads,
    7:1; the order of the expansion is the reading taken).
    Scores are q.k / sqrt(D) ([HET] section 4.3 kernel comment); a query at
    position p sees keys 0..p (causal mask including the diagonal, [QWEN]
    architecture overview "Causal mask + softmax").  Masked keys are left out.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Tq, Hq, D = q.shape
    Hkv = K.shape[1]
    n_rep = Hq // Hkv
    out = np.empty((Tq, Hq, D))
    for i in range(Tq):
        n_vis = int(q_pos[i]) + 1
        assert n_vis <= K.shape[0]
        for h in range(Hq):
            g = h // n_rep
            s = K[:n_vis, g, :] @ q[i, h] / math.sqrt(D)
            m = s.max()
            e = np.exp(s - m)
            out[i, h] = (e @ V[:n_vis, g, :]) / e.sum()
    return out


def attention_online(q, q_pos, K, V, tile: int) -> np.ndarray:
    """The same attention, computed tile by tile with a running max m,
    running denominator l and rescaled accumulator ([TFF] section 3.7.2
    item 5, online softmax).  The page's update adds one exp term per tile,
    which is only right for one score at a time; the reading used is
    m' = max(m, max s), l' = l e^(m-m') + sum e^(s-m'),
    acc' = acc e^(m-m') + sum e^(s-m') v, o = acc / l."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Tq, Hq, D = q.shape
    n_rep = Hq // K.shape[1]
    out = np.empty((Tq, Hq, D))
    for i in range(Tq):
        n_vis = int(q_pos[i]) + 1
        for h in range(Hq):
            g = h // n_rep
            m, l, acc = -np.inf, 0.0, np.zeros(D)
            for j0 in range(0, n_vis, tile):
                j1 = min(j0 + tile, n_vis)
                s = K[j0:j1, g, :] @ q[i, h] / math.sqrt(D)
                m_new = max(m, s.max())
                alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
                p = np.exp(s - m_new)
                l = l * alpha + p.sum()
                acc = acc * alpha + p @ V[j0:j1, g, :]
                m = m_new
            out[i, h] = acc / l
    return out


# --------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------

# the activation each projection multiplies, as the layer stores it: xn, o
# and hn in fp16, the SwiGLU product a in bf16
A8W8_ACT = {"wq": "f16", "wk": "f16", "wv": "f16", "wo": "f16", "wg": "f16", "wu": "f16", "wd": "bf16"}


def expand_weights(shape, w: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """float64 copies of the weights; Q8_0 and per-channel int8 matrices
    expanded exactly; A8W8 projections kept as codes and scales
    (A8W8Weight)."""
    out = {}
    for name, a in w.items():
        if name.endswith("_scale") or name.endswith("_zp"):
            continue
        if shape.weight_dtype == "a8w8" and name + "_scale" in w:
            out[name] = A8W8Weight(a, w[name + "_scale"], A8W8_ACT[name])
        elif shape.weight_dtype == "q80" and name + "_scale" in w:
            out[name] = q80_expand(a, w[name + "_scale"])
        elif shape.weight_dtype == "iq8" and name + "_scale" in w:
            out[name] = iq8_expand(a, w[name + "_scale"], w[name + "_zp"])
        else:
            out[name] = np.asarray(a, np.float64)
    return out


def layer_forward(shape, w: Dict[str, np.ndarray], x: np.ndarray, q_start, q_len, ctx_len,
                  table: Optional[np.ndarray], cache: Optional[PagedCache],
                  want_stages: bool = False, rows_out=None):
    """Forward pass of one pre-norm Qwen-style GQA decoder layer over a batch
    of sequences.

    Sequence i owns rows q_start[i] .. q_start[i]+q_len[i]-1 of x [rows, H];
    its new tokens sit at positions ctx_len[i] + 0..q_len[i]-1 and its first
    ctx_len[i] tokens are already in ``cache``.  With ``cache`` None (no KV
    cache) each sequence must have ctx_len 0 and attends over its own exact
    keys.  Steps ([QWEN] architecture overview; [TFF] section 4.1 decode
    flow; weights already expanded by ``expand_weights``):

      1. xn = RMSNorm(x, ln1)
      2. q, k, v = xn Wq^T (+bq), xn Wk^T (+bk), xn Wv^T (+bv)
      3. (Qwen3) per-head RMSNorm of q and k over head_dim, gains q_norm/k_norm,
         before RoPE (reading: same eps; gains shared by all heads)
      4. RoPE (half-split) on q and k at each token's position
      5. k, v of new tokens written to the cache (rounded to its dtype), then
         every key/value is read back from the cache ([TFF] 3.6.4; decode
         appends the token at position ctx_len first)
      6. o = causal GQA attention
      7. h = x + o Wo^T                      (residual)
      8. hn = RMSNorm(h, ln2)
      9. a = silu(hn Wg^T) * (hn Wu^T)
     10. y = h + a Wd^T                      (second residual; reading: the
         standard pre-norm layer with two residual adds)

    ``rows_out`` (optional, sorted row indices) restricts steps 6-10 to those
    rows -- every row's k and v still reach the cache -- so long prompts can
    be checked on a sample of rows.  The result then has one row per entry.
    """
    H, D = shape.hidden, shape.head_dim
    Hq, Hkv = shape.n_q_heads, shape.n_kv_heads
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    sel = np.arange(rows) if rows_out is None else np.asarray(rows_out)
    xn = rms_norm(x, w["ln1"], shape.rms_eps)
    q = np.zeros((rows, Hq, D))
    q[sel] = linear(xn[sel], w["wq"], w.get("bq")).reshape(len(sel), Hq, D)
    k = linear(xn, w["wk"], w.get("bk")).reshape(rows, Hkv, D)
    v = linear(xn, w["wv"], w.get("bv")).reshape(rows, Hkv, D)
    if shape.qk_norm:
        q = rms_norm(q, w["q_norm"], shape.rms_eps)
        k = rms_norm(k, w["k_norm"], shape.rms_eps)
    pos = np.empty(rows, np.int64)
    for i in range(len(q_len)):
        r0 = int(q_start[i])
        pos[r0:r0 + int(q_len[i])] = int(ctx_len[i]) + np.arange(int(q_len[i]))
    q = rope_neox(q, pos[:, None], shape.rope_theta)
    k = rope_neox(k, pos[:, None], shape.rope_theta)
    o = np.zeros((rows, Hq, D))
    in_sel = np.zeros(rows, bool)
    in_sel[sel] = True
    for i in range(len(q_len)):
        r0, n, c = int(q_start[i]), int(q_len[i]), int(ctx_len[i])
        if n == 0:
            continue
        if cache is None:
            assert c == 0, "prior context needs a KV cache"
            Ks, Vs = k[r0:r0 + n], v[r0:r0 + n]
        else:
            cache.write_tokens(table[i], c, k[r0:r0 + n], v[r0:r0 + n])
            Ks, Vs = cache.read(table[i], c + n)
        mine = np.arange(r0, r0 + n)[in_sel[r0:r0 + n]]
        if len(mine):
            o[mine] = attention(q[mine], pos[mine], Ks, Vs)
    o2 = o[sel].reshape(len(sel), Hq * D)
    h = x[sel] + linear(o2, w["wo"])
    hn = rms_norm(h, w["ln2"], shape.rms_eps)
    a = swiglu(linear(hn, w["wg"]), linear(hn, w["wu"]))
    y = h + linear(a, w["wd"])
    if want_stages:
        return y, dict(xn=xn[sel], q=q[sel], k=k, v=v, o=o2, h=h, hn=hn, a=a, pos=pos[sel])
    return y


def fill_cache(cache: PagedCache, table: np.ndarray, ctx_len, cache_k, cache_v):
    """Write the already-cached tokens: sequence i's positions 0..ctx_len[i]-1
    come from consecutive rows of cache_k / cache_v ([n, Hkv, D])."""
    r = 0
    for i, c in enumerate(ctx_len):
        cache.write_tokens(table[i], 0, cache_k[r:r + int(c)], cache_v[r:r + int(c)])
        r += int(c)
    assert r == (0 if cache_k is None else cache_k.shape[0])
