"""Test harness: runs one workload call through the C-ABI (GPU) and through
the oracle (CPU) on the same seeded inputs, and measures the difference.

Tolerance (the bf16 bar): max |y - r| <= 2e-2 * max |r| and
sum |y - r| / sum |r| <= 5e-3 (a normalised L1; a per-element ratio is
ill-conditioned near zero).  The GPU tests apply it to the layer output y and
to the stage buffers (RMSNorm output, rotated q, attention output, the
attention branch h - x, the SwiGLU product, the MLP branch y - h), so a
residual add cannot hide an error in a branch."""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth

MAX_ABS_FRAC = 2e-2
MEAN_REL = 5e-3


@dataclasses.dataclass
class Err:
    max_abs: float
    max_ref: float
    mean_rel: float

    @property
    def ok(self) -> bool:
        return self.max_abs <= MAX_ABS_FRAC * self.max_ref and self.mean_rel <= MEAN_REL

    def __str__(self):
        return (f"max_abs={self.max_abs:.3e} (limit {MAX_ABS_FRAC * self.max_ref:.3e}) "
                f"mean_rel={self.mean_rel:.3e} (limit {MEAN_REL:.1e})")


def compare(y, ref) -> Err:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), "non-finite output"
    d = np.abs(y - ref)
    return Err(float(d.max()), float(np.abs(ref).max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300)))


def compare_branch_bf16(y, h, y_ref, h_ref) -> Err:
    """The MLP branch y - h of a layer whose output y is bf16.  y is the GPU's
    fp32 sum h + branch rounded once to bf16, so y - h carries up to half a
    bf16 quantum of |y| that is no error of the branch; only the part of
    |(y - h) - (y_ref - h_ref)| beyond that half quantum counts, against the
    same bar as every other stage (relative to the branch, not to y)."""
    y = np.asarray(y, np.float64)
    h = np.asarray(h, np.float64)
    br_ref = np.asarray(y_ref, np.float64) - np.asarray(h_ref, np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    _, e = np.frexp(y)
    half_quantum = np.ldexp(np.ones_like(y), np.maximum(e - 9, -134))
    d = np.maximum(np.abs((y - h) - br_ref) - half_quantum, 0.0)
    return Err(float(d.max()), float(np.abs(br_ref).max()),
               float(d.sum() / max(np.abs(br_ref).sum(), 1e-300)))


def unpack_u4(kt, vt):
    """Codes of a u4 pool from its byte views (KvCache.tensors): K [blocks,
    Hkv, 16, D], V [blocks, Hkv, D, 16].  Byte layout as include/tdl.h states
    it: K byte 4j + i of a row holds channels 8j + i (low nibble) and 8j + 4
    + i (high); V byte (c, slot) holds channels 2c and 2c + 1."""
    k = kt.cpu().numpy()
    v = vt.cpu().numpy()
    hd = k.shape[-1]
    K = np.empty(k.shape[:-1] + (2 * hd,), np.uint8)
    j, i = np.arange(hd) // 4, np.arange(hd) % 4
    K[..., 8 * j + i] = k & 15
    K[..., 8 * j + 4 + i] = k >> 4
    V = np.empty(v.shape[:2] + (2 * hd, v.shape[3]), np.uint8)
    V[:, :, 0::2, :] = v & 15
    V[:, :, 1::2, :] = v >> 4
    return K, V


# ------------------------------------------------------------------ oracle

def oracle_cache(inp: synth.LayerInputs, seqs=None) -> Optional[oracle.PagedCache]:
    """The oracle's cache holding the already-cached tokens of the chosen
    sequences (all by default).  u8 / u4 parameters come from every cached
    token."""
    wl, shape, b = inp.workload, inp.workload.shape, inp.batch
    if wl.kv_dtype == "none":
        return None
    if wl.kv_dtype == "bf16":
        cache = oracle.PagedCache(b.n_blocks, shape.n_kv_heads, shape.head_dim, "bf16")
    else:
        bits = 4 if wl.kv_dtype == "u4" else 8
        ck = inp.cache_k if inp.calib_k is None else inp.calib_k
        cv = inp.cache_v if inp.calib_v is None else inp.calib_v
        kp = oracle.kv_calibrate(ck, bits)
        vp = oracle.kv_calibrate(cv, bits)
        cache = oracle.PagedCache(b.n_blocks, shape.n_kv_heads, shape.head_dim, wl.kv_dtype, kp, vp,
                                  block_scales=inp.block_scales)
    if inp.cache_k is not None:
        # one call writes every sequence's cached tokens from position 0
        seqs = range(b.n_seqs) if seqs is None else seqs
        off = np.concatenate([[0], np.cumsum(b.ctx_len)])
        for i in seqs:
            n = int(b.ctx_len[i])
            cache.write_tokens(b.table[i], 0, inp.cache_k[off[i]:off[i] + n], inp.cache_v[off[i]:off[i] + n])
    return cache


def run_oracle(inp: synth.LayerInputs, seqs: Optional[List[int]] = None, want_stages=False,
               rows_out=None, weights=None):
    """Oracle output rows of the chosen sequences (all by default), in row
    order, with their row indices.  ``rows_out`` (absolute row indices within
    the chosen sequences) restricts the outputs to a sample of rows;
    ``weights`` replaces the expanded weights (oracle.expand_weights)."""
    shape, b = inp.workload.shape, inp.batch
    W = oracle.expand_weights(shape, inp.weights) if weights is None else weights
    seqs = list(range(b.n_seqs)) if seqs is None else list(seqs)
    cache = oracle_cache(inp, seqs)
    rows = np.concatenate([np.arange(b.q_start[i], b.q_start[i] + b.q_len[i]) for i in seqs])
    q_len = b.q_len[seqs]
    q_start = np.concatenate([[0], np.cumsum(q_len)[:-1]])
    sel = None
    if rows_out is not None:
        pos_of = {int(r): k for k, r in enumerate(rows)}
        sel = np.array(sorted(pos_of[int(r)] for r in rows_out))
    out = oracle.layer_forward(shape, W, inp.x[rows], q_start, q_len, b.ctx_len[seqs],
                               b.table[seqs], cache, want_stages=want_stages, rows_out=sel)
    if sel is not None:
        rows = rows[sel]
    return rows, out, cache


# --------------------------------------------------------------------- GPU

def device_weights(shape: synth.LayerShape, w: Dict[str, np.ndarray]):
    import torch
    out = {}
    for name, a in w.items():
        if name.endswith("_scale"):
            out[name] = torch.from_numpy(a).cuda()
        elif a.dtype == np.int8:
            out[name] = torch.from_numpy(a).cuda()
        elif name.startswith("w") and shape.weight_dtype == "bf16":
            out[name] = torch.from_numpy(a).to(torch.bfloat16).cuda()
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return out


@dataclasses.dataclass
class GpuRun:
    y: np.ndarray
    layer: object
    kv: object
    tensors: dict


def gpu_setup(inp: synth.LayerInputs, max_tokens: Optional[int] = None, max_position: int = 16384,
              rope_fused: bool = False):
    """Creates the layer and the cache (filled with the cached tokens) and
    uploads x and the batch arrays."""
    import torch
    import transformer_decoder_layer_amd as tdl
    wl, shape, b = inp.workload, inp.workload.shape, inp.batch
    n_rows = b.n_rows
    cfg = tdl.make_config(shape, max_tokens=max_tokens or max(n_rows, 1), max_seqs=max(b.n_seqs, 1),
                          max_position=max_position, rope_fused=rope_fused)
    layer = tdl.Layer(cfg, device_weights(shape, inp.weights))
    kv = None
    t = {}
    t["x"] = torch.from_numpy(inp.x).to(torch.bfloat16).cuda()
    t["y"] = torch.full_like(t["x"], float("nan"))
    t["table"] = torch.from_numpy(b.table).cuda()
    t["q_start"] = torch.from_numpy(b.q_start).cuda()
    t["q_len"] = torch.from_numpy(b.q_len).cuda()
    t["ctx_len"] = torch.from_numpy(b.ctx_len).cuda()
    if wl.kv_dtype != "none":
        kv = tdl.KvCache(b.n_blocks, shape.n_kv_heads, shape.head_dim, wl.kv_dtype,
                         block_scales=inp.block_scales)
        if inp.calib_k is not None and wl.kv_dtype in ("u8", "u4"):
            kv.calibrate(torch.from_numpy(inp.calib_k).cuda(), torch.from_numpy(inp.calib_v).cuda())
        if inp.cache_k is not None:
            ck = torch.from_numpy(inp.cache_k).cuda()
            cv = torch.from_numpy(inp.cache_v).cuda()
            if wl.kv_dtype in ("u8", "u4") and inp.calib_k is None:
                kv.calibrate(ck, cv)
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(b.ctx_len)]).astype(np.int32)).cuda()
            zero = torch.zeros(b.n_seqs, dtype=torch.int32, device="cuda")
            kv.write(cu, zero, t["table"], ck, cv)
            del ck, cv
    return layer, kv, t


def gpu_call(inp: synth.LayerInputs, layer, kv, t, stream=None):
    wl, b = inp.workload, inp.batch
    if wl.kind == "prefill":
        layer.prefill(t["x"], t["y"], int(b.ctx_len[0]), kv, t["table"] if kv else None, stream=stream)
    elif wl.kind == "decode":
        max_ctx = int((b.ctx_len + 1).max())
        layer.decode_paged(t["x"], t["y"], t["ctx_len"], t["table"], max_ctx, kv, stream=stream)
    else:
        n_pre = int((b.q_len > 1).sum())
        max_q = int(b.q_len[:n_pre].max()) if n_pre else 0
        layer.step(t["x"], t["y"], t["q_start"], t["q_len"], t["ctx_len"], t["table"], n_pre, max_q,
                   int((b.ctx_len + b.q_len).max()), kv, stream=stream)


def run_gpu(inp: synth.LayerInputs, **kw) -> GpuRun:
    import torch
    layer, kv, t = gpu_setup(inp, **kw)
    gpu_call(inp, layer, kv, t)
    torch.cuda.synchronize()
    y = t["y"].float().cpu().numpy()
    return GpuRun(y, layer, kv, t)
