"""Pins of the oracle to facts other than itself: worked examples printed in
tests/golden (each with its citation), closed forms, invariants, library
routines for special cases, and brute force on tiny inputs.

Each test names the plausible mistake it would catch."""
import json
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bf16 ----

def test_round_bf16_matches_torch_cast():
    # special case reducing to a library routine: torch's fp32 -> bf16 cast
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.float32([0.0, -0.0, 1.0, 1e-40, 3e38])]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies exactly between 1 and 1 + 2^-7: even mantissa is 1.0
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert oracle.round_bf16(-(1 + 2 ** -8 + 2 ** -30)) == -(1 + 2 ** -7)


# ------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_worked_example():
    g = load("rmsnorm_worked.json")
    y = oracle.rms_norm(np.array([g["x"]]), g["g"], g["eps"])[0]
    np.testing.assert_allclose(y, g["y"], atol=g["atol"])


def test_rmsnorm_constant_row_and_gain():
    # constant row c -> c / sqrt(c^2 + eps) * g (catches eps outside the sqrt,
    # mean over H-1, dropped gain)
    c, eps = 3.0, 1e-6
    gains = np.linspace(0.5, 1.5, 8)
    y = oracle.rms_norm(np.full((1, 8), c), gains, eps)[0]
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * gains, rtol=1e-15)
    # large eps makes its placement visible: mean(x^2) = 1, eps = 3 -> 1/2
    y = oracle.rms_norm(np.ones((1, 4)), np.ones(4), 3.0)[0]
    np.testing.assert_allclose(y, 0.5, rtol=1e-15)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    y = oracle.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, np.ones(64), 0.0), y, rtol=1e-13)


# ---------------------------------------------------------------- RoPE ----

def test_rope_worked_example_both_pairings():
    g = load("rope_worked.json")
    x = np.array(g["x"])
    np.testing.assert_allclose(oracle.rope_neox(x, g["pos"], g["theta"]), g["neox"], atol=g["atol"])
    np.testing.assert_allclose(oracle.rope_interleaved(x, g["pos"], g["theta"]), g["interleaved"],
                               atol=g["atol"])


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    D, theta = 128, 1e6
    x = rng.standard_normal((6, D))
    np.testing.assert_allclose(oracle.rope_neox(x, np.zeros(6), theta), x, rtol=0, atol=0)
    y = oracle.rope_neox(x, np.arange(6) * 977, theta)
    pair_norm = lambda a: a[..., :D // 2] ** 2 + a[..., D // 2:] ** 2
    np.testing.assert_allclose(pair_norm(y), pair_norm(x), rtol=1e-12)
    # <R_p q, R_p' k> depends only on p - p'
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    d1 = oracle.rope_neox(q, 1000, theta) @ oracle.rope_neox(k, 990, theta)
    d2 = oracle.rope_neox(q, 4011, theta) @ oracle.rope_neox(k, 4001, theta)
    assert abs(d1 - d2) < 1e-10
    d3 = oracle.rope_neox(q, 4012, theta) @ oracle.rope_neox(k, 4001, theta)
    assert abs(d1 - d3) > 1e-6


def test_rope_frequency_per_pair():
    # a unit vector in pair i at position p rotates by exactly p * theta^(-2i/D)
    D, theta, p = 16, 1e4, 37
    for i in range(D // 2):
        x = np.zeros(D)
        x[i] = 1.0
        y = oracle.rope_neox(x, p, theta)
        ang = math.atan2(y[i + D // 2], y[i])
        want = math.remainder(p * theta ** (-2 * i / D), 2 * math.pi)
        assert abs(ang - want) < 1e-12


# ------------------------------------------------------------- linear -----

def test_linear_layout_against_loops_and_torch():
    # W is [out, in]: Y[m, n] = sum_k X[m, k] W[n, k] (catches a transposed W)
    rng = np.random.default_rng(4)
    X, W, b = rng.standard_normal((3, 7)), rng.standard_normal((5, 7)), rng.standard_normal(5)
    Y = oracle.linear(X, W, b)
    for m in range(3):
        for n in range(5):
            assert abs(Y[m, n] - (sum(X[m, k] * W[n, k] for k in range(7)) + b[n])) < 1e-12
    X, W = rng.standard_normal((32, 688)), rng.standard_normal((256, 688))
    ref = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(W)).numpy()
    np.testing.assert_allclose(oracle.linear(X, W), ref, rtol=1e-12, atol=1e-12)


def test_silu_values():
    g = load("silu_values.json")
    np.testing.assert_allclose(oracle.silu(g["z"]), g["silu"], atol=g["atol"])
    # swiglu: silu on the gate, not on up (catches swapped branches)
    assert oracle.swiglu(1.0, 2.0) == pytest.approx(2 * 0.7310585786)
    assert oracle.swiglu(2.0, 1.0) == pytest.approx(2.0 / (1 + math.exp(-2.0)))


def test_q80_expand_exact():
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, (4, 96), dtype=np.int8)
    scales = np.abs(rng.standard_normal((4, 3)) * 0.002).astype(np.float16)
    W = oracle.q80_expand(codes, scales)
    for n in range(4):
        for k in range(96):
            assert W[n, k] == float(scales[n, k // 32]) * int(codes[n, k])
    # the block index runs along the input dimension (catches [n, k % 3])
    s = np.array([[1, 2, 4]], np.float16)
    c = np.ones((1, 96), np.int8)
    assert list(oracle.q80_expand(c, s)[0, ::32]) == [1.0, 2.0, 4.0]


def test_q80_from_gguf_hand_blocks():
    """Hand-written 34-byte blocks (tests/golden/q80_gguf_blocks.json): the
    scale bytes come first and are little-endian binary16, the codes are
    signed, and a row's blocks precede the next row's."""
    g = load("q80_gguf_blocks.json")
    for case in g["cases"]:
        raw = bytes.fromhex(case["hex"])
        codes, scales = oracle.q80_from_gguf(raw, case["rows"], case["cols"])
        assert codes.dtype == np.int8 and scales.dtype == np.float16
        assert scales.astype(float).tolist() == case["scales"]
        nb = case["cols"] // 32
        heads = [codes[r, 32 * b:32 * b + 5].tolist() for r in range(case["rows"]) for b in range(nb)]
        assert heads == case["codes_head"]
        W = oracle.q80_expand(codes, scales)
        vals = [W[r, 32 * b:32 * b + 5].tolist() for r in range(case["rows"]) for b in range(nb)]
        assert vals == case["values_head"]
    # every byte of a block lands somewhere: all 256 code bytes round-trip
    raw = b"".join(b"\x00\x3c" + bytes(range(32 * i, 32 * i + 32)) for i in range(8))
    codes, scales = oracle.q80_from_gguf(raw, 1, 256)
    assert codes.view(np.uint8).tolist()[0] == list(range(256))
    assert (scales == 1.0).all()


# ------------------------------------------------------ A8W8 projections ---

def test_quantize_rows_int8_worked_example():
    """Row 0 (exact in fp16): s = 127 / 127 = 1, codes 127, round(-63.5) =
    -64 and round(0.5) = 0 (ties to even), 0.25 -> 0; row 1 all zero: s = 1,
    codes 0; a bf16 row: 300 is exact in bf16, its code is 127 and 1 rounds to
    0 at s = 300/127."""
    x = np.array([[127.0, -63.5, 0.5, 0.25, 0.0], [0.0, 0.0, 0.0, 0.0, 0.0]])
    codes, s = oracle.quantize_rows_int8(x, "f16")
    assert codes.tolist() == [[127, -64, 0, 0, 0], [0, 0, 0, 0, 0]]
    assert s.tolist() == [1.0, 1.0]
    codes, s = oracle.quantize_rows_int8(np.array([[300.0, 1.0, -300.0]]), "bf16")
    assert codes.tolist() == [[127, 0, -127]]
    assert s[0] == np.float32(np.float32(300.0) / np.float32(127.0))
    # the row is rounded to its storage type first: 1 + 2^-9 is 1 in bf16
    # (8 significant bits) but not in fp16 (11): it sets the scale only there
    x = np.array([[1.0 + 2.0 ** -9, 0.5]])
    assert oracle.quantize_rows_int8(x, "bf16")[1][0] == np.float32(1.0) / np.float32(127.0)
    assert oracle.quantize_rows_int8(x, "f16")[1][0] == np.float32(1.0 + 2.0 ** -9) / np.float32(127.0)


def test_a8w8_linear_exact_on_grid_and_orientation():
    """Activations on their own int8 grid (each row's largest entry 127 s_m)
    quantise exactly, so the A8W8 product equals X (codes x row scale)^T; the
    activation scale runs over rows of X and the weight scale over rows of W
    (catches a transposed scale)."""
    rng = np.random.default_rng(23)
    M, N, K = 5, 7, 64
    qa = rng.integers(-127, 128, (M, K))
    qa[:, 3] = 127
    sa = np.array([0.5, 0.25, 1.0, 2.0, 0.125])  # powers of two: exact in fp16
    x = qa * sa[:, None]
    wc = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ws = (rng.random(N) * 0.01 + 0.001).astype(np.float32)
    W = oracle.A8W8Weight(wc, ws, "f16")
    y = oracle.linear(x, W)
    ref = x @ (wc.astype(np.float64) * ws.astype(np.float64)[:, None]).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    b = rng.standard_normal(N)
    np.testing.assert_allclose(oracle.linear(x, W, b), ref + b, rtol=1e-12, atol=1e-12)


def test_a8w8_layer_close_to_expanded_weights():
    """A tiny layer on the A8W8 path stays within the int8 activation
    quantisation's error of the same layer with the weights expanded
    (codes x scale) in float64: a few tenths of a percent."""
    shape = dataclasses.replace(synth.TINY, weight_dtype="a8w8")
    inp = synth.make_inputs(synth.Workload("tiny_a8w8", shape, "prefill", prefill_len=24, kv_dtype="none"),
                            seed=5, random_gains=True)
    W = oracle.expand_weights(shape, inp.weights)
    E = {k: (np.asarray(v.codes, np.float64) * v.scale.astype(np.float64)[:, None]
             if isinstance(v, oracle.A8W8Weight) else v) for k, v in W.items()}
    q0, ql, ctx = np.array([0]), np.array([24]), np.array([0])
    y = oracle.layer_forward(shape, W, inp.x, q0, ql, ctx, None, None)
    ye = oracle.layer_forward(shape, E, inp.x, q0, ql, ctx, None, None)
    x = inp.x.astype(np.float64)
    rel = np.abs((y - x) - (ye - x)).sum() / np.abs(ye - x).sum()
    assert 1e-4 < rel < 2e-2


# ------------------------------------------- per-channel int8 weights ---

def test_iq8_expand_worked_example():
    g = load("iq8_worked.json")
    codes = np.array(g["codes"], np.int8)
    zp = np.array(g["zero_point"], np.int8)
    scale = np.array([float.fromhex(h) for h in g["scale_hex"]], np.float32)
    W = oracle.iq8_expand(codes, scale, zp)
    assert W[:2].tolist() == g["expect_rows_0_1"]
    assert [float(v) for v in W[2]] == [float.fromhex(h) for h in g["expect_row_2_hex"]]


def test_iq8_expand_special_cases_and_orientation():
    rng = np.random.default_rng(8)
    codes = rng.integers(-128, 128, size=(6, 40), dtype=np.int8)
    # zero point 0, scale 1: the codes themselves
    W = oracle.iq8_expand(codes, np.ones(6, np.float32), np.zeros(6, np.int8))
    assert np.array_equal(W, codes.astype(np.float64))
    # a zero point equal to a row's constant code gives a zero row
    c = np.full((2, 8), 7, np.int8)
    assert not oracle.iq8_expand(c, np.float32([3, 3]), np.int8([7, 0])).any(axis=1)[0]
    # parameters belong to output rows (n), not to input columns (k)
    sc = np.float32([1, 2, 4, 8, 16, 32])
    zp = np.int8([0, 1, 2, 3, 4, 5])
    W = oracle.iq8_expand(codes, sc, zp)
    for n in range(6):
        assert np.array_equal(W[n], (codes[n].astype(np.float64) - zp[n]) * sc[n])
    # linear through the expanded matrix: y = s[n] * sum_k x[k] (q[n,k] - zp[n])
    x = rng.standard_normal((3, 40))
    y = oracle.linear(x, W)
    ref = (x @ codes.T.astype(np.float64) - x.sum(1, keepdims=True) * zp.astype(np.float64)) * sc
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_a8w8_gemm_brute_force_and_extremes():
    rng = np.random.default_rng(9)
    A = rng.integers(-128, 128, size=(3, 7), dtype=np.int8)
    B = rng.integers(-128, 128, size=(5, 7), dtype=np.int8)
    sa = np.float32([0.5, 2.0, 0.25])
    sb = np.float32([1.0, 0.125, 4.0, 3.0, 0.5])
    C, out = oracle.a8w8_gemm(A, B, sa, sb)
    for m in range(3):                           # explicit loops, Python ints
        for n in range(5):
            acc = 0
            for k in range(7):
                acc += int(A[m, k]) * int(B[n, k])
            assert C[m, n] == acc
            assert out[m, n] == acc * float(sa[m]) * float(sb[n])   # power-of-two scales: exact
    # the scale of row m multiplies row m, the scale of column n column n
    C1, out1 = oracle.a8w8_gemm(A, B, np.float32([1, 1, 1]), np.float32([1, 0, 0, 0, 0]))
    assert np.array_equal(out1[:, 0], C1[:, 0]) and not out1[:, 1:].any()
    # extremes: -128 * -128 over K = 4096 is 2^26, well inside int32
    big = np.full((1, 4096), -128, np.int8)
    Cb, _ = oracle.a8w8_gemm(big, big, np.float32([1]), np.float32([1]))
    assert Cb[0, 0] == 1 << 26


# ------------------------------------------------- int8 KV quantisation ---

def test_kv_quant_worked_examples():
    g = load("kv_quant_worked.json")
    for case in g["cases"]:
        x = np.array(case["x"], np.float32).reshape(4, 1, 1)
        scale, zp = oracle.kv_calibrate(x)
        assert float(scale[0, 0]) == float.fromhex(case["scale_hex"])
        assert int(zp[0, 0]) == case["zp"]
        codes = oracle.kv_quantize(x, scale, zp)
        assert codes.ravel().tolist() == case["codes"]


def test_kv_quant_invariants_and_error_bound():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((500, 3, 8)) * rng.uniform(0.1, 5, (1, 3, 8))
         + rng.uniform(-2, 2, (1, 3, 8))).astype(np.float32)
    scale, zp = oracle.kv_calibrate(x)
    codes = oracle.kv_quantize(x, scale, zp)
    amin, amax = x.argmin(axis=0), x.argmax(axis=0)
    for h in range(3):
        for d in range(8):
            assert codes[amin[h, d], h, d] == 0
            assert codes[amax[h, d], h, d] in (254, 255)
    deq = oracle.kv_dequantize(codes, scale, zp)
    bound = scale / 2 + 2.0 ** -23 * np.maximum(np.abs(x.min(0)), np.abs(x.max(0))) * 4
    assert np.all(np.abs(deq - x) <= bound[None] * (1 + 1e-6))
    # per-channel: a channel's parameters ignore the other channels
    x2 = x.copy()
    x2[:, 0, 0] *= 100
    s2, z2 = oracle.kv_calibrate(x2)
    assert np.array_equal(s2[1:], scale[1:]) and np.array_equal(z2[:, 1:], zp[:, 1:])
    # values outside the calibrated range clamp
    assert oracle.kv_quantize(np.float32([[[1e6]]]), scale[:1, :1], zp[:1, :1])[0, 0, 0] == 255
    # a flat channel gets scale 1
    s, z = oracle.kv_calibrate(np.full((4, 1, 1), 2.5, np.float32))
    assert s[0, 0] == 1.0 and z[0, 0] == -2


def test_kv_quant_u4_worked_examples():
    g = load("kv_quant_u4_worked.json")
    assert oracle.kv_levels(g["n_bits"]) == 15 and oracle.kv_levels(8) == 255
    for case in g["cases"]:
        x = np.array(case["x"], np.float32).reshape(4, 1, 1)
        scale, zp = oracle.kv_calibrate(x, 4)
        assert float(scale[0, 0]) == float.fromhex(case["scale_hex"])
        assert int(zp[0, 0]) == case["zp"]
        codes = oracle.kv_quantize(x, scale, zp, 4)
        assert codes.ravel().tolist() == case["codes"]


def test_kv_quant_u4_invariants_and_error_bound():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal((300, 2, 8)) * rng.uniform(0.1, 5, (1, 2, 8))
         + rng.uniform(-2, 2, (1, 2, 8))).astype(np.float32)
    scale, zp = oracle.kv_calibrate(x, 4)
    # 15 steps span each channel's range (a 255-step scale would be 17x finer)
    rng_c = x.max(0).astype(np.float64) - x.min(0)
    np.testing.assert_allclose(scale, rng_c / 15, rtol=2 ** -22)
    codes = oracle.kv_quantize(x, scale, zp, 4)
    assert codes.max() <= 15
    amin, amax = x.argmin(axis=0), x.argmax(axis=0)
    for h in range(2):
        for d in range(8):
            assert codes[amin[h, d], h, d] == 0
            assert codes[amax[h, d], h, d] in (14, 15)
            # every level in between is reachable: 300 spread values hit most
            assert len(np.unique(codes[:, h, d])) >= 12
    deq = oracle.kv_dequantize(codes, scale, zp)
    bound = scale / 2 + 2.0 ** -23 * np.maximum(np.abs(x.min(0)), np.abs(x.max(0))) * 4
    assert np.all(np.abs(deq - x) <= bound[None] * (1 + 1e-6))
    # a channel of exactly 16 equally spaced values (step a power of two)
    # takes the codes 0..15 in order
    lv = (np.arange(16, dtype=np.float32) * np.float32(0.125) - np.float32(1)).reshape(16, 1, 1)
    s, z = oracle.kv_calibrate(lv, 4)
    assert s[0, 0] == 0.125 and z[0, 0] == 8
    assert oracle.kv_quantize(lv, s, z, 4).ravel().tolist() == list(range(16))
    # values outside the calibrated range clamp at both ends
    assert oracle.kv_quantize(np.float32([[[1e6]]]), s, z, 4)[0, 0, 0] == 15
    assert oracle.kv_quantize(np.float32([[[-1e6]]]), s, z, 4)[0, 0, 0] == 0


# ------------------------------------------------------------ attention ---

def brute_force_attention(q, q_pos, K, V):
    """Full-matrix attention with an explicit repeat_kv and an explicit mask
    matrix (a different construction from the oracle's per-row loop)."""
    Tq, Hq, D = q.shape
    n_rep = Hq // K.shape[1]
    Kr = np.repeat(K, n_rep, axis=1)          # [Tk, Hq, D]
    Vr = np.repeat(V, n_rep, axis=1)
    S = np.einsum("qhd,khd->hqk", q, Kr) / math.sqrt(D)
    mask = np.arange(K.shape[0])[None, :] <= np.asarray(q_pos)[:, None]
    S = np.where(mask[None], S, -np.inf)
    P = np.exp(S - S.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    return np.einsum("hqk,khd->qhd", P, Vr)


@pytest.mark.parametrize("Hq,Hkv,D,Tq,Tk", [(4, 2, 64, 32, 32), (6, 2, 16, 5, 9), (7, 1, 8, 3, 20),
                                            (3, 3, 4, 4, 4)])
def test_attention_brute_force(Hq, Hkv, D, Tq, Tk):
    rng = np.random.default_rng(Hq * 100 + Tk)
    q = rng.standard_normal((Tq, Hq, D))
    K, V = rng.standard_normal((Tk, Hkv, D)), rng.standard_normal((Tk, Hkv, D))
    q_pos = np.arange(Tk - Tq, Tk)
    np.testing.assert_allclose(oracle.attention(q, q_pos, K, V),
                               brute_force_attention(q, q_pos, K, V), rtol=1e-12, atol=1e-12)


def test_attention_against_torch_sdpa_gqa():
    # library routine: torch SDPA (fp64 CPU, causal, enable_gqa -> query head h
    # reads KV head h // n_rep)
    rng = np.random.default_rng(7)
    T, Hq, Hkv, D = 12, 6, 2, 16
    q, K, V = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(K), t(V), is_causal=True,
                                                           enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.attention(q, np.arange(T), K, V), ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    K, V = rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8))
    q = rng.standard_normal((1, 4, 8))
    # one visible key: the output is that key's value, for every head of the group
    o = oracle.attention(q, [0], K, V)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[0, h // 2], rtol=1e-14)
    # all keys equal: uniform weights, the mean of the visible values
    Ke = np.repeat(K[:1], 10, axis=0)
    o = oracle.attention(q, [6], Ke, V)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[:7, h // 2].mean(axis=0), rtol=1e-12)


@pytest.mark.parametrize("tile", [1, 5, 16])
def test_online_softmax_equals_two_pass(tile):
    rng = np.random.default_rng(9)
    q, K, V = rng.standard_normal((6, 4, 16)) * 3, rng.standard_normal((40, 2, 16)), rng.standard_normal((40, 2, 16))
    pos = np.array([0, 1, 15, 16, 17, 39])
    np.testing.assert_allclose(oracle.attention_online(q, pos, K, V, tile), oracle.attention(q, pos, K, V),
                               rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ paged KV ----

def test_paged_equals_contiguous_bit_exact():
    rng = np.random.default_rng(10)
    Hkv, D, n = 2, 8, 70
    K = synth.to_bf16_values(rng.standard_normal((n, Hkv, D)).astype(np.float32)).astype(np.float64)
    V = synth.to_bf16_values(rng.standard_normal((n, Hkv, D)).astype(np.float32)).astype(np.float64)
    table = synth.random_tables(rng, [n], n_blocks=9)
    cache = oracle.PagedCache(9, Hkv, D, "bf16")
    for t in range(n):
        cache.write(table[0], t, K[t], V[t])
    Kp, Vp = cache.read(table[0], n)
    assert np.array_equal(Kp, K) and np.array_equal(Vp, V)
    q = rng.standard_normal((3, 4, D))
    pos = np.array([5, 40, 69])
    assert np.array_equal(oracle.attention(q, pos, Kp, Vp), oracle.attention(q, pos, K, V))
    # slot addressing: token t at (table[t // 16], t % 16)
    blk, off = cache.location(table[0], 37)
    assert blk == table[0][2] and off == 5
    assert np.array_equal(cache.k[blk, :, off, :], K[37])


def test_paged_u8_roundtrip():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 2, 8)).astype(np.float32)
    params = oracle.kv_calibrate(x)
    cache = oracle.PagedCache(4, 2, 8, "u8", params, params)
    table = np.array([[3, 0, 2]], np.int32)
    for t in range(40):
        cache.write(table[0], t, x[t], x[t])
    Kp, _ = cache.read(table[0], 40)
    np.testing.assert_allclose(Kp, oracle.kv_dequantize(oracle.kv_quantize(x, *params), *params), rtol=0)
    assert np.all(np.abs(Kp - x) <= params[0][None] * 0.5001)


def test_paged_u4_roundtrip():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 2, 8)).astype(np.float32)
    params = oracle.kv_calibrate(x, 4)
    cache = oracle.PagedCache(4, 2, 8, "u4", params, params)
    table = np.array([[1, 3, 0]], np.int32)
    for t in range(40):
        cache.write(table[0], t, x[t], -x[t])
    Kp, Vp = cache.read(table[0], 40)
    assert cache.k.max() <= 15
    np.testing.assert_allclose(Kp, oracle.kv_dequantize(oracle.kv_quantize(x, *params, 4), *params),
                               rtol=0)
    assert np.all(np.abs(Kp - x) <= params[0][None] * 0.5001)
    # the negated values fall outside the range on one side and clamp there
    assert np.all(Vp >= oracle.kv_dequantize(np.zeros((1, 2, 8)), *params) - 1e-12)


# -------------------------------------------- per-block x per-channel KV ---

def test_kv_block_exponent_worked_example():
    """Hand-worked u8 block, D = 2, scale (0.5, 0.25), zero point (128, 10).
    q = x / scale: token 0 (20, 4), token 1 (-140, 248), token 2 (1, 3).
    e = 0 clamps -140 + 128 < 0; e = 1 fits every value, so e = 1 and the
    codes are 128 + rint(q / 2), 10 + rint(q / 2) with ties to even:
    (138, 12), (58, 134), (128 [0.5 -> 0], 12 [1.5 -> 2]); back: (c - zp) * scale * 2."""
    scale = np.array([0.5, 0.25], np.float32)
    zp = np.array([128, 10], np.int32)
    x = np.array([[10.0, 1.0], [-70.0, 62.0], [0.5, 0.75]], np.float32)
    assert oracle.kv_block_exponent(x, scale, zp, 8) == 1
    codes = oracle.kv_quantize_block(x, scale, zp, 1, 8)
    assert codes.tolist() == [[138, 12], [58, 134], [128, 12]]
    back = oracle.kv_dequantize(codes, scale, zp, 1)
    assert back.tolist() == [[10.0, 1.0], [-70.0, 62.0], [0.0, 1.0]]
    # the same block without its outlier token needs no factor
    assert oracle.kv_block_exponent(x[[0, 2]], scale, zp, 8) == 0
    # beyond 2^7 times the range the largest factor is kept and the rest clamps
    assert oracle.kv_block_exponent(np.array([[1e6, 0.0]], np.float32), scale, zp, 8) == oracle.KV_MAX_BLOCK_EXP


def test_kv_block_exponent_brute_force():
    """e is the smallest exponent whose codes need no clamping, found here by
    another route: the pinned per-channel quantiser with the scale itself
    multiplied by 2^e (exact in float32), against the unclamped codes."""
    rng = np.random.default_rng(21)
    for bits in (8, 4):
        L = (1 << bits) - 1
        for trial in range(60):
            scale = (rng.random(6) * 0.2 + 0.01).astype(np.float32)
            zp = rng.integers(0, L + 1, 6).astype(np.int32)
            x = (rng.standard_normal((5, 6)) * rng.choice([0.1, 1.0, 5.0, 40.0])).astype(np.float32)
            e = oracle.kv_block_exponent(x, scale, zp, bits)

            def fits(k):
                sk = (scale * np.float32(2.0 ** k)).astype(np.float32)
                raw = np.rint(x / sk).astype(np.int64) + zp
                return np.all((raw >= 0) & (raw <= L))
            want = next((k for k in range(oracle.KV_MAX_BLOCK_EXP + 1) if fits(k)), oracle.KV_MAX_BLOCK_EXP)
            assert e == want
            sk = (scale * np.float32(2.0 ** e)).astype(np.float32)
            assert np.array_equal(oracle.kv_quantize_block(x, scale, zp, e, bits), oracle.kv_quantize(x, sk, zp, bits))


def test_paged_block_scales_calls():
    """A call that writes a block's first slot sets its factor from the
    tokens it writes there; a later call appending to the block keeps it and
    clamps; values inside the calibrated range give the per-channel cache
    exactly."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((40, 2, 8)).astype(np.float32)
    params = oracle.kv_calibrate(x)
    table = np.array([[3, 0, 2]], np.int32)
    plain = oracle.PagedCache(4, 2, 8, "u8", params, params)
    blk = oracle.PagedCache(4, 2, 8, "u8", params, params, block_scales=True)
    for c in (plain, blk):
        c.write_tokens(table[0], 0, x[:20], x[:20])
        c.write_tokens(table[0], 20, x[20:40], x[20:40])
    assert np.array_equal(plain.k, blk.k) and not blk.ek.any()
    np.testing.assert_array_equal(plain.read(table[0], 40)[0], blk.read(table[0], 40)[0])
    # tokens 0..9 of a new sequence, scaled by 3: the block takes e = 2 (x 4)
    # where the values leave the range (per head), and the call's values
    # come back within half a (widened) step
    big = 3.0 * x[:10]
    c2 = oracle.PagedCache(4, 2, 8, "u8", params, params, block_scales=True)
    t2 = np.array([[1, 2, 3]], np.int32)
    c2.write_tokens(t2[0], 0, big, -big)
    for g in range(2):
        assert c2.ek[1, g] == oracle.kv_block_exponent(big[:, g], params[0][g], params[1][g])
        assert c2.ek[1, g] >= 1
    K, V = c2.read(t2[0], 10)
    step = params[0][None] * (2.0 ** c2.ek[1])[:, None]
    assert np.all(np.abs(K - big) <= 0.5001 * step)
    # a later call appends tokens 10..13 (same block) with the factor kept
    e_before = c2.ek.copy()
    c2.write_tokens(t2[0], 10, 10.0 * x[10:14], x[10:14])
    assert np.array_equal(c2.ek, e_before)
    K2, _ = c2.read(t2[0], 14)
    hi = (255 - params[1].astype(np.float64)) * params[0] * 2.0 ** c2.ek[1][:, None]
    assert np.all(K2[10:14] <= hi[None] + 1e-9)  # clamped at the block's top code
    # the next block (tokens 16..) gets its own factor from its first call
    c2.write_tokens(t2[0], 14, x[14:20], x[14:20])
    assert np.array_equal(c2.ek[2], [oracle.kv_block_exponent(x[16:20, g], params[0][g], params[1][g])
                                     for g in range(2)])


# ---------------------------------------------------------------- layer ---

def tiny_shape(**kw):
    base = dict(name="t", hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, intermediate=40,
                rms_eps=1e-6, rope_theta=1e4, qkv_bias=True, qk_norm=False, weight_dtype="f32")
    base.update(kw)
    return synth.LayerShape(**base)


def run_prefill(shape, w, x, cache=None, start=0, table=None):
    T = x.shape[0]
    return oracle.layer_forward(shape, oracle.expand_weights(shape, w), x, [0], [T], [start],
                                table, cache, want_stages=True)


def test_layer_single_token_closed_form():
    # T = 1: attention returns v itself, so the layer reduces to plain matrix
    # algebra (catches a wrong residual source, a missing bias, swapped MLP
    # branches, or the wrong KV head for a query head)
    shape = tiny_shape()
    w = synth.make_weights(shape, seed=1, random_gains=True)
    x = np.random.default_rng(2).standard_normal((1, 32))
    y, _ = run_prefill(shape, w, x)
    W = {k: np.asarray(v, np.float64) for k, v in w.items()}
    r = lambda a, g: a / np.sqrt(np.mean(a * a) + 1e-6) * g
    xn = r(x[0], W["ln1"])
    v = (W["wv"] @ xn + W["bv"]).reshape(2, 8)
    o = np.concatenate([v[h // 2] for h in range(4)])
    h = x[0] + W["wo"] @ o
    hn = r(h, W["ln2"])
    gte, up = W["wg"] @ hn, W["wu"] @ hn
    want = h + W["wd"] @ (gte / (1 + np.exp(-gte)) * up)
    np.testing.assert_allclose(y[0], want, rtol=1e-12, atol=1e-12)


def test_layer_two_token_closed_form_qk_norm_gains():
    # T = 2 with per-head Q/K RMSNorm and distinct random gains everywhere
    # (ln1, ln2, q_norm, k_norm).  Written as plain matrix algebra: RoPE as an
    # explicit D x D rotation matrix per position, softmax over the two keys
    # by hand.  Non-uniform gains do not commute with the rotation (pair
    # members i and i + D/2 get different gains), so this fails if the Q/K
    # norm runs after RoPE, if q_norm and k_norm are swapped, or if a gain is
    # dropped.  [QWEN] section 2 (RMSNorm times the weight; RoPE on Q and K).
    D, Hq, Hkv = 8, 4, 2
    shape = tiny_shape(qkv_bias=False, qk_norm=True)
    w = synth.make_weights(shape, seed=21, random_gains=True)
    assert not np.allclose(w["q_norm"], w["k_norm"])
    x = np.random.default_rng(22).standard_normal((2, 32))
    y, st = run_prefill(shape, w, x)
    W = {k: np.asarray(v, np.float64) for k, v in w.items()}

    def rms(a, g):
        return a / np.sqrt(np.mean(a * a) + 1e-6) * g

    def rot(p):
        R = np.zeros((D, D))
        for i in range(D // 2):
            ang = p * 1e4 ** (-2.0 * i / D)
            c, s = np.cos(ang), np.sin(ang)
            R[i, i], R[i, i + D // 2] = c, -s
            R[i + D // 2, i], R[i + D // 2, i + D // 2] = s, c
        return R

    q = np.zeros((2, Hq, D))
    k = np.zeros((2, Hkv, D))
    v = np.zeros((2, Hkv, D))
    for t in range(2):
        xn = rms(x[t], W["ln1"])
        qr, kr, vr = W["wq"] @ xn, W["wk"] @ xn, W["wv"] @ xn
        for hh in range(Hq):
            q[t, hh] = rot(t) @ rms(qr[hh * D:(hh + 1) * D], W["q_norm"])
        for g in range(Hkv):
            k[t, g] = rot(t) @ rms(kr[g * D:(g + 1) * D], W["k_norm"])
            v[t, g] = vr[g * D:(g + 1) * D]
    np.testing.assert_allclose(st["q"], q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st["k"], k, rtol=1e-12, atol=1e-12)
    want = np.zeros((2, 32))
    for t in range(2):
        o = np.zeros(Hq * D)
        for hh in range(Hq):
            g = hh // (Hq // Hkv)
            if t == 0:
                o[hh * D:(hh + 1) * D] = v[0, g]
            else:
                s0 = q[1, hh] @ k[0, g] / np.sqrt(D)
                s1 = q[1, hh] @ k[1, g] / np.sqrt(D)
                p0 = 1.0 / (1.0 + np.exp(s1 - s0))
                o[hh * D:(hh + 1) * D] = p0 * v[0, g] + (1.0 - p0) * v[1, g]
        h = x[t] + W["wo"] @ o
        hn = rms(h, W["ln2"])
        gte, up = W["wg"] @ hn, W["wu"] @ hn
        want[t] = h + W["wd"] @ (gte / (1 + np.exp(-gte)) * up)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    # the norm's gains matter here: swapping q_norm and k_norm changes q
    w_sw = dict(w, q_norm=w["k_norm"], k_norm=w["q_norm"])
    _, st_sw = run_prefill(shape, w_sw, x)
    assert np.abs(st_sw["q"] - q).max() > 1e-3


def test_layer_zero_branches():
    shape = tiny_shape()
    w = synth.make_weights(shape, seed=3)
    x = np.random.default_rng(4).standard_normal((5, 32))
    w0 = dict(w, wo=np.zeros_like(w["wo"]), wd=np.zeros_like(w["wd"]))
    y, _ = run_prefill(shape, w0, x)
    assert np.array_equal(y, x)
    w1 = dict(w, wd=np.zeros_like(w["wd"]))
    y, st = run_prefill(shape, w1, x)
    assert np.array_equal(y, st["h"])


def test_layer_qk_norm_step():
    # with qk_norm each head of q and k has unit RMS (gains 1) before RoPE; RoPE
    # preserves pair norms, so the stage output still has unit RMS per head
    shape = tiny_shape(qkv_bias=False, qk_norm=True, rms_eps=1e-12)
    w = synth.make_weights(shape, seed=5)
    x = np.random.default_rng(6).standard_normal((3, 32)) * 4
    _, st = run_prefill(shape, w, x)
    np.testing.assert_allclose(np.sqrt(np.mean(st["q"] ** 2, -1)), 1.0, rtol=1e-5)
    np.testing.assert_allclose(np.sqrt(np.mean(st["k"] ** 2, -1)), 1.0, rtol=1e-5)


def test_prefill_decode_consistency():
    # the last row of prefill over S+1 tokens equals a decode step at context S
    shape = tiny_shape()
    w = synth.make_weights(shape, seed=7)
    W = oracle.expand_weights(shape, w)
    S = 21
    x = synth.to_bf16_values(np.random.default_rng(8).standard_normal((S + 1, 32)).astype(np.float32))
    table = np.array([[4, 1]], np.int32)
    c1 = oracle.PagedCache(6, 2, 8, "bf16")
    y_full = oracle.layer_forward(shape, W, x, [0], [S + 1], [0], table, c1)
    c2 = oracle.PagedCache(6, 2, 8, "bf16")
    oracle.layer_forward(shape, W, x[:S], [0], [S], [0], table, c2)
    y_dec = oracle.layer_forward(shape, W, x[S:], [0], [1], [S], table, c2)
    np.testing.assert_allclose(y_dec[0], y_full[S], rtol=1e-13, atol=1e-13)
    # chunked prefill (two chunks) equals the one-shot rows
    c3 = oracle.PagedCache(6, 2, 8, "bf16")
    y_a = oracle.layer_forward(shape, W, x[:9], [0], [9], [0], table, c3)
    y_b = oracle.layer_forward(shape, W, x[9:], [0], [S + 1 - 9], [9], table, c3)
    np.testing.assert_allclose(np.concatenate([y_a, y_b]), y_full, rtol=1e-13, atol=1e-13)


def test_batch_rows_independent():
    # a mixed batch gives each sequence the result it gets alone
    shape = tiny_shape()
    W = oracle.expand_weights(shape, synth.make_weights(shape, seed=9))
    rng = np.random.default_rng(10)
    x = rng.standard_normal((7, 32))
    table = np.array([[0, 1, -1], [2, 3, 4]], np.int32)
    cache = oracle.PagedCache(5, 2, 8, "bf16")
    kv = rng.standard_normal((40, 2, 8))
    oracle.fill_cache(cache, table, [0, 40], kv, kv)
    import copy
    c_alone = copy.deepcopy(cache)
    y = oracle.layer_forward(shape, W, x, [0, 6], [6, 1], [0, 40], table, cache)
    y1 = oracle.layer_forward(shape, W, x[6:], [0], [1], [40], table[1:], c_alone)
    np.testing.assert_allclose(y[6], y1[0], rtol=1e-13)


def test_sampled_rows_equal_full_rows():
    # restricting the output rows changes nothing in the rows that are kept
    shape = tiny_shape()
    W = oracle.expand_weights(shape, synth.make_weights(shape, seed=11))
    x = np.random.default_rng(12).standard_normal((20, 32))
    table = np.array([[2, 0]], np.int32)
    y_all = oracle.layer_forward(shape, W, x, [0], [20], [0], table, oracle.PagedCache(3, 2, 8, "bf16"))
    sel = np.array([0, 7, 19])
    y_sel = oracle.layer_forward(shape, W, x, [0], [20], [0], table, oracle.PagedCache(3, 2, 8, "bf16"),
                                 rows_out=sel)
    assert np.array_equal(y_sel, y_all[sel])
