"""int8 x int8 GEMM ([HET] 4.5) through the C ABI: the int32 sums bit for bit
against the oracle's exact integer products, the dequantised output to fp32
rounding, on ragged shapes that span several 128 x 128 tiles and a partial
64-wide k step, the int8 extremes, and sampled rows of a full-size shape."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(A, B, sa, sb, with_c=True):
    import torch
    import transformer_decoder_layer_amd as tdl
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    M, N = A.shape[0], B.shape[0]
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    c = torch.zeros((M, N), dtype=torch.int32, device="cuda") if with_c else None
    print(f"[a8w8] M={M} N={N} K={A.shape[1]}", flush=True)
    tdl.gemm_a8w8(dev(A), dev(B), dev(sa), dev(sb), out, c)
    torch.cuda.synchronize()
    return (c.cpu().numpy() if with_c else None), out.cpu().numpy()


def _check_out(out, ref):
    # out = fl(fl(float(C) * a) * b): within a few float32 ulps of the exact product
    assert np.all(np.isfinite(out))
    assert np.all(np.abs(out - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-30)


# K % 64 == 0 (1024, 960): the direct-to-LDS kernel; otherwise the
# register-staged one
@pytest.mark.parametrize("M,N,K", [(77, 200, 208), (300, 520, 1024), (300, 520, 960), (1, 1, 16), (129, 127, 80)])
def test_a8w8_matches_oracle(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    sa = (np.abs(rng.standard_normal(M)) * 0.01 + 1e-4).astype(np.float32)
    sb = (np.abs(rng.standard_normal(N)) * 0.01 + 1e-4).astype(np.float32)
    C, out = _run(A, B, sa, sb)
    Cref, ref = oracle.a8w8_gemm(A, B, sa, sb)
    assert np.array_equal(C.astype(np.int64), Cref)
    _check_out(out, ref)
    _, out2 = _run(A, B, sa, sb, with_c=False)   # no int32 output: same result
    assert np.array_equal(out2, out)


def test_a8w8_extremes():
    K = 4096
    A = np.full((130, K), -128, np.int8)
    A[1] = 127
    B = np.full((3, K), -128, np.int8)
    C, out = _run(A, B, np.ones(130, np.float32), np.float32([1, 0.5, 2]))
    assert (C[0] == 1 << 26).all() and (C[1] == -127 * 128 * K).all()
    assert out[0].tolist() == [2.0 ** 26, 2.0 ** 25, 2.0 ** 27]


def test_a8w8_full_size_sampled_rows():
    # the Qwen2.5-7B gate/up shape (M 4096 tokens, N 2 x 18944, K 3584):
    # every row computed on the GPU, a sample of rows checked exactly
    M, N, K = 4096, 37888, 3584
    rng = np.random.default_rng(5)
    A = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    sa = (np.abs(rng.standard_normal(M)) * 0.01 + 1e-4).astype(np.float32)
    sb = (np.abs(rng.standard_normal(N)) * 0.01 + 1e-4).astype(np.float32)
    C, out = _run(A, B, sa, sb)
    rows = [0, 1, 127, 128, 2047, 4000, 4095]
    cols = np.r_[0:200, 18000:18200, N - 200:N]
    Cref, ref = oracle.a8w8_gemm(A[rows], B[cols], sa[rows], sb[cols])
    assert np.array_equal(C[np.ix_(rows, cols)].astype(np.int64), Cref)
    _check_out(out[np.ix_(rows, cols)], ref)
