"""GGUF Q8_0 import (q80_import_gguf) against the oracle's block parser:
codes and scales bit for bit, and a Q8_0 layer built from the imported
arrays gives the same output bits as one built from the original arrays."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (64, 4096), (1000, 4096 + 32)])
def test_import_matches_oracle_parser(rows, cols):
    import torch
    import transformer_decoder_layer_amd as tdl
    print(f"[gguf import {rows}x{cols}]", flush=True)
    rng = np.random.default_rng(rows * 7 + cols)
    codes = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    scales = (rng.standard_normal((rows, cols // 32)) * 0.01).astype(np.float16)
    raw = synth.gguf_q80_bytes(codes, scales)
    blocks = torch.from_numpy(raw).cuda()
    c = torch.full((rows, cols), 77, dtype=torch.int8, device="cuda")
    s = torch.full((rows, cols // 32), float("nan"), dtype=torch.float16, device="cuda")
    tdl.q80_import_gguf(blocks, rows, cols, c, s)
    torch.cuda.synchronize()
    n_check = min(rows, 40)  # the struct-based parser is slow: a leading slice of rows
    ref_c, ref_s = oracle.q80_from_gguf(raw[:n_check * (cols // 32) * 34], n_check, cols)
    got_c, got_s = c.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(got_c[:n_check], ref_c)
    assert np.array_equal(got_s[:n_check].view(np.uint16), ref_s.view(np.uint16))
    # every row: the original arrays (the serialiser's input) come back
    assert np.array_equal(got_c, codes)
    assert np.array_equal(got_s.view(np.uint16), scales.view(np.uint16))


def test_layer_from_imported_weights_is_identical():
    import torch
    import transformer_decoder_layer_amd as tdl
    from harness import device_weights
    from test_gpu_layer import TINY_Q80 as shape
    print("[gguf layer]", flush=True)
    w = synth.make_weights(shape, seed=3, random_gains=True)
    dw = device_weights(shape, w)
    dw2 = dict(dw)
    for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        rows, cols = w[name].shape
        raw = torch.from_numpy(synth.gguf_q80_bytes(w[name], w[name + "_scale"])).cuda()
        c = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
        s = torch.empty((rows, cols // 32), dtype=torch.float16, device="cuda")
        tdl.q80_import_gguf(raw, rows, cols, c, s)
        dw2[name], dw2[name + "_scale"] = c, s
    outs = []
    for weights in (dw, dw2):
        cfg = tdl.make_config(shape, max_tokens=200)
        layer = tdl.Layer(cfg, weights)
        x = torch.from_numpy(synth.make_x(np.random.default_rng(4), 150, shape.hidden)).to(torch.bfloat16).cuda()
        y = torch.empty_like(x)
        layer.prefill(x, y, 0, None, None)
        torch.cuda.synchronize()
        outs.append(y.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
