"""GPU parity of the quantization kernels against the oracle: bit-exact codes
and scales (integer work), including every bf16 bit pattern."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import mx
from tests import layout

pytestmark = pytest.mark.gpu


def _all_bf16_finite():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = mx.bf16_bits_to_f64(bits)
    return bits[np.isfinite(v)]


def _special_rows(cols):
    """Rows built to hit the corner cases: zero blocks, subnormal maxima,
    exact ties, values past the saturation point, signed zeros."""
    rng = np.random.default_rng(42)
    rows = []
    rows.append(np.zeros(cols, np.float32))
    r = np.zeros(cols, np.float32); r[::3] = -0.0; rows.append(r)
    rows.append((rng.standard_normal(cols) * 1e-40).astype(np.float32))           # subnormals
    rows.append(np.tile(np.array([4, 5, 7, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 6, -5, -7, 7.5, 1e-3, 0, -0.0], np.float32), cols // 16))
    rows.append(np.tile(np.array([448, 464, 465, 480, 256, 300, -460, 1.0, 2.0 ** -9, 2.0 ** -10, 2.0 ** -6, 0, 3, 5, 7, 9], np.float32), cols // 16))
    rows.append((rng.standard_normal(cols) * 3e38 / 4).astype(np.float32))          # near fp32 max
    rows.append(np.ldexp(rng.uniform(1, 2, cols), rng.integers(-149, 127, cols)).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_weight_quant_rowmajor_matches_oracle(fmt):
    rng = np.random.default_rng(1)
    w = np.concatenate([(rng.standard_normal((57, 256)) * 0.02).astype(np.float32), _special_rows(256)])
    codes, scales = binding.mx_quantize_weights(torch.from_numpy(w).cuda(), fmt, "rowmajor")
    rc, rs = mx.mx_quantize(w.astype(np.float64), fmt)
    if fmt == "fp4":
        rc = mx.pack_fp4(rc)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_weight_quant_every_bf16_value(fmt):
    bits = _all_bf16_finite()
    vals = mx.bf16_bits_to_f64(bits).astype(np.float32)
    rng = np.random.default_rng(2)
    n = len(vals) // 256 * 256
    for arr in (np.sort(vals)[:n], rng.permutation(vals)[:n]):   # similar and mixed magnitudes per block
        w = arr.reshape(-1, 256)
        codes, scales = binding.mx_quantize_weights(torch.from_numpy(np.ascontiguousarray(w)).cuda(), fmt, "rowmajor")
        rc, rs = mx.mx_quantize(w.astype(np.float64), fmt)
        if fmt == "fp4":
            rc = mx.pack_fp4(rc)
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt,shape", [("fp4", (32, 640)), ("fp8", (32, 640)), ("fp4", (2048, 3072)), ("fp8", (3072, 1024))])
def test_weight_quant_tiled_matches_oracle_layout(fmt, shape):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    codes, scales = binding.mx_quantize_weights(torch.from_numpy(w).cuda(), fmt, "tiled")
    rc, rs = mx.mx_quantize(w.astype(np.float64), fmt)
    tc, ts = layout.tile_weight(rc, rs, fmt)
    assert np.array_equal(codes.cpu().numpy(), tc)
    assert np.array_equal(scales.cpu().numpy(), ts)


def test_act_quant_every_bf16_pattern():
    bits = _all_bf16_finite()
    rng = np.random.default_rng(4)
    n = len(bits) // 256 * 256
    for arr in (np.sort(bits)[:n], rng.permutation(bits)[:n]):
        x = np.ascontiguousarray(arr.reshape(-1, 256))
        codes, scales = binding.mxfp4_quant_act(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
        rc, rs = mx.mx_quantize(mx.bf16_bits_to_f64(x), "fp4")
        assert np.array_equal(codes.cpu().numpy(), mx.pack_fp4(rc))
        assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("name", ["tiny", "decode16", "prefill"])
def test_act_quant_workload_shapes(name):
    cfg = synth.workload(name)
    x = synth.activations(cfg)
    codes, scales = binding.mxfp4_quant_act(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
    rows = np.arange(x.shape[0]) if x.shape[0] <= 16 else np.random.default_rng(5).choice(x.shape[0], 256, replace=False)
    rc, rs = mx.mx_quantize(mx.bf16_bits_to_f64(x[rows]), "fp4")
    assert np.array_equal(codes.cpu().numpy()[rows], mx.pack_fp4(rc))
    assert np.array_equal(scales.cpu().numpy()[rows], rs)
