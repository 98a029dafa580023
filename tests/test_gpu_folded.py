"""The shared expert folded into the expert table as an MXFP4 expert: the
MXFP8 -> MXFP4 re-quantization kernel bit for bit against the oracle's, and
the folded layer (expert E selected by every row with weight 1) on the fused
decode and grouped paths against the oracle's folded layer."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe, mx
from tests import helpers
from tests import layout as layout_mod

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("which", ["ws13", "ws2"])
def test_requant_full_size_shared_matrices_tiled(which):
    """The full-size shared expert (gate/up [2048, 3072], down [3072, 1024]):
    fp32 draws -> the library's MXFP8 (tiled) -> its MXFP4 re-quantization,
    against the oracle's MXFP8 quantization and re-quantization of the same
    draws, laid out tiled."""
    cfg = synth.workload("decode1")
    w = synth.device_shared_w13(cfg) if which == "ws13" else synth.device_shared_w2(cfg)
    rows, cols = w.shape
    q8, q8s = binding.mx_quantize_weights(w, "fp8", "tiled")
    c4, s4 = binding.mx_requant_fp8_to_fp4(q8, q8s, rows, cols, "tiled")
    torch.cuda.synchronize()
    oc8, os8 = mx.mx_quantize(w.cpu().numpy().astype(np.float64), "fp8")
    oc4, os4 = mx.requant_fp8_to_fp4(oc8, os8)
    tc, ts = layout_mod.tile_weight(oc4, os4, "fp4")
    assert np.array_equal(c4.cpu().numpy(), tc)
    assert np.array_equal(s4.cpu().numpy(), ts)


def test_requant_every_e4m3_code_rowmajor():
    """Row-major MXFP8 input written directly: every finite E4M3 code in every
    block position, with scale codes from 100 to 154, against the oracle."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # 254 codes
    rng = np.random.default_rng(3)
    rows, cols = 64, 256
    c8 = np.empty((rows, cols), np.uint8)
    flat = np.concatenate([rng.permutation(codes) for _ in range(rows * cols // codes.size + 1)])
    c8[:] = flat[:rows * cols].reshape(rows, cols)
    s8 = rng.integers(100, 155, size=(rows, cols // 32)).astype(np.uint8)
    d8 = torch.from_numpy(c8).cuda().contiguous()
    ds8 = torch.from_numpy(s8).cuda().contiguous()
    c4, s4 = binding.mx_requant_fp8_to_fp4(d8, ds8, rows, cols, "rowmajor")
    torch.cuda.synchronize()
    oc4, os4 = mx.requant_fp8_to_fp4(c8, s8)
    assert np.array_equal(s4.cpu().numpy(), os4)
    assert np.array_equal(c4.cpu().numpy(), mx.pack_fp4(oc4))


_CACHE = {}


def _folded(name):
    """(cfg, GPU folded layer, oracle folded layer) for workload ``name``:
    the GPU layer re-quantizes the library's MXFP8 shared expert, the oracle
    folds its own."""
    if name not in _CACHE:
        cfg = synth.workload(name)
        gl = helpers.gpu_layer(cfg)
        H, I = cfg["H"], cfg["I"]
        c13, s13 = binding.mx_requant_fp8_to_fp4(gl.ws13, gl.ws13_scale, 2 * I, H)
        c2, s2 = binding.mx_requant_fp8_to_fp4(gl.ws2, gl.ws2_scale, H, I)
        gf = gl.folded_from(c13, s13, c2, s2)
        torch.cuda.synchronize()
        of = moe.fold_shared_expert(helpers.oracle_layer(cfg))
        _CACHE[name] = (cfg, gf, of)
    return _CACHE[name]


@pytest.mark.parametrize("name,T", [("decode1", 1), ("decode16", 16), ("tp4", 16)])
def test_folded_decode_matches_oracle(name, T):
    cfg, gf, of = _folded(name)
    x = synth.activations(cfg, T=T, index=60 + T)
    r = synth.activations(cfg, T=T, index=70 + T)
    print(f"[folded] {name} decode T={T}", flush=True)
    y, ids, w = binding.fused_moe_mxfp4_decode(gf, _dev(x), residual=_dev(r), return_routing=True)
    torch.cuda.synchronize()
    y, ids, w = _host(y), ids.cpu().numpy(), w.cpu().numpy()
    assert ids.shape == (T, cfg["k"]) and ids.max() < cfg["E"]
    helpers.compare_with_oracle(dict(cfg, I_s=0), gf, of, x, y, ids, w, residual_bits=r, label="folded decode")


@pytest.mark.parametrize("name,T", [("tp4", 200), ("decode16", 37)])
def test_folded_grouped_matches_oracle_and_decode(name, T):
    cfg, gf, of = _folded(name)
    x = synth.activations(cfg, T=T, index=80 + T)
    print(f"[folded] {name} grouped T={T}", flush=True)
    y = binding.fused_moe_mxfp4_grouped(gf, _dev(x))
    torch.cuda.synchronize()
    y = _host(y)
    helpers.compare_with_oracle(dict(cfg, I_s=0), gf, of, x, y, label="folded grouped")
    ws = binding.decode_workspace(gf)
    for t0 in range(0, T, 16):
        yd = binding.fused_moe_mxfp4_decode(gf, _dev(x[t0:t0 + 16]), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(_host(yd), y[t0:t0 + 16]), t0


def _nvfp4_dev(codes, bscales, gscale):
    packed = mx.pack_fp4(codes)
    return (torch.from_numpy(packed).cuda().contiguous(), torch.from_numpy(bscales).cuda().contiguous(),
            torch.from_numpy(gscale).cuda().contiguous())


@pytest.mark.parametrize("layout", ["tiled", "rowmajor"])
def test_nvfp4_requant_full_size_expert_gate_up(layout):
    """A synthetic NVFP4 gate/up matrix of the full-size expert ([2048, 3072],
    gate and up halves with their own fp32 second-level scales) re-quantized
    to MXFP4 by the library, against the oracle, bit for bit."""
    cfg = synth.workload("decode1")
    rows, cols = 2 * cfg["I"], cfg["H"]
    codes, bscales, gscale = synth.nvfp4_matrix(cfg, 0, 0, rows, cols, n_global=2)
    c, bs, g = _nvfp4_dev(codes, bscales, gscale)
    c4, s4 = binding.mx_requant_nvfp4_to_fp4(c, bs, g, rows // 2, layout)
    torch.cuda.synchronize()
    oc4, os4 = mx.requant_nvfp4_to_mxfp4(codes, bscales, gscale, rows // 2)
    if layout == "tiled":
        tc, ts = layout_mod.tile_weight(oc4, os4, "fp4")
        assert np.array_equal(c4.cpu().numpy(), tc)
        assert np.array_equal(s4.cpu().numpy(), ts)
    else:
        assert np.array_equal(c4.cpu().numpy(), mx.pack_fp4(oc4))
        assert np.array_equal(s4.cpu().numpy(), os4)


def test_nvfp4_requant_every_code_and_block_scale():
    """Every E2M1 code under every finite E4M3 block scale (with and without
    the sign bit) and several second-level scales, row-major."""
    rows, cols = 256, 512
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    bscales = rng.choice(finite, size=(rows, cols // 16)).astype(np.uint8)
    gscale = np.array([1.0, 0.3, 2.0 ** -10, 7.25e-6], np.float32)
    c, bs, g = _nvfp4_dev(codes, bscales, gscale)
    c4, s4 = binding.mx_requant_nvfp4_to_fp4(c, bs, g, rows // 4, "rowmajor")
    torch.cuda.synchronize()
    oc4, os4 = mx.requant_nvfp4_to_mxfp4(codes, bscales, gscale, rows // 4)
    assert np.array_equal(s4.cpu().numpy(), os4)
    assert np.array_equal(c4.cpu().numpy(), mx.pack_fp4(oc4))
