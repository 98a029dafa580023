"""The pre-router RMSNorm fused into the layer call: the input is the
residual stream h, the MoE runs on RMSNorm(h) (fp32, straight into the router
and the MX quantizers) and h is added back.  Against the oracle's normed layer
on the fused decode and grouped paths (MXFP8 and folded shared experts), bit
for bit between the two paths, and bit for bit across batch sizes."""

import copy

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe
from tests import helpers

pytestmark = pytest.mark.gpu

_CACHE = {}


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _normed(name, fold=False):
    key = (name, fold)
    if key not in _CACHE:
        cfg = synth.workload(name)
        gl = helpers.gpu_layer(cfg)
        ol = helpers.oracle_layer(cfg)
        if fold:
            H, I = cfg["H"], cfg["I"]
            c13, s13 = binding.mx_requant_fp8_to_fp4(gl.ws13, gl.ws13_scale, 2 * I, H)
            c2, s2 = binding.mx_requant_fp8_to_fp4(gl.ws2, gl.ws2_scale, H, I)
            gl = gl.folded_from(c13, s13, c2, s2)
            ol = moe.fold_shared_expert(ol)
        g = synth.norm_weight(cfg)
        gn = gl.with_norm(torch.from_numpy(g).cuda(), 1e-6)
        on = copy.copy(ol)
        on.norm_weight, on.norm_eps = g.astype(np.float64), 1e-6
        torch.cuda.synchronize()
        _CACHE[key] = (cfg, gn, on)
    return _CACHE[key]


@pytest.mark.parametrize("name,T,fold", [("decode1", 1, False), ("decode16", 16, False), ("tp4", 16, False),
                                         ("odd", 16, False), ("decode16", 16, True)])
def test_normed_decode_matches_oracle(name, T, fold):
    cfg, gl, ol = _normed(name, fold)
    x = synth.activations(cfg, T=T, index=90 + T)
    print(f"[norm] {name} decode T={T} folded={fold}", flush=True)
    y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(x), return_routing=True)
    torch.cuda.synchronize()
    y, ids, w = _host(y), ids.cpu().numpy(), w.cpu().numpy()
    helpers.compare_with_oracle(dict(cfg, I_s=0 if fold else cfg["I_s"]), gl, ol, x, y, ids, w,
                                label=f"normed decode{' folded' if fold else ''}")


@pytest.mark.parametrize("name,T,fold", [("tp4", 200, False), ("decode16", 37, True)])
def test_normed_grouped_matches_oracle_and_decode(name, T, fold):
    cfg, gl, ol = _normed(name, fold)
    x = synth.activations(cfg, T=T, index=95 + T)
    print(f"[norm] {name} grouped T={T} folded={fold}", flush=True)
    y = binding.fused_moe_mxfp4_grouped(gl, _dev(x))
    torch.cuda.synchronize()
    y = _host(y)
    helpers.compare_with_oracle(dict(cfg, I_s=0 if fold else cfg["I_s"]), gl, ol, x, y,
                                label=f"normed grouped{' folded' if fold else ''}")
    ws = binding.decode_workspace(gl)
    for t0 in range(0, T, 16):
        yd = binding.fused_moe_mxfp4_decode(gl, _dev(x[t0:t0 + 16]), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(_host(yd), y[t0:t0 + 16]), t0


def test_normed_layer_rejects_a_separate_residual():
    cfg, gl, _ = _normed("decode1")
    x = _dev(synth.activations(cfg))
    with pytest.raises(binding.MoeError) as ei:
        binding.fused_moe_mxfp4_decode(gl, x, residual=x.clone())
    assert ei.value.status == -1


@pytest.mark.parametrize("fold", [False, True])
def test_normed_decode_rows_independent_of_batch(fold):
    """Above four rows the fused launch hands the phase-B and phase-C units
    out by weight (the workgroups that normalize and quantize every row in
    phase A take fewer); each row's result must not depend on that."""
    cfg, gl, ol = _normed("decode16", fold)
    x = synth.activations(cfg, T=16, index=7)
    ws = binding.decode_workspace(gl)
    print(f"[norm] decode16 batches folded={fold}", flush=True)
    y16 = _host(binding.fused_moe_mxfp4_decode(gl, _dev(x), workspace=ws))
    torch.cuda.synchronize()
    for T in (1, 4, 5, 8, 12):
        yT = _host(binding.fused_moe_mxfp4_decode(gl, _dev(x[:T]), workspace=ws))
        torch.cuda.synchronize()
        assert np.array_equal(yT, y16[:T]), T
    assert binding.moe_decode_status(ws) == 0
