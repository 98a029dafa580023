"""Wide fused steps (17..64 rows in one launch): the instance that runs every
unit's rows in 16-row groups on the same weight tiles.  Against the oracle;
every output row bit-identical to the 16-row instance on the same row (the
per-row arithmetic is the same); bit-identical to the grouped path; skewed
routing that puts 64 rows on one expert's units; the folded shared expert,
the fused norm, the run-time shape instance; and the dispatch rule."""

import copy

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe
from tests import helpers

pytestmark = pytest.mark.gpu

_CACHE = {}


def _layers(name):
    if name not in _CACHE:
        cfg = synth.workload(name)
        _CACHE[name] = (cfg, helpers.gpu_layer(cfg), helpers.oracle_layer(cfg))
    return _CACHE[name]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _decode(gl, x, residual=None, ws=None):
    print(f"[wide] T={x.shape[0]} H={x.shape[1]} E={gl.num_experts}", flush=True)
    y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(x), residual=None if residual is None else _dev(residual),
                                               workspace=ws, return_routing=True)
    torch.cuda.synchronize()
    return _host(y), ids.cpu().numpy(), w.cpu().numpy()


def _narrow(gl, x, residual=None):
    """The 16-row instance over the rows in batches of 16."""
    ws = binding.decode_workspace(gl, max_rows=16)
    out = []
    for t0 in range(0, x.shape[0], 16):
        out.append(_decode(gl, x[t0:t0 + 16], None if residual is None else residual[t0:t0 + 16], ws))
    return tuple(np.concatenate([o[i] for o in out]) for i in range(3))


@pytest.mark.parametrize("T", [17, 64])
def test_wide_decode_matches_oracle_and_narrow(T):
    cfg, gl, ol = _layers("decode16")
    x = synth.activations(cfg, T=T, index=200 + T)
    r = synth.activations(cfg, T=T, index=300 + T)
    y, ids, w = _decode(gl, x, r)
    yn, idsn, wn = _narrow(gl, x, r)
    assert np.array_equal(ids, idsn) and np.array_equal(w, wn)
    assert np.array_equal(y, yn)
    helpers.compare_with_oracle(cfg, gl, ol, x, y, ids, w, residual_bits=r, label="wide")


def test_wide_decode_every_size_equals_narrow_and_grouped():
    cfg, gl, _ = _layers("decode16")
    x = synth.activations(cfg, T=64, index=400)
    ws = binding.decode_workspace(gl)
    y64, _, _ = _decode(gl, x, ws=ws)
    assert np.array_equal(y64, _narrow(gl, x)[0])
    for T in (18, 31, 33, 48, 63):
        yT, _, _ = _decode(gl, x[:T], ws=ws)
        assert np.array_equal(yT, y64[:T]), T
    yg = binding.fused_moe_mxfp4_grouped(gl, _dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(_host(yg), y64)
    assert binding.moe_decode_status(ws) == 0


@pytest.mark.timeout(900)
def test_wide_decode_sixty_four_rows_on_four_experts():
    """A router bias sending all 64 rows to the same 4 experts: every gate/up
    and down unit of those experts runs four 16-row groups."""
    cfg, gl, ol = _layers("decode16")
    hot = [5, 33, 90, 127]
    bias = np.zeros(cfg["E"], np.float32)
    bias[hot] = 64.0
    gl2 = binding.MoELayer(gl.hidden, gl.inter, gl.num_experts, gl.top_k, gl.shared_inter, gl.router_w,
                           torch.from_numpy(bias).cuda(), gl.w13, gl.w13_scale, gl.w2, gl.w2_scale,
                           gl.ws13, gl.ws13_scale, gl.ws2, gl.ws2_scale)
    ol2 = moe.Layer(ol.H, ol.I, ol.E, ol.k, ol.I_s, ol.router_w, bias, ol.w13_codes, ol.w13_scales,
                    ol.w2_codes, ol.w2_scales, ol.ws13_codes, ol.ws13_scales, ol.ws2_codes, ol.ws2_scales)
    x = synth.activations(cfg, T=64, index=500)
    y, ids, w = _decode(gl2, x)
    assert all(sorted(r) == hot for r in ids.tolist())
    assert np.array_equal(y, _narrow(gl2, x)[0])
    helpers.compare_with_oracle(cfg, gl2, ol2, x, y, ids, w, label="wide skewed")


def test_wide_decode_folded_and_normed():
    cfg, gl, ol = _layers("decode16")
    H, I = cfg["H"], cfg["I"]
    c13, s13 = binding.mx_requant_fp8_to_fp4(gl.ws13, gl.ws13_scale, 2 * I, H)
    c2, s2 = binding.mx_requant_fp8_to_fp4(gl.ws2, gl.ws2_scale, H, I)
    g = synth.norm_weight(cfg)
    gf = gl.folded_from(c13, s13, c2, s2).with_norm(torch.from_numpy(g).cuda())
    of = copy.copy(moe.fold_shared_expert(ol))
    of.norm_weight, of.norm_eps = g.astype(np.float64), 1e-6
    x = synth.activations(cfg, T=40, index=600)
    y, ids, w = _decode(gf, x)
    assert np.array_equal(y, _narrow(gf, x)[0])
    helpers.compare_with_oracle(dict(cfg, I_s=0), gf, of, x, y, ids, w, label="wide folded normed")


@pytest.mark.parametrize("name,T", [("tp4", 64), ("odd", 50)])
def test_wide_decode_runtime_shape(name, T):
    cfg, gl, ol = _layers(name)
    x = synth.activations(cfg, T=T, index=700 + T)
    y, ids, w = _decode(gl, x)
    assert np.array_equal(y, _narrow(gl, x)[0])
    helpers.compare_with_oracle(cfg, gl, ol, x, y, ids, w, label="wide")


def test_dispatch_with_wide_fused_steps():
    cfg, gl, _ = _layers("decode16")
    fwd = binding.MoEForward(gl, fused_max_rows=64)
    x40 = synth.activations(cfg, T=40, index=800)
    x65 = synth.activations(cfg, T=65, index=801)
    y40 = fwd(_dev(x40))
    assert fwd.last_path == "decode"
    y65 = fwd(_dev(x65))
    assert fwd.last_path == "grouped"
    torch.cuda.synchronize()
    assert np.array_equal(_host(y40), _narrow(gl, x40)[0])
    g65 = binding.fused_moe_mxfp4_grouped(gl, _dev(x65))
    torch.cuda.synchronize()
    assert np.array_equal(_host(y65), _host(g65))
