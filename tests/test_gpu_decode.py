"""GPU parity of the single-launch fused decode layer against the oracle, at
the tiny size and at the full MiniMax-shaped sizes (1 and 16 rows, and the
8-layer residual chain), plus the invariants the kernel promises: output rows
independent of the batch they are in and of row order, bit-identical repeats."""

import sys

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe, mx
from tests import helpers

pytestmark = pytest.mark.gpu

_CACHE = {}


def _layers(name, layer=0):
    key = (name, layer)
    if key not in _CACHE:
        cfg = synth.workload(name)
        _CACHE[key] = (cfg, helpers.gpu_layer(cfg, layer), helpers.oracle_layer(cfg, layer))
    return _CACHE[key]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(gl, x_bits, residual_bits=None, ws=None):
    print(f"[decode] T={x_bits.shape[0]} H={x_bits.shape[1]}", flush=True)
    res = _dev(residual_bits) if residual_bits is not None else None
    y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(x_bits), residual=res, workspace=ws, return_routing=True)
    torch.cuda.synchronize()
    return _host(y), ids.cpu().numpy(), w.cpu().numpy()


def _compare(cfg, gl, ol, x_bits, y, ids, w, residual_bits=None, layer=0, ulp_frac=None):
    """Oracle comparison with the near-tie rule for routing."""
    ref = moe.moe_layer(x_bits, ol, residual_bits)
    if not np.array_equal(ids, ref["ids"]):
        ids_r, _, logits = binding.moe_router_topk(gl, _dev(x_bits), want_logits=True)
        logits = logits.cpu().numpy()
        bound = helpers.logit_bound(x_bits, synth.router_weights(cfg, layer), ref["logits"])
        helpers.check_logits(logits, ref["logits"], bound)
        helpers.check_topk(ids, logits, ref["logits"], bound, cfg["k"])
        ref = moe.moe_layer(x_bits, ol, residual_bits, ids=ids)
    np.testing.assert_allclose(w, ref["weights"], rtol=1e-5, atol=1e-6)
    err, within = helpers.check_layer_output(y, ref, ulp_frac=ulp_frac)
    print(f"[decode] {cfg['name']} T={x_bits.shape[0]}: max row err {err:.3e}, within 1 ulp {within:.4f}", flush=True)
    return ref


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode16"])
def test_decode_matches_oracle(name):
    cfg, gl, ol = _layers(name)
    x = synth.activations(cfg)
    y, ids, w = _run(gl, x)
    _compare(cfg, gl, ol, x, y, ids, w)


@pytest.mark.timeout(900)
def test_decode_routed_experts_alone_match_to_one_ulp():
    """Without the shared expert every MXFP4 partial sum is exact in fp32, so
    the GPU and the oracle differ only in the final bf16 rounding."""
    cfg, gl, ol = _layers("decode16")
    gl2 = binding.MoELayer(gl.hidden, gl.inter, gl.num_experts, gl.top_k, 0, gl.router_w, gl.router_bias,
                           gl.w13, gl.w13_scale, gl.w2, gl.w2_scale)
    ol2 = moe.Layer(ol.H, ol.I, ol.E, ol.k, 0, ol.router_w, ol.router_bias, ol.w13_codes, ol.w13_scales,
                    ol.w2_codes, ol.w2_scales)
    x = synth.activations(cfg)
    y, ids, w = _run(gl2, x)
    _compare(dict(cfg, I_s=0), gl2, ol2, x, y, ids, w, ulp_frac=0.999)


@pytest.mark.timeout(900)
def test_decode_chain_of_eight_layers_with_residual():
    cfg = synth.workload("chain8")
    x = synth.activations(cfg)
    ws = None
    for layer in range(cfg["layers"]):
        gl = helpers.gpu_layer(cfg, layer)
        ol = helpers.oracle_layer(cfg, layer)
        if ws is None:
            ws = binding.decode_workspace(gl)
        y, ids, w = _run(gl, x, residual_bits=x, ws=ws)
        _compare(cfg, gl, ol, x, y, ids, w, residual_bits=x, layer=layer)
        x = y  # the next layer reads this layer's output
        del gl
    assert binding.moe_decode_status(ws) == 0


def test_rows_independent_of_batch_and_order():
    cfg, gl, ol = _layers("decode16")
    x = synth.activations(cfg)
    ws = binding.decode_workspace(gl)
    y16, ids16, w16 = _run(gl, x, ws=ws)
    # same call again: bit-identical
    y16b, _, _ = _run(gl, x, ws=ws)
    assert np.array_equal(y16, y16b)
    # every row alone, and every prefix batch size, gives the same bits
    for t in range(16):
        y1, ids1, w1 = _run(gl, x[t:t + 1], ws=ws)
        assert np.array_equal(y1[0], y16[t]), t
        assert np.array_equal(ids1[0], ids16[t]) and np.array_equal(w1[0], w16[t])
    for T in (2, 3, 5, 8, 13):
        yT, _, _ = _run(gl, x[:T], ws=ws)
        assert np.array_equal(yT, y16[:T]), T
    perm = np.random.default_rng(0).permutation(16)
    yp, _, _ = _run(gl, x[perm], ws=ws)
    assert np.array_equal(yp, y16[perm])
    assert binding.moe_decode_status(ws) == 0


def test_decode_routing_matches_standalone_router():
    cfg, gl, ol = _layers("decode16")
    x = synth.activations(cfg)
    _, ids, w = _run(gl, x)
    ids_r, w_r = binding.moe_router_topk(gl, _dev(x))
    assert np.array_equal(ids, ids_r.cpu().numpy())
    assert np.array_equal(w, w_r.cpu().numpy())


def test_decode_rejects_more_than_16_rows():
    cfg, gl, ol = _layers("tiny")
    x = _dev(synth.activations(cfg, T=17))
    with pytest.raises(binding.MoeError) as ei:
        binding.fused_moe_mxfp4_decode(gl, x)
    assert ei.value.status == -2


@pytest.mark.timeout(900)
def test_decode_sixteen_rows_on_four_experts():
    """A router bias that sends all 16 rows to the same 4 experts: every
    workgroup's gate/up units then read all 16 rows of x, so the MXFP4 copy of
    x it makes once routing is known spans several batches.  Checked against
    the oracle and bit for bit against the grouped path."""
    cfg, gl, ol = _layers("decode16")
    hot = [3, 40, 77, 120]
    bias = np.zeros(cfg["E"], np.float32)
    bias[hot] = 64.0
    gl2 = binding.MoELayer(gl.hidden, gl.inter, gl.num_experts, gl.top_k, gl.shared_inter, gl.router_w,
                           torch.from_numpy(bias).cuda(), gl.w13, gl.w13_scale, gl.w2, gl.w2_scale,
                           gl.ws13, gl.ws13_scale, gl.ws2, gl.ws2_scale)
    ol2 = moe.Layer(ol.H, ol.I, ol.E, ol.k, ol.I_s, ol.router_w, bias, ol.w13_codes, ol.w13_scales,
                    ol.w2_codes, ol.w2_scales, ol.ws13_codes, ol.ws13_scales, ol.ws2_codes, ol.ws2_scales)
    x = synth.activations(cfg)
    y, ids, w = _run(gl2, x)
    assert all(sorted(r) == hot for r in ids.tolist())
    _compare(cfg, gl2, ol2, x, y, ids, w)
    yg = binding.fused_moe_mxfp4_grouped(gl2, _dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(_host(yg), y)
