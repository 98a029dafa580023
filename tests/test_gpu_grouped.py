"""GPU parity of the grouped (any number of rows) MoE path.

* against the oracle at the tiny size, with enough rows that expert segments
  span several 128-row blocks and end ragged;
* against the fused decode kernel, bit for bit, at the full MiniMax-shaped
  sizes for 1..16 rows (both paths promise the same arithmetic), with and
  without the residual;
* at the 8192-row prefill size: sampled rows against the oracle, and against
  the decode kernel run on those rows alone (bit for bit).
"""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe
from tests import helpers

pytestmark = pytest.mark.gpu

_CACHE = {}


def _layers(name, layer=0, oracle=True):
    key = (name, layer)
    if key not in _CACHE:
        cfg = synth.workload(name)
        _CACHE[key] = (cfg, helpers.gpu_layer(cfg, layer), helpers.oracle_layer(cfg, layer) if oracle else None)
    return _CACHE[key]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _grouped(gl, x_bits, residual_bits=None):
    print(f"[grouped] T={x_bits.shape[0]} H={x_bits.shape[1]} E={gl.num_experts}", flush=True)
    res = _dev(residual_bits) if residual_bits is not None else None
    y = binding.fused_moe_mxfp4_grouped(gl, _dev(x_bits), residual=res)
    torch.cuda.synchronize()
    return _host(y)


def _decode(gl, x_bits, residual_bits=None, ws=None):
    """Decode kernel over the rows in batches of at most 16."""
    out = []
    for t0 in range(0, x_bits.shape[0], 16):
        xb = x_bits[t0:t0 + 16]
        res = _dev(residual_bits[t0:t0 + 16]) if residual_bits is not None else None
        y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(xb), residual=res, workspace=ws, return_routing=True)
        torch.cuda.synchronize()
        out.append((_host(y), ids.cpu().numpy(), w.cpu().numpy()))
    return (np.concatenate([o[0] for o in out]), np.concatenate([o[1] for o in out]),
            np.concatenate([o[2] for o in out]))


def _oracle_compare(cfg, gl, ol, x_bits, y, residual_bits=None, layer=0):
    """Oracle comparison; rows whose routing is a near tie are recomputed with
    the GPU router's (valid) choice."""
    ref = moe.moe_layer(x_bits, ol, residual_bits)
    ids_g, _, logits = binding.moe_router_topk(gl, _dev(x_bits), want_logits=True)
    ids_g = ids_g.cpu().numpy()
    if not np.array_equal(ids_g, ref["ids"]):
        logits = logits.cpu().numpy()
        bound = helpers.logit_bound(x_bits, synth.router_weights(cfg, layer), ref["logits"])
        helpers.check_logits(logits, ref["logits"], bound)
        helpers.check_topk(ids_g, logits, ref["logits"], bound, cfg["k"])
        ref = moe.moe_layer(x_bits, ol, residual_bits, ids=ids_g)
    err, within = helpers.check_layer_output(y, ref)
    print(f"[grouped] {cfg['name']} T={x_bits.shape[0]}: max row err {err:.3e}, within 1 ulp {within:.4f}",
          flush=True)


@pytest.mark.parametrize("T", [1, 4, 37, 1000])
def test_grouped_matches_oracle_tiny(T):
    """tiny: 8 experts top-2; at T=1000 every expert gets about 250 slots,
    i.e. two full 128-row blocks and a ragged third."""
    cfg, gl, ol = _layers("tiny")
    x = synth.activations(cfg, T=T, index=T)
    y = _grouped(gl, x)
    _oracle_compare(cfg, gl, ol, x, y)


def test_grouped_matches_oracle_tiny_with_residual():
    cfg, gl, ol = _layers("tiny")
    x = synth.activations(cfg, T=300, index=1)
    r = synth.activations(cfg, T=300, index=2)
    y = _grouped(gl, x, residual_bits=r)
    _oracle_compare(cfg, gl, ol, x, y, residual_bits=r)


@pytest.mark.parametrize("T", [1, 5, 16])
def test_grouped_equals_decode_bitwise(T):
    cfg, gl, _ = _layers("decode16", oracle=False)
    x = synth.activations(cfg, T=T, index=100 + T)
    yd, _, _ = _decode(gl, x)
    yg = _grouped(gl, x)
    assert np.array_equal(yg, yd)


def test_grouped_equals_decode_ragged_with_residual():
    """37 rows (two full decode batches and a ragged one) with a residual."""
    cfg, gl, _ = _layers("decode1", oracle=False)
    x = synth.activations(cfg, T=37, index=7)
    r = synth.activations(cfg, T=37, index=8)
    yd, _, _ = _decode(gl, x, residual_bits=r)
    yg = _grouped(gl, x, residual_bits=r)
    assert np.array_equal(yg, yd)


@pytest.mark.timeout(1200)
def test_grouped_prefill_8192_sampled_rows():
    """Full prefill size: 8192 rows, about 256 slots per expert.  Sampled
    rows (first, last, and spread ones) against the oracle and against the
    decode kernel run on those rows alone."""
    cfg, gl, ol = _layers("prefill")
    x = synth.activations(cfg)
    assert x.shape == (8192, 3072)
    y = _grouped(gl, x)
    rows = np.array([0, 1, 2047, 4444, 8190, 8191])
    yd, _, _ = _decode(gl, x[rows])
    assert np.array_equal(y[rows], yd)
    _oracle_compare(cfg, gl, ol, x[rows], y[rows])
    # every row is finite bf16 (no NaN/Inf pattern: exponent field not all ones)
    assert not np.any((y & 0x7f80) == 0x7f80)
