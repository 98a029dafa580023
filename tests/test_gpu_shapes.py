"""GPU parity at layer shapes other than the MiniMax one, which run the
generic (run-time shape) instance of the fused decode kernel with a shared
expert, and the grouped path:

* ``tp4``: the per-GPU share under 4-way tensor parallelism over the
  intermediate dimension (H 3072, 128 experts top-4, I = I_s = 256), the shape
  one GPU shows of the sharded layer;
* ``wide``: 256 experts top-8 (I = I_s = 256);
* ``odd``: H 1280, 16 experts top-3, I 384, I_s 640, whose K-tile counts
  10 / 3 / 5 split the dot products into 2 / 1 / 1 chunks and leave the scale
  groups part-filled;
* ``h640``: H 640, 16 experts top-2, I 256, I_s 384: H is not a multiple of
  256, so the grouped routed down runs its 128-column tiles (256 otherwise);
* ``h384``: H 384, 16 experts top-2, I = I_s = 512: the same, with the down
  products' K a multiple of 512 (the scale-group loop).

Each against the oracle (decode at 16 rows, grouped at more rows), and decode
and grouped bit for bit against each other."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
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


@pytest.mark.parametrize("name", ["tp4", "wide", "odd", "h640", "h384"])
def test_shape_decode_matches_oracle_and_grouped(name):
    cfg, gl, ol = _layers(name)
    x = synth.activations(cfg)
    r = synth.activations(cfg, index=1)
    print(f"[shapes] {name} decode T={cfg['T']} H={cfg['H']} I={cfg['I']} I_s={cfg['I_s']} "
          f"E={cfg['E']} k={cfg['k']}", flush=True)
    y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(x), residual=_dev(r), return_routing=True)
    torch.cuda.synchronize()
    y, ids, w = _host(y), ids.cpu().numpy(), w.cpu().numpy()
    helpers.compare_with_oracle(cfg, gl, ol, x, y, ids, w, residual_bits=r, label="decode")
    yg = binding.fused_moe_mxfp4_grouped(gl, _dev(x), residual=_dev(r))
    torch.cuda.synchronize()
    assert np.array_equal(_host(yg), y)


@pytest.mark.parametrize("name,T", [("tp4", 200), ("odd", 300), ("h640", 300), ("odd", 700), ("h384", 300)])
def test_shape_grouped_matches_oracle(name, T):
    """Enough rows that expert segments span several 128-row blocks (odd: 16
    experts top-3, about 56 slots each at 300 rows; tp4: about 6 per expert).
    At 700 rows the odd shape averages more than one 128-row block per
    expert, so its routed gate/up takes the 256-column tiles, with K-tile
    counts that are not whole scale groups."""
    cfg, gl, ol = _layers(name)
    x = synth.activations(cfg, T=T, index=T)
    print(f"[shapes] {name} grouped T={T}", flush=True)
    y = binding.fused_moe_mxfp4_grouped(gl, _dev(x))
    torch.cuda.synchronize()
    y = _host(y)
    helpers.compare_with_oracle(cfg, gl, ol, x, y, label="grouped")
    # and bit for bit against the fused kernel in 16-row batches
    ws = binding.decode_workspace(gl)
    for t0 in range(0, T, 16):
        yd = binding.fused_moe_mxfp4_decode(gl, _dev(x[t0:t0 + 16]), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(_host(yd), y[t0:t0 + 16]), t0
