"""GPU parity of the grouped (any number of rows) MoE path.

* against the oracle at the tiny size, with enough rows that expert segments
  span several 128-row blocks and end ragged;
* against the fused decode kernel, bit for bit, at the full MiniMax-shaped
  sizes for 1..16 rows (both paths promise the same arithmetic), with and
  without the residual;
* at the 8192-row prefill size: every row bit for bit against the decode
  kernel, and the rows at 128-row block boundaries and segment tails of
  twelve experts against the oracle;
* at the TP4 per-GPU shape, with 256 experts top-8, and at a shape whose K
  splits into 2 / 1 / 1 chunks (test_gpu_shapes.py);
* the two-stream schedule of the plain call against the one-stream timed
  call, bit for bit, on a non-default stream, for back-to-back calls and
  from two host threads at once.
"""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe, mx
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


def _oracle_compare(cfg, gl, ol, x_bits, y, residual_bits=None, layer=0, label=""):
    helpers.compare_with_oracle(cfg, gl, ol, x_bits, y, residual_bits=residual_bits, layer=layer, label=label)


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


def _boundary_rows(ids, experts, block_m=128):
    """Rows whose slots sit at the first and last position of each 128-row
    block of the given experts' segments, and at each segment's ragged tail
    (the sorted order is by slot, i.e. by row, inside a segment)."""
    rows = set()
    T, k = ids.shape
    for e in experts:
        seg = (np.flatnonzero(ids.reshape(-1) == e) // k).tolist()
        n = len(seg)
        for p in range(0, n, block_m):
            rows.add(seg[p])
            rows.add(seg[min(p + block_m - 1, n - 1)])
        rows.add(seg[n - 1])
        if n >= 2:
            rows.add(seg[n - 2])
    return sorted(rows)


@pytest.mark.timeout(1200)
def test_grouped_prefill_8192_every_row():
    """Full prefill size: 8192 rows, about 256 slots per expert.  Every row
    equals the fused decode kernel run on it (512 calls of 16 rows, bit for
    bit: both promise the same arithmetic).  Rows at the first and last
    position of the 128-row blocks of twelve experts' segments and at their
    ragged tails are compared with the oracle."""
    cfg, gl, ol = _layers("prefill")
    x = synth.activations(cfg)
    assert x.shape == (8192, 3072)
    y = _grouped(gl, x)
    assert not np.any((y & 0x7f80) == 0x7f80)  # finite bf16 everywhere
    ws = binding.decode_workspace(gl)
    yd, _, _ = _decode(gl, x, ws=ws)
    mismatch = np.flatnonzero(np.any(y != yd, axis=1))
    assert mismatch.size == 0, f"{mismatch.size} rows differ from the decode kernel, first {mismatch[:8]}"
    logits = moe.router_logits(mx.bf16_bits_to_f64(x), ol.router_w, ol.router_bias)
    ids, _ = moe.select_topk(logits, cfg["k"])
    experts = [0, 11, 23, 37, 50, 63, 64, 77, 90, 101, 115, 127]
    rows = _boundary_rows(ids, experts)
    assert len(rows) >= 64, len(rows)
    print(f"[grouped] oracle on {len(rows)} boundary rows", flush=True)
    xr = x[rows]
    helpers.prefetch(ol, np.unique(ids[rows]))
    _oracle_compare(cfg, gl, ol, xr, y[rows], label="block boundaries")


def test_grouped_side_stream_matches_one_stream():
    """The plain call runs the quantization and the shared gate/up on the
    library's side stream; the timed call runs every step on the caller's
    stream.  Both give the same bits, from a non-default caller stream too,
    and back-to-back plain calls on one workspace (different inputs and row
    counts, no synchronization between them) each give their own result."""
    cfg, gl, _ = _layers("odd", oracle=False)
    ws = binding.grouped_workspace(gl, 700)
    xs = [_dev(synth.activations(cfg, T=T, index=j)) for j, T in enumerate((700, 37, 300))]
    ref = []
    for x in xs:
        print(f"[grouped] timed T={x.shape[0]}", flush=True)
        y, _ = binding.fused_moe_mxfp4_grouped_timed(gl, x, workspace=ws)
        torch.cuda.synchronize()
        ref.append(_host(y))
    s = torch.cuda.Stream()
    for rep in range(2):
        print(f"[grouped] back-to-back plain calls, pass {rep}", flush=True)
        with torch.cuda.stream(s):
            ys = [binding.fused_moe_mxfp4_grouped(gl, x, workspace=ws) for x in xs]
        s.synchronize()
        for y, r in zip(ys, ref):
            assert np.array_equal(_host(y), r)
    ys = [binding.fused_moe_mxfp4_grouped(gl, x, workspace=ws) for x in xs]
    torch.cuda.synchronize()
    for y, r in zip(ys, ref):
        assert np.array_equal(_host(y), r)


def test_grouped_two_host_threads():
    """Two host threads make plain grouped calls at the same time, each on its
    own stream, workspace and inputs; they share the device's side stream, and
    every result equals the one-stream timed call's."""
    import threading

    cfg, gl, _ = _layers("odd", oracle=False)
    xs = [_dev(synth.activations(cfg, T=T, index=10 + j)) for j, T in enumerate((300, 211))]
    wss = [binding.grouped_workspace(gl, x.shape[0]) for x in xs]
    ref = []
    for x, ws in zip(xs, wss):
        y, _ = binding.fused_moe_mxfp4_grouped_timed(gl, x, workspace=ws)
        torch.cuda.synchronize()
        ref.append(_host(y))
    outs = [[], []]
    errors = []

    def worker(j):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    outs[j].append(binding.fused_moe_mxfp4_grouped(gl, xs[j], workspace=wss[j]))
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    print("[grouped] two host threads, 4 calls each", flush=True)
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for j in range(2):
        assert len(outs[j]) == 4
        for y in outs[j]:
            assert np.array_equal(_host(y), ref[j])
