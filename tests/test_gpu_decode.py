"""GPU parity of the single-launch fused decode layer against the oracle, at
the tiny size and at the full MiniMax-shaped sizes (1 and 16 rows, and the
8-layer residual chain, eager and replayed from a captured HIP graph), plus
the invariants the kernel promises: output rows independent of the batch they
are in and of row order, bit-identical repeats, a call counter that wraps
safely, a poisoned workspace after a timed-out wait, and the 16-row dispatch
rule between the fused and the grouped path."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe
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
    print(f"[decode] T={x_bits.shape[0]} H={x_bits.shape[1]} E={gl.num_experts}", flush=True)
    res = _dev(residual_bits) if residual_bits is not None else None
    y, ids, w = binding.fused_moe_mxfp4_decode(gl, _dev(x_bits), residual=res, workspace=ws, return_routing=True)
    torch.cuda.synchronize()
    return _host(y), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode16"])
def test_decode_matches_oracle(name):
    cfg, gl, ol = _layers(name)
    x = synth.activations(cfg)
    y, ids, w = _run(gl, x)
    helpers.compare_with_oracle(cfg, gl, ol, x, y, ids, w)


@pytest.mark.timeout(900)
def test_decode_routed_experts_alone_match_to_one_ulp():
    """Without the shared expert the GPU and the oracle differ only by the
    fp32 rounding of the chunked sums and the final bf16 rounding: besides the
    element bound, 99.9% of elements are within one bf16 ulp."""
    cfg, gl, ol = _layers("decode16")
    gl2 = binding.MoELayer(gl.hidden, gl.inter, gl.num_experts, gl.top_k, 0, gl.router_w, gl.router_bias,
                           gl.w13, gl.w13_scale, gl.w2, gl.w2_scale)
    ol2 = moe.Layer(ol.H, ol.I, ol.E, ol.k, 0, ol.router_w, ol.router_bias, ol.w13_codes, ol.w13_scales,
                    ol.w2_codes, ol.w2_scales)
    x = synth.activations(cfg)
    y, ids, w = _run(gl2, x)
    ref = helpers.compare_with_oracle(dict(cfg, I_s=0), gl2, ol2, x, y, ids, w)
    helpers.check_layer_output(y, ref, ulp_frac=0.999)


@pytest.mark.timeout(900)
def test_decode_chain_of_eight_layers_with_residual_and_graph_replay():
    """The 8-layer chain (4 rows, Zipf-biased routers, residual add).  Each
    layer is checked against the oracle on the oracle's own chain input.  The
    GPU's own chain (each layer reading the previous GPU output) is then
    captured once into a HIP graph of 8 launches and replayed: every replay,
    with eager work and synchronizations in between, equals the eager chain
    bit for bit."""
    cfg = synth.workload("chain8")
    L = cfg["layers"]
    gls = [helpers.gpu_layer(cfg, layer) for layer in range(L)]
    ols = [helpers.oracle_layer(cfg, layer) for layer in range(L)]
    ws = binding.decode_workspace(gls[0])
    x = synth.activations(cfg)
    # per layer on the oracle's chain input
    xo = x
    for layer in range(L):
        y, ids, w = _run(gls[layer], xo, residual_bits=xo, ws=ws)
        ref = helpers.compare_with_oracle(cfg, gls[layer], ols[layer], xo, y, ids, w, residual_bits=xo,
                                          layer=layer, label=f"layer {layer}")
        xo = ref["y_bits"]
    # the GPU's own chain, eager
    bufs = [_dev(x)] + [torch.empty_like(_dev(x)) for _ in range(L)]
    for layer in range(L):
        binding.fused_moe_mxfp4_decode(gls[layer], bufs[layer], residual=bufs[layer], out=bufs[layer + 1],
                                       workspace=ws)
    torch.cuda.synchronize()
    eager = [_host(b) for b in bufs[1:]]
    # captured once, replayed three times
    for b in bufs[1:]:
        b.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for layer in range(L):
            binding.fused_moe_mxfp4_decode(gls[layer], bufs[layer], residual=bufs[layer], out=bufs[layer + 1],
                                           workspace=ws)
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(0)
        # eager work between replays: a decode call on another layer's weights
        binding.fused_moe_mxfp4_decode(gls[rep], bufs[0], out=torch.empty_like(bufs[0]), workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[decode] graph replay {rep}", flush=True)
        for layer in range(L):
            assert np.array_equal(_host(bufs[layer + 1]), eager[layer]), (rep, layer)
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


def test_decode_rejects_more_than_64_rows():
    cfg, gl, ol = _layers("tiny")
    x = _dev(synth.activations(cfg, T=65))
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
    helpers.compare_with_oracle(cfg, gl2, ol2, x, y, ids, w)
    yg = binding.fused_moe_mxfp4_grouped(gl2, _dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(_host(yg), y)


# Workspace words (byte offsets of the sync block, one 256-byte line each).
_STATUS, _EPOCH = 0, 3 * 256
_TRACE_BYTES = 2048 * 16 * 8   # per-workgroup trace words after the four sync lines
_TAGGED_FROM = 4 * 256 + _TRACE_BYTES  # then the tagged words, to the end


def _word(ws, off):
    return int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0])


def _set_word(ws, off, value):
    ws[off:off + 4] = torch.from_numpy(np.array([value], np.uint32).view(np.uint8)).cuda()
    torch.cuda.synchronize()


def test_call_counter_wrap_clears_tagged_words():
    """A call whose tag is the last 32-bit value clears every tagged word and
    restarts the counter, so the next call (tag 1 again) cannot take words
    left by the earlier call that also had tag 1.  Forced from the host by
    setting the counter word."""
    cfg, gl, _ = _layers("decode16")
    xa, xb, xc = (synth.activations(cfg, index=i) for i in (11, 12, 13))
    ref_ws = binding.decode_workspace(gl)
    ref_b, _, _ = _run(gl, xb, ws=ref_ws)
    ref_c, _, _ = _run(gl, xc, ws=ref_ws)
    ws = binding.decode_workspace(gl)
    _run(gl, xa, ws=ws)                      # leaves words tagged 1
    assert _word(ws, _EPOCH) == 1
    _set_word(ws, _EPOCH, 0xFFFFFFFE)        # the next call's tag is 0xFFFFFFFF
    yb, _, _ = _run(gl, xb, ws=ws)
    assert np.array_equal(yb, ref_b)
    assert _word(ws, _EPOCH) == 0
    tagged = ws[_TAGGED_FROM:].cpu().numpy()
    assert not tagged.any(), "tagged words left after the wrap"
    yc, _, _ = _run(gl, xc, ws=ws)           # tag 1 again
    assert np.array_equal(yc, ref_c)
    assert _word(ws, _EPOCH) == 1
    assert binding.moe_decode_status(ws) == 0


def test_status_word_poisons_later_calls_until_reinitialized():
    """Once a wait has given up (forced here by setting the status word from
    the host, so no wait runs out), calls on that workspace write NaN and
    report the timeout; zero-filling the workspace restores normal calls."""
    cfg, gl, _ = _layers("decode16")
    x = synth.activations(cfg, index=21)
    ref, _, _ = _run(gl, x)
    ws = binding.decode_workspace(gl)
    _set_word(ws, _STATUS, 1)
    y, _, _ = _run(gl, x, ws=ws)
    assert np.all(y == 0x7FC0)
    assert binding.moe_decode_status(ws) == -5
    binding.load().moe_workspace_init(binding._ptr(ws), ws.numel(), binding._stream())
    y2, _, _ = _run(gl, x, ws=ws)
    assert np.array_equal(y2, ref)
    assert binding.moe_decode_status(ws) == 0


def test_dispatch_sixteen_rows_fused_seventeen_grouped():
    """The layer call for any T with the pages' rule (fused_max_rows = 16): up
    to 16 rows one fused launch, wider steps the grouped path; each result
    equals the direct call of its path.  The default takes up to 64 rows
    fused."""
    cfg, gl, _ = _layers("decode16")
    assert binding.MoEForward(gl).fused_max_rows == binding.WIDE_MAX_ROWS
    fwd = binding.MoEForward(gl, fused_max_rows=16)
    x16 = synth.activations(cfg, T=16, index=31)
    x17 = synth.activations(cfg, T=17, index=32)
    y16 = fwd(_dev(x16))
    assert fwd.last_path == "decode"
    y17 = fwd(_dev(x17))
    assert fwd.last_path == "grouped"
    torch.cuda.synchronize()
    d16, _, _ = _run(gl, x16)
    g17 = binding.fused_moe_mxfp4_grouped(gl, _dev(x17))
    torch.cuda.synchronize()
    assert np.array_equal(_host(y16), d16)
    assert np.array_equal(_host(y17), _host(g17))
    # rows of the 17-row step equal the fused kernel on them (same arithmetic)
    d17a, _, _ = _run(gl, x17[:16])
    d17b, _, _ = _run(gl, x17[16:])
    assert np.array_equal(_host(y17), np.concatenate([d17a, d17b]))
