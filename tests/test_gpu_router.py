"""GPU parity of router + top-k and of the token sort against the oracle."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from oracle import moe, mx
from tests import helpers

pytestmark = pytest.mark.gpu


def _x_dev(x):
    return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)


def _router_only_layer(cfg):
    """A layer whose expert weights are tiny placeholders: the router call
    reads only router_w / router_bias."""
    H, E = cfg["H"], cfg["E"]
    wr = torch.from_numpy(synth.router_weights(cfg)).cuda()
    b = synth.router_bias(cfg)
    bias = torch.from_numpy(b).cuda() if b is not None else None
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    return binding.MoELayer(H, cfg["I"], E, cfg["k"], 0, wr, bias, dummy, dummy, dummy, dummy)


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode1", 1), ("decode16", 16), ("chain8", 4),
                                    ("decode16", 37), ("prefill", 8192)])
def test_router_topk_matches_oracle(name, T):
    cfg = synth.workload(name)
    layer = _router_only_layer(cfg)
    x = synth.activations(cfg, T=T)
    ids, w, logits = binding.moe_router_topk(layer, _x_dev(x), want_logits=True)
    torch.cuda.synchronize()
    ids, w, logits = ids.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    wr = synth.router_weights(cfg)
    l_ref = moe.router_logits(mx.bf16_bits_to_f64(x), wr, synth.router_bias(cfg))
    bound = helpers.logit_bound(x, wr, l_ref)
    helpers.check_logits(logits, l_ref, bound)
    exact = helpers.check_topk(ids, logits, l_ref, bound, cfg["k"])
    assert exact >= int(0.99 * T)
    # weights: softmax over the chosen logits, from the GPU's own logits
    for t in range(T):
        z = logits[t, ids[t]].astype(np.float64)
        p = np.exp(z - z[0])
        np.testing.assert_allclose(w[t], p / p.sum(), rtol=2e-6, atol=1e-7)
        assert abs(w[t].astype(np.float64).sum() - 1.0) < 4 * 2.0 ** -23


def test_router_ties_go_to_lower_expert():
    """All router rows equal -> every logit ties -> experts 0..k-1, equal weights."""
    cfg = synth.workload("tiny")
    H, E, k = cfg["H"], cfg["E"], cfg["k"]
    wr = torch.full((E, H), 0.01, dtype=torch.float32, device="cuda")
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    layer = binding.MoELayer(H, cfg["I"], E, k, 0, wr, None, dummy, dummy, dummy, dummy)
    x = synth.activations(cfg, T=5)
    ids, w = binding.moe_router_topk(layer, _x_dev(x))
    assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(k), (5, 1)))
    assert np.all(w.cpu().numpy() == np.float32(1.0 / k))


@pytest.mark.parametrize("T,k,E,block_m,skew", [(1, 4, 128, 1, 0), (4, 2, 8, 1, 0), (16, 4, 128, 1, 0),
                                                 (16, 4, 128, 16, 1), (37, 4, 12, 4, 0), (8192, 4, 128, 64, 0),
                                                 (8192, 4, 128, 128, 1), (300, 8, 256, 32, 0), (2000, 1, 3, 64, 1)])
def test_align_sort_matches_oracle(T, k, E, block_m, skew):
    rng = np.random.default_rng(T * 7 + k)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
        ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)])
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    ids = ids.astype(np.int32)
    slots, bexp, offs, npad = binding.moe_align_sort(torch.from_numpy(ids).cuda(), E, block_m)
    torch.cuda.synchronize()
    r_slots, r_bexp, r_offs, r_npad = moe.align_sort(ids, E, block_m)
    npad_g = int(npad.cpu().numpy()[0])
    assert npad_g == r_npad
    s = slots.cpu().numpy()
    assert np.array_equal(s[:r_npad], r_slots)
    assert np.all(s[r_npad:] == T * k)
    b = bexp.cpu().numpy()
    assert np.array_equal(b[:len(r_bexp)], r_bexp)
    assert np.all(b[len(r_bexp):] == -1)
    assert np.array_equal(offs.cpu().numpy(), r_offs)


def test_align_sort_all_to_one_expert():
    T, k, E = 3000, 1, 16
    ids = np.full((T, k), 5, np.int32)
    slots, bexp, offs, npad = binding.moe_align_sort(torch.from_numpy(ids).cuda(), E, 64)
    r_slots, r_bexp, r_offs, r_npad = moe.align_sort(ids, E, 64)
    assert int(npad.cpu()[0]) == r_npad
    assert np.array_equal(slots.cpu().numpy()[:r_npad], r_slots)
    assert np.array_equal(offs.cpu().numpy(), r_offs)


@pytest.mark.parametrize("H,E,k,T,with_bias", [(384, 40, 3, 77, True), (3072, 128, 4, 300, False),
                                                 (3072, 128, 4, 5, True)])
def test_router_tiled_equals_rowwise(H, E, k, T, with_bias):
    """A call that returns the logits takes the register-tiled kernel (16-row x
    32-expert workgroup tiles; here with a partial 256-wide stride, a partial
    row tile and a partial expert tile), one without takes the per-row kernel.
    Both follow the documented order, so the routing ids and weights must
    agree bit for bit, and the tiled logits lie within the fp32 bound of the
    oracle's."""
    rng = np.random.default_rng(1000 * H + E + T)
    wr_np = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    b_np = rng.standard_normal(E).astype(np.float32) if with_bias else None
    wr = torch.from_numpy(wr_np).cuda()
    bias = torch.from_numpy(b_np).cuda() if with_bias else None
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    layer = binding.MoELayer(H, 128, E, k, 0, wr, bias, dummy, dummy, dummy, dummy)
    xf = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
    x_bits = xf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xd = _x_dev(x_bits)
    ids_t, w_t, l_t = binding.moe_router_topk(layer, xd, want_logits=True)
    ids_r, w_r = binding.moe_router_topk(layer, xd, want_logits=False)
    torch.cuda.synchronize()
    ids_r, w_r = ids_r.cpu().numpy(), w_r.cpu().numpy()
    l_t, ids_t, w_t = l_t.cpu().numpy(), ids_t.cpu().numpy(), w_t.cpu().numpy()
    assert np.array_equal(ids_t, ids_r)
    assert np.array_equal(w_t.view(np.uint32), w_r.view(np.uint32))
    l_ref = moe.router_logits(mx.bf16_bits_to_f64(x_bits), wr_np, b_np)
    helpers.check_logits(l_t, l_ref, helpers.logit_bound(x_bits, wr_np, l_ref))
