"""Pins of the oracle's layer: hand-worked closed forms, the k = E identity
with a dense softmax mixture, linearity, token-permutation equivariance, and
top-k / sort invariants checked against numpy and scipy routines."""

import math

import numpy as np
import pytest
import scipy.special

from oracle import moe, mx
from mxfp4_moe_decode_amd import synth


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _row(first, n):
    r = np.zeros(n, np.float32)
    r[0] = first
    return r


def _hand_layer(k, with_shared=False, I_s=32):
    """H = I = 32, E = 2.  Router: expert 0 weight +1 on x[0], expert 1 -1.
    Expert 0: gate rows [-1, 0, ..], up rows [4, 0, ..], down rows [0.5, 0, ..].
    Expert 1: gate rows [2, 0, ..],  up rows [1, 0, ..], down rows [1, 0, ..].
    Shared: gate rows [1.5, 0, ..], up rows [2, 0, ..], down rows [0.25, 0, ..]."""
    H = I = 32
    wr = np.stack([_row(1.0, H), _row(-1.0, H)])
    w13 = [np.stack([_row(-1.0, H)] * I + [_row(4.0, H)] * I),
           np.stack([_row(2.0, H)] * I + [_row(1.0, H)] * I)]
    w2 = [np.stack([_row(0.5, I)] * H), np.stack([_row(1.0, I)] * H)]
    kw = {}
    if with_shared:
        kw = dict(ws13=np.stack([_row(1.5, H)] * I_s + [_row(2.0, H)] * I_s),
                  ws2=np.stack([_row(0.25, I_s)] * H))
    return moe.quantize_layer(H, I, 2, k, I_s if with_shared else 0, wr, None, w13, w2, **kw)


def test_hand_worked_single_expert():
    # x = e_0 -> logits (1, -1) -> expert 0 with weight 1.
    # xq = 1 exactly (block max 1 -> X = 2^-2, 4 -> code 6).
    # g = -1, u = 4 -> a = silu(-1) * 4 = -1.0757657 -> X = 2^-2, -4.303 -> -4 -> aq = -1.
    # d[h] = aq_0 * 0.5 = -0.5.  (Gate and up swapped would give silu(4) * -1 -> -6 * 2^-1 -> d = -1.5.)
    layer = _hand_layer(k=1)
    x = _bf16([_row(1.0, 32)])
    out = moe.moe_layer(x, layer)
    assert out["ids"].tolist() == [[0]]
    assert out["weights"][0, 0] == 1.0
    assert np.all(out["y"] == -0.5)
    assert np.all(out["y_bits"] == _bf16([-0.5])[0])


def test_hand_worked_two_experts_softmax_weights():
    # expert 1: g = 2, u = 1 -> a = silu(2) = 1.7615942 -> X = 2^-2, 7.05 saturates to 6 -> aq = 1.5,
    # d = 1.5 * 1 = 1.5.  Weights: softmax of (1, -1).
    layer = _hand_layer(k=2)
    x = _bf16([_row(1.0, 32)])
    out = moe.moe_layer(x, layer)
    w0 = 1.0 / (1.0 + math.exp(-2.0))
    w1 = 1.0 - w0
    assert out["ids"].tolist() == [[0, 1]]
    np.testing.assert_allclose(out["weights"][0], [w0, w1], rtol=1e-14)
    np.testing.assert_allclose(out["y"], w0 * -0.5 + w1 * 1.5, rtol=1e-14)


def test_hand_worked_shared_expert_mxfp8_and_residual():
    # shared: x -> E4M3 exactly; g = 1.5, u = 2 -> a = silu(1.5) * 2 = 2.4527235;
    # X = 2^(1 - 8) = 2^-7, 313.95 -> nearest E4M3 in [256, 512) (step 32) is 320 -> aq = 2.5;
    # s[h] = 2.5 * 0.25 = 0.625.  Routed part as in the single-expert case (-0.5); residual 1.
    layer = _hand_layer(k=1, with_shared=True)
    x = _bf16([_row(1.0, 32)])
    r = _bf16([np.full(32, 1.0, np.float32)])
    out = moe.moe_layer(x, layer, residual_bits=r)
    assert np.all(out["s"] == 0.625)
    assert np.all(out["y"] == 1.0 - 0.5 + 0.625)


def test_all_ones_weights_closed_form():
    """Every weight 1.0 (stored as 4 * 2^-2): g = u = S = sum_h xq[h] for every
    row, so a is constant, aq = MX(a) is constant and d[h] = I * aq for every
    expert; the k weights sum to one, so y = I * aq."""
    H, I, E, k, T = 256, 128, 4, 2, 3
    rng = np.random.default_rng(0)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    ones13 = np.ones((2 * I, H), np.float32)
    ones2 = np.ones((H, I), np.float32)
    layer = moe.quantize_layer(H, I, E, k, 0, wr, None, [ones13] * E, [ones2] * E)
    assert np.all(mx.mx_dequantize(layer.w13_codes[0], layer.w13_scales[0], "fp4") == 1.0)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = moe.moe_layer(x, layer)
    xc, xs = mx.mx_quantize(mx.bf16_bits_to_f64(x), "fp4")
    S = mx.mx_dequantize(xc, xs, "fp4").sum(axis=1)
    S = S.astype(np.float32).astype(np.float64)
    a = (S / (1 + np.exp(-S)) * S).astype(np.float32).astype(np.float64)
    for t in range(T):
        ac, asc = mx.mx_quantize(np.full((1, I), a[t]), "fp4")
        aq = mx.mx_dequantize(ac, asc, "fp4")[0, 0]
        np.testing.assert_allclose(out["y"][t], I * aq, rtol=1e-14)


def _random_layer(H=256, I=128, E=8, k=2, I_s=0, seed=0):
    rng = np.random.default_rng(seed)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    w13 = [(rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32) for _ in range(E)]
    w2 = [(rng.standard_normal((H, I)) * 0.02).astype(np.float32) for _ in range(E)]
    kw = {}
    if I_s:
        kw = dict(ws13=(rng.standard_normal((2 * I_s, H)) * 0.02).astype(np.float32),
                  ws2=(rng.standard_normal((H, I_s)) * 0.02).astype(np.float32))
    return moe.quantize_layer(H, I, E, k, I_s, wr, None, w13, w2, **kw), rng


def test_k_equals_E_is_dense_softmax_mixture():
    layer, rng = _random_layer(E=4, k=4)
    x = synth.f32_to_bf16_bits(rng.standard_normal((5, 256)).astype(np.float32))
    out = moe.moe_layer(x, layer)
    xf = mx.bf16_bits_to_f64(x)
    logits = (xf @ layer.router_w.T).astype(np.float32).astype(np.float64)
    p = scipy.special.softmax(logits, axis=1)
    dense = np.zeros_like(xf)
    for e in range(4):
        d, _ = moe.mx_ffn(xf, layer.w13_codes[e], layer.w13_scales[e], layer.w2_codes[e], layer.w2_scales[e], "fp4")
        dense += p[:, e:e + 1] * d
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


def test_down_scale_doubling_doubles_routed_output():
    layer, rng = _random_layer()
    x = synth.f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    y1 = moe.moe_layer(x, layer)["y"]
    layer.w2_scales = [s + 1 for s in layer.w2_scales]
    y2 = moe.moe_layer(x, layer)["y"]
    assert np.array_equal(y2, 2 * y1)


def test_zero_routed_down_leaves_the_shared_expert():
    layer, rng = _random_layer(I_s=64)
    layer.w2_codes = [np.zeros_like(c) for c in layer.w2_codes]
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    out = moe.moe_layer(x, layer)
    s, _ = moe.mx_ffn(mx.bf16_bits_to_f64(x), layer.ws13_codes, layer.ws13_scales,
                      layer.ws2_codes, layer.ws2_scales, "fp8")
    assert np.array_equal(out["y"], s)
    assert np.any(s != 0)


def test_token_permutation_equivariance():
    layer, rng = _random_layer(I_s=64)
    x = synth.f32_to_bf16_bits(rng.standard_normal((6, 256)).astype(np.float32))
    perm = rng.permutation(6)
    a = moe.moe_layer(x, layer)
    b = moe.moe_layer(x[perm], layer)
    assert np.array_equal(a["y_bits"][perm], b["y_bits"])
    assert np.array_equal(a["ids"][perm], b["ids"])


def test_topk_invariants_with_ties():
    rng = np.random.default_rng(9)
    logits = rng.integers(-3, 4, (200, 7)).astype(np.float64)  # many exact ties
    ids, w = moe.select_topk(logits, 3)
    for t in range(200):
        sel = list(ids[t])
        rest = [e for e in range(7) if e not in sel]
        for a in sel:
            for f in rest:
                assert logits[t, a] > logits[t, f] or (logits[t, a] == logits[t, f] and a < f)
        for a, b in zip(sel, sel[1:]):
            assert logits[t, a] > logits[t, b] or (logits[t, a] == logits[t, b] and a < b)
        # order agrees with numpy's lexsort on (index, -logit)
        ref = np.lexsort((np.arange(7), -logits[t]))[:3]
        assert sel == list(ref)
        full = scipy.special.softmax(logits[t])
        np.testing.assert_allclose(w[t], full[sel] / full[sel].sum(), rtol=1e-14)
        assert abs(w[t].sum() - 1.0) < 1e-15 * 4


@pytest.mark.parametrize("block_m", [1, 4, 16])
def test_align_sort_matches_numpy_stable_argsort(block_m):
    rng = np.random.default_rng(block_m)
    T, k, E = 37, 4, 12
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    slots, bexp, offs, npad = moe.align_sort(ids, E, block_m)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)]))
    real = slots[slots != T * k]
    assert np.array_equal(real, order)
    assert npad == sum(-(-c // block_m) * block_m for c in counts)
    assert npad % block_m == 0 and len(bexp) == npad // block_m
    for b, e in enumerate(bexp):
        blk = slots[b * block_m:(b + 1) * block_m]
        assert all(s == T * k or flat[s] == e for s in blk)
    assert list(bexp) == sorted(bexp)


def test_router_logits_are_fp32_rounded_exact_products():
    rng = np.random.default_rng(11)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 64)).astype(np.float32))
    wr = rng.standard_normal((3, 64)).astype(np.float32)
    l = moe.router_logits(mx.bf16_bits_to_f64(x), wr)
    from fractions import Fraction
    xf = mx.bf16_bits_to_f64(x)
    for t in range(2):
        for e in range(3):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wr[e]))
            assert l[t, e] == float(np.float32(float(exact)))


def test_ids_override_with_the_topk_itself_changes_nothing():
    layer, rng = _random_layer(I_s=64)
    x = synth.f32_to_bf16_bits(rng.standard_normal((6, 256)).astype(np.float32))
    out = moe.moe_layer(x, layer)
    again = moe.moe_layer(x, layer, ids=out["ids"])
    assert np.array_equal(again["y_bits"], out["y_bits"])
    np.testing.assert_allclose(again["weights"], out["weights"], rtol=1e-15)


def test_ids_override_hand_worked():
    # The hand layer's logits are (1, -1).  Forcing the second expert alone:
    # weight 1 and d = 1.5 (its hand-worked output, see the two-expert case),
    # not the top choice's -0.5.  Forcing both in swapped order: the weights
    # follow the order given, softmax of (-1, 1), and y is unchanged.
    layer = _hand_layer(k=1)
    x = _bf16([_row(1.0, 32)])
    out = moe.moe_layer(x, layer, ids=np.array([[1]]))
    assert out["weights"][0, 0] == 1.0
    assert np.all(out["y"] == 1.5)
    layer2 = _hand_layer(k=2)
    out2 = moe.moe_layer(x, layer2, ids=np.array([[1, 0]]))
    w0 = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(out2["weights"][0], [1.0 - w0, w0], rtol=1e-14)
    np.testing.assert_allclose(out2["y"], (1.0 - w0) * 1.5 + w0 * -0.5, rtol=1e-14)


def test_ids_override_any_order_of_all_experts_is_dense_mixture():
    # k = E with every row's experts given in a shuffled order: the weights
    # are the softmax of the logits in that order, so the layer is still the
    # dense softmax mixture.
    layer, rng = _random_layer(E=4, k=4)
    x = synth.f32_to_bf16_bits(rng.standard_normal((5, 256)).astype(np.float32))
    ids = np.stack([rng.permutation(4) for _ in range(5)]).astype(np.int32)
    out = moe.moe_layer(x, layer, ids=ids)
    xf = mx.bf16_bits_to_f64(x)
    logits = (xf @ layer.router_w.T).astype(np.float32).astype(np.float64)
    p = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(out["weights"], np.take_along_axis(p, ids, axis=1), rtol=1e-12)
    dense = np.zeros_like(xf)
    for e in range(4):
        d, _ = moe.mx_ffn(xf, layer.w13_codes[e], layer.w13_scales[e], layer.w2_codes[e], layer.w2_scales[e], "fp4")
        dense += p[:, e:e + 1] * d
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)


def test_folded_shared_expert_hand_worked():
    # The hand layer with its shared expert (gate 1.5, up 2, down 0.25; all on
    # the E2M1 grid, so the MXFP8 -> MXFP4 weight re-quantization is exact)
    # folded in as expert 2 with weight 1.  Its activations are now MXFP4:
    # xq = 1; g = 1.5, u = 2 -> a = silu(1.5) * 2 = 2.4527235 -> block exponent
    # -1, 4.905 -> nearest 4 -> aq = 2.0 (MXFP8 gave 2.5); s = 2.0 * 0.25 = 0.5.
    # Routed part -0.5 as before, residual 1: y = 1.0.
    layer = moe.fold_shared_expert(_hand_layer(k=1, with_shared=True, I_s=32))
    assert layer.shared_folded and layer.I_s == 0 and layer.E == 2
    x = _bf16([_row(1.0, 32)])
    r = _bf16([np.full(32, 1.0, np.float32)])
    out = moe.moe_layer(x, layer, residual_bits=r)
    assert out["ids"].tolist() == [[0]]
    assert np.all(out["s"] == 0.5)
    assert np.all(out["y"] == 1.0)


def test_folded_layer_routes_over_the_original_experts_only():
    # The folded expert is not a router candidate: ids stay in 0..E-1 and the
    # routed part is unchanged; only the always-on part differs.
    layer, rng = _random_layer(I=128, I_s=128)
    folded = moe.fold_shared_expert(layer)
    x = synth.f32_to_bf16_bits(rng.standard_normal((6, 256)).astype(np.float32))
    a = moe.moe_layer(x, layer)
    b = moe.moe_layer(x, folded)
    assert np.array_equal(a["ids"], b["ids"]) and np.array_equal(a["d"], b["d"])
    assert b["ids"].max() < layer.E
    # the folded part is the MXFP4 FFN of the re-quantized shared weights
    c13, s13 = mx.requant_fp8_to_fp4(layer.ws13_codes, layer.ws13_scales)
    c2, s2 = mx.requant_fp8_to_fp4(layer.ws2_codes, layer.ws2_scales)
    s_ref, _ = moe.mx_ffn(mx.bf16_bits_to_f64(x), c13, s13, c2, s2, "fp4")
    assert np.array_equal(b["s"], s_ref)


def test_rmsnorm_closed_forms():
    # constant rows: mean square c^2, so x = c / sqrt(c^2 + eps) * weight
    H = 64
    wgt = np.linspace(0.5, 1.5, H)
    h = np.stack([np.full(H, 3.0), np.full(H, -0.25)])
    x = moe.rmsnorm(h, wgt, 1e-6)
    np.testing.assert_allclose(x[0], 3.0 / math.sqrt(9.0 + 1e-6) * wgt, rtol=1e-15)
    np.testing.assert_allclose(x[1], -0.25 / math.sqrt(0.0625 + 1e-6) * wgt, rtol=1e-15)
    # eps = 0: invariant to scaling the row by a power of two (exact)
    rng = np.random.default_rng(2)
    r = rng.standard_normal((3, H))
    assert np.array_equal(moe.rmsnorm(r * 8.0, wgt, 0.0), moe.rmsnorm(r, wgt, 0.0))
    # every normalized row has mean square 1 (unit weight, eps = 0)
    np.testing.assert_allclose(np.mean(moe.rmsnorm(r, np.ones(H), 0.0) ** 2, axis=1), 1.0, rtol=1e-14)


def test_normed_layer_on_unit_rms_rows_is_the_plain_layer_with_residual():
    # rows of +-1 have mean square 1: with unit weight and eps = 0 the norm
    # is the identity, so the normed layer equals the plain layer with its
    # input added back as the residual
    layer, rng = _random_layer(I_s=64)
    x = synth.f32_to_bf16_bits(rng.choice([-1.0, 1.0], size=(5, 256)).astype(np.float32))
    plain = moe.moe_layer(x, layer, residual_bits=x)
    layer.norm_weight, layer.norm_eps = np.ones(256), 0.0
    normed = moe.moe_layer(x, layer)
    assert np.array_equal(normed["y"], plain["y"]) and np.array_equal(normed["ids"], plain["ids"])
    # a row scaled by 4 normalizes to the same x, so only the residual differs
    x4 = synth.f32_to_bf16_bits((4.0 * mx.bf16_bits_to_f64(x)).astype(np.float32))
    normed4 = moe.moe_layer(x4, layer)
    assert np.array_equal(normed4["ids"], normed["ids"])
    np.testing.assert_allclose(normed4["y"] - mx.bf16_bits_to_f64(x4), normed["y"] - mx.bf16_bits_to_f64(x),
                               rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        moe.moe_layer(x, layer, residual_bits=x)
