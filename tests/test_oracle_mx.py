"""Pins of the oracle's MX formats against the OCP MX closed forms, torch's
float8 dtypes (a library conversion written independently of the oracle),
brute force over every bf16 pattern, and invariants of the block scale rule."""

import math

import numpy as np
import pytest
import torch

from oracle import mx
from tests import layout
from tests.conftest import read_golden


def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = mx.bf16_bits_to_f64(bits)
    return v[np.isfinite(v)]


# --------------------------------------------------------------------------- decoders

def test_e2m1_table_matches_ocp_golden():
    for code, val in read_golden("e2m1_values.txt"):
        got = mx.e2m1_value(int(code))
        assert float(got) == float(val), code
        assert math.copysign(1.0, float(got)) == math.copysign(1.0, float(val))


def test_e4m3_specials_match_ocp_golden():
    for code, val in read_golden("e4m3_specials.txt"):
        got = float(mx.e4m3_value(int(code, 16)))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = mx.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e8m0_matches_golden_and_torch():
    for code, lg in read_golden("e8m0_specials.txt"):
        got = float(mx.e8m0_value(int(code)))
        if lg == "nan":
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, int(lg))
    ref = torch.arange(255, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(ref, mx.e8m0_value(np.arange(255)))


# --------------------------------------------------------------------------- element rounding

def test_e4m3_rounding_matches_torch_for_every_bf16_value():
    """torch's fp32 -> float8_e4m3fn conversion rounds to nearest even and
    returns NaN past the 448/480 midpoint; the MX conversion saturates there."""
    v = _all_bf16_values()
    got = mx.round_to_element(v, "fp8")
    inr = np.abs(v) <= 464.0
    ref = torch.from_numpy(v[inr].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], ref)
    out = ~inr
    assert np.all((got[out] & 0x7F) == 0x7E)
    assert np.array_equal(got[out] >> 7, np.signbit(v[out]).astype(np.uint8))


def _brute_force_codes(v, fmt):
    """Nearest element value by exhaustive comparison against every finite
    code; equal distances go to the even magnitude code; sign copied."""
    maxc = mx.FORMATS[fmt]["max_code"]
    grid = np.array([float(mx.element_value(c, fmt)) for c in range(maxc + 1)])
    mag = np.abs(v)
    dist = np.abs(mag[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equally near codes prefer the even one (there are at most two)
    even = cand & (np.arange(maxc + 1)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = np.where(mag >= grid[-1], maxc, code)
    return (code | (np.signbit(v).astype(np.int64) << mx.FORMATS[fmt]["sign_bit"])).astype(np.uint8)


@pytest.mark.parametrize("shift", [-3, 0, 2, 7])
def test_e2m1_rounding_brute_force_every_bf16_value(shift):
    v = _all_bf16_values()
    v = np.ldexp(v, shift)
    assert np.array_equal(mx.round_to_element(v, "fp4"), _brute_force_codes(v, "fp4"))


def test_e2m1_ties_go_to_even_codes():
    # midpoints between neighbouring E2M1 values and the expected even code
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7}
    for v, c in cases.items():
        assert int(mx.round_to_element(np.array([v]), "fp4")[0]) == c, v
        assert int(mx.round_to_element(np.array([-v]), "fp4")[0]) == c | 8, -v
    # sign kept for values that round to zero and for -0.0
    assert int(mx.round_to_element(np.array([-0.1]), "fp4")[0]) == 8
    assert int(mx.round_to_element(np.array([-0.0]), "fp4")[0]) == 8
    assert int(mx.round_to_element(np.array([1e30]), "fp4")[0]) == 7


def test_e4m3_fp32_midpoints_and_neighbours_match_torch():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7E, 2000)
    lo = mx.e4m3_value(codes)
    hi = mx.e4m3_value(codes + 1)
    mid = (lo + hi) / 2  # exact in fp32 for E4M3 neighbours
    for d in (0, 1, -1):
        v = np.nextafter(mid.astype(np.float32), np.float32(np.inf) if d > 0 else np.float32(-np.inf)) if d else mid.astype(np.float32)
        ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(mx.round_to_element(v.astype(np.float64), "fp8"), ref)


# --------------------------------------------------------------------------- block scale

@pytest.mark.parametrize("fmt,lo,hi", [("fp4", 4.0, 8.0), ("fp8", 256.0, 512.0)])
def test_scaled_block_max_in_top_binade(fmt, lo, hi):
    """floor(log2 amax) - emax puts amax / X in [2^emax, 2^(emax+1))."""
    rng = np.random.default_rng(1)
    amax = np.ldexp(rng.uniform(1, 2, 5000), rng.integers(-100, 100, 5000))
    e = mx.shared_exponent(amax, fmt)
    s = np.ldexp(amax, -e)
    assert np.all((s >= lo) & (s < hi))


def test_scale_clamps_and_zero_block():
    assert int(mx.shared_exponent(0.0, "fp4")) == -127
    assert int(mx.shared_exponent(2.0 ** -140, "fp4")) == -127
    assert int(mx.shared_exponent(2.0 ** 127, "fp4")) == 125
    codes, scales = mx.mx_quantize(np.zeros((1, 32)), "fp4")
    assert scales[0, 0] == 0 and np.all(codes == 0)


def test_quantize_error_within_half_quantum():
    """|dequant - v| <= half the element spacing at |v| (or the saturation gap)."""
    rng = np.random.default_rng(2)
    for fmt, mbits, emin in (("fp4", 1, 0), ("fp8", 3, -6)):
        v = rng.standard_normal((64, 256)).astype(np.float32).astype(np.float64)
        c, s = mx.mx_quantize(v, fmt)
        dq = mx.mx_dequantize(c, s, fmt)
        X = np.repeat(mx.e8m0_value(s), 32, axis=1)
        y = np.abs(v) / X
        p = np.floor(np.log2(np.maximum(y, 2.0 ** -30)))
        half = 0.5 * np.ldexp(1.0, (np.maximum(p, emin) - mbits).astype(int)) * X
        maxv = float(mx.element_value(mx.FORMATS[fmt]["max_code"], fmt))
        sat = y > maxv
        assert np.all(np.abs(dq - v)[~sat] <= half[~sat])
        assert np.all(np.abs(dq[sat]) == maxv * X[sat])


def test_quantize_requantize_is_identity():
    rng = np.random.default_rng(3)
    for fmt in ("fp4", "fp8"):
        v = rng.standard_normal((16, 128)).astype(np.float32).astype(np.float64)
        c, s = mx.mx_quantize(v, fmt)
        c2, s2 = mx.mx_quantize(mx.mx_dequantize(c, s, fmt), fmt)
        # the block max may drop a binade when it saturated; codes then shift, so
        # compare values instead of codes
        assert np.array_equal(mx.mx_dequantize(c2, s2, fmt), mx.mx_dequantize(c, s, fmt))


# --------------------------------------------------------------------------- lossless BF16 widening

def test_e4m3_times_power_of_two_is_exact_in_bf16():
    """vLLM PR "[ROCm] MiniMax-M3: allow the AMD monokernel decode on
    MiniMax-M3.1", section "Purpose": E4M3 times a power-of-two scale is exact
    in BF16.  Checked for every finite code and scales 2^-100..2^100."""
    vals = mx.e4m3_value(np.arange(256))
    vals = vals[np.isfinite(vals)]
    for k in range(-100, 101, 7):
        y = np.ldexp(vals, k)
        back = mx.bf16_bits_to_f64(mx.round_to_bf16_bits(y))
        assert np.array_equal(back, y)
    vals4 = mx.e2m1_value(np.arange(16))
    y = np.ldexp(vals4, 5)
    assert np.array_equal(mx.bf16_bits_to_f64(mx.round_to_bf16_bits(y)), y)


# --------------------------------------------------------------------------- bf16 rounding / packing

def test_round_to_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(20000), np.ldexp(rng.standard_normal(2000), -130)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx.round_to_bf16_bits(v.astype(np.float64)), ref)


def test_round_to_bf16_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint 1 + 2^-8; a detour
    # through fp32 would land on the midpoint and round to even (1.0)
    y = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert mx.bf16_bits_to_f64(mx.round_to_bf16_bits(y))[0] == 1.0 + 2.0 ** -7


def test_fp4_nibble_order():
    assert mx.pack_fp4(np.array([[0x1, 0xF]]))[0, 0] == 0xF1
    c = np.random.default_rng(0).integers(0, 16, (3, 64)).astype(np.uint8)
    assert np.array_equal(mx.unpack_fp4(mx.pack_fp4(c)), c)


# --------------------------------------------------------------------------- tiled layout

@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_tiled_layout_is_a_bijection_with_hand_checked_entries(fmt):
    N, K = 32, 640  # K/128 = 5 tiles -> scale groups padded to 8
    rng = np.random.default_rng(7)
    maxc = 16 if fmt == "fp4" else 256
    codes = rng.integers(0, maxc, (N, K)).astype(np.uint8)
    scales = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
    tc, ts = layout.tile_weight(codes, scales, fmt)
    TB = 1024 if fmt == "fp4" else 2048
    assert tc.size == N // 16 * (K // 128) * TB
    assert ts.size == N // 16 * 2 * 256
    if fmt == "fp4":
        # row 17 (strip 1, lane 1 + 16*q), column 300 = tile 2, q = 1, j = 6 (even -> low nibble)
        byte = tc[(1 * 5 + 2) * 1024 + 16 * (1 + 16 * 1) + 6]
        assert byte & 0xF == codes[17, 300] and byte >> 4 == codes[17, 301]
        assert np.array_equal(np.sort(mx.unpack_fp4(tc)), np.sort(codes.reshape(-1)))
    else:
        # row 3, column 128*4 + 64 + 16*2 + 5 = 613: tile 4, c = 1, q = 2, j = 5
        assert tc[(0 * 5 + 4) * 2048 + 1024 + 16 * (3 + 16 * 2) + 5] == codes[3, 613]
        assert np.array_equal(np.sort(tc), np.sort(codes.reshape(-1)))
    # scale of row 20, block 4*(4*1 + 0) + 3 = 19: strip 1, group 1, lane 4 + 16*3, byte 0
    assert ts[((1 * 2 + 1) * 64 + 4 + 48) * 4 + 0] == scales[20, 19]
    # padding (K-tiles 5..7) holds 127
    assert ts[((0 * 2 + 1) * 64 + 0) * 4 + 1] == 127


def test_requant_fp8_to_fp4_hand_worked():
    # One MXFP8 block, scale 2^-7: element 0 = E4M3 0x7A (320) -> 2.5, element
    # 1 = E4M3 0xE2 (-40) -> -0.3125.  MXFP4: block max 2.5 -> exponent
    # floor(log2 2.5) - 2 = -1; 2.5 * 2 = 5 lies halfway between 4 (code 6) and
    # 6 (code 7) -> even code 6, value 4 * 2^-1 = 2.0 (the loss); -0.3125 * 2 =
    # -0.625 -> nearest 0.5 -> code 0x9, value -0.25.
    c8 = np.zeros((1, 32), np.uint8)
    c8[0, 0], c8[0, 1] = 0x7A, 0xE2
    s8 = np.array([[127 - 7]], np.uint8)
    c4, s4 = mx.requant_fp8_to_fp4(c8, s8)
    assert s4.tolist() == [[126]]
    assert c4[0, 0] == 6 and c4[0, 1] == 0x9 and not c4[0, 2:].any()
    v = mx.mx_dequantize(c4, s4, "fp4")
    assert v[0, 0] == 2.0 and v[0, 1] == -0.25


def test_requant_fp8_to_fp4_brute_force_every_e4m3_code():
    # Block: element 0 carries every finite E4M3 code in turn, element 1 is
    # fixed at +448 (the E4M3 maximum), so the MXFP4 block exponent is
    # floor(log2(448 * X)) - 2 = 6 + (s - 127) for scale code s.  Each code's
    # requantized value must be the E2M1 grid point nearest to its exact value
    # (found by exhaustive search over the 8 magnitudes, ties to the even code).
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for s in (120, 127, 131):
        codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
        c8 = np.zeros((codes.size, 32), np.uint8)
        c8[:, 0] = codes
        c8[:, 1] = 0x7E  # 448
        s8 = np.full((codes.size, 1), s, np.uint8)
        c4, s4 = mx.requant_fp8_to_fp4(c8, s8)
        e = 6 + (s - 127)
        assert np.all(s4 == e + 127)
        for i, c in enumerate(codes.tolist()):
            v = mx.e4m3_value(c) * 2.0 ** (s - 127) / 2.0 ** e
            mag = abs(v)
            dist = [abs(mag - g) for g in grid]
            best = min(dist)
            cands = [j for j in range(8) if dist[j] == best]
            j = cands[0] if len(cands) == 1 else [j for j in cands if j % 2 == 0][0]
            if mag > 6:
                j = 7
            want = j | (8 if (c & 0x80) else 0)
            assert c4[i, 0] == want, (s, hex(c), v, c4[i, 0], want)
        # the fixed 448 element: 448 * X / 2^e = 7 -> saturates to 6 (code 7)
        assert np.all(c4[:, 1] == 7)


def test_requant_fp8_to_fp4_lossless_on_the_fp4_grid():
    # Values that are E2M1 values times a common power of two survive the
    # round trip fp32 -> MXFP8 -> MXFP4 unchanged.
    rng = np.random.default_rng(5)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    w = rng.choice(grid, size=(16, 128)) * rng.choice([-1.0, 1.0], size=(16, 128)) * 2.0 ** -9
    w[:, ::32] = 6 * 2.0 ** -9  # every block reaches the top binade
    c8, s8 = mx.mx_quantize(w, "fp8")
    c4, s4 = mx.requant_fp8_to_fp4(c8, s8)
    assert np.array_equal(mx.mx_dequantize(c4, s4, "fp4"), w)


def _e4m3_code(v):
    """E4M3 code of an exactly representable positive value (test helper)."""
    vals = mx.e4m3_value(np.arange(0x7F))
    return int(np.flatnonzero(vals == v)[0])


def test_nvfp4_requant_hand_worked():
    # Block scale 1.5 (E4M3), global 0.5: E2M1 6 -> 6 * 1.5 * 0.5 = 4.5 and
    # E2M1 -1 -> -0.75.  MXFP4 of the 32-block: max 4.5 -> exponent
    # floor(log2 4.5) - 2 = 0; 4.5 -> nearest of 4 / 6 is 4 (code 6): lossy;
    # -0.75 halfway between 0.5 (code 1) and 1 (code 2) -> even code 2 -> -1.
    c = np.zeros((1, 32), np.uint8)
    c[0, 0], c[0, 17] = 7, 0xA  # +6 in the first 16-block, -1 in the second
    bs = np.array([[_e4m3_code(1.5), _e4m3_code(1.5)]], np.uint8)
    v = mx.nvfp4_dequantize(c, bs, [0.5], 1)
    assert v[0, 0] == 4.5 and v[0, 17] == -0.75
    c4, s4 = mx.requant_nvfp4_to_mxfp4(c, bs, [0.5], 1)
    assert s4.tolist() == [[127]]
    assert c4[0, 0] == 6 and c4[0, 17] == 0xA and not np.delete(c4[0], [0, 17]).any()


def test_nvfp4_requant_is_lossless_for_power_of_two_scales():
    # Block scales that are powers of two, equal over each pair of 16-blocks,
    # and a power-of-two global scale: every 32-block is E2M1 codes times a
    # common power of two, so MXFP4 holds it exactly (with a top-binade element
    # the MX exponent is that power and the codes are unchanged).
    rng = np.random.default_rng(1)
    rows, cols = 8, 128
    c = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    c[:, ::32] = 6  # magnitude 4: top binade of E2M1
    k = rng.integers(-6, 6, size=(rows, cols // 32))
    bs = np.repeat(np.vectorize(lambda e: _e4m3_code(2.0 ** e))(k), 2, axis=1).astype(np.uint8)
    g = [2.0 ** -3, 2.0 ** 2]
    c4, s4 = mx.requant_nvfp4_to_mxfp4(c, bs, g, rows // 2)
    assert np.array_equal(c4, c)
    gexp = np.repeat(np.log2(g), rows // 2)[:, None]
    assert np.array_equal(s4.astype(np.int64), (127 + k + gexp).astype(np.int64))
    assert np.array_equal(mx.mx_dequantize(c4, s4, "fp4"), mx.nvfp4_dequantize(c, bs, g, rows // 2))


def test_nvfp4_requant_brute_force_every_element_and_block_scale():
    # Every E2M1 code next to a fixed +6 element, under every finite positive
    # E4M3 block scale and a non-power-of-two global scale: the MXFP4 code is
    # the grid point nearest to the exact scaled value (exhaustive search,
    # ties to the even code, saturation), and the block exponent is
    # floor(log2(6 * s_block * g)) - 2.
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    g = 0.3
    scales = np.array([b for b in range(1, 0x7F)], np.uint8)
    for s in scales.tolist():
        c = np.zeros((16, 32), np.uint8)
        c[:, 0] = np.arange(16)
        c[:, 1] = 7
        bs = np.full((16, 2), s, np.uint8)
        v = mx.nvfp4_dequantize(c, bs, [g], 16)
        c4, s4 = mx.requant_nvfp4_to_mxfp4(c, bs, [g], 16)
        amax = float(np.float32(6 * mx.e4m3_value(s)) * np.float32(g))
        e = math.floor(math.log2(amax)) - 2
        if amax == 0 or e < -127:
            continue
        assert np.all(s4 == e + 127), s
        for i in range(16):
            q = abs(v[i, 0]) / 2.0 ** e
            dist = [abs(q - p) for p in grid]
            best = min(dist)
            cands = [j for j in range(8) if dist[j] == best]
            j = cands[0] if len(cands) == 1 else [j for j in cands if j % 2 == 0][0]
            if q > 6:
                j = 7
            want = j | (8 if (i & 8) else 0)
            assert c4[i, 0] == want, (s, i, q, c4[i, 0], want)
