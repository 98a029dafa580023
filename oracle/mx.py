"""OCP MX element formats and block quantization, written out plainly in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

What the pages fix: routed-expert weights are OCP MXFP4 with static scales and
routed-expert activations are OCP MXFP4 with dynamic scales (model card
"amd/MiniMax-M3.1-Flash-Quark-MXFP4", section "Model Overview"); the shared
expert is MXFP8 (article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and
optimization", section "MiniMax-M3.1 at a glance"); an E4M3 value times a
power-of-two scale is exact in BF16 (vLLM PR "[ROCm] MiniMax-M3: allow the AMD
monokernel decode on MiniMax-M3.1", section "Purpose").  The pages do not spell
the formats out; the definitions below are those of the OCP Microscaling
Formats (MX) v1.0 specification:

* a block is 32 consecutive elements along the reduction axis sharing one
  E8M0 scale X = 2**(code - 127) (code 255 is NaN and never produced);
* E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf or NaN;
* E4M3 (FP8, the "FN" variant): sign, 4 exponent bits (bias 7), 3 mantissa
  bits; subnormals 2**-6 * m/8; S.1111.111 is NaN; max magnitude 448;
* conversion: shared exponent = floor(log2(max|v|)) - emax_elem (emax_elem = 2
  for E2M1, 8 for E4M3), then each v / X is rounded to the nearest element
  value, ties to the even code, saturating to the largest finite magnitude.

Readings taken where the specification leaves a choice (each one is listed
with its reason in the design notes of the repository):

* the shared exponent is clamped to [-127, 127]; an all-zero block gets -127;
* the sign of v is kept even when v / X rounds to zero (and for -0.0);
* FP4 codes are packed two per byte, element 2i in the low nibble of byte i.
"""

import numpy as np

BLOCK = 32

# Per-format constants: exponent of the largest power of two in the element
# format (emax_elem), sign-bit position, largest finite magnitude code.
FORMATS = {
    "fp4": {"emax": 2, "sign_bit": 3, "max_code": 0x7},
    "fp8": {"emax": 8, "sign_bit": 7, "max_code": 0x7E},
}


# ---------------------------------------------------------------------------
# Element and scale decoders (closed forms of the OCP MX element formats)
# ---------------------------------------------------------------------------

def e2m1_value(codes):
    """Value of E2M1 codes (0..15): (-1)^s * 2^(e-1) * (1 + m/2) for e >= 1,
    (-1)^s * 0.5 * m for e == 0 (OCP MX v1.0, FP4 E2M1 element type)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e4m3_value(codes):
    """Value of E4M3 codes (0..255): (-1)^s * 2^(e-7) * (1 + m/8) for e >= 1,
    (-1)^s * 2^-6 * m/8 for e == 0; NaN for S.1111.111 (OCP MX v1.0, FP8
    E4M3 element type)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e8m0_value(codes):
    """Value of E8M0 scale codes: 2^(c - 127); 255 is NaN (OCP MX v1.0, E8M0
    scale type)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def element_value(codes, fmt):
    return e2m1_value(codes) if fmt == "fp4" else e4m3_value(codes)


def _magnitude_grid(fmt):
    """Magnitudes of the non-negative finite codes 0..max_code, ascending (both
    formats are monotone in their magnitude code)."""
    return element_value(np.arange(FORMATS[fmt]["max_code"] + 1), fmt)


# ---------------------------------------------------------------------------
# Conversion to an element code (round to nearest, ties to even, saturate)
# ---------------------------------------------------------------------------

def round_to_element(v, fmt):
    """Codes of the element values nearest to v (fp64 array, already divided
    by the block scale).  Ties go to the even code; magnitudes beyond the
    largest finite value saturate to it; the sign bit is copied from v."""
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    grid = _magnitude_grid(fmt)
    max_code = FORMATS[fmt]["max_code"]
    mag = np.abs(v)
    # grid[i - 1] <= mag < grid[i]
    i = np.searchsorted(grid, mag, side="right")
    lo = np.clip(i - 1, 0, max_code)
    hi = np.clip(i, 0, max_code)
    d_lo = mag - np.take(grid, lo)
    d_hi = np.take(grid, hi) - mag
    code = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(mag >= grid[max_code], max_code, code)
    sign = np.signbit(v).astype(np.int64) << FORMATS[fmt]["sign_bit"]
    return (code | sign).astype(np.uint8).reshape(shape)


def shared_exponent(amax, fmt):
    """Block scale exponent floor(log2(amax)) - emax_elem, clamped to the E8M0
    range [-127, 127]; an all-zero block gets -127 (OCP MX v1.0 conversion
    rule; clamp and zero-block handling are readings, see module docstring)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)          # amax = f * 2^ex with 0.5 <= f < 1
    floor_log2 = ex.astype(np.int64) - 1
    e = floor_log2 - FORMATS[fmt]["emax"]
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127)


def mx_quantize(values, fmt):
    """Quantize ``values`` (fp64 array whose entries are exact bf16 / fp32
    numbers; last axis a multiple of 32) to MX blocks along the last axis.

    Returns (codes, scales): codes uint8 of the same shape, one element code
    per entry (unpacked); scales uint8 with last axis K/32 (E8M0 codes)."""
    v = np.asarray(values, dtype=np.float64)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    blocks = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    e = shared_exponent(amax, fmt)
    scaled = np.ldexp(blocks, -e[..., None])  # exact: division by a power of two
    codes = round_to_element(scaled, fmt).reshape(v.shape)
    return codes, (e + 127).astype(np.uint8)


def mx_dequantize(codes, scales, fmt):
    """Element value times its block's E8M0 scale, fp64 (exact)."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    vals = element_value(codes, fmt)
    sc = np.repeat(e8m0_value(scales), BLOCK, axis=-1)
    assert sc.shape[-1] == K
    return vals * sc


def requant_fp8_to_fp4(codes8, scales8):
    """Re-quantize an MXFP8 matrix to MXFP4 along the same 32-element blocks:
    each element's exact value (E4M3 value times its E8M0 scale) is quantized
    again by the MX conversion with the E2M1 element type (the shared expert
    re-quantized to MXFP4 so that it runs as one more MXFP4 expert; vLLM PR
    "[ROCm] MiniMax-M3: allow the AMD monokernel decode on MiniMax-M3.1",
    section "Purpose", which notes that this re-quantization is lossy; model
    card "amd/MiniMax-M3.1-Flash-Quark-MXFP4", section "Experimental MXFP4
    shared experts").  Returns (codes, scales) of the MXFP4 matrix."""
    return mx_quantize(mx_dequantize(codes8, scales8, "fp8"), "fp4")


def nvfp4_dequantize(codes, block_scales, global_scales, rows_per_scale):
    """Values of an NVFP4 matrix, the format of the checkpoint's routed experts
    (article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and
    optimization", section "MiniMax-M3.1 at a glance").  The pages name the
    format without defining it; the definition used is the public NVFP4 one:
    E2M1 elements (unpacked ``codes`` [rows, cols]) in blocks of 16
    consecutive elements along a row, each block with an unsigned E4M3 scale
    (``block_scales`` [rows, cols/16] codes), and a second-level fp32 scale per
    group of ``rows_per_scale`` rows (``global_scales``):
        v = E2M1(c) * E4M3(s_block) * s_global.
    E2M1 times E4M3 is exact (at most 6 significant bits); the product with
    the fp32 global scale is rounded once to fp32, the precision a loader
    holds weights in.  Returns fp64 values (each an fp32 number)."""
    codes = np.asarray(codes)
    rows, cols = codes.shape
    bs = np.repeat(e4m3_value(block_scales), 16, axis=-1)
    g = np.repeat(np.asarray(global_scales, np.float64), rows_per_scale)[:rows, None]
    return to_f32(e2m1_value(codes) * bs * g)


def requant_nvfp4_to_mxfp4(codes, block_scales, global_scales, rows_per_scale):
    """NVFP4 -> MXFP4: the MX conversion (E2M1 elements, 32-element blocks,
    E8M0 scales) of the NVFP4 matrix's fp32 values (the load-time conversion of
    the NVFP4 routed experts to the MXFP4 datapath: article above, TL;DR and
    section "Day 0 support for AMD Instinct GPUs"; vLLM PR #64273, squash
    commit notes "Re-quantize the NVFP4 routed experts to MXFP8 (or MXFP4) at
    load").  Returns (codes, scales) of the MXFP4 matrix."""
    return mx_quantize(nvfp4_dequantize(codes, block_scales, global_scales, rows_per_scale), "fp4")


def pack_fp4(codes):
    """Two E2M1 codes per byte along the last axis: element 2i in the low
    nibble of byte i, element 2i+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# bf16 / fp32 helpers (plain IEEE conversions used by the oracle)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """Exact value of bf16 numbers given as uint16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(y):
    """Round fp64 values to the nearest bf16, ties to even (one rounding, no
    detour through fp32); returns uint16 bit patterns.  bf16 keeps 8
    significant bits and the fp32 exponent range (subnormal quantum 2^-133)."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite value")
    _, ex = np.frexp(y)
    q = np.maximum(ex.astype(np.int64) - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(y, -q)), q)       # np.rint: ties to even
    if np.any(np.abs(r) >= 2.0 ** 128):
        raise OverflowError("bf16 overflow")
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def to_f32(y):
    """Round fp64 to the nearest fp32 (ties to even), returned as fp64."""
    return np.asarray(y, dtype=np.float64).astype(np.float32).astype(np.float64)


