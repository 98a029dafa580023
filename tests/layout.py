"""The GPU library's tiled MX weight layout, written out from its definition
(include/mxmoe.h), as test plumbing: the tests compare the library's tiled
quantizer with the oracle's row-major codes through this map.  It holds no
arithmetic of the layer and is not part of the oracle."""

import numpy as np

from oracle import mx

# ---------------------------------------------------------------------------
# A weight matrix W[N, K] (N % 16 == 0, K % 128 == 0) is cut into tiles of 16
# rows x 128 columns.  Tile (nt, kt) holds TB bytes (1024 for FP4, 2048 for
# FP8) at byte offset (nt * K/128 + kt) * TB.  Inside a tile, with lane
# l = 0..63, r = nt*16 + l % 16, q = l // 16 and j = 0..15:
#   FP4: byte 16*l + j  = codes of W[r, kt*128 + 32*q + 2*j]  (low nibble)
#                         and   W[r, kt*128 + 32*q + 2*j + 1] (high nibble);
#   FP8: byte 1024*c + 16*l + j (c = 0, 1) = code of W[r, kt*128 + 64*c + 16*q + j].
# Scales: KG = ceil(K/512) groups of four K-tiles per 16-row strip.  Byte
#   ((nt * KG + g) * 64 + l) * 4 + i  = scale of W[r, block 4*(4*g + i) + q],
# and 127 where 4*g + i is beyond the last K-tile.

def tile_weight(codes, scales, fmt):
    """Tiled layout of an MX weight matrix given unpacked ``codes`` [N, K] and
    ``scales`` [N, K/32]; returns (tiled_codes, tiled_scales) as flat uint8."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, K = codes.shape
    if N % 16 or K % 128:
        raise ValueError("tiled layout needs N % 16 == 0 and K % 128 == 0")
    KT = K // 128
    KG = (KT + 3) // 4
    TB = 1024 if fmt == "fp4" else 2048
    out = np.zeros(N // 16 * KT * TB, dtype=np.uint8)
    osc = np.full(N // 16 * KG * 256, 127, dtype=np.uint8)
    for nt in range(N // 16):
        for kt in range(KT):
            base = (nt * KT + kt) * TB
            for l in range(64):
                r = nt * 16 + l % 16
                q = l // 16
                if fmt == "fp4":
                    k0 = kt * 128 + 32 * q
                    seg = codes[r, k0:k0 + 32]
                    out[base + 16 * l: base + 16 * l + 16] = mx.pack_fp4(seg)
                else:
                    for c in range(2):
                        k0 = kt * 128 + 64 * c + 16 * q
                        out[base + 1024 * c + 16 * l: base + 1024 * c + 16 * l + 16] = codes[r, k0:k0 + 16]
        for g in range(KG):
            for l in range(64):
                r = nt * 16 + l % 16
                q = l // 16
                for i in range(4):
                    kt = 4 * g + i
                    if kt < KT:
                        osc[((nt * KG + g) * 64 + l) * 4 + i] = scales[r, 4 * kt + q]
    return out, osc
