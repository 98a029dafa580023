"""The bench's algorithmic bytes and FLOPs (the roofline denominators) against
the library's own tiled weight sizes and the layer's shapes."""

import bench
from mxfp4_moe_decode_amd import binding


def _expert_bytes(H, I):
    """W13 [2I, H] and W2 [H, I] in MXFP4 as the library lays them out."""
    return (binding.mx_codes_bytes(2 * I, H, "fp4") + binding.mx_scales_bytes(2 * I, H)
            + binding.mx_codes_bytes(H, I, "fp4") + binding.mx_scales_bytes(H, I))


def _shared_bytes(H, Is):
    return (binding.mx_codes_bytes(2 * Is, H, "fp8") + binding.mx_scales_bytes(2 * Is, H)
            + binding.mx_codes_bytes(H, Is, "fp8") + binding.mx_scales_bytes(H, Is))


def test_decode_layer_bytes_match_library_sizes():
    H, I, E, Is = 3072, 1024, 128, 1024
    for D, T in ((4, 1), (50, 16), (64, 16)):
        want = E * H * 4 + D * _expert_bytes(H, I) + _shared_bytes(H, Is) + 2 * T * H * 2
        assert bench.layer_bytes(H, I, E, Is, D, T) == want
    # the 1-row figure the roofline is quoted on
    assert bench.layer_bytes(H, I, E, Is, 4, 1) == 31_371_264
    # with a residual the bf16 residual row is read too
    assert bench.layer_bytes(H, I, E, Is, 4, 1, residual=True) == 31_371_264 + H * 2


def test_prefill_flops():
    routed, shared, router = bench.prefill_flops(8192, 3072, 1024, 128, 4, 1024)
    # gate/up is [2I, H] per chosen expert, down [H, I]: 3 I H multiply-adds per row and choice
    assert routed == 2 * 8192 * 4 * (2 * 1024 * 3072 + 3072 * 1024)
    assert shared == 2 * 8192 * (2 * 1024 * 3072 + 3072 * 1024)
    assert router == 2 * 8192 * 128 * 3072
    assert round(routed / 1e9, 1) == 618.5 and round(shared / 1e9, 1) == 154.6 and round(router / 1e9, 2) == 6.44


def test_folded_layer_bytes():
    """Folded: the MXFP8 shared expert's 9,732,096 B become one more MXFP4
    expert of 5,013,504 B."""
    H, I, E, Is = 3072, 1024, 128, 1024
    assert bench.layer_bytes(H, I, E, Is, 4, 1, folded=True) == 31_371_264 - 9_732_096 + 5_013_504
    assert bench.layer_bytes(H, I, E, Is, 4, 1, folded=True) == E * H * 4 + 5 * _expert_bytes(H, I) + 2 * H * 2
