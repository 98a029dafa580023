"""Seeded synthetic inputs shaped like the MiniMax-M3.1 MoE layer.

This module only draws random numbers; it holds none of the layer's
arithmetic (no quantization, routing or FFN).  Both the GPU path and the CPU
oracle take their inputs from here, so the two never share anything else.

Workloads (sizes from the layer the pages describe: 128 routed experts, 4 active
per token, plus a shared expert, article "MiniMax-M3.1 on AMD Instinct GPUs:
Day-0 support and optimization", section "MiniMax-M3.1 at a glance"; hidden and
intermediate sizes are not on the pages and are taken as 3072 / 1024):

* ``tiny``     T=4,    H=256,  E=8,   k=2, I=128,  no shared expert, seed 0
* ``decode1``  T=1,    H=3072, E=128, k=4, I=1024, shared expert I_s=1024
* ``decode16`` T=16,   same layer, router weights U(-1/sqrt(H), 1/sqrt(H))
* ``chain8``   T=4,    8 layers with distinct weights, Zipf(s=1.2) router bias,
               residual add between layers
* ``prefill``  T=8192, same layer as ``decode1``
* ``tp4``      T=16, the per-GPU share of the layer under 4-way tensor
               parallelism over the intermediate dimension: H=3072, E=128,
               k=4, I=256, shared I_s=256
* ``wide``     T=16, H=3072, 256 experts top-8, I=256, shared I_s=256
* ``odd``      T=16, H=1280, 16 experts top-3, I=384, shared I_s=640: K-tile
               counts 10 / 3 / 5, so the dot products split into 2 / 1 / 1
               K-chunks and the scale groups end part-filled
* ``h640``     T=16, H=640, 16 experts top-2, I=256, shared I_s=384: H not a
               multiple of 256 (the grouped routed down keeps 128-column
               tiles), K-tile counts 5 / 2 / 3
* ``h384``     T=16, H=384, 16 experts top-2, I=512, shared I_s=512: H not a
               multiple of 256 with whole scale groups in the down products
               (K-tile counts 3 / 4 / 4)

Draws: expert and shared weights fp32 N(0, 0.02); router weights fp32 N(0, 0.02)
(``decode16``: uniform); activations N(0, 1) stored as bf16 (round to nearest
even of the fp32 draw).  Zipf bias: b_e = -s * ln(rank_e) with rank a seeded
permutation of 1..E, so the prior over experts is proportional to rank^-s.

Every tensor has its own stream, so any single expert can be regenerated on
its own: on the host a PCG64 ``default_rng([seed, workload, layer, tag,
index])``; for full-size expert and shared weights, torch's device Philox
generator seeded from the same key (``device_*`` functions).
"""

import math

import numpy as np

WORKLOADS = {
    "tiny": dict(T=4, H=256, E=8, k=2, I=128, I_s=0, router="normal", layers=1,
                 zipf=None, residual=False),
    "decode1": dict(T=1, H=3072, E=128, k=4, I=1024, I_s=1024, router="normal", layers=1,
                    zipf=None, residual=False),
    "decode16": dict(T=16, H=3072, E=128, k=4, I=1024, I_s=1024, router="uniform", layers=1,
                     zipf=None, residual=False),
    "chain8": dict(T=4, H=3072, E=128, k=4, I=1024, I_s=1024, router="normal", layers=8,
                   zipf=1.2, residual=True),
    "prefill": dict(T=8192, H=3072, E=128, k=4, I=1024, I_s=1024, router="normal", layers=1,
                    zipf=None, residual=False),
    "tp4": dict(T=16, H=3072, E=128, k=4, I=256, I_s=256, router="normal", layers=1,
                zipf=None, residual=False),
    "wide": dict(T=16, H=3072, E=256, k=8, I=256, I_s=256, router="normal", layers=1,
                 zipf=None, residual=False),
    "odd": dict(T=16, H=1280, E=16, k=3, I=384, I_s=640, router="normal", layers=1,
                zipf=None, residual=False),
    "h640": dict(T=16, H=640, E=16, k=2, I=256, I_s=384, router="normal", layers=1,
                 zipf=None, residual=False),
    "h384": dict(T=16, H=384, E=16, k=2, I=512, I_s=512, router="normal", layers=1,
                 zipf=None, residual=False),
}
_WID = {name: i + 1 for i, name in enumerate(WORKLOADS)}
_TAG = {"router": 1, "w13": 2, "w2": 3, "ws13": 4, "ws2": 5, "bias": 6, "x": 7, "nvfp4": 8, "norm": 9}
WEIGHT_STD = 0.02


def workload(name, **overrides):
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    cfg["name"] = name
    cfg.setdefault("seed", 0)
    return cfg


def _rng(cfg, layer, tag, index=0):
    return np.random.default_rng([cfg["seed"], _WID[cfg["name"]], layer, _TAG[tag], index])


def router_weights(cfg, layer=0):
    """fp32 [E, H]."""
    g = _rng(cfg, layer, "router")
    E, H = cfg["E"], cfg["H"]
    if cfg["router"] == "uniform":
        b = 1.0 / math.sqrt(H)
        return g.uniform(-b, b, size=(E, H)).astype(np.float32)
    return (g.standard_normal((E, H), dtype=np.float32) * np.float32(WEIGHT_STD)).astype(np.float32)


def router_bias(cfg, layer=0):
    """fp32 [E] Zipf offsets, or None."""
    if not cfg.get("zipf"):
        return None
    g = _rng(cfg, layer, "bias")
    rank = g.permutation(cfg["E"]) + 1
    return (-cfg["zipf"] * np.log(rank.astype(np.float64))).astype(np.float32)


def _normal(cfg, layer, tag, index, shape):
    g = _rng(cfg, layer, tag, index)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(WEIGHT_STD)).astype(np.float32)


def expert_w13(cfg, layer, e):
    """fp32 [2I, H]: gate rows 0..I-1, up rows I..2I-1."""
    return _normal(cfg, layer, "w13", e, (2 * cfg["I"], cfg["H"]))


def expert_w2(cfg, layer, e):
    """fp32 [H, I]."""
    return _normal(cfg, layer, "w2", e, (cfg["H"], cfg["I"]))


def shared_w13(cfg, layer=0):
    return _normal(cfg, layer, "ws13", 0, (2 * cfg["I_s"], cfg["H"]))


def shared_w2(cfg, layer=0):
    return _normal(cfg, layer, "ws2", 0, (cfg["H"], cfg["I_s"]))


def f32_to_bf16_bits(a):
    """Storage rounding of an fp32 draw to bf16 (nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations(cfg, layer=0, T=None, index=0):
    """bf16 bit patterns [T, H] of N(0, 1) draws."""
    T = cfg["T"] if T is None else T
    g = _rng(cfg, layer, "x", index)
    return f32_to_bf16_bits(g.standard_normal((T, cfg["H"]), dtype=np.float32))


def _device_seed(cfg, layer, tag, index):
    """64-bit seed for torch's device generator, mixed from the same key as
    the host streams."""
    h = 1469598103934665603
    for v in (cfg["seed"], _WID[cfg["name"]], layer, _TAG[tag], index):
        h = ((h ^ (int(v) & 0xFFFFFFFFFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def _device_normal(cfg, layer, tag, index, shape, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(cfg, layer, tag, index))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    return t.normal_(0.0, WEIGHT_STD, generator=g)


def device_expert_w13(cfg, layer, e, device="cuda"):
    """fp32 [2I, H] N(0, 0.02) drawn on the device (torch's seeded Philox
    generator): the full-size layers have 128 experts of 9.4M weights each,
    too many to draw on the host for every test and benchmark run.  The oracle
    reads the very same values back with ``.cpu()``."""
    return _device_normal(cfg, layer, "w13", e, (2 * cfg["I"], cfg["H"]), device)


def device_expert_w2(cfg, layer, e, device="cuda"):
    """fp32 [H, I], as ``device_expert_w13``."""
    return _device_normal(cfg, layer, "w2", e, (cfg["H"], cfg["I"]), device)


def device_shared_w13(cfg, layer=0, device="cuda"):
    return _device_normal(cfg, layer, "ws13", 0, (2 * cfg["I_s"], cfg["H"]), device)


def device_shared_w2(cfg, layer=0, device="cuda"):
    return _device_normal(cfg, layer, "ws2", 0, (cfg["H"], cfg["I_s"]), device)


def nvfp4_matrix(cfg, layer, index, rows, cols, n_global=1):
    """A synthetic NVFP4 matrix (the checkpoint format of the routed experts):
    E2M1 codes uniform over all 16 codes, unpacked [rows, cols]; E4M3 block
    scale codes [rows, cols/16] uniform over 0x40..0x7E (values 2 .. 448);
    ``n_global`` fp32 second-level scales log-uniform around 2e-5, so that the
    values have the spread of N(0, 0.02) weights (block maxima ~1e-2 .. 6e-2)."""
    g = _rng(cfg, layer, "nvfp4", index)
    codes = g.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    bscales = g.integers(0x40, 0x7F, size=(rows, cols // 16)).astype(np.uint8)
    gscale = (2e-5 * np.exp(g.uniform(-0.5, 0.5, size=n_global))).astype(np.float32)
    return codes, bscales, gscale


def norm_weight(cfg, layer=0):
    """fp32 [H] weight of the pre-router RMSNorm: 1 + 0.1 N(0, 1)."""
    g = _rng(cfg, layer, "norm")
    return (1.0 + 0.1 * g.standard_normal(cfg["H"])).astype(np.float32)
