"""The block-sparse MoE layer written out plainly in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed (article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support
and optimization", section "MiniMax-M3.1 at a glance"; model card
"amd/MiniMax-M3.1-Flash-Quark-MXFP4", section "Model Overview"):

    logits[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e])        router, fp32 weights
    ids[t, :]    = the k experts with the largest logits
    w[t, j]      = softmax over the k selected logits
    xq[t]        = MXFP4(x[t])                                 dynamic activation quant
    g, u         = xq[t] . W13[e][n], xq[t] . W13[e][I + n]     E2M1 weights, E8M0 scales
    a            = MXFP4(silu(g) * u)
    d[t, j]      = a . W2[e]
    s[t]         = the same FFN with MXFP8 activations and weights (shared expert)
    y[t]         = bf16( r[t] + sum_j w[t, j] * d[t, j] + s[t] )

The arithmetic is fp64 throughout.  Where a floating-point value decides an
integer (the top-k choice, an activation code), the value is first rounded to
fp32, the precision the GPU kernels hold it in: router logits, and the g, u and
a of both FFNs.  Everything else stays fp64, so the oracle is exact up to fp64
rounding and the documented fp32 roundings.

Readings of points the pages leave open: softmax over fp32 router logits,
top-k, renormalise over the k chosen (ties between equal logits go to the lower
expert index; output in descending logit order); SwiGLU = silu(gate) * up with
gate rows first in W13; the shared expert is added with weight 1; an optional
residual is added in the same fp32/fp64 sum before the single bf16 rounding.
"""

import numpy as np

from . import mx


# ---------------------------------------------------------------------------
# Router and top-k
# ---------------------------------------------------------------------------

def router_logits(x, w_r, bias=None):
    """Router logits for activations ``x`` [T, H] (exact bf16 values, fp64)
    and fp32 router weights ``w_r`` [E, H] (fp64): x @ w_r^T (+ bias), in fp64,
    then rounded to fp32 (returned as fp64).  The router is kept in high
    precision (article, "MiniMax-M3.1 at a glance")."""
    l = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return mx.to_f32(l)


def select_topk(logits, k):
    """Per row, the k experts with the largest logits (4 of 128 in the model,
    article "MiniMax-M3.1 at a glance"); ties between equal logits go to the
    lower expert index; ids are listed in descending logit order.  Weights are
    the softmax over the chosen logits, which equals a softmax over all E
    followed by renormalisation over the k chosen."""
    logits = np.asarray(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        sel = order[:k]
        ids[t] = sel
        z = logits[t, sel]
        p = np.exp(z - z[0])
        w[t] = p / p.sum()
    return ids, w


# ---------------------------------------------------------------------------
# Token sort by expert
# ---------------------------------------------------------------------------

def align_sort(ids, num_experts, block_m):
    """Group the slots s = t*k + j by expert: a stable counting sort of the
    slots by ids[t, j].  Each expert's segment is padded to a multiple of
    block_m with the pad value T*k; experts with no slots own no block.

    Returns (sorted_slots, block_expert, expert_offsets, num_padded):
    sorted_slots [num_padded] int32, block_expert [num_padded / block_m]
    int32, expert_offsets [E + 1] int32 (exclusive scan of the unpadded
    counts), num_padded int."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    pad = T * k
    counts = np.zeros(num_experts, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_slots = []
    block_expert = []
    for e in range(num_experts):
        seg = [s for s in range(T * k) if flat[s] == e]
        if not seg:
            continue
        nblk = (len(seg) + block_m - 1) // block_m
        seg = seg + [pad] * (nblk * block_m - len(seg))
        sorted_slots.extend(seg)
        block_expert.extend([e] * nblk)
    return (np.asarray(sorted_slots, np.int32), np.asarray(block_expert, np.int32),
            offsets.astype(np.int32), len(sorted_slots))


# ---------------------------------------------------------------------------
# Layer weights
# ---------------------------------------------------------------------------

class Layer:
    """Quantized layer weights as unpacked element codes plus E8M0 scales.

    Routed expert e: ``w13_codes[e]`` [2I, H] (rows 0..I-1 gate, I..2I-1 up),
    ``w13_scales[e]`` [2I, H/32]; ``w2_codes[e]`` [H, I], ``w2_scales[e]``
    [H, I/32]; all MXFP4.  Shared expert (I_s > 0): ``ws13_*`` [2I_s, H],
    ``ws2_*`` [H, I_s], MXFP8.  Router: ``router_w`` [E, H] fp32 values,
    optional ``router_bias`` [E]."""

    def __init__(self, H, I, E, k, I_s, router_w, router_bias,
                 w13_codes, w13_scales, w2_codes, w2_scales,
                 ws13_codes=None, ws13_scales=None, ws2_codes=None, ws2_scales=None, shared_folded=False,
                 norm_weight=None, norm_eps=1e-6):
        self.H, self.I, self.E, self.k, self.I_s = H, I, E, k, I_s
        # norm_weight [H] (or None): the layer's input is the residual stream
        # h and the MoE runs on RMSNorm(h), see moe_layer
        self.norm_weight = None if norm_weight is None else np.asarray(norm_weight, np.float64)
        self.norm_eps = float(norm_eps)
        # shared_folded: expert E of the (E + 1)-expert table is the shared
        # expert in MXFP4, selected for every token with weight 1 (I_s is 0)
        self.shared_folded = shared_folded
        self.router_w = np.asarray(router_w, np.float64)
        self.router_bias = None if router_bias is None else np.asarray(router_bias, np.float64)
        self.w13_codes, self.w13_scales = w13_codes, w13_scales
        self.w2_codes, self.w2_scales = w2_codes, w2_scales
        self.ws13_codes, self.ws13_scales = ws13_codes, ws13_scales
        self.ws2_codes, self.ws2_scales = ws2_codes, ws2_scales


def quantize_layer(H, I, E, k, I_s, router_w, router_bias, w13, w2, ws13=None, ws2=None):
    """Static MX quantization of fp32 layer weights (routed experts to MXFP4,
    shared expert to MXFP8).  ``w13`` / ``w2`` are sequences (or callables
    e -> array) of per-expert fp32 arrays [2I, H] / [H, I]."""
    get13 = w13 if callable(w13) else (lambda e: w13[e])
    get2 = w2 if callable(w2) else (lambda e: w2[e])
    c13, s13, c2, s2 = [], [], [], []
    for e in range(E):
        c, s = mx.mx_quantize(np.asarray(get13(e), np.float64), "fp4")
        c13.append(c)
        s13.append(s)
        c, s = mx.mx_quantize(np.asarray(get2(e), np.float64), "fp4")
        c2.append(c)
        s2.append(s)
    sc = {}
    if I_s > 0:
        sc["ws13_codes"], sc["ws13_scales"] = mx.mx_quantize(np.asarray(ws13, np.float64), "fp8")
        sc["ws2_codes"], sc["ws2_scales"] = mx.mx_quantize(np.asarray(ws2, np.float64), "fp8")
    return Layer(H, I, E, k, I_s, router_w, router_bias, c13, s13, c2, s2, **sc)


class _Appended:
    """Sequence view: ``base`` (indexed by expert) with one more entry at E."""

    def __init__(self, base, E, extra):
        self.base, self.E, self.extra = base, E, extra

    def __getitem__(self, e):
        return self.extra if int(e) == self.E else self.base[e]


def fold_shared_expert(layer):
    """The layer with its MXFP8 shared expert re-quantized to MXFP4 and folded
    into the routed expert table as expert E, which every token selects with
    weight 1 (the AITER fused MoE "with the shared expert optionally folded
    into the expert table", article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0
    support and optimization", section "Serving with vLLM / What we
    Optimized"; re-quantization to MXFP4 as in vLLM PR #64273, section
    "Purpose").  Requires I_s == I (the table's experts share one shape)."""
    if layer.I_s != layer.I:
        raise ValueError("folding needs the shared expert's intermediate size to equal the routed one")
    c13, s13 = mx.requant_fp8_to_fp4(layer.ws13_codes, layer.ws13_scales)
    c2, s2 = mx.requant_fp8_to_fp4(layer.ws2_codes, layer.ws2_scales)
    E = layer.E
    return Layer(layer.H, layer.I, E, layer.k, 0, layer.router_w, layer.router_bias,
                 _Appended(layer.w13_codes, E, c13), _Appended(layer.w13_scales, E, s13),
                 _Appended(layer.w2_codes, E, c2), _Appended(layer.w2_scales, E, s2), shared_folded=True)


# ---------------------------------------------------------------------------
# Expert FFN (SwiGLU) on MX operands
# ---------------------------------------------------------------------------

def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def mx_ffn(x, w13_codes, w13_scales, w2_codes, w2_scales, fmt):
    """SwiGLU FFN of rows ``x`` [n, H] (exact input values, fp64) with MX
    weights of format ``fmt`` ("fp4" routed, "fp8" shared):

        xq = MX(x); g, u = xq . W13 gate / up rows (fp64, then fp32)
        a  = fp32(silu(g) * u); aq = MX(a); d = aq . W2 rows (fp64)

    Returns d [n, H] fp64 and, for inspection, the intermediates: the
    dequantized operands (xq, w13, aq, w2), g, u, a and the intermediate's
    codes and scales."""
    I = w13_codes.shape[0] // 2
    xc, xs = mx.mx_quantize(x, fmt)
    xq = mx.mx_dequantize(xc, xs, fmt)
    w13 = mx.mx_dequantize(w13_codes, w13_scales, fmt)
    gu = mx.to_f32(xq @ w13.T)
    g, u = gu[:, :I], gu[:, I:]
    a = mx.to_f32(silu(g) * u)
    ac, as_ = mx.mx_quantize(a, fmt)
    aq = mx.mx_dequantize(ac, as_, fmt)
    w2 = mx.mx_dequantize(w2_codes, w2_scales, fmt)
    d = aq @ w2.T
    return d, {"x": x, "x_codes": xc, "x_scales": xs, "g": g, "u": u, "a": a, "a_codes": ac, "a_scales": as_,
               "xq": xq, "w13": w13, "aq": aq, "w2": w2, "fmt": fmt}


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def rmsnorm(h, weight, eps):
    """RMSNorm of rows h [T, H] (fp64): h / sqrt(mean(h^2) + eps) * weight,
    the normalization in front of the router that mono decode fuses into the
    MoE launch (article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and
    optimization", section "Serving with vLLM / What we Optimized": "the
    RMSNorm and router").  The result is not rounded to bf16: inside one fused
    launch it goes straight to the router and the MX quantizers."""
    h = np.asarray(h, np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(weight, np.float64)[None, :]


def moe_layer(x_bits, layer, residual_bits=None, ids=None, on_ffn=None):
    """One MoE layer on bf16 rows ``x_bits`` [T, H] (uint16 patterns).

    ``ids`` may override the routing choice (used only where the top-k is a
    near-tie and another choice is equally valid); the weights are then the
    softmax over the given experts' logits, in the given order.  ``on_ffn``,
    if given, is called after each expert FFN as on_ffn(kind, e, rows, info)
    with kind "routed" (rows: the (t, j) pairs of expert e) or "shared" (e and
    rows None) and mx_ffn's intermediates; it changes nothing.  Returns a dict
    with ``y_bits`` (bf16 output patterns), ``y`` (fp64 before rounding),
    ``logits``, ``ids``, ``weights``, ``d`` [T, k, H], ``s`` [T, H]."""
    x = mx.bf16_bits_to_f64(x_bits)
    T, H = x.shape
    k = layer.k
    h_res = None
    if layer.norm_weight is not None:
        # the input is the residual stream h: the MoE runs on RMSNorm(h) and h
        # itself is added back (the fused residual); no separate residual
        if residual_bits is not None:
            raise ValueError("a layer with a pre-router norm adds its own input as the residual")
        h_res = x
        x = rmsnorm(x, layer.norm_weight, layer.norm_eps)
    logits = router_logits(x, layer.router_w, layer.router_bias)
    if ids is None:
        ids, w = select_topk(logits, k)
    else:
        ids = np.asarray(ids, np.int32)
        w = np.empty((T, k))
        for t in range(T):
            z = logits[t, ids[t]]
            p = np.exp(z - z.max())
            w[t] = p / p.sum()
    d = np.zeros((T, k, H))
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        rows = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == e]
        xt = np.stack([x[t] for t, _ in rows])
        de, info = mx_ffn(xt, layer.w13_codes[e], layer.w13_scales[e],
                          layer.w2_codes[e], layer.w2_scales[e], "fp4")
        if on_ffn is not None:
            on_ffn("routed", e, rows, info)
        for r, (t, j) in enumerate(rows):
            d[t, j] = de[r]
    s = np.zeros((T, H))
    if layer.I_s > 0:
        s, info = mx_ffn(x, layer.ws13_codes, layer.ws13_scales,
                         layer.ws2_codes, layer.ws2_scales, "fp8")
        if on_ffn is not None:
            on_ffn("shared", None, None, info)
    elif layer.shared_folded:
        # expert E, selected by every token with weight 1: its output is added
        # like the shared expert's, after the routed experts
        E = layer.E
        s, info = mx_ffn(x, layer.w13_codes[E], layer.w13_scales[E],
                         layer.w2_codes[E], layer.w2_scales[E], "fp4")
        if on_ffn is not None:
            on_ffn("shared", E, None, info)
    y = np.einsum("tj,tjh->th", w, d) + s
    if residual_bits is not None:
        y = y + mx.bf16_bits_to_f64(residual_bits)
    if h_res is not None:
        y = y + h_res
    return {"y_bits": mx.round_to_bf16_bits(y), "y": y, "logits": logits,
            "ids": ids, "weights": w, "d": d, "s": s}


def activation_quant(x_bits, fmt="fp4"):
    """Dynamic MX quantization of bf16 rows (the model card's "Routed-expert
    activation quantization: OCP MXFP4, Dynamic"): returns packed codes
    [rows, cols/2] for FP4 (or [rows, cols] for FP8) and scales [rows, cols/32]."""
    codes, scales = mx.mx_quantize(mx.bf16_bits_to_f64(x_bits), fmt)
    if fmt == "fp4":
        codes = mx.pack_fp4(codes)
    return codes, scales
