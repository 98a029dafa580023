"""Shared test plumbing: seeded layers for the GPU path and the oracle (each
quantizes the same fp32 draws itself), and the comparison rules.

Comparison rules (written here once, used by every parity test):
* integer / byte results (codes, scales, ids, sorted order): bit-exact;
* router logits: within the fp32 error bound of the kernel's documented
  summation (a 48-term sequential FMA chain per lane, then a 6-level
  butterfly, then the bias): |l_gpu - l| <= gamma_56 * sum_h |x_h w_h| + 2u|l|,
  u = 2^-24, gamma_n = n u / (1 - n u);
* top-k ids: bit-exact for every row whose top-k is decided by more than twice
  that bound; a row with a closer call must hold a valid top-k of the GPU's own
  logits (several answers are correct there);
* layer output: per row max|y - y_ref| / max|y_ref| <= 2e-2, the stated
  tolerance, on every layer; and every element within its own derived bound
  (``LayerBound``): the kernels' fp32 sums round, and where a gate/up value
  lies that close to a rounding boundary of the re-quantized intermediate
  (E2M1 routed, E4M3 shared) its code may differ by a step, which moves the
  down output by that step times the weight column.  The bound follows this
  through every step of the layer, element by element.  The share of
  elements within one bf16 ulp of the oracle is printed as a diagnostic.
"""

import concurrent.futures

import numpy as np

from mxfp4_moe_decode_amd import synth
from oracle import moe, mx

U32 = 2.0 ** -24
SILU_SLOPE = 1.1  # max over z of |d/dz z*sigmoid(z)| = 1.0998...


def gamma(n):
    return n * U32 / (1 - n * U32)


class LazyExperts:
    """Sequence of oracle-quantized expert matrices, generated on demand from
    the seeded generator (the oracle only ever touches the experts it uses)."""

    def __init__(self, make, fmt="fp4"):
        self.make, self.fmt, self.cache = make, fmt, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = mx.mx_quantize(np.asarray(self.make(e), np.float64), self.fmt)
        return self.cache[e]


def prefetch(ol, experts, threads=16):
    """Quantize the given experts of an oracle layer ahead of use, several at
    a time (numpy releases the GIL in the heavy array work)."""
    todo = sorted({int(e) for e in experts if int(e) < ol.E})  # a folded expert E is held already
    base13 = getattr(ol.w13_codes, "base", ol.w13_codes)
    base2 = getattr(ol.w2_codes, "base", ol.w2_codes)
    w13, w2 = base13.lazy, base2.lazy
    host13 = {e: w13.make(e) for e in todo if e not in w13.cache}
    host2 = {e: w2.make(e) for e in todo if e not in w2.cache}

    def q(item):
        lazy, e, a = item
        return lazy, e, mx.mx_quantize(np.asarray(a, np.float64), lazy.fmt)

    items = [(w13, e, a) for e, a in host13.items()] + [(w2, e, a) for e, a in host2.items()]
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        for lazy, e, res in ex.map(q, items):
            lazy.cache[e] = res


def oracle_experts(x_bits, ol, ids=None):
    """Experts the oracle's routing (or the given ids) selects for x."""
    if ids is None:
        x = mx.bf16_bits_to_f64(x_bits)
        if ol.norm_weight is not None:
            x = moe.rmsnorm(x, ol.norm_weight, ol.norm_eps)
        logits = moe.router_logits(x, ol.router_w, ol.router_bias)
        ids, _ = moe.select_topk(logits, ol.k)
    return np.unique(np.asarray(ids))


class _Part:
    def __init__(self, lazy, idx):
        self.lazy, self.idx = lazy, idx

    def __getitem__(self, e):
        return self.lazy[e][self.idx]


def oracle_layer(cfg, layer=0, device_weights=True):
    """oracle.moe.Layer for workload ``cfg`` (experts quantized lazily).  With
    ``device_weights`` the fp32 draws are the device-generated ones (read
    back to the host), as used by ``gpu_layer``."""
    if device_weights:
        g13 = lambda e: synth.device_expert_w13(cfg, layer, e).cpu().numpy()
        g2 = lambda e: synth.device_expert_w2(cfg, layer, e).cpu().numpy()
        gs13 = lambda: synth.device_shared_w13(cfg, layer).cpu().numpy()
        gs2 = lambda: synth.device_shared_w2(cfg, layer).cpu().numpy()
    else:
        g13 = lambda e: synth.expert_w13(cfg, layer, e)
        g2 = lambda e: synth.expert_w2(cfg, layer, e)
        gs13 = lambda: synth.shared_w13(cfg, layer)
        gs2 = lambda: synth.shared_w2(cfg, layer)
    w13 = LazyExperts(g13)
    w2 = LazyExperts(g2)
    kw = {}
    if cfg["I_s"]:
        kw["ws13_codes"], kw["ws13_scales"] = mx.mx_quantize(gs13().astype(np.float64), "fp8")
        kw["ws2_codes"], kw["ws2_scales"] = mx.mx_quantize(gs2().astype(np.float64), "fp8")
    return moe.Layer(cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"],
                     synth.router_weights(cfg, layer), synth.router_bias(cfg, layer),
                     _Part(w13, 0), _Part(w13, 1), _Part(w2, 0), _Part(w2, 1), **kw)


def gpu_layer(cfg, layer=0, device="cuda"):
    """binding.MoELayer for workload ``cfg`` from the device-generated draws,
    quantized by the library."""
    from mxfp4_moe_decode_amd import binding
    sh = {}
    if cfg["I_s"]:
        sh = dict(shared_w13=synth.device_shared_w13(cfg, layer, device),
                  shared_w2=synth.device_shared_w2(cfg, layer, device))
    return binding.MoELayer.from_fp32(
        cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"], synth.router_weights(cfg, layer),
        synth.router_bias(cfg, layer), lambda e: synth.device_expert_w13(cfg, layer, e, device),
        lambda e: synth.device_expert_w2(cfg, layer, e, device), device=device, **sh)


def logit_bound(x_bits, w_r, logits_ref, x=None, x_rel=0.0):
    """Per-(row, expert) bound on |l_gpu - l| for the kernel's fp32 order.
    ``x`` (fp64, default the bf16 rows) is the router input; ``x_rel`` bounds
    the relative error of the GPU's copy of it (the fp32 pre-router norm)."""
    xa = np.abs(mx.bf16_bits_to_f64(x_bits) if x is None else np.asarray(x, np.float64))
    s = xa @ np.abs(np.asarray(w_r, np.float64)).T
    return (gamma(56) + x_rel) * s + 2 * U32 * np.abs(logits_ref)


def norm_rel_error(H):
    """Relative error bound of the GPU's normalized x = (h * r) * g against the
    exact one: the fp32 sum of squares (positive terms, at most H/256 * 4 + 6
    roundings each), the division by H, the epsilon add, the square root and
    the reciprocal (one rounding each, the square root halving the sum's
    relative error), then the two products."""
    n = 4 * ((H + 255) // 256) + 6
    return gamma(n) / 2 + 6 * U32


def check_logits(l_gpu, l_ref, bound):
    diff = np.abs(np.asarray(l_gpu, np.float64) - l_ref)
    assert np.all(diff <= bound), f"logit error {diff.max()} above bound {bound[diff > bound].min()}"


def check_topk(ids_gpu, l_gpu, l_ref, bound, k):
    """Returns the number of rows compared bit-exactly."""
    ids_gpu = np.asarray(ids_gpu)
    exact = 0
    T, E = l_ref.shape
    ids_ref, _ = moe.select_topk(l_ref, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l_ref[t, e], e))
        lv = l_ref[t, order]
        eps = 2 * bound[t].max()
        decided = lv[k - 1] - lv[k] > eps and all(lv[j] - lv[j + 1] > eps for j in range(k - 1))
        if decided:
            assert list(ids_gpu[t]) == list(ids_ref[t]), f"row {t}: {ids_gpu[t]} vs {ids_ref[t]}"
            exact += 1
        else:
            own, _ = moe.select_topk(np.asarray(l_gpu[t:t + 1], np.float64), k)
            assert list(ids_gpu[t]) == list(own[0]), f"row {t}: not a top-k of the GPU's own logits"
    return exact


def check_layer_output(y_bits, ref, tol=2e-2, ulp_frac=None):
    """``ref`` is the oracle's output dict.  Returns (max row error, fraction
    of elements within one bf16 ulp); ``ulp_frac`` enforces a minimum share."""
    y = mx.bf16_bits_to_f64(np.asarray(y_bits).astype(np.uint16))
    yr = ref["y"]
    row_err = np.abs(y - yr).max(axis=1) / np.maximum(np.abs(yr).max(axis=1), 1e-30)
    assert np.all(row_err <= tol), f"row errors {row_err}"
    yb = mx.bf16_bits_to_f64(ref["y_bits"])
    _, ex = np.frexp(np.maximum(np.abs(yb), 2.0 ** -126))
    ulp = np.ldexp(1.0, ex.astype(np.int64) - 8)
    within = float(np.mean(np.abs(y - yb) <= ulp))
    if ulp_frac is not None:
        assert within >= ulp_frac, f"only {within:.4f} of elements within one bf16 ulp"
    return float(row_err.max()), within


# ---------------------------------------------------------------------------
# Derived element-wise bound on |y_gpu - y_oracle|
# ---------------------------------------------------------------------------

def gemm_roundings(K):
    """Most fp32 roundings one product passes through in the kernels' dot
    product over K: inside a 16x16x128 scaled matrix instruction (at most 128,
    as if it summed sequentially), one per later instruction of its K-chunk
    chain, and one per chunk sum added after it (NC = 4, 2 or 1 chunks)."""
    kt = K // 128
    nc = 4 if kt % 4 == 0 else (2 if kt % 2 == 0 else 1)
    return 128 + kt // nc + nc


def requant_deviation(a, da, fmt):
    """Largest |MX(a') - MX(a)| (dequantized, element by element) over every
    a' with |a' - a| <= da, where MX(a') may use any block scale that the
    block maximum of such a' can give.  The element rounding is monotone, so
    the interval ends decide it."""
    n, I = a.shape
    nb = I // mx.BLOCK
    ab = a.reshape(n, nb, mx.BLOCK)
    db = da.reshape(n, nb, mx.BLOCK)
    e_o = mx.shared_exponent(np.abs(ab).max(axis=-1), fmt)
    e_lo = mx.shared_exponent(np.maximum(np.abs(ab) - db, 0.0).max(axis=-1), fmt)
    e_hi = mx.shared_exponent((np.abs(ab) + db).max(axis=-1), fmt)
    aq = mx.element_value(mx.round_to_element(np.ldexp(ab, -e_o[..., None]), fmt), fmt)
    aq = np.ldexp(aq, e_o[..., None])
    dev = np.zeros_like(ab)
    for shift in (-1, 0, 1):
        e = e_o + shift
        ok = ((e >= e_lo) & (e <= e_hi))[..., None]
        for end in (ab - db, ab + db):
            v = mx.element_value(mx.round_to_element(np.ldexp(end, -e[..., None]), fmt), fmt)
            v = np.ldexp(v, e[..., None])
            dev = np.where(ok, np.maximum(dev, np.abs(v - aq)), dev)
    return dev.reshape(n, I)


def ffn_deviation(info, fmt, x_rel=0.0):
    """Bound on |d_gpu - d_oracle| [n, H] for one SwiGLU FFN of the oracle
    (``info`` from oracle.moe.mx_ffn): with ``x_rel`` > 0 (the GPU's x has
    that relative error), the MX codes of x that can differ; fp32 rounding of
    the gate/up sums, of SwiGLU (the hardware exp2 and reciprocal, one ulp
    each, after an exponent -g log2 e rounded twice: (2|g| + 7) u relative,
    taken as (2|g| + 16) u, plus 2^-120 where the exponential overflows) and
    the oracle's own fp32 roundings of g, u, a, then the re-quantization steps
    that can follow, then the down product's rounding."""
    xq, w13, g, u, a, aq, w2 = (info[k] for k in ("xq", "w13", "g", "u", "a", "aq", "w2"))
    I = g.shape[1]
    H = xq.shape[1]
    w13a = np.abs(w13)
    dxq = np.zeros_like(xq)
    if x_rel > 0:
        x = np.asarray(info["x"], np.float64)
        dxq = requant_deviation(x, x_rel * np.abs(x), fmt)
    s13 = (np.abs(xq) + dxq) @ w13a.T
    e13 = dxq @ w13a.T
    dg = gamma(gemm_roundings(H)) * s13[:, :I] + e13[:, :I] + 2 * U32 * np.abs(g)
    du = gamma(gemm_roundings(H)) * s13[:, I:] + e13[:, I:] + 2 * U32 * np.abs(u)
    sil = g / (1.0 + np.exp(-g))
    da = (SILU_SLOPE * np.abs(u) * dg + np.abs(sil) * du + SILU_SLOPE * dg * du
          + (2 * np.abs(g) + 16) * U32 * np.abs(a) + 2.0 ** -120)
    daq = requant_deviation(a, da, fmt)
    w2a = np.abs(w2)
    return daq @ w2a.T + gamma(gemm_roundings(I)) * ((np.abs(aq) + daq) @ w2a.T)


class LayerBound:
    """Collects per-FFN deviations through the oracle's ``on_ffn`` hook and
    turns them into a bound on every output element."""

    W_RTOL, W_ATOL = 1e-5, 1e-6  # the routing-weight tolerance the tests assert

    def __init__(self, T, k, H, x_rel=0.0):
        self.dd = np.zeros((T, k, H))
        self.ds = np.zeros((T, H))
        self.x_rel = x_rel

    def __call__(self, kind, e, rows, info):
        if kind == "routed":
            dev = ffn_deviation(info, "fp4", self.x_rel)
            for r, (t, j) in enumerate(rows):
                self.dd[t, j] = dev[r]
        else:
            self.ds[:] = ffn_deviation(info, info["fmt"], self.x_rel)

    def bound(self, ref, residual_bits=None):
        w, d, s = ref["weights"], ref["d"], ref["s"]
        k = w.shape[1]
        aw = np.abs(w)[:, :, None]
        dw = (self.W_RTOL * np.abs(w) + self.W_ATOL)[:, :, None]
        r = np.abs(mx.bf16_bits_to_f64(residual_bits)) if residual_bits is not None else 0.0
        B = (aw * self.dd + dw * (np.abs(d) + self.dd)).sum(axis=1) + self.ds
        terms = (aw * (np.abs(d) + self.dd)).sum(axis=1) + np.abs(s) + self.ds + r
        B = B + gamma(k + 2) * terms
        # the single rounding to bf16 (8 significant bits): half an ulp, at
        # most 2^-8 relative, or half the smallest subnormal step
        return B + 2.0 ** -8 * (np.abs(ref["y"]) + B) + 2.0 ** -134


def check_elementwise(y_bits, ref, bound):
    """Every element within its bound; returns the largest ratio |err| / bound."""
    y = mx.bf16_bits_to_f64(np.asarray(y_bits).astype(np.uint16))
    err = np.abs(y - ref["y"])
    bad = err > bound
    if np.any(bad):
        t, h = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} elements beyond the derived bound, first at row {t} column {h}: "
                             f"|err| {err[t, h]:.3e} > bound {bound[t, h]:.3e} (y_ref {ref['y'][t, h]:.4e})")
    return float((err / bound).max())


def oracle_with_bound(x_bits, layer, residual_bits=None, ids=None):
    """Oracle layer output plus the element-wise bound of its comparison."""
    T = np.asarray(x_bits).shape[0]
    normed = layer.norm_weight is not None
    lb = LayerBound(T, layer.k, layer.H, norm_rel_error(layer.H) if normed else 0.0)
    ref = moe.moe_layer(x_bits, layer, residual_bits, ids=ids, on_ffn=lb)
    # with the norm the layer adds its own input back
    return ref, lb.bound(ref, x_bits if normed else residual_bits)


def compare_with_oracle(cfg, gl, ol, x_bits, y, ids=None, w=None, residual_bits=None, layer=0,
                        router_w=None, label=""):
    """The full comparison of one layer call with the oracle: routing ids
    bit-exact where decided (else a valid top-k of the GPU's own logits, and
    the oracle is evaluated on the GPU's choice), routing weights within
    1e-5, the per-row 2e-2 tolerance and every element within its derived
    bound.  ``ids`` / ``w`` are the call's routing outputs (None: taken from
    the standalone router).  Returns the oracle's result."""
    import torch
    from mxfp4_moe_decode_amd import binding

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    prefetch(ol, oracle_experts(x_bits, ol))
    ids_r, w_r, logits = binding.moe_router_topk(gl, dev(x_bits), want_logits=True)
    torch.cuda.synchronize()
    ids_r, w_r, logits = ids_r.cpu().numpy(), w_r.cpu().numpy(), logits.cpu().numpy()
    if ids is None:
        ids, w = ids_r, w_r
    else:
        assert np.array_equal(ids, ids_r), "the call's routing differs from the standalone router's"
        assert np.array_equal(w, w_r), "the call's routing weights differ from the standalone router's"
    xr = mx.bf16_bits_to_f64(x_bits)
    x_rel = 0.0
    if ol.norm_weight is not None:
        xr = moe.rmsnorm(xr, ol.norm_weight, ol.norm_eps)
        x_rel = norm_rel_error(ol.H)
    ref_logits = moe.router_logits(xr, ol.router_w, ol.router_bias)
    wr = synth.router_weights(cfg, layer) if router_w is None else router_w
    bound_l = logit_bound(x_bits, wr, ref_logits, x=xr, x_rel=x_rel)
    check_logits(logits, ref_logits, bound_l)
    ref_ids, _ = moe.select_topk(ref_logits, ol.k)
    use_ids = None
    if not np.array_equal(ids, ref_ids):
        check_topk(ids, logits, ref_logits, bound_l, ol.k)
        use_ids = ids
        prefetch(ol, oracle_experts(x_bits, ol, ids))
    ref, bound = oracle_with_bound(x_bits, ol, residual_bits, ids=use_ids)
    np.testing.assert_allclose(w, ref["weights"], rtol=LayerBound.W_RTOL, atol=LayerBound.W_ATOL)
    err, within = check_layer_output(y, ref)
    ratio = check_elementwise(y, ref, bound)
    print(f"[oracle] {cfg['name']} {label} T={np.asarray(x_bits).shape[0]}: max row err {err:.3e}, "
          f"within 1 ulp {within:.4f}, largest err/bound {ratio:.3f}", flush=True)
    return ref
