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
  tolerance, on every layer.  Stricter, for layers of routed experts alone:
  99.9% of elements within one bf16 ulp of the oracle's correctly rounded
  value, since their MXFP4 partial sums are exact in fp32 and only the final
  rounding differs.  With the MXFP8 shared expert no element-share check is
  made: its fp32 sums round, and where one lands within that rounding of an
  E4M3 boundary of the re-quantized intermediate the code differs by one step
  and the whole shared-output row moves by a few 1e-3 of its scale (within the
  2e-2 tolerance); the share is printed as a diagnostic.
"""

import numpy as np

from mxfp4_moe_decode_amd import synth
from oracle import moe, mx

U32 = 2.0 ** -24


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


def logit_bound(x_bits, w_r, logits_ref):
    """Per-(row, expert) bound on |l_gpu - l| for the kernel's fp32 order."""
    x = np.abs(mx.bf16_bits_to_f64(x_bits))
    s = x @ np.abs(np.asarray(w_r, np.float64)).T
    return gamma(56) * s + 2 * U32 * np.abs(logits_ref)


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
