"""Thin Python binding of libmxmoe.so (ctypes).  Argument marshalling only:
torch provides device memory and the current stream; every computation runs in
the library's HIP kernels.  Importing works without a GPU; calling a compute
function needs the built library and a GPU, and fails loudly otherwise."""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxmoe.so")

MX_FMT = {"fp4": 0, "fp8": 1}
MX_LAYOUT = {"rowmajor": 0, "tiled": 1}

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARGUMENT", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE_TOO_SMALL", -4: "MOE_ERR_HIP", -5: "MOE_ERR_TIMEOUT"}

EXPORTS = [
    "mx_codes_bytes", "mx_scales_bytes", "mx_quantize_weights", "mx_requant_fp8_to_fp4", "mx_requant_nvfp4_to_fp4",
    "mxfp4_quant_act",
    "moe_router_topk", "moe_align_sort_capacity", "moe_align_sort_workspace_bytes", "moe_align_sort",
    "moe_workspace_bytes", "moe_workspace_init", "fused_moe_mxfp4_decode", "fused_moe_mxfp4_decode_noalloc",
    "fused_moe_mxfp4_grouped", "fused_moe_mxfp4_grouped_timed",
    "moe_decode_status", "moe_decode_trace", "moe_status_string",
]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({_lib_or_none_string(status)})")


class MoeLayerC(ctypes.Structure):
    """moe_layer_t of mxmoe.h."""
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("ws13", ctypes.c_void_p), ("ws13_scale", ctypes.c_void_p),
        ("ws2", ctypes.c_void_p), ("ws2_scale", ctypes.c_void_p),
        ("shared_folded", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
    ]


_lib = None


def load():
    """Load the built library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mxfp4_moe_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
    LP = ctypes.POINTER(MoeLayerC)
    sig = {
        "mx_codes_bytes": (Z, [I, I, I, I]),
        "mx_scales_bytes": (Z, [I, I, I]),
        "mx_quantize_weights": (S, [P, I, I, I, I, P, P, P]),
        "mx_requant_fp8_to_fp4": (S, [P, P, I, I, I, P, P, P]),
        "mx_requant_nvfp4_to_fp4": (S, [P, P, P, I, I, I, I, P, P, P]),
        "mxfp4_quant_act": (S, [P, I, I, P, P, P]),
        "moe_router_topk": (S, [LP, P, I, P, P, P, P]),
        "moe_align_sort_capacity": (Z, [I, I, I, I]),
        "moe_align_sort_workspace_bytes": (Z, [I, I, I]),
        "moe_align_sort": (S, [P, I, I, I, I, P, P, P, P, P, Z, P]),
        "moe_workspace_bytes": (Z, [LP, I, I]),
        "moe_workspace_init": (S, [P, Z, P]),
        "fused_moe_mxfp4_decode": (S, [LP, P, I, P, P, P, Z, P, P, P]),
        "fused_moe_mxfp4_decode_noalloc": (S, [LP, P, I, P, P, P, P, P]),
        "fused_moe_mxfp4_grouped": (S, [LP, P, I, P, P, P, Z, P]),
        "fused_moe_mxfp4_grouped_timed": (S, [LP, P, I, P, P, P, Z, P, P]),
        "moe_decode_status": (S, [P, Z]),
        "moe_decode_trace": (I, [LP, P, Z, P, Z]),
        "moe_status_string": (ctypes.c_char_p, [S]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _lib_or_none_string(status):
    try:
        return load().moe_status_string(status).decode()
    except Exception:
        return "?"


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA tensors")


# --------------------------------------------------------------------------- quantization

def mx_codes_bytes(rows, cols, fmt="fp4", layout="tiled"):
    return load().mx_codes_bytes(rows, cols, MX_FMT[fmt], MX_LAYOUT[layout])


def mx_scales_bytes(rows, cols, layout="tiled"):
    return load().mx_scales_bytes(rows, cols, MX_LAYOUT[layout])


def mx_quantize_weights(w, fmt="fp4", layout="tiled", codes=None, scales=None):
    """Static MX quantization of an fp32 [rows, cols] CUDA tensor.  Returns
    (codes, scales) uint8 tensors (flat for the tiled layout)."""
    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    rows, cols = w.shape
    nc, ns = mx_codes_bytes(rows, cols, fmt, layout), mx_scales_bytes(rows, cols, layout)
    if nc == 0 or ns == 0:
        raise ValueError(f"unsupported shape {tuple(w.shape)} for layout {layout}")
    if codes is None:
        codes = torch.empty(nc, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(ns, dtype=torch.uint8, device=w.device)
    _check("mx_quantize_weights", load().mx_quantize_weights(
        _ptr(w), rows, cols, MX_FMT[fmt], MX_LAYOUT[layout], _ptr(codes), _ptr(scales), _stream()))
    if layout == "rowmajor":
        codes = codes.view(rows, cols // 2 if fmt == "fp4" else cols)
        scales = scales.view(rows, cols // 32)
    return codes, scales


def mx_requant_fp8_to_fp4(codes8, scales8, rows, cols, layout="tiled", codes4=None, scales4=None):
    """MXFP8 matrix (codes, scales uint8 CUDA tensors) re-quantized to MXFP4
    along the same blocks.  Returns (codes4, scales4)."""
    _need_cuda(codes8, scales8)
    nc, ns = mx_codes_bytes(rows, cols, "fp4", layout), mx_scales_bytes(rows, cols, layout)
    if nc == 0 or ns == 0:
        raise ValueError(f"unsupported shape {(rows, cols)} for layout {layout}")
    if codes4 is None:
        codes4 = torch.empty(nc, dtype=torch.uint8, device=codes8.device)
    if scales4 is None:
        scales4 = torch.empty(ns, dtype=torch.uint8, device=codes8.device)
    _check("mx_requant_fp8_to_fp4", load().mx_requant_fp8_to_fp4(
        _ptr(codes8), _ptr(scales8), rows, cols, MX_LAYOUT[layout], _ptr(codes4), _ptr(scales4), _stream()))
    if layout == "rowmajor":
        codes4, scales4 = codes4.view(rows, cols // 2), scales4.view(rows, cols // 32)
    return codes4, scales4


def mx_requant_nvfp4_to_fp4(codes, block_scales, global_scales, rows_per_scale, layout="tiled",
                            codes4=None, scales4=None):
    """NVFP4 matrix (packed codes [rows, cols/2], E4M3 block scales [rows,
    cols/16] uint8, fp32 global scales, CUDA tensors) re-quantized to MXFP4.
    Returns (codes4, scales4)."""
    _need_cuda(codes, block_scales, global_scales)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    nc, ns = mx_codes_bytes(rows, cols, "fp4", layout), mx_scales_bytes(rows, cols, layout)
    if nc == 0 or ns == 0:
        raise ValueError(f"unsupported shape {(rows, cols)} for layout {layout}")
    if codes4 is None:
        codes4 = torch.empty(nc, dtype=torch.uint8, device=codes.device)
    if scales4 is None:
        scales4 = torch.empty(ns, dtype=torch.uint8, device=codes.device)
    _check("mx_requant_nvfp4_to_fp4", load().mx_requant_nvfp4_to_fp4(
        _ptr(codes), _ptr(block_scales), _ptr(global_scales), rows_per_scale, rows, cols, MX_LAYOUT[layout],
        _ptr(codes4), _ptr(scales4), _stream()))
    if layout == "rowmajor":
        codes4, scales4 = codes4.view(rows, cols // 2), scales4.view(rows, cols // 32)
    return codes4, scales4


def mxfp4_quant_act(x):
    """Dynamic MXFP4 quantization of bf16 [rows, cols]: (codes [rows, cols/2],
    scales [rows, cols/32]) uint8."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    rows, cols = x.shape
    codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device)
    _check("mxfp4_quant_act", load().mxfp4_quant_act(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


# --------------------------------------------------------------------------- layer weights

class MoELayer:
    """Device weights of one layer in the library's tiled MX layout."""

    def __init__(self, hidden, inter, num_experts, top_k, shared_inter, router_w, router_bias,
                 w13, w13_scale, w2, w2_scale, ws13=None, ws13_scale=None, ws2=None, ws2_scale=None,
                 shared_folded=False, norm_weight=None, norm_eps=1e-6):
        self.hidden, self.inter, self.num_experts, self.top_k, self.shared_inter = (
            hidden, inter, num_experts, top_k, shared_inter)
        self.shared_folded = bool(shared_folded)
        self.norm_weight, self.norm_eps = norm_weight, float(norm_eps)
        self.router_w, self.router_bias = router_w, router_bias
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        self.ws13, self.ws13_scale, self.ws2, self.ws2_scale = ws13, ws13_scale, ws2, ws2_scale
        self._c = MoeLayerC(hidden, inter, num_experts, top_k, shared_inter,
                            router_w.data_ptr(), router_bias.data_ptr() if router_bias is not None else None,
                            w13.data_ptr(), w13_scale.data_ptr(), w2.data_ptr(), w2_scale.data_ptr(),
                            ws13.data_ptr() if ws13 is not None else None,
                            ws13_scale.data_ptr() if ws13_scale is not None else None,
                            ws2.data_ptr() if ws2 is not None else None,
                            ws2_scale.data_ptr() if ws2_scale is not None else None, int(self.shared_folded),
                            norm_weight.data_ptr() if norm_weight is not None else None, self.norm_eps)

    @property
    def c(self):
        return ctypes.byref(self._c)

    @classmethod
    def from_fp32(cls, hidden, inter, num_experts, top_k, shared_inter, router_w, router_bias,
                  expert_w13, expert_w2, shared_w13=None, shared_w2=None, device="cuda", fold_shared=False):
        """Quantize fp32 weights on the device.  ``expert_w13(e)`` /
        ``expert_w2(e)`` return the fp32 [2I, H] / [H, I] matrices of expert e
        (host arrays or device tensors); ``router_w`` [E, H]; ``router_bias``
        [E] or None; shared weights [2I_s, H] / [H, I_s] or None.  With
        ``fold_shared`` the shared expert is quantized to MXFP8, re-quantized
        to MXFP4 and stored as expert E of an (E + 1)-expert table."""
        H, I, E, Is = hidden, inter, num_experts, shared_inter
        dev = torch.device(device)
        if fold_shared and Is != I:
            raise ValueError("folding needs the shared intermediate size to equal the routed one")
        n_tab = E + 1 if fold_shared else E

        def dev_f32(a):
            return torch.as_tensor(a, dtype=torch.float32).to(dev).contiguous()

        c13, s13 = mx_codes_bytes(2 * I, H, "fp4"), mx_scales_bytes(2 * I, H)
        c2, s2 = mx_codes_bytes(H, I, "fp4"), mx_scales_bytes(H, I)
        w13 = torch.empty(n_tab * c13, dtype=torch.uint8, device=dev)
        w13s = torch.empty(n_tab * s13, dtype=torch.uint8, device=dev)
        w2 = torch.empty(n_tab * c2, dtype=torch.uint8, device=dev)
        w2s = torch.empty(n_tab * s2, dtype=torch.uint8, device=dev)
        for e in range(E):
            mx_quantize_weights(dev_f32(expert_w13(e)), "fp4", "tiled",
                                w13[e * c13:(e + 1) * c13], w13s[e * s13:(e + 1) * s13])
            mx_quantize_weights(dev_f32(expert_w2(e)), "fp4", "tiled",
                                w2[e * c2:(e + 1) * c2], w2s[e * s2:(e + 1) * s2])
        sh = {}
        rb = None if router_bias is None else dev_f32(router_bias)
        if Is > 0:
            q13, q13s = mx_quantize_weights(dev_f32(shared_w13), "fp8", "tiled")
            q2, q2s = mx_quantize_weights(dev_f32(shared_w2), "fp8", "tiled")
            if fold_shared:
                mx_requant_fp8_to_fp4(q13, q13s, 2 * I, H, "tiled", w13[E * c13:], w13s[E * s13:])
                mx_requant_fp8_to_fp4(q2, q2s, H, I, "tiled", w2[E * c2:], w2s[E * s2:])
                return cls(H, I, E, top_k, 0, dev_f32(router_w), rb, w13, w13s, w2, w2s, shared_folded=True)
            sh = dict(ws13=q13, ws13_scale=q13s, ws2=q2, ws2_scale=q2s)
        return cls(H, I, E, top_k, Is, dev_f32(router_w), rb, w13, w13s, w2, w2s, **sh)

    def with_norm(self, weight, eps=1e-6):
        """The same layer with the pre-router RMSNorm fused in (``weight``: an
        fp32 [H] CUDA tensor): its input is then the residual stream."""
        return MoELayer(self.hidden, self.inter, self.num_experts, self.top_k, self.shared_inter, self.router_w,
                        self.router_bias, self.w13, self.w13_scale, self.w2, self.w2_scale, self.ws13,
                        self.ws13_scale, self.ws2, self.ws2_scale, self.shared_folded, weight.contiguous(), eps)

    def folded_from(self, fp4_13, fp4_13s, fp4_2, fp4_2s):
        """A folded-shared copy of this layer sharing its routed weights:
        the routed tables are copied into (E + 1)-expert tables and expert E
        is set from the given MXFP4 tiled shared-expert matrices."""
        E = self.num_experts
        cat = lambda a, b: torch.cat([a, b.reshape(-1)]).contiguous()
        return MoELayer(self.hidden, self.inter, E, self.top_k, 0, self.router_w, self.router_bias,
                        cat(self.w13, fp4_13), cat(self.w13_scale, fp4_13s), cat(self.w2, fp4_2),
                        cat(self.w2_scale, fp4_2s), shared_folded=True, norm_weight=self.norm_weight,
                        norm_eps=self.norm_eps)


# --------------------------------------------------------------------------- router / sort

def moe_router_topk(layer, x, want_logits=False):
    _need_cuda(x)
    T = x.shape[0]
    ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=x.device)
    w = torch.empty(T, layer.top_k, dtype=torch.float32, device=x.device)
    logits = torch.empty(T, layer.num_experts, dtype=torch.float32, device=x.device) if want_logits else None
    _check("moe_router_topk", load().moe_router_topk(layer.c, _ptr(x), T, _ptr(logits), _ptr(ids), _ptr(w), _stream()))
    return (ids, w, logits) if want_logits else (ids, w)


def moe_align_sort(topk_ids, num_experts, block_m):
    _need_cuda(topk_ids)
    T, k = topk_ids.shape
    lib = load()
    cap = lib.moe_align_sort_capacity(T, k, num_experts, block_m)
    wsb = lib.moe_align_sort_workspace_bytes(T, k, num_experts)
    if cap == 0 or wsb == 0:
        raise ValueError("invalid align_sort arguments")
    dev = topk_ids.device
    sorted_slots = torch.empty(cap, dtype=torch.int32, device=dev)
    block_expert = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    num_padded = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check("moe_align_sort", lib.moe_align_sort(
        _ptr(topk_ids), T, k, num_experts, block_m, _ptr(sorted_slots), _ptr(block_expert),
        _ptr(offsets), _ptr(num_padded), _ptr(ws), wsb, _stream()))
    return sorted_slots, block_expert, offsets, num_padded


# --------------------------------------------------------------------------- fused layer

def moe_workspace_bytes(layer, T, path):
    return load().moe_workspace_bytes(layer.c, T, path)


def decode_workspace(layer, device="cuda", max_rows=64):
    """A zero-initialized workspace for fused_moe_mxfp4_decode, for steps of
    up to ``max_rows`` rows (16: mono decode steps; 64: also the wide steps)."""
    n = moe_workspace_bytes(layer, max_rows, 0)
    if n == 0:
        raise ValueError("invalid layer")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check("moe_workspace_init", load().moe_workspace_init(_ptr(ws), n, _stream()))
    return ws


def fused_moe_mxfp4_decode(layer, x, residual=None, out=None, workspace=None, return_routing=False):
    _need_cuda(x, residual, out, workspace)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = decode_workspace(layer, x.device)
    ids = w = None
    if return_routing:
        ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=x.device)
        w = torch.empty(T, layer.top_k, dtype=torch.float32, device=x.device)
    _check("fused_moe_mxfp4_decode", load().fused_moe_mxfp4_decode(
        layer.c, _ptr(x), T, _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(),
        _ptr(ids), _ptr(w), _stream()))
    return (out, ids, w) if return_routing else out


def fused_moe_mxfp4_decode_noalloc(layer, x, residual=None, out=None, return_routing=False):
    """fused_moe_mxfp4_decode on the library's own per-device workspace (no
    workspace argument; see mxmoe.h for the sharing rules)."""
    _need_cuda(x, residual, out)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    ids = w = None
    if return_routing:
        ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=x.device)
        w = torch.empty(T, layer.top_k, dtype=torch.float32, device=x.device)
    _check("fused_moe_mxfp4_decode_noalloc", load().fused_moe_mxfp4_decode_noalloc(
        layer.c, _ptr(x), T, _ptr(residual), _ptr(out), _ptr(ids), _ptr(w), _stream()))
    return (out, ids, w) if return_routing else out


def grouped_workspace(layer, T, device="cuda"):
    n = moe_workspace_bytes(layer, T, 1)
    if n == 0:
        raise MoeError("moe_workspace_bytes", -2)
    return torch.empty(n, dtype=torch.uint8, device=device)


def fused_moe_mxfp4_grouped(layer, x, residual=None, out=None, workspace=None):
    _need_cuda(x, residual, out, workspace)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = grouped_workspace(layer, T, x.device)
    _check("fused_moe_mxfp4_grouped", load().fused_moe_mxfp4_grouped(
        layer.c, _ptr(x), T, _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


# The pages' dispatch rule: steps of at most DECODE_MAX_ROWS rows run as one
# fused launch, wider ones stay on the original path (the article "MiniMax-M3.1
# on AMD Instinct GPUs: Day-0 support and optimization", section "Performance,
# mono decode on vs off").  The library's fused launch also takes wide steps of
# up to WIDE_MAX_ROWS rows (the same article's next kernel item, section
# "What's next": wider mono steps), and MoEForward uses them by default.
DECODE_MAX_ROWS = 16
WIDE_MAX_ROWS = 64


class MoEForward:
    """One MoE layer call for any number of rows: the fused single launch for
    T <= ``fused_max_rows``, falling back to the grouped path when the library
    reports the shape as unsupported by it; the grouped path otherwise.  The
    default is 64 rows: the wide fused launch is faster than the grouped path
    at every row count from 17 to 64 on the MiniMax-M3.1 layer (85 against
    150 us at 17 rows, 187 against 215 us at 64, one MI355X).  16 gives the
    pages' own rule.  Keeps the decode workspace (zero-filled once) and a
    grouped workspace grown on demand."""

    def __init__(self, layer, device="cuda", fused_max_rows=WIDE_MAX_ROWS):
        if not 1 <= fused_max_rows <= WIDE_MAX_ROWS:
            raise ValueError(f"fused_max_rows must be in 1..{WIDE_MAX_ROWS}")
        self.layer, self.device = layer, torch.device(device)
        self.fused_max_rows = fused_max_rows
        self.decode_ws = None
        self.grouped_ws = None
        self.last_path = None

    def _grouped(self, x, residual, out):
        n = moe_workspace_bytes(self.layer, x.shape[0], 1)
        if n == 0:
            raise MoeError("moe_workspace_bytes", -2)
        if self.grouped_ws is None or self.grouped_ws.numel() < n:
            self.grouped_ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        self.last_path = "grouped"
        return fused_moe_mxfp4_grouped(self.layer, x, residual, out, self.grouped_ws)

    def __call__(self, x, residual=None, out=None):
        if x.shape[0] <= self.fused_max_rows:
            if self.decode_ws is None:
                self.decode_ws = decode_workspace(self.layer, self.device,
                                                  DECODE_MAX_ROWS if self.fused_max_rows <= DECODE_MAX_ROWS
                                                  else WIDE_MAX_ROWS)
            try:
                y = fused_moe_mxfp4_decode(self.layer, x, residual, out, self.decode_ws)
                self.last_path = "decode"
                return y
            except MoeError as err:
                if err.status != -2:  # MOE_ERR_UNSUPPORTED: shape beyond the fused kernel
                    raise
        return self._grouped(x, residual, out)


GROUPED_STEPS = ("router", "sort", "x_quant", "routed_gate_up", "routed_down", "shared_gate_up",
                 "shared_down_combine")


def fused_moe_mxfp4_grouped_timed(layer, x, residual=None, out=None, workspace=None):
    """fused_moe_mxfp4_grouped with HIP events around each launch step.
    Returns (out, events); after a synchronize, events[i].elapsed_time(
    events[i + 1]) is step GROUPED_STEPS[i] in ms."""
    _need_cuda(x, residual, out, workspace)
    T = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = grouped_workspace(layer, T, x.device)
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(len(GROUPED_STEPS) + 1)]
    for e in events:  # creates the HIP events
        e.record(stream)
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("fused_moe_mxfp4_grouped_timed", load().fused_moe_mxfp4_grouped_timed(
        layer.c, _ptr(x), T, _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(), handles, _stream()))
    return out, events


def moe_decode_status(workspace):
    return load().moe_decode_status(_ptr(workspace), workspace.numel())


def moe_decode_trace(layer, workspace):
    """Per-workgroup phase timestamps (device clock ticks) of the last decode
    call on ``workspace``: an int64 array [grid, 16] (see mxmoe.h)."""
    import numpy as np
    buf = np.zeros(2048 * 16, dtype=np.uint64)
    g = load().moe_decode_trace(layer.c, _ptr(workspace), workspace.numel(),
                                buf.ctypes.data_as(ctypes.c_void_p), buf.size)
    if g < 0:
        raise MoeError("moe_decode_trace", g)
    return buf[: g * 16].reshape(g, 16).astype(np.int64)
