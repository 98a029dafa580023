// C-ABI entry points of libmxmoe.so (declared in include/mxmoe.h).  Every call
// validates its arguments on the host and returns before enqueueing anything
// if they are wrong; only then does it reach a HIP launch.
#include <cstdint>

#include "internal.h"

using namespace mxmoe;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_layer(const moe_layer_t* L) {
  if (!L) return MOE_ERR_INVALID_ARGUMENT;
  const int H = L->hidden, I = L->inter, E = L->num_experts, k = L->top_k, Is = L->shared_inter;
  if (H <= 0 || I <= 0 || H % 128 || I % 128) return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || E > 256) return MOE_ERR_INVALID_ARGUMENT;
  if (k < 1 || k > 8 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (Is < 0 || Is % 128) return MOE_ERR_INVALID_ARGUMENT;
  if (!L->router_w || !L->w13 || !L->w13_scale || !L->w2 || !L->w2_scale) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(L->router_w, 16) || !aligned(L->router_bias, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(L->w13, 16) || !aligned(L->w2, 16) || !aligned(L->w13_scale, 4) || !aligned(L->w2_scale, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(L->norm_weight, 16) || !(L->norm_eps >= 0.f)) return MOE_ERR_INVALID_ARGUMENT;
  if (L->shared_folded != 0 && L->shared_folded != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (L->shared_folded && (Is != 0 || k > 7 || E > 255)) return MOE_ERR_INVALID_ARGUMENT;
  if (Is > 0) {
    if (!L->ws13 || !L->ws13_scale || !L->ws2 || !L->ws2_scale) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(L->ws13, 16) || !aligned(L->ws2, 16) || !aligned(L->ws13_scale, 4) ||
        !aligned(L->ws2_scale, 4))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

bool valid_fmt(int fmt) { return fmt == MX_FMT_FP4 || fmt == MX_FMT_FP8; }
bool valid_layout(int layout) { return layout == MX_LAYOUT_ROWMAJOR || layout == MX_LAYOUT_TILED; }
bool valid_shape(int rows, int cols, int layout) {
  if (rows <= 0 || cols <= 0 || cols % 32) return false;
  if (layout == MX_LAYOUT_TILED && (rows % 16 || cols % 128)) return false;
  return true;
}

}  // namespace

extern "C" {

size_t mx_codes_bytes(int rows, int cols, int fmt, int layout) {
  if (!valid_fmt(fmt) || !valid_layout(layout) || !valid_shape(rows, cols, layout)) return 0;
  if (layout == MX_LAYOUT_TILED) return tiled_codes_bytes(rows, cols, fmt);
  return (size_t)rows * (size_t)(fmt == MX_FMT_FP4 ? cols / 2 : cols);
}

size_t mx_scales_bytes(int rows, int cols, int layout) {
  if (!valid_layout(layout) || !valid_shape(rows, cols, layout)) return 0;
  if (layout == MX_LAYOUT_TILED) return tiled_scales_bytes(rows, cols);
  return (size_t)rows * (size_t)(cols / 32);
}

moe_status mx_quantize_weights(const float* w, int rows, int cols, int fmt, int layout,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_fmt(fmt) || !valid_layout(layout) || !valid_shape(rows, cols, layout))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_quant_weights(w, rows, cols, fmt, layout, codes, scales, stream));
}

moe_status mx_requant_fp8_to_fp4(const uint8_t* codes8, const uint8_t* scales8, int rows, int cols, int layout,
                                 uint8_t* codes4, uint8_t* scales4, hipStream_t stream) {
  if (!codes8 || !scales8 || !codes4 || !scales4) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_layout(layout) || !valid_shape(rows, cols, layout)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(codes8, 16) || !aligned(codes4, 16) || !aligned(scales4, 4)) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_requant_fp8_fp4(codes8, scales8, rows, cols, layout, codes4, scales4, stream));
}

moe_status mx_requant_nvfp4_to_fp4(const uint8_t* codes, const uint8_t* block_scales, const float* global_scales,
                                   int rows_per_scale, int rows, int cols, int layout, uint8_t* codes4,
                                   uint8_t* scales4, hipStream_t stream) {
  if (!codes || !block_scales || !global_scales || !codes4 || !scales4) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_layout(layout) || !valid_shape(rows, cols, layout)) return MOE_ERR_INVALID_ARGUMENT;
  if (rows_per_scale <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, 16) || !aligned(global_scales, 4) || !aligned(codes4, 16) || !aligned(scales4, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_requant_nvfp4(codes, block_scales, global_scales, rows_per_scale, rows, cols, layout, codes4,
                                       scales4, stream));
}

moe_status mxfp4_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARGUMENT;
  if (rows <= 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes, 16)) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_quant_act(x, rows, cols, MX_FMT_FP4, codes, scales, stream));
}

moe_status moe_router_topk(const moe_layer_t* layer, const uint16_t* x, int T, float* logits,
                           int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  const moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (T <= 0 || !x || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16)) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_router_topk(*layer, x, T, logits, topk_ids, topk_w, layer->top_k, -1, stream));
}

size_t moe_align_sort_capacity(int T, int k, int E, int block_m) {
  if (T <= 0 || k <= 0 || E <= 0 || E > 256 || block_m <= 0) return 0;
  const size_t S = (size_t)T * k;
  const size_t used = S < (size_t)E ? S : (size_t)E;
  return S + used * (size_t)(block_m - 1);
}

size_t moe_align_sort_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0 || E > 256) return 0;
  return align_sort_ws_bytes(T, k, E);
}

moe_status moe_align_sort(const int32_t* topk_ids, int T, int k, int E, int block_m,
                          int32_t* sorted_slots, int32_t* block_expert, int32_t* expert_offsets,
                          int32_t* num_padded, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!topk_ids || !sorted_slots || !block_expert || !expert_offsets || !num_padded || !ws)
    return MOE_ERR_INVALID_ARGUMENT;
  if (T <= 0 || k <= 0 || E <= 0 || E > 256 || block_m <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((size_t)T * k > (size_t)INT32_MAX / 2) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(ws, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < align_sort_ws_bytes(T, k, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_align_sort(topk_ids, T, k, E, block_m, sorted_slots, block_expert,
                                    expert_offsets, num_padded, ws, stream));
}

size_t moe_workspace_bytes(const moe_layer_t* layer, int T, int path) {
  if (check_layer(layer) != MOE_OK) return 0;
  if (path == 0) return (T >= 1 && T <= kDecodeWideMaxT) ? decode_ws_bytes(*layer, T) : 0;
  if (path == 1) return T >= 1 ? grouped_ws_bytes(*layer, T) : 0;
  return 0;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || ws_bytes == 0 || !aligned(ws, 4) || ws_bytes % 4) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_fill_u32(ws, ws_bytes / 4, 0u, stream));
}

moe_status fused_moe_mxfp4_decode(const moe_layer_t* layer, const uint16_t* x, int T,
                                  const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                  int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream) {
  const moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws || T <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (layer->norm_weight && residual) return MOE_ERR_INVALID_ARGUMENT;  // the norm adds its own input
  if (T > kDecodeWideMaxT || !decode_supported(*layer, T)) return MOE_ERR_UNSUPPORTED;
  if (static_cast<const void*>(y) == static_cast<const void*>(x)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(residual, 4) || !aligned(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < decode_ws_bytes(*layer, T)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_decode(*layer, x, T, residual, y, ws, topk_ids_out, topk_w_out, stream));
}

moe_status fused_moe_mxfp4_decode_noalloc(const moe_layer_t* layer, const uint16_t* x, int T,
                                          const uint16_t* residual, uint16_t* y, int32_t* topk_ids_out,
                                          float* topk_w_out, hipStream_t stream) {
  const moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y || T <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (layer->norm_weight && residual) return MOE_ERR_INVALID_ARGUMENT;  // the norm adds its own input
  if (T > kDecodeMaxT || !decode_supported(*layer, T)) return MOE_ERR_UNSUPPORTED;
  if (static_cast<const void*>(y) == static_cast<const void*>(x)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(residual, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (decode_ws_bytes(*layer, T) > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = noalloc_scratch(stream);
  if (!ws) return MOE_ERR_HIP;
  return from_hip(launch_decode(*layer, x, T, residual, y, ws, topk_ids_out, topk_w_out, stream));
}

namespace {
moe_status grouped_call(const moe_layer_t* layer, const uint16_t* x, int T, const uint16_t* residual, uint16_t* y,
                        void* ws, size_t ws_bytes, hipStream_t stream, const hipEvent_t* events) {
  const moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws || T <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (layer->norm_weight && residual) return MOE_ERR_INVALID_ARGUMENT;  // the norm adds its own input
  if (static_cast<const void*>(y) == static_cast<const void*>(x)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(residual, 16) || !aligned(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = grouped_ws_bytes(*layer, T);
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(launch_grouped(*layer, x, T, residual, y, ws, stream, events));
}
}  // namespace

moe_status fused_moe_mxfp4_grouped(const moe_layer_t* layer, const uint16_t* x, int T,
                                   const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return grouped_call(layer, x, T, residual, y, ws, ws_bytes, stream, nullptr);
}

moe_status fused_moe_mxfp4_grouped_timed(const moe_layer_t* layer, const uint16_t* x, int T,
                                         const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                         const hipEvent_t* events, hipStream_t stream) {
  if (!events) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i <= kGroupedSteps; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARGUMENT;
  return grouped_call(layer, x, T, residual, y, ws, ws_bytes, stream, events);
}

moe_status moe_decode_status(const void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < 4) return MOE_ERR_INVALID_ARGUMENT;
  uint32_t status = 0;
  if (hipMemcpy(&status, static_cast<const char*>(ws) + kDecodeStatusOffset, 4, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return status ? MOE_ERR_TIMEOUT : MOE_OK;
}

int moe_decode_trace(const moe_layer_t* layer, const void* ws, size_t ws_bytes, uint64_t* host,
                     size_t n_words) {
  if (check_layer(layer) != MOE_OK || !ws || !host) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < decode_ws_bytes(*layer, 1)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  uint32_t grid = 0;
  if (hipMemcpy(&grid, static_cast<const char*>(ws) + kDecodeGridOffset, 4, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return MOE_ERR_HIP;
  size_t n = (size_t)grid * kTraceWords;
  if (n > n_words) n = n_words;
  if (n && hipMemcpy(host, static_cast<const char*>(ws) + decode_trace_offset(*layer), n * 8,
                     hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  return (int)grid;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported by this entry point";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime or launch error";
    case MOE_ERR_TIMEOUT: return "a device-side wait timed out";
  }
  return "unknown status";
}

}  // extern "C"
