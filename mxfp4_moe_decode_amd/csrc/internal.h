// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "mxmoe.h"

namespace mxmoe {

// Tiled layout sizes (see mxmoe.h).
inline size_t tiled_codes_bytes(int rows, int cols, int fmt) {
  return (size_t)(rows / 16) * (size_t)(cols / 128) * (fmt == MX_FMT_FP4 ? 1024u : 2048u);
}
inline int tiled_scale_groups(int cols) { return (cols / 128 + 3) / 4; }
inline size_t tiled_scales_bytes(int rows, int cols) {
  return (size_t)(rows / 16) * (size_t)tiled_scale_groups(cols) * 256u;
}

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Per-device host tables (launch geometry, the no-allocation scratch) hold
// this many devices.
constexpr int kMaxDevices = 64;
// The current HIP device, or -1 if it cannot be queried or is beyond the tables.
inline int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

// ------------------------------------------------------------------ quantization
hipError_t launch_quant_weights(const float* w, int rows, int cols, int fmt, int layout,
                                uint8_t* codes, uint8_t* scales, hipStream_t stream);
// Row-major activation quantization: codes [rows, cols/2] (FP4) or [rows, cols]
// (FP8), scales [rows, cols/32].  With gamma: of the RMS-normalized rows
// (h * rnorm[row]) * gamma[col] instead of x itself.
hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int fmt, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream, const float* rnorm = nullptr,
                            const float* gamma = nullptr);
// Both copies at once: MXFP4 codes [rows, cols/2] and MXFP8 codes [rows, cols],
// each with scales [rows, cols/32].
hipError_t launch_quant_act_dual(const uint16_t* x, int rows, int cols, uint8_t* codes4, uint8_t* scales4,
                                 uint8_t* codes8, uint8_t* scales8, hipStream_t stream,
                                 const float* rnorm = nullptr, const float* gamma = nullptr);
// rnorm[t] = 1 / sqrt(mean(x[t]^2) + eps) (the fixed order of row_rms_inv).
hipError_t launch_rms_rows(const uint16_t* x, int rows, int cols, float eps, float* rnorm, hipStream_t stream);
hipError_t launch_fill_u32(void* p, size_t words, uint32_t value, hipStream_t stream);
// MXFP8 -> MXFP4 along the same blocks, either layout.
hipError_t launch_requant_fp8_fp4(const uint8_t* codes8, const uint8_t* scales8, int rows, int cols, int layout,
                                  uint8_t* codes4, uint8_t* scales4, hipStream_t stream);

// NVFP4 (row-major codes, E4M3 block scales per 16, fp32 scale per row group)
// -> MXFP4 in either layout.
hipError_t launch_requant_nvfp4(const uint8_t* codes, const uint8_t* block_scales, const float* global_scales,
                                int rows_per_scale, int rows, int cols, int layout, uint8_t* codes4,
                                uint8_t* scales4, hipStream_t stream);

// Slots per row of a layer call: the k routed choices, plus the folded shared
// expert when there is one.
inline int layer_slots(const moe_layer_t& L) { return L.top_k + (L.shared_folded ? 1 : 0); }

// ------------------------------------------------------------------ router
// With a logits buffer the call takes the tiled logits kernel and a separate
// top-k pass; without, the per-row kernel (same arithmetic, identical results).
// ids / w rows are `ld` apart (>= k); with fold_e >= 0 entry k of every row
// is set to (fold_e, 1.0): the folded shared expert's slot.
hipError_t launch_router_topk(const moe_layer_t& L, const uint16_t* x, int T, float* logits,
                              int32_t* ids, float* w, int ld, int fold_e, hipStream_t stream);

// ------------------------------------------------------------------ align / sort
constexpr int kSortChunk = 1024;
size_t align_sort_ws_bytes(int T, int k, int E);
hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int block_m,
                             int32_t* sorted_slots, int32_t* block_expert, int32_t* expert_offsets,
                             int32_t* num_padded, void* ws, hipStream_t stream);

// ------------------------------------------------------------------ fused decode
constexpr int kDecodeMaxT = 16;      // rows of a decode step (mono decode's limit)
constexpr int kDecodeWideMaxT = 64;  // rows of a wide fused step
constexpr int kDecodeMaxGrid = 2048;
constexpr int kTraceWords = 16;
// Workspace for steps of T rows (sized for 16 rows up to T = 16, else for 64).
size_t decode_ws_bytes(const moe_layer_t& L, int T);
// Shapes and row counts the fused decode kernel handles (T <= 64, a gate/up
// K-chunk fits its register buffers, its LDS fits a workgroup).
bool decode_supported(const moe_layer_t& L, int T);
hipError_t launch_decode(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                         uint16_t* y, void* ws, int32_t* ids_out, float* w_out,
                         hipStream_t stream);
// Offset of the status word inside a decode workspace.
constexpr size_t kDecodeStatusOffset = 0;
// Bytes of the counter region at the start of a decode workspace (zero at rest).
size_t decode_sync_bytes(const moe_layer_t& L);
size_t decode_trace_offset(const moe_layer_t& L);
constexpr size_t kDecodeGridOffset = 2 * 256;  // word holding the grid size of the last call
// No-allocation decode: the library's own per-device workspace (a file-scope
// device array of this many bytes).  Returns its address on the current
// device, zero-filling it on `stream` the first time; nullptr on failure.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
void* noalloc_scratch(hipStream_t stream);

// ------------------------------------------------------------------ grouped path
size_t grouped_ws_bytes(const moe_layer_t& L, int T);
// Launch steps of the grouped path: router, sort, x quantization, routed
// gate/up, routed down, shared gate/up (without a shared expert: the
// combine), shared down with the combine.
constexpr int kGroupedSteps = 7;
hipError_t launch_grouped(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                          uint16_t* y, void* ws, hipStream_t stream, const hipEvent_t* ev = nullptr);

}  // namespace mxmoe
