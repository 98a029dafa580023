// Router logits and top-k for any number of rows (used on its own and by the
// grouped path).  A workgroup takes a group of rows, keeps them in LDS, computes
// the E logits of each row with the fixed-order dot product of mx_device.h and
// then 16 lanes per row select the top k.
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRouterRows = 8;  // rows a workgroup keeps in LDS

__global__ void __launch_bounds__(kThreads) router_topk_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, int k, int rows_per_wg,
    const float* __restrict__ wr, const float* __restrict__ bias, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                               // [rows][H]
  float* ls = reinterpret_cast<float*>(smem + align_up((size_t)rows_per_wg * H * 2, 16));  // [rows][E]
  const int t0 = blockIdx.x * rows_per_wg;
  const int nrows = min(rows_per_wg, T - t0);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;

  // stage the rows (16-byte copies; H % 128 == 0)
  const int vec_per_row = H / 8;
  for (int i = threadIdx.x; i < nrows * vec_per_row; i += kThreads) {
    const int r = i / vec_per_row, c = i % vec_per_row;
    reinterpret_cast<uint4*>(xs + (size_t)r * H)[c] =
        reinterpret_cast<const uint4*>(x + (size_t)(t0 + r) * H)[c];
  }
  __syncthreads();

  // A wavefront per expert: each batch of up to 16 strides of the expert's
  // weights is loaded once into registers and applied to every staged row, so
  // each (row, expert) sum keeps the order of router_lane_partial.
  for (int e = wave; e < E; e += kWaves) {
    const float* wrow = wr + (size_t)e * H;
    float p[kRouterRows];
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r) p[r] = 0.f;
    for (int h0 = 4 * lane; h0 < H; h0 += 16 * 256) {
      float4 w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (h0 + 256 * j < H) w[j] = *reinterpret_cast<const float4*>(wrow + h0 + 256 * j);
#pragma unroll
      for (int r = 0; r < kRouterRows; ++r) {
        if (r < nrows) {
          const uint16_t* xr = xs + (size_t)r * H;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (h0 + 256 * j < H) {
              const uint2 xv = *reinterpret_cast<const uint2*>(xr + h0 + 256 * j);
              p[r] = fmaf(bf16_to_f32(xv.x & 0xffffu), w[j].x, p[r]);
              p[r] = fmaf(bf16_to_f32(xv.x >> 16), w[j].y, p[r]);
              p[r] = fmaf(bf16_to_f32(xv.y & 0xffffu), w[j].z, p[r]);
              p[r] = fmaf(bf16_to_f32(xv.y >> 16), w[j].w, p[r]);
            }
        }
      }
    }
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r)
      if (r < nrows) {
        float v = wave_sum_butterfly(p[r]);
        if (bias) v = v + b;
        if (lane == 0) ls[r * E + e] = v;
      }
  }
  __syncthreads();

  if (logits_out) {
    for (int i = threadIdx.x; i < nrows * E; i += kThreads)
      logits_out[(size_t)t0 * E + i] = ls[i];
  }
  for (int r0 = 0; r0 < nrows; r0 += kThreads / 16) {
    const int r = r0 + (int)threadIdx.x / 16;
    const bool act = r < nrows;
    const int rr = act ? r : 0;
    rows_topk16(ls + rr * E, act, E, k, threadIdx.x & 15, ids_out + (size_t)(t0 + rr) * k,
                w_out + (size_t)(t0 + rr) * k);
  }
}

}  // namespace

hipError_t launch_router_topk(const moe_layer_t& L, const uint16_t* x, int T, float* logits,
                              int32_t* ids, float* w, hipStream_t stream) {
  const int H = L.hidden, E = L.num_experts;
  int rows = 65536 / H;
  rows = rows < 1 ? 1 : (rows > kRouterRows ? kRouterRows : rows);
  const size_t lds = align_up((size_t)rows * H * 2, 16) + (size_t)rows * E * 4;
  const unsigned grid = (unsigned)((T + rows - 1) / rows);
  hipLaunchKernelGGL(router_topk_kernel, dim3(grid), dim3(kThreads), lds, stream, x, T, H, E,
                     L.top_k, rows, L.router_w, L.router_bias, logits, ids, w);
  return hipGetLastError();
}

}  // namespace mxmoe
