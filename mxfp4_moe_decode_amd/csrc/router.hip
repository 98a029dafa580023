// Router logits and top-k for any number of rows (used on its own and by the
// grouped path).  With a logits buffer, a register-tiled kernel spread over
// row x expert tiles writes the logits with the fixed-order dot product of
// mx_device.h and a second pass selects the top k.  Without one, a workgroup
// takes up to 8 rows, keeps them in LDS, computes all E logits of each row
// (a wavefront per expert) and selects the top k itself: one workgroup per 8
// rows, so the tiled path is much faster at every row count.
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
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int ld, int fold_e, const float* __restrict__ gamma,
    float eps) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float rn[kRouterRows];  // pre-router RMSNorm factors of the staged rows (with gamma)
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
  if (gamma) {
    for (int r = wave; r < nrows; r += kWaves) {
      const float v = row_rms_inv(xs + (size_t)r * H, H, eps, lane);
      if (lane == 0) rn[r] = v;
    }
    __syncthreads();
  }

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
      if (gamma) {
        float4 g[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (h0 + 256 * j < H) g[j] = *reinterpret_cast<const float4*>(gamma + h0 + 256 * j);
#pragma unroll
        for (int r = 0; r < kRouterRows; ++r) {
          if (r < nrows) {
            const uint16_t* xr = xs + (size_t)r * H;
            const float rr = rn[r];
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (h0 + 256 * j < H) {
                const uint2 xv = *reinterpret_cast<const uint2*>(xr + h0 + 256 * j);
                p[r] = fmaf(__uint_as_float(normed_bits((xv.x & 0xffffu) << 16, rr, g[j].x)), w[j].x, p[r]);
                p[r] = fmaf(__uint_as_float(normed_bits(xv.x & 0xffff0000u, rr, g[j].y)), w[j].y, p[r]);
                p[r] = fmaf(__uint_as_float(normed_bits((xv.y & 0xffffu) << 16, rr, g[j].z)), w[j].z, p[r]);
                p[r] = fmaf(__uint_as_float(normed_bits(xv.y & 0xffff0000u, rr, g[j].w)), w[j].w, p[r]);
              }
          }
        }
      } else {
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
    rows_topk16(ls + rr * E, act, E, k, threadIdx.x & 15, ids_out + (size_t)(t0 + rr) * ld,
                w_out + (size_t)(t0 + rr) * ld);
    if (act && fold_e >= 0 && (threadIdx.x & 15) == 0) {
      ids_out[(size_t)(t0 + rr) * ld + k] = fold_e;
      w_out[(size_t)(t0 + rr) * ld + k] = 1.0f;
    }
  }
}


// ------------------------------------------------------------------ many rows
// Logits for many rows with the same per-logit arithmetic, organized for
// throughput: a wavefront owns a tile of 16 rows x 8 experts and keeps its
// 128 partial sums in registers, so each loaded x value feeds 8 FMAs and each
// loaded weight 16.  Lane l visits h = 256 i + 4 l + c (i ascending, c =
// 0..3) for every (row, expert) of the tile, exactly as router_lane_partial
// does for one pair.  The 64 lanes' partial sums are then added by a halving
// exchange: at lane distance d (32, 16, ..., 1) each lane keeps one half of
// its values and adds its partner's copy of that half, so every sum it forms
// is the sum the butterfly forms at that distance (same two operands), and
// lane l ends with the finished logits of tile entries 2l and 2l + 1.
constexpr int kTileRows = 16;
constexpr int kTileExperts = 8;   // per wavefront
constexpr int kTileVals = kTileRows * kTileExperts;

// With the pre-router norm (kNorm) every x value becomes (x r) g first; that
// instance has its own kernel, since the norm's registers would push the
// plain one into scratch memory.
template <bool kNorm>
__device__ __forceinline__ void router_tiled_body(const uint16_t* __restrict__ x, int T, int H, int E,
                                                  const float* __restrict__ wr, const float* __restrict__ bias,
                                                  float* __restrict__ logits, int n_rblk, int n_eblk,
                                                  const float* __restrict__ gamma, float eps, float* rn) {
  // workgroups are dealt to the 8 XCDs in turn; renumber so that each XCD
  // takes a contiguous run of tiles (the expert groups of one row block share
  // that XCD's L2)
  const int per = gridDim.x / 8;
  const int tile = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (tile >= n_rblk * n_eblk) return;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t0 = (tile / n_eblk) * kTileRows;
  const int e0 = (tile % n_eblk) * (kTileExperts * kWaves) + wave * kTileExperts;
  if constexpr (kNorm) {
    for (int r = wave; r < kTileRows; r += kWaves) {
      const float v = row_rms_inv(x + (size_t)min(t0 + r, T - 1) * H, H, eps, lane);
      if (lane == 0) rn[r] = v;
    }
    __syncthreads();
  }
  if (e0 >= E) return;
  const uint16_t* xr[kTileRows];
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) xr[r] = x + (size_t)min(t0 + r, T - 1) * H;
  const float* wp[kTileExperts];
#pragma unroll
  for (int e = 0; e < kTileExperts; ++e) wp[e] = wr + (size_t)min(e0 + e, E - 1) * H;

  float acc[kTileVals];
#pragma unroll
  for (int s = 0; s < kTileVals; ++s) acc[s] = 0.f;
  for (int h = 4 * lane; h < H; h += 256) {  // a lane past the end of a partial stride does nothing
    uint2 xv[kTileRows];
    float4 wv[kTileExperts];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) xv[r] = *reinterpret_cast<const uint2*>(xr[r] + h);
#pragma unroll
    for (int e = 0; e < kTileExperts; ++e) wv[e] = *reinterpret_cast<const float4*>(wp[e] + h);
    float4 gv = make_float4(1.f, 1.f, 1.f, 1.f);
    if constexpr (kNorm) gv = *reinterpret_cast<const float4*>(gamma + h);
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      float x0 = bf16_to_f32(xv[r].x & 0xffffu), x1 = bf16_to_f32(xv[r].x >> 16);
      float x2 = bf16_to_f32(xv[r].y & 0xffffu), x3 = bf16_to_f32(xv[r].y >> 16);
      if constexpr (kNorm) {
        const float rr = rn[r];
        x0 = (x0 * rr) * gv.x;
        x1 = (x1 * rr) * gv.y;
        x2 = (x2 * rr) * gv.z;
        x3 = (x3 * rr) * gv.w;
      }
#pragma unroll
      for (int e = 0; e < kTileExperts; ++e) {
        float& a = acc[r * kTileExperts + e];
        a = fmaf(x0, wv[e].x, a);
        a = fmaf(x1, wv[e].y, a);
        a = fmaf(x2, wv[e].z, a);
        a = fmaf(x3, wv[e].w, a);
      }
    }
  }
  // halving exchange: before distance d the lane holds 2d values (entries
  // whose higher index bits equal its lane bits above d); it keeps the upper
  // half if lane & d, the lower half otherwise
#pragma unroll
  for (int d = 32, half = kTileVals / 2; d >= 1; d >>= 1, half >>= 1) {
    const bool up = (lane & d) != 0;
#pragma unroll
    for (int s = 0; s < half; ++s) {
      const float lo = acc[s], hi = acc[s + half];
      const float send = up ? lo : hi;
      const float keep = up ? hi : lo;
      acc[s] = keep + __shfl_xor(send, d);
    }
  }
  // lane l: entries 2l, 2l + 1 = row l / 4, experts 2 (l % 4) + j
  const int t = t0 + lane / 4;
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + 2 * (lane % 4) + j;
      if (e < E) {
        float v = acc[j];
        if (bias) v = v + bias[e];
        logits[(size_t)t * E + e] = v;
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads, 2) router_logits_tiled_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int n_rblk, int n_eblk) {
  router_tiled_body<false>(x, T, H, E, wr, bias, logits, n_rblk, n_eblk, nullptr, 0.f, nullptr);
}

__global__ void __launch_bounds__(kThreads, 1) router_logits_tiled_norm_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ logits, int n_rblk, int n_eblk,
    const float* __restrict__ gamma, float eps) {
  __shared__ float rn[kTileRows];  // pre-router RMSNorm factors of the tile's rows
  router_tiled_body<true>(x, T, H, E, wr, bias, logits, n_rblk, n_eblk, gamma, eps, rn);
}

// Top k of each row of a logits matrix: 16 lanes per row.
__global__ void __launch_bounds__(kThreads) topk_rows_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                             int32_t* __restrict__ ids_out,
                                                             float* __restrict__ w_out, int ld, int fold_e) {
  const int r = blockIdx.x * (kThreads / 16) + (int)threadIdx.x / 16;
  const bool act = r < T;
  const int rr = act ? r : T - 1;
  rows_topk16(logits + (size_t)rr * E, act, E, k, threadIdx.x & 15, ids_out + (size_t)rr * ld,
              w_out + (size_t)rr * ld);
  if (act && fold_e >= 0 && (threadIdx.x & 15) == 0) {
    ids_out[(size_t)rr * ld + k] = fold_e;
    w_out[(size_t)rr * ld + k] = 1.0f;
  }
}

}  // namespace

hipError_t launch_router_topk(const moe_layer_t& L, const uint16_t* x, int T, float* logits,
                              int32_t* ids, float* w, int ld, int fold_e, hipStream_t stream) {
  const int H = L.hidden, E = L.num_experts;
  if (logits) {  // expert-parallel: tiles of rows x experts, then the top-k pass
    const int n_rblk = (T + kTileRows - 1) / kTileRows;
    const int n_eblk = (E + kTileExperts * kWaves - 1) / (kTileExperts * kWaves);
    const unsigned grid = (unsigned)((n_rblk * n_eblk + 7) / 8 * 8);
    if (L.norm_weight)
      hipLaunchKernelGGL(router_logits_tiled_norm_kernel, dim3(grid), dim3(kThreads), 0, stream, x, T, H, E,
                         L.router_w, L.router_bias, logits, n_rblk, n_eblk, L.norm_weight, L.norm_eps);
    else
      hipLaunchKernelGGL(router_logits_tiled_kernel, dim3(grid), dim3(kThreads), 0, stream, x, T, H, E,
                         L.router_w, L.router_bias, logits, n_rblk, n_eblk);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)((T + 15) / 16)), dim3(kThreads), 0, stream, logits, T, E,
                       L.top_k, ids, w, ld, fold_e);
    return hipGetLastError();
  }
  int rows = 65536 / H;
  rows = rows < 1 ? 1 : (rows > kRouterRows ? kRouterRows : rows);
  const size_t lds = align_up((size_t)rows * H * 2, 16) + (size_t)rows * E * 4;
  const unsigned grid = (unsigned)((T + rows - 1) / rows);
  hipLaunchKernelGGL(router_topk_kernel, dim3(grid), dim3(kThreads), lds, stream, x, T, H, E,
                     L.top_k, rows, L.router_w, L.router_bias, logits, ids, w, ld, fold_e, L.norm_weight,
                     L.norm_eps);
  return hipGetLastError();
}

}  // namespace mxmoe
