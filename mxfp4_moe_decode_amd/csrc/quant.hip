// MX quantization kernels: static weight quantization (fp32 -> MXFP4 / MXFP8,
// row-major or tiled) and dynamic MXFP4 activation quantization (bf16 -> MXFP4).
// One thread per 32-element block.  Each element is scaled by 2^-e (exact)
// and converted by gfx950's rounding fp32 -> E2M1 / E4M3 instructions
// (quant_block32 in mx_device.h), so the codes are the specification's.
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;

// Destination of the packed codes of block (r, b) of a [rows][cols] matrix.
// Row-major: FP4 bytes [r][16b .. 16b+16), FP8 bytes [r][32b .. 32b+32).
// Tiled (see mxmoe.h): FP4: one 16-byte piece; FP8: two 16-byte pieces.
template <class F, bool Tiled>
__device__ __forceinline__ void store_block(uint8_t* codes, uint8_t* scales, int r, int b, int cols,
                                            const uint32_t* words, uint32_t scale) {
  const int KT = cols / 128;
  if constexpr (!Tiled) {
    if constexpr (F::MB == 1) {
      *reinterpret_cast<uint4*>(codes + (size_t)r * (cols / 2) + 16 * b) =
          make_uint4(words[0], words[1], words[2], words[3]);
    } else {
      uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)r * cols + 32 * b);
      dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
      dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
    }
    scales[(size_t)r * (cols / 32) + b] = (uint8_t)scale;
  } else {
    const int nt = r / 16, kt = b / 4, q = b % 4;
    const int lane = (r % 16) + 16 * q;
    if constexpr (F::MB == 1) {
      uint8_t* tile = codes + ((size_t)nt * KT + kt) * 1024;
      *reinterpret_cast<uint4*>(tile + 16 * lane) = make_uint4(words[0], words[1], words[2], words[3]);
    } else {
      // K offsets 32q .. 32q+32 inside the tile: the first 16 go to (c, q') =
      // ((32q)/64, (32q%64)/16), the next 16 to the following q'.
      uint8_t* tile = codes + ((size_t)nt * KT + kt) * 2048;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k0 = 32 * q + 16 * h;
        const int c = k0 / 64, qq = (k0 % 64) / 16;
        const int ll = (r % 16) + 16 * qq;
        *reinterpret_cast<uint4*>(tile + 1024 * c + 16 * ll) =
            make_uint4(words[4 * h], words[4 * h + 1], words[4 * h + 2], words[4 * h + 3]);
      }
    }
    const int KG = (KT + 3) / 4;
    const int g = kt / 4, i = kt % 4;
    scales[(((size_t)nt * KG + g) * 64 + lane) * 4 + i] = (uint8_t)scale;
  }
}

// Codes and scale of MXFP8 block (r, b) of a [rows][cols] matrix in either
// layout (the inverse of store_block<FP8, Tiled>).
template <bool Tiled>
__device__ __forceinline__ uint32_t load_block_fp8(const uint8_t* codes, const uint8_t* scales, int r, int b,
                                                   int cols, uint32_t (&words)[8]) {
  const int KT = cols / 128;
  if constexpr (!Tiled) {
    const uint4* src = reinterpret_cast<const uint4*>(codes + (size_t)r * cols + 32 * b);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 v = src[h];
      words[4 * h] = v.x;
      words[4 * h + 1] = v.y;
      words[4 * h + 2] = v.z;
      words[4 * h + 3] = v.w;
    }
    return scales[(size_t)r * (cols / 32) + b];
  } else {
    const int nt = r / 16, kt = b / 4, q = b % 4;
    const uint8_t* tile = codes + ((size_t)nt * KT + kt) * 2048;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k0 = 32 * q + 16 * h;
      const int c = k0 / 64, qq = (k0 % 64) / 16;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + 1024 * c + 16 * ((r % 16) + 16 * qq));
      words[4 * h] = v.x;
      words[4 * h + 1] = v.y;
      words[4 * h + 2] = v.z;
      words[4 * h + 3] = v.w;
    }
    const int KG = (KT + 3) / 4;
    return scales[(((size_t)nt * KG + kt / 4) * 64 + (r % 16) + 16 * q) * 4 + kt % 4];
  }
}

// Exact fp32 value of E4M3 code c times 2^(s - 127): the code is M * 2^(E - 10)
// with M = 8 + m, E = e for a normal (e >= 1) and M = m, E = 1 for a subnormal;
// M has at most four significant bits, so the product is exact whenever it is
// finite in fp32 (down to 2^-136, inside fp32's subnormal range).
__device__ __forceinline__ uint32_t e4m3_scaled_bits(uint32_t c, uint32_t s) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float M = (float)(e ? 8u + m : m);
  const float v = ldexpf(M, (int)(e ? e : 1u) - 10 + (int)s - 127);
  return __float_as_uint(v) | ((c & 0x80u) << 24);
}

// MXFP8 -> MXFP4 re-quantization along the same 32-element blocks: every
// element's exact value goes through the MX conversion again with the E2M1
// element type.  One thread per block.
template <bool Tiled>
__global__ void __launch_bounds__(kThreads) requant_fp8_fp4_kernel(const uint8_t* __restrict__ codes8,
                                                                   const uint8_t* __restrict__ scales8, int rows,
                                                                   int cols, uint8_t* __restrict__ codes4,
                                                                   uint8_t* __restrict__ scales4) {
  const int nb = cols / 32;
  const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= (size_t)rows * nb) return;
  const int r = (int)(blk / nb), b = (int)(blk % nb);
  uint32_t w8[8];
  const uint32_t s = load_block_fp8<Tiled>(codes8, scales8, r, b, cols, w8);
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) bits[i] = e4m3_scaled_bits((w8[i / 4] >> (8 * (i % 4))) & 0xffu, s);
  uint32_t words[8];
  const uint32_t s4 = quant_block32<FP4>(bits, words);
  store_block<FP4, Tiled>(codes4, scales4, r, b, cols, words, s4);
}

// NVFP4 -> MXFP4 re-quantization.  NVFP4 (the public format: E2M1 elements,
// an E4M3 scale per 16 consecutive elements, an fp32 scale per tensor or row
// group): v = E2M1(c) * E4M3(s_block) * s_global, where the first product is
// exact in fp32 and the second is rounded once (round to nearest even).  The
// fp32 values then go through the MX conversion with the E2M1 element type,
// 32 elements per block.  One thread per 32-element block: the row-major codes
// [rows][cols/2] (element 2i in the low nibble of byte i), block scales
// [rows][cols/16], scale group r / rows_per_scale.
template <bool Tiled>
__global__ void __launch_bounds__(kThreads) requant_nvfp4_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ block_scales,
                                                                 const float* __restrict__ global_scales,
                                                                 int rows_per_scale, int rows, int cols,
                                                                 uint8_t* __restrict__ codes4,
                                                                 uint8_t* __restrict__ scales4) {
  const int nb = cols / 32;
  const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= (size_t)rows * nb) return;
  const int r = (int)(blk / nb), b = (int)(blk % nb);
  const uint4 v = *reinterpret_cast<const uint4*>(codes + (size_t)r * (cols / 2) + 16 * b);
  const uint32_t packed[4] = {v.x, v.y, v.z, v.w};
  const uint8_t* bs = block_scales + (size_t)r * (cols / 16) + 2 * b;
  const float s[2] = {__uint_as_float(e4m3_scaled_bits(bs[0], 127u)), __uint_as_float(e4m3_scaled_bits(bs[1], 127u))};
  const float g = global_scales[r / rows_per_scale];
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    // E2M1 magnitude code m = 2e + f: M * 2^(max(e, 1) - 2) with M = 2 + f for
    // e >= 1 and M = f for e = 0 (0, 0.5, 1, 1.5, 2, 3, 4, 6)
    const uint32_t c = (packed[i / 8] >> (4 * (i % 8))) & 0xfu;
    const uint32_t e = (c >> 1) & 3u, f = c & 1u;
    const float a = ldexpf((float)(e ? 2u + f : f) * s[i / 16], (int)(e ? e : 1u) - 2);  // exact
    bits[i] = __float_as_uint(a * g) ^ ((c & 8u) << 28);
  }
  uint32_t words[8];
  const uint32_t s4 = quant_block32<FP4>(bits, words);
  store_block<FP4, Tiled>(codes4, scales4, r, b, cols, words, s4);
}

template <class F, bool Tiled>
__global__ void __launch_bounds__(kThreads) quant_weights_kernel(const float* __restrict__ w,
                                                                 int rows, int cols,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const int nb = cols / 32;
  const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= (size_t)rows * nb) return;
  const int r = (int)(blk / nb), b = (int)(blk % nb);
  const uint4* src = reinterpret_cast<const uint4*>(w + (size_t)r * cols + 32 * b);
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = src[i];
    bits[4 * i] = v.x;
    bits[4 * i + 1] = v.y;
    bits[4 * i + 2] = v.z;
    bits[4 * i + 3] = v.w;
  }
  uint32_t words[8];
  const uint32_t s = quant_block32<F>(bits, words);
  store_block<F, Tiled>(codes, scales, r, b, cols, words, s);
}

// The pre-router RMSNorm on a 32-value block of a row: (h * r) * g.
__device__ __forceinline__ void apply_norm(uint32_t (&bits)[32], float r, const float* g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 gv = *reinterpret_cast<const float4*>(g + 4 * i);
    bits[4 * i] = normed_bits(bits[4 * i], r, gv.x);
    bits[4 * i + 1] = normed_bits(bits[4 * i + 1], r, gv.y);
    bits[4 * i + 2] = normed_bits(bits[4 * i + 2], r, gv.z);
    bits[4 * i + 3] = normed_bits(bits[4 * i + 3], r, gv.w);
  }
}

// r[t] = 1 / sqrt(mean(h[t]^2) + eps) for every row, a wavefront per row.
__global__ void __launch_bounds__(kThreads) rms_rows_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                            float eps, float* __restrict__ rnorm) {
  const int r = blockIdx.x * (kThreads / kWave) + (int)threadIdx.x / kWave;
  if (r >= rows) return;  // whole wavefront
  const float v = row_rms_inv(x + (size_t)r * cols, cols, eps, threadIdx.x % kWave);
  if (threadIdx.x % kWave == 0) rnorm[r] = v;
}

template <class F>
__global__ void __launch_bounds__(kThreads) quant_act_kernel(const uint16_t* __restrict__ x, int rows,
                                                             int cols, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             const float* __restrict__ rnorm,
                                                             const float* __restrict__ gamma) {
  const int nb = cols / 32;
  const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= (size_t)rows * nb) return;
  const int r = (int)(blk / nb), b = (int)(blk % nb);
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)r * cols + 32 * b);
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bits[8 * i + 2 * j] = p[j] << 16;
      bits[8 * i + 2 * j + 1] = p[j] & 0xffff0000u;
    }
  }
  if (gamma) apply_norm(bits, rnorm[r], gamma + 32 * b);
  constexpr int kWords = F::MB == 1 ? 4 : 8;  // 16 or 32 code bytes per block
  uint32_t words[kWords];
  const uint32_t s = quant_block32<F>(bits, words);
  uint4* dst = reinterpret_cast<uint4*>(codes + ((size_t)r * nb + b) * (4 * kWords));
#pragma unroll
  for (int w = 0; w < kWords; w += 4) dst[w / 4] = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
  scales[(size_t)r * nb + b] = (uint8_t)s;
}

// Both MX copies of the activations (MXFP4 and MXFP8) from one read of x:
// the same block arithmetic as quant_act_kernel for each format.
__global__ void __launch_bounds__(kThreads) quant_act_dual_kernel(const uint16_t* __restrict__ x, int rows,
                                                                  int cols, uint8_t* __restrict__ codes4,
                                                                  uint8_t* __restrict__ scales4,
                                                                  uint8_t* __restrict__ codes8,
                                                                  uint8_t* __restrict__ scales8,
                                                                  const float* __restrict__ rnorm,
                                                                  const float* __restrict__ gamma) {
  const int nb = cols / 32;
  const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= (size_t)rows * nb) return;
  const int r = (int)(blk / nb), b = (int)(blk % nb);
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)r * cols + 32 * b);
  uint32_t bits[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bits[8 * i + 2 * j] = p[j] << 16;
      bits[8 * i + 2 * j + 1] = p[j] & 0xffff0000u;
    }
  }
  if (gamma) apply_norm(bits, rnorm[r], gamma + 32 * b);
  uint32_t w4[4], w8[8];
  const uint32_t s4 = quant_block32<FP4>(bits, w4);
  const uint32_t s8 = quant_block32<FP8>(bits, w8);
  const size_t o = (size_t)r * nb + b;
  *reinterpret_cast<uint4*>(codes4 + o * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  uint4* d8 = reinterpret_cast<uint4*>(codes8 + o * 32);
  d8[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
  d8[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
  scales4[o] = (uint8_t)s4;
  scales8[o] = (uint8_t)s8;
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_requant_fp8_fp4(const uint8_t* codes8, const uint8_t* scales8, int rows, int cols, int layout,
                                  uint8_t* codes4, uint8_t* scales4, hipStream_t stream) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const unsigned grid = (unsigned)((nblk + kThreads - 1) / kThreads);
  if (layout == MX_LAYOUT_TILED) {
    hipError_t err = launch_fill_u32(scales4, tiled_scales_bytes(rows, cols) / 4, 0x7f7f7f7fu, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(requant_fp8_fp4_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, codes8, scales8, rows,
                       cols, codes4, scales4);
  } else {
    hipLaunchKernelGGL(requant_fp8_fp4_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, codes8, scales8, rows,
                       cols, codes4, scales4);
  }
  return hipGetLastError();
}

hipError_t launch_requant_nvfp4(const uint8_t* codes, const uint8_t* block_scales, const float* global_scales,
                                int rows_per_scale, int rows, int cols, int layout, uint8_t* codes4,
                                uint8_t* scales4, hipStream_t stream) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const unsigned grid = (unsigned)((nblk + kThreads - 1) / kThreads);
  if (layout == MX_LAYOUT_TILED) {
    hipError_t err = launch_fill_u32(scales4, tiled_scales_bytes(rows, cols) / 4, 0x7f7f7f7fu, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(requant_nvfp4_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, codes, block_scales,
                       global_scales, rows_per_scale, rows, cols, codes4, scales4);
  } else {
    hipLaunchKernelGGL(requant_nvfp4_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, codes, block_scales,
                       global_scales, rows_per_scale, rows, cols, codes4, scales4);
  }
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, size_t words, uint32_t value, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  const unsigned grid = (unsigned)((words + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, stream, (uint32_t*)p, words, value);
  return hipGetLastError();
}

hipError_t launch_quant_weights(const float* w, int rows, int cols, int fmt, int layout,
                                uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const unsigned grid = (unsigned)((nblk + kThreads - 1) / kThreads);
  if (layout == MX_LAYOUT_TILED) {
    // scale bytes of K-tiles past the end of a group hold 127
    const size_t sb = tiled_scales_bytes(rows, cols);
    hipError_t err = launch_fill_u32(scales, sb / 4, 0x7f7f7f7fu, stream);
    if (err != hipSuccess) return err;
  }
  if (fmt == MX_FMT_FP4) {
    if (layout == MX_LAYOUT_TILED)
      hipLaunchKernelGGL((quant_weights_kernel<FP4, true>), dim3(grid), dim3(kThreads), 0, stream, w, rows, cols, codes, scales);
    else
      hipLaunchKernelGGL((quant_weights_kernel<FP4, false>), dim3(grid), dim3(kThreads), 0, stream, w, rows, cols, codes, scales);
  } else {
    if (layout == MX_LAYOUT_TILED)
      hipLaunchKernelGGL((quant_weights_kernel<FP8, true>), dim3(grid), dim3(kThreads), 0, stream, w, rows, cols, codes, scales);
    else
      hipLaunchKernelGGL((quant_weights_kernel<FP8, false>), dim3(grid), dim3(kThreads), 0, stream, w, rows, cols, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_rms_rows(const uint16_t* x, int rows, int cols, float eps, float* rnorm, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + kThreads / kWave - 1) / (kThreads / kWave));
  hipLaunchKernelGGL(rms_rows_kernel, dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, eps, rnorm);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, int fmt, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream, const float* rnorm, const float* gamma) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const unsigned grid = (unsigned)((nblk + kThreads - 1) / kThreads);
  if (fmt == MX_FMT_FP4)
    hipLaunchKernelGGL(quant_act_kernel<FP4>, dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, codes, scales,
                       rnorm, gamma);
  else
    hipLaunchKernelGGL(quant_act_kernel<FP8>, dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, codes, scales,
                       rnorm, gamma);
  return hipGetLastError();
}

hipError_t launch_quant_act_dual(const uint16_t* x, int rows, int cols, uint8_t* codes4, uint8_t* scales4,
                                 uint8_t* codes8, uint8_t* scales8, hipStream_t stream, const float* rnorm,
                                 const float* gamma) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const unsigned grid = (unsigned)((nblk + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(quant_act_dual_kernel, dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, codes4, scales4,
                     codes8, scales8, rnorm, gamma);
  return hipGetLastError();
}

}  // namespace mxmoe
