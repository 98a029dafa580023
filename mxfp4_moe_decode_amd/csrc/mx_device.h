// Device helpers shared by the gfx950 kernels: MX block quantization (block
// exponent from the exponent bits, elements by the hardware conversions or the
// branch-free software rounding), scaled FP4/FP8 matrix-core wrappers, the
// router's fixed-order dot product and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MX element formats (OCP Microscaling Formats v1.0).  MB: mantissa bits,
// EMIN: exponent of the smallest normal, EMAX: exponent of the largest power
// of two (emax_elem of the scale rule), MAXC: largest finite magnitude code,
// SIGN: sign bit position.
// ---------------------------------------------------------------------------
struct FP4 { static constexpr int MB = 1, EMIN = 0, EMAX = 2, MAXC = 0x7, SIGN = 3; };
struct FP8 { static constexpr int MB = 3, EMIN = -6, EMAX = 8, MAXC = 0x7E, SIGN = 7; };

// Block exponent floor(log2(amax)) - emax_elem, clamped below at -127, from
// the fp32 bit pattern of the block's largest magnitude (sign cleared).  Zero
// and subnormal maxima give -127.  fp32 inputs never reach the upper clamp.
template <class F>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  int e = (int)(amax_bits >> 23) - 127 - F::EMAX;
  return e < -127 ? -127 : e;
}

// 2^-e as an fp32 value (e = block exponent, -127 <= e <= 126).
__device__ __forceinline__ float block_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// SwiGLU: silu(g) * u = g / (1 + e^-g) * u, with the hardware base-2
// exponential and reciprocal: g * rcp(1 + 2^(-g log2 e)) * u.  Relative error
// against the exact value, to first order in u = 2^-24: the exponent -g log2 e
// carries two roundings (the constant and the product), which move 2^t by at
// most 2|g| u; the exponential and the reciprocal are within one ulp (2u) each;
// the sum and the two products round once each: (2|g| + 7) u.  Overflow of the
// exponential (g < -88) gives 0 where the exact value is below 2^-120.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return (g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g * 1.44269504f))) * u;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two E4M3 codes (element a in the low byte) of v * 2^-e for fp32 bit
// patterns a, b and inv = block_inv_scale(e), by the hardware conversion:
// q = v * inv is exact (a power-of-two scaling) and |q| < 2^9; clamped to
// +-448 (the largest E4M3 magnitude) first, its round-to-nearest-even
// conversion equals rounding and then saturating, sign of zero included.
__device__ __forceinline__ uint32_t quant_pair_fp8(uint32_t a, uint32_t b, float inv) {
  const float qa = __builtin_amdgcn_fmed3f(__uint_as_float(a) * inv, -448.f, 448.f);
  const float qb = __builtin_amdgcn_fmed3f(__uint_as_float(b) * inv, -448.f, 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, 0, false) & 0xffffu;
}

// E2M1 codes of v * 2^-e for four fp32 bit patterns (element i in nibble i)
// by the hardware conversion, with a unit scale: q = v * inv is exact and
// |q| < 2^3, and the conversion rounds to nearest even and saturates at 6.
__device__ __forceinline__ uint32_t quant_quad_fp4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, float inv) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(b0) * inv, __uint_as_float(b1) * inv,
                                                        1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(b2) * inv, __uint_as_float(b3) * inv, 1.0f, 1);
  return w & 0xffffu;
}

// Quantize 32 consecutive values (fp32 bit patterns) of one MX block held by
// one lane.  FP4: 16 packed bytes (element 2i in the low nibble of byte i);
// FP8: 32 bytes.  Returns the E8M0 scale code.
template <class F>
__device__ __forceinline__ uint32_t quant_block32(const uint32_t* bits, uint32_t* out_words) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, bits[i] & 0x7fffffffu);
  const int e = block_exponent<F>(amax);
  const float inv = block_inv_scale(e);
  if constexpr (F::MB == 1) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      out_words[w] = quant_quad_fp4(bits[8 * w], bits[8 * w + 1], bits[8 * w + 2], bits[8 * w + 3], inv) |
                     (quant_quad_fp4(bits[8 * w + 4], bits[8 * w + 5], bits[8 * w + 6], bits[8 * w + 7], inv) << 16);
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w)
      out_words[w] = quant_pair_fp8(bits[4 * w], bits[4 * w + 1], inv) |
                     (quant_pair_fp8(bits[4 * w + 2], bits[4 * w + 3], inv) << 16);
  }
  return (uint32_t)(e + 127);
}

// ---------------------------------------------------------------------------
// Scaled matrix instructions, 16x16x128 (gfx950).  Operand layout, verified on
// the device: lane l supplies row l%16 of its operand.  FP4: 16 bytes holding
// K = 32*(l/16) .. +32 (element 2i in the low nibble of byte i).  FP8: bytes
// 0..15 hold K = 16*(l/16) .. +16, bytes 16..31 hold K = 64 + 16*(l/16) .. +16.
// Scale operands: lane l gives the E8M0 of (row l%16, K block l/16) in the low
// byte.  Result: lane l, element i = C[4*(l/16) + i][l%16] with C = A * B^T.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_fp4(v4i a, v4i b, v4f c, uint32_t sa, uint32_t sb) {
  v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ v4f mfma_fp8(v4i a0, v4i a1, v4i b0, v4i b1, v4f c, uint32_t sa,
                                        uint32_t sb) {
  v8i A = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  v8i B = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// Streaming loads of weights read once per call (non-temporal: on gfx950 a
// cold burst of these completes about twice as fast as plain loads).
__device__ __forceinline__ v4i load_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}
__device__ __forceinline__ uint32_t load_stream4(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float4 load_stream_f4(const float* p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------
// Router dot product, the fixed order every router path uses: lane l
// accumulates with fp32 FMA the products for h = 256*i + 4*l + c (i ascending,
// c = 0..3), then wave_sum_butterfly adds the 64 partial sums.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float router_lane_partial(const uint16_t* xrow, const float* wrow, int H,
                                                     int lane) {
  float p = 0.f;
  // batches of 16 strides: all loads of a batch are issued before its FMAs
  for (int h0 = 4 * lane; h0 < H; h0 += 16 * 256) {
    float4 w[16];
    uint2 xv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int h = h0 + 256 * j;
      if (h < H) {
        w[j] = *reinterpret_cast<const float4*>(wrow + h);
        xv[j] = *reinterpret_cast<const uint2*>(xrow + h);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (h0 + 256 * j < H) {
        p = fmaf(bf16_to_f32(xv[j].x & 0xffffu), w[j].x, p);
        p = fmaf(bf16_to_f32(xv[j].x >> 16), w[j].y, p);
        p = fmaf(bf16_to_f32(xv[j].y & 0xffffu), w[j].z, p);
        p = fmaf(bf16_to_f32(xv[j].y >> 16), w[j].w, p);
      }
    }
  }
  return p;
}

// Butterfly sum over the 64 lanes; every lane ends with the same value
// (fp32 addition is commutative, so partners compute identical sums).
__device__ __forceinline__ float wave_sum_butterfly(float p) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off);
  return p;
}

// ---------------------------------------------------------------------------
// Pre-router RMSNorm, the fixed arithmetic every path uses: the sum of
// squares of a bf16 row with lane l FMA-ing h = 256 i + 4 l + c (i ascending,
// c = 0..3), the butterfly over the lanes, r = 1 / sqrtf(S / H + eps); the
// normalized value is (h * r) * g, two fp32 products.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float row_rms_inv(const uint16_t* row, int H, float eps, int lane) {
  float p = 0.f;
  for (int h0 = 4 * lane; h0 < H; h0 += 256) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + h0);
    const float a = bf16_to_f32(v.x & 0xffffu), b = bf16_to_f32(v.x >> 16);
    const float c = bf16_to_f32(v.y & 0xffffu), d = bf16_to_f32(v.y >> 16);
    p = fmaf(a, a, p);
    p = fmaf(b, b, p);
    p = fmaf(c, c, p);
    p = fmaf(d, d, p);
  }
  const float s = wave_sum_butterfly(p);
  return 1.0f / sqrtf(s / (float)H + eps);
}

// fp32 bits of the normalized value of bf16 bits-as-fp32 `hbits`.
__device__ __forceinline__ uint32_t normed_bits(uint32_t hbits, float r, float g) {
  return __float_as_uint((__uint_as_float(hbits) * r) * g);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v, int width) {
  for (int off = width / 2; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

// Top-k key: order-preserving fp32 bits (with -0 folded onto +0) above the
// complemented expert index, so the largest key is the largest logit and,
// among equal logits, the lowest expert index.
__device__ __forceinline__ uint64_t topk_key(float logit, int e) {
  uint32_t b = __float_as_uint(logit + 0.0f);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xffffu - (uint32_t)e);
}

__device__ __forceinline__ float topk_key_logit(uint64_t key) {
  uint32_t b = (uint32_t)(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;
  return __uint_as_float(b);
}

__device__ __forceinline__ int topk_key_expert(uint64_t key) {
  return (int)(0xffffu - (uint32_t)(key & 0xffffu));
}

// Weights of a chosen top-k: z_j = exp(l_j - l_0), w_j = z_j / sum_j z_j in
// fp32 with the sum taken in j order (l_0 is the largest logit).  In place:
// w[] holds the chosen logits on entry.
__device__ __forceinline__ void topk_weights_inplace(float* w, int k) {
  const float l0 = w[0];
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += expf(w[j] - l0);
  for (int j = 0; j < k; ++j) w[j] = expf(w[j] - l0) / sum;
}

constexpr int kTopkMax = 8;

// Moves a 64-bit value between the lanes of a 16-lane row with one data-parallel
// permutation (CTRL: quad_perm or row mirror patterns, which stay inside the row).
template <int CTRL>
__device__ __forceinline__ uint64_t row_move64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the 16 lanes of a row: swap neighbours, swap pairs, mirror
// each half row, mirror the row.  Every lane ends with the maximum.
__device__ __forceinline__ uint64_t row16_max64(uint64_t v) {
  v = max_u64(v, row_move64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, row_move64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, row_move64<0x141>(v));  // row_half_mirror
  v = max_u64(v, row_move64<0x140>(v));  // row_mirror
  return v;
}

// Order-preserving 32-bit image of a logit (-0 counted as +0): a larger
// image means a larger logit, and 0 is below every image.
__device__ __forceinline__ uint32_t logit_order_bits(float logit) {
  const uint32_t b = __float_as_uint(logit + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float logit_from_order_bits(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

// Maximum over the wavefront, returned uniform: each step moves a value with
// one data-parallel permutation (swap neighbours, swap pairs, mirror each half
// row, mirror the row, then lane 15 of rows 0/2 into rows 1/3 and lane 31
// into rows 2/3); lane 63 ends with the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top k of one row of E <= 256 logits on a whole wavefront (lane l holds the
// logits of experts l, l+64, ...); same result and outputs as rows_topk16.
// Each of the k rounds takes the wavefront maximum of the 32-bit logit images
// and, among the experts holding it, the lowest index (first set bit of the
// ballots, expert l + 64 r in r-major order), then retires that expert.  Lane j
// keeps round j's logit; the weights are formed in parallel with the sum taken
// in j order, as topk_weights_inplace does.  Lanes j < k of an active row
// write ids[j] and w[j].  Every lane must call it; k is uniform.
__device__ __forceinline__ void row_topk64(const float* logits_row, bool active, int E, int k, int lane,
                                           int32_t* ids, float* w) {
  // A key can be 0 (the logit with all bits set), so whether an expert is
  // still in the running is kept apart from its key.
  uint32_t kv[4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + 64 * r;
    live[r] = active && e < E;
    kv[r] = live[r] ? logit_order_bits(logits_row[e]) : 0u;
  }
  float my_l = 0.f;
  int my_e = 0;
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j) {
    if (j < k) {
      const uint32_t m = wave_max_u32(max(max(kv[0], kv[1]), max(kv[2], kv[3])));
      int best = -1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint64_t bal = __ballot(live[r] && kv[r] == m);
        if (best < 0 && bal != 0ull) best = 64 * r + (__ffsll((unsigned long long)bal) - 1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (lane + 64 * r == best) {
          kv[r] = 0u;
          live[r] = false;
        }
      if (lane == j) {
        my_l = logit_from_order_bits(m);
        my_e = best;
      }
    }
  }
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float z = expf(my_l - l0);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j)
    if (j < k) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
  if (active && lane < k) {
    ids[lane] = my_e;
    w[lane] = z / sum;
  }
}

// Top k of one row of E <= 256 logits on the 16 lanes of a row: lane `sub`
// holds the keys of experts sub, sub+16, ...; k rounds each take the row-wide
// largest key and retire it.  Keys are unique (they carry the expert index), so
// the result is the top k under the key order.  Lane sub == 0 of an active row
// writes ids[0..k) (descending logit, ties to the lower expert) and w[0..k)
// (it reads w back to form the weights).  All 64 lanes of the wavefront must
// call it, rows past the end with active = false; k is uniform.
__device__ __forceinline__ void rows_topk16(const float* logits_row, bool active, int E, int k, int sub,
                                            int32_t* ids, float* w) {
  uint64_t key[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int e = sub + 16 * r;
    key[r] = (active && e < E) ? topk_key(logits_row[e], e) : 0ull;  // 0 is below every real key
  }
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = max_u64(m, key[r]);
    m = row16_max64(m);
#pragma unroll
    for (int r = 0; r < 16; ++r) key[r] = key[r] == m ? 0ull : key[r];
    if (active && sub == 0) {
      ids[j] = topk_key_expert(m);
      w[j] = topk_key_logit(m);
    }
  }
  if (active && sub == 0) topk_weights_inplace(w, k);
}

}  // namespace mxmoe
