// The whole MoE layer for 1..16 rows in one kernel launch ("mono decode": one
// fused launch per MoE layer for a pure decode step of at most 16 tokens,
// article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and optimization",
// section "Serving with vLLM / What we Optimized").
//
// Structure.  A persistent grid (at most the device's co-resident capacity) of
// 4-wavefront workgroups.  Every wavefront is a worker that takes work units
// w, w + W, w + 2W, ... (W = number of wavefronts) from three lists in order:
//
//   phase 1  x quantization (one unit per row: MXFP4 and MXFP8 copies of x),
//            router logits (one unit per expert and row),
//            shared-expert gate/up (one unit per 16-row strip of Ws13 and
//            K-chunk of 4 tiles; waits for x quantization);
//   phase 2  each workgroup waits for all logits, takes the top k of every row
//            and builds the same expert list; then routed gate/up units
//            (selected expert, 16-row strip of W13, K-chunk);
//   phase 3  shared down units (16 rows of Ws2, K half) and routed down units
//            (selected expert, 16 rows of W2); each waits for its expert's
//            intermediate activations.
//
// A unit only ever waits for units earlier in this order, so with every
// workgroup resident the smallest unfinished unit can always progress.
// Gate/up partial sums go to the workspace; the wavefront that completes a
// 32-column block of an expert's intermediate (last arrival on a counter)
// sums the K-chunk partials in chunk order, applies SwiGLU and re-quantizes
// (MXFP4 routed, MXFP8 shared).  The wavefront that completes a 16-column
// block of the output combines sum_j w_j d_j + s (+ residual) in fixed order
// and rounds once to bf16.  Every sum has a fixed order independent of the
// number of rows, so output row t depends on x[t] only.
//
// Weights are streamed as whole 1 KiB tiles of the tiled MX layout straight
// into the operands of the scaled 16x16x128 matrix instruction; the weight
// loads of a unit are issued before its wait, so they overlap the dependency.
// Counters live in the workspace, are zero at rest and are reset by the last
// user before the launch ends.  Waits give up after about one second and then
// mark the workspace status word instead of hanging.
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWG = kThreads / kWave;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kDecodeMaxT * kMaxK;
constexpr uint64_t kSpinTicks = 100000000ull;  // ~1 s of the 100 MHz constant clock

enum { S_STATUS = 0, S_DONE = 1, S_ROUTER = 2, S_XQ = 3, S_SA = 4, S_HEAD = 64 };

struct DecodeArgs {
  int T, H, I, E, k, Is;
  int KT1, KC1, KS1, KG1;        // gate/up: K-tiles of H, tiles per chunk, chunks, scale groups
  int KT2, KG2;                  // routed down: K-tiles of I, scale groups
  int KTs2, KGs2, KCs2, SDS;     // shared down: K-tiles of I_s, scale groups, tiles per split, splits
  int G;
  const float* router_w;
  const float* router_bias;
  const uint8_t *w13, *w13s, *w2, *w2s, *ws13, *ws13s, *ws2, *ws2s;
  size_t w13_stride, w13s_stride, w2_stride, w2s_stride;
  const uint16_t* x;
  const uint16_t* residual;
  uint16_t* y;
  int32_t* ids_out;
  float* w_out;
  uint32_t *sync, *gu_cnt, *sgu_cnt, *a_ready, *comb_cnt;
  float* logits;
  uint8_t *xq4, *xs4, *xq8, *xs8;
  float *gu_part, *sgu_part;
  uint8_t *a4, *as4, *a8, *as8;
  float *d_part, *s_part;
};

struct Smem {
  float logits[kDecodeMaxT * 256];
  int32_t ids[kMaxSlots];
  float w[kMaxSlots];
  uint8_t elist[kMaxSlots];
  uint8_t ecount[kMaxSlots];
  uint8_t tl[kMaxSlots][kDecodeMaxT];  // slots routed to each selected expert, ascending
  int wave_cnt[kWavesPerWG];
  int D;
};

// ------------------------------------------------------------------ synchronisation
// Data handed from one workgroup to another (logits, quantized x, partial
// sums, intermediate codes) is written and read with relaxed agent-scope
// atomic accesses, which gfx950 issues with the sc1 bit: they are served at
// the device's coherence point, past the per-XCD L2 caches, so no L2
// write-back or invalidate is needed.  A producer waits for its stores to be
// acknowledged (vmcnt 0) before it bumps a counter; a consumer polls the
// counter and issues its data loads only after the poll has returned.
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ v4i ld_dev16(const uint8_t* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = ld_dev(q), b = ld_dev(q + 1);
  return v4i{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)(uint32_t)b, (int)(uint32_t)(b >> 32)};
}
__device__ __forceinline__ void st_dev16(uint8_t* p, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  st_dev(q, (uint64_t)w0 | ((uint64_t)w1 << 32));
  st_dev(q + 1, (uint64_t)w2 | ((uint64_t)w3 << 32));
}
// Wait until every vector memory access of this wavefront is acknowledged.
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Keeps the compiler from moving memory accesses across this point.
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

__device__ __forceinline__ void wait_count(uint32_t* ctr, uint32_t target, uint32_t* status) {
  const uint64_t t0 = wall_clock64();
  while (ld_dev(ctr) < target) {
    if (ld_dev(status)) return;
    if (wall_clock64() - t0 > kSpinTicks) {
      __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ void wave_wait(uint32_t* ctr, uint32_t target, uint32_t* status, int lane) {
  compiler_fence();
  if (lane == 0) wait_count(ctr, target, status);
  compiler_fence();
}

__device__ __forceinline__ void wave_release_add(uint32_t* ctr, int lane) {
  compiler_fence();
  drain_stores();
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every lane of the wavefront whose arrival completes the count.
__device__ __forceinline__ bool wave_arrive_last(uint32_t* ctr, uint32_t target, int lane) {
  compiler_fence();
  drain_stores();
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = (uint32_t)__shfl((int)old, 0);
  compiler_fence();
  return old + 1 == target;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.f + expf(-g))) * u; }

// ------------------------------------------------------------------ phase 1
__device__ void unit_xq(const DecodeArgs& A, int t, int lane) {
  const int nb = A.H / 32;
  for (int b = lane; b < nb; b += kWave) {
    const uint4* src = reinterpret_cast<const uint4*>(A.x + (size_t)t * A.H + 32 * b);
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
    uint32_t words[8];
    uint32_t s = quant_block32<FP4>(bits, words);
    st_dev16(A.xq4 + (size_t)t * (A.H / 2) + 16 * b, words[0], words[1], words[2], words[3]);
    st_dev(&A.xs4[t * nb + b], (uint8_t)s);
    if (A.Is) {
      s = quant_block32<FP8>(bits, words);
      uint8_t* dst = A.xq8 + (size_t)t * A.H + 32 * b;
      st_dev16(dst, words[0], words[1], words[2], words[3]);
      st_dev16(dst + 16, words[4], words[5], words[6], words[7]);
      st_dev(&A.xs8[t * nb + b], (uint8_t)s);
    }
  }
  wave_release_add(&A.sync[S_XQ], lane);
}

__device__ void unit_router(const DecodeArgs& A, int e, int t, int lane) {
  float p = router_lane_partial(A.x + (size_t)t * A.H, A.router_w + (size_t)e * A.H, A.H, lane);
  p = wave_sum_butterfly(p);
  if (A.router_bias) p = p + A.router_bias[e];
  if (lane == 0) st_dev(&A.logits[t * A.E + e], p);
  wave_release_add(&A.sync[S_ROUTER], lane);
}

__device__ void finalize_shared(const DecodeArgs& A, int nb, int lane) {
  const int col = lane & 31, half = lane >> 5;
  const int Is = A.Is;
  for (int m0 = 0; m0 < A.T; m0 += 2) {
    const int m = m0 + half;
    const bool act = m < A.T;
    float g = 0.f, u = 0.f;
    if (act) {
      const float* gp = A.sgu_part + (size_t)m * A.KS1 * (2 * Is) + 32 * nb + col;
      g = ld_dev(gp);
      u = ld_dev(gp + Is);
      for (int kc = 1; kc < A.KS1; ++kc) {
        g = g + ld_dev(gp + (size_t)kc * 2 * Is);
        u = u + ld_dev(gp + (size_t)kc * 2 * Is + Is);
      }
    }
    const uint32_t ab = __float_as_uint(silu_mul(g, u));
    const int e = block_exponent<FP8>(wave_max_u32(ab & 0x7fffffffu, 32));
    const uint32_t code = quant_elem<FP8>(ab, e);
    if (act) {
      st_dev(&A.a8[(size_t)m * Is + 32 * nb + col], (uint8_t)code);
      if (col == 0) st_dev(&A.as8[m * (Is / 32) + nb], (uint8_t)(e + 127));
    }
  }
}

__device__ void unit_shared_gu(const DecodeArgs& A, int st, int kc, int lane) {
  const int Is = A.Is;
  const uint8_t* wb = A.ws13 + ((size_t)st * A.KT1 + (size_t)kc * A.KC1) * 2048 + lane * 16;
  v4i B0[4], B1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KC1) {
      B0[i] = load_stream16(wb + i * 2048);
      B1[i] = load_stream16(wb + i * 2048 + 1024);
    }
  const int kt0 = kc * A.KC1;
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(
      A.ws13s + (((size_t)st * A.KG1 + kt0 / 4) * 64 + lane) * 4);
  wave_wait(&A.sync[S_XQ], (uint32_t)A.T, A.sync, lane);
  const int m = lane & 15, q = lane >> 4;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KC1) {
      const int kt = kt0 + i;
      v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      uint32_t sa = 127;
      if (m < A.T) {
        const uint8_t* ap = A.xq8 + (size_t)m * A.H + kt * 128 + 16 * q;
        a0 = ld_dev16(ap);
        a1 = ld_dev16(ap + 64);
        sa = ld_dev(&A.xs8[m * (A.H / 32) + 4 * kt + q]);
      }
      acc = mfma_fp8(a0, a1, B0[i], B1[i], acc, sa, (sb >> (8 * ((kt0 + i) & 3))) & 0xffu);
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < A.T) st_dev(&A.sgu_part[((size_t)mm * A.KS1 + kc) * (2 * Is) + 16 * st + (lane & 15)], acc[r]);
  }
  const int nb = ((16 * st) % Is) / 32;
  if (wave_arrive_last(&A.sgu_cnt[nb], 4 * A.KS1, lane)) {
    finalize_shared(A, nb, lane);
    if (lane == 0) st_dev(&A.sgu_cnt[nb], 0u);
    wave_release_add(&A.sync[S_SA], lane);
  }
}

// ------------------------------------------------------------------ phase 2
__device__ void build_expert_list(const DecodeArgs& A, Smem& sm, int lane, int wave) {
  const int S = A.T * A.k;
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < A.E)
    for (int s = 0; s < S; ++s) cnt += (sm.ids[s] == e);
  const bool used = cnt > 0;
  const uint64_t mask = __ballot(used);
  if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sm.wave_cnt[w];
  if (used) {
    const int dd = base + __popcll(mask & ((1ull << lane) - 1ull));
    sm.elist[dd] = (uint8_t)e;
    sm.ecount[dd] = (uint8_t)cnt;
    int pos = 0;
    for (int s = 0; s < S; ++s)
      if (sm.ids[s] == e) sm.tl[dd][pos++] = (uint8_t)s;
  }
  if (threadIdx.x == 0) {
    int D = 0;
    for (int w = 0; w < kWavesPerWG; ++w) D += sm.wave_cnt[w];
    sm.D = D;
  }
}

__device__ void finalize_routed(const DecodeArgs& A, const Smem& sm, int dd, int nb, int lane) {
  const int col = lane & 31, half = lane >> 5;
  const int n = sm.ecount[dd], I = A.I;
  for (int m0 = 0; m0 < n; m0 += 2) {
    const int m = m0 + half;
    const bool act = m < n;
    const int slot = act ? sm.tl[dd][m] : 0;
    float g = 0.f, u = 0.f;
    if (act) {
      const float* gp = A.gu_part + (size_t)slot * A.KS1 * (2 * I) + 32 * nb + col;
      g = ld_dev(gp);
      u = ld_dev(gp + I);
      for (int kc = 1; kc < A.KS1; ++kc) {
        g = g + ld_dev(gp + (size_t)kc * 2 * I);
        u = u + ld_dev(gp + (size_t)kc * 2 * I + I);
      }
    }
    const uint32_t ab = __float_as_uint(silu_mul(g, u));
    const int e = block_exponent<FP4>(wave_max_u32(ab & 0x7fffffffu, 32));
    const uint32_t code = quant_elem<FP4>(ab, e);
    const uint32_t hi = (uint32_t)__shfl_down((int)code, 1);
    if (act && !(col & 1))
      st_dev(&A.a4[(size_t)slot * (I / 2) + 16 * nb + col / 2], (uint8_t)((code & 0xfu) | ((hi & 0xfu) << 4)));
    if (act && col == 0) st_dev(&A.as4[slot * (I / 32) + nb], (uint8_t)(e + 127));
  }
}

__device__ void unit_routed_gu(const DecodeArgs& A, const Smem& sm, int dd, int st, int kc, int lane) {
  const int e = sm.elist[dd], n = sm.ecount[dd];
  const int I = A.I;
  const uint8_t* wb = A.w13 + (size_t)e * A.w13_stride +
                      ((size_t)st * A.KT1 + (size_t)kc * A.KC1) * 1024 + lane * 16;
  v4i B[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KC1) B[i] = load_stream16(wb + i * 1024);
  const int kt0 = kc * A.KC1;
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(
      A.w13s + (size_t)e * A.w13s_stride + (((size_t)st * A.KG1 + kt0 / 4) * 64 + lane) * 4);
  const int m = lane & 15, q = lane >> 4;
  const int tok = m < n ? sm.tl[dd][m] / A.k : -1;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KC1) {
      const int kt = kt0 + i;
      v4i a = {0, 0, 0, 0};
      uint32_t sa = 127;
      if (tok >= 0) {
        a = ld_dev16(A.xq4 + (size_t)tok * (A.H / 2) + kt * 64 + 16 * q);
        sa = ld_dev(&A.xs4[tok * (A.H / 32) + 4 * kt + q]);
      }
      acc = mfma_fp4(a, B[i], acc, sa, (sb >> (8 * ((kt0 + i) & 3))) & 0xffu);
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < n)
      st_dev(&A.gu_part[((size_t)sm.tl[dd][mm] * A.KS1 + kc) * (2 * I) + 16 * st + (lane & 15)], acc[r]);
  }
  const int nb = ((16 * st) % I) / 32;
  uint32_t* cnt = &A.gu_cnt[e * (I / 32) + nb];
  if (wave_arrive_last(cnt, 4 * A.KS1, lane)) {
    finalize_routed(A, sm, dd, nb, lane);
    if (lane == 0) st_dev(cnt, 0u);
    wave_release_add(&A.a_ready[e], lane);
  }
}

// ------------------------------------------------------------------ phase 3
__device__ void combine(const DecodeArgs& A, const Smem& sm, int hs, int lane) {
  const int H = A.H, k = A.k;
  for (int idx = lane; idx < A.T * 16; idx += kWave) {
    const int t = idx >> 4, h = 16 * hs + (idx & 15);
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(sm.w[t * k + j], ld_dev(&A.d_part[(size_t)(t * k + j) * H + h]), acc);
    if (A.Is) {
      float s = ld_dev(&A.s_part[(size_t)t * H + h]);
      for (int kh = 1; kh < A.SDS; ++kh) s = s + ld_dev(&A.s_part[((size_t)kh * kDecodeMaxT + t) * H + h]);
      acc = acc + s;
    }
    if (A.residual) acc = acc + bf16_to_f32(A.residual[(size_t)t * H + h]);
    A.y[(size_t)t * H + h] = f32_to_bf16(acc);
  }
}

__device__ void arrive_output(const DecodeArgs& A, const Smem& sm, int hs, int lane) {
  uint32_t* cnt = &A.comb_cnt[hs];
  if (wave_arrive_last(cnt, (uint32_t)(A.SDS + sm.D), lane)) {
    combine(A, sm, hs, lane);
    if (lane == 0) st_dev(cnt, 0u);
  }
}

__device__ void unit_shared_down(const DecodeArgs& A, const Smem& sm, int hs, int kh, int lane) {
  const int Is = A.Is;
  const int kt0 = kh * A.KCs2;
  const uint8_t* wb = A.ws2 + ((size_t)hs * A.KTs2 + kt0) * 2048 + lane * 16;
  v4i B0[4], B1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KCs2) {
      B0[i] = load_stream16(wb + i * 2048);
      B1[i] = load_stream16(wb + i * 2048 + 1024);
    }
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(
      A.ws2s + (((size_t)hs * A.KGs2 + kt0 / 4) * 64 + lane) * 4);
  wave_wait(&A.sync[S_SA], (uint32_t)(Is / 32), A.sync, lane);
  const int m = lane & 15, q = lane >> 4;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < A.KCs2) {
      const int kt = kt0 + i;
      v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      uint32_t sa = 127;
      if (m < A.T) {
        const uint8_t* ap = A.a8 + (size_t)m * Is + kt * 128 + 16 * q;
        a0 = ld_dev16(ap);
        a1 = ld_dev16(ap + 64);
        sa = ld_dev(&A.as8[m * (Is / 32) + 4 * kt + q]);
      }
      acc = mfma_fp8(a0, a1, B0[i], B1[i], acc, sa, (sb >> (8 * ((kt0 + i) & 3))) & 0xffu);
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < A.T) st_dev(&A.s_part[((size_t)kh * kDecodeMaxT + mm) * A.H + 16 * hs + (lane & 15)], acc[r]);
  }
  arrive_output(A, sm, hs, lane);
}

__device__ void unit_routed_down(const DecodeArgs& A, const Smem& sm, int dd, int hs, int lane) {
  const int e = sm.elist[dd], n = sm.ecount[dd];
  const int I = A.I;
  const uint8_t* wb = A.w2 + (size_t)e * A.w2_stride + (size_t)hs * A.KT2 * 1024 + lane * 16;
  const uint8_t* sbp = A.w2s + (size_t)e * A.w2s_stride + ((size_t)hs * A.KG2 * 64 + lane) * 4;
  const int m = lane & 15, q = lane >> 4;
  const int slot = m < n ? sm.tl[dd][m] : -1;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 0; kt0 < A.KT2; kt0 += 8) {
    v4i B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (kt0 + i < A.KT2) B[i] = load_stream16(wb + (size_t)(kt0 + i) * 1024);
    const uint32_t sb0 = *reinterpret_cast<const uint32_t*>(sbp + (size_t)(kt0 / 4) * 256);
    const uint32_t sb1 = kt0 + 4 < A.KT2 ? *reinterpret_cast<const uint32_t*>(sbp + (size_t)(kt0 / 4 + 1) * 256) : 0u;
    if (kt0 == 0) wave_wait(&A.a_ready[e], (uint32_t)(I / 32), A.sync, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (kt0 + i < A.KT2) {
        const int kt = kt0 + i;
        v4i a = {0, 0, 0, 0};
        uint32_t sa = 127;
        if (slot >= 0) {
          a = ld_dev16(A.a4 + (size_t)slot * (I / 2) + kt * 64 + 16 * q);
          sa = ld_dev(&A.as4[slot * (I / 32) + 4 * kt + q]);
        }
        const uint32_t sbw = i < 4 ? sb0 : sb1;
        acc = mfma_fp4(a, B[i], acc, sa, (sbw >> (8 * (i & 3))) & 0xffu);
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < n) st_dev(&A.d_part[(size_t)sm.tl[dd][mm] * A.H + 16 * hs + (lane & 15)], acc[r]);
  }
  arrive_output(A, sm, hs, lane);
}

// ------------------------------------------------------------------ kernel
__global__ void __launch_bounds__(kThreads) fused_decode_kernel(DecodeArgs A) {
  __shared__ Smem sm;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int W = gridDim.x * kWavesPerWG;
  const int wid = blockIdx.x * kWavesPerWG + wave;
  const int T = A.T, E = A.E;

  // phase 1
  const int n_xq = T, n_router = T * E;
  const int n_sgu = A.Is ? (2 * A.Is / 16) * A.KS1 : 0;
  for (int u = wid; u < n_xq + n_router + n_sgu; u += W) {
    if (u < n_xq) {
      unit_xq(A, u, lane);
    } else if (u < n_xq + n_router) {
      const int v = u - n_xq;
      unit_router(A, v / T, v % T, lane);
    } else {
      const int v = u - n_xq - n_router;
      unit_shared_gu(A, v / A.KS1, v % A.KS1, lane);
    }
  }

  // phase 2: routing, identical in every workgroup
  if (threadIdx.x == 0) {
    wait_count(&A.sync[S_ROUTER], (uint32_t)(T * E), A.sync);
    wait_count(&A.sync[S_XQ], (uint32_t)T, A.sync);
  }
  __syncthreads();
  compiler_fence();
  for (int i = threadIdx.x; i < T * E; i += kThreads) sm.logits[i] = ld_dev(&A.logits[i]);
  __syncthreads();
  for (int t = wave; t < T; t += kWavesPerWG)
    wave_topk(sm.logits + t * E, E, A.k, lane, sm.ids + t * A.k, sm.w + t * A.k);
  __syncthreads();
  build_expert_list(A, sm, lane, wave);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < T * A.k; i += kThreads) {
      if (A.ids_out) A.ids_out[i] = sm.ids[i];
      if (A.w_out) A.w_out[i] = sm.w[i];
    }
  }
  const int D = sm.D;
  const int per_expert = (2 * A.I / 16) * A.KS1;
  for (int u = wid; u < D * per_expert; u += W) {
    const int dd = u / per_expert, r = u % per_expert;
    unit_routed_gu(A, sm, dd, r / A.KS1, r % A.KS1, lane);
  }

  // phase 3
  const int nhs = A.H / 16;
  const int n_sd = A.Is ? nhs * A.SDS : 0;
  for (int u = wid; u < n_sd + D * nhs; u += W) {
    if (u < n_sd) {
      unit_shared_down(A, sm, u / A.SDS, u % A.SDS, lane);
    } else {
      const int v = u - n_sd;
      unit_routed_down(A, sm, v / nhs, v % nhs, lane);
    }
  }

  // exit: the last workgroup resets the launch-wide counters
  __syncthreads();
  if (threadIdx.x == 0) {
    compiler_fence();
    drain_stores();
    const uint32_t old = __hip_atomic_fetch_add(&A.sync[S_DONE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    compiler_fence();
    if (old + 1 == (uint32_t)A.G) {
      st_dev(&A.sync[S_ROUTER], 0u);
      st_dev(&A.sync[S_XQ], 0u);
      st_dev(&A.sync[S_SA], 0u);
      for (int e = 0; e < E; ++e) st_dev(&A.a_ready[e], 0u);
      drain_stores();
      st_dev(&A.sync[S_DONE], 0u);
    }
  }
}

// ------------------------------------------------------------------ workspace map
struct Carve {
  size_t sync, gu_cnt, sgu_cnt, a_ready, comb_cnt, sync_end;
  size_t logits, xq4, xs4, xq8, xs8, gu_part, sgu_part, a4, as4, a8, as8, d_part, s_part, total;
};

int pick_chunk(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }

Carve carve(const moe_layer_t& L) {
  const size_t T = kDecodeMaxT, H = L.hidden, I = L.inter, E = L.num_experts, k = L.top_k,
               Is = L.shared_inter;
  const size_t KS1 = (H / 128) / pick_chunk((int)(H / 128));
  const size_t SDS = Is ? (Is / 128) / pick_chunk((int)(Is / 128)) : 0;
  Carve c{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  c.sync = take(S_HEAD * 4);
  c.gu_cnt = take(E * (I / 32) * 4);
  c.sgu_cnt = take((Is / 32) * 4 + 4);
  c.a_ready = take(E * 4);
  c.comb_cnt = take((H / 16) * 4);
  c.sync_end = o;
  c.logits = take(T * E * 4);
  c.xq4 = take(T * H / 2);
  c.xs4 = take(T * H / 32);
  c.xq8 = take(T * H);
  c.xs8 = take(T * H / 32);
  c.gu_part = take(T * k * KS1 * 2 * I * 4);
  c.sgu_part = take(T * KS1 * 2 * Is * 4 + 4);
  c.a4 = take(T * k * I / 2);
  c.as4 = take(T * k * I / 32);
  c.a8 = take(T * Is + 4);
  c.as8 = take(T * Is / 32 + 4);
  c.d_part = take(T * k * H * 4);
  c.s_part = take((SDS ? SDS : 1) * T * H * 4);
  c.total = o;
  return c;
}

int grid_size() {
  static int cached_dev = -1, cached_grid = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == cached_dev) return cached_grid;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_decode_kernel, kThreads, 0) != hipSuccess)
    return 0;
  if (occ > 2) occ = 2;
  cached_dev = dev;
  cached_grid = occ * cus;
  return cached_grid;
}

}  // namespace

size_t decode_ws_bytes(const moe_layer_t& L) { return carve(L).total; }
size_t decode_sync_bytes(const moe_layer_t& L) { return carve(L).sync_end; }

hipError_t launch_decode(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                         uint16_t* y, void* ws, int32_t* ids_out, float* w_out, hipStream_t stream) {
  const Carve c = carve(L);
  char* base = reinterpret_cast<char*>(ws);
  DecodeArgs A{};
  A.T = T;
  A.H = L.hidden;
  A.I = L.inter;
  A.E = L.num_experts;
  A.k = L.top_k;
  A.Is = L.shared_inter;
  A.KT1 = A.H / 128;
  A.KC1 = pick_chunk(A.KT1);
  A.KS1 = A.KT1 / A.KC1;
  A.KG1 = (A.KT1 + 3) / 4;
  A.KT2 = A.I / 128;
  A.KG2 = (A.KT2 + 3) / 4;
  A.KTs2 = A.Is / 128;
  A.KGs2 = (A.KTs2 + 3) / 4;
  A.KCs2 = A.Is ? pick_chunk(A.KTs2) : 1;
  A.SDS = A.Is ? A.KTs2 / A.KCs2 : 0;
  A.G = grid_size();
  if (A.G <= 0) return hipErrorInvalidDeviceFunction;
  A.router_w = L.router_w;
  A.router_bias = L.router_bias;
  A.w13 = L.w13;
  A.w13s = L.w13_scale;
  A.w2 = L.w2;
  A.w2s = L.w2_scale;
  A.ws13 = L.ws13;
  A.ws13s = L.ws13_scale;
  A.ws2 = L.ws2;
  A.ws2s = L.ws2_scale;
  A.w13_stride = tiled_codes_bytes(2 * A.I, A.H, MX_FMT_FP4);
  A.w13s_stride = tiled_scales_bytes(2 * A.I, A.H);
  A.w2_stride = tiled_codes_bytes(A.H, A.I, MX_FMT_FP4);
  A.w2s_stride = tiled_scales_bytes(A.H, A.I);
  A.x = x;
  A.residual = residual;
  A.y = y;
  A.ids_out = ids_out;
  A.w_out = w_out;
  A.sync = reinterpret_cast<uint32_t*>(base + c.sync);
  A.gu_cnt = reinterpret_cast<uint32_t*>(base + c.gu_cnt);
  A.sgu_cnt = reinterpret_cast<uint32_t*>(base + c.sgu_cnt);
  A.a_ready = reinterpret_cast<uint32_t*>(base + c.a_ready);
  A.comb_cnt = reinterpret_cast<uint32_t*>(base + c.comb_cnt);
  A.logits = reinterpret_cast<float*>(base + c.logits);
  A.xq4 = reinterpret_cast<uint8_t*>(base + c.xq4);
  A.xs4 = reinterpret_cast<uint8_t*>(base + c.xs4);
  A.xq8 = reinterpret_cast<uint8_t*>(base + c.xq8);
  A.xs8 = reinterpret_cast<uint8_t*>(base + c.xs8);
  A.gu_part = reinterpret_cast<float*>(base + c.gu_part);
  A.sgu_part = reinterpret_cast<float*>(base + c.sgu_part);
  A.a4 = reinterpret_cast<uint8_t*>(base + c.a4);
  A.as4 = reinterpret_cast<uint8_t*>(base + c.as4);
  A.a8 = reinterpret_cast<uint8_t*>(base + c.a8);
  A.as8 = reinterpret_cast<uint8_t*>(base + c.as8);
  A.d_part = reinterpret_cast<float*>(base + c.d_part);
  A.s_part = reinterpret_cast<float*>(base + c.s_part);
  hipLaunchKernelGGL(fused_decode_kernel, dim3(A.G), dim3(kThreads), 0, stream, A);
  return hipGetLastError();
}

}  // namespace mxmoe
