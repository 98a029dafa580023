// The whole MoE layer for 1..16 rows in one kernel launch ("mono decode": one
// fused launch per MoE layer for a pure decode step of at most 16 tokens,
// article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and optimization",
// section "Serving with vLLM / What we Optimized").
//
// Structure.  A persistent grid of G 4-wavefront workgroups (G at most the
// device's co-resident capacity).  Workgroup b takes work units b, b+G, ...
// from three lists, in order:
//
//   phase 1  x quantization (one unit per row: MXFP4 and MXFP8 copies),
//            router logits (one unit per expert, all rows),
//            shared-expert gate/up (one unit per 32-column block of the shared
//            intermediate and K-chunk: the four waves take the two gate and two
//            up strips of 16 rows);
//   phase 2  every workgroup waits for all logits, takes the top k of each row,
//            builds the same list of selected experts and stages the MXFP4 x
//            in LDS; then routed gate/up units (selected expert, 32-column
//            block, share S of the K-chunks);
//   phase 3  shared down units and routed down units (64 output columns, one
//            strip of 16 per wave), then the combine.
//
// A unit only waits for units of an earlier phase, so with every workgroup
// resident the smallest unfinished unit can always progress.
//
// Arithmetic (fixed, independent of the number of rows and of the grid): every
// dot product is cut into K-chunks of CT tiles of 128; a chunk is one chain of
// scaled 16x16x128 matrix instructions in tile order starting from zero, and
// the chunk sums are added in chunk order in fp32.  A routed gate/up block may
// be split over S workgroups (S is picked per launch to fill the grid); the
// chunk sums then travel through the workspace and the workgroup that
// completes the block adds them in the same order, so S never changes a bit.
// SwiGLU and re-quantization (MXFP4 routed, MXFP8 shared) follow on the
// 32-column block; the combine adds sum_j w_j d_j in j order, then s, then the
// residual, and rounds once to bf16.  Output row t therefore depends on x[t]
// only.
//
// Weights stream as whole 1 KiB tiles of the tiled MX layout straight into the
// matrix-instruction operands; a workgroup issues the next unit's weight loads
// before the current unit's epilogue.
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWG = kThreads / kWave;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kDecodeMaxT * kMaxK;
constexpr int kMaxChunksPerUnit = 6;   // routed gate/up chunks one unit holds in registers
constexpr int kGuRegTiles = 24;        // = kMaxChunksPerUnit * 4
constexpr int kDownRegTiles = 16;      // FP4 tiles (FP8 tiles count double) per down batch
constexpr uint64_t kSpinTicks = 100000000ull;  // ~1 s of the 100 MHz constant clock

// Every counter sits on a 256-byte line of its own: device-scope atomics on
// one line are serialized by the memory side.
constexpr int kLine = 64;  // words
__device__ __forceinline__ uint32_t* ctr(uint32_t* base, int i) { return base + (size_t)i * kLine; }
// Lines of the sync block: status, done, x-quant, shared-intermediate ready,
// grid size of the last call, then kRouterCtrs router counters.
enum { S_STATUS = 0, S_DONE = 1, S_XQ = 2, S_SA = 3, S_GRID = 4, S_ROUTER = 8 };
constexpr int kRouterCtrs = 8;
constexpr int kSyncLines = S_ROUTER + kRouterCtrs;

// Timestamps each workgroup records (100 MHz device clock).
enum { TR_START = 0, TR_P1 = 1, TR_ROUTED = 2, TR_P2 = 3, TR_P3 = 4, TR_UNIT1 = 5, TR_LOGITS = 6, TR_XQ = 7 };

struct DecodeArgs {
  int T, H, I, E, k, Is, G;
  // K geometry: KT = K-tiles of 128, CT = tiles per chunk, KS = chunks, KG = scale groups
  int KT1, CT1, KS1, KG1;  // K = H (gate/up)
  int KT2, CT2, KS2, KG2;  // K = I (routed down)
  int KTs, CTs, KSs, KGs;  // K = I_s (shared down)
  int S;                   // workgroups sharing one routed gate/up block
  const float* router_w;
  const float* router_bias;
  const uint8_t *w13, *w13s, *w2, *w2s, *ws13, *ws13s, *ws2, *ws2s;
  size_t w13_stride, w13s_stride, w2_stride, w2s_stride;
  const uint16_t* x;
  const uint16_t* residual;
  uint16_t* y;
  int32_t* ids_out;
  float* w_out;
  uint32_t *sync, *gu_cnt, *sgu_cnt, *a_ready, *comb_cnt, *sd_cnt;
  float* logits;
  uint8_t *xq4, *xs4, *xq8, *xs8;
  float *gu_part, *sgu_part;
  uint8_t *a4, *as4, *a8, *as8;
  float *d_part, *s_part;
  uint64_t* trace;
};

struct Smem {
  int32_t ids[kMaxSlots];
  float w[kMaxSlots];
  uint8_t elist[kMaxSlots];
  uint8_t ecount[kMaxSlots];
  uint8_t tl[kMaxSlots][kDecodeMaxT];  // slots routed to each selected expert, ascending
  float fin[2][32][kDecodeMaxT];       // gate / up sums of one 32-column block
  int wave_cnt[kWavesPerWG];
  int D;
  int flag;
};

// ------------------------------------------------------------------ synchronisation
// Data handed from one workgroup to another (logits, quantized x, partial
// sums, intermediate codes) is written and read with relaxed agent-scope
// atomic accesses, which gfx950 issues with the sc1 bit: they are served at
// the device's coherence point, past the per-XCD L2 caches, so no L2
// write-back or invalidate is needed.  Each wavefront waits for its stores to
// be acknowledged (vmcnt 0) before the workgroup barrier that precedes a
// counter bump; a consumer polls the counter and issues its data loads only
// after the poll has returned.
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

__device__ __forceinline__ void wait_count(uint32_t* c, uint32_t target, uint32_t* status) {
  const uint64_t t0 = wall_clock64();
  while (ld_dev(c) < target) {
    if (ld_dev(status)) return;
    if (wall_clock64() - t0 > kSpinTicks) {
      __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Workgroup-wide wait: thread 0 polls, the barrier releases everyone.
__device__ __forceinline__ void wg_wait(uint32_t* c, uint32_t target, uint32_t* status) {
  compiler_fence();
  if (threadIdx.x == 0) wait_count(c, target, status);
  __syncthreads();
  compiler_fence();
}

// All of the workgroup's stores are acknowledged, then thread 0 adds to *c.
__device__ __forceinline__ void wg_release_add(uint32_t* c, uint32_t v) {
  compiler_fence();
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// As wg_release_add with 1; true in every thread if this arrival completed
// the count to `target`.
__device__ __forceinline__ bool wg_arrive_last(uint32_t* c, uint32_t target, Smem& sm) {
  compiler_fence();
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    sm.flag = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == target;
  __syncthreads();
  compiler_fence();
  return sm.flag != 0;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.f + expf(-g))) * u; }

__device__ __forceinline__ uint32_t scale_byte(uint32_t word, int tile) { return (word >> (8 * (tile & 3))) & 0xffu; }

// Strip of a 32-column intermediate block nb handled by wave w: waves 0, 1
// take the gate rows, waves 2, 3 the up rows (I_ = intermediate size).
__device__ __forceinline__ int gu_strip(int nb, int w, int I_) {
  return w < 2 ? 2 * nb + w : I_ / 16 + 2 * nb + (w - 2);
}

// ------------------------------------------------------------------ phase 1
// x quantization: block task i of T * nb * F (nb = H/32 blocks per row, F = 2
// formats with a shared expert, else 1) is (row, format, block); eight lanes
// take one task, four elements each, and agree on the block scale with three
// butterfly steps.  A unit is 32 tasks.
__device__ __forceinline__ void unit_xq(const DecodeArgs& A, int u) {
  const int nb = A.H / 32, F = A.Is ? 2 : 1;
  const int task = u * (kThreads / 8) + (int)threadIdx.x / 8;
  const int j = threadIdx.x & 7;
  const bool act = task < A.T * nb * F;
  int t = 0, fp8 = 0, b = 0;
  if (act) {
    t = task / (nb * F);
    const int r = task % (nb * F);
    fp8 = r / nb;
    b = r % nb;
  }
  uint32_t bits[4] = {0u, 0u, 0u, 0u};
  if (act) {
    const uint2 v = *reinterpret_cast<const uint2*>(A.x + (size_t)t * A.H + 32 * b + 4 * j);
    bits[0] = v.x << 16;
    bits[1] = v.x & 0xffff0000u;
    bits[2] = v.y << 16;
    bits[3] = v.y & 0xffff0000u;
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) am = max(am, bits[i] & 0x7fffffffu);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 8));
  if (act) {
    if (fp8) {
      const int e = block_exponent<FP8>(am);
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= quant_elem<FP8>(bits[i], e) << (8 * i);
      st_dev(reinterpret_cast<uint32_t*>(A.xq8 + (size_t)t * A.H + 32 * b + 4 * j), word);
      if (j == 0) st_dev(&A.xs8[t * nb + b], (uint8_t)(e + 127));
    } else {
      const int e = block_exponent<FP4>(am);
      uint32_t half = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) half |= quant_elem<FP4>(bits[i], e) << (4 * i);
      st_dev(reinterpret_cast<uint16_t*>(A.xq4 + (size_t)t * (A.H / 2) + 16 * b + 2 * j), (uint16_t)half);
      if (j == 0) st_dev(&A.xs4[t * nb + b], (uint8_t)(e + 127));
    }
  }
  wg_release_add(ctr(A.sync, S_XQ), 1u);
}

__host__ __device__ __forceinline__ int xq_units(int T, int H, int Is) {
  return (T * (H / 32) * (Is ? 2 : 1) + kThreads / 8 - 1) / (kThreads / 8);
}

// Logits of expert e for all rows; wave w takes rows w, w+4, ...  Same
// per-row arithmetic as router_lane_partial: each batch of up to 16 strides
// of the expert's weights is loaded once, then the rows go through it two at
// a time.
__device__ __forceinline__ void unit_router(const DecodeArgs& A, int e, int lane, int wave) {
  const float* wrow = A.router_w + (size_t)e * A.H;
  const int H = A.H;
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  int nr = 0;
  for (int t = wave; t < A.T; t += kWavesPerWG) ++nr;
  for (int h0 = 4 * lane; h0 < H; h0 += 16 * 256) {
    float4 w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (h0 + 256 * j < H) w[j] = *reinterpret_cast<const float4*>(wrow + h0 + 256 * j);
#pragma unroll
    for (int r0 = 0; r0 < 4; r0 += 2) {
      if (r0 < nr) {
        uint2 xv[2][16];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (r0 + r < nr) {
            const uint16_t* xr = A.x + (size_t)(wave + 4 * (r0 + r)) * H;
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (h0 + 256 * j < H) xv[r][j] = *reinterpret_cast<const uint2*>(xr + h0 + 256 * j);
          }
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (r0 + r < nr) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (h0 + 256 * j < H) {
                float& acc = p[r0 + r];
                acc = fmaf(bf16_to_f32(xv[r][j].x & 0xffffu), w[j].x, acc);
                acc = fmaf(bf16_to_f32(xv[r][j].x >> 16), w[j].y, acc);
                acc = fmaf(bf16_to_f32(xv[r][j].y & 0xffffu), w[j].z, acc);
                acc = fmaf(bf16_to_f32(xv[r][j].y >> 16), w[j].w, acc);
              }
          }
      }
    }
  }
  const float b = A.router_bias ? A.router_bias[e] : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < nr) {
      float v = wave_sum_butterfly(p[r]);
      if (A.router_bias) v = v + b;
      if (lane == 0) st_dev(&A.logits[(wave + 4 * r) * A.E + e], v);
    }
  wg_release_add(ctr(A.sync, S_ROUTER + e % kRouterCtrs), 1u);
}

// SwiGLU of the gate / up sums in sm.fin for rows m < n (slot of row m:
// slot_of(m)), re-quantized per 32-column block nb.  Wave w takes rows
// 2w, 2w+1 (+8, ...): half a wave per row, one column per lane.
template <class F, class SlotOf>
__device__ __forceinline__ void swiglu_requant(const Smem& sm, int n, int nb, int inter, uint8_t* codes,
                               uint8_t* scales, SlotOf slot_of, int lane, int wave) {
  const int col = lane & 31, half = lane >> 5;
  for (int m0 = 2 * wave; m0 < n; m0 += 2 * kWavesPerWG) {
    const int m = m0 + half;
    const bool act = m < n;
    const float g = act ? sm.fin[0][col][m] : 0.f;
    const float u = act ? sm.fin[1][col][m] : 0.f;
    const uint32_t ab = __float_as_uint(silu_mul(g, u));
    const int e = block_exponent<F>(wave_max_u32(ab & 0x7fffffffu, 32));
    const uint32_t code = quant_elem<F>(ab, e);
    const int slot = act ? slot_of(m) : 0;
    if constexpr (F::MB == 1) {
      const uint32_t hi = (uint32_t)__shfl_down((int)code, 1);
      if (act && !(col & 1))
        st_dev(&codes[(size_t)slot * (inter / 2) + 16 * nb + col / 2], (uint8_t)((code & 0xfu) | ((hi & 0xfu) << 4)));
    } else {
      if (act) st_dev(&codes[(size_t)slot * inter + 32 * nb + col], (uint8_t)code);
    }
    if (act && col == 0) st_dev(&scales[slot * (inter / 32) + nb], (uint8_t)(e + 127));
  }
}

__device__ __forceinline__ void unit_shared_gu(const DecodeArgs& A, Smem& sm, int nb, int kc, int lane, int wave) {
  const int Is = A.Is, CT = A.CT1;
  const int st = gu_strip(nb, wave, Is);
  const uint8_t* wb = A.ws13 + ((size_t)st * A.KT1 + (size_t)kc * CT) * 2048 + lane * 16;
  v4i B0[4], B1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < CT) {
      B0[i] = load_stream16(wb + i * 2048);
      B1[i] = load_stream16(wb + i * 2048 + 1024);
    }
  const int kt0 = kc * CT;
  const uint32_t sb = *reinterpret_cast<const uint32_t*>(A.ws13s + (((size_t)st * A.KG1 + kt0 / 4) * 64 + lane) * 4);
  wg_wait(ctr(A.sync, S_XQ), (uint32_t)xq_units(A.T, A.H, A.Is), A.sync);
  const int m = lane & 15, q = lane >> 4;
  v4i a0[4], a1[4];
  uint32_t sa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] = a1[i] = v4i{0, 0, 0, 0};
    sa[i] = 127;
    if (i < CT && m < A.T) {
      const int kt = kt0 + i;
      const uint8_t* ap = A.xq8 + (size_t)m * A.H + kt * 128 + 16 * q;
      a0[i] = ld_dev16(ap);
      a1[i] = ld_dev16(ap + 64);
      sa[i] = ld_dev(&A.xs8[m * (A.H / 32) + 4 * kt + q]);
    }
  }
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < CT) acc = mfma_fp8(a0[i], a1[i], B0[i], B1[i], acc, sa[i], scale_byte(sb, kt0 + i));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < A.T) st_dev(&A.sgu_part[((size_t)mm * A.KS1 + kc) * (2 * Is) + 16 * st + (lane & 15)], acc[r]);
  }
  if (wg_arrive_last(ctr(A.sgu_cnt, nb), (uint32_t)A.KS1, sm)) {
    // chunk sums of this wave's strip, added in chunk order
    for (int idx = lane; idx < 16 * A.T; idx += kWave) {
      const int n = idx & 15, mm = idx >> 4;
      const float* gp = A.sgu_part + (size_t)mm * A.KS1 * (2 * Is) + 16 * st + n;
      float v = ld_dev(gp);
      for (int c = 1; c < A.KS1; ++c) v = v + ld_dev(gp + (size_t)c * 2 * Is);
      sm.fin[wave >> 1][16 * (wave & 1) + n][mm] = v;
    }
    __syncthreads();
    swiglu_requant<FP8>(sm, A.T, nb, Is, A.a8, A.as8, [](int m_) { return m_; }, lane, wave);
    if (threadIdx.x == 0) st_dev(ctr(A.sgu_cnt, nb), 0u);
    wg_release_add(ctr(A.sync, S_SA), 1u);
  }
}

// ------------------------------------------------------------------ phase 2
__device__ __forceinline__ void build_expert_list(const DecodeArgs& A, Smem& sm, int lane, int wave) {
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

struct GuUnit {
  int dd, nb, c0, nch;
};

__device__ __forceinline__ GuUnit gu_unit(const DecodeArgs& A, int u) {
  const int per_expert = (A.I / 32) * A.S;
  const int r = u % per_expert;
  const int nch = A.KS1 / A.S;
  return GuUnit{u / per_expert, r / A.S, (r % A.S) * nch, nch};
}

// Issue the weight loads of a routed gate/up unit (this wave's strip).
__device__ __forceinline__ void gu_issue(const DecodeArgs& A, const Smem& sm, const GuUnit& U, int lane,
                                         int wave, v4i (&B)[kGuRegTiles], uint32_t (&sb)[kMaxChunksPerUnit]) {
  const int e = sm.elist[U.dd];
  const int st = gu_strip(U.nb, wave, A.I);
  const int t0 = U.c0 * A.CT1, nt = U.nch * A.CT1;
  const uint8_t* wb = A.w13 + (size_t)e * A.w13_stride + ((size_t)st * A.KT1 + t0) * 1024 + lane * 16;
#pragma unroll
  for (int i = 0; i < kGuRegTiles; ++i)
    if (i < nt) B[i] = load_stream16(wb + (size_t)i * 1024);
  const uint8_t* sp = A.w13s + (size_t)e * A.w13s_stride + ((size_t)st * A.KG1 * 64 + lane) * 4;
#pragma unroll
  for (int g = 0; g < kMaxChunksPerUnit; ++g)
    if (4 * g < nt + (t0 & 3)) sb[g] = *reinterpret_cast<const uint32_t*>(sp + (size_t)(t0 / 4 + g) * 256);
}

// Scale word g of a unit, picked with compile-time register indices.
__device__ __forceinline__ uint32_t pick_word(const uint32_t (&sb)[kMaxChunksPerUnit], int g) {
  uint32_t w = sb[0];
#pragma unroll
  for (int i = 1; i < kMaxChunksPerUnit; ++i)
    if (g == i) w = sb[i];
  return w;
}

// Matrix instructions of a routed gate/up unit.  With S == 1 the chunk sums
// are added in chunk order and returned; otherwise each chunk sum goes to the
// workspace as soon as its chain ends.  kAligned: the unit starts on a scale
// group (always so for chunks of four tiles), so scale words are picked with
// compile-time indices.
template <bool kAligned>
__device__ __forceinline__ v4f unit_routed_gu(const DecodeArgs& A, const Smem& sm, const uint8_t* xq4_lds,
                                              const uint8_t* xs4_lds, const GuUnit& U,
                                              const v4i (&B)[kGuRegTiles],
                                              const uint32_t (&sb)[kMaxChunksPerUnit], int lane, int wave) {
  const int n = sm.ecount[U.dd];
  const int m = lane & 15, q = lane >> 4;
  const int tok = m < n ? sm.tl[U.dd][m] / A.k : -1;
  const int CT = A.CT1, t0 = U.c0 * CT, nt = U.nch * CT;
  const int st = gu_strip(U.nb, wave, A.I);
  v4f acc = {0.f, 0.f, 0.f, 0.f}, sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ti = 0; ti < kGuRegTiles; ++ti) {
    if (ti < nt) {
      const int kt = t0 + ti;
      v4i a = {0, 0, 0, 0};
      uint32_t sa = 127;
      if (tok >= 0) {
        a = *reinterpret_cast<const v4i*>(xq4_lds + (size_t)tok * (A.H / 2) + kt * 64 + 16 * q);
        sa = xs4_lds[tok * (A.H / 32) + 4 * kt + q];
      }
      const uint32_t word = kAligned ? sb[ti >> 2] : pick_word(sb, ((t0 & 3) + ti) >> 2);
      acc = mfma_fp4(a, B[ti], acc, sa, scale_byte(word, kt));
      if ((ti + 1) % CT == 0) {  // the chain of one chunk ends here
        if (A.S == 1) {
          sum = ti + 1 == CT ? acc : sum + acc;
        } else {
          const int c = U.c0 + ti / CT;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mm = 4 * q + r;
            if (mm < n)
              st_dev(&A.gu_part[((size_t)sm.tl[U.dd][mm] * A.KS1 + c) * (2 * A.I) + 16 * st + (lane & 15)], acc[r]);
          }
        }
        acc = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  return sum;
}

__device__ __forceinline__ void routed_gu_epilogue(const DecodeArgs& A, Smem& sm, const GuUnit& U, v4f sum,
                                                   int lane, int wave) {
  const int e = sm.elist[U.dd], n = sm.ecount[U.dd], I = A.I;
  const int st = gu_strip(U.nb, wave, I);
  const int q = lane >> 4, col = lane & 15;
  bool finalize = true;
  if (A.S == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 4 * q + r;
      if (mm < n) sm.fin[wave >> 1][16 * (wave & 1) + col][mm] = sum[r];
    }
    __syncthreads();
  } else {
    finalize = wg_arrive_last(ctr(A.gu_cnt, e * (I / 32) + U.nb), (uint32_t)A.S, sm);
    if (finalize) {
      for (int idx = lane; idx < 16 * n; idx += kWave) {
        const int nn = idx & 15, mm = idx >> 4;
        const float* gp = A.gu_part + (size_t)sm.tl[U.dd][mm] * A.KS1 * (2 * I) + 16 * st + nn;
        float v = ld_dev(gp);
        for (int c = 1; c < A.KS1; ++c) v = v + ld_dev(gp + (size_t)c * 2 * I);
        sm.fin[wave >> 1][16 * (wave & 1) + nn][mm] = v;
      }
      __syncthreads();
    }
  }
  if (finalize) {
    const int dd = U.dd;
    swiglu_requant<FP4>(sm, n, U.nb, I, A.a4, A.as4, [&](int m_) { return (int)sm.tl[dd][m_]; }, lane, wave);
    if (A.S > 1 && threadIdx.x == 0) st_dev(ctr(A.gu_cnt, e * (I / 32) + U.nb), 0u);
    wg_release_add(ctr(A.a_ready, e), 1u);
  }
  __syncthreads();  // sm.fin is reused by the next unit
}

// ------------------------------------------------------------------ phase 3
__device__ __forceinline__ void combine(const DecodeArgs& A, const Smem& sm, int hg) {
  const int H = A.H, k = A.k;
  for (int idx = threadIdx.x; idx < A.T * 64; idx += kThreads) {
    const int t = idx >> 6, h = 64 * hg + (idx & 63);
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(sm.w[t * k + j], ld_dev(&A.d_part[(size_t)(t * k + j) * H + h]), acc);
    if (A.Is) acc = acc + ld_dev(&A.s_part[(size_t)t * H + h]);
    if (A.residual) acc = acc + bf16_to_f32(A.residual[(size_t)t * H + h]);
    A.y[(size_t)t * H + h] = f32_to_bf16(acc);
  }
}

// Routed down units of a column group count in; the last one waits for the
// group's shared-expert part (computed in phase 1) and combines.
__device__ __forceinline__ void arrive_output(const DecodeArgs& A, Smem& sm, int hg) {
  uint32_t* c = ctr(A.comb_cnt, hg);
  if (wg_arrive_last(c, (uint32_t)sm.D, sm)) {
    if (A.Is) wg_wait(ctr(A.sd_cnt, hg), 1u, A.sync);
    combine(A, sm, hg);
    if (threadIdx.x == 0) {
      st_dev(c, 0u);
      if (A.Is) st_dev(ctr(A.sd_cnt, hg), 0u);
    }
  }
}

// Down unit: shared (dd < 0) or routed expert dd, output columns 64 hg .. +64
// (this wave: strip 4 hg + wave).
struct DownUnit {
  int dd, hg;
};

__device__ __forceinline__ DownUnit down_unit(const DecodeArgs& A, int u) {
  const int nhg = A.H / 64;
  return DownUnit{u / nhg, u % nhg};
}

// Weight tiles a down unit holds in registers per batch: FP4 routed tiles
// take one register quad, FP8 shared tiles two.
template <bool kShared>
constexpr int down_batch() { return kShared ? 4 : kDownRegTiles; }

// Issue the loads of tiles [t0, t0 + batch) of the unit's strip into B.
template <bool kShared>
__device__ __forceinline__ void down_issue(const DecodeArgs& A, const Smem& sm, const DownUnit& U, int t0,
                                           int lane, int wave, v4i (&B)[kDownRegTiles]) {
  const int hs = 4 * U.hg + wave;
  constexpr int batch = down_batch<kShared>();
  if constexpr (kShared) {
    const int nt = min(batch, A.KTs - t0);
    const uint8_t* wb = A.ws2 + ((size_t)hs * A.KTs + t0) * 2048 + lane * 16;
#pragma unroll
    for (int i = 0; i < batch; ++i)
      if (i < nt) {
        B[2 * i] = load_stream16(wb + (size_t)i * 2048);
        B[2 * i + 1] = load_stream16(wb + (size_t)i * 2048 + 1024);
      }
  } else {
    const int e = sm.elist[U.dd];
    const int nt = min(batch, A.KT2 - t0);
    const uint8_t* wb = A.w2 + (size_t)e * A.w2_stride + ((size_t)hs * A.KT2 + t0) * 1024 + lane * 16;
#pragma unroll
    for (int i = 0; i < batch; ++i)
      if (i < nt) B[i] = load_stream16(wb + (size_t)i * 1024);
  }
}

// Down projection of one unit (kShared: the shared expert, U.dd unused); B
// holds its first batch of weight tiles.
template <bool kShared>
__device__ __forceinline__ void unit_down(const DecodeArgs& A, Smem& sm, const DownUnit& U, v4i (&B)[kDownRegTiles],
                                          int lane, int wave) {
  const int hs = 4 * U.hg + wave;
  const int KT = kShared ? A.KTs : A.KT2, CT = kShared ? A.CTs : A.CT2, KG = kShared ? A.KGs : A.KG2;
  constexpr int batch = down_batch<kShared>();
  const int e = kShared ? 0 : sm.elist[U.dd];
  const int n = kShared ? A.T : sm.ecount[U.dd];
  const uint8_t* sp = kShared ? A.ws2s + ((size_t)hs * KG * 64 + lane) * 4
                              : A.w2s + (size_t)e * A.w2s_stride + ((size_t)hs * KG * 64 + lane) * 4;
  if (kShared)
    wg_wait(ctr(A.sync, S_SA), (uint32_t)(A.Is / 32), A.sync);
  else
    wg_wait(ctr(A.a_ready, e), (uint32_t)(A.I / 32), A.sync);
  const int m = lane & 15, q = lane >> 4;
  const int row = m < n ? (kShared ? m : (int)sm.tl[U.dd][m]) : -1;
  float out[4] = {0.f, 0.f, 0.f, 0.f};
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < KT; t0 += batch) {
    if (t0 > 0) down_issue<kShared>(A, sm, U, t0, lane, wave, B);
#pragma unroll
    for (int i = 0; i < batch; ++i) {
      const int kt = t0 + i;
      if (kt < KT) {
        const uint32_t word = *reinterpret_cast<const uint32_t*>(sp + (size_t)(kt / 4) * 256);
        uint32_t sa = 127;
        if constexpr (kShared) {
          v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
          if (row >= 0) {
            const uint8_t* ap = A.a8 + (size_t)row * A.Is + kt * 128 + 16 * q;
            a0 = ld_dev16(ap);
            a1 = ld_dev16(ap + 64);
            sa = ld_dev(&A.as8[row * (A.Is / 32) + 4 * kt + q]);
          }
          acc = mfma_fp8(a0, a1, B[2 * i], B[2 * i + 1], acc, sa, scale_byte(word, kt));
        } else {
          v4i a = {0, 0, 0, 0};
          if (row >= 0) {
            a = ld_dev16(A.a4 + (size_t)row * (A.I / 2) + kt * 64 + 16 * q);
            sa = ld_dev(&A.as4[row * (A.I / 32) + 4 * kt + q]);
          }
          acc = mfma_fp4(a, B[i], acc, sa, scale_byte(word, kt));
        }
        if ((kt + 1) % CT == 0) {  // end of a chunk: add its sum in chunk order
#pragma unroll
          for (int r = 0; r < 4; ++r) out[r] = kt + 1 == CT ? acc[r] : out[r] + acc[r];
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = 4 * q + r;
    if (mm < n) {
      if (kShared)
        st_dev(&A.s_part[(size_t)mm * A.H + 16 * hs + (lane & 15)], out[r]);
      else
        st_dev(&A.d_part[(size_t)sm.tl[U.dd][mm] * A.H + 16 * hs + (lane & 15)], out[r]);
    }
  }
}

// ------------------------------------------------------------------ kernel
__global__ void __launch_bounds__(kThreads) fused_decode_kernel(DecodeArgs A) {
  __shared__ Smem sm;
  extern __shared__ __align__(16) unsigned char dyn[];  // logits, then MXFP4 x
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int G = A.G;
  const int T = A.T, E = A.E;
  uint64_t* tr = A.trace + (size_t)blockIdx.x * kTraceWords;
  if (threadIdx.x == 0) tr[TR_START] = wall_clock64();

  // phase 1
  const int n_xq = xq_units(T, A.H, A.Is);
  const int n_sgu = A.Is ? (A.Is / 32) * A.KS1 : 0;
  const int n_sd = A.Is ? A.H / 64 : 0;
  for (int u = blockIdx.x; u < n_xq + E + n_sgu + n_sd; u += G) {
    if (u < n_xq) {
      unit_xq(A, u);
    } else if (u < n_xq + E) {
      unit_router(A, u - n_xq, lane, wave);
    } else if (u < n_xq + E + n_sgu) {
      const int v = u - n_xq - E;
      unit_shared_gu(A, sm, v / A.KS1, v % A.KS1, lane, wave);
    } else {
      const DownUnit U{-1, u - n_xq - E - n_sgu};
      v4i B[kDownRegTiles];
      down_issue<true>(A, sm, U, 0, lane, wave, B);
      unit_down<true>(A, sm, U, B, lane, wave);
      wg_release_add(ctr(A.sd_cnt, U.hg), 1u);
    }
    if (threadIdx.x == 0) tr[TR_UNIT1] = wall_clock64();
  }

  // phase 2: routing, identical in every workgroup
  if (threadIdx.x == 0) {
    tr[TR_P1] = wall_clock64();
    for (int r = 0; r < kRouterCtrs; ++r)
      wait_count(ctr(A.sync, S_ROUTER + r), (uint32_t)((E - r + kRouterCtrs - 1) / kRouterCtrs), A.sync);
    tr[TR_LOGITS] = wall_clock64();
  }
  __syncthreads();
  compiler_fence();
  float* logits_lds = reinterpret_cast<float*>(dyn);
  for (int i = threadIdx.x; i < T * E; i += kThreads) logits_lds[i] = ld_dev(&A.logits[i]);
  __syncthreads();
  {
    const int row = threadIdx.x / 16;  // 16 lanes per row, 16 rows per pass
    rows_topk16(logits_lds + (row < T ? row : 0) * E, row < T, E, A.k, threadIdx.x & 15,
                sm.ids + (row < T ? row : 0) * A.k, sm.w + (row < T ? row : 0) * A.k);
  }
  __syncthreads();
  build_expert_list(A, sm, lane, wave);
  if (threadIdx.x == 0) {
    wait_count(ctr(A.sync, S_XQ), (uint32_t)n_xq, A.sync);
    tr[TR_XQ] = wall_clock64();
  }
  __syncthreads();
  compiler_fence();
  // stage the MXFP4 copy of x (codes then scales) over the logits
  uint8_t* xq4_lds = dyn;
  uint8_t* xs4_lds = dyn + (size_t)T * (A.H / 2);
  {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(A.xq4);
    uint64_t* dst = reinterpret_cast<uint64_t*>(xq4_lds);
    for (int i = threadIdx.x; i < T * A.H / 16; i += kThreads) dst[i] = ld_dev(src + i);
    for (int i = threadIdx.x; i < T * A.H / 32; i += kThreads) xs4_lds[i] = ld_dev(&A.xs4[i]);
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < T * A.k; i += kThreads) {
      if (A.ids_out) A.ids_out[i] = sm.ids[i];
      if (A.w_out) A.w_out[i] = sm.w[i];
    }
  }
  __syncthreads();
  const int D = sm.D;
  if (threadIdx.x == 0) tr[TR_ROUTED] = wall_clock64();

  {
    const int n2 = D * (A.I / 32) * A.S;
    v4i B[kGuRegTiles];
    uint32_t sb[kMaxChunksPerUnit];
    int u = blockIdx.x;
    if (u < n2) gu_issue(A, sm, gu_unit(A, u), lane, wave, B, sb);
    for (; u < n2; u += G) {
      const GuUnit U = gu_unit(A, u);
      const v4f sum = ((U.c0 * A.CT1) & 3) == 0
                          ? unit_routed_gu<true>(A, sm, xq4_lds, xs4_lds, U, B, sb, lane, wave)
                          : unit_routed_gu<false>(A, sm, xq4_lds, xs4_lds, U, B, sb, lane, wave);
      if (u + G < n2) gu_issue(A, sm, gu_unit(A, u + G), lane, wave, B, sb);
      routed_gu_epilogue(A, sm, U, sum, lane, wave);
    }
  }
  if (threadIdx.x == 0) tr[TR_P2] = wall_clock64();

  // phase 3: routed down projections and the combine
  {
    const int n3 = D * (A.H / 64);
    v4i B[kDownRegTiles];
    int u = blockIdx.x;
    if (u < n3) down_issue<false>(A, sm, down_unit(A, u), 0, lane, wave, B);
    for (; u < n3; u += G) {
      const DownUnit U = down_unit(A, u);
      unit_down<false>(A, sm, U, B, lane, wave);
      if (u + G < n3) down_issue<false>(A, sm, down_unit(A, u + G), 0, lane, wave, B);
      arrive_output(A, sm, U.hg);
    }
  }

  // exit: the last workgroup resets the launch-wide counters
  __syncthreads();
  if (threadIdx.x == 0) {
    tr[TR_P3] = wall_clock64();
    if (blockIdx.x == 0) st_dev(ctr(A.sync, S_GRID), (uint32_t)G);
    compiler_fence();
    drain_stores();
    const uint32_t old = __hip_atomic_fetch_add(ctr(A.sync, S_DONE), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    compiler_fence();
    if (old + 1 == (uint32_t)G) {
      for (int r = 0; r < kRouterCtrs; ++r) st_dev(ctr(A.sync, S_ROUTER + r), 0u);
      st_dev(ctr(A.sync, S_XQ), 0u);
      st_dev(ctr(A.sync, S_SA), 0u);
      for (int e = 0; e < E; ++e) st_dev(ctr(A.a_ready, e), 0u);
      drain_stores();
      st_dev(ctr(A.sync, S_DONE), 0u);
    }
  }
}

// ------------------------------------------------------------------ host side
struct Carve {
  size_t sync, gu_cnt, sgu_cnt, a_ready, comb_cnt, sd_cnt, sync_end;
  size_t logits, xq4, xs4, xq8, xs8, gu_part, sgu_part, a4, as4, a8, as8, d_part, s_part, trace, total;
};

int pick_chunk(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }

Carve carve(const moe_layer_t& L) {
  const size_t T = kDecodeMaxT, H = L.hidden, I = L.inter, E = L.num_experts, k = L.top_k,
               Is = L.shared_inter;
  const size_t KS1 = (H / 128) / pick_chunk((int)(H / 128));
  Carve c{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  const size_t line = kLine * 4;
  c.sync = take(kSyncLines * line);
  c.gu_cnt = take(E * (I / 32) * line);
  c.sgu_cnt = take((Is / 32 + 1) * line);
  c.a_ready = take(E * line);
  c.comb_cnt = take((H / 64) * line);
  c.sd_cnt = take((H / 64) * line);
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
  c.a8 = take(T * Is + 16);
  c.as8 = take(T * Is / 32 + 16);
  c.d_part = take(T * k * H * 4);
  c.s_part = take(T * H * 4);
  c.trace = take((size_t)kDecodeMaxGrid * kTraceWords * 8);
  c.total = o;
  return c;
}

size_t dyn_lds_bytes(const moe_layer_t& L) {
  const size_t T = kDecodeMaxT;
  const size_t logits = T * L.num_experts * 4;
  const size_t xq = T * (L.hidden / 2 + L.hidden / 32);
  return align_up(logits > xq ? logits : xq, 16);
}

int grid_size(size_t lds) {
  static int cached_dev = -1, cached_grid = 0;
  static size_t cached_lds = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == cached_dev && lds == cached_lds) return cached_grid;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_decode_kernel, kThreads, lds) != hipSuccess)
    return 0;
  if (occ > 2) occ = 2;
  cached_dev = dev;
  cached_lds = lds;
  cached_grid = occ * cus;
  if (cached_grid > kDecodeMaxGrid) cached_grid = kDecodeMaxGrid;
  return cached_grid;
}

}  // namespace

size_t decode_ws_bytes(const moe_layer_t& L) { return carve(L).total; }
size_t decode_sync_bytes(const moe_layer_t& L) { return carve(L).sync_end; }
size_t decode_trace_offset(const moe_layer_t& L) { return carve(L).trace; }

hipError_t launch_decode(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                         uint16_t* y, void* ws, int32_t* ids_out, float* w_out, hipStream_t stream) {
  const Carve c = carve(L);
  const size_t lds = dyn_lds_bytes(L);
  char* base = reinterpret_cast<char*>(ws);
  DecodeArgs A{};
  A.T = T;
  A.H = L.hidden;
  A.I = L.inter;
  A.E = L.num_experts;
  A.k = L.top_k;
  A.Is = L.shared_inter;
  A.KT1 = A.H / 128;
  A.CT1 = pick_chunk(A.KT1);
  A.KS1 = A.KT1 / A.CT1;
  A.KG1 = (A.KT1 + 3) / 4;
  A.KT2 = A.I / 128;
  A.CT2 = pick_chunk(A.KT2);
  A.KS2 = A.KT2 / A.CT2;
  A.KG2 = (A.KT2 + 3) / 4;
  A.KTs = A.Is / 128;
  A.CTs = A.Is ? pick_chunk(A.KTs) : 1;
  A.KSs = A.Is ? A.KTs / A.CTs : 0;
  A.KGs = (A.KTs + 3) / 4;
  A.G = grid_size(lds);
  if (A.G <= 0) return hipErrorInvalidDeviceFunction;
  // Workgroups per routed gate/up block: the smallest divisor of the chunk
  // count that gives at least 1.5 units per workgroup (with the expected
  // number of distinct experts) and keeps a unit's chunks in registers.
  {
    const int Dexp = T * A.k < A.E ? T * A.k : A.E;
    const int blocks = Dexp * (A.I / 32);
    A.S = A.KS1;
    for (int s = 1; s <= A.KS1; ++s) {
      if (A.KS1 % s || A.KS1 / s > kMaxChunksPerUnit || (A.KS1 / s) * A.CT1 > kGuRegTiles) continue;
      if (2 * blocks * s >= 3 * A.G) { A.S = s; break; }
    }
    if (A.KS1 / A.S > kMaxChunksPerUnit || (A.KS1 / A.S) * A.CT1 > kGuRegTiles) return hipErrorInvalidValue;
  }
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
  A.sd_cnt = reinterpret_cast<uint32_t*>(base + c.sd_cnt);
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
  A.trace = reinterpret_cast<uint64_t*>(base + c.trace);
  hipLaunchKernelGGL(fused_decode_kernel, dim3(A.G), dim3(kThreads), lds, stream, A);
  return hipGetLastError();
}

}  // namespace mxmoe
