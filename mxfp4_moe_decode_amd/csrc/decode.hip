// The whole MoE layer for 1..16 rows in one kernel launch ("mono decode": one
// fused launch per MoE layer for a pure decode step of at most 16 tokens,
// article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and optimization",
// section "Serving with vLLM / What we Optimized").
//
// Structure.  A persistent grid of G 4-wavefront workgroups (G at most the
// device's co-resident capacity) runs three lists of work units:
//
//   phase A  (workgroup b takes units b, b+G, ...)
//            x quantization blocks (MXFP4 and, with a shared expert, MXFP8),
//            router logits (one unit per expert, all rows),
//            shared-expert gate/up (one unit per 16-column strip: the gate
//            strip and the matching up strip; the four wavefronts split K);
//   routing  every workgroup waits for all logits, takes the top k of each
//            row and builds the same list of the D selected experts, then
//            stages the MXFP4 copy of x in LDS;
//   phase B  routed gate/up units (selected expert, 16-column strip; the four
//            wavefronts split K), SwiGLU, fp32 result per (row, choice) slot;
//   phase C  routed down units (selected expert, 64 output columns, one
//            16-column strip per wavefront) and shared down units; a down unit
//            re-quantizes the intermediate it needs (MXFP4 routed, MXFP8
//            shared) into LDS itself;
//   combine  workgroup b combines the 64-column groups b, b+G, ... once all
//            their down outputs are in.
//
// Phases B and C give each workgroup a contiguous run of units and are one
// software pipeline over three register buffers: while a unit computes from
// one, the next two units' tiles land in the others, and as soon as its matrix
// products have read its buffer a unit requests the tiles of the unit three
// places on into it.  Results of phases B and C carry the call's tag (below), so no unit
// waits for its own stores.  A unit only waits for
// units of an earlier phase, so with every workgroup resident the smallest
// unfinished unit can always progress.
//
// Arithmetic (fixed, independent of the number of rows and of the grid): every
// dot product is cut into NC = 4 (or 2, or 1) K-chunks of CT tiles of 128; a
// chunk is one chain of scaled 16x16x128 matrix instructions in tile order
// starting from zero, and the chunk sums are added in chunk order in fp32.
// SwiGLU and re-quantization (MXFP4 routed, MXFP8 shared) follow per 32-column
// block; the combine adds sum_j w_j d_j in j order, then s, then the residual,
// and rounds once to bf16.  Output row t therefore depends on x[t] only.
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxK = 8;
constexpr int kMaxSlots = kDecodeMaxT * kMaxK;
constexpr int kMaxCT = 6;      // tiles of a gate/up K-chunk held in registers
constexpr int kBufQuads = 12;  // 16-byte weight loads one prefetch buffer holds per lane
constexpr int kBufWords = 6;   // scale words one prefetch buffer holds per lane
constexpr int kBufs = 3;       // register buffers of the unit pipeline
constexpr int kDownBatch = 8;  // routed (MXFP4) down tiles per register batch; MXFP8: half
constexpr uint64_t kSpinTicks = 100000000ull;  // ~1 s of the 100 MHz constant clock

// Every counter sits on a 256-byte line of its own: device-scope atomics on
// one line are serialized by the memory side.
constexpr int kLine = 64;  // words
__device__ __forceinline__ uint32_t* ctr(uint32_t* base, int i) { return base + (size_t)i * kLine; }
// Lines of the sync block: status, done, x-quant, shared-intermediate ready,
// grid size of the last call, call epoch.
enum { S_STATUS = 0, S_DONE = 1, S_XQ = 2, S_SA = 3, S_GRID = 4, S_EPOCH = 5, kSyncLines = 6 };

// Timestamps each workgroup records (100 MHz device clock).
enum {
  TR_START = 0, TR_A = 1, TR_LOGITS = 2, TR_ROUTED = 3, TR_B = 4, TR_C = 5, TR_FIRST = 6,
  TR_LOGITS_LDS = 7, TR_TOPK = 8, TR_ELIST = 9,
  TR_B_MMA = 10, TR_B_STORED = 11, TR_B_NEXT = 12, TR_B_RELEASED = 13, TR_C_STAGED = 14
};

struct DecodeArgs {
  int T, H, I, E, k, Is, G;
  int KT1, CT1, NC1;  // K = H: tiles of 128, tiles per chunk, chunks
  int KT2, CT2;       // K = I
  int KTs, CTs;       // K = I_s
  const float* router_w;
  const float* router_bias;
  const uint8_t *w13, *w13s, *w2, *w2s, *ws13, *ws13s, *ws2, *ws2s;
  const uint16_t* x;
  const uint16_t* residual;
  uint16_t* y;
  int32_t* ids_out;
  float* w_out;
  uint32_t* sync;
  uint64_t* logits;  // tagged [T][E]
  uint8_t *xq4, *xs4, *xq8, *xs8;
  uint64_t* a_r;  // tagged [T*k][I]
  float* a_s;
  uint64_t *d_part, *s_part;  // tagged [T*k][H], [T][H]
  uint64_t* trace;
};

// The shape as the kernel sees it: compile-time constants where the launch
// picked a specialization for the layer's shape (H_, I_, IS_, E_, K_ non-zero,
// IS_ = -1 for no shared expert), the run-time fields otherwise.
constexpr int n_chunks_of(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }
template <int H_, int I_, int IS_, int E_, int K_>
struct DArgs : DecodeArgs {
  __device__ __forceinline__ int h() const { return H_ ? H_ : H; }
  __device__ __forceinline__ int i() const { return I_ ? I_ : I; }
  __device__ __forceinline__ int is() const { return IS_ ? (IS_ < 0 ? 0 : IS_) : Is; }
  __device__ __forceinline__ int e() const { return E_ ? E_ : E; }
  __device__ __forceinline__ int kk() const { return K_ ? K_ : k; }
  __device__ __forceinline__ int kt1() const { return h() / 128; }
  __device__ __forceinline__ int nc1() const { return n_chunks_of(kt1()); }
  __device__ __forceinline__ int ct1() const { return kt1() / nc1(); }
  __device__ __forceinline__ int kt2() const { return i() / 128; }
  __device__ __forceinline__ int ct2() const { return kt2() / n_chunks_of(kt2()); }
  __device__ __forceinline__ int kts() const { return is() / 128; }
  __device__ __forceinline__ int cts() const { return is() ? kts() / n_chunks_of(kts()) : 1; }
};

// Thread 0 records the device clock in trace word i of its workgroup.
template <class DA>
__device__ __forceinline__ void trace_at(const DA& A, int i) {
  if (threadIdx.x == 0) A.trace[(size_t)blockIdx.x * kTraceWords + i] = wall_clock64();
}

struct Smem {
  int32_t ids[kMaxSlots];
  float w[kMaxSlots];
  int hist[256];
  int epos[256];
  int fill[kMaxSlots];
  uint8_t elist[kMaxSlots];
  uint8_t ecount[kMaxSlots];
  uint8_t tl[kMaxSlots][kDecodeMaxT];           // slots routed to each selected expert
  float red[kWaves][2][kDecodeMaxT][16];        // chunk sums [chunk][gate/up][row][column]
  int wave_cnt[kWaves];
  int D;
  int flag;
  int staged;                                   // expert whose intermediate is in LDS (-1 shared, -2 none)
};

// ------------------------------------------------------------------ synchronisation
// Data handed from one workgroup to another (logits, quantized x, fp32
// intermediates and partial outputs) is written and read with relaxed
// agent-scope atomic accesses, which gfx950 issues with the sc1 bit: they are
// served at the device's coherence point, past the per-XCD L2 caches, so no L2
// write-back or invalidate is needed.  Before a counter is bumped each
// wavefront waits for its stores to be acknowledged (vector memory operations
// complete in issue order, so it waits until no more than the operations
// issued after the stores are outstanding), then the workgroup barrier, then
// one atomic add.  A consumer polls the counter and issues its data loads
// only after the poll has returned.
//
// Where many producers feed one consumer set (128 router units, 64 gate/up
// strips per expert), a shared counter would serialize the atomics at the
// memory side; there the data carries the call's tag instead: each value is
// stored as one 64-bit word (tag << 32 | fp32 bits), single-copy atomic, and a
// consumer reads the words until every tag is this call's.  The tag is one
// more than the epoch word, which the last workgroup of a call advances, so
// words of an earlier call (or the zero-filled workspace) never match.
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
__device__ __forceinline__ float4 ld_dev_f4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = ld_dev(q), b = ld_dev(q + 1);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                     __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}
// Keeps the compiler from moving memory accesses (and, for the machine
// scheduler, any instruction) across this point.
__device__ __forceinline__ void compiler_fence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}
// s_waitcnt vmcnt(n), expcnt and lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
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

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.f + expf(-g))) * u; }

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Workgroup-uniform bounded retry: true to go on polling.  Gives up (marking
// the status word) after the spin bound or once another wait has given up.
__device__ __forceinline__ bool keep_polling(bool all_ok, uint64_t t0, uint32_t* status) {
  if (__syncthreads_and(all_ok)) return false;
  const bool late = wall_clock64() - t0 > kSpinTicks || ld_dev(status) != 0;
  if (__syncthreads_or(late)) {
    if (threadIdx.x == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

__device__ __forceinline__ uint32_t scale_byte(uint32_t word, int tile) { return (word >> (8 * (tile & 3))) & 0xffu; }

// w[i] for a run-time i in 0..2, without indexing a register array.
__device__ __forceinline__ uint32_t pick3(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
  return i == 0 ? w0 : (i == 1 ? w1 : w2);
}

// ------------------------------------------------------------------ MX block quantization by 8 lanes
// Eight consecutive lanes hold the 32 values of one block (lane j: values
// 4j..4j+3, fp32 bit patterns) and agree on the block scale with three
// butterfly steps.  Returns the four codes packed (FP4: 16 bits, element 4j+i
// in nibble i; FP8: 32 bits, byte i) and the E8M0 code in *scale.
template <class F>
__device__ __forceinline__ uint32_t quant_block8(const uint32_t (&bits)[4], uint32_t* scale) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) am = max(am, bits[i] & 0x7fffffffu);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 8));
  const int e = block_exponent<F>(am);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) packed |= quant_elem<F>(bits[i], e) << ((F::MB == 1 ? 4 : 8) * i);
  *scale = (uint32_t)(e + 127);
  return packed;
}

// ------------------------------------------------------------------ phase A
// x quantization: block task i of T * nb * F (nb = H/32 blocks per row, F = 2
// formats with a shared expert, else 1) is (row, format, block); a unit is 32
// tasks.
__host__ __device__ __forceinline__ int xq_units(int T, int H, int Is) {
  return (T * (H / 32) * (Is ? 2 : 1) + kThreads / 8 - 1) / (kThreads / 8);
}

template <class DA>
__device__ __forceinline__ void unit_xq(const DA& A, int u) {
  const int nb = A.h() / 32, F = A.is() ? 2 : 1;
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
    const uint2 v = *reinterpret_cast<const uint2*>(A.x + (size_t)t * A.h() + 32 * b + 4 * j);
    bits[0] = v.x << 16;
    bits[1] = v.x & 0xffff0000u;
    bits[2] = v.y << 16;
    bits[3] = v.y & 0xffff0000u;
  }
  // the eight lanes of a task share fp8 (same task), so the branch is uniform per group
  uint32_t sc;
  if (fp8) {
    const uint32_t word = quant_block8<FP8>(bits, &sc);
    if (act) {
      st_dev(reinterpret_cast<uint32_t*>(A.xq8 + (size_t)t * A.h() + 32 * b + 4 * j), word);
      if (j == 0) st_dev(&A.xs8[t * nb + b], (uint8_t)sc);
    }
  } else {
    const uint32_t half = quant_block8<FP4>(bits, &sc);
    if (act) {
      st_dev(reinterpret_cast<uint16_t*>(A.xq4 + (size_t)t * (A.h() / 2) + 16 * b + 2 * j), (uint16_t)half);
      if (j == 0) st_dev(&A.xs4[t * nb + b], (uint8_t)sc);
    }
  }
  compiler_fence();
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr(A.sync, S_XQ), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Logits of expert e for all rows; wave w takes rows w, w+4, ...  Same
// per-row arithmetic as router_lane_partial: each batch of up to 16 strides
// of the expert's weights is loaded once, then the rows go through it two at
// a time.
template <class DA>
__device__ __forceinline__ void unit_router(const DA& A, uint32_t tag, int e, int lane, int wave) {
  const float* wrow = A.router_w + (size_t)e * A.h();
  const int H = A.h();
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  int nr = 0;
  for (int t = wave; t < A.T; t += kWaves) ++nr;
  for (int h0 = 4 * lane; h0 < H; h0 += 16 * 256) {
    float4 w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (h0 + 256 * j < H) w[j] = load_stream_f4(wrow + h0 + 256 * j);
#pragma unroll
    for (int r0 = 0; r0 < 4; r0 += 2) {
      if (r0 < nr) {
        uint2 xv[2][16];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (r0 + r < nr) {
            const uint16_t* xr = A.x + (size_t)(wave + kWaves * (r0 + r)) * H;
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
      if (lane == 0) st_dev(&A.logits[(wave + kWaves * r) * A.e() + e], tagged(tag, v));
    }
}

// Chunk sums of a gate/up unit in sm.red, added in chunk order, then SwiGLU:
// thread (row, column) for row < n; returns false for idle threads.
__device__ __forceinline__ bool gu_finish(const Smem& sm, int nc, int n, int* row, int* col, float* a) {
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  if (r >= n) return false;
  float g = sm.red[0][0][r][c], u = sm.red[0][1][r][c];
  for (int ch = 1; ch < nc; ++ch) {
    g = g + sm.red[ch][0][r][c];
    u = u + sm.red[ch][1][r][c];
  }
  *row = r;
  *col = c;
  *a = silu_mul(g, u);
  return true;
}

// Shared gate/up strip i: wave w computes K-chunk w of the gate strip i and
// the up strip I_s/16 + i (MXFP8 x MXFP8); the chunk sums meet in LDS.
template <class DA>
__device__ __forceinline__ void unit_shared_gu(const DA& A, Smem& sm, int i, int lane, int wave) {
  const int CT = A.ct1(), KG = (A.kt1() + 3) / 4;
  const int m = lane & 15, q = lane >> 4;
  const bool act = wave < A.nc1();
  const int t0 = wave * CT;
  v4i B[2][kMaxCT][2];
  uint32_t sw[2][3];
  if (act) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int st = s == 0 ? i : A.is() / 16 + i;
      const uint8_t* wb = A.ws13 + ((size_t)st * A.kt1() + t0) * 2048 + lane * 16;
#pragma unroll
      for (int j = 0; j < kMaxCT; ++j)
        if (j < CT) {
          B[s][j][0] = load_stream16(wb + j * 2048);
          B[s][j][1] = load_stream16(wb + j * 2048 + 1024);
        }
      const uint8_t* sp = A.ws13s + ((size_t)st * KG * 64 + lane) * 4;
#pragma unroll
      for (int g = 0; g < 3; ++g)
        sw[s][g] = load_stream4(sp + (size_t)min(t0 / 4 + g, KG - 1) * 256);
    }
  }
  wg_wait(ctr(A.sync, S_XQ), (uint32_t)xq_units(A.T, A.h(), A.is()), A.sync);
  if (act) {
    v4i a0[kMaxCT], a1[kMaxCT];
    uint32_t sa[kMaxCT];
#pragma unroll
    for (int j = 0; j < kMaxCT; ++j) {
      a0[j] = a1[j] = v4i{0, 0, 0, 0};
      sa[j] = 127;
      if (j < CT && m < A.T) {
        const int kt = t0 + j;
        const uint8_t* ap = A.xq8 + (size_t)m * A.h() + kt * 128 + 16 * q;
        a0[j] = ld_dev16(ap);
        a1[j] = ld_dev16(ap + 64);
        sa[j] = ld_dev(&A.xs8[m * (A.h() / 32) + 4 * kt + q]);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxCT; ++j)
        if (j < CT) {
          const int kt = t0 + j;
          const uint32_t word = pick3(sw[s][0], sw[s][1], sw[s][2], kt / 4 - t0 / 4);
          acc = mfma_fp8(a0[j], a1[j], B[s][j][0], B[s][j][1], acc, sa[j], scale_byte(word, kt));
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[wave][s][4 * q + r][m] = acc[r];
    }
  }
  __syncthreads();
  int row, col;
  float a;
  if (gu_finish(sm, A.nc1(), A.T, &row, &col, &a)) st_dev(&A.a_s[(size_t)row * A.is() + 16 * i + col], a);
  compiler_fence();
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr(A.sync, S_SA), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ routing
// Selected experts in ascending expert order (every workgroup builds the same
// list) and the slots routed to each.  The order of slots inside a list is
// not fixed; nothing depends on it, since every result is addressed by slot.
template <class DA>
__device__ __forceinline__ void build_expert_list(const DA& A, Smem& sm, int lane, int wave) {
  const int S = A.T * A.kk(), tid = threadIdx.x;
  sm.hist[tid] = 0;
  if (tid < kMaxSlots) sm.fill[tid] = 0;
  __syncthreads();
  if (tid < S) atomicAdd(&sm.hist[sm.ids[tid]], 1);
  __syncthreads();
  const int cnt = sm.hist[tid];
  const bool used = cnt > 0;
  const uint64_t mask = __ballot(used);
  if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sm.wave_cnt[w];
  if (used) {
    const int dd = base + __popcll(mask & ((1ull << lane) - 1ull));
    sm.elist[dd] = (uint8_t)tid;
    sm.ecount[dd] = (uint8_t)cnt;
    sm.epos[tid] = dd;
  }
  if (tid == 0) sm.D = sm.wave_cnt[0] + sm.wave_cnt[1] + sm.wave_cnt[2] + sm.wave_cnt[3];
  __syncthreads();
  if (tid < S) {
    const int dd = sm.epos[sm.ids[tid]];
    sm.tl[dd][atomicAdd(&sm.fill[dd], 1)] = (uint8_t)tid;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ phases B and C
// Unit j of a workgroup's sequence: its phase-B units [b0, b1) then its
// phase-C units [c0, c1).
struct Seq {
  int b0, nb, c0, nc;
  int D, nhg;
};

struct Buf {
  v4i q[kBufQuads];
  uint32_t w[kBufWords];
};

// Requests the weight tiles and scale words of sequence entry j into buf.
template <class DA>
__device__ __forceinline__ void issue(const DA& A, const Smem& sm, const Seq& S, int j, int lane, int wave,
                                      Buf& buf) {
  if (j >= S.nb + S.nc) return;
  if (j < S.nb) {
    if (wave >= A.nc1()) return;
    const int u = S.b0 + j;
    const int per = A.i() / 16;
    const int e = sm.elist[u / per], i = u % per;
    const int CT = A.ct1(), KG = (A.kt1() + 3) / 4, t0 = wave * CT;
    const uint8_t* base = A.w13 + (size_t)e * ((size_t)A.i() * A.h());
    const uint8_t* sbase = A.w13s + (size_t)e * ((size_t)(2 * A.i() / 16) * KG * 256);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int st = s == 0 ? i : A.i() / 16 + i;
      const uint8_t* wb = base + ((size_t)st * A.kt1() + t0) * 1024 + lane * 16;
#pragma unroll
      for (int jj = 0; jj < kMaxCT; ++jj)
        if (jj < CT) buf.q[kMaxCT * s + jj] = load_stream16(wb + jj * 1024);
      const uint8_t* sp = sbase + ((size_t)st * KG * 64 + lane) * 4;
#pragma unroll
      for (int g = 0; g < 3; ++g)
        buf.w[3 * s + g] = load_stream4(sp + (size_t)min(t0 / 4 + g, KG - 1) * 256);
    }
    return;
  }
  const int u = S.c0 + j - S.nb;
  if (u < S.D * S.nhg) {
    const int e = sm.elist[u / S.nhg], hs = 4 * (u % S.nhg) + wave;
    const int KG = (A.kt2() + 3) / 4, nt = min(A.kt2(), kDownBatch);
    const uint8_t* wb = A.w2 + (size_t)e * ((size_t)A.h() * A.i() / 2) + (size_t)hs * A.kt2() * 1024 + lane * 16;
#pragma unroll
    for (int jj = 0; jj < kDownBatch; ++jj)
      if (jj < nt) buf.q[jj] = load_stream16(wb + jj * 1024);
    const uint8_t* sp = A.w2s + (size_t)e * ((size_t)(A.h() / 16) * KG * 256) + ((size_t)hs * KG * 64 + lane) * 4;
#pragma unroll
    for (int g = 0; g < 2; ++g) buf.w[g] = load_stream4(sp + (size_t)min(g, KG - 1) * 256);
  } else {
    const int hs = 4 * (u - S.D * S.nhg) + wave;
    const int KG = (A.kts() + 3) / 4, nt = min(A.kts(), kDownBatch / 2);
    const uint8_t* wb = A.ws2 + (size_t)hs * A.kts() * 2048 + lane * 16;
#pragma unroll
    for (int jj = 0; jj < kDownBatch / 2; ++jj)
      if (jj < nt) {
        buf.q[2 * jj] = load_stream16(wb + jj * 2048);
        buf.q[2 * jj + 1] = load_stream16(wb + jj * 2048 + 1024);
      }
    const uint8_t* sp = A.ws2s + ((size_t)hs * KG * 64 + lane) * 4;
#pragma unroll
    for (int g = 0; g < 2; ++g) buf.w[g] = load_stream4(sp + (size_t)min(g, KG - 1) * 256);
  }
}

// Routed gate/up: MFMA chain of this wave's K-chunk for both strips into
// sm.red (A operand: the MXFP4 x rows of the routed slots, from LDS).
template <class DA>
__device__ __forceinline__ void gu_compute(const DA& A, Smem& sm, const uint8_t* xq4_lds,
                                           const uint8_t* xs4_lds, int dd, const Buf& buf, int lane, int wave) {
  if (wave >= A.nc1()) return;
  const int n = sm.ecount[dd];
  const int m = lane & 15, q = lane >> 4;
  const int tok = m < n ? sm.tl[dd][m] / A.kk() : -1;
  const int CT = A.ct1(), t0 = wave * CT;
  v4i a[kMaxCT];
  uint32_t sa[kMaxCT];
#pragma unroll
  for (int jj = 0; jj < kMaxCT; ++jj) {
    a[jj] = v4i{0, 0, 0, 0};
    sa[jj] = 127;
    if (jj < CT && tok >= 0) {
      const int kt = t0 + jj;
      a[jj] = *reinterpret_cast<const v4i*>(xq4_lds + (size_t)tok * (A.h() / 2) + kt * 64 + 16 * q);
      sa[jj] = xs4_lds[tok * (A.h() / 32) + 4 * kt + q];
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < kMaxCT; ++jj)
      if (jj < CT) {
        const int kt = t0 + jj;
        const uint32_t word = pick3(buf.w[3 * s], buf.w[3 * s + 1], buf.w[3 * s + 2], kt / 4 - t0 / 4);
        acc = mfma_fp4(a[jj], buf.q[kMaxCT * s + jj], acc, sa[jj], scale_byte(word, kt));
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.red[wave][s][4 * q + r][m] = acc[r];
  }
}

// Four consecutive fp32 values, plain or tagged (the value is the low word).
__device__ __forceinline__ float4 load4(const float* p) { return ld_dev_f4(p); }
__device__ __forceinline__ float4 load4(const uint64_t* p) {
  return make_float4(__uint_as_float((uint32_t)ld_dev(p)), __uint_as_float((uint32_t)ld_dev(p + 1)),
                     __uint_as_float((uint32_t)ld_dev(p + 2)), __uint_as_float((uint32_t)ld_dev(p + 3)));
}

// Waits until rows slots[0..n) of a tagged [*, K] array all carry this call's
// tag (only the tag halves are read).
template <class DA>
__device__ __forceinline__ void wait_tagged_rows(const DA& A, uint32_t tag, const uint64_t* src, int K, int n,
                                                 const uint8_t* slots) {
  const uint64_t t0 = wall_clock64();
  const uint32_t* hi = reinterpret_cast<const uint32_t*>(src) + 1;
  bool ok;
  do {
    ok = true;
    for (int idx = threadIdx.x; idx < n * K; idx += kThreads) {
      const int m = idx / K, c = idx % K;
      ok &= ld_dev(&hi[2 * ((size_t)slots[m] * K + c)]) == tag;
    }
  } while (keep_polling(ok, t0, A.sync));
}

// Re-quantizes the fp32 intermediate rows of one down unit into LDS (row m of
// the staged block = routed slot tl[dd][m], or shared row m): codes [n, K/2]
// (FP4) or [n, K] (FP8), scales [n, K/32].
template <class F, class Src>
__device__ __forceinline__ void stage_intermediate(const Src* src, int K, int n, const uint8_t* slots,
                                                   uint8_t* codes, uint8_t* scales) {
  const int nb = K / 32, tasks = n * nb;
  const int j = threadIdx.x & 7;
  for (int t0 = 0; t0 < tasks; t0 += 4 * (kThreads / 8)) {
    float4 v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {  // all loads first
      const int task = t0 + p * (kThreads / 8) + (int)threadIdx.x / 8;
      v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (task < tasks) {
        const int m = task / nb, b = task % nb;
        const int row = slots ? slots[m] : m;
        v[p] = load4(src + (size_t)row * K + 32 * b + 4 * j);
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int task = t0 + p * (kThreads / 8) + (int)threadIdx.x / 8;
      if (t0 + p * (kThreads / 8) >= tasks) break;  // uniform: whole pass beyond the end
      const uint32_t bits[4] = {__float_as_uint(v[p].x), __float_as_uint(v[p].y), __float_as_uint(v[p].z),
                                __float_as_uint(v[p].w)};
      uint32_t sc;
      const uint32_t packed = quant_block8<F>(bits, &sc);
      if (task < tasks) {
        const int m = task / nb, b = task % nb;
        if constexpr (F::MB == 1)
          *reinterpret_cast<uint16_t*>(codes + (size_t)m * (K / 2) + 16 * b + 2 * j) = (uint16_t)packed;
        else
          *reinterpret_cast<uint32_t*>(codes + (size_t)m * K + 32 * b + 4 * j) = packed;
        if (j == 0) scales[m * nb + b] = (uint8_t)sc;
      }
    }
  }
}

// Down unit MFMA (this wave's 16-column strip hs, all K-tiles): the first
// batch of weight tiles is in buf, later batches are loaded here.  Returns the
// chunk-ordered sums for rows 4q+r.
template <class F>
__device__ __forceinline__ v4f down_compute(const uint8_t* w, const uint8_t* ws_scale, int KT, int CT,
                                            const uint8_t* codes, const uint8_t* scales, int n, Buf& buf,
                                            int lane) {
  constexpr int R = F::MB == 1 ? 1 : 2;  // register quads per tile
  constexpr int NB = kDownBatch / R;     // tiles per batch
  const int KG = (KT + 3) / 4;
  const int m = lane & 15, q = lane >> 4;
  const int K = KT * 128;
  v4f out = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < KT; b0 += NB) {
    if (b0 > 0) {
      const int nt = min(KT - b0, NB);
#pragma unroll
      for (int jj = 0; jj < NB; ++jj)
        if (jj < nt) {
#pragma unroll
          for (int r = 0; r < R; ++r) buf.q[R * jj + r] = load_stream16(w + (size_t)(b0 + jj) * 1024 * R + 1024 * r);
        }
#pragma unroll
      for (int g = 0; g < 2; ++g)
        buf.w[g] = load_stream4(ws_scale + (size_t)min(b0 / 4 + g, KG - 1) * 256);
    }
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int kt = b0 + jj;
      if (kt < KT) {
        v4i a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
        uint32_t sa = 127;
        if (m < n) {
          const uint8_t* ap = codes + (size_t)m * (F::MB == 1 ? K / 2 : K) + kt * 64 * R + 16 * q;
          a0 = *reinterpret_cast<const v4i*>(ap);
          if (R == 2) a1 = *reinterpret_cast<const v4i*>(ap + 64);
          sa = scales[m * (K / 32) + 4 * kt + q];
        }
        const uint32_t sb = scale_byte(buf.w[jj / 4], kt);
        if constexpr (F::MB == 1)
          acc = mfma_fp4(a0, buf.q[jj], acc, sa, sb);
        else
          acc = mfma_fp8(a0, a1, buf.q[2 * jj], buf.q[2 * jj + 1], acc, sa, sb);
        if ((kt + 1) % CT == 0) {  // end of a chunk: add its sum in chunk order
          out = kt + 1 == CT ? acc : out + acc;
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  return out;
}

// Combine of output columns 64 hg .. +64 for every row: reads the tagged down
// outputs of the group until all are this call's, then
// y = bf16( sum_j w_j d_j (j in order) + s + residual ).
template <class DA>
__device__ __forceinline__ void combine(const DA& A, uint32_t tag, const Smem& sm, int hg) {
  const int H = A.h(), k = A.kk();
  constexpr int kPer = kDecodeMaxT * 64 / kThreads;  // (row, column) pairs per thread
  float d[kPer][kMaxK], s[kPer];
  const uint64_t t0 = wall_clock64();
  bool ok;
  do {
    ok = true;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      if (idx < A.T * 64) {
        const int t = idx >> 6, h = 64 * hg + (idx & 63);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
          if (j < k) {
            const uint64_t w = ld_dev(&A.d_part[(size_t)(t * k + j) * H + h]);
            ok &= tag_ok(w, tag);
            d[p][j] = __uint_as_float((uint32_t)w);
          }
        if (A.is()) {
          const uint64_t w = ld_dev(&A.s_part[(size_t)t * H + h]);
          ok &= tag_ok(w, tag);
          s[p] = __uint_as_float((uint32_t)w);
        }
      }
    }
  } while (keep_polling(ok, t0, A.sync));
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const int idx = threadIdx.x + p * kThreads;
    if (idx < A.T * 64) {
      const int t = idx >> 6, h = 64 * hg + (idx & 63);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) acc = fmaf(sm.w[t * k + j], d[p][j], acc);
      if (A.is()) acc = acc + s[p];
      if (A.residual) acc = acc + bf16_to_f32(A.residual[(size_t)t * H + h]);
      A.y[(size_t)t * H + h] = f32_to_bf16(acc);
    }
  }
}

// One sequence entry: compute from buf, request entry j + kBufs into buf,
// store the results.
template <class DA>
__device__ __forceinline__ void run_entry(const DA& A, uint32_t tag, Smem& sm, const Seq& S, int j, Buf& buf,
                                          uint8_t* xq4_lds, uint8_t* xs4_lds, uint8_t* stage, int lane, int wave) {
  if (j < S.nb) {
    const int u = S.b0 + j, per = A.i() / 16;
    const int dd = u / per, i = u % per;
    gu_compute(A, sm, xq4_lds, xs4_lds, dd, buf, lane, wave);
    if (j == 0) trace_at(A, TR_B_MMA);
    issue(A, sm, S, j + kBufs, lane, wave, buf);  // buf is free once the matrix products have read it
    if (j == 0) trace_at(A, TR_B_NEXT);
    __syncthreads();
    int row, col;
    float a;
    if (gu_finish(sm, A.nc1(), sm.ecount[dd], &row, &col, &a))
      st_dev(&A.a_r[(size_t)sm.tl[dd][row] * A.i() + 16 * i + col], tagged(tag, a));
    if (j == 0) trace_at(A, TR_B_STORED);
    __syncthreads();  // sm.red is rewritten by the next unit
    if (j == 0) trace_at(A, TR_B_RELEASED);
    return;
  }
  const int u = S.c0 + j - S.nb;
  const bool routed = u < S.D * S.nhg;
  const int dd = routed ? u / S.nhg : -1;
  const int hg = routed ? u % S.nhg : u - S.D * S.nhg;  // 64-column group
  const int hs = 4 * hg + wave;
  const int m = lane & 15, q = lane >> 4;
  v4f out;
  if (routed) {
    const int e = sm.elist[dd], n = sm.ecount[dd];
    const int K = A.i();
    uint8_t* codes = stage;
    uint8_t* scales = stage + kDecodeMaxT * (K / 2);
    if (sm.staged != e) {
      wait_tagged_rows(A, tag, A.a_r, K, n, sm.tl[dd]);
      stage_intermediate<FP4>(A.a_r, K, n, sm.tl[dd], codes, scales);
      __syncthreads();
      if (threadIdx.x == 0) sm.staged = e;
      if (j == S.nb) trace_at(A, TR_C_STAGED);
    }
    const int KG = (A.kt2() + 3) / 4;
    const uint8_t* w = A.w2 + (size_t)e * ((size_t)A.h() * A.i() / 2) + (size_t)hs * A.kt2() * 1024 + lane * 16;
    const uint8_t* sw = A.w2s + (size_t)e * ((size_t)(A.h() / 16) * KG * 256) + ((size_t)hs * KG * 64 + lane) * 4;
    out = down_compute<FP4>(w, sw, A.kt2(), A.ct2(), codes, scales, n, buf, lane);
    issue(A, sm, S, j + kBufs, lane, wave, buf);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q + r < n)
        st_dev(&A.d_part[(size_t)sm.tl[dd][4 * q + r] * A.h() + 16 * hs + m], tagged(tag, out[r]));
  } else {
    const int K = A.is();
    uint8_t* codes = stage;
    uint8_t* scales = stage + kDecodeMaxT * K;
    if (sm.staged != -1) {
      wg_wait(ctr(A.sync, S_SA), (uint32_t)(A.is() / 16), A.sync);
      stage_intermediate<FP8>(A.a_s, K, A.T, static_cast<const uint8_t*>(nullptr), codes, scales);
      __syncthreads();
      if (threadIdx.x == 0) sm.staged = -1;
    }
    const int KG = (A.kts() + 3) / 4;
    const uint8_t* w = A.ws2 + (size_t)hs * A.kts() * 2048 + lane * 16;
    const uint8_t* sw = A.ws2s + ((size_t)hs * KG * 64 + lane) * 4;
    out = down_compute<FP8>(w, sw, A.kts(), A.cts(), codes, scales, A.T, buf, lane);
    issue(A, sm, S, j + kBufs, lane, wave, buf);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q + r < A.T) st_dev(&A.s_part[(size_t)(4 * q + r) * A.h() + 16 * hs + m], tagged(tag, out[r]));
  }
}

// ------------------------------------------------------------------ kernel
template <class DA>
__global__ void __launch_bounds__(kThreads) fused_decode_kernel(DA A) {
  __shared__ Smem sm;
  extern __shared__ __align__(16) unsigned char dyn[];  // logits, then MXFP4 x; staged intermediates
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int G = A.G, T = A.T, E = A.e();
  const uint32_t tag = ld_dev(ctr(A.sync, S_EPOCH)) + 1u;
  uint64_t* tr = A.trace + (size_t)blockIdx.x * kTraceWords;
  if (threadIdx.x == 0) {
    tr[TR_START] = wall_clock64();
    for (int i = 1; i < kTraceWords; ++i) tr[i] = 0;
  }

  // phase A
  const int n_xq = xq_units(T, A.h(), A.is());
  const int n_sgu = A.is() ? A.is() / 16 : 0;
  for (int u = blockIdx.x; u < n_xq + E + n_sgu; u += G) {
    if (u < n_xq)
      unit_xq(A, u);
    else if (u < n_xq + E)
      unit_router(A, tag, u - n_xq, lane, wave);
    else
      unit_shared_gu(A, sm, u - n_xq - E, lane, wave);
    if (threadIdx.x == 0 && u == (int)blockIdx.x) tr[TR_FIRST] = wall_clock64();
  }
  trace_at(A, TR_A);
  compiler_fence();

  // routing, identical in every workgroup: read the tagged logits until all
  // are this call's
  float* logits_lds = reinterpret_cast<float*>(dyn);
  {
    const uint64_t t0 = wall_clock64();
    bool ok;
    do {
      ok = true;
      for (int i = threadIdx.x; i < T * E; i += kThreads) {
        const uint64_t w = ld_dev(&A.logits[i]);
        ok &= tag_ok(w, tag);
        logits_lds[i] = __uint_as_float((uint32_t)w);
      }
    } while (keep_polling(ok, t0, A.sync));
  }
  trace_at(A, TR_LOGITS);
  trace_at(A, TR_LOGITS_LDS);
  if (T <= kWaves) {  // a wavefront per row
    const int row = wave < T ? wave : 0;
    row_topk64(logits_lds + row * E, wave < T, E, A.kk(), lane, sm.ids + row * A.kk(), sm.w + row * A.kk());
  } else {  // 16 lanes per row, 16 rows
    const int row = threadIdx.x / 16;
    rows_topk16(logits_lds + (row < T ? row : 0) * E, row < T, E, A.kk(), threadIdx.x & 15,
                sm.ids + (row < T ? row : 0) * A.kk(), sm.w + (row < T ? row : 0) * A.kk());
  }
  __syncthreads();
  trace_at(A, TR_TOPK);
  build_expert_list(A, sm, lane, wave);
  trace_at(A, TR_ELIST);
  if (threadIdx.x == 0) {
    wait_count(ctr(A.sync, S_XQ), (uint32_t)n_xq, A.sync);
    sm.staged = -2;
  }
  __syncthreads();
  compiler_fence();
  uint8_t* xq4_lds = dyn;
  uint8_t* xs4_lds = dyn + (size_t)T * (A.h() / 2);
  {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(A.xq4);
    uint64_t* dst = reinterpret_cast<uint64_t*>(xq4_lds);
    for (int i = threadIdx.x; i < T * A.h() / 16; i += kThreads) dst[i] = ld_dev(src + i);
    for (int i = threadIdx.x; i < T * A.h() / 32; i += kThreads) xs4_lds[i] = ld_dev(&A.xs4[i]);
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < T * A.kk(); i += kThreads) {
      if (A.ids_out) A.ids_out[i] = sm.ids[i];
      if (A.w_out) A.w_out[i] = sm.w[i];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) tr[TR_ROUTED] = wall_clock64();

  // phases B and C: contiguous runs of units per workgroup, one pipeline
  Seq S;
  S.D = sm.D;
  S.nhg = A.h() / 64;
  {
    const int NB = S.D * (A.i() / 16);
    const int NCU = S.D * S.nhg + (A.is() ? S.nhg : 0);
    const unsigned b = blockIdx.x, g = (unsigned)G;  // products stay below 2^24
    S.b0 = (int)((unsigned)NB * b / g);
    S.nb = (int)((unsigned)NB * (b + 1) / g) - S.b0;
    S.c0 = (int)((unsigned)NCU * b / g);
    S.nc = (int)((unsigned)NCU * (b + 1) / g) - S.c0;
  }
  uint8_t* stage = dyn + align_up((size_t)kDecodeMaxT * (A.h() / 2 + A.h() / 32), 16);
  const int total = S.nb + S.nc;
  Buf X, Y, Z;
  issue(A, sm, S, 0, lane, wave, X);
  issue(A, sm, S, 1, lane, wave, Y);
  issue(A, sm, S, 2, lane, wave, Z);
  for (int j = 0; j < total; j += kBufs) {  // entries rotate over the three buffers
    run_entry(A, tag, sm, S, j, X, xq4_lds, xs4_lds, stage, lane, wave);
    if (j == S.nb - 1 && threadIdx.x == 0) tr[TR_B] = wall_clock64();
    if (j + 1 < total) {
      run_entry(A, tag, sm, S, j + 1, Y, xq4_lds, xs4_lds, stage, lane, wave);
      if (j + 1 == S.nb - 1 && threadIdx.x == 0) tr[TR_B] = wall_clock64();
    }
    if (j + 2 < total) {
      run_entry(A, tag, sm, S, j + 2, Z, xq4_lds, xs4_lds, stage, lane, wave);
      if (j + 2 == S.nb - 1 && threadIdx.x == 0) tr[TR_B] = wall_clock64();
    }
  }

  // combines: workgroup b takes column groups b, b + G, ...
  for (int hg = blockIdx.x; hg < S.nhg; hg += G) combine(A, tag, sm, hg);

  // exit: the last workgroup resets the launch-wide counters
  __syncthreads();
  if (threadIdx.x == 0) {
    tr[TR_C] = wall_clock64();
    if (blockIdx.x == 0) st_dev(ctr(A.sync, S_GRID), (uint32_t)G);
    compiler_fence();
    wait_vm<0>();
    const uint32_t old = __hip_atomic_fetch_add(ctr(A.sync, S_DONE), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    compiler_fence();
    if (old + 1 == (uint32_t)G) {
      st_dev(ctr(A.sync, S_EPOCH), tag);  // the next call's tag is one more
      st_dev(ctr(A.sync, S_XQ), 0u);
      st_dev(ctr(A.sync, S_SA), 0u);
      compiler_fence();
      wait_vm<0>();
      st_dev(ctr(A.sync, S_DONE), 0u);
    }
  }
}

// ------------------------------------------------------------------ host side
struct Carve {
  size_t sync, sync_end;
  size_t logits, xq4, xs4, xq8, xs8, a_r, a_s, d_part, s_part, trace, total;
};

Carve carve(const moe_layer_t& L) {
  const size_t T = kDecodeMaxT, H = L.hidden, I = L.inter, E = L.num_experts, k = L.top_k,
               Is = L.shared_inter;
  Carve c{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  const size_t line = kLine * 4;
  c.sync = take(kSyncLines * line);
  c.sync_end = o;
  c.logits = take(T * E * 8);
  c.xq4 = take(T * H / 2);
  c.xs4 = take(T * H / 32);
  c.xq8 = take(T * H);
  c.xs8 = take(T * H / 32);
  c.a_r = take(T * k * I * 8);
  c.a_s = take(T * Is * 4 + 16);
  c.d_part = take(T * k * H * 8);
  c.s_part = take(T * H * 8);
  c.trace = take((size_t)kDecodeMaxGrid * kTraceWords * 8);
  c.total = o;
  return c;
}

// Dynamic LDS: max(logits, MXFP4 x) followed by the staged intermediate.
size_t dyn_lds_bytes(const moe_layer_t& L) {
  const size_t T = kDecodeMaxT;
  const size_t logits = T * L.num_experts * 4;
  const size_t xq = align_up(T * (L.hidden / 2 + L.hidden / 32), 16);
  const size_t st4 = T * (L.inter / 2 + L.inter / 32);
  const size_t st8 = T * ((size_t)L.shared_inter + L.shared_inter / 32);
  return align_up(logits > xq ? logits : xq, 16) + align_up(st4 > st8 ? st4 : st8, 16);
}

template <class DA>
int grid_size(size_t lds) {
  static int cached_dev = -1, cached_grid = 0;
  static size_t cached_lds = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev == cached_dev && lds == cached_lds) return cached_grid;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fused_decode_kernel<DA>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_decode_kernel<DA>, kThreads, lds) != hipSuccess)
    return 0;
  if (occ > 1) occ = 1;
  cached_dev = dev;
  cached_lds = lds;
  cached_grid = occ * cus;
  if (cached_grid > kDecodeMaxGrid) cached_grid = kDecodeMaxGrid;
  return cached_grid;
}

template <class DA>
hipError_t launch_instance(const DecodeArgs& args, size_t lds, hipStream_t stream) {
  DA A;
  static_cast<DecodeArgs&>(A) = args;
  A.G = grid_size<DA>(lds);
  if (A.G <= 0) return hipErrorInvalidDeviceFunction;
  hipLaunchKernelGGL(fused_decode_kernel<DA>, dim3(A.G), dim3(kThreads), lds, stream, A);
  return hipGetLastError();
}

// The MiniMax-M3.1 layer shape (hidden 3072, 128 experts top-4, intermediate
// 1024, shared intermediate 1024) has its own compiled instance.
using MiniMaxShape = DArgs<3072, 1024, 1024, 128, 4>;
using AnyShape = DArgs<0, 0, 0, 0, 0>;

int n_chunks(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }

}  // namespace

size_t decode_ws_bytes(const moe_layer_t& L) { return carve(L).total; }
size_t decode_sync_bytes(const moe_layer_t& L) { return carve(L).sync_end; }
size_t decode_trace_offset(const moe_layer_t& L) { return carve(L).trace; }

bool decode_supported(const moe_layer_t& L) {
  // a K-chunk of the gate/up (K = H) must fit the register buffers
  const int KT1 = L.hidden / 128;
  return KT1 / n_chunks(KT1) <= kMaxCT && dyn_lds_bytes(L) + sizeof(Smem) <= 160 * 1024;
}

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
  A.NC1 = n_chunks(A.KT1);
  A.CT1 = A.KT1 / A.NC1;
  A.KT2 = A.I / 128;
  A.CT2 = A.KT2 / n_chunks(A.KT2);
  A.KTs = A.Is / 128;
  A.CTs = A.Is ? A.KTs / n_chunks(A.KTs) : 1;
  if (A.CT1 > kMaxCT) return hipErrorInvalidValue;
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
  A.x = x;
  A.residual = residual;
  A.y = y;
  A.ids_out = ids_out;
  A.w_out = w_out;
  A.sync = reinterpret_cast<uint32_t*>(base + c.sync);
  A.logits = reinterpret_cast<uint64_t*>(base + c.logits);
  A.xq4 = reinterpret_cast<uint8_t*>(base + c.xq4);
  A.xs4 = reinterpret_cast<uint8_t*>(base + c.xs4);
  A.xq8 = reinterpret_cast<uint8_t*>(base + c.xq8);
  A.xs8 = reinterpret_cast<uint8_t*>(base + c.xs8);
  A.a_r = reinterpret_cast<uint64_t*>(base + c.a_r);
  A.a_s = reinterpret_cast<float*>(base + c.a_s);
  A.d_part = reinterpret_cast<uint64_t*>(base + c.d_part);
  A.s_part = reinterpret_cast<uint64_t*>(base + c.s_part);
  A.trace = reinterpret_cast<uint64_t*>(base + c.trace);
  if (A.H == 3072 && A.I == 1024 && A.Is == 1024 && A.E == 128 && A.k == 4)
    return launch_instance<MiniMaxShape>(A, lds, stream);
  return launch_instance<AnyShape>(A, lds, stream);
}

}  // namespace mxmoe
