// The whole MoE layer for 1..16 rows in one kernel launch ("mono decode": one
// fused launch per MoE layer for a pure decode step of at most 16 tokens,
// article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and optimization",
// section "Serving with vLLM / What we Optimized").
//
// Structure.  A persistent grid of G 4-wavefront workgroups (G at most the
// device's co-resident capacity) runs three lists of work units:
//
//   phase A  (workgroup b takes units b, b+G, ...)
//            router logits (one unit per expert, all rows),
//            shared-expert gate/up (one unit per 16-column strip of the gate
//            or the up half, on an MXFP8 copy of x the workgroup makes in
//            LDS; the four wavefronts split K);
//   routing  every workgroup waits for all logits, takes the top k of each
//            row and builds the same list of the D selected experts; the
//            MXFP4 copy of x its gate/up units read is in LDS by then (up to
//            4 rows: all rows, made while waiting for the logits) or is made
//            now (more rows: only the rows routed to its experts);
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
#include <atomic>
#include <mutex>

#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxK = 8;
constexpr int kGroup = 16;     // rows of one matrix-instruction row block
constexpr int kMaxCT = 6;      // tiles of a gate/up K-chunk held in registers
constexpr int kBufQuads = 12;  // 16-byte weight loads one prefetch buffer holds per lane
constexpr int kBufs = 3;       // register buffers of the unit pipeline
constexpr int kDownBatch = 8;  // routed (MXFP4) down tiles per register batch; MXFP8: half
constexpr uint64_t kSpinTicks = 100000000ull;  // ~1 s of the 100 MHz constant clock
constexpr uint16_t kBf16NaN = 0x7fc0;

// Every counter sits on a 256-byte line of its own: device-scope atomics on
// one line are serialized by the memory side.
constexpr int kLine = 64;  // words
__device__ __forceinline__ uint32_t* ctr(uint32_t* base, int i) { return base + (size_t)i * kLine; }
// Lines of the sync block: status, done, x-quant, shared-intermediate ready,
// grid size of the last call, call epoch.
enum { S_STATUS = 0, S_DONE = 1, S_GRID = 2, S_EPOCH = 3, kSyncLines = 4 };
static_assert(kDecodeGridOffset == (size_t)S_GRID * kLine * 4, "grid word offset");
static_assert(kDecodeStatusOffset == (size_t)S_STATUS * kLine * 4, "status word offset");

// Timestamps each workgroup records (100 MHz device clock).
enum {
  TR_START = 0, TR_A = 1, TR_LOGITS = 2, TR_ROUTED = 3, TR_B = 4, TR_C = 5, TR_FIRST = 6,
  TR_XQ = 7, TR_TOPK = 8, TR_ELIST = 9,
  TR_B_MMA = 10, TR_B_STORED = 11, TR_S_MMA = 12, TR_B_RELEASED = 13, TR_C_STAGED = 14, TR_TAG = 15
};

struct DecodeArgs {
  int T, H, I, E, k, Is, G;
  int fold;           // the shared expert is expert E of the table (1) or MXFP8 (0)
  const float* norm_w;  // pre-router RMSNorm weight [H], or null
  float norm_eps;
  int gamma_off;        // dynamic-LDS byte offsets: the norm weight's copy,
  int off_xq4, off_stage, off_x8;  // the MXFP4 x, the staged intermediate, the MXFP8 x
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
  uint64_t* a_r;  // tagged [T*k][I]
  uint64_t* a_s;  // tagged [T][2 I_s]
  uint64_t *d_part, *s_part;  // tagged [T*k][H], [T][H]
  uint64_t* tagged;           // every tagged word above: one contiguous range
  uint32_t n_tagged;
  uint64_t* trace;
};

// The shape as the kernel sees it: compile-time constants where the launch
// picked a specialization for the layer's shape (H_, I_, IS_, E_, K_ non-zero,
// IS_ = -1 for no MXFP8 shared expert; FOLD_ 0 or 1, -1 for run time), the
// run-time fields otherwise.  kr() is the router's k; kk() the slots per row:
// the k routed choices and, with the shared expert folded into the table, one
// more slot (expert E, weight 1).
constexpr int n_chunks_of(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }
template <int H_, int I_, int IS_, int E_, int K_, int FOLD_, int MT_>
struct DArgs : DecodeArgs {
  static constexpr bool kFixedShape = H_ != 0;  // a compiled instance for one layer shape
  static constexpr int kMaxT = MT_;              // rows the instance takes (16, or 64 for wide steps)
  static constexpr bool kWide = MT_ > kGroup;
  __device__ __forceinline__ int h() const { return H_ ? H_ : H; }
  __device__ __forceinline__ int i() const { return I_ ? I_ : I; }
  __device__ __forceinline__ int is() const { return IS_ ? (IS_ < 0 ? 0 : IS_) : Is; }
  __device__ __forceinline__ int e() const { return E_ ? E_ : E; }
  __device__ __forceinline__ int kr() const { return K_ ? K_ : k; }
  __device__ __forceinline__ int fd() const { return FOLD_ >= 0 ? FOLD_ : fold; }
  __device__ __forceinline__ int kk() const { return kr() + fd(); }
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

// Per-workgroup state for an instance taking up to MT rows.  The slots routed
// to selected expert dd are slist[eoff[dd] .. eoff[dd] + ecount[dd]).
template <int MT>
struct SmemT {
  static constexpr int kSlots = MT * kMaxK;
  int32_t ids[kSlots];
  float w[kSlots];
  uint64_t rmask[256];  // rows selecting each expert (an expert takes at most one slot per row)
  int epos[256];
  uint8_t elist[kSlots];
  uint8_t ecount[kSlots];
  uint16_t eoff[kSlots];
  uint16_t slist[kSlots];
  // wide instance: expert-groups q = (selected expert qd[q], rows 16 qg[q] ..
  // +16), experts in list order; the folded shared expert's are the last NQF
  uint16_t qd[kSlots];
  uint8_t qg[kSlots];
  int NQ, NQF;
  float red[kWaves][2][kGroup][16];             // chunk sums [chunk][gate/up][row][column]
  int wave_cnt[kWaves];
  int wave_sum[kWaves];
  uint8_t qrows[MT];                            // rows of x quantized for this workgroup's gate/up units
  float rnorm[MT];                              // pre-router RMSNorm factor of each row
  int D;
  int flag;
  int last;                                     // this workgroup is the call's last to finish
  __device__ __forceinline__ int slot(int dd, int i) const { return slist[eoff[dd] + i]; }
};
template <class DA>
using SmemOf = SmemT<DA::kMaxT>;

// ------------------------------------------------------------------ synchronisation
// Data handed from one workgroup to another (logits, gate/up results,
// partial outputs) is written and read with relaxed agent-scope atomic
// accesses, which gfx950 issues with the sc1 bit: they are served at the
// device's coherence point, past the per-XCD L2 caches, so no L2 write-back
// or invalidate is needed.  Each value is stored as one 64-bit word (tag << 32
// | fp32 bits), single-copy atomic, and a consumer reads the words until
// every tag is this call's: no counter is bumped, so producers never wait for
// their stores to be acknowledged and many producers never serialize on one
// address.  The tag is one more than the epoch word, which the last workgroup
// of a call advances, so words of an earlier call (or the zero-filled
// workspace) never match.
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

__device__ __forceinline__ uint64_t tagged_u(uint32_t tag, uint32_t v) { return ((uint64_t)tag << 32) | v; }
__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) { return tagged_u(tag, __float_as_uint(v)); }
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
// Eight consecutive lanes (8i .. 8i+7) hold the 32 values of one block (lane
// j: values 4j..4j+3, fp32 bit patterns) and agree on the block scale in
// three steps.  Returns the four codes packed (FP4: 16 bits, element 4j+i
// in nibble i; FP8: 32 bits, byte i) and the E8M0 code in *scale.
template <class F>
__device__ __forceinline__ uint32_t quant_block8(const uint32_t (&bits)[4], uint32_t* scale) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) am = max(am, bits[i] & 0x7fffffffu);
  // maximum over the eight lanes with data-parallel moves (every lane of the
  // group is active): swap neighbours, swap pairs, mirror the half row
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xf, 0xf, false));
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0x4E, 0xf, 0xf, false));
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0x141, 0xf, 0xf, false));
  const int e = block_exponent<F>(am);
  const float inv = block_inv_scale(e);
  uint32_t packed = 0;
  if constexpr (F::MB == 1) {
    packed = quant_quad_fp4(bits[0], bits[1], bits[2], bits[3], inv);
  } else {
    packed = quant_pair_fp8(bits[0], bits[1], inv) | (quant_pair_fp8(bits[2], bits[3], inv) << 16);
  }
  *scale = (uint32_t)(e + 127);
  return packed;
}

// ------------------------------------------------------------------ x quantization
// Every workgroup quantizes the rows of x it needs itself, into LDS: a shared
// gate/up strip all T rows (MXFP8); for the routed gate/up units, with at most
// kEarlyQuantT rows all rows before routing (while the workgroup would wait
// for the logits anyway; a strip quantizes them from the x values it already
// holds), with more rows only the rows of the tokens routed to their experts,
// once routing is known (quantizing all 16 rows in every workgroup would cost
// far more than the wait it fills).  A task
// is one 32-value block (row, block b) of a list of rows: task t covers row
// rows[t / (H/32)] (row t / (H/32) without a list) and block t mod (H/32).
// The eight lanes of group g = threadIdx / 8 handle tasks t0 + p * 32 + g of a
// batch (p < kQBatch), lane j taking values 4j .. 4j+3 (bf16 x, read with
// plain loads: x does not change during the call).  A batch's loads are all
// issued before any of its blocks is quantized.
constexpr int kQBatch = 16;
constexpr int kEarlyQuantT = 4;
// phase-B/C parts of the late and the other workgroups with the pre-router
// norm above kEarlyQuantT rows (see decode_body)
constexpr unsigned kNormEarly = 3, kNormLate = 2;
static_assert(kNormEarly <= 3 && kNormLate <= kNormEarly, "the unit cut's 32-bit products assume parts of at most 3");
constexpr int kQGroups = kThreads / 8;

// Without a row list (kRows false) task t is block t of x in row-major
// order, so every offset is linear in t: x elements 32 t, MXFP8 code bytes
// 32 t, MXFP4 code bytes 16 t, scale t.
template <bool kRows, class DA>
__device__ __forceinline__ void x_batch_load(const DA& A, int t0, int tasks, const uint8_t* rows,
                                             uint32_t (&bits)[kQBatch][4], int blk0 = 0) {
  const int H = A.h(), nb = H / 32, j = threadIdx.x & 7, grp = threadIdx.x / 8;
#pragma unroll
  for (int p = 0; p < kQBatch; ++p) {
    const int task = t0 + p * kQGroups + grp;
    bits[p][0] = bits[p][1] = bits[p][2] = bits[p][3] = 0u;
    if (task < tasks) {
      const size_t off = kRows ? (size_t)rows[task / nb] * H + 32 * (task % nb) : 32 * ((size_t)blk0 + task);
      const uint2 v = *reinterpret_cast<const uint2*>(A.x + off + 4 * j);
      bits[p][0] = v.x << 16;
      bits[p][1] = v.x & 0xffff0000u;
      bits[p][2] = v.y << 16;
      bits[p][3] = v.y & 0xffff0000u;
    }
  }
}

// With the pre-router norm, before the workgroup's first x quantization: the
// norm weight copied into LDS and, unless a router unit of this workgroup has
// left them in sm.rnorm, every row's norm factor.
template <class DA>
__device__ __forceinline__ void norm_setup(const DA& A, SmemOf<DA>& sm, float* gamma_lds, bool need_r, int lane, int wave) {
  if (!DA::kWide)
    for (int i = threadIdx.x; i < A.h() / 4; i += kThreads)
      reinterpret_cast<float4*>(gamma_lds)[i] = reinterpret_cast<const float4*>(A.norm_w)[i];
  if (need_r)
    for (int t = wave; t < A.T; t += kWaves) {
      const float v = row_rms_inv(A.x + (size_t)t * A.h(), A.h(), A.norm_eps, lane);
      if (lane == 0) sm.rnorm[t] = v;
    }
  __syncthreads();
}

// With the pre-router norm: the loaded batch becomes (h * r) * g.
template <bool kRows, class DA>
__device__ __forceinline__ void x_batch_norm(const DA& A, const SmemOf<DA>& sm, const float* gamma_lds, int t0, int tasks,
                                             const uint8_t* rows, uint32_t (&bits)[kQBatch][4], int blk0 = 0) {
  const int H = A.h(), nb = H / 32, j = threadIdx.x & 7, grp = threadIdx.x / 8;
#pragma unroll
  for (int p = 0; p < kQBatch; ++p) {
    const int task = t0 + p * kQGroups + grp;
    if (task < tasks) {
      const int row = kRows ? rows[task / nb] : (blk0 + task) / nb;
      const float r = sm.rnorm[row];
      const float* gp = DA::kWide ? A.norm_w : gamma_lds;  // the wide instance keeps no LDS copy
      const float4 g = *reinterpret_cast<const float4*>(gp + 32 * (task % nb) + 4 * j);
      bits[p][0] = normed_bits(bits[p][0], r, g.x);
      bits[p][1] = normed_bits(bits[p][1], r, g.y);
      bits[p][2] = normed_bits(bits[p][2], r, g.z);
      bits[p][3] = normed_bits(bits[p][3], r, g.w);
    }
  }
}

// Quantizes a loaded batch to format F: codes [T][H * bytes per element],
// scales [T][H/32] (indexed by the real row).
template <class F, bool kRows, class DA>
__device__ __forceinline__ void x_batch_quant(const DA& A, int t0, int tasks, const uint8_t* rows,
                                              const uint32_t (&bits)[kQBatch][4], uint8_t* codes,
                                              uint8_t* scales) {
  const int H = A.h(), nb = H / 32, j = threadIdx.x & 7, grp = threadIdx.x / 8;
#pragma unroll
  for (int p = 0; p < kQBatch; ++p) {
    if (t0 + p * kQGroups >= tasks) break;  // uniform
    const int task = t0 + p * kQGroups + grp;
    uint32_t sc;
    const uint32_t packed = quant_block8<F>(bits[p], &sc);
    if (task < tasks) {
      // block index in row-major order: task itself without a row list
      const int blk = kRows ? rows[task / nb] * nb + task % nb : task;
      if constexpr (F::MB == 1)
        *reinterpret_cast<uint16_t*>(codes + 16 * blk + 2 * j) = (uint16_t)packed;
      else
        *reinterpret_cast<uint32_t*>(codes + 32 * blk + 4 * j) = packed;
      if (j == 0) scales[blk] = (uint8_t)sc;
    }
  }
}

// ------------------------------------------------------------------ phase A
// Logits of expert e for all rows; wave w takes rows w, w+4, ...  Same
// per-row arithmetic as router_lane_partial: each batch of up to 16 strides
// of the expert's weights is loaded once, then the rows go through it two at
// a time.
// Rows wave + 4 (rc + r), r < nr (at most 4) of one router unit.
template <class DA>
__device__ __forceinline__ void router_rows(const DA& A, SmemOf<DA>& sm, uint32_t tag, int e, int rc, int nr,
                                            int lane, int wave) {
  const float* wrow = A.router_w + (size_t)e * A.h();
  const int H = A.h();
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  if (A.norm_w) {
    // The normalized rows (h * r) * g.  With H <= 4096 the unit loads the
    // expert's weights and g once, then takes the rows two at a time: each
    // row's norm factor comes from the x values already in registers (same
    // order as row_rms_inv: lane partial sums over h = 256 i + 4 l + c, then
    // the butterfly) and is left in sm.rnorm for the workgroup's own x
    // quantization.  Wider rows, and the run-time shape instance (whose
    // registers this would exhaust), take the factor from row_rms_inv first.
    if (DA::kFixedShape && H <= 16 * 256) {
      float4 w[16], g[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (4 * lane + 256 * j < H) {
          w[j] = load_stream_f4(wrow + 4 * lane + 256 * j);
          g[j] = *reinterpret_cast<const float4*>(A.norm_w + 4 * lane + 256 * j);
        }
#pragma unroll
      for (int r0 = 0; r0 < 4; r0 += 2) {
        if (r0 < nr) {
          uint2 xv[2][16];
#pragma unroll
          for (int r = 0; r < 2; ++r)
            if (r0 + r < nr) {
              const uint16_t* xr = A.x + (size_t)(wave + kWaves * (rc + r0 + r)) * H;
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (4 * lane + 256 * j < H) xv[r][j] = *reinterpret_cast<const uint2*>(xr + 4 * lane + 256 * j);
            }
#pragma unroll
          for (int r = 0; r < 2; ++r)
            if (r0 + r < nr) {
              float sq = 0.f;
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (4 * lane + 256 * j < H) {
                  const float a = bf16_to_f32(xv[r][j].x & 0xffffu), b = bf16_to_f32(xv[r][j].x >> 16);
                  const float c = bf16_to_f32(xv[r][j].y & 0xffffu), d = bf16_to_f32(xv[r][j].y >> 16);
                  sq = fmaf(a, a, sq);
                  sq = fmaf(b, b, sq);
                  sq = fmaf(c, c, sq);
                  sq = fmaf(d, d, sq);
                }
              const float rr = 1.0f / sqrtf(wave_sum_butterfly(sq) / (float)H + A.norm_eps);
              if (lane == 0) sm.rnorm[wave + kWaves * (rc + r0 + r)] = rr;
              float& acc = p[r0 + r];
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (4 * lane + 256 * j < H) {
                  acc = fmaf(__uint_as_float(normed_bits((xv[r][j].x & 0xffffu) << 16, rr, g[j].x)), w[j].x, acc);
                  acc = fmaf(__uint_as_float(normed_bits(xv[r][j].x & 0xffff0000u, rr, g[j].y)), w[j].y, acc);
                  acc = fmaf(__uint_as_float(normed_bits((xv[r][j].y & 0xffffu) << 16, rr, g[j].z)), w[j].z, acc);
                  acc = fmaf(__uint_as_float(normed_bits(xv[r][j].y & 0xffff0000u, rr, g[j].w)), w[j].w, acc);
                }
            }
        }
      }
    } else {
      for (int r = 0; r < nr; ++r) {
        const int row = wave + kWaves * (rc + r);
        const float rr = row_rms_inv(A.x + (size_t)row * H, H, A.norm_eps, lane);
        if (lane == 0) sm.rnorm[row] = rr;
        const uint16_t* xr = A.x + (size_t)row * H;
        float& acc = p[r];
        for (int h0 = 4 * lane; h0 < H; h0 += 256) {
          const float4 w = load_stream_f4(wrow + h0), g = *reinterpret_cast<const float4*>(A.norm_w + h0);
          const uint2 xv = *reinterpret_cast<const uint2*>(xr + h0);
          acc = fmaf(__uint_as_float(normed_bits((xv.x & 0xffffu) << 16, rr, g.x)), w.x, acc);
          acc = fmaf(__uint_as_float(normed_bits(xv.x & 0xffff0000u, rr, g.y)), w.y, acc);
          acc = fmaf(__uint_as_float(normed_bits((xv.y & 0xffffu) << 16, rr, g.z)), w.z, acc);
          acc = fmaf(__uint_as_float(normed_bits(xv.y & 0xffff0000u, rr, g.w)), w.w, acc);
        }
      }
    }
    const float b = A.router_bias ? A.router_bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < nr) {
        float v = wave_sum_butterfly(p[r]);
        if (A.router_bias) v = v + b;
        if (lane == 0) st_dev(&A.logits[(wave + kWaves * (rc + r)) * A.e() + e], tagged(tag, v));
      }
    return;
  }
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
            const uint16_t* xr = A.x + (size_t)(wave + kWaves * (rc + r0 + r)) * H;
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
      if (lane == 0) st_dev(&A.logits[(wave + kWaves * (rc + r)) * A.e() + e], tagged(tag, v));
    }
}

template <class DA>
__device__ __forceinline__ void unit_router(const DA& A, SmemOf<DA>& sm, uint32_t tag, int e, int lane, int wave) {
  int nr = 0;
  for (int t = wave; t < A.T; t += kWaves) ++nr;
  // four rows per pass (one pass unless the wide instance has more rows)
  for (int rc = 0; rc < (DA::kWide ? nr : 1); rc += 4)
    if (rc < nr) router_rows(A, sm, tag, e, rc, min(nr - rc, 4), lane, wave);
}

// Shared gate/up strip st (0 <= st < 2 I_s/16: gate strips, then up strips):
// wave w computes K-chunk w (MXFP8 x MXFP8); the chunk sums meet in LDS and
// are added in chunk order.  The workgroup first quantizes x itself to MXFP8
// (x8: codes [16][H], scales at 16 H; 16-row groups in turn) and, with at most
// kEarlyQuantT rows, to MXFP4 (the copy the routed gate/up units read later);
// the first batch of x is requested before the weights, so that quantizing
// does not wait for them.  The fp32 result
// goes to a_s[row][16 st + col] as tagged words (gate columns, then up
// columns); SwiGLU is applied where it is staged.
template <class DA>
__device__ __forceinline__ void unit_shared_strip(const DA& A, uint32_t tag, SmemOf<DA>& sm, const float* gamma_lds, int st,
                                                  int g0, uint8_t* x8, uint8_t* xq4, uint8_t* xs4, int lane,
                                                  int wave) {
  const int CT = A.ct1(), KG = (A.kt1() + 3) / 4, nb = A.h() / 32;
  const int m = lane & 15, q = lane >> 4;
  const bool act = wave < A.nc1();
  const int t0 = wave * CT;
  uint8_t* xs8 = x8 + (size_t)kGroup * A.h();
  uint32_t bits[kQBatch][4];
  x_batch_load<false>(A, 0, min(A.T - g0, kGroup) * nb, nullptr, bits, g0 * nb);
  v4i B[kMaxCT][2];
  uint32_t sw[3];
  if (act) {
    const uint8_t* wb = A.ws13 + ((size_t)st * A.kt1() + t0) * 2048 + lane * 16;
#pragma unroll
    for (int j = 0; j < kMaxCT; ++j)
      if (j < CT) {
        B[j][0] = load_stream16(wb + j * 2048);
        B[j][1] = load_stream16(wb + j * 2048 + 1024);
      }
    const uint8_t* sp = A.ws13s + ((size_t)st * KG * 64 + lane) * 4;
#pragma unroll
    for (int g = 0; g < 3; ++g) sw[g] = load_stream4(sp + (size_t)min(t0 / 4 + g, KG - 1) * 256);
  }
  // the strip's 16-row group of x (the wide instance schedules one unit per group)
  {
    const int ng = min(A.T - g0, kGroup), tasks = ng * nb;
    for (int b0 = 0; b0 < tasks; b0 += kQBatch * kQGroups) {
      if (b0 > 0) x_batch_load<false>(A, b0, tasks, nullptr, bits, g0 * nb);
      if (A.norm_w) x_batch_norm<false>(A, sm, gamma_lds, b0, tasks, nullptr, bits, g0 * nb);
      x_batch_quant<FP8, false>(A, b0, tasks, nullptr, bits, x8, xs8);
      if (A.T <= kEarlyQuantT) x_batch_quant<FP4, false>(A, b0, tasks, nullptr, bits, xq4, xs4);
    }
    trace_at(A, TR_XQ);
    __syncthreads();
    if (act) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxCT; ++j)
        if (j < CT) {
          const int kt = t0 + j;
          // rows past the group repeat its last row: their sums are never read
          const int mr = m < ng ? m : ng - 1;
          const uint8_t* ap = x8 + (size_t)mr * A.h() + kt * 128 + 16 * q;
          const v4i a0 = *reinterpret_cast<const v4i*>(ap);
          const v4i a1 = *reinterpret_cast<const v4i*>(ap + 64);
          const uint32_t sa = xs8[mr * (A.h() / 32) + 4 * kt + q];
          const uint32_t word = pick3(sw[0], sw[1], sw[2], kt / 4 - t0 / 4);
          acc = mfma_fp8(a0, a1, B[j][0], B[j][1], acc, sa, scale_byte(word, kt));
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[wave][0][4 * q + r][m] = acc[r];
    }
    trace_at(A, TR_S_MMA);
    __syncthreads();
    const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (r < ng) {
      float v = sm.red[0][0][r][c];
      for (int ch = 1; ch < A.nc1(); ++ch) v = v + sm.red[ch][0][r][c];
      st_dev(&A.a_s[(size_t)(g0 + r) * (2 * A.is()) + 16 * st + c], tagged(tag, v));
    }
    __syncthreads();  // sm.red and x8 are reused
  }
}

// Gate/up unit i of the folded shared expert (expert E of the table, every
// row in slot k of its row), run in phase A since every row selects it: the
// workgroup makes the MXFP4 copy of all rows of x (its first loads issued
// ahead of the weight tiles), then the unit computes like a routed one and
// stores the SwiGLU values of slots t*kk + k as tagged words.
template <class DA>
__device__ __forceinline__ void unit_fold_gu(const DA& A, uint32_t tag, SmemOf<DA>& sm, const float* gamma_lds, int i,
                                             uint8_t* xq4, uint8_t* xs4, bool& have_x4, int lane, int wave);

// Chunk sums of a routed gate/up unit in sm.red, added in chunk order, then
// SwiGLU: thread (row, column) for row < n; returns false for idle threads.
template <class SM>
__device__ __forceinline__ bool gu_finish(const SM& sm, int nc, int n, int* row, int* col, float* a) {
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

// ------------------------------------------------------------------ routing
// Selected experts in ascending expert order and the slots routed to each, in
// ascending row order.  Every workgroup builds the same lists: the wide
// instance cuts a list into 16-slot groups, and the workgroup writing a
// group's gate/up results and the one reading them must agree on its slots.
// A row takes an expert at most once, so the rows selecting expert e form a
// bit mask, and a slot's place in e's list is the number of earlier rows in it.
template <class DA>
__device__ __forceinline__ void build_expert_list(const DA& A, SmemOf<DA>& sm, int lane, int wave) {
  static_assert(DA::kMaxT <= 64, "one mask bit per row");
  const int S = A.T * A.kk(), tid = threadIdx.x;
  if (!DA::kWide && A.T == 1) {
    // One row: its kk experts are distinct, so an expert's place in the list
    // is its rank among them and its slot list is its own slot (the lists
    // below come out the same).
    const int kk = A.kk();
    if (tid < kk) {
      const int e = sm.ids[tid];
      int dd = 0;
      for (int j = 0; j < kk; ++j) dd += sm.ids[j] < e ? 1 : 0;
      sm.elist[dd] = (uint8_t)e;
      sm.ecount[dd] = 1;
      sm.eoff[dd] = (uint16_t)dd;
      sm.slist[dd] = (uint16_t)tid;
    }
    if (tid == 0) sm.D = kk;
    __syncthreads();
    return;
  }
  sm.rmask[tid] = 0ull;
  __syncthreads();
  for (int sl = tid; sl < S; sl += kThreads) atomicOr(&sm.rmask[sm.ids[sl]], 1ull << (sl / A.kk()));
  __syncthreads();
  const int cnt = __popcll(sm.rmask[tid]);
  const bool used = cnt > 0;
  const uint64_t mask = __ballot(used);
  // inclusive scan of the counts over the wavefront (expert order)
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
  if (lane == kWave - 1) sm.wave_sum[wave] = incl;
  __syncthreads();
  int base = 0, sbase = 0;
  for (int w = 0; w < wave; ++w) {
    base += sm.wave_cnt[w];
    sbase += sm.wave_sum[w];
  }
  if (used) {
    const int dd = base + __popcll(mask & ((1ull << lane) - 1ull));
    sm.elist[dd] = (uint8_t)tid;
    sm.ecount[dd] = (uint8_t)cnt;
    sm.eoff[dd] = (uint16_t)(sbase + incl - cnt);
    sm.epos[tid] = dd;
  }
  if (tid == 0) sm.D = sm.wave_cnt[0] + sm.wave_cnt[1] + sm.wave_cnt[2] + sm.wave_cnt[3];
  __syncthreads();
  for (int sl = tid; sl < S; sl += kThreads) {
    const int e = sm.ids[sl];
    const uint64_t before = sm.rmask[e] & ((1ull << (sl / A.kk())) - 1ull);
    sm.slist[sm.eoff[sm.epos[e]] + __popcll(before)] = (uint16_t)sl;
  }
  if constexpr (DA::kWide) {
    // expert-groups: ceil(count / 16) per selected expert (thread tid = dd)
    const int D = sm.D;
    const int ng = tid < D ? (sm.ecount[tid] + kGroup - 1) / kGroup : 0;
    int gi = ng;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(gi, d);
      if (lane >= d) gi += v;
    }
    __syncthreads();  // sm.wave_sum is reused
    if (lane == kWave - 1) sm.wave_sum[wave] = gi;
    __syncthreads();
    int gbase = 0;
    for (int w = 0; w < wave; ++w) gbase += sm.wave_sum[w];
    for (int g = 0; g < ng; ++g) {
      sm.qd[gbase + gi - ng + g] = (uint16_t)tid;
      sm.qg[gbase + gi - ng + g] = (uint8_t)g;
    }
    if (tid == 0) {
      sm.NQ = sm.wave_sum[0] + sm.wave_sum[1] + sm.wave_sum[2] + sm.wave_sum[3];
      sm.NQF = A.fd() ? (A.T + kGroup - 1) / kGroup : 0;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ phases B and C
// Unit j of a workgroup's sequence: its phase-B units [b0, b1) then its
// phase-C units [c0, c1).
struct Seq {
  int b0, nb, c0, nc;
  int D, nhg, ns;  // selected experts, 64-column groups, shared down units
  int fold;        // the last selected expert is the folded shared expert (gate/up done in phase A)
  int NQ, NQF;     // wide instance: expert-groups, of which the folded expert's (the last)
};

struct Buf {
  v4i q[kBufQuads];
  // scale words as separate members: every index below is a constant once
  // the loops are unrolled, and an array here has ended up in scratch memory
  uint32_t w0, w1, w2, w3, w4, w5;
  __device__ __forceinline__ uint32_t& w(int i) {
    switch (i) {
      case 0: return w0;
      case 1: return w1;
      case 2: return w2;
      case 3: return w3;
      case 4: return w4;
      default: return w5;
    }
  }
  __device__ __forceinline__ uint32_t w(int i) const { return const_cast<Buf*>(this)->w(i); }
};

// Requests the weight tiles and scale words of sequence entry j into buf.
// The scale words are gathered in scalars and stored to buf once, on a single
// path: stores to different members on different paths get merged into one
// store through a pointer, which keeps buf in scratch memory.
// The weight tiles and scale words of a gate/up unit (expert e, 16-column
// strip i of the gate half and of the up half; this wavefront's K-chunk).
// The scale words come back in n0..n5 (the caller stores them to buf on its
// single store path); false for a wavefront without a K-chunk.
template <class DA>
__device__ __forceinline__ bool issue_gu(const DA& A, int e, int i, int lane, int wave, Buf& buf, uint32_t& n0,
                                         uint32_t& n1, uint32_t& n2, uint32_t& n3, uint32_t& n4, uint32_t& n5) {
  if (wave >= A.nc1()) return false;
  {
    const int CT = A.ct1(), KG = (A.kt1() + 3) / 4, t0 = wave * CT;
    const uint8_t* base = A.w13 + (size_t)e * ((size_t)A.i() * A.h());
    const uint8_t* sbase = A.w13s + (size_t)e * ((size_t)(2 * A.i() / 16) * KG * 256);
    const int st0 = i, st1 = A.i() / 16 + i;
    const uint8_t* wb0 = base + ((size_t)st0 * A.kt1() + t0) * 1024 + lane * 16;
    const uint8_t* wb1 = base + ((size_t)st1 * A.kt1() + t0) * 1024 + lane * 16;
#pragma unroll
    for (int jj = 0; jj < kMaxCT; ++jj)
      if (jj < CT) buf.q[jj] = load_stream16(wb0 + jj * 1024);
#pragma unroll
    for (int jj = 0; jj < kMaxCT; ++jj)
      if (jj < CT) buf.q[kMaxCT + jj] = load_stream16(wb1 + jj * 1024);
    const uint8_t* sp0 = sbase + ((size_t)st0 * KG * 64 + lane) * 4;
    const uint8_t* sp1 = sbase + ((size_t)st1 * KG * 64 + lane) * 4;
    n0 = load_stream4(sp0 + (size_t)min(t0 / 4, KG - 1) * 256);
    n1 = load_stream4(sp0 + (size_t)min(t0 / 4 + 1, KG - 1) * 256);
    n2 = load_stream4(sp0 + (size_t)min(t0 / 4 + 2, KG - 1) * 256);
    n3 = load_stream4(sp1 + (size_t)min(t0 / 4, KG - 1) * 256);
    n4 = load_stream4(sp1 + (size_t)min(t0 / 4 + 1, KG - 1) * 256);
    n5 = load_stream4(sp1 + (size_t)min(t0 / 4 + 2, KG - 1) * 256);
  }
  return true;
}

// Phase-B unit u: selected expert dd, first row g0 of its 16-row group (the
// wide instance schedules each expert-group separately), 16-column strip i.
template <class DA>
__device__ __forceinline__ void b_unit(const DA& A, const SmemOf<DA>& sm, int u, int& dd, int& g0, int& i) {
  const int per = A.i() / 16, q = u / per;
  i = u % per;
  if constexpr (DA::kWide) {
    dd = sm.qd[q];
    g0 = kGroup * sm.qg[q];
  } else {
    dd = q;
    g0 = 0;
  }
}

// Routed phase-C unit ur (counted after the shared ones): selected expert dd,
// first row g0, 64-column group hg.  With the shared expert folded in (the
// list's last expert) its units come first.
template <class DA>
__device__ __forceinline__ void c_unit(const DA& A, const SmemOf<DA>& sm, const Seq& S, int ur, int& dd, int& g0,
                                       int& hg) {
  const int qc = ur / S.nhg;
  hg = ur % S.nhg;
  if constexpr (DA::kWide) {
    const int q = S.fold ? (qc + S.NQ - S.NQF) % S.NQ : qc;
    dd = sm.qd[q];
    g0 = kGroup * sm.qg[q];
  } else {
    dd = S.fold ? (qc == 0 ? S.D - 1 : qc - 1) : qc;
    g0 = 0;
  }
}

// Requests the weight tiles and scale words of sequence entry j into buf.
// The scale words are gathered in scalars and stored to buf once, on a single
// path: stores to different members on different paths get merged into one
// store through a pointer, which keeps buf in scratch memory.
template <class DA>
__device__ __forceinline__ void issue(const DA& A, const SmemOf<DA>& sm, const Seq& S, int j, int lane, int wave,
                                      Buf& buf) {
  if (j >= S.nb + S.nc) return;
  uint32_t n0 = 0, n1 = 0, n2 = 0, n3 = 0, n4 = 0, n5 = 0;
  if (j < S.nb) {
    int dd, g0, i;
    b_unit(A, sm, S.b0 + j, dd, g0, i);
    if (!issue_gu(A, sm.elist[dd], i, lane, wave, buf, n0, n1, n2, n3, n4, n5)) return;
  } else {
    // down units: both kinds load 1 KB weight blocks at a 1 KB stride (a
    // routed FP4 tile is one block, a shared FP8 tile two) and two scale words
    const int u = S.c0 + j - S.nb;
    const uint8_t *wb, *sp;
    int nq, KG;
    if (u >= S.ns) {
      int dd, g0, hg;
      c_unit(A, sm, S, u - S.ns, dd, g0, hg);
      const int e = sm.elist[dd], hs = 4 * hg + wave;
      KG = (A.kt2() + 3) / 4;
      nq = min(A.kt2(), kDownBatch);
      wb = A.w2 + (size_t)e * ((size_t)A.h() * A.i() / 2) + (size_t)hs * A.kt2() * 1024 + lane * 16;
      sp = A.w2s + (size_t)e * ((size_t)(A.h() / 16) * KG * 256) + ((size_t)hs * KG * 64 + lane) * 4;
    } else {
      const int hs = 4 * (u % S.nhg) + wave;
      KG = (A.kts() + 3) / 4;
      nq = 2 * min(A.kts(), kDownBatch / 2);
      wb = A.ws2 + (size_t)hs * A.kts() * 2048 + lane * 16;
      sp = A.ws2s + ((size_t)hs * KG * 64 + lane) * 4;
    }
#pragma unroll
    for (int jj = 0; jj < kDownBatch; ++jj)
      if (jj < nq) buf.q[jj] = load_stream16(wb + jj * 1024);
    n0 = load_stream4(sp);
    n1 = load_stream4(sp + (size_t)min(1, KG - 1) * 256);
  }
  buf.w0 = n0;
  buf.w1 = n1;
  buf.w2 = n2;
  buf.w3 = n3;
  buf.w4 = n4;
  buf.w5 = n5;
}

// Routed gate/up: MFMA chain of this wave's K-chunk for both strips into
// sm.red (A operand: the MXFP4 x rows of the routed slots, from LDS).
// Row m of the unit's A operand for its row group starting at g0 is x row
// tok (from the unit's slot list, or the row itself for the folded shared
// expert's units, which take every row).
template <class DA>
__device__ __forceinline__ void gu_compute(const DA& A, SmemOf<DA>& sm, const uint8_t* xq4_lds,
                                           const uint8_t* xs4_lds, int dd, int g0, const Buf& buf, int lane,
                                           int wave) {
  if (wave >= A.nc1()) return;
  const int m = lane & 15;
  int tok;
  if (dd >= 0) {
    const int n = min(sm.ecount[dd] - g0, kGroup);
    // rows past the group's slot count repeat its last token: their
    // products land in result rows that are never read
    tok = sm.slot(dd, g0 + (m < n ? m : n - 1)) / A.kk();
  } else {  // the folded expert's units: the group's rows of x, local in LDS
    const int ng = min(A.T - g0, kGroup);
    tok = m < ng ? m : ng - 1;
  }
  const int q = lane >> 4;
  const int CT = A.ct1(), t0 = wave * CT;
  v4i a[kMaxCT];
  uint32_t sa[kMaxCT];
#pragma unroll
  for (int jj = 0; jj < kMaxCT; ++jj) {
    if (jj < CT) {
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
        const uint32_t word = pick3(buf.w(3 * s), buf.w(3 * s + 1), buf.w(3 * s + 2), kt / 4 - t0 / 4);
        acc = mfma_fp4(a[jj], buf.q[kMaxCT * s + jj], acc, sa[jj], scale_byte(word, kt));
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.red[wave][s][4 * q + r][m] = acc[r];
  }
}

template <class DA>
__device__ __forceinline__ void unit_fold_gu(const DA& A, uint32_t tag, SmemOf<DA>& sm, const float* gamma_lds, int i,
                                             int g0, uint8_t* xq4, uint8_t* xs4, int& x4_group, int lane, int wave) {
  const int nb = A.h() / 32, ng = min(A.T - g0, kGroup), tasks = ng * nb;
  uint32_t bits[kQBatch][4];
  const bool quant = x4_group != g0;  // uniform: the group's rows are not in LDS yet
  if (quant) x_batch_load<false>(A, 0, tasks, nullptr, bits, g0 * nb);
  Buf buf;
  uint32_t n0 = 0, n1 = 0, n2 = 0, n3 = 0, n4 = 0, n5 = 0;
  issue_gu(A, A.e(), i, lane, wave, buf, n0, n1, n2, n3, n4, n5);
  buf.w0 = n0;
  buf.w1 = n1;
  buf.w2 = n2;
  buf.w3 = n3;
  buf.w4 = n4;
  buf.w5 = n5;
  if (quant) {
    __syncthreads();  // earlier readers of the LDS rows are done
    for (int b0 = 0; b0 < tasks; b0 += kQBatch * kQGroups) {
      if (b0 > 0) x_batch_load<false>(A, b0, tasks, nullptr, bits, g0 * nb);
      if (A.norm_w) x_batch_norm<false>(A, sm, gamma_lds, b0, tasks, nullptr, bits, g0 * nb);
      x_batch_quant<FP4, false>(A, b0, tasks, nullptr, bits, xq4, xs4);
    }
    x4_group = g0;
    trace_at(A, TR_XQ);
  }
  __syncthreads();  // the x rows are in LDS
  gu_compute(A, sm, xq4, xs4, -1, g0, buf, lane, wave);
  trace_at(A, TR_S_MMA);
  __syncthreads();
  int row, col;
  float a;
  if (gu_finish(sm, A.nc1(), ng, &row, &col, &a))
    st_dev(&A.a_r[(size_t)((g0 + row) * A.kk() + A.kr()) * A.i() + 16 * i + col], tagged(tag, a));
  __syncthreads();  // sm.red is rewritten by the next unit
}

// Staging of a down unit's intermediate rows into LDS as MX blocks: codes
// [n, K/2] (FP4) or [n, K] (FP8), scales [n, K/32].  Task t = (row m, block b)
// of n * K/32 is handled by the eight lanes 8(t mod 32) .. +8 of pass t / 128
// slot (t / 32) mod 4; each lane holds four consecutive values.
constexpr int kStagePass = 4 * (kThreads / 8);  // tasks per pass

template <class F>
__device__ __forceinline__ void stage_quantize(const float4 (&v)[4], int t0, int tasks, int K, uint8_t* codes,
                                               uint8_t* scales) {
  const int nb = K / 32, j = threadIdx.x & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int task = t0 + p * (kThreads / 8) + (int)threadIdx.x / 8;
    if (t0 + p * (kThreads / 8) >= tasks) break;  // uniform: whole slot beyond the end
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

// Routed intermediate: the tagged SwiGLU values of slots[0..n) (row stride
// K), polled pass by pass until every word of the pass carries this call's
// tag, then quantized to MXFP4.
template <class DA>
__device__ __forceinline__ void stage_routed(const DA& A, uint32_t tag, int K, int n, const uint16_t* slots,
                                             uint8_t* codes, uint8_t* scales) {
  const int nb = K / 32, tasks = n * nb, j = threadIdx.x & 7;
  const uint64_t tw = wall_clock64();
  for (int t0 = 0; t0 < tasks; t0 += kStagePass) {
    float4 v[4];
    bool ok;
    do {
      ok = true;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int task = t0 + p * (kThreads / 8) + (int)threadIdx.x / 8;
        v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (task < tasks) {
          const uint64_t* src = A.a_r + (size_t)slots[task / nb] * K + 32 * (task % nb) + 4 * j;
          const uint64_t w0 = ld_dev(src), w1 = ld_dev(src + 1), w2 = ld_dev(src + 2), w3 = ld_dev(src + 3);
          ok &= tag_ok(w0, tag);
          ok &= tag_ok(w1, tag);
          ok &= tag_ok(w2, tag);
          ok &= tag_ok(w3, tag);
          v[p] = make_float4(__uint_as_float((uint32_t)w0), __uint_as_float((uint32_t)w1),
                             __uint_as_float((uint32_t)w2), __uint_as_float((uint32_t)w3));
        }
      }
    } while (keep_polling(ok, tw, A.sync));
    stage_quantize<FP4>(v, t0, tasks, K, codes, scales);
  }
}

// Shared intermediate: SwiGLU of the tagged gate and up sums of a_s (row
// stride 2K: gate columns, then up columns), polled pass by pass until every
// word of the pass carries this call's tag, then quantized to MXFP8.
template <class DA>
__device__ __forceinline__ void stage_shared(const DA& A, uint32_t tag, int K, int g0, int n, uint8_t* codes,
                                             uint8_t* scales) {
  const int nb = K / 32, tasks = n * nb, j = threadIdx.x & 7;
  const uint64_t tw = wall_clock64();
  for (int t0 = 0; t0 < tasks; t0 += kStagePass) {
    float g[4][4], u[4][4];
    bool ok;
    do {
      ok = true;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int task = t0 + p * (kThreads / 8) + (int)threadIdx.x / 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) g[p][i] = u[p][i] = 0.f;
        if (task < tasks) {
          const uint64_t* src = A.a_s + (size_t)(g0 + task / nb) * (2 * K) + 32 * (task % nb) + 4 * j;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint64_t wg = ld_dev(src + i), wu = ld_dev(src + K + i);
            ok &= tag_ok(wg, tag);
            ok &= tag_ok(wu, tag);
            g[p][i] = __uint_as_float((uint32_t)wg);
            u[p][i] = __uint_as_float((uint32_t)wu);
          }
        }
      }
    } while (keep_polling(ok, tw, A.sync));
    float4 v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      v[p] = make_float4(silu_mul(g[p][0], u[p][0]), silu_mul(g[p][1], u[p][1]), silu_mul(g[p][2], u[p][2]),
                         silu_mul(g[p][3], u[p][3]));
    stage_quantize<FP8>(v, t0, tasks, K, codes, scales);
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
        buf.w(g) = load_stream4(ws_scale + (size_t)min(b0 / 4 + g, KG - 1) * 256);
    }
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int kt = b0 + jj;
      if (kt < KT) {
        // rows past n repeat row n - 1: their products land in result rows
        // that are never stored
        const int mr = m < n ? m : n - 1;
        const uint8_t* ap = codes + (size_t)mr * (F::MB == 1 ? K / 2 : K) + kt * 64 * R + 16 * q;
        const v4i a0 = *reinterpret_cast<const v4i*>(ap);
        v4i a1 = a0;
        if constexpr (R == 2) a1 = *reinterpret_cast<const v4i*>(ap + 64);
        const uint32_t sa = scales[mr * (K / 32) + 4 * kt + q];
        const uint32_t sb = scale_byte(buf.w(jj / 4), kt);
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
// y = bf16( sum_j w_j d_j (j in order) + s + residual ).  If any wait of the
// call has given up by then (the status word, read with the last polls), the
// group's output is NaN instead.
template <class DA>
__device__ __forceinline__ void combine(const DA& A, uint32_t tag, const SmemOf<DA>& sm, int hg, int g0) {
  const int H = A.h(), k = A.kk(), T = min(A.T, g0 + kGroup);  // rows g0 .. T - 1
  constexpr int kPer = kGroup * 64 / kThreads;  // (row, column) pairs per thread
  float d[kPer][kMaxK], s[kPer];
  const uint64_t t0 = wall_clock64();
  bool ok;
  uint32_t status;
  do {
    ok = true;
    status = ld_dev(ctr(A.sync, S_STATUS));  // read with the polls: no extra round trip
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = 64 * g0 + threadIdx.x + p * kThreads;
      if (idx < T * 64) {
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
    const int idx = 64 * g0 + threadIdx.x + p * kThreads;
    if (idx < T * 64) {
      const int t = idx >> 6, h = 64 * hg + (idx & 63);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) acc = fmaf(sm.w[t * k + j], d[p][j], acc);
      if (A.is()) acc = acc + s[p];
      if (A.residual) acc = acc + bf16_to_f32(A.residual[(size_t)t * H + h]);
      // a wait of this call that gave up (status set) leaves NaN, not stale data
      A.y[(size_t)t * H + h] = (ok && status == 0u) ? f32_to_bf16(acc) : kBf16NaN;
    }
  }
}

// One sequence entry: compute from buf, request entry j + kBufs into buf,
// store the results.  An entry covers at most 16 rows: the wide instance
// schedules each 16-row group of an expert as a unit of its own.
template <class DA>
__device__ __forceinline__ void run_entry(const DA& A, uint32_t tag, SmemOf<DA>& sm, const Seq& S, int j, Buf& buf,
                                          uint8_t* xq4_lds, uint8_t* xs4_lds, uint8_t* stage, int lane, int wave) {
  if (j < S.nb) {
    int dd, g0, i;
    b_unit(A, sm, S.b0 + j, dd, g0, i);
    gu_compute(A, sm, xq4_lds, xs4_lds, dd, g0, buf, lane, wave);
    if (j == 0) trace_at(A, TR_B_MMA);
    issue(A, sm, S, j + kBufs, lane, wave, buf);  // buf is free once the matrix products have read it
    __syncthreads();
    int row, col;
    float a;
    if (gu_finish(sm, A.nc1(), min(sm.ecount[dd] - g0, kGroup), &row, &col, &a))
      st_dev(&A.a_r[(size_t)sm.slot(dd, g0 + row) * A.i() + 16 * i + col], tagged(tag, a));
    if (j == 0) trace_at(A, TR_B_STORED);
    __syncthreads();  // sm.red is rewritten by the next unit
    if (j == 0) trace_at(A, TR_B_RELEASED);
    return;
  }
  const int u = S.c0 + j - S.nb;  // shared down units first, then routed
  const int m = lane & 15, q = lane >> 4;
  // The staged intermediate is the previous entry's when that entry was a
  // down unit of the same kind and (expert-)group.  Every thread derives this
  // from the sequence itself, so the whole workgroup takes the same branch.
  const int pu = u - 1;
  v4f out;
  if (u >= S.ns) {
    int dd, g0, hg;
    c_unit(A, sm, S, u - S.ns, dd, g0, hg);
    const bool staged = j > S.nb && pu >= S.ns && (pu - S.ns) / S.nhg == (u - S.ns) / S.nhg;
    const int hs = 4 * hg + wave;
    const int e = sm.elist[dd], n = min(sm.ecount[dd] - g0, kGroup);
    const int K = A.i();
    uint8_t* codes = stage;
    uint8_t* scales = stage + kGroup * (K / 2);
    if (!staged) {
      stage_routed(A, tag, K, n, &sm.slist[sm.eoff[dd] + g0], codes, scales);
      __syncthreads();
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
        st_dev(&A.d_part[(size_t)sm.slot(dd, g0 + 4 * q + r) * A.h() + 16 * hs + m], tagged(tag, out[r]));
  } else {
    const int g0 = kGroup * (u / S.nhg), hs = 4 * (u % S.nhg) + wave, n = min(A.T - g0, kGroup);
    const bool staged = j > S.nb && pu / S.nhg == u / S.nhg;
    const int K = A.is();
    uint8_t* codes = stage;
    uint8_t* scales = stage + kGroup * K;
    if (!staged) {
      stage_shared(A, tag, K, g0, n, codes, scales);
      __syncthreads();
    }
    const int KG = (A.kts() + 3) / 4;
    const uint8_t* w = A.ws2 + (size_t)hs * A.kts() * 2048 + lane * 16;
    const uint8_t* sw = A.ws2s + ((size_t)hs * KG * 64 + lane) * 4;
    out = down_compute<FP8>(w, sw, A.kts(), A.cts(), codes, scales, n, buf, lane);
    issue(A, sm, S, j + kBufs, lane, wave, buf);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q + r < n) st_dev(&A.s_part[(size_t)(g0 + 4 * q + r) * A.h() + 16 * hs + m], tagged(tag, out[r]));
  }
}

// ------------------------------------------------------------------ kernel
// The layer itself: phases A, B, C and the combines of this workgroup.
template <class DA>
__device__ __forceinline__ void decode_body(const DA& A, uint32_t tag, SmemOf<DA>& sm, unsigned char* dyn, uint64_t* tr,
                                            int lane, int wave) {
  const int G = A.G, T = A.T, E = A.e();

  // dynamic LDS (offsets from the host, see lds_layout): the logits; the
  // MXFP4 x; the MXFP8 x of a shared strip (phase A) or the staged down-unit
  // intermediate (phase C); the norm weight.  The wide instance overlays the
  // staged intermediate on the logits and the MXFP8 x on the MXFP4 x.
  float* logits_lds = reinterpret_cast<float*>(dyn);
  uint8_t* xq4_lds = dyn + A.off_xq4;
  uint8_t* xs4_lds = xq4_lds + (size_t)T * (A.h() / 2);
  uint8_t* stage = dyn + A.off_stage;
  uint8_t* x8_lds = dyn + A.off_x8;
  float* gamma_lds = reinterpret_cast<float*>(dyn + A.gamma_off);  // the norm weight (with the norm)

  // phase A: router units, then shared gate/up strips, strided over the grid.
  // With few rows a strip leaves the MXFP4 copy of x in LDS and the other
  // workgroups make it after their units.
  // the pre-router norm's factor of every row, in every workgroup (the same
  // arithmetic everywhere, so all agree)
  // pre-router norm: a router unit leaves the norm factors of all rows in
  // sm.rnorm (have_r); norm_setup stages the weight (and the factors if
  // missing) before the workgroup's first x quantization (have_norm)
  bool have_r = false, have_norm = false;

  // units after the router's: MXFP8 shared gate/up strips, or the folded
  // shared expert's gate/up units (all rows select it)
  // (one unit per strip and 16-row group of x)
  const int n_base = A.is() ? 2 * A.is() / 16 : (A.fd() ? A.i() / 16 : 0);
  const int n_ss = n_base * (DA::kWide ? (T + kGroup - 1) / kGroup : 1);
  const bool early_x4 = T <= kEarlyQuantT;
  bool have_x4 = false;      // the MXFP4 copy of x in LDS holds the rows the units need
  bool have_all_x4 = false;  // ... and it holds every row, at its own position
  int x4_group = -1;         // the 16-row group a folded expert's unit left in LDS
  for (int u = blockIdx.x; u < E + n_ss; u += G) {
    if (u < E) {
      unit_router(A, sm, tag, u, lane, wave);
      have_r = true;
    } else {
      if (A.norm_w && !have_norm) {
        __syncthreads();  // the router unit's factors are in sm.rnorm
        norm_setup(A, sm, gamma_lds, !have_r, lane, wave);
        have_norm = have_r = true;
      }
      const int v = u - E, g0 = kGroup * (v / n_base);
      if (A.fd()) {
        unit_fold_gu(A, tag, sm, gamma_lds, v % n_base, g0, xq4_lds, xs4_lds, x4_group, lane, wave);
        have_x4 = have_all_x4 = !DA::kWide;  // up to 16 rows: every row, at its own position
      } else {
        unit_shared_strip(A, tag, sm, gamma_lds, v % n_base, g0, x8_lds, xq4_lds, xs4_lds, lane, wave);
        have_x4 = early_x4;
      }
    }
    if (threadIdx.x == 0 && u == (int)blockIdx.x) tr[TR_FIRST] = wall_clock64();
  }
  if (A.norm_w && !have_norm) {  // workgroups with router units only, or with no phase-A unit
    __syncthreads();
    norm_setup(A, sm, gamma_lds, !have_r, lane, wave);
    have_norm = have_r = true;
  }
  if (early_x4 && !have_x4) {
    const int tasks = T * (A.h() / 32);
    for (int t0 = 0; t0 < tasks; t0 += kQBatch * kQGroups) {
      uint32_t bits[kQBatch][4];
      x_batch_load<false>(A, t0, tasks, nullptr, bits);
      if (A.norm_w) x_batch_norm<false>(A, sm, gamma_lds, t0, tasks, nullptr, bits);
      x_batch_quant<FP4, false>(A, t0, tasks, nullptr, bits, xq4_lds, xs4_lds);
    }
    trace_at(A, TR_XQ);
  }
  trace_at(A, TR_A);
  compiler_fence();

  // routing, identical in every workgroup: read the tagged logits until all
  // are this call's
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
  // the k routed choices of row t go to slots t*kk .. t*kk + k - 1
  if (T <= kWaves) {  // a wavefront per row
    const int row = wave < T ? wave : 0;
    row_topk64(logits_lds + row * E, wave < T, E, A.kr(), lane, sm.ids + row * A.kk(), sm.w + row * A.kk());
  } else {  // 16 lanes per row, 16 rows per pass
    for (int r0 = 0; r0 < (DA::kWide ? T : 1); r0 += kThreads / 16) {
      const int row = r0 + (int)threadIdx.x / 16;
      rows_topk16(logits_lds + (row < T ? row : 0) * E, row < T, E, A.kr(), threadIdx.x & 15,
                  sm.ids + (row < T ? row : 0) * A.kk(), sm.w + (row < T ? row : 0) * A.kk());
    }
  }
  if (A.fd() && threadIdx.x >= kThreads - kGroup) {  // the folded shared expert: last slot of each row
    for (int t = threadIdx.x - (kThreads - kGroup); t < T; t += kGroup) {
      sm.ids[t * A.kk() + A.kr()] = E;
      sm.w[t * A.kk() + A.kr()] = 1.0f;
    }
  }
  __syncthreads();
  trace_at(A, TR_TOPK);
  build_expert_list(A, sm, lane, wave);
  trace_at(A, TR_ELIST);
  if (blockIdx.x == 0) {  // the routing outputs: the k routed choices per row
    for (int i = threadIdx.x; i < T * A.kr(); i += kThreads) {
      const int sl = (i / A.kr()) * A.kk() + i % A.kr();
      if (A.ids_out) A.ids_out[i] = sm.ids[sl];
      if (A.w_out) A.w_out[i] = sm.w[sl];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) tr[TR_ROUTED] = wall_clock64();

  // phases B and C: contiguous runs of units per workgroup, one pipeline
  Seq S;
  S.D = sm.D;
  S.nhg = A.h() / 64;
  S.ns = A.is() ? S.nhg : 0;
  S.fold = A.fd();
  int NQB = S.D - S.fold, NQC = S.D;  // expert(-group)s of phases B and C
  if constexpr (DA::kWide) {
    S.NQ = sm.NQ;
    S.NQF = sm.NQF;
    NQB = S.NQ - S.NQF;
    NQC = S.NQ;
    S.ns = A.is() ? S.nhg * ((T + kGroup - 1) / kGroup) : 0;
  }
  {
    const int NB = NQB * (A.i() / 16);  // the folded expert's gate/up ran in phase A
    const int NCU = S.ns + NQC * S.nhg;
    // 32-bit products: decode_supported keeps the phase-B unit count and the
    // phase-C cost below 2^19 and the grid is at most kDecodeMaxGrid (2^11),
    // so with parts of at most 3 every cut position below stays under 2^32.
    const unsigned b = blockIdx.x, g = (unsigned)G;
    // With the pre-router norm and more than kEarlyQuantT rows, the
    // workgroups that ran a shared strip or a folded gate/up unit after the
    // router units (they form the norm factors of every row and quantize
    // every row first) reach routing long after the router workgroups, so
    // they take kNormLate parts of the phase-B and phase-C work to the
    // others' kNormEarly; otherwise every workgroup takes one part.
    const bool weigh = !DA::kWide && A.norm_w && T > kEarlyQuantT;
    const unsigned we = weigh ? kNormEarly : 1u, wl = weigh ? kNormLate : 1u;
    const unsigned l0 = (unsigned)min(E, G), l1 = (unsigned)min(E + n_ss, G);  // the late ones: [l0, l1)
    auto wsum = [&](unsigned x) -> unsigned {  // weight of workgroups 0 .. x - 1
      const unsigned late = min(x, l1) > l0 ? min(x, l1) - l0 : 0u;
      return we * x - (we - wl) * late;
    };
    const unsigned wt = wsum(g), w0 = wsum(b), w1 = wsum(b + 1);
    S.b0 = (int)((unsigned)NB * w0 / wt);
    S.nb = (int)((unsigned)NB * w1 / wt) - S.b0;
    if (T > 1) {
      // Above one row phase C is cut by cost: a shared down unit (MXFP8)
      // moves twice the weight bytes of a routed (MXFP4) one and counts
      // twice.  (At one row there are fewer units than workgroups, and a cut
      // by cost would give some workgroups two routed units.)  Shared unit
      // u < ns covers cost positions [2u, 2u + 2), routed unit u >= ns covers
      // [ns + u, ns + u + 1); workgroup b takes the units whose range starts
      // in [ct w0 / wt, ct w1 / wt), so every unit has one owner and each run
      // stays contiguous.
      const unsigned ns = (unsigned)S.ns, ct = 2u * ns + ((unsigned)NCU - ns);
      auto first_at = [&](unsigned p) -> int { return (int)(p <= 2u * ns ? (p + 1u) / 2u : p - ns); };
      S.c0 = first_at(ct * w0 / wt);
      S.nc = first_at(ct * w1 / wt) - S.c0;
    } else {
      S.c0 = (int)((unsigned)NCU * w0 / wt);
      S.nc = (int)((unsigned)NCU * w1 / wt) - S.c0;
    }
  }
  const int total = S.nb + S.nc;

  // With more than kEarlyQuantT rows: the MXFP4 copy of the x rows this
  // workgroup's gate/up units read (the tokens routed to the experts of its
  // run of phase-B units), listed in ascending order in sm.qrows.  It is made
  // before the pipeline's weight tiles are requested: a wait for x issued
  // after them would also wait for every tile in flight.
  uint64_t need = 0;
  if (!early_x4 && !have_all_x4 && S.nb > 0) {
    const int per = A.i() / 16;
    for (int u = S.b0 - S.b0 % per; u < S.b0 + S.nb; u += per) {  // each expert(-group) of the run
      int dd, g0, i;
      b_unit(A, sm, u, dd, g0, i);
      for (int s = g0; s < min(sm.ecount[dd], g0 + kGroup); ++s) need |= 1ull << (sm.slot(dd, s) / A.kk());
    }
  }
  if (need) {  // uniform
    if (threadIdx.x < DA::kMaxT && ((need >> threadIdx.x) & 1ull))
      sm.qrows[__popcll(need & ((1ull << threadIdx.x) - 1ull))] = (uint8_t)threadIdx.x;
    __syncthreads();
    const int q_tasks = __popcll(need) * (A.h() / 32);
    for (int t0 = 0; t0 < q_tasks; t0 += kQBatch * kQGroups) {
      uint32_t bits[kQBatch][4];
      x_batch_load<true>(A, t0, q_tasks, sm.qrows, bits);
      if (A.norm_w) x_batch_norm<true>(A, sm, gamma_lds, t0, q_tasks, sm.qrows, bits);
      x_batch_quant<FP4, true>(A, t0, q_tasks, sm.qrows, bits, xq4_lds, xs4_lds);
    }
    trace_at(A, TR_XQ);
    __syncthreads();  // the x rows are in LDS before any gate/up unit reads them
  }

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
  for (int hg = blockIdx.x; hg < S.nhg; hg += G)
    for (int g0 = 0; g0 < (DA::kWide ? T : 1); g0 += kGroup) combine(A, tag, sm, hg, g0);
}

// A call on a workspace whose status word is set (an earlier call gave up a
// wait, so its tagged words cannot be trusted) computes nothing: its output
// is the bf16 NaN pattern, until the workspace is zero-filled again.
template <class DA>
__device__ __forceinline__ void poison_output(const DA& A) {
  const int nhg = A.h() / 64;
  for (int hg = blockIdx.x; hg < nhg; hg += A.G)
    for (int idx = threadIdx.x; idx < A.T * 64; idx += kThreads)
      A.y[(size_t)(idx >> 6) * A.h() + 64 * hg + (idx & 63)] = kBf16NaN;
}

template <class DA>
__global__ void __launch_bounds__(kThreads) fused_decode_kernel(DA A) {
  const uint64_t t_entry = wall_clock64();
  __shared__ SmemOf<DA> sm;
  extern __shared__ __align__(16) unsigned char dyn[];
  // the wavefront index as a uniform value: everything derived from it stays
  // in scalar registers, which leaves the vector registers to the pipeline
  // buffers (fewer of them move through AGPRs)
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int G = A.G;
  const uint32_t tag = ld_dev(ctr(A.sync, S_EPOCH)) + 1u;
  const uint32_t status = ld_dev(ctr(A.sync, S_STATUS));
  uint64_t* tr = A.trace + (size_t)blockIdx.x * kTraceWords;
  if (threadIdx.x == 0) {
    tr[TR_START] = t_entry;
    for (int i = 1; i < kTraceWords - 1; ++i) tr[i] = 0;
    wait_vm<0>();
    tr[TR_TAG] = wall_clock64() + (tag == 0u ? 1u : 0u);
  }
  if (status == 0u)
    decode_body(A, tag, sm, dyn, tr, lane, wave);
  else
    poison_output(A);

  // exit: the last workgroup to finish advances the epoch (the next call's
  // tag is one more) and resets the arrival counter.  Tags are unique per
  // call, so neither needs this call's stores to have landed first: the next
  // call starts only after they all have.  The call whose tag is the last
  // 32-bit value (once in 2^32 calls) is the exception, below.
  const bool wrap = tag == 0xffffffffu;  // uniform
  __syncthreads();
  if (threadIdx.x == 0) {
    tr[TR_C] = wall_clock64();
    if (blockIdx.x == 0) st_dev(ctr(A.sync, S_GRID), (uint32_t)G);
    compiler_fence();
    if (wrap) wait_vm<0>();
    const uint32_t old = __hip_atomic_fetch_add(ctr(A.sync, S_DONE), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    compiler_fence();
    const bool last = old + 1 == (uint32_t)G;
    if (last && !wrap) {
      st_dev(ctr(A.sync, S_EPOCH), tag);
      st_dev(ctr(A.sync, S_DONE), 0u);
    }
    sm.last = last;
  }
  if (!wrap) return;  // uniform
  __syncthreads();
  if (sm.last) {  // uniform
    // After 2^32 - 1 calls the tag would wrap to 0, the tag of zero-filled
    // words, and later tags would match words written 2^32 calls earlier.
    // Instead every tagged word is cleared, once every workgroup's stores
    // have landed (each waited for its own before counting itself in), and
    // the epoch restarts at 0.
    for (uint32_t i = threadIdx.x; i < A.n_tagged; i += kThreads) st_dev(&A.tagged[i], (uint64_t)0);
    compiler_fence();
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      st_dev(ctr(A.sync, S_EPOCH), 0u);
      compiler_fence();
      wait_vm<0>();
      st_dev(ctr(A.sync, S_DONE), 0u);
    }
  }
}

// ------------------------------------------------------------------ host side
struct Carve {
  size_t sync, sync_end;
  size_t trace, logits, a_r, a_s, d_part, s_part, total;
};

// Workspace of an instance taking up to MT rows: the sync block, the trace
// words (offsets independent of MT), then the tagged words.
Carve carve(const moe_layer_t& L, int MT) {
  const size_t T = MT, H = L.hidden, I = L.inter, E = L.num_experts, k = layer_slots(L), Is = L.shared_inter;
  Carve c{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  const size_t line = kLine * 4;
  c.sync = take(kSyncLines * line);
  c.sync_end = o;
  c.trace = take((size_t)kDecodeMaxGrid * kTraceWords * 8);
  c.logits = take(T * E * 8);
  c.a_r = take(T * k * I * 8);
  c.a_s = take(T * 2 * Is * 8 + 16);
  c.d_part = take(T * k * H * 8);
  c.s_part = take(T * H * 8);
  c.total = o;
  return c;
}

// Dynamic LDS of an instance taking up to MT rows.  Up to 16 rows: logits,
// the MXFP4 x, then either the MXFP8 x of a shared strip (phase A) or a
// staged down-unit intermediate (phase C), then the norm weight.  Wide
// instance: the staged intermediate over the logits (dead after routing) and
// the MXFP8 x over the MXFP4 x (a strip's copy is dead before the copy for
// phase B is made); the norm weight is read from memory.
struct LdsLayout {
  size_t xq4, stage, x8, gamma, total;
};

LdsLayout lds_layout(const moe_layer_t& L, int MT) {
  const size_t H = L.hidden, I = L.inter, E = L.num_experts, Is = L.shared_inter;
  const size_t logits = align_up((size_t)MT * E * 4, 16);
  const size_t xq = align_up((size_t)MT * (H / 2 + H / 32), 16);
  const size_t st4 = (size_t)kGroup * (I / 2 + I / 32), st8 = (size_t)kGroup * (Is + Is / 32);
  const size_t st = align_up(st4 > st8 ? st4 : st8, 16);
  const size_t x8 = Is ? align_up((size_t)kGroup * (H + H / 32), 16) : 0;
  LdsLayout o{};
  if (MT <= kGroup) {
    o.xq4 = logits;
    o.stage = o.x8 = logits + xq;
    o.gamma = o.stage + (st > x8 ? st : x8);
    o.total = o.gamma + (L.norm_weight ? H * 4 : 0);
  } else {
    o.stage = 0;
    o.xq4 = o.x8 = logits > st ? logits : st;
    o.gamma = 0;
    o.total = o.xq4 + (xq > x8 ? xq : x8);
  }
  return o;
}

int max_rows_for(int T) { return T <= kDecodeMaxT ? kDecodeMaxT : kDecodeWideMaxT; }

// Grid of the persistent launch: as many workgroups as the device keeps
// resident at once (one per CU), since every workgroup must run concurrently.
// Kept per device in a lock-free table of (dynamic LDS bytes << 32 | grid);
// two threads that race on a device's first call compute the same entry.
template <class DA>
int grid_size(size_t lds) {
  static std::atomic<uint64_t> cache[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return 0;
  const uint64_t c = cache[dev].load(std::memory_order_relaxed);
  if (c != 0 && (c >> 32) == lds) return (int)(uint32_t)c;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (lds + sizeof(SmemOf<DA>) > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fused_decode_kernel<DA>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_decode_kernel<DA>, kThreads, lds) != hipSuccess)
    return 0;
  int grid = (occ > 1 ? 1 : occ) * cus;
  if (grid > kDecodeMaxGrid) grid = kDecodeMaxGrid;
  if (grid > 0) cache[dev].store(((uint64_t)lds << 32) | (uint32_t)grid, std::memory_order_relaxed);
  return grid;
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
using MiniMaxShape = DArgs<3072, 1024, 1024, 128, 4, 0, kDecodeMaxT>;
using MiniMaxFolded = DArgs<3072, 1024, -1, 128, 4, 1, kDecodeMaxT>;  // shared expert folded in as expert 128
using AnyShape = DArgs<0, 0, 0, 0, 0, -1, kDecodeMaxT>;
// wide steps (17..64 rows)
using MiniMaxShapeW = DArgs<3072, 1024, 1024, 128, 4, 0, kDecodeWideMaxT>;
using MiniMaxFoldedW = DArgs<3072, 1024, -1, 128, 4, 1, kDecodeWideMaxT>;
using AnyShapeW = DArgs<0, 0, 0, 0, 0, -1, kDecodeWideMaxT>;

int n_chunks(int tiles) { return tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1); }

}  // namespace

size_t decode_ws_bytes(const moe_layer_t& L, int T) { return carve(L, max_rows_for(T)).total; }
size_t decode_sync_bytes(const moe_layer_t& L) { return carve(L, kDecodeMaxT).sync_end; }
size_t decode_trace_offset(const moe_layer_t& L) { return carve(L, kDecodeMaxT).trace; }

bool decode_supported(const moe_layer_t& L, int T) {
  if (T < 1 || T > kDecodeWideMaxT) return false;
  // a K-chunk of the gate/up (K = H) must fit the register buffers, the LDS a workgroup
  const int KT1 = L.hidden / 128;
  const size_t smem = T <= kDecodeMaxT ? sizeof(SmemT<kDecodeMaxT>) : sizeof(SmemT<kDecodeWideMaxT>);
  // the kernel cuts the unit sequences with 32-bit products (unit count or
  // cost times a cumulative weight of at most 3 * kDecodeMaxGrid)
  const size_t groups = (size_t)max_rows_for(T) / 16, nq = ((size_t)L.num_experts + 1) * groups;
  const size_t nhg = (size_t)L.hidden / 64, nb_units = nq * (L.inter / 16);
  const size_t c_cost = 2 * nhg * groups + nq * nhg;
  if (nb_units >= (1u << 19) || c_cost >= (1u << 19)) return false;
  static_assert(3ull * kDecodeMaxGrid * (1u << 19) <= 0xffffffffull, "32-bit unit cut");
  return KT1 / n_chunks(KT1) <= kMaxCT && lds_layout(L, max_rows_for(T)).total + smem <= 160 * 1024;
}

hipError_t launch_decode(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                         uint16_t* y, void* ws, int32_t* ids_out, float* w_out, hipStream_t stream) {
  const int MT = max_rows_for(T);
  const Carve c = carve(L, MT);
  const LdsLayout lay = lds_layout(L, MT);
  const size_t lds = lay.total;
  char* base = reinterpret_cast<char*>(ws);
  DecodeArgs A{};
  A.T = T;
  A.H = L.hidden;
  A.I = L.inter;
  A.E = L.num_experts;
  A.k = L.top_k;
  A.fold = L.shared_folded ? 1 : 0;
  A.norm_w = L.norm_weight;
  A.norm_eps = L.norm_eps;
  A.gamma_off = (int)lay.gamma;
  A.off_xq4 = (int)lay.xq4;
  A.off_stage = (int)lay.stage;
  A.off_x8 = (int)lay.x8;
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
  A.residual = L.norm_weight ? x : residual;  // with the norm: its own input is the residual
  A.y = y;
  A.ids_out = ids_out;
  A.w_out = w_out;
  A.sync = reinterpret_cast<uint32_t*>(base + c.sync);
  A.logits = reinterpret_cast<uint64_t*>(base + c.logits);
  A.a_r = reinterpret_cast<uint64_t*>(base + c.a_r);
  A.a_s = reinterpret_cast<uint64_t*>(base + c.a_s);

  A.d_part = reinterpret_cast<uint64_t*>(base + c.d_part);
  A.s_part = reinterpret_cast<uint64_t*>(base + c.s_part);
  A.trace = reinterpret_cast<uint64_t*>(base + c.trace);
  A.tagged = A.logits;
  A.n_tagged = (uint32_t)((c.total - c.logits) / 8);
  const bool minimax = A.H == 3072 && A.I == 1024 && A.E == 128 && A.k == 4;
  if (MT > kDecodeMaxT) {
    if (minimax && A.Is == 1024 && !A.fold) return launch_instance<MiniMaxShapeW>(A, lds, stream);
    if (minimax && A.Is == 0 && A.fold) return launch_instance<MiniMaxFoldedW>(A, lds, stream);
    return launch_instance<AnyShapeW>(A, lds, stream);
  }
  if (minimax && A.Is == 1024 && !A.fold) return launch_instance<MiniMaxShape>(A, lds, stream);
  if (minimax && A.Is == 0 && A.fold) return launch_instance<MiniMaxFolded>(A, lds, stream);
  return launch_instance<AnyShape>(A, lds, stream);
}

// ------------------------------------------------------------------ no-allocation variant
// The workspace of fused_moe_mxfp4_decode_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol): each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;                       // guards the first call on each device
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // this device's copy of `scratch`, once set up
}  // namespace

void* noalloc_scratch(hipStream_t stream) {
  const int dev = current_device();
  if (dev < 0) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  // The decode protocol needs zero-filled words before its first call; the
  // fill is a kernel on the caller's stream, ordered before that call.
  if (launch_fill_u32(ptr, kNoAllocScratchBytes / 4, 0u, stream) != hipSuccess) return nullptr;
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace mxmoe
