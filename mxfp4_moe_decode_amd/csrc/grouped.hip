// The MoE layer for any number of rows as a short sequence of launches on one
// stream (the path the article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support
// and optimization" takes beyond the fused decode sizes, section "Serving with
// vLLM / What we Optimized"):
//
//   1. router logits and top-k per row;
//   2. align-sort of the T*k (row, choice) slots by expert, each expert's
//      segment padded to kBM rows;
//   3. MXFP4 (and, with a shared expert, MXFP8) quantization of x;
//   4. routed gate/up: one grouped scaled-FP4 GEMM over the kBM-row blocks,
//      epilogue SwiGLU and MXFP4 re-quantization of the intermediate;
//   5. shared gate/up: dense scaled-FP8 GEMM, epilogue SwiGLU and MXFP8
//      re-quantization;
//   6. routed down: grouped scaled-FP4 GEMM, fp32 result per slot;
//   7. shared down: dense scaled-FP8 GEMM whose epilogue is the combine
//      (without a shared expert a separate combine kernel runs instead).
//
// Arithmetic is that of the fused decode kernel, step for step: the same
// 16x16x128 scaled matrix instructions in K-chunks of CT tiles whose sums are
// added in chunk order, the same SwiGLU / re-quantization and the same combine
// order.  For the same rows and routing both paths give identical bits.
//
// GEMM tiling.  A workgroup of four wavefronts (2 x 2) owns a tile of rows x
// columns; each wavefront holds MF row fragments of 16 and four column strips
// of 16 (gate/up: two gate strips and the two matching up strips of one
// 32-column intermediate block, so SwiGLU and the block re-quantization stay
// inside the wavefront).  Weight tiles stream from the tiled MX layout straight
// into the matrix-instruction operands; activation rows are read in place
// (gathered through the sorted slots for the routed gate/up).  Operands of the
// next K-tile are loaded while the current one is multiplied.  Workgroups are
// numbered so that each XCD receives a contiguous run of tiles: the tiles of
// one expert's blocks then share that XCD's L2.
#include <atomic>
#include <type_traits>

#include <mutex>

#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;  // rows of a routed block (the align-sort block size)

enum Mode { GU_ROUTED = 0, GU_SHARED = 1, DOWN_ROUTED = 2, DOWN_SHARED = 3 };

struct GemmArgs {
  int T, k, H;
  int MB, NT;               // row blocks and column tiles of the launch
  int KT, CT, KG;           // K-tiles of 128, tiles per chunk, scale groups of 4 tiles
  const uint8_t* a;         // activation codes, row-major
  const uint8_t* as;        // activation scales, row-major [rows, K/32]
  size_t a_stride, as_stride;
  const uint8_t* b;         // weight codes, tiled layout
  const uint8_t* bs;        // weight scales, tiled layout
  size_t b_estride, bs_estride;  // per expert
  const int32_t* sorted_slots;
  const int32_t* block_expert;
  const int32_t* num_padded;
  int inter;                // gate/up: intermediate size
  uint8_t* oc;              // gate/up: intermediate codes
  uint8_t* os;              // gate/up: intermediate scales
  float* d_part;            // routed down output [T*k, H]
  const float* topk_w;      // shared down: routing weights [T, k]
  const uint16_t* residual; // shared down: optional residual [T, H]
  uint16_t* y;              // shared down: output [T, H]
};

// Workgroup tile geometry per format.  A 16x128 operand tile is one 1 KiB
// block (FP4) or two (FP8, R = 2 halves); lane l's 16 bytes of a block are the
// bytes that lane feeds the matrix instruction.
// Wavefronts form a 2 x WN grid; each holds MF row fragments of 16 and four
// column strips of 16.
template <class F, int WN>
struct Geo {
  static constexpr int R = F::MB == 1 ? 1 : 2;
  static constexpr int MF = F::MB == 1 ? 4 : 2;  // row fragments per wavefront
  static constexpr int WAVES = 2 * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 2 * 16 * MF;         // rows per workgroup
  static constexpr int STRIPS = 4 * WN;          // 16-column weight strips per workgroup
  static constexpr int A_TILES = (BM / 16) * R;  // 1 KiB blocks of A per K-tile
  static constexpr int B_TILES = STRIPS * R;     // 1 KiB blocks of B per K-tile
  static constexpr int TILES = A_TILES + B_TILES;
  static constexpr int TPW = TILES / WAVES;      // code blocks each wavefront moves per K-tile
  static constexpr int A_SC = BM / 64;           // 256-byte A-scale pieces per K-tile (waves 0..A_SC-1)
  static constexpr int B_SC = STRIPS / WAVES;    // 256-byte B-scale lines each wavefront moves
  static constexpr int NS = F::MB == 1 ? 4 : 3;  // K-tiles in the LDS ring
  static constexpr int A_SC_OFF = TILES * 1024;  // stage layout: code blocks, A scales, B scales
  static constexpr int B_SC_OFF = A_SC_OFF + BM * 4;
  static constexpr int STAGE = B_SC_OFF + STRIPS * 256;
  static_assert(TILES % WAVES == 0 && STRIPS % WAVES == 0, "work splits evenly over the wavefronts");
  static_assert(NS >= 2 && NS <= 5, "the waits count at most three K-tiles in flight behind the current one");
  // loads per wavefront per K-tile, for the wavefronts that move an A-scale piece and for the others
  static constexpr int CNT_A = TPW + 1 + B_SC, CNT_B = TPW + B_SC;
  // Scale groups (K a multiple of 512): the ring's stages hold code blocks
  // only, and the scales of four K-tiles at a time go into a two-slot ring of
  // groups after it: A, [BM rows][16 bytes] (one 16-byte load per row, by
  // wavefronts < A_SC); B, [STRIPS][64 lanes][4 bytes].
  static constexpr int STAGE4 = TILES * 1024;
  static constexpr int GSA = BM * 16;
  static constexpr int GSTAGE = GSA + STRIPS * 256;
  template <bool G4>
  static constexpr int ring_bytes() { return G4 ? NS * STAGE4 + 2 * GSTAGE : NS * STAGE; }
};

__device__ __forceinline__ uint32_t row_move32(uint32_t v) {  // neighbour swap inside a quad
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row16_max32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
  return v;
}

// s_waitcnt vmcnt(N), other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One K-tile of matrix instructions; the first tile of a chunk starts its
// chain from zero.
template <class F, int MF, int R>
__device__ __forceinline__ void mma_tile(const v4i (&a)[MF][R], const v4i (&b)[4][R], const uint32_t (&sa)[MF],
                                         const uint32_t (&sb)[4], bool first, v4f (&acc)[MF][4]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (F::MB == 1) {
        acc[i][j] = first ? mfma_fp4(a[i][0], b[j][0], zero, sa[i], sb[j])
                          : mfma_fp4(a[i][0], b[j][0], acc[i][j], sa[i], sb[j]);
      } else {
        acc[i][j] = first ? mfma_fp8(a[i][0], a[i][R - 1], b[j][0], b[j][R - 1], zero, sa[i], sb[j])
                          : mfma_fp8(a[i][0], a[i][R - 1], b[j][0], b[j][R - 1], acc[i][j], sa[i], sb[j]);
      }
    }
}

// Operand row of the workgroup's row rl: padding rows read the block's first
// row (a real one) and their results are discarded.
template <int MODE, int BM>
__device__ __forceinline__ int a_row(const GemmArgs& g, const int32_t* slots, int S, int mb, int rl) {
  const int rr = slots[rl] < S ? rl : 0;
  if constexpr (MODE == GU_ROUTED) return slots[rr] / g.k;
  return mb * BM + rr;
}

// Weight strip of the workgroup's strip s (0..4 WN - 1): gate/up tiles take the
// two gate strips and the two matching up strips of each of their WN 32-column
// intermediate blocks; down tiles take 4 WN consecutive strips.
template <int MODE, int WN>
__device__ __forceinline__ int w_strip(const GemmArgs& g, int nt, int s) {
  if constexpr (MODE == GU_ROUTED || MODE == GU_SHARED) {
    const int nb = WN * nt + (s >> 2), jj = s & 3;
    return (jj < 2 ? 0 : g.inter / 16) + 2 * nb + (jj & 1);
  }
  return 4 * WN * nt + s;
}

// Direct global -> LDS load of BYTES (4 or 16) per lane: lane l's bytes land
// at lds + l * BYTES (M0 holds the wavefront's LDS address).  Written as asm
// so that the compiler does not see it: it would otherwise order every LDS
// read of the kernel behind all direct loads in flight (a full lgkmcnt
// drain before each matrix instruction), although their completion is
// counted by vmcnt alone.  The kernel waits for them with explicit vmcnt
// waits; the load has no register result.
// M0 is a reserved register: clang warns that it does not preserve it across
// the asm.  The GEMM kernels have no other user of M0 (every M0 write in their
// code is this sequence; tests/test_build_cpu.py checks the compiled code), so
// nothing depends on a value the asm overwrites; the clobber documents it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* src, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)  // the asm is device code only
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

// Direct global -> LDS loads of this wavefront's share of K-tile kt into its
// ring slot: code blocks t = wave + WAVES i (1 KiB each, lane l's 16 bytes at
// l*16), one 256-byte piece of the rows' A scales (wavefronts < A_SC: lane l
// brings the 4 scale bytes of row 64*wave + l) and B_SC lines of B scales
// (lane l's word of strip wave + WAVES i, for the K-tile's group of 4).
template <class Gm>
__device__ __forceinline__ void issue_ktile(const uint8_t* (&src)[Gm::TPW], const int (&step)[Gm::TPW],
                                            const uint8_t* as_src, const uint8_t* (&bs_src)[Gm::B_SC],
                                            unsigned char* ring, int wave, int kt) {
  unsigned char* st = ring + (kt % Gm::NS) * Gm::STAGE;
#pragma unroll
  for (int i = 0; i < Gm::TPW; ++i)
    lds_dma<16>(src[i] + (size_t)kt * step[i], st + (wave + Gm::WAVES * i) * 1024);
  if (wave < Gm::A_SC) lds_dma<4>(as_src + 4 * kt, st + Gm::A_SC_OFF + wave * 256);
#pragma unroll
  for (int i = 0; i < Gm::B_SC; ++i)
    lds_dma<4>(bs_src[i] + (size_t)(kt >> 2) * 256, st + Gm::B_SC_OFF + (wave + Gm::WAVES * i) * 256);
}

// As issue_ktile with scale groups: the code blocks of K-tile kt into its ring
// stage and, when kt opens a group of four (kt % 4 == 0), that group's scales
// into group slot (kt / 4) % 2: 16 bytes of each row's A scales (the four
// K-tiles' four bytes each) and the lane's B-scale word of each strip.
template <class Gm>
__device__ __forceinline__ void issue_ktile_g4(const uint8_t* (&src)[Gm::TPW], const int (&step)[Gm::TPW],
                                               const uint8_t* as_src, const uint8_t* (&bs_src)[Gm::B_SC],
                                               unsigned char* ring, int wave, int kt) {
  unsigned char* st = ring + (kt % Gm::NS) * Gm::STAGE4;
#pragma unroll
  for (int i = 0; i < Gm::TPW; ++i)
    lds_dma<16>(src[i] + (size_t)kt * step[i], st + (wave + Gm::WAVES * i) * 1024);
  if ((kt & 3) == 0) {
    unsigned char* gs = ring + Gm::NS * Gm::STAGE4 + ((kt >> 2) & 1) * Gm::GSTAGE;
    if (wave < Gm::A_SC) lds_dma<16>(as_src + 4 * kt, gs + wave * 1024);
#pragma unroll
    for (int i = 0; i < Gm::B_SC; ++i) lds_dma<4>(bs_src[i] + (size_t)(kt >> 2) * 256, gs + Gm::GSA + (wave + Gm::WAVES * i) * 256);
  }
}

// s_waitcnt until only the loads of K-tiles kt+1 .. kt+ahead are pending, with
// scale groups: each K-tile brings TPW code-block loads, and the one opening a
// group SC more (at most one of up to three consecutive K-tiles does).
template <int TPW, int SC>
__device__ __forceinline__ void wait_ktiles_g4(int ahead, int kt) {
  const int ph = kt & 3;  // K-tile kt + 4 - ph opens the next group
  const bool extra = ahead >= 4 - ph;
  switch (2 * ahead + (extra ? 1 : 0)) {
    case 0: case 1: wait_vm<0>(); break;
    case 2: wait_vm<TPW>(); break;
    case 3: wait_vm<TPW + SC>(); break;
    case 4: wait_vm<2 * TPW>(); break;
    case 5: wait_vm<2 * TPW + SC>(); break;
    case 6: wait_vm<3 * TPW>(); break;
    default: wait_vm<3 * TPW + SC>(); break;
  }
}

// f(std::integral_constant<int, I>{}) for I = B .. E - 1, in order.
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One K-tile of FP4 products with the B scales taken as byte OPB of each
// strip's scale word (the word holds the scales of four K-tiles); the first
// tile of a chunk starts its chain from zero.
template <class F, int MF, int R, int OPB>
__device__ __forceinline__ void mma_tile_sel(const v4i (&a)[MF][R], const v4i (&b)[4][R], const uint32_t (&sa)[MF],
                                             const uint32_t (&sbw)[4], bool first, v4f (&acc)[MF][4]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  constexpr int FMT = F::MB == 1 ? 4 : 0;  // cbsz / blgp: E2M1 or E4M3 operands
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v8i A = {a[i][0][0], a[i][0][1], a[i][0][2], a[i][0][3],
                     R == 2 ? a[i][R - 1][0] : 0, R == 2 ? a[i][R - 1][1] : 0, R == 2 ? a[i][R - 1][2] : 0,
                     R == 2 ? a[i][R - 1][3] : 0};
      const v8i B = {b[j][0][0], b[j][0][1], b[j][0][2], b[j][0][3],
                     R == 2 ? b[j][R - 1][0] : 0, R == 2 ? b[j][R - 1][1] : 0, R == 2 ? b[j][R - 1][2] : 0,
                     R == 2 ? b[j][R - 1][3] : 0};
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, first ? zero : acc[i][j], FMT, FMT, 0,
                                                                    (int)sa[i], OPB, (int)sbw[j]);
    }
}

// issue_ktile_g4 with whether kt opens a scale group known at compile time.
template <class Gm, bool OPEN>
__device__ __forceinline__ void issue_ktile_g4c(const uint8_t* (&src)[Gm::TPW], const int (&step)[Gm::TPW],
                                                const uint8_t* as_src, const uint8_t* (&bs_src)[Gm::B_SC],
                                                unsigned char* ring, int wave, int kt) {
  unsigned char* st = ring + (kt % Gm::NS) * Gm::STAGE4;
#pragma unroll
  for (int i = 0; i < Gm::TPW; ++i) lds_dma<16>(src[i] + (size_t)kt * step[i], st + (wave + Gm::WAVES * i) * 1024);
  if constexpr (OPEN) {
    unsigned char* gs = ring + Gm::NS * Gm::STAGE4 + ((kt >> 2) & 1) * Gm::GSTAGE;
    if (wave < Gm::A_SC) lds_dma<16>(as_src + 4 * kt, gs + wave * 1024);
#pragma unroll
    for (int i = 0; i < Gm::B_SC; ++i) lds_dma<4>(bs_src[i] + (size_t)(kt >> 2) * 256, gs + Gm::GSA + (wave + Gm::WAVES * i) * 256);
  }
}

// s_waitcnt until at most `ahead` K-tiles of this wavefront's loads are pending.
template <int CNT>
__device__ __forceinline__ void wait_ktiles(int ahead) {
  switch (ahead) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<CNT>(); break;
    case 2: wait_vm<2 * CNT>(); break;
    default: wait_vm<3 * CNT>(); break;
  }
}

// Main loop.  The operands of K-tile kt travel global -> LDS with direct
// (LDS-destination) 16-byte loads into slot kt % NS of a ring, NS - 1 K-tiles
// ahead of the matrix instructions; each wavefront moves TPW of the tile's
// 1 KiB blocks and its share of the K-tile's block scales (4-byte direct
// loads of the activation scales, the weight-scale words of the K-tile's
// group of four).  Two workgroups share a CU (LDS), so the registers are held
// to two wavefronts per SIMD (256 per lane, accumulators included).
template <class F, int MODE, int WN, bool G4>
__global__ void __launch_bounds__(128 * WN) __attribute__((amdgpu_waves_per_eu(2)))
grouped_gemm_kernel(GemmArgs g) {  // 2 x WN wavefronts
  using Gm = Geo<F, WN>;
  constexpr int MF = Gm::MF, BM = Gm::BM, R = Gm::R, TPW = Gm::TPW, NS = Gm::NS;
  constexpr int WAVES = Gm::WAVES, THREADS = Gm::THREADS, STRIPS = Gm::STRIPS;
  constexpr bool kRouted = MODE == GU_ROUTED || MODE == DOWN_ROUTED;
  constexpr bool kGateUp = MODE == GU_ROUTED || MODE == GU_SHARED;
  extern __shared__ __align__(16) unsigned char smem[];

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so XCD x
  // is given the contiguous run of tiles x*per .. (x+1)*per - 1.  The grid is
  // sized for the largest padded row count; the live tile count is read here,
  // so the tiles past the sorted rows' end are spread over every XCD instead
  // of all falling into the last ones' runs (which would leave those idle).
  const int L = blockIdx.x;
  int ntiles = g.MB * g.NT;
  if constexpr (kRouted) ntiles = min(ntiles, (*g.num_padded + BM - 1) / BM * g.NT);
  const int per = (ntiles + 7) >> 3;  // tiles per XCD; gridDim.x / 8 >= per
  if ((L >> 3) >= per) return;
  // The routed gate/up with 256-column tiles (one workgroup per CU) runs a
  // persistent grid: the workgroup at position p of its XCD takes tiles
  // x*per + p, x*per + p + G/8, ... in turn (G the grid size); the others
  // take one tile each.
  constexpr bool kPersist = G4 && WN == 4 && MODE == GU_ROUTED;
  const int xcd = L & 7, stride = kPersist ? (int)(gridDim.x >> 3) : per;
  int it = L >> 3;
  int tile = xcd * per + it;
  if (tile >= ntiles) return;
  auto locate = [&](int t, int& mb_, int& nt_, int& e_) {
    int mb = t / g.NT, nt = t % g.NT;
    if constexpr (MODE == GU_SHARED) {
      // every row block multiplies the same weights: bands of GM row blocks
      // taken column by column, so the tiles that run together on an XCD share
      // their weight blocks GM ways (row-major, the XCD's 64 concurrent tiles
      // would cover four row blocks and every weight block; 3.5% faster at
      // 8192 rows).  Not for the shared down: its combine reads whole rows of
      // the routed outputs, which row-major order keeps contiguous.
      constexpr int GM = 16;
      const int band = t / (GM * g.NT), idx = t % (GM * g.NT);
      const int gm = min(GM, g.MB - band * GM);
      mb = band * GM + idx % gm;
      nt = idx / gm;
    }
    mb_ = mb;
    nt_ = nt;
    e_ = kRouted ? g.block_expert[mb] : 0;
  };
  int mb, nt, e;
  locate(tile, mb, nt, e);
  // the wavefront index as a uniform value: everything derived from it stays
  // in scalar registers (the persistent loop needs the vector registers)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int m = lane & 15, q = lane >> 4;
  const int S = g.T * g.k;
  const int KT = g.KT, KG = g.KG;

  unsigned char* ring = smem;
  int32_t* slots = reinterpret_cast<int32_t*>(smem + Gm::template ring_bytes<G4>());
  int32_t* slots_next = slots + BM;  // the next tile's (persistent grid)
  // the gate/up epilogue's output tile, apart from the ring that the next
  // tile's loads are filling (persistent grid)
  unsigned char* out_tile = reinterpret_cast<unsigned char*>(slots + 2 * BM);

  // A tile's rows and operand sources: slots, then (scales) A, the 4 bytes of
  // K-tile 0 of row 64*wave + lane; B, lane's word of group 0 of each strip
  // this wavefront moves; (codes) block t = wave + WAVES i of every K-tile
  const uint8_t* as_src;
  const uint8_t* bs_src[Gm::B_SC];
  const uint8_t* src[TPW];
  int step[TPW];
  auto setup = [&](int mb_, int nt_, int e_, int32_t* sl, const uint8_t*& as_s, const uint8_t* (&bs_s)[Gm::B_SC],
                   const uint8_t* (&sr)[TPW], int (&st)[TPW]) {
    if (threadIdx.x < BM) {
      const int r = mb_ * BM + (int)threadIdx.x;
      sl[threadIdx.x] = kRouted ? g.sorted_slots[r] : (r < g.T ? r : S);
    }
    __syncthreads();
    as_s = g.as + (size_t)a_row<MODE, BM>(g, sl, S, mb_, (64 * wave + lane) % BM) * g.as_stride;
    const uint8_t* bsb = g.bs + (size_t)e_ * g.bs_estride;
#pragma unroll
    for (int i = 0; i < Gm::B_SC; ++i)
      bs_s[i] = bsb + ((size_t)w_strip<MODE, WN>(g, nt_, wave + WAVES * i) * KG * 64 + lane) * 4;
    const uint8_t* bb = g.b + (size_t)e_ * g.b_estride;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + WAVES * i;
      if (t < Gm::A_TILES) {
        const int f = t / R, r = t % R;
        sr[i] = g.a + (size_t)a_row<MODE, BM>(g, sl, S, mb_, 16 * f + m) * g.a_stride + 64 * r + 16 * q;
        st[i] = 64 * R;
      } else {
        const int sb = (t - Gm::A_TILES) / R, r = (t - Gm::A_TILES) % R;
        sr[i] = bb + (size_t)w_strip<MODE, WN>(g, nt_, sb) * KT * 1024 * R + 1024 * r + lane * 16;
        st[i] = 1024 * R;
      }
    }
  };
  setup(mb, nt, e, slots, as_src, bs_src, src, step);

  v4f acc[MF][4], sum[MF][4];
  auto issue = [&](int kt) {
    if constexpr (G4)
      issue_ktile_g4<Gm>(src, step, as_src, bs_src, ring, wave, kt);
    else
      issue_ktile<Gm>(src, step, as_src, bs_src, ring, wave, kt);
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < KT) issue(s0);
  for (;;) {
    // chunk sums: -0 + x == x bit for bit (signed zeros included), so starting
    // from -0 and always adding equals taking the first chunk's sum as it is
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = sum[i][j] = v4f{-0.f, -0.f, -0.f, -0.f};

    if constexpr (G4) {
      // Scale groups, the loop unrolled by the group: the group's scales sit in
      // group slot (kg / 4) % 2 and K-tile kg + j's B scales are byte j of each
      // strip's scale word, so the waits and the scale bytes are constants (with
      // a four-stage ring the stage, j, is too).  Away from the last group NS - 2
      // K-tiles are in flight behind the current one, and when one of them opens
      // the next group (j >= 4 - (NS - 2)) its scale loads are in flight too.
      const bool a_wave = __builtin_amdgcn_readfirstlane(wave) < Gm::A_SC;  // uniform
      int t_in = 0;
      for (int g4 = 0; g4 < KT / 4; ++g4) {
        const int kg = 4 * g4;
        const bool last = kg + 4 >= KT;
        const unsigned char* gs = ring + NS * Gm::STAGE4 + ((kg >> 2) & 1) * Gm::GSTAGE;
        uint32_t sbw[4];
        static_for<0, 4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          const int kt = kg + j;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (!last) {
            if constexpr (j < 4 - (NS - 2)) {
              wait_vm<(NS - 2) * TPW>();
            } else {
              if (a_wave)
                wait_vm<(NS - 2) * TPW + 1 + Gm::B_SC>();
              else
                wait_vm<(NS - 2) * TPW + Gm::B_SC>();
            }
          } else {
            const int ahead = min(NS - 2, KT - 1 - kt);
            if (a_wave)
              wait_ktiles_g4<TPW, 1 + Gm::B_SC>(ahead, kt);
            else
              wait_ktiles_g4<TPW, Gm::B_SC>(ahead, kt);
          }
          // the barrier, as in the general loop below
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (kt + NS - 1 < KT) issue_ktile_g4c<Gm, (j + NS - 1) % 4 == 0>(src, step, as_src, bs_src, ring, wave, kt + NS - 1);
          const unsigned char* st = ring + (kt % NS) * Gm::STAGE4;
          v4i a[MF][R], b[4][R];
          uint32_t sa[MF];
          if constexpr (j == 0) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sbw[jj] = reinterpret_cast<const uint32_t*>(gs + Gm::GSA)[(4 * wn + jj) * 64 + lane];
          }
#pragma unroll
          for (int i = 0; i < MF; ++i) sa[i] = gs[(16 * (wm * MF + i) + m) * 16 + 4 * j + q];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int r = 0; r < R; ++r)
              b[jj][r] = *reinterpret_cast<const v4i*>(st + (Gm::A_TILES + (4 * wn + jj) * R + r) * 1024 + lane * 16);
#pragma unroll
          for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int r = 0; r < R; ++r)
              a[i][r] = *reinterpret_cast<const v4i*>(st + ((wm * MF + i) * R + r) * 1024 + lane * 16);
          __builtin_amdgcn_sched_barrier(0);
          if (t_in == 0)
            mma_tile_sel<F, MF, R, j>(a, b, sa, sbw, true, acc);
          else
            mma_tile_sel<F, MF, R, j>(a, b, sa, sbw, false, acc);
          if (++t_in == g.CT) {  // end of a chunk: add its sum in chunk order
            t_in = 0;
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) sum[i][jj] = sum[i][jj] + acc[i][jj];
          }
        });
      }
    } else {  // the general loop: scales per K-tile
      for (int kt = 0, t_in = 0; kt < KT; ++kt) {
        // K-tile kt has landed once only the K-tiles issued after it are pending
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int ahead = min(NS - 2, KT - 1 - kt);  // K-tiles issued after kt
        if (wave < Gm::A_SC)
          wait_ktiles<Gm::CNT_A>(ahead);
        else
          wait_ktiles<Gm::CNT_B>(ahead);
        // Each wavefront's own loads of K-tile kt are in LDS (the wait above); the
        // barrier makes that hold for all of them.  It is a bare s_barrier: the
        // workgroup fence of __syncthreads() would wait for every direct-to-LDS
        // load in flight, the later K-tiles' included, and empty the ring.  The
        // LDS reads of K-tile kt - 1 are complete (its matrix instructions have
        // consumed them), so its slot may be refilled once every wavefront is here.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + NS - 1 < KT) issue(kt + NS - 1);
        const unsigned char* st = ring + (kt % NS) * Gm::STAGE;
        const unsigned char* sc_a = st + Gm::A_SC_OFF;  // the K-tile's scales sit in its stage
        const uint32_t* sc_b = reinterpret_cast<const uint32_t*>(st + Gm::B_SC_OFF);
        v4i a[MF][R], b[4][R];
        uint32_t sa[MF], sb[4], sbw[4];
        // LDS reads in the order the matrix instructions consume them: scales,
        // the B strips, then A fragment by fragment, so that the instructions of
        // fragment i wait only for the reads up to a[i]
#pragma unroll
        for (int j = 0; j < 4; ++j) sbw[j] = sc_b[(4 * wn + j) * 64 + lane];
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const int f = wm * MF + i;
          sa[i] = sc_a[(16 * f + m) * 4 + q];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = 4 * wn + j;
#pragma unroll
          for (int r = 0; r < R; ++r)
            b[j][r] = *reinterpret_cast<const v4i*>(st + (Gm::A_TILES + s * R + r) * 1024 + lane * 16);
        }
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const int f = wm * MF + i;
#pragma unroll
          for (int r = 0; r < R; ++r) a[i][r] = *reinterpret_cast<const v4i*>(st + (f * R + r) * 1024 + lane * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) sb[j] = (sbw[j] >> (8 * (kt & 3))) & 0xffu;
        if (t_in == 0)
          mma_tile<F, MF, R>(a, b, sa, sb, true, acc);
        else
          mma_tile<F, MF, R>(a, b, sa, sb, false, acc);
        if (++t_in == g.CT) {  // end of a chunk: add its sum in chunk order
          t_in = 0;
#pragma unroll
          for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sum[i][j] = sum[i][j] + acc[i][j];
        }
      }
    }


    // Persistent grid: the next tile's rows, sources and first K-tiles are
    // requested here, so their latency overlaps this tile's epilogue (which
    // uses its own output tile in LDS, not the ring).  Only the routed gate/up
    // does this: the routed down's fp32 stores would sit in the in-order vmcnt
    // queue ahead of the next tile's first loads (it ran 3% slower persistent).
    it += stride;
    const int tile2 = xcd * per + it;
    const bool more = kPersist && it < per && tile2 < ntiles;  // uniform
    int mb2 = 0, nt2 = 0, e2 = 0;
    const uint8_t* as_src2 = nullptr;
    const uint8_t* bs_src2[Gm::B_SC];
    const uint8_t* src2[TPW];
    int step2[TPW];
    if constexpr (kPersist) {
      if (more) {
        locate(tile2, mb2, nt2, e2);
        __syncthreads();  // every wavefront is done reading the ring
        setup(mb2, nt2, e2, slots_next, as_src2, bs_src2, src2, step2);
#pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0)
          if (s0 < KT) issue_ktile_g4<Gm>(src2, step2, as_src2, bs_src2, ring, wave, s0);
      }
    }

    // ---------------------------------------------------------------- epilogues
    // The routed gate/up and down epilogues assemble the workgroup's output tile
    // in the (now idle) LDS ring and write it out with 16-byte row-contiguous
    // stores.
    if constexpr (kGateUp) {
      // SwiGLU on the 32 columns of block nb, then MX re-quantization of each
      // row's block.  sum[i][0], sum[i][1]: gate columns m and 16 + m; sum[i][2],
      // sum[i][3]: the matching up columns.  Output row of the intermediate: the
      // sorted position (routed) or the row (shared).
      constexpr int BPB = F::MB == 1 ? 16 : 32;  // code bytes of a row's 32-column block
      constexpr int RB = WN * BPB;               // code bytes of a row of the tile
      uint8_t* tc = kPersist ? out_tile : ring;   // [BM][RB] codes
      uint8_t* ts = tc + BM * RB;                // [BM][WN] scales
      __syncthreads();  // every wavefront is done reading the ring
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = wm * 16 * MF + 16 * i + 4 * q + r;
          const uint32_t a0 = __float_as_uint(silu_mul(sum[i][0][r], sum[i][2][r]));
          const uint32_t a1 = __float_as_uint(silu_mul(sum[i][1][r], sum[i][3][r]));
          const uint32_t am = row16_max32(max(a0 & 0x7fffffffu, a1 & 0x7fffffffu));
          const int ex = block_exponent<F>(am);
          const float inv = block_inv_scale(ex);
          uint8_t* op = tc + rl * RB + BPB * wn;
          if constexpr (F::MB == 1) {
            // even lanes pack columns m, m + 1 (the neighbour's value) into one
            // byte, low nibble first; the codes are those of quant_quad_fp4
            const uint32_t w = quant_quad_fp4(a0, row_move32(a0), a1, row_move32(a1), inv);
            if (!(m & 1)) {
              op[m / 2] = (uint8_t)w;
              op[8 + m / 2] = (uint8_t)(w >> 8);
            }
          } else {
            const uint32_t w = quant_pair_fp8(a0, a1, inv);
            op[m] = (uint8_t)w;
            op[16 + m] = (uint8_t)(w >> 8);
          }
          if (m == 0) ts[rl * WN + wn] = (uint8_t)(ex + 127);
        }
      __syncthreads();
      const size_t row_bytes = F::MB == 1 ? (size_t)g.inter / 2 : (size_t)g.inter;
      constexpr int PARTS = RB / 16;
      for (int t = threadIdx.x; t < BM * PARTS; t += THREADS) {
        const int rl = t / PARTS, part = t % PARTS;
        if (slots[rl] < S)
          *reinterpret_cast<uint4*>(g.oc + (size_t)(mb * BM + rl) * row_bytes + (size_t)(WN * nt) * BPB + 16 * part) =
              *reinterpret_cast<const uint4*>(tc + rl * RB + 16 * part);
      }
      for (int rl = threadIdx.x; rl < BM; rl += THREADS)
        if (slots[rl] < S) {
#pragma unroll
          for (int w = 0; w < WN; ++w) g.os[(size_t)(mb * BM + rl) * (g.inter / 32) + WN * nt + w] = ts[rl * WN + w];
        }
    } else if constexpr (MODE == DOWN_ROUTED && WN == 4) {
      // fp32 results straight from the registers (the 128 x 256 tile is too
      // large to assemble in the ring): for each of its rows a lane stores one
      // column of each strip, 16 lanes one 64-byte run
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = slots[wm * 16 * MF + 16 * i + 4 * q + r];
          if (slot < S) {
            float* dp = g.d_part + (size_t)slot * g.H + (size_t)(16 * STRIPS) * nt + m;
#pragma unroll
            for (int j = 0; j < 4; ++j) dp[16 * (4 * wn + j)] = sum[i][j][r];
          }
        }
    } else if constexpr (MODE == DOWN_ROUTED) {
      // fp32 result rows per slot: tile [BM][16 STRIPS] (row stride padded by
      // four floats against bank conflicts), columns 16 STRIPS nt onwards
      constexpr int CW = 16 * STRIPS;
      constexpr int LD = CW + 4;
      static_assert(BM * LD * 4 <= Gm::template ring_bytes<G4>(), "the output tile fits the ring");
      float* tf = reinterpret_cast<float*>(ring);
      __syncthreads();  // every wavefront is done reading the ring
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = wm * 16 * MF + 16 * i + 4 * q + r;
#pragma unroll
          for (int j = 0; j < 4; ++j) tf[rl * LD + 16 * (4 * wn + j) + m] = sum[i][j][r];
        }
      __syncthreads();
      constexpr int V = CW / 4;  // float4 per row
      for (int t = threadIdx.x; t < BM * V; t += THREADS) {
        const int rl = t / V, c4 = t % V;
        const int slot = slots[rl];
        if (slot < S)
          *reinterpret_cast<float4*>(g.d_part + (size_t)slot * g.H + (size_t)CW * nt + 4 * c4) =
              *reinterpret_cast<const float4*>(tf + rl * LD + 4 * c4);
      }
    } else {
      // combine: y = bf16( sum_j w_j d_j (j in order) + s + residual ).  Per
      // row fragment, every load of a batch of four choices (weights, routed
      // outputs, residual) is issued before any of them is used, so the
      // fragment waits for memory once rather than once per output.
      const int k = g.k;
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        int tr[4];
        float c[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tr[r] = mb * BM + wm * 16 * MF + 16 * i + 4 * q + r;
#pragma unroll
          for (int j = 0; j < 4; ++j) c[r][j] = 0.f;
        }
        for (int jc = 0; jc < k; jc += 4) {
          float wv[4][4], dv[4][4][4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tc = min(tr[r], g.T - 1);  // rows past the end read a real row, nothing is stored
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const bool on = jc + jj < k;
              wv[r][jj] = on ? g.topk_w[(size_t)tc * k + jc + jj] : 0.f;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int h = 16 * w_strip<MODE, WN>(g, nt, 4 * wn + j) + m;
                dv[r][j][jj] = on ? g.d_part[((size_t)tc * k + jc + jj) * g.H + h] : 0.f;
              }
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (jc + jj < k) {
#pragma unroll
                for (int j = 0; j < 4; ++j) c[r][j] = fmaf(wv[r][jj], dv[r][j][jj], c[r][j]);
              }
        }
        float rv[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int h = 16 * w_strip<MODE, WN>(g, nt, 4 * wn + j) + m;
            rv[r][j] = g.residual ? bf16_to_f32(g.residual[(size_t)min(tr[r], g.T - 1) * g.H + h]) : 0.f;
          }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tr[r] < g.T) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int h = 16 * w_strip<MODE, WN>(g, nt, 4 * wn + j) + m;
              float v = c[r][j] + sum[i][j][r];
              if (g.residual) v = v + rv[r][j];
              g.y[(size_t)tr[r] * g.H + h] = f32_to_bf16(v);
            }
          }
      }
    }

    if (!more) break;
    mb = mb2;
    nt = nt2;
    e = e2;
    {
      int32_t* t = slots;
      slots = slots_next;
      slots_next = t;
    }
    as_src = as_src2;
#pragma unroll
    for (int i = 0; i < Gm::B_SC; ++i) bs_src[i] = bs_src2[i];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      src[i] = src2[i];
      step[i] = step2[i];
    }
  }
}

// Combine without a shared expert: y = bf16( sum_j w_j d_j + residual ).
__global__ void __launch_bounds__(kThreads) combine_kernel(int T, int k, int H, const float* __restrict__ topk_w,
                                                           const float* __restrict__ d_part,
                                                           const uint16_t* residual, uint16_t* y) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)T * H) return;
  const int t = (int)(idx / H), h = (int)(idx % H);
  float c = 0.f;
  for (int j = 0; j < k; ++j) c = fmaf(topk_w[t * k + j], d_part[(size_t)(t * k + j) * H + h], c);
  if (residual) c = c + bf16_to_f32(residual[idx]);
  y[idx] = f32_to_bf16(c);
}

// Tiles per K-chunk: the dot product is cut into 4 (else 2, else 1) chunks.
int pick_chunk(int tiles) { return tiles / (tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1)); }

struct GCarve {
  size_t ids, w, logits, sort_ws, sorted, bexp, eoff, npad, xq4, xs4, xq8, xs8, a4, as4, a8, as8, d_part, rnorm, total;
  size_t cap, nblk;
};

GCarve gcarve(const moe_layer_t& L, int T) {
  // slots per row and experts in the table (with the folded shared expert: one more of each)
  const size_t H = L.hidden, I = L.inter, E = L.num_experts + (L.shared_folded ? 1 : 0), k = layer_slots(L),
               Is = L.shared_inter;
  const size_t S = (size_t)T * k;
  GCarve c{};
  c.cap = S + (S < E ? S : E) * (kBM - 1);
  c.nblk = (c.cap + kBM - 1) / kBM;
  const size_t rows = c.nblk * kBM;  // every sorted position a block can touch
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  c.ids = take(S * 4);
  c.w = take(S * 4);
  c.logits = take((size_t)T * E * 4);
  c.sort_ws = take(align_sort_ws_bytes(T, (int)k, (int)E));
  c.sorted = take(rows * 4);
  c.bexp = take(c.nblk * 4);
  c.eoff = take((E + 1) * 4);
  c.npad = take(4);
  c.xq4 = take((size_t)T * H / 2);
  c.xs4 = take((size_t)T * H / 32);
  c.xq8 = Is ? take((size_t)T * H) : 0;
  c.xs8 = Is ? take((size_t)T * H / 32) : 0;
  c.a4 = take(rows * I / 2);
  c.as4 = take(rows * I / 32);
  c.a8 = Is ? take((size_t)T * Is) : 0;
  c.as8 = Is ? take((size_t)T * Is / 32) : 0;
  c.d_part = take(S * H * 4);
  c.rnorm = L.norm_weight ? take((size_t)T * 4) : 0;
  c.total = o;
  return c;
}

unsigned grid8(int tiles) { return (unsigned)((tiles + 7) / 8 * 8); }

// Compute units of the current device, cached per device (lock-free; racing
// first calls store the same value).
int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices) return -1;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <class F, int MODE, int WN, bool G4>
hipError_t launch_gemm_as(const GemmArgs& g, hipStream_t stream) {
  using Gm = Geo<F, WN>;
  constexpr bool kPersist = G4 && WN == 4 && MODE == GU_ROUTED;
  // ring, slots (two sets when persistent) and the gate/up output tile
  const size_t lds = (size_t)Gm::template ring_bytes<G4>() + (size_t)Gm::BM * 4 * (kPersist ? 2 : 1) +
                     (kPersist ? (size_t)Gm::BM * (WN * 16 + WN) : 0);
  // the kernel's dynamic LDS limit is raised once per device (a lock-free
  // flag per device; racing first calls both set the same attribute)
  static std::atomic<bool> lds_set[kMaxDevices];
  if (lds > 64 * 1024) {
    const int dev = current_device();
    if (dev < 0) return hipErrorInvalidDevice;
    if (!lds_set[dev].load(std::memory_order_relaxed)) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_gemm_kernel<F, MODE, WN, G4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
      lds_set[dev].store(true, std::memory_order_relaxed);
    }
  }
  unsigned grid = grid8(g.MB * g.NT);
  if (kPersist) {  // one workgroup per CU, looping over tiles
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const unsigned cap = (unsigned)(cus / 8 * 8);
    if (cap > 0 && grid > cap) grid = cap;
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<F, MODE, WN, G4>), dim3(grid), dim3(Gm::THREADS), lds, stream, g);
  return hipGetLastError();
}

// Scale groups need whole groups of four K-tiles and 16-byte aligned rows of
// A scales (K a multiple of 512); other shapes load the scales per K-tile.
template <class F, int MODE, int WN>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
  const bool g4 = g.KT % 4 == 0 && g.as_stride % 16 == 0 && reinterpret_cast<uintptr_t>(g.as) % 16 == 0;
  return g4 ? launch_gemm_as<F, MODE, WN, true>(g, stream) : launch_gemm_as<F, MODE, WN, false>(g, stream);
}

}  // namespace

size_t grouped_ws_bytes(const moe_layer_t& L, int T) { return gcarve(L, T).total; }

// The grouped path's second stream on each device (default priority, created
// with the device current on its first untimed call) and its events: fork
// (recorded on the caller's stream, waited for by the side stream), quant
// (the side stream's quantization done) and join (all of its work done).
// Callers hold g_side_mu from the fork's record to the join's wait, so that
// concurrent host threads cannot interleave their records of these events.
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join, quant;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];
bool g_side_made[kMaxDevices];

hipError_t side_stream(const SideStream** out) {  // g_side_mu held
  *out = nullptr;
  const int dev = current_device();
  if (dev < 0) return hipErrorInvalidDevice;
  SideStream& S = g_side[dev];
  if (!g_side_made[dev]) {
    hipError_t err = hipStreamCreateWithFlags(&S.s, hipStreamNonBlocking);
    if (err != hipSuccess) return err;
    if ((err = hipEventCreateWithFlags(&S.fork, hipEventDisableTiming)) != hipSuccess ||
        (err = hipEventCreateWithFlags(&S.join, hipEventDisableTiming)) != hipSuccess ||
        (err = hipEventCreateWithFlags(&S.quant, hipEventDisableTiming)) != hipSuccess)
      return err;
    g_side_made[dev] = true;
  }
  *out = &S;
  return hipSuccess;
}

hipError_t launch_grouped(const moe_layer_t& L, const uint16_t* x, int T, const uint16_t* residual,
                          uint16_t* y, void* ws, hipStream_t stream, const hipEvent_t* ev) {
  // ev (optional): kGroupedSteps + 1 events, recorded before each step and at the end
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  const GCarve c = gcarve(L, T);
  char* base = reinterpret_cast<char*>(ws);
  auto at = [&](size_t off) { return base + off; };
  // k: slots per row, E: experts in the table; with the shared expert folded
  // in, slot k_routed of every row holds expert num_experts with weight 1
  const int H = L.hidden, I = L.inter, Is = L.shared_inter, k = layer_slots(L);
  const int E = L.num_experts + (L.shared_folded ? 1 : 0);
  int32_t* ids = reinterpret_cast<int32_t*>(at(c.ids));
  float* w = reinterpret_cast<float*>(at(c.w));
  int32_t* sorted = reinterpret_cast<int32_t*>(at(c.sorted));
  int32_t* bexp = reinterpret_cast<int32_t*>(at(c.bexp));
  int32_t* npad = reinterpret_cast<int32_t*>(at(c.npad));
  uint8_t* xq4 = reinterpret_cast<uint8_t*>(at(c.xq4));
  uint8_t* xs4 = reinterpret_cast<uint8_t*>(at(c.xs4));
  uint8_t* a4 = reinterpret_cast<uint8_t*>(at(c.a4));
  uint8_t* as4 = reinterpret_cast<uint8_t*>(at(c.as4));
  float* d_part = reinterpret_cast<float*>(at(c.d_part));
  hipError_t err;
  // Untimed and not under stream capture, the steps that do not depend on the
  // routing (x's MX quantization, the shared gate/up GEMM) run on the
  // device's side stream, forked from `stream` before the router: they fill
  // the GPU while the router's tail, the top-k and the token sort leave it
  // partly idle.  The routed gate/up waits for the quantization only, the
  // shared down (or the combine) for all of the side stream's work.
  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  const SideStream* side = nullptr;
  if (!ev) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((err = hipStreamIsCapturing(stream, &cs)) != hipSuccess) return err;
    if (cs == hipStreamCaptureStatusNone) {
      lock.lock();
      if ((err = side_stream(&side)) != hipSuccess) return err;
    }
  }
  const hipStream_t sq = side ? side->s : stream;  // stream of the quantization and the shared gate/up
  bool forked = false;
  auto join = [&]() -> hipError_t {
    forked = false;
    hipError_t e = hipEventRecord(side->join, side->s);
    return e == hipSuccess ? hipStreamWaitEvent(stream, side->join, 0) : e;
  };
  // on an error return after the fork, still order the side stream's work
  // before whatever the caller does next on `stream`
  struct JoinGuard {
    bool& f;
    decltype(join)& j;
    ~JoinGuard() {
      if (f) (void)j();
    }
  } guard{forked, join};
  if (side) {
    if ((err = hipEventRecord(side->fork, stream)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess) return err;
    forked = true;
  }
  if ((err = mark(0)) != hipSuccess) return err;
  if ((err = launch_router_topk(L, x, T, reinterpret_cast<float*>(at(c.logits)), ids, w,
                               k, L.shared_folded ? L.num_experts : -1, stream)) != hipSuccess)
    return err;
  if ((err = mark(1)) != hipSuccess) return err;
  if ((err = launch_align_sort(ids, T, k, E, kBM, sorted, bexp, reinterpret_cast<int32_t*>(at(c.eoff)), npad,
                               at(c.sort_ws), stream)) != hipSuccess)
    return err;
  if ((err = mark(2)) != hipSuccess) return err;
  // MXFP4 x (and, with a shared expert, MXFP8 x) from one read of x; with
  // the pre-router norm, of the normalized rows (the router normalizes its own)
  float* rnorm = nullptr;
  if (L.norm_weight) {
    rnorm = reinterpret_cast<float*>(at(c.rnorm));
    if ((err = launch_rms_rows(x, T, H, L.norm_eps, rnorm, sq)) != hipSuccess) return err;
    residual = x;  // the fused residual: the layer's own input
  }
  if (Is > 0)
    err = launch_quant_act_dual(x, T, H, xq4, xs4, reinterpret_cast<uint8_t*>(at(c.xq8)),
                                reinterpret_cast<uint8_t*>(at(c.xs8)), sq, rnorm, L.norm_weight);
  else
    err = launch_quant_act(x, T, H, MX_FMT_FP4, xq4, xs4, sq, rnorm, L.norm_weight);
  if (err != hipSuccess) return err;
  if ((err = mark(3)) != hipSuccess) return err;

  GemmArgs g{};
  g.T = T;
  g.k = k;
  g.H = H;
  g.sorted_slots = sorted;
  g.block_expert = bexp;
  g.num_padded = npad;
  uint8_t* xq8 = reinterpret_cast<uint8_t*>(at(c.xq8));
  uint8_t* xs8 = reinterpret_cast<uint8_t*>(at(c.xs8));
  uint8_t* a8 = reinterpret_cast<uint8_t*>(at(c.a8));
  uint8_t* as8 = reinterpret_cast<uint8_t*>(at(c.as8));
  constexpr int BM8 = Geo<FP8, 2>::BM;
  // shared gate/up: A = MXFP8 x, B = Ws13.  With at least 512 tiles of
  // 64 x 256 (two rounds of workgroups) and K on the scale-group loop,
  // eight-wavefront 64 x 256 tiles: each K-tile's 40 KB of operands feed
  // twice the products of a 64 x 128 tile's 24 KB (4% faster at 8192 rows);
  // with fewer rows the 64 x 128 tiles keep more workgroups busy.
  const bool wide_sgu = H % 512 == 0 && (size_t)((T + BM8 - 1) / BM8) * (Is / 128) >= 512;
  auto shared_gate_up = [&](hipStream_t s) -> hipError_t {
    GemmArgs r = g;
    r.MB = (T + BM8 - 1) / BM8;
    r.NT = Is / (wide_sgu ? 128 : 64);
    r.KT = H / 128;
    r.CT = pick_chunk(r.KT);
    r.KG = (r.KT + 3) / 4;
    r.a = xq8;
    r.as = xs8;
    r.a_stride = H;
    r.as_stride = H / 32;
    r.b = L.ws13;
    r.bs = L.ws13_scale;
    r.inter = Is;
    r.oc = a8;
    r.os = as8;
    return wide_sgu ? launch_gemm<FP8, GU_SHARED, 4>(r, s) : launch_gemm<FP8, GU_SHARED, 2>(r, s);
  };
  if (side) {
    if (Is > 0) {
      if ((err = hipEventRecord(side->quant, sq)) != hipSuccess) return err;
      if ((err = shared_gate_up(sq)) != hipSuccess) return err;
      if ((err = hipStreamWaitEvent(stream, side->quant, 0)) != hipSuccess) return err;
    } else {
      if ((err = join()) != hipSuccess) return err;
      lock.unlock();
    }
  }
  // routed gate/up: A = MXFP4 x gathered by slot, B = W13[e].  With at
  // least a full 128-row block per expert on average the products dominate:
  // 128 x 256 tiles (eight wavefronts, one workgroup per CU), whose K-tile of
  // 24 KB of operands feeds twice the products of a 128 x 128 tile's 16 KB
  // (routed gate/up 5% faster at 8192 rows).  With fewer rows the weights
  // dominate, and two 128 x 128 workgroups per CU keep more of them in
  // flight (the wide tile was 4% slower at 64 rows).
  const bool wide_gu = (size_t)T * k >= (size_t)128 * E;
  {
    GemmArgs r = g;
    r.MB = (int)c.nblk;
    r.NT = I / (wide_gu ? 128 : 64);
    r.KT = H / 128;
    r.CT = pick_chunk(r.KT);
    r.KG = (r.KT + 3) / 4;
    r.a = xq4;
    r.as = xs4;
    r.a_stride = H / 2;
    r.as_stride = H / 32;
    r.b = L.w13;
    r.bs = L.w13_scale;
    r.b_estride = tiled_codes_bytes(2 * I, H, MX_FMT_FP4);
    r.bs_estride = tiled_scales_bytes(2 * I, H);
    r.inter = I;
    r.oc = a4;
    r.os = as4;
    err = wide_gu ? launch_gemm<FP4, GU_ROUTED, 4>(r, stream) : launch_gemm<FP4, GU_ROUTED, 2>(r, stream);
    if (err != hipSuccess) return err;
  }
  if ((err = mark(4)) != hipSuccess) return err;
  // routed down: A = intermediate in sorted order, B = W2[e], out d_part[slot];
  // 256-column tiles (eight wavefronts) when H allows: each block's
  // intermediate is then read by half as many workgroups
  {
    const bool wide = H % 256 == 0;
    GemmArgs r = g;
    r.MB = (int)c.nblk;
    r.NT = H / (wide ? 256 : 128);
    r.KT = I / 128;
    r.CT = pick_chunk(r.KT);
    r.KG = (r.KT + 3) / 4;
    r.a = a4;
    r.as = as4;
    r.a_stride = I / 2;
    r.as_stride = I / 32;
    r.b = L.w2;
    r.bs = L.w2_scale;
    r.b_estride = tiled_codes_bytes(H, I, MX_FMT_FP4);
    r.bs_estride = tiled_scales_bytes(H, I);
    r.d_part = d_part;
    err = wide ? launch_gemm<FP4, DOWN_ROUTED, 4>(r, stream) : launch_gemm<FP4, DOWN_ROUTED, 2>(r, stream);
    if (err != hipSuccess) return err;
  }
  if ((err = mark(5)) != hipSuccess) return err;
  if (Is == 0) {
    const size_t n = (size_t)T * H;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                       T, k, H, w, d_part, residual, y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = mark(6)) != hipSuccess) return err;
    return mark(7);
  }
  if (!side && (err = shared_gate_up(stream)) != hipSuccess) return err;
  if (side) {
    if ((err = join()) != hipSuccess) return err;
    lock.unlock();
  }
  if ((err = mark(6)) != hipSuccess) return err;
  // shared down + combine
  {
    GemmArgs r = g;
    r.MB = (T + BM8 - 1) / BM8;
    r.NT = H / 128;
    r.KT = Is / 128;
    r.CT = pick_chunk(r.KT);
    r.KG = (r.KT + 3) / 4;
    r.a = a8;
    r.as = as8;
    r.a_stride = Is;
    r.as_stride = Is / 32;
    r.b = L.ws2;
    r.bs = L.ws2_scale;
    r.d_part = d_part;
    r.topk_w = w;
    r.residual = residual;
    r.y = y;
    if ((err = launch_gemm<FP8, DOWN_SHARED, 2>(r, stream)) != hipSuccess) return err;
  }
  return mark(7);
}

}  // namespace mxmoe
