// Stable counting sort of the routing slots by expert, padded per expert to a
// multiple of block_m.  Three passes over chunks of kSortChunk slots:
//   1. per chunk: histogram and each slot's stable rank among the chunk's
//      slots of the same expert (wavefront ballots, then a prefix over waves);
//   2. one workgroup: totals, padded offsets, per-chunk bases, block owners,
//      pad entries;
//   3. per chunk: scatter slot s to base[chunk][e] + rank(s).
#include "internal.h"
#include "mx_device.h"

namespace mxmoe {
namespace {

constexpr int kThreads = kSortChunk;  // one slot per thread
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxE = 256;
constexpr int kScanBatch = 16;  // chunk counts loaded together by the scan

__global__ void __launch_bounds__(kThreads) sort_rank_kernel(const int32_t* __restrict__ ids, int S,
                                                             int E, int32_t* __restrict__ hist,
                                                             int32_t* __restrict__ rank) {
  __shared__ int32_t wave_cnt[kWaves][kMaxE];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kWaves * kMaxE; i += kThreads) (&wave_cnt[0][0])[i] = 0;
  __syncthreads();
  const int s = blockIdx.x * kThreads + threadIdx.x;
  const int e = s < S ? ids[s] : -1;
  const bool valid = e >= 0 && e < E;  // ids outside [0, E) are left out
  // rank among the lanes below with the same expert
  int r = 0;
  uint64_t pending = __ballot(valid);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int le = __shfl(e, leader);
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) {
      r = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == leader) wave_cnt[wave][le] = __popcll(m);
    }
    pending &= ~m;
  }
  __syncthreads();
  // exclusive prefix over waves, per expert; chunk totals to the histogram
  for (int ee = threadIdx.x; ee < E; ee += kThreads) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_cnt[w][ee];
      wave_cnt[w][ee] = run;
      run += c;
    }
    hist[(size_t)blockIdx.x * E + ee] = run;
  }
  __syncthreads();
  if (valid) rank[s] = wave_cnt[wave][e] + r;
}

__global__ void __launch_bounds__(256) sort_scan_kernel(int32_t* __restrict__ hist, int nchunks, int S,
                                                        int E, int block_m, int capacity,
                                                        int32_t* __restrict__ sorted_slots,
                                                        int32_t* __restrict__ block_expert,
                                                        int32_t* __restrict__ expert_offsets,
                                                        int32_t* __restrict__ num_padded) {
  __shared__ int32_t total[kMaxE], padded[kMaxE], poff[kMaxE + 1], uoff[kMaxE + 1];
  const int tid = threadIdx.x;
  // the chunk counts of an expert are read kScanBatch at a time, all loads of
  // a batch issued before any is used
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) h[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) run += h[i];
    }
    total[e] = run;
    padded[e] = (run + block_m - 1) / block_m * block_m;
  }
  __syncthreads();
  // exclusive prefixes over the experts: thread e sums the entries below e
  // (independent LDS reads, so they pipeline); thread E forms the totals
  for (int e = tid; e <= E; e += blockDim.x) {
    int p = 0, u = 0;
    for (int e2 = 0; e2 < e; ++e2) {
      p += padded[e2];
      u += total[e2];
    }
    poff[e] = p;
    uoff[e] = u;
    if (e == E) *num_padded = p;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) expert_offsets[e] = uoff[e];
  // per-chunk destination bases (overwrite the histogram in place)
  for (int e = tid; e < E; e += blockDim.x) {
    int run = poff[e];
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) h[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (c0 + i < nchunks) {
          hist[(size_t)(c0 + i) * E + e] = run;
          run += h[i];
        }
    }
  }
  const int npad = poff[E];
  const int nblk_cap = capacity / block_m;
  // block owners: each expert marks its own blocks, blocks past the padded
  // length get -1
  for (int e = tid; e < E; e += blockDim.x)
    for (int b = poff[e] / block_m; b < (poff[e] + padded[e]) / block_m; ++b) block_expert[b] = e;
  for (int b = npad / block_m + tid; b < nblk_cap; b += blockDim.x) block_expert[b] = -1;
  // pad entries inside segments and everything past the padded length
  for (int e = tid; e < E; e += blockDim.x)
    for (int i = poff[e] + total[e]; i < poff[e] + padded[e]; ++i) sorted_slots[i] = S;
  for (int i = npad + tid; i < capacity; i += blockDim.x) sorted_slots[i] = S;
}

__global__ void __launch_bounds__(kThreads) sort_scatter_kernel(const int32_t* __restrict__ ids, int S,
                                                                int E, const int32_t* __restrict__ base,
                                                                const int32_t* __restrict__ rank,
                                                                int32_t* __restrict__ sorted_slots) {
  const int s = blockIdx.x * kThreads + threadIdx.x;
  if (s >= S) return;
  const int e = ids[s];
  if (e < 0 || e >= E) return;
  sorted_slots[base[(size_t)blockIdx.x * E + e] + rank[s]] = s;
}

}  // namespace

size_t align_sort_ws_bytes(int T, int k, int E) {
  const size_t S = (size_t)T * k;
  const size_t nchunks = (S + kSortChunk - 1) / kSortChunk;
  return align_up(nchunks * E * 4, 256) + align_up(S * 4, 256);
}

hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int block_m,
                             int32_t* sorted_slots, int32_t* block_expert, int32_t* expert_offsets,
                             int32_t* num_padded, void* ws, hipStream_t stream) {
  const int S = T * k;
  const int nchunks = (S + kSortChunk - 1) / kSortChunk;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                             align_up((size_t)nchunks * E * 4, 256));
  const int capacity = (int)moe_align_sort_capacity(T, k, E, block_m);
  hipLaunchKernelGGL(sort_rank_kernel, dim3(nchunks), dim3(kThreads), 0, stream, ids, S, E, hist, rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(256), 0, stream, hist, nchunks, S, E, block_m,
                     capacity, sorted_slots, block_expert, expert_offsets, num_padded);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(nchunks), dim3(kThreads), 0, stream, ids, S, E, hist,
                     rank, sorted_slots);
  return hipGetLastError();
}

}  // namespace mxmoe
