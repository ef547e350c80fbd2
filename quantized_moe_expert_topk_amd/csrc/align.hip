// align.hip -- moe_align for gfx950: a stable counting sort of the T*k flat (token, slot)
// pairs by expert, each expert's run padded to a multiple of block_m.  The FreeToken pages
// name this step (PR #637 "Notes": the moe_align fallback on ROCm) without defining it;
// the definition implemented here is the one stated in include/qmoe.h.
//
// Three passes over chunks of 1024 pairs, none of them ordered by atomics, so the result
// is deterministic:
//   1. k_align_hist    per-chunk expert histograms -> hist[chunk][E]; also fills every slot
//                      of sorted_ids with the sentinel (pass 3 overwrites the pairs' slots)
//   2. k_align_scan    per-expert exclusive prefix over chunks (in place), counts, padded
//                      offsets and block_expert
//   3. k_align_scatter stable rank of each pair inside its chunk (ballot match masks per
//                      64-pair row, prefix over the 16 rows of the chunk) -> sorted_ids
#include "device_common.h"
#include "launch.h"
#include "route_align_dev.h"

namespace qmoe {

constexpr int kChunk = 1024;  // pairs per chunk = 16 rows of 64

__global__ __launch_bounds__(256) void k_align_hist(const int32_t *__restrict__ ids, int P, int E,
                                                    int32_t *__restrict__ hist, int nchunk, int cap,
                                                    int32_t *__restrict__ sorted_ids) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < cap; p += gridDim.x * blockDim.x) sorted_ids[p] = P;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int f = base + i;
    if (f < P) {
      const int e = ids[f];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);  // a count does not depend on the order
    }
  }
  __syncthreads();
  if ((int)blockIdx.x < nchunk)
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads.  Thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void k_align_scan(int32_t *__restrict__ hist, int nchunk, int E, int BM,
                                                     int P, int cap, int32_t *__restrict__ block_expert,
                                                     int32_t *__restrict__ counts,
                                                     int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ total_padded) {
  __shared__ int32_t start_of[1025];  // padded start of expert e; start_of[E] = total
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // exclusive prefix over chunks, 32 independent loads at a time: each batch is one round trip
    // to the histograms the previous kernel wrote (T = 8192, k = 8: 64 chunks in 2 round trips;
    // measured 7.2 -> 6.3 us against batches of 8)
    for (int c0 = 0; c0 < nchunk; c0 += 32) {
      int v[32];
#pragma unroll
      for (int u = 0; u < 32; u++) v[u] = c0 + u < nchunk ? hist[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 32; u++) {
        if (c0 + u < nchunk) hist[(size_t)(c0 + u) * E + e] = run;  // where chunk c's pairs of e start
        run += v[u];
      }
    }
    counts[e] = run;
  }
  const int padded = e < E ? (run + BM - 1) / BM * BM : 0;
  // block-wide exclusive scan of padded (wave scan, then scan of the 16 wave totals)
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int inc = padded;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; w++) wbase += wsum[w];
  const int start = wbase + inc - padded;
  int total = 0;
  for (int w = 0; w < 16; w++) total += wsum[w];
  if (e < E) {
    offsets[e] = start;
    start_of[e] = start;
  }
  if (e == 0) {
    offsets[E] = total;
    total_padded[0] = total;
    start_of[E] = total;
  }
  __syncthreads();
  // block b belongs to the last expert whose padded start is <= b*BM (starts ascend; an
  // empty expert shares its start with the next one), or to none past the total
  for (int b = threadIdx.x; b < cap / BM; b += blockDim.x) {
    const int p = b * BM;
    int owner = -1;
    if (p < total) {
      int lo = 0, hi = E - 1;  // largest e with start_of[e] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start_of[mid] <= p) lo = mid; else hi = mid - 1;
      }
      owner = lo;
    }
    block_expert[b] = owner;
  }
}

// One workgroup (256 threads = 4 waves) per chunk; wave w handles rows 4w..4w+3 of 64 pairs.
__global__ __launch_bounds__(256) void k_align_scatter(const int32_t *__restrict__ ids, int P, int E,
                                                       const int32_t *__restrict__ hist,
                                                       const int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ sorted_ids) {
  extern __shared__ int32_t rowcnt[];  // [16][E]: pairs of expert e in row r of this chunk
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 16 * E; i += blockDim.x) rowcnt[i] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int myexp[4], myrank[4];
  const int base = blockIdx.x * kChunk;
#pragma unroll
  for (int rr = 0; rr < 4; rr++) {
    const int row = wave * 4 + rr;
    const int f = base + row * 64 + lane;
    int e = f < P ? ids[f] : -1;
    if (e < 0 || e >= E) e = -1;
    uint64_t peers = __ballot(e >= 0);
    for (int bit = 0; bit < nbits; bit++) {
      const uint64_t m = __ballot(e >= 0 && ((e >> bit) & 1));
      peers &= ((e >> bit) & 1) ? m : ~m;
    }
    myexp[rr] = e;
    myrank[rr] = __popcll(peers & below);
    if (e >= 0 && myrank[rr] == 0) rowcnt[row * E + e] = __popcll(peers);  // row leader
  }
  __syncthreads();
  // exclusive prefix over the 16 rows, per expert
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int r = 0; r < 16; r++) {
      const int v = rowcnt[r * E + e];
      rowcnt[r * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 4; rr++) {
    const int row = wave * 4 + rr;
    const int e = myexp[rr];
    if (e >= 0) {
      const int f = base + row * 64 + lane;
      const int pos = offsets[e] + hist[(size_t)blockIdx.x * E + e] + rowcnt[row * E + e] + myrank[rr];
      sorted_ids[pos] = f;
    }
  }
}

// Single-workgroup path (decode and mid-size batches): histogram, scan, sentinels and the
// stable scatter in one launch of 1024 threads, for P <= 1024 pairs and E <= 512 (RPW = 1), or
// P <= 4096 and E <= 256 (RPW = 4: four rows of 64 pairs per wave; at T = 256, k = 8 one launch
// instead of the three chunked passes).
template <int RPW>
__global__ __launch_bounds__(1024) void k_align_small(const int32_t *__restrict__ ids, int P, int E, int BM,
                                                      int cap, int32_t *__restrict__ sorted_ids,
                                                      int32_t *__restrict__ block_expert,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ total_padded) {
  extern __shared__ int32_t lds[];  // rowcnt [16 RPW][E], then start [E]
  align_block<RPW>(ids, P, E, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded, lds);
}

hipError_t launch_align(const int32_t *ids, int T, int k, int E, int BM, int cap, int32_t *sorted_ids,
                        int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded,
                        int32_t *hist, hipStream_t s) {
  const int P = T * k;
  if (P <= kChunk && E <= 512) {
    hipLaunchKernelGGL(k_align_small<1>, dim3(1), dim3(1024), 17 * E * sizeof(int32_t), s, ids, P, E, BM, cap,
                       sorted_ids, block_expert, counts, offsets, total_padded);
    return hipGetLastError();
  }
  if (P <= 4 * kChunk && E <= 256) {
    hipLaunchKernelGGL(k_align_small<4>, dim3(1), dim3(1024), 65 * E * sizeof(int32_t), s, ids, P, E, BM, cap,
                       sorted_ids, block_expert, counts, offsets, total_padded);
    return hipGetLastError();
  }
  const int nchunk = (P + kChunk - 1) / kChunk;
  // at least one workgroup, which also writes the sentinels when there are no pairs
  hipLaunchKernelGGL(k_align_hist, dim3(nchunk > 0 ? nchunk : 1), dim3(256), E * sizeof(int32_t), s, ids, P, E,
                     hist, nchunk, cap, sorted_ids);
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(1024), 0, s, hist, nchunk, E, BM, P, cap, block_expert, counts,
                     offsets, total_padded);
  if (nchunk > 0) {
    hipLaunchKernelGGL(k_align_scatter, dim3(nchunk), dim3(256), 16 * E * sizeof(int32_t), s, ids, P, E,
                       hist, offsets, sorted_ids);
  }
  return hipGetLastError();
}

}  // namespace qmoe
