// route_align_dev.h -- device routines shared by the routing kernels (route.hip) and the
// alignment kernels (align.hip): the per-wave router tile, the per-token top-k selection
// and the single-workgroup counting sort.  Each kernel that uses them computes exactly what
// its stand-alone counterpart computes, in the same order.
#pragma once

#include "device_common.h"

namespace qmoe {

// One wave's split-K router tile: 16 tokens [t0, t0+16) x 16 experts [e0, e0+16) over K
// [kbeg, kend) of H.  K advances 128 per step: lane group g = l/16 loads the contiguous
// 32-element run [kc + 32g, kc + 32g + 32) of its row for both operands.  Tokens past T
// and experts past E read zeros.  PLANES: the wave also writes the MXFP4 activation planes of
// its tokens for every 128-wide step s of [kbeg, kend) with s % 4 == plane_wave (the 4 waves of
// a workgroup that load the same x rows share the work; -1: none), from the x runs it loaded,
// each lane one whole 32-element block: pq [2][T][H] e4m3 (hi, then lo) and ps [2][T][H/32]
// e8m0, the split the activation kernel makes (the same mx8_split on the same block).
template <bool PLANES = false>
__device__ __forceinline__ f32x4_t router_wave_partial(const uint16_t *__restrict__ x, int T, int H,
                                                       const uint16_t *__restrict__ w, int E, int t0, int e0,
                                                       int kbeg, int kend, uint8_t *__restrict__ pq = nullptr,
                                                       uint8_t *__restrict__ ps = nullptr, int plane_wave = -1) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4;
  const int ta = t0 + r, eb = e0 + r;
  const bool va = ta < T, vb = eb < E;
  const uint4 *xa = reinterpret_cast<const uint4 *>(x + (size_t)(va ? ta : 0) * H);
  const uint4 *wb = reinterpret_cast<const uint4 *>(w + (size_t)(vb ? eb : 0) * H);
  f32x4_t acc = zero4();
  for (int kc = kbeg; kc < kend; kc += 256) {  // two steps' loads in flight, then their MFMAs in order
    frag8 a[2][4], b[2][4];
#pragma unroll
    for (int st = 0; st < 2; st++) {
      const bool in = kc + 128 * st < kend;
      const int q = (kc + 128 * st + 32 * g) >> 3;  // uint4 index (8 bf16 each)
#pragma unroll
      for (int s = 0; s < 4; s++) {
        a[st][s].q = va && in ? xa[q + s] : make_uint4(0, 0, 0, 0);
        b[st][s].q = vb && in ? wb[q + s] : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int st = 0; st < 2; st++)
      if (kc + 128 * st < kend)
#pragma unroll
        for (int s = 0; s < 4; s++) acc = mfma_bf16(a[st][s], b[st][s], acc);
    if constexpr (PLANES) {
      if (plane_wave >= 0 && va) {
#pragma unroll
        for (int st = 0; st < 2; st++) {
          if (kc + 128 * st >= kend) break;
          if ((((kc - kbeg) >> 7) + st) % 4 != plane_wave) continue;
          float v[32];
#pragma unroll
          for (int s = 0; s < 4; s++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
              v[8 * s + 2 * j] = __uint_as_float(a[st][s].u[j] << 16);
              v[8 * s + 2 * j + 1] = __uint_as_float(a[st][s].u[j] & 0xFFFF0000u);
            }
          uint32_t qh[16], ql[16], s1, s2;
          mx8_split<32>(v, [](float m) { return m; }, qh, ql, s1, s2);
          const size_t k0 = (size_t)kc + 128 * st + 32 * g, o = (size_t)ta * H + k0, plane = (size_t)T * H;
#pragma unroll
          for (int h = 0; h < 2; h++) {
            *reinterpret_cast<uint4 *>(pq + o + 16 * h) =
                make_uint4(qh[8 * h] | (qh[8 * h + 1] << 16), qh[8 * h + 2] | (qh[8 * h + 3] << 16),
                           qh[8 * h + 4] | (qh[8 * h + 5] << 16), qh[8 * h + 6] | (qh[8 * h + 7] << 16));
            *reinterpret_cast<uint4 *>(pq + plane + o + 16 * h) =
                make_uint4(ql[8 * h] | (ql[8 * h + 1] << 16), ql[8 * h + 2] | (ql[8 * h + 3] << 16),
                           ql[8 * h + 4] | (ql[8 * h + 5] << 16), ql[8 * h + 6] | (ql[8 * h + 7] << 16));
          }
          ps[(size_t)ta * (H / 32) + k0 / 32] = (uint8_t)s1;
          ps[(size_t)T * (H / 32) + (size_t)ta * (H / 32) + k0 / 32] = (uint8_t)s2;
        }
      }
    }
  }
  return acc;
}

// Ordered 64-bit key: larger logit first, then lower index.  Float bits are mapped to an
// unsigned order (sign flip) in the upper half; the lower half is ~index.  -0.0 and +0.0
// are one score (equal logits tie to the lower index), so zero is made +0.0 first.
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)idx);
}

__device__ __forceinline__ int key_index(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

// 32-bit wave reductions.  The DPP row steps (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror) combine every lane of a 16-lane row exactly once, so each lane holds its row's
// result; row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3, fold rows 0-2
// into row 3, and lane 63 holds the wave's result, which is returned to every lane.  Lanes a
// step does not write keep their own value (update_dpp's `old`).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <typename F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t identity, F op) {
  v = op(v, dpp_u32<0xB1>(v, identity));   // quad_perm [1,0,3,2]
  v = op(v, dpp_u32<0x4E>(v, identity));   // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0x141>(v, identity));  // row_half_mirror
  v = op(v, dpp_u32<0x140>(v, identity));  // row_mirror
  v = op(v, dpp_u32<0x142, 0xA>(v, identity));  // row_bcast:15
  v = op(v, dpp_u32<0x143, 0xC>(v, identity));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Top-k of token t by one wave from its E logits `lg` (any memory; E <= 64 NS): each lane
// sorts its NS keys (experts l + 64q) descending; each round takes the wave-wide maximum of
// the lanes' heads and the winning lane shifts its keys.  Writes ids[t*k + j] in rank order
// and the softmax weights (over the k picks when renormalize, else over all E).  COPY: the
// ids also go to ids_copy (same index), e.g. an LDS array that a later step of the kernel reads.
template <int NS, bool COPY = false>
__device__ __forceinline__ void select_topk(const float *lg, int E, int k, int renormalize, int t,
                                            int32_t *__restrict__ ids, float *__restrict__ wts,
                                            int32_t *ids_copy = nullptr) {
  const int lane = lane_id();
  uint64_t key[NS];
  float vals[NS];
#pragma unroll
  for (int q = 0; q < NS; q++) {
    const int e = lane + 64 * q;
    vals[q] = e < E ? lg[e] : -INFINITY;
    key[q] = e < E ? rank_key(vals[q] != vals[q] ? -INFINITY : vals[q], e) : 0;  // NaN ranks last
  }
  // descending sort of the lane's keys (odd-even transposition network)
#pragma unroll
  for (int pass = 0; pass < NS; pass++)
#pragma unroll
    for (int q = pass & 1; q + 1 < NS; q += 2)
      if (key[q] < key[q + 1]) {
        const uint64_t tmp = key[q];
        key[q] = key[q + 1];
        key[q + 1] = tmp;
      }
  // Each round: the largest score among the lanes' heads (the upper half of the key), then the
  // lowest expert index among the heads holding it (ties only), then the winner's lane shifts.
  // A lane whose keys are used up holds 0, below every score (k <= E).
  float mine = 0.f, top = 0.f;
  for (int j = 0; j < k; j++) {
    const uint32_t hv = (uint32_t)(key[0] >> 32);
    const uint32_t m = wave_max_u32(hv);
    const uint64_t cand = __ballot(hv == m);
    int wl = __ffsll((unsigned long long)cand) - 1;
    if (__popcll(cand) > 1) {
      const uint32_t iv = hv == m ? (uint32_t)key_index(key[0]) : 0xFFFFFFFFu;
      wl = __ffsll((unsigned long long)__ballot(iv == wave_min_u32(iv))) - 1;
    }
    const int bi = __builtin_amdgcn_readlane(key_index(key[0]), wl);
    const float bv = key_value((uint64_t)m << 32);
    if (lane == wl) {
#pragma unroll
      for (int q = 0; q + 1 < NS; q++) key[q] = key[q + 1];
      key[NS - 1] = 0;
    }
    if (lane == j) mine = bv;
    if (j == 0) top = bv;
    if (lane == 0) ids[(size_t)t * k + j] = bi;
    if (COPY && lane == 0) ids_copy[t * k + j] = bi;
  }
  // softmax weights
  float z;
  if (renormalize) {
    z = lane < k ? expf(mine - top) : 0.f;
  } else {
    z = 0.f;
#pragma unroll
    for (int q = 0; q < NS; q++)
      if (lane + 64 * q < E) z += expf(vals[q] - top);
  }
  z = wave_sum_f32(z);
  if (lane < k) wts[(size_t)t * k + lane] = expf(mine - top) / z;
}

// Inclusive prefix sum over the wave (lane l gets the sum of lanes 0..l): row_shr 1, 2, 4, 8
// within each 16-lane row (lanes shifted in from outside the row add 0), then row_bcast:15
// and row_bcast:31 carry the rows' totals forward.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += (int)dpp_u32<0x111>((uint32_t)v, 0u);  // row_shr:1
  v += (int)dpp_u32<0x112>((uint32_t)v, 0u);  // row_shr:2
  v += (int)dpp_u32<0x114>((uint32_t)v, 0u);  // row_shr:4
  v += (int)dpp_u32<0x118>((uint32_t)v, 0u);  // row_shr:8
  v += (int)dpp_u32<0x142, 0xA>((uint32_t)v, 0u);  // row_bcast:15
  v += (int)dpp_u32<0x143, 0xC>((uint32_t)v, 0u);  // row_bcast:31
  return v;
}

// Stable counting sort of P <= 1024 * RPW pairs (ids[f], f < P) over E experts by one
// workgroup of exactly 1024 threads: histogram, scan, sentinels and the stable scatter.
// The pairs form 16 * RPW rows of 64; wave w owns rows [RPW w, RPW w + RPW) and ranks each
// pair among the equal ids of its row (ballot match masks); thread x owns expert x in the
// scan (E <= 1024).  Every slot of sorted_ids and block_expert is first written as padding
// (P, -1); the experts' blocks and the pairs overwrite theirs after the workgroup barriers.
// lds: (16 * RPW + 1) * E int32 of dynamic LDS (rowcnt [16 RPW][E], then start [E]).
template <int RPW>
__device__ __forceinline__ void align_block(const int32_t *__restrict__ ids, int P, int E, int BM, int cap,
                                            int32_t *__restrict__ sorted_ids, int32_t *__restrict__ block_expert,
                                            int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ total_padded, int32_t *lds) {
  constexpr int NR = 16 * RPW;  // rows of 64 pairs
  int32_t *rowcnt = lds;
  int32_t *start_of = lds + NR * E;
  __shared__ int32_t wsum[16];
  const int lane = lane_id(), wave = threadIdx.x >> 6, x = threadIdx.x;
  // block arithmetic: shifts when BM is a power of two, else divisions (uniform branch)
  const bool pow2 = (BM & (BM - 1)) == 0;
  const int sh = __builtin_ctz((unsigned)BM);
  auto blocks = [&](int v) { return pow2 ? v >> sh : v / BM; };
  int e[RPW];
#pragma unroll
  for (int q = 0; q < RPW; q++) {  // in flight while the padding is written and the counters cleared
    const int f = (RPW * wave + q) * 64 + lane;
    e[q] = f < P ? ids[f] : -1;
  }
  const int nblk = blocks(cap);
  for (int p = x; p < cap; p += blockDim.x) sorted_ids[p] = P;
  for (int b = x; b < nblk; b += blockDim.x) block_expert[b] = -1;
  for (int i = x; i < NR * E; i += blockDim.x) rowcnt[i] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank[RPW];
#pragma unroll
  for (int q = 0; q < RPW; q++) {
    rank[q] = 0;
    if (RPW * wave * 64 + q * 64 >= P) continue;  // no pair in this row (uniform)
    if (e[q] < 0 || e[q] >= E) e[q] = -1;
    uint64_t peers = __ballot(e[q] >= 0);
    for (int bit = 0; bit < nbits; bit++) {
      const uint64_t m = __ballot(e[q] >= 0 && ((e[q] >> bit) & 1));
      peers &= ((e[q] >> bit) & 1) ? m : ~m;
    }
    rank[q] = __popcll(peers & below);
    if (e[q] >= 0 && rank[q] == 0) rowcnt[(RPW * wave + q) * E + e[q]] = __popcll(peers);
  }
  __syncthreads();
  // per expert: exclusive prefix over the rows and the total count
  int run = 0;
  if (x < E) {
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += 16) {
      int v[16];  // 16 reads before their writes
#pragma unroll
      for (int rr = 0; rr < 16; rr++) v[rr] = rowcnt[(r0 + rr) * E + x];
#pragma unroll
      for (int rr = 0; rr < 16; rr++) {
        rowcnt[(r0 + rr) * E + x] = run;
        run += v[rr];
      }
    }
    counts[x] = run;
  }
  const int padded = x < E ? blocks(run + BM - 1) * BM : 0;
  const int inc = wave_inclusive_scan(padded);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int wbase = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    const int ws = wsum[w];
    wbase += w < wave ? ws : 0;
    total += ws;
  }
  const int start = wbase + inc - padded;
  if (x < E) {
    start_of[x] = start;
    offsets[x] = start;
    for (int b = blocks(start); b < blocks(start + padded); b++) block_expert[b] = x;
  }
  if (x == 0) {
    offsets[E] = total;
    total_padded[0] = total;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RPW; q++) {
    const int row = RPW * wave + q;
    if (e[q] >= 0) sorted_ids[start_of[e[q]] + rowcnt[row * E + e[q]] + rank[q]] = row * 64 + lane;
  }
}

}  // namespace qmoe
