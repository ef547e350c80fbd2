// route.hip -- replicated router and top-k selection for gfx950.
//
// logits[t, e] = sum_h x[t, h] W[e, h] + bias[e] on bf16 MFMA with fp32 accumulation,
// then per token the k experts ranking first under (logit descending, index ascending)
// and their softmax weights (renormalised over the k picks when norm_topk_prob is set:
// FreeToken issue #62, second comment; PR #70 ownership table, "Router ... Replicated").
//
// Kernels:
//   k_router_partial  split-K GEMM: KS workgroup layers each reduce H/KS of K and write
//                     their own partial [KS][T][E] (no atomics), so decode-sized batches
//                     still spread the router weight over the whole chip.
//   k_topk            sums the KS partials in a fixed order (plus bias), writes the
//                     logits, then one wave per token selects k experts by k rounds of a
//                     wave-wide (value, lower index) maximum built from DPP row steps.
//   k_topk_align      for T <= 8 (it handles up to 16): k_topk's work for every token in one workgroup of 1024
//                     threads, then moe_align's single-workgroup counting sort on the picks,
//                     which stay in LDS (moe_route_align; the same results as k_topk followed
//                     by k_align_small, one launch and one global round trip fewer).
#include "device_common.h"
#include "launch.h"
#include "route_align_dev.h"

namespace qmoe {

// One workgroup = 4 waves = 16 tokens x 64 experts x one K split; wave w owns experts
// [16w, 16w+16).  K advances 128 per step: lane group g = l/16 loads the contiguous
// 32-element run [kc + 32g, kc + 32g + 32) of its row for both operands.
// PLANES: the 4 waves of the first expert group also write the MXFP4 activation planes of
// their tokens over their K range, a quarter of the steps each (router_wave_partial; measured on
// MI355X against wave 0 alone: DeepSeek-shaped layer T = 256, 373.3 -> 371.9 us per step).
template <bool PLANES>
__global__ __launch_bounds__(256) void k_router_partial(const uint16_t *__restrict__ x, int T, int H,
                                                        const uint16_t *__restrict__ w, int E,
                                                        const float *__restrict__ bias, int kchunk,
                                                        float *__restrict__ part, uint8_t *__restrict__ pq,
                                                        uint8_t *__restrict__ ps) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.y * 16, e0 = blockIdx.x * 64 + wave * 16;
  // a wave past the last expert has no logits to compute, but in the first expert group it still
  // writes its share of the activation planes (its weight loads read zeros)
  if (e0 >= E && !(PLANES && blockIdx.x == 0)) return;
  const int ks = blockIdx.z;
  const int kbeg = ks * kchunk;
  const f32x4_t acc = router_wave_partial<PLANES>(x, T, H, w, E, t0, e0, kbeg, kbeg + kchunk, pq, ps,
                                                  PLANES && blockIdx.x == 0 ? wave : -1);
  const int eb = e0 + r;
  if (eb < E) {
    const float bv = (bias && ks == 0 && gridDim.z == 1) ? bias[eb] : 0.f;
    float *dst = part + (size_t)ks * T * E;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int t = t0 + 4 * g + j;
      if (t < T) dst[(size_t)t * E + eb] = acc[j] + bv;
    }
  }
}

// ---------------------------------------------------------------------------- top-k

// Four tokens per workgroup.  Phase 1: all threads sum the KS partials of the 4 tokens'
// logits (fixed order, independent loads), add the bias, write the logits and stage them
// in LDS.  Phase 2: wave w selects for token w.  Each lane sorts its NS keys (experts
// l + 64q) descending; each round takes the wave-wide maximum of the lanes' heads and the
// winning lane shifts its keys.
// Phase 1 for tokens [t0, t0 + 4) by 256 threads (u = thread index among them): lg[tt][e].
template <int NS, int KSMAX>
__device__ __forceinline__ void topk_gather(const float *__restrict__ part, int KS, int T, int E,
                                            const float *__restrict__ bias, float *__restrict__ logits_out,
                                            int t0, int u, float (*lg)[NS * 64]) {
  for (int e = u; e < E; e += 256) {
    // 4 tokens x KSMAX partials, every load unconditional (indices clamped) so all are in
    // flight at once; values past KS or T are masked, sums run in split order
    float v[4][KSMAX];
    const rsrc_t pr = make_rsrc(part, (uint32_t)KS * T * E * 4);
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const uint32_t vo = ((uint32_t)min(t0 + tt, T - 1) * E + e) * 4;  // token + expert (VGPR)
#pragma unroll
      for (int q = 0; q < KSMAX; q++)  // split slice (SGPR offset)
        v[tt][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 pr, (int)vo, (int)((uint32_t)min(q, KS - 1) * T * E * 4), 0));
    }
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < KSMAX; q++) s += q < KS ? v[tt][q] : 0.f;
      s += b;
      if (t0 + tt < T && logits_out) logits_out[(size_t)(t0 + tt) * E + e] = s;
      lg[tt][e] = s;
    }
  }
}

template <int NS, int KSMAX>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ part, int KS, int T, int E,
                                              const float *__restrict__ bias, int k, int renormalize,
                                              float *__restrict__ logits_out, int32_t *__restrict__ ids,
                                              float *__restrict__ wts) {
  __shared__ float lg[4][NS * 64];
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 4;
  topk_gather<NS, KSMAX>(part, KS, T, E, bias, logits_out, t0, threadIdx.x, lg);
  __syncthreads();
  const int t = t0 + wave;
  if (t < T) select_topk<NS>(lg[wave], E, k, renormalize, t, ids, wts);
}

// T <= 16 tokens, E <= 512 (NS <= 8), T * k <= 1024: thread group g = tid / 256 gathers tokens
// [4g, 4g + 4), wave w selects token w, then the whole workgroup aligns the T * k picks.
// Dynamic LDS: 17 * E int32 for the counting sort.  (Larger batches in chunks of 16 tokens
// measured slower than k_topk's workgroups in parallel followed by k_align_small: at T = 64,
// 34 us against 11 us, every chunk paying the partial-sum loads' latency alone.)
template <int NS, int KSMAX>
__global__ __launch_bounds__(1024) void k_topk_align(const float *__restrict__ part, int KS, int T, int E,
                                                     const float *__restrict__ bias, int k, int renormalize,
                                                     float *__restrict__ logits_out, int32_t *__restrict__ ids,
                                                     float *__restrict__ wts, int BM, int cap,
                                                     int32_t *__restrict__ sorted_ids,
                                                     int32_t *__restrict__ block_expert, int32_t *__restrict__ counts,
                                                     int32_t *__restrict__ offsets,
                                                     int32_t *__restrict__ total_padded) {
  extern __shared__ int32_t align_lds[];
  __shared__ float lg[16][NS * 64];
  __shared__ int32_t picks[1024];
  const int wave = threadIdx.x >> 6, grp = threadIdx.x >> 8;
  if (4 * grp < T) topk_gather<NS, KSMAX>(part, KS, T, E, bias, logits_out, 4 * grp, threadIdx.x & 255, &lg[4 * grp]);
  __syncthreads();
  if (wave < T) select_topk<NS, true>(lg[wave], E, k, renormalize, wave, ids, wts, picks);
  __syncthreads();
  align_block<1>(picks, T * k, E, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded, align_lds);
}

template <int KSMAX>
static void launch_topk_ks(const float *part, int KS, int T, int E, const float *bias, int k, int renormalize,
                           float *logits_out, int32_t *ids, float *wts, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  const int slots = (E + 63) / 64;
  if (slots <= 1)
    hipLaunchKernelGGL((k_topk<1, KSMAX>), grid, block, 0, s, part, KS, T, E, bias, k, renormalize, logits_out, ids, wts);
  else if (slots <= 2)
    hipLaunchKernelGGL((k_topk<2, KSMAX>), grid, block, 0, s, part, KS, T, E, bias, k, renormalize, logits_out, ids, wts);
  else if (slots <= 4)
    hipLaunchKernelGGL((k_topk<4, KSMAX>), grid, block, 0, s, part, KS, T, E, bias, k, renormalize, logits_out, ids, wts);
  else if (slots <= 8)
    hipLaunchKernelGGL((k_topk<8, KSMAX>), grid, block, 0, s, part, KS, T, E, bias, k, renormalize, logits_out, ids, wts);
  else
    hipLaunchKernelGGL((k_topk<16, KSMAX>), grid, block, 0, s, part, KS, T, E, bias, k, renormalize, logits_out, ids, wts);
}

static hipError_t launch_topk_ns(const float *part, int KS, int T, int E, const float *bias, int k, int renormalize,
                                 float *logits_out, int32_t *ids, float *wts, hipStream_t s) {
  // the partial loads are unrolled KSMAX times (indices past KS clamped), so KSMAX follows KS
  if (KS <= 1)
    launch_topk_ks<1>(part, 1, T, E, bias, k, renormalize, logits_out, ids, wts, s);
  else if (KS <= 2)
    launch_topk_ks<2>(part, KS, T, E, bias, k, renormalize, logits_out, ids, wts, s);
  else if (KS <= 4)
    launch_topk_ks<4>(part, KS, T, E, bias, k, renormalize, logits_out, ids, wts, s);
  else if (KS <= 8)
    launch_topk_ks<8>(part, KS, T, E, bias, k, renormalize, logits_out, ids, wts, s);
  else
    launch_topk_ks<16>(part, KS, T, E, bias, k, renormalize, logits_out, ids, wts, s);
  return hipGetLastError();
}

// K splits for the router GEMM: enough workgroups to cover the chip at small T.
// Large batches run the router on the LDS-tiled GEMM (128 tokens x 128 experts per
// workgroup), small ones on k_router_partial.  k_router_partial splits K until about 512
// workgroups are in flight (at most 16 splits): a workgroup's K loop is a chain of dependent
// load round trips, so shorter ones finish sooner (T = 256, H = 4096: 2 -> 8 splits, step
// 409 -> 402 us).  The tiled GEMM splits until about 256 workgroups: every split adds T x E
// fp32 partials that the top-k kernel reads back (E = 256: T = 8192 4 -> 2 splits, step
// 646 -> 640 us; T = 4096 8 -> 4 splits, 269 -> 264 us).
static bool router_tiled(int T) { return T >= 1024; }
bool router_writes_planes(int T) { return !router_tiled(T); }

int router_ksplit(int T, int E, int H) {
  if (router_tiled(T)) {  // K ranges stay whole 64-wide stages
    const int base = ((T + 127) / 128) * ((E + 127) / 128);
    int ks = 1;
    while (base * ks < 256 && ks < 8 && (H / 64) % (ks * 2) == 0) ks *= 2;
    return ks;
  }
  const int base = ((E + 63) / 64) * ((T + 15) / 16);
  int ks = 1;
  while (base * ks < 512 && ks < 16 && ks * 2 <= H / 128 && (H / 128) % (ks * 2) == 0) ks *= 2;
  return ks;
}

size_t router_workspace_bytes(int T, int E, int H) {
  const int ks = router_ksplit(T, E, H);
  return ks > 1 ? (size_t)ks * T * E * sizeof(float) : 0;
}

// The router GEMM into part: the K-split partials [ks][T][E] when ks > 1, else the logits
// with the bias added.
static hipError_t launch_router_gemm(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias,
                                     int ks, float *part, const XPlanes *xp, hipStream_t s) {
  if (router_tiled(T)) return launch_router_tiled(x, T, H, w, E, bias, ks, part, s);
  dim3 grid((E + 63) / 64, (T + 15) / 16, ks);
  if (xp)
    hipLaunchKernelGGL(k_router_partial<true>, grid, dim3(256), 0, s, x, T, H, w, E, bias, H / ks, part, xp->q, xp->s);
  else
    hipLaunchKernelGGL(k_router_partial<false>, grid, dim3(256), 0, s, x, T, H, w, E, bias, H / ks, part, nullptr,
                       nullptr);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias,
                         float *logits, float *partial, int *ks, const XPlanes *xp, hipStream_t s) {
  *ks = router_ksplit(T, E, H);
  return launch_router_gemm(x, T, H, w, E, bias, *ks, *ks > 1 ? partial : logits, xp, s);
}

hipError_t launch_route(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int k,
                        int renormalize, float *logits, int32_t *ids, float *wts, float *partial,
                        hipStream_t s) {
  const int ks = router_ksplit(T, E, H);
  float *part = ks > 1 ? partial : logits;
  const hipError_t e = launch_router_gemm(x, T, H, w, E, bias, ks, part, nullptr, s);
  if (e != hipSuccess) return e;
  // with one split the GEMM already added the bias and wrote the logits in place
  return launch_topk_ns(part, ks, T, E, ks > 1 ? bias : nullptr, k, renormalize, ks > 1 ? logits : nullptr, ids, wts,
                        s);
}

hipError_t launch_topk(const float *logits, int T, int E, const float *bias, int k, int renormalize,
                       int32_t *ids, float *wts, hipStream_t s) {
  return launch_topk_ns(logits, 1, T, E, bias, k, renormalize, nullptr, ids, wts, s);
}

// The one workgroup loads every token's split-K partials itself (T x E x splits), so past a few
// tokens the parallel top-k workgroups and k_align_small win.  Measured on MI355X, E = 256, k = 8
// (step, us): T = 8 fused 36.5 vs 37.0; T = 16 fused 45.2 vs 43.1 (NVFP4 decode layer) and 134.7 vs
// 132.5 (DeepSeek-shaped MXFP4 layer).
bool route_align_fused(int T, int E, int k) { return T >= 1 && T <= 8 && E <= 512 && T * k <= 1024; }

template <int NS>
static void launch_topk_align_ns(const float *part, int KS, int T, int E, const float *bias, int k, int renormalize,
                                 float *logits_out, int32_t *ids, float *wts, int BM, int cap, int32_t *sorted_ids,
                                 int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded,
                                 hipStream_t s) {
  const size_t lds = 17 * (size_t)E * sizeof(int32_t);
  if (KS <= 1)
    hipLaunchKernelGGL((k_topk_align<NS, 1>), dim3(1), dim3(1024), lds, s, part, 1, T, E, bias, k, renormalize,
                       logits_out, ids, wts, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded);
  else if (KS <= 8)
    hipLaunchKernelGGL((k_topk_align<NS, 8>), dim3(1), dim3(1024), lds, s, part, KS, T, E, bias, k, renormalize,
                       logits_out, ids, wts, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded);
  else
    hipLaunchKernelGGL((k_topk_align<NS, 16>), dim3(1), dim3(1024), lds, s, part, KS, T, E, bias, k, renormalize,
                       logits_out, ids, wts, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded);
}

hipError_t launch_route_align(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int k,
                              int renormalize, float *logits, int32_t *ids, float *wts, float *partial, int BM,
                              int cap, int32_t *sorted_ids, int32_t *block_expert, int32_t *counts,
                              int32_t *offsets, int32_t *total_padded, int32_t *hist, hipStream_t s,
                              const XPlanes *xp) {
  if (!route_align_fused(T, E, k)) {
    hipError_t e;
    if (xp) {  // launch_route with the planes written by its router GEMM
      const int ks = router_ksplit(T, E, H);
      float *part = ks > 1 ? partial : logits;
      e = launch_router_gemm(x, T, H, w, E, bias, ks, part, xp, s);
      if (e == hipSuccess)
        e = launch_topk_ns(part, ks, T, E, ks > 1 ? bias : nullptr, k, renormalize, ks > 1 ? logits : nullptr, ids,
                           wts, s);
    } else {
      e = launch_route(x, T, H, w, E, bias, k, renormalize, logits, ids, wts, partial, s);
    }
    if (e != hipSuccess) return e;
    return launch_align(ids, T, k, E, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded, hist, s);
  }
  const int ks = router_ksplit(T, E, H);  // the router GEMM exactly as launch_route runs it
  float *part = ks > 1 ? partial : logits;
  const hipError_t e = launch_router_gemm(x, T, H, w, E, bias, ks, part, xp, s);
  if (e != hipSuccess) return e;
  const float *b = ks > 1 ? bias : nullptr;
  float *lo = ks > 1 ? logits : nullptr;
  const int slots = (E + 63) / 64;
  if (slots <= 1)
    launch_topk_align_ns<1>(part, ks, T, E, b, k, renormalize, lo, ids, wts, BM, cap, sorted_ids, block_expert, counts,
                            offsets, total_padded, s);
  else if (slots <= 2)
    launch_topk_align_ns<2>(part, ks, T, E, b, k, renormalize, lo, ids, wts, BM, cap, sorted_ids, block_expert, counts,
                            offsets, total_padded, s);
  else if (slots <= 4)
    launch_topk_align_ns<4>(part, ks, T, E, b, k, renormalize, lo, ids, wts, BM, cap, sorted_ids, block_expert, counts,
                            offsets, total_padded, s);
  else
    launch_topk_align_ns<8>(part, ks, T, E, b, k, renormalize, lo, ids, wts, BM, cap, sorted_ids, block_expert, counts,
                            offsets, total_padded, s);
  return hipGetLastError();
}

}  // namespace qmoe
