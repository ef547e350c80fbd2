// route.hip -- replicated router and top-k selection for gfx950.
//
// logits[t, e] = sum_h x[t, h] W[e, h] + bias[e] on bf16 MFMA with fp32 accumulation,
// then per token the k experts ranking first under (logit descending, index ascending)
// and their softmax weights (renormalised over the k picks when norm_topk_prob is set:
// FreeToken issue #62, second comment; PR #70 ownership table, "Router ... Replicated").
#include "device_common.h"
#include "launch.h"

namespace qmoe {

// One workgroup = 4 waves = 16 tokens x 64 experts; wave w owns experts [16w, 16w+16).
// K advances 128 per step: lane group g = l/16 loads the contiguous 32-element run
// [kc + 32g, kc + 32g + 32) of its row for both operands (64 B per lane per operand).
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t *__restrict__ x, int T, int H,
                                                       const uint16_t *__restrict__ w, int E,
                                                       const float *__restrict__ bias,
                                                       float *__restrict__ logits) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.y * 16, e0 = blockIdx.x * 64 + wave * 16;
  if (e0 >= E) return;
  const int ta = t0 + r, eb = e0 + r;
  const bool va = ta < T, vb = eb < E;
  const uint4 *xa = reinterpret_cast<const uint4 *>(x + (size_t)(va ? ta : 0) * H);
  const uint4 *wb = reinterpret_cast<const uint4 *>(w + (size_t)(vb ? eb : 0) * H);
  f32x4_t acc = zero4();
  for (int kc = 0; kc < H; kc += 128) {
    const int q = (kc + 32 * g) >> 3;  // uint4 index (8 bf16 each)
    frag8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      a[s].q = va ? xa[q + s] : make_uint4(0, 0, 0, 0);
      b[s].q = vb ? wb[q + s] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; s++) acc = mfma_bf16(a[s], b[s], acc);
  }
  if (vb) {
    const float bv = bias ? bias[eb] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int t = t0 + 4 * g + j;
      if (t < T) logits[(size_t)t * E + eb] = acc[j] + bv;
    }
  }
}

// Top-k: one wave per token.  Lane l holds experts e = l + 64 q.  Each of the k rounds
// takes the wave-wide best (value, then lower index) among the not-yet-taken experts.
constexpr int kMaxSlots = 16;  // E <= 1024

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E,
                                              const float *__restrict__ bias, int k, int renormalize,
                                              int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nslot = (E + 63) >> 6;
  float v[kMaxSlots];
#pragma unroll
  for (int q = 0; q < kMaxSlots; q++) {
    const int e = lane + 64 * q;
    v[q] = (q < nslot && e < E) ? logits[(size_t)t * E + e] + (bias ? bias[e] : 0.f) : -INFINITY;
    if (v[q] != v[q]) v[q] = -INFINITY;  // a NaN logit ranks last (selection stays in range)
  }
  uint32_t taken = 0;
  float mine = 0.f;  // lane j < k keeps the j-th selected logit
  float top = 0.f;
  for (int j = 0; j < k; j++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kMaxSlots; q++) {
      const int e = lane + 64 * q;
      if (q < nslot && e < E && !(taken >> q & 1u) && better(v[q], e, bv, bi)) {
        bv = v[q];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) mine = bv;
    if (j == 0) top = bv;
    if (lane == 0) ids[(size_t)t * k + j] = bi;
  }
  // softmax weights
  float z;
  if (renormalize) {
    z = lane < k ? expf(mine - top) : 0.f;
  } else {
    z = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSlots; q++)
      if (q < nslot && lane + 64 * q < E) z += expf(v[q] - top);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  if (lane < k) wts[(size_t)t * k + lane] = expf(mine - top) / z;
}

hipError_t launch_router_logits(const uint16_t *x, int T, int H, const uint16_t *w, int E,
                                const float *bias, float *logits, hipStream_t s) {
  dim3 grid((E + 63) / 64, (T + 15) / 16);
  hipLaunchKernelGGL(k_router_logits, grid, dim3(256), 0, s, x, T, H, w, E, bias, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int E, const float *bias, int k, int renormalize,
                       int32_t *ids, float *wts, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, bias, k, renormalize,
                     ids, wts);
  return hipGetLastError();
}

}  // namespace qmoe
