// expert.hip -- the expert layer's launch entry points (gate_up, down, the one-token down +
// combine, the MXFP4 activation split and the combine) for every format; the kernels are in
// expert_kernels.h, and the MXFP4 instantiations in expert_mxfp4.hip.
#include "expert_kernels.h"

namespace qmoe {

// x [rows, K] bf16 -> two e4m3 planes + e8m0 scales (ActMX layout).  A thread converts 8
// consecutive elements; the 4 lanes of a quad hold one 32-element block (K % 32 == 0).
__global__ __launch_bounds__(256) void k_act_mx8(const uint16_t *__restrict__ x, int rows, int K,
                                                 uint8_t *__restrict__ q, uint8_t *__restrict__ sc) {
  const size_t n8 = (size_t)rows * (K / 8);
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;  // n8 is a multiple of 4: quads leave together
  const uint4 raw = *reinterpret_cast<const uint4 *>(x + i * 8);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
  uint32_t qh[4], ql[4], s1, s2;
  mx8_split<8>(v, [](float m) { return quad_max(m); }, qh, ql, s1, s2);
  const size_t plane = (size_t)rows * K;
  *reinterpret_cast<uint2 *>(q + i * 8) = make_uint2(qh[0] | (qh[1] << 16), qh[2] | (qh[3] << 16));
  *reinterpret_cast<uint2 *>(q + plane + i * 8) = make_uint2(ql[0] | (ql[1] << 16), ql[2] | (ql[3] << 16));
  if ((i & 3) == 0) {
    sc[i / 4] = (uint8_t)s1;
    sc[plane / 32 + i / 4] = (uint8_t)s2;
  }
}

hipError_t launch_gate_up(int fmt, const GateUpArgs &a, int n_shared_sub, hipStream_t s) {
  switch (fmt) {
    case MOE_FMT_NVFP4: launch_gate_up_grid<MOE_FMT_NVFP4>(a, n_shared_sub, s); break;
    case MOE_FMT_MXFP4_E8M0: launch_gate_up_mxfp4(a, n_shared_sub, s); break;
    case MOE_FMT_BF16: launch_gate_up_grid<MOE_FMT_BF16>(a, n_shared_sub, s); break;
    case MOE_FMT_Q4_0: launch_gate_up_grid<MOE_FMT_Q4_0>(a, n_shared_sub, s); break;
    default: launch_gate_up_grid<MOE_FMT_FP8_BLOCK128>(a, n_shared_sub, s); break;
  }
  return hipGetLastError();
}

// Where the one-token kernel measured faster than down + combine (MI355X, steps of 200): fp8-block
// 24.7 -> 22.2 us, bf16 28.2 -> 26.0, MXFP4 (slice 1024) 40.8 -> 40.3, NVFP4 and q4_0 on a 256
// slice 24.5 -> 24.1 and 24.9 -> 24.5.  NVFP4 and q4_0 runs longer than two K steps do not fit
// the 128 registers of a 1024-thread workgroup (NVFP4 at slice 512: 27.0 -> 29.0 us), so they
// keep the two kernels.
bool down_t1_fused(int fmt, const DownArgs &a, int has_shared) {
  const int kph = fmt == MOE_FMT_Q4_0 ? a.lo & 127 : 0;
  const int steps = (a.Il + kph + 127) / 128;
  const bool fits = !(fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_Q4_0) || steps <= 2;
  return a.T == 1 && a.k <= 15 && a.n_routed_sub + (has_shared ? 1 : 0) <= 16 && fits;
}

hipError_t launch_down_t1(int fmt, const DownArgs &a, const float *topk_w, void *out, int out_bf16, hipStream_t s) {
  switch (fmt) {
    case MOE_FMT_NVFP4: launch_down_t1_fmt<MOE_FMT_NVFP4>(a, topk_w, out, out_bf16, s); break;
    case MOE_FMT_MXFP4_E8M0: launch_down_t1_mxfp4(a, topk_w, out, out_bf16, s); break;
    case MOE_FMT_BF16: launch_down_t1_fmt<MOE_FMT_BF16>(a, topk_w, out, out_bf16, s); break;
    case MOE_FMT_Q4_0: launch_down_t1_fmt<MOE_FMT_Q4_0>(a, topk_w, out, out_bf16, s); break;
    default: launch_down_t1_fmt<MOE_FMT_FP8_BLOCK128>(a, topk_w, out, out_bf16, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(int fmt, const DownArgs &a, int n_shared_sub, hipStream_t s) {
  const int nsub = a.n_routed_sub + n_shared_sub, ncol = (a.H + 64 * DNT - 1) / (64 * DNT);
  const dim3 grid = a.cols_fastest ? dim3(ncol, nsub) : dim3(nsub, ncol);
  switch (fmt) {
    case MOE_FMT_NVFP4: launch_down_fmt<MOE_FMT_NVFP4>(a, grid, s); break;
    case MOE_FMT_MXFP4_E8M0: launch_down_mxfp4(a, grid, s); break;
    case MOE_FMT_BF16: launch_down_fmt<MOE_FMT_BF16>(a, grid, s); break;
    case MOE_FMT_Q4_0: launch_down_fmt<MOE_FMT_Q4_0>(a, grid, s); break;
    default: launch_down_fmt<MOE_FMT_FP8_BLOCK128>(a, grid, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_act_mx8(const uint16_t *x, int rows, int K, uint8_t *q, uint8_t *sc, hipStream_t s) {
  const size_t n8 = (size_t)rows * (K / 8);
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_act_mx8, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, rows, K, q, sc);
  return hipGetLastError();
}

hipError_t launch_combine(const void *Y, bool y_bf16, const float *topk_w, int T, int k, int H, int has_shared,
                          void *out, int out_bf16, hipStream_t s) {
  dim3 grid((H / (y_bf16 ? 8 : 4) + 255) / 256, T);
  if (y_bf16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, Y, topk_w, T, k, H, has_shared, out, out_bf16);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, Y, topk_w, T, k, H, has_shared, out, out_bf16);
  return hipGetLastError();
}

}  // namespace qmoe
