// expert.hip -- quantized SwiGLU expert layer on an intermediate slice [lo, lo + Il) for gfx950.
//
// gate_up: for every row of the aligned pair list (and every token for the shared expert)
//   g_i = x . Wg[lo+i],  u_i = x . Wu[I+lo+i],  h_i = silu(g_i) * u_i  (bf16)
// down:    y_n = sum_i h_i Wd[n, lo+i], scaled by the routing weight and written per pair
// combine: out[t] = sum_j Y[t*k+j] + Y_shared[t]  (fixed order, deterministic)
// The slice geometry is the pages' (gate rows [lo,hi), up rows [I+lo, I+hi), down columns
// [lo,hi): FreeToken issue #62 "What it touches" item 1), and so is the math (issue #520
// section 4 "Expert sharding": silu(gate)*up @ down, linear in the intermediate index).
//
// Weights are dequantized in registers to bf16 and fed to v_mfma_f32_16x16x32_bf16 (W4A16
// for the FP4 formats, W8A16 for fp8-block):
//   NVFP4      e2m1 * e4m3 group scale (exact in bf16); the fp32 per-row global is applied
//              to the fp32 accumulator in the epilogue.
//   MXFP4      e2m1 * 2^(e8m0-127) by the scaled conversion instruction (exact).
//   FP8_BLOCK  e4m3 -> bf16 exact; the fp32 128x128 block scale multiplies each 128-wide
//              K chunk's partial sum.
//
// Tiling: a workgroup is 4 waves and covers 16 rows of the pair list x 64 output columns;
// wave w owns columns [16w, 16w+16) and runs the whole K loop.  K advances 128 per step;
// lane group g = l/16 reads the contiguous K run [kc+32g, kc+32g+32) of its row of both
// operands (the MFMA slots of A and B carry the same K indices).
#include "device_common.h"
#include "launch.h"

namespace qmoe {

// ---------------------------------------------------------------------------- B operand

// Load + dequantize the 32-element K run [k0, k0+32) of one weight row into 4 fragments
// (fragment s = K [k0+8s, k0+8s+8)).  `row` is the row index inside the expert's matrix,
// `K` the matrix width (elements).  For FP8_BLOCK the block scale is applied by the caller.
template <int FMT>
__device__ __forceinline__ void load_b(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                       size_t row, int K, int k0, frag8 (&b)[4]) {
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const uint4 c = *reinterpret_cast<const uint4 *>(codes + row * (size_t)(K / 2) + k0 / 2);
    const uint8_t *sp = scales + row * (size_t)(K / 16) + k0 / 16;
    const float s0 = e4m3_to_f32(sp[0]), s1 = e4m3_to_f32(sp[1]);
    fp4x8_mul_to_bf16(c.x, s0, b[0]);
    fp4x8_mul_to_bf16(c.y, s0, b[1]);
    fp4x8_mul_to_bf16(c.z, s1, b[2]);
    fp4x8_mul_to_bf16(c.w, s1, b[3]);
  } else if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    const uint4 c = *reinterpret_cast<const uint4 *>(codes + row * (size_t)(K / 2) + k0 / 2);
    const float p = e8m0_to_f32(scales[row * (size_t)(K / 32) + k0 / 32]);
    fp4x8_pow2_to_bf16(c.x, p, b[0]);
    fp4x8_pow2_to_bf16(c.y, p, b[1]);
    fp4x8_pow2_to_bf16(c.z, p, b[2]);
    fp4x8_pow2_to_bf16(c.w, p, b[3]);
  } else {
    const uint4 *cp = reinterpret_cast<const uint4 *>(codes + row * (size_t)K + k0);
    const uint4 c0 = cp[0], c1 = cp[1];
    fp8x8_to_bf16(c0.x, c0.y, b[0]);
    fp8x8_to_bf16(c0.z, c0.w, b[1]);
    fp8x8_to_bf16(c1.x, c1.y, b[2]);
    fp8x8_to_bf16(c1.z, c1.w, b[3]);
  }
}

__device__ __forceinline__ void load_a(const uint16_t *__restrict__ rowp, int k0, bool valid, frag8 (&a)[4]) {
  const uint4 *p = reinterpret_cast<const uint4 *>(rowp + k0);
#pragma unroll
  for (int s = 0; s < 4; s++) a[s].q = valid ? p[s] : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------- gate_up

template <int FMT>
__global__ __launch_bounds__(256) void k_gate_up(GateUpArgs a) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int sb = blockIdx.x;
  const int c0 = blockIdx.y * 64 + wave * 16;  // first slice column of this wave
  if (c0 >= a.Il) return;
  const bool is_shared = sb >= a.n_routed_sub;
  int p0, e, tok;
  const uint8_t *codes;
  const uint8_t *scales;
  const float *glob;
  if (!is_shared) {
    p0 = sb * 16;
    if (p0 >= a.total_padded[0]) return;
    e = a.block_expert[p0 / a.block_m];
    if (e < 0) return;
    const int f = a.sorted_ids[p0 + r];
    tok = f < a.T * a.k ? f / a.k : -1;
    codes = a.gu;
    scales = a.gus;
    glob = a.gug;
  } else {
    const int t0 = (sb - a.n_routed_sub) * 16;
    p0 = a.cap + t0;
    e = 0;
    tok = t0 + r < a.T ? t0 + r : -1;
    codes = a.sgu;
    scales = a.sgus;
    glob = a.sgug;
  }
  const int H = a.H, I = a.I;
  const size_t gate_row = (size_t)e * 2 * I + a.lo + c0 + r;  // row inside the bank's [E*2I] rows
  const size_t up_row = gate_row + I;
  const uint16_t *xrow = a.x + (size_t)(tok >= 0 ? tok : 0) * H;
  f32x4_t accg = zero4(), accu = zero4();
  for (int kc = 0; kc < H; kc += 128) {
    const int k0 = kc + 32 * g;
    frag8 av[4], bg[4], bu[4];
    load_a(xrow, k0, tok >= 0, av);
    load_b<FMT>(codes, scales, gate_row, H, k0, bg);
    load_b<FMT>(codes, scales, up_row, H, k0, bu);
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
      // block scale of rows [row/128] and K block kc/128 (uniform over the wave)
      const float *si = reinterpret_cast<const float *>(scales);
      const float sg = si[(gate_row / 128) * (size_t)(H / 128) + kc / 128];
      const float su = si[(up_row / 128) * (size_t)(H / 128) + kc / 128];
      f32x4_t tg = zero4(), tu = zero4();
#pragma unroll
      for (int s = 0; s < 4; s++) {
        tg = mfma_bf16(av[s], bg[s], tg);
        tu = mfma_bf16(av[s], bu[s], tu);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        accg[j] += sg * tg[j];
        accu[j] += su * tu[j];
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; s++) {
        accg = mfma_bf16(av[s], bg[s], accg);
        accu = mfma_bf16(av[s], bu[s], accu);
      }
    }
  }
  float gsc = 1.f, usc = 1.f;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    gsc = glob[gate_row];
    usc = glob[up_row];
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float gv = accg[j] * gsc, uv = accu[j] * usc;
    const float hv = gv / (1.f + __expf(-gv)) * uv;
    a.h[(size_t)(p0 + 4 * g + j) * a.Il + c0 + r] = bf16_bits(hv);
  }
}

// ---------------------------------------------------------------------------- down

template <int FMT>
__global__ __launch_bounds__(256) void k_down(DownArgs a) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int sb = blockIdx.x;
  const int n0 = blockIdx.y * 64 + wave * 16;  // first output column (hidden index)
  if (n0 >= a.H) return;
  const bool is_shared = sb >= a.n_routed_sub;
  int p0, e;
  const uint8_t *codes;
  const uint8_t *scales;
  const float *glob;
  if (!is_shared) {
    p0 = sb * 16;
    if (p0 >= a.total_padded[0]) return;
    e = a.block_expert[p0 / a.block_m];
    if (e < 0) return;
    codes = a.dn;
    scales = a.dns;
    glob = a.dng;
  } else {
    p0 = a.cap + (sb - a.n_routed_sub) * 16;
    e = 0;
    codes = a.sdn;
    scales = a.sdns;
    glob = a.sdng;
  }
  const int H = a.H, I = a.I, Il = a.Il;
  const size_t drow = (size_t)e * H + n0 + r;  // down row of output column n0 + r
  const uint16_t *hrow = a.h + (size_t)(p0 + r) * Il;
  f32x4_t acc = zero4();
  for (int kc = 0; kc < Il; kc += 128) {
    const int k0 = kc + 32 * g;
    const bool valid = k0 < Il;  // Il % 32 == 0: a lane group's run is all in or all out
    frag8 av[4], bv[4];
    load_a(hrow, k0, valid, av);
    if (valid) {
      load_b<FMT>(codes, scales, drow, I, a.lo + k0, bv);
    } else {
#pragma unroll
      for (int s = 0; s < 4; s++) bv[s].q = make_uint4(0, 0, 0, 0);
    }
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
      const float *si = reinterpret_cast<const float *>(scales);
      const float sc = si[(drow / 128) * (size_t)(I / 128) + (a.lo + kc) / 128];
      f32x4_t t = zero4();
#pragma unroll
      for (int s = 0; s < 4; s++) t = mfma_bf16(av[s], bv[s], t);
#pragma unroll
      for (int j = 0; j < 4; j++) acc[j] += sc * t[j];
    } else {
#pragma unroll
      for (int s = 0; s < 4; s++) acc = mfma_bf16(av[s], bv[s], acc);
    }
  }
  float dsc = 1.f;
  if constexpr (FMT == MOE_FMT_NVFP4) dsc = glob[drow];
  const int P = a.T * a.k;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int p = p0 + 4 * g + j;
    const float y = acc[j] * dsc;
    if (!is_shared) {
      const int f = a.sorted_ids[p];
      if (f < P) a.Y[(size_t)f * H + n0 + r] = a.topk_w[f] * y;
    } else {
      const int t = p - a.cap;
      if (t < a.T) a.Y[(size_t)(P + t) * H + n0 + r] = y;
    }
  }
}

// ---------------------------------------------------------------------------- combine

__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ Y, int T, int k, int H, int has_shared,
                                                 void *__restrict__ out, int out_bf16) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; j++) {
    const float4 v = *reinterpret_cast<const float4 *>(Y + (size_t)(t * k + j) * H + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (has_shared) {
    const float4 v = *reinterpret_cast<const float4 *>(Y + (size_t)(T * k + t) * H + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (out_bf16) {
    uint16_t *o = reinterpret_cast<uint16_t *>(out) + (size_t)t * H + n;
    uint2 pk;
    pk.x = (uint32_t)bf16_bits(acc.x) | ((uint32_t)bf16_bits(acc.y) << 16);
    pk.y = (uint32_t)bf16_bits(acc.z) | ((uint32_t)bf16_bits(acc.w) << 16);
    *reinterpret_cast<uint2 *>(o) = pk;
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (size_t)t * H + n) = acc;
  }
}

// ---------------------------------------------------------------------------- launchers

hipError_t launch_gate_up(int fmt, const GateUpArgs &a, int n_shared_sub, hipStream_t s) {
  dim3 grid(a.n_routed_sub + n_shared_sub, (a.Il + 63) / 64);
  switch (fmt) {
    case MOE_FMT_NVFP4: hipLaunchKernelGGL(k_gate_up<MOE_FMT_NVFP4>, grid, dim3(256), 0, s, a); break;
    case MOE_FMT_MXFP4_E8M0: hipLaunchKernelGGL(k_gate_up<MOE_FMT_MXFP4_E8M0>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_gate_up<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(int fmt, const DownArgs &a, int n_shared_sub, hipStream_t s) {
  dim3 grid(a.n_routed_sub + n_shared_sub, (a.H + 63) / 64);
  switch (fmt) {
    case MOE_FMT_NVFP4: hipLaunchKernelGGL(k_down<MOE_FMT_NVFP4>, grid, dim3(256), 0, s, a); break;
    case MOE_FMT_MXFP4_E8M0: hipLaunchKernelGGL(k_down<MOE_FMT_MXFP4_E8M0>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_down<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const float *Y, int T, int k, int H, int has_shared, void *out, int out_bf16,
                          hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, Y, T, k, H, has_shared, out, out_bf16);
  return hipGetLastError();
}

}  // namespace qmoe
