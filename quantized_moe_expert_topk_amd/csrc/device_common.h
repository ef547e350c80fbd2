// device_common.h -- gfx950 building blocks shared by the routing, alignment and expert
// kernels: vector types, the bf16 MFMA, and in-register weight decoders.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64, lane l, i = 0..7, j = 0..3):
//   A (16x32, M x K): lane l holds A[l % 16][8 * (l / 16) + i]
//   B (32x16, K x N): lane l holds B[8 * (l / 16) + i][l % 16]
//   D (16x16, M x N): lane l holds D[4 * (l / 16) + j][l % 16]
// A contraction does not care which K index a (lane group, i) slot carries as long as A
// and B agree, so the kernels hand each lane group a contiguous run of K and load it with
// wide vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

union frag8 {  // 8 bf16 = 4 dwords = one MFMA operand slot of one lane
  bf16x8_t v;
  bf16x2_t h[4];
  uint32_t u[4];
  uint4 q;
};

__device__ __forceinline__ f32x4_t mfma_bf16(const frag8 &a, const frag8 &b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16 (wave64, lane l, h = l / 32, i = 0..7, j = 0..15), as measured:
//   A (32x16): lane l holds A[l % 32][8 h + i];  B (16x32): lane l holds B[8 h + i][l % 32]
//   D (32x32): lane l register j holds D[8 (j / 4) + 4 h + j % 4][l % 32]
// One wave issuing these back to back keeps the matrix core near its peak, which the
// 16x16x32 form does not reach with a single wave per SIMD.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32_bf16(const frag8 &a, const frag8 &b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x2_t pack_bf16(float a, float b) {  // round to nearest even
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}

__device__ __forceinline__ uint16_t bf16_bits(float a) {
  __bf16 h = (__bf16)a;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// e4m3fn byte -> f32 (gfx950 decodes the OCP E4M3 encoding natively).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)(byte & 0xFFu), 0);
}

// e8m0 byte (1..254) -> the f32 2^(b-127); the conversion instructions use only the
// exponent field of their f32 scale operand.
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) { return __uint_as_float((byte & 0xFFu) << 23); }

// 8 e2m1 codes (dword; element i in nibble i, low nibble first) -> 8 bf16 of code * s.
// The e2m1 -> f32 conversion is exact; e2m1 * e4m3 has at most 6 significant bits, so the
// product and its bf16 rounding are exact.
__device__ __forceinline__ void fp4x8_mul_to_bf16(uint32_t codes, float s, frag8 &out) {
  f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  out.h[0] = pack_bf16(p0[0] * s, p0[1] * s);
  out.h[1] = pack_bf16(p1[0] * s, p1[1] * s);
  out.h[2] = pack_bf16(p2[0] * s, p2[1] * s);
  out.h[3] = pack_bf16(p3[0] * s, p3[1] * s);
}

// 8 e2m1 codes -> 8 bf16 of code * 2^x, where pow2 is the f32 2^x (MXFP4 e8m0 scale).
__device__ __forceinline__ void fp4x8_pow2_to_bf16(uint32_t codes, float pow2, frag8 &out) {
  out.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 0);
  out.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 1);
  out.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 2);
  out.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 3);
}

// Q4_0 codes of 8 elements (one dword: element 2i in bits [4i, 4i+4), element 2i+1 in bits
// [16+4i, 20+4i)) -> 8 bf16 of 128 + q.  0x4300 is bf16 128, whose last mantissa bit is
// worth 1, so or-ing a 4-bit code into the mantissa adds it exactly.
__device__ __forceinline__ void q4x8_to_bf16_biased(uint32_t d, frag8 &out) {
  out.u[0] = (d & 0x000F000Fu) | 0x43004300u;
  out.u[1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
  out.u[2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
  out.u[3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// 8 e4m3 codes (two dwords, element i in byte i) -> 8 bf16 (exact).
__device__ __forceinline__ void fp8x8_to_bf16(uint32_t lo, uint32_t hi, frag8 &out) {
  out.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  out.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  out.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  out.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
}

// Buffer resources (wave-uniform, in SGPRs): loads take a 32-bit byte offset, fold
// constant offsets into the instruction, and return 0 past `bytes` (hardware range check).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Callers pass values that are the same in every lane; readfirstlane states that to the
// compiler so the descriptor is built in SGPRs.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// NT: the non-temporal hint, for bytes read once (streamed expert weights), so that they do
// not push reused lines (activation rows, scales) out of the caches.
template <bool NT>
__device__ __forceinline__ uint4 buf_load16w(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? 2 : 0));
}

__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ---------------------------------------------------------------------------- weights

// One expert's weight matrix [rows, K] (K = row width in elements) as buffer resources.
template <int FMT>
struct WMat {
  rsrc_t codes, scales;
  int K;
};

template <int FMT>
__device__ __forceinline__ WMat<FMT> weight_matrix(const uint8_t *codes, const uint8_t *scales, int e, int rows,
                                                   int K) {
  WMat<FMT> m;
  m.K = K;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    m.codes = make_rsrc(codes + (size_t)e * rows * (K / 2), (uint32_t)rows * (K / 2));
    m.scales = make_rsrc(scales + (size_t)e * rows * (K / 16), (uint32_t)rows * (K / 16));
  } else if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    m.codes = make_rsrc(codes + (size_t)e * rows * (K / 2), (uint32_t)rows * (K / 2));
    m.scales = make_rsrc(scales + (size_t)e * rows * (K / 32), (uint32_t)rows * (K / 32));
  } else if constexpr (FMT == MOE_FMT_Q4_0) {  // fp16 scale per 32 elements
    m.codes = make_rsrc(codes + (size_t)e * rows * (K / 2), (uint32_t)rows * (K / 2));
    m.scales = make_rsrc(scales + (size_t)e * rows * (K / 16), (uint32_t)rows * (K / 16));
  } else if constexpr (FMT == MOE_FMT_BF16) {
    m.codes = make_rsrc(codes + (size_t)e * rows * K * 2, (uint32_t)rows * K * 2);
    m.scales = m.codes;  // unused
  } else {
    m.codes = make_rsrc(codes + (size_t)e * rows * K, (uint32_t)rows * K);
    m.scales = make_rsrc(scales + (size_t)e * (rows / 128) * (K / 128) * 4, (uint32_t)(rows / 128) * (K / 128) * 4);
  }
  return m;
}

__device__ __forceinline__ void zero_frags(frag8 (&b)[4]) {
#pragma unroll
  for (int q = 0; q < 4; q++) b[q].q = make_uint4(0, 0, 0, 0);
}

// Wave-wide helpers (wave64).
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// ---------------------------------------------------------------------------- scaled FP4 MFMA
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = fp8 e4m3 (cbsz 0) and B = fp4 e2m1 (blgp 4),
// operand layouts as measured on gfx950 (wave64, lane l, g = l / 16):
//   A (16 x 128): lane l holds row l % 16; bytes 0..15 are K [16g, 16g+16) and bytes
//                 16..31 are K [64+16g, 64+16g+16)
//   B (128 x 16): lane l holds column l % 16, K [32g, 32g+32) as 32 nibbles (low nibble
//                 first) in the first 4 dwords
//   scales:       byte 0 of lane l's scale operand is the e8m0 scale of row (A) or
//                 column (B) l % 16 over the 32-wide K block g
//   D:            as the bf16 MFMA (lane l holds D[4g + j][l % 16])
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

__device__ __forceinline__ f32x4_t mfma_scale_e4m3_e2m1(const uint4 &a0, const uint4 &a1, const uint4 &b, uint32_t sa,
                                                        uint32_t sb, f32x4_t c) {
  const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, (int)sa, 0, (int)sb);
}

// Two f32 -> two e4m3 bytes (round to nearest even; inputs clamped to the format's +-448).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// e8m0 block scale for values of magnitude up to amax: the smallest power of two X with
// amax / X <= 448 (e4m3's largest finite value), so that the top binade of the block uses
// all of e4m3's precision and nothing saturates; at least 2^-126 so that X is a normal f32.
// Returns the byte e (X = 2^(e-127)).
__device__ __forceinline__ uint32_t e8m0_for_amax(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int eb = (int)((b >> 23) & 0xFFu);                        // biased exponent of amax
  const int e = eb - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);   // mantissa above 1.75 -> next binade
  return (uint32_t)max(e, 1);
}
__device__ __forceinline__ float e8m0_inv(uint32_t e) { return __uint_as_float((254u - e) << 23); }

// Wave-internal max over the 16 lanes of each row (lanes 16q .. 16q+15) and over quads.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));  // quad_perm [1,0,3,2]
  return fmaxf(v, dpp_f32<0x4E>(v));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}

// Split values into two e4m3 planes with one e8m0 scale each for their 32-element block:
//   hi = e4m3(v / X1) * X1,  lo = e4m3((v - hi) / X2) * X2
// amax_fn reduces a magnitude over the lanes that share the block.  Returns the plane
// bytes of NV values (NV = 2: 16 bits per plane) and the two scale bytes.
template <int NV, typename AmaxFn>
__device__ __forceinline__ void mx8_split(const float (&v)[NV], AmaxFn amax_fn, uint32_t (&qhi)[NV / 2],
                                          uint32_t (&qlo)[NV / 2], uint32_t &s1, uint32_t &s2) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NV; i++) m = fmaxf(m, fabsf(v[i]));
  s1 = e8m0_for_amax(amax_fn(m));
  const float inv1 = e8m0_inv(s1), x1 = __uint_as_float(s1 << 23);
  float res[NV];
  float m2 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; i += 2) {
    const uint32_t q = e4m3x2(v[i] * inv1, v[i + 1] * inv1);
    qhi[i / 2] = q;
    res[i] = v[i] - e4m3_to_f32(q) * x1;
    res[i + 1] = v[i + 1] - e4m3_to_f32(q >> 8) * x1;
    m2 = fmaxf(m2, fmaxf(fabsf(res[i]), fabsf(res[i + 1])));
  }
  s2 = e8m0_for_amax(amax_fn(m2));
  const float inv2 = e8m0_inv(s2);
#pragma unroll
  for (int i = 0; i < NV; i += 2) qlo[i / 2] = e4m3x2(res[i] * inv2, res[i + 1] * inv2);
}
