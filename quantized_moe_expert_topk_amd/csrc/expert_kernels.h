// expert_kernels.h -- the expert kernels (templates) and their launch helpers, included by
// expert.hip (every format but MXFP4, and the dispatch of every format) and by expert_mxfp4.hip
// (the MXFP4 instantiations, compiled with their own scheduling options).  What the kernels
// compute, their tiling and their number formats are described below.
//
// The quantized SwiGLU expert layer on an intermediate slice [lo, lo + Il), gfx950.
//
// gate_up: for every row of the aligned pair list (and every token for the shared expert)
//   g_i = x . Wg[lo+i],  u_i = x . Wu[I+lo+i],  h_i = silu(g_i) * u_i  (bf16)
// down:    y_n = sum_i h_i Wd[n, lo+i], written per pair
// combine: out[t] = sum_j topk_w[t,j] Y[t*k+j] + Y_shared[t]  (fixed order, deterministic; the
//          routing weight is applied here, where it is a direct load, not in down, where it
//          would be a load through sorted_ids behind another load)
// The slice geometry is the pages' (gate rows [lo,hi), up rows [I+lo, I+hi), down columns
// [lo,hi): FreeToken issue #62 "What it touches" item 1), and so is the math (issue #520
// section 4 "Expert sharding": silu(gate)*up @ down, linear in the intermediate index).
//
// NVFP4 and fp8-block weights are dequantized in registers and fed to the 16x16x32 MFMA
// (W4A16 / W8A16):
//   NVFP4      e2m1 * e4m3 group scale has at most 6 significant bits: exact in bf16, so the
//              bf16 activations meet exact weights in v_mfma_f32_16x16x32_bf16 (W4A16, fp32
//              accumulation); the fp32 per-row global is applied in the epilogue.
//   FP8_BLOCK  e4m3 -> bf16 exact; the fp32 128x128 block scale multiplies each 128-wide
//              K chunk's partial sum.
//   BF16       used as stored.
//   Q4_0       codes -> bf16 128 + q exactly; the -136 offset and the fp16 block scale are
//              applied per 32-wide block to the fp32 MFMA results (mma_run).
// MXFP4 (e8m0 per 32) runs on the native scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4: the
// raw e2m1 codes and e8m0 bytes are the B operand and its scales, with no dequantization.
// Its A operand cannot be 16-bit, so x (and h) are carried as two e4m3 planes with e8m0
// block scales, hi = e4m3(v/X1)*X1 and lo = e4m3((v-hi)/X2)*X2 (about 8 significant bits,
// the precision of bf16), and each chunk takes one MFMA per plane.
//
// Tiling: a workgroup is 4 waves over 16 rows of the pair list (one aligned sub-block of a
// single expert).  gate_up: 32 slice columns of gate and of up (4 MFMA tiles), K split over
// the 4 waves and reduced through LDS.  down: each wave owns 4 x 16 hidden columns over the
// whole slice.  K advances in 128-wide chunks: lane group g = l/16 reads the run
// [kc+32g, kc+32g+32) of its row of both operands (FP4; the MFMA slots of A and B carry the
// same K indices).  The weights are in the tile-16 layout (MOE_LAYOUT_TILE16), so one wave
// load of a tile is a contiguous 1 KB run already in operand order.  A wave issues the
// loads of 2 chunks before decoding either of them, so the weight bytes are in flight while
// the VALU dequantizes.
#pragma once

#include "device_common.h"
#include "launch.h"
#include "route_align_dev.h"

namespace qmoe {

// Scale run of one lane: NB consecutive scale bytes starting at byte `off` (any
// alignment), gathered with dword loads and funnel shifts.  Bytes past the resource read
// as 0 (buffer range check).
template <int NB>
struct ScaleRun {
  uint32_t w[(NB + 3) / 4];
};

template <int NB>
__device__ __forceinline__ void load_scale_run(rsrc_t r, uint32_t off, ScaleRun<NB> &s) {
  if constexpr (NB == 1) {
    s.w[0] = buf_load1(r, off);
  } else if constexpr (NB == 2) {
    s.w[0] = buf_load2(r, off);  // NVFP4 runs start at even bytes
  } else {
    constexpr int ND = NB / 4 + 1;  // dwords covering NB bytes at any alignment
    const uint32_t base = off & ~3u, sh = (off & 3u) * 8;
    uint32_t d[ND + (ND & 1)];
    if constexpr (ND == 2) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)base, 0, 0));
      d[0] = v.x;
      d[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < ND; q += 4) {
        const uint4 v = buf_load16(r, base + 4 * q);
        d[q] = v.x;
        if (q + 1 < ND) d[q + 1] = v.y;
        if (q + 2 < ND) d[q + 2] = v.z;
        if (q + 3 < ND) d[q + 3] = v.w;
      }
    }
#pragma unroll
    for (int q = 0; q < NB / 4; q++) s.w[q] = __builtin_amdgcn_alignbit(d[q + 1], d[q], sh);
  }
}

template <int NB>
__device__ __forceinline__ uint32_t run_byte(const ScaleRun<NB> &s, int i) {  // i: compile-time after unrolling
  return (s.w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

struct ARaw {
  uint4 q[4];  // 32 bf16 = one 32-wide K piece of one activation row
};

// Dequantize a 32-wide piece to 4 bf16 fragments (fragment s = K [8s, 8s+8) of the piece).
//   NVFP4: codes c (32 nibbles), e4m3 scales s0 (first 16) and s1 (last 16)
__device__ __forceinline__ void decode_nvfp4(const uint4 &c, uint32_t s0, uint32_t s1, frag8 (&b)[4]) {
  const float f0 = e4m3_to_f32(s0), f1 = e4m3_to_f32(s1);
  fp4x8_mul_to_bf16(c.x, f0, b[0]);
  fp4x8_mul_to_bf16(c.y, f0, b[1]);
  fp4x8_mul_to_bf16(c.z, f1, b[2]);
  fp4x8_mul_to_bf16(c.w, f1, b[3]);
}

__device__ __forceinline__ void decode_mxfp4(const uint4 &c, uint32_t e8, frag8 (&b)[4]) {
  const float p = e8m0_to_f32(e8);
  fp4x8_pow2_to_bf16(c.x, p, b[0]);
  fp4x8_pow2_to_bf16(c.y, p, b[1]);
  fp4x8_pow2_to_bf16(c.z, p, b[2]);
  fp4x8_pow2_to_bf16(c.w, p, b[3]);
}

// Scale bytes of one row-major row for a group of 2 K steps (chunk mapping): NVFP4 16 bytes
// (2 steps x 4 lane groups x 2 groups of 16), MXFP4 8 bytes (2 x 4 x 1).  All four lane
// groups of a row load the same span; each lane then selects its own bytes.  Used for the
// MXFP4 activation planes, which are row-major.
template <int FMT>
__device__ __forceinline__ uint4 load_scale_span(rsrc_t r, uint32_t off, bool aligned) {
  constexpr int NB = FMT == MOE_FMT_NVFP4 ? 16 : 8;
  if (aligned) {  // uniform: a dword-aligned start for every lane
    if constexpr (NB == 16) return buf_load16(r, off);
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    return make_uint4(v.x, v.y, 0, 0);
  }
  ScaleRun<NB> run;
  load_scale_run(r, off, run);
  if constexpr (NB == 16) return make_uint4(run.w[0], run.w[1], run.w[2], run.w[3]);
  return make_uint4(run.w[0], run.w[1], 0, 0);
}

// This lane's scale bytes of step s (0/1) of a span (lane group g).
//   NVFP4: the two e4m3 bytes at 8s + 2g, 8s + 2g + 1 (low 16 bits of the result)
//   MXFP4: the e8m0 byte at 4s + g
template <int FMT>
__device__ __forceinline__ uint32_t span_scales(const uint4 &sp, int s, int g) {
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const uint32_t lo = s ? sp.z : sp.x, hi = s ? sp.w : sp.y;
    return ((g & 2) ? hi : lo) >> (16 * (g & 1));
  } else {
    return (s ? sp.y : sp.x) >> (8 * g);
  }
}

// Weight rows are stored in 16-row tiles, piece-major (MOE_LAYOUT_TILE16): piece c (16
// code bytes) of row R sits at tile_off(R) + 256 c, with tile_off(R) = (R & ~15) * P +
// (R & 15) * 16 for P code bytes per row, and the FP4 scale bytes of piece c (SP of them) at
// (R & ~15) * S + 16 SP c + (R & 15) SP for S scale bytes per row.  A wave's load of one
// piece index over the 16 rows of a tile is then one contiguous 1 KB run.
template <int FMT>
__device__ __forceinline__ uint32_t code_tile_off(uint32_t row, uint32_t K) {
  return (row & ~15u) * (FMT == MOE_FMT_BF16 ? 2 * K : FMT == MOE_FMT_FP8_BLOCK128 ? K : K / 2) + (row & 15u) * 16;
}

template <int FMT>
__device__ __forceinline__ uint32_t scale_tile_off(uint32_t row, uint32_t K) {
  constexpr uint32_t SP = FMT == MOE_FMT_NVFP4 ? 2 : 1;
  return (row & ~15u) * (K / 32) * SP + (row & 15u) * SP;
}

// Multiply-accumulate a wave's K range [kw0, kw0 + 128*COUNT) of one 16-row A block against
// NT weight tiles.  Step i is the 128-wide chunk [kw0 + 128 i, +128).  FP4: lane group
// g = l/16 takes the 32-element piece [32 g, 32 g + 32) of the step from both operands.
// FP8: lane group g takes [16 g, 16 g + 16) and [64 + 16 g, +16), so each of the two code
// loads covers 4 consecutive pieces of every tile row (one 1 KB run per tile).  BF16: MFMA q
// of the step takes [32 q, 32 q + 32), lane group g its 8 elements [32 q + 8 g, +8) (pieces
// 4q..4q+3: again one 1 KB run per tile and MFMA, no dequantization).  Q4_0: MFMA q of the
// step is block q (K [32 q, 32 q + 32)), lane group g its elements [8 g, 8 g + 8); the lane's
// one 16-byte piece (step, g) holds one dword of each of the 4 blocks.  Either way
// every MFMA stays inside one 128x128 FP8 scale block.  Positions at or past kvalid
// (relative to kw0) contribute zero and load from clamped in-bounds offsets.  Steps are
// taken in groups of 2 (FP4, Q4_0) or 1 (FP8, BF16) whose loads are all issued before decoding.
// Q4_0 keeps the weights exact in bf16 without a subtraction per weight: the codes become
// bf16 128 + q by bit operations alone, and since (q - 8) d = ((128 + q) - 136) d, block q's
// partial sum is d (x . (128 + q) - 136 sum(x)), where the second term is one MFMA of x
// against a constant -136 operand per block, shared by the NT tiles and fed in as the
// accumulator input of each tile's MFMA; d (fp16, per weight row and block) then scales the
// fp32 result.  Q4_0 steps are 128-wide and aligned to the row (b_k0 + kw0 a multiple of 128);
// a K range that starts or ends inside a step (a down slice on a multiple of 32) is given as
// QMASK with kphase, the offset of the range's first element inside its first step: the
// blocks of a step before kphase (counted from kw0 = 0) or at or past kvalid are skipped, and
// the activation row is read kphase elements later than the step offsets say.
//   ra, a_row: activation buffer and the byte offset of this lane's row; a row past the
//              buffer end reads as zeros without a memory request (padding rows)
//   m, rows:   weight matrix (tile-16 layout) and this lane's row of each tile (the NT
//              tiles start on multiples of 16);  b_k0: K offset in the row
//   lsc:       FP4 with RB = 4 * COUNT * SP a multiple of 16: this wave's LDS region of
//              NT x 16 RB bytes.  The run's scale bytes (one contiguous 16 RB-byte run per
//              tile in this layout) are fetched with 16-byte loads issued before the first
//              group's weight loads, staged there and read back per lane.  Shorter runs
//              (lsc unused) load each lane's SP scale bytes per step and tile.  Q4_0 stages
//              the same way (its 2 scale bytes per 32 elements give NVFP4's run length) and
//              reads back the 8 bytes of its row per step.
//   NTW:       weight code loads carry the non-temporal hint
template <int FMT, int NT, int COUNT, bool QMASK = false, bool NTW = false>
__device__ __forceinline__ void mma_run(rsrc_t ra, uint32_t a_row, const WMat<FMT> &m, const uint32_t (&rows)[NT],
                                        int b_k0, int kw0, int kvalid, int g, f32x4_t (&acc)[NT],
                                        uint8_t *lsc = nullptr, int kphase = 0) {
  static_assert(!QMASK || FMT == MOE_FMT_Q4_0, "block masks are for Q4_0 steps");
  constexpr bool FP4 = FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_MXFP4_E8M0;
  constexpr bool BF16 = FMT == MOE_FMT_BF16;
  constexpr bool Q4 = FMT == MOE_FMT_Q4_0;
  constexpr int NPF = (FP4 || Q4) ? 2 : 1;
  constexpr int SP = (FMT == MOE_FMT_NVFP4 || Q4) ? 2 : 1;  // scale bytes per 32 elements
  constexpr bool STAGE = FP4 || Q4;                          // formats with per-row scale runs
  const uint32_t K = (uint32_t)m.K;
  const int lane = lane_id(), r = lane & 15;
  uint32_t cb[NT], sb[NT];
#pragma unroll
  for (int t = 0; t < NT; t++) {
    cb[t] = code_tile_off<FMT>(rows[t], K);
    // Q4_0 scales: tile-16 order in units of one step's 4 fp16 (8 bytes)
    sb[t] = FP4 ? scale_tile_off<FMT>(rows[t], K) : Q4 ? (rows[t] & ~15u) * (K / 16) + (rows[t] & 15u) * 8 : 0;
  }
  constexpr int RB = STAGE ? 4 * COUNT * SP : 16;  // staged scale bytes per lane (16 lanes per tile)
  constexpr int SQ = RB / 16;
  static_assert(NT % 4 == 0, "whole tiles per 16-lane group when staging scale runs");
  constexpr int TPG = NT / 4;  // tiles whose scale runs one 16-lane group stages
  uint4 stg[TPG][SQ > 0 ? SQ : 1];
  if constexpr (STAGE && SQ > 0) {
#pragma unroll
    for (int u = 0; u < TPG; u++) {  // lanes 16t..16t+15 fetch the runs of tiles t, t + 4, ...
      const uint32_t run = (rows[(lane >> 4) + 4 * u] & ~15u) * (K / 32) * SP + ((b_k0 + kw0) / 32) * 16 * SP;
#pragma unroll
      for (int q = 0; q < SQ; q++) stg[u][q] = buf_load16(m.scales, run + r * RB + 16 * q);
    }
  }
#pragma unroll
  for (int i0 = 0; i0 < COUNT; i0 += NPF) {
    ARaw ar[NPF];
    uint4 c0[NPF][NT], c1[NPF][NT], c2[NPF][NT], c3[NPF][NT];
    uint32_t lsv[NPF][NT];
    float bs[NPF][NT];
    uint2 qsv[NPF][NT];  // Q4_0: the 4 fp16 block scales of the step
#pragma unroll
    for (int ii = 0; ii < NPF; ii++) {
      const int i = i0 + ii;
      if (i >= COUNT) break;
      if constexpr (FP4) {
        const int kr = 128 * i + 32 * g;
        const int k = kw0 + (kr < kvalid ? kr : 0);  // this lane's piece, relative to b_k0
#pragma unroll
        for (int q = 0; q < 4; q++) ar[ii].q[q] = buf_load16(ra, a_row + k * 2 + 16 * q);
        const uint32_t pc = (uint32_t)(b_k0 + k) / 32;
#pragma unroll
        for (int t = 0; t < NT; t++) c0[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + pc * 256);
        if constexpr (SQ == 0) {
#pragma unroll
          for (int t = 0; t < NT; t++)
            lsv[ii][t] = SP == 2 ? buf_load2(m.scales, sb[t] + pc * 32) : buf_load1(m.scales, sb[t] + pc * 16);
        }
      } else if constexpr (Q4) {
        const int kc = kw0 + (128 * i < kvalid ? 128 * i : 0);  // the step
#pragma unroll
        for (int q = 0; q < 4; q++) {  // blocks before kphase read element 0 (skipped below)
          const int ka = kc + 32 * q + 8 * g - kphase;
          ar[ii].q[q] = buf_load16(ra, a_row + (ka > 0 ? ka : 0) * 2);
        }
        const uint32_t st = (uint32_t)(b_k0 + kc) / 128;
#pragma unroll
        for (int t = 0; t < NT; t++) {
          c0[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + (4 * st + g) * 256);
          if constexpr (SQ == 0) qsv[ii][t] = buf_load8(m.scales, sb[t] + st * 128);
        }
      } else if constexpr (BF16) {
        const int kc = kw0 + (128 * i < kvalid ? 128 * i : 0);  // the step
#pragma unroll
        for (int q = 0; q < 4; q++) ar[ii].q[q] = buf_load16(ra, a_row + (kc + 32 * q + 8 * g) * 2);
        const uint32_t pc = (uint32_t)(b_k0 + kc) / 8 + g;
#pragma unroll
        for (int t = 0; t < NT; t++) {
          c0[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + pc * 256);
          c1[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + (pc + 4) * 256);
          c2[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + (pc + 8) * 256);
          c3[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + (pc + 12) * 256);
        }
      } else {
        const int kc = kw0 + (128 * i < kvalid ? 128 * i : 0);  // the step
#pragma unroll
        for (int q = 0; q < 4; q++)
          ar[ii].q[q] = buf_load16(ra, a_row + (kc + 16 * g + (q >= 2 ? 64 : 0)) * 2 + 16 * (q & 1));
        const uint32_t pc = (uint32_t)(b_k0 + kc) / 16 + g;
#pragma unroll
        for (int t = 0; t < NT; t++) {
          c0[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + pc * 256);
          c1[ii][t] = buf_load16w<NTW>(m.codes, cb[t] + (pc + 4) * 256);
          bs[ii][t] = buf_load_f32(m.scales, ((rows[t] / 128) * (K / 128) + (b_k0 + kw0 + 128 * i) / 128) * 4);
        }
      }
    }
    if constexpr (STAGE && SQ > 0) {
      {  // scale bytes from the wave's LDS region (staged once per run)
        {
          if (i0 == 0) {  // the first group's weight loads are in flight by now
#pragma unroll
            for (int u = 0; u < TPG; u++)
#pragma unroll
              for (int q = 0; q < SQ; q++) *reinterpret_cast<uint4 *>(lsc + (lane + 64 * u) * RB + 16 * q) = stg[u][q];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
        }
#pragma unroll
        for (int ii = 0; ii < NPF; ii++) {
          if constexpr (Q4) {  // the 4 scales of this lane's row for the step (a run of 128-byte steps)
            const int ist = 128 * (i0 + ii) < kvalid ? i0 + ii : 0;
#pragma unroll
            for (int t = 0; t < NT; t++)
              qsv[ii][t] = *reinterpret_cast<const uint2 *>(lsc + 16 * t * RB + ist * 128 + r * 8);
          } else {
            const int kr = 128 * (i0 + ii) + 32 * g;
            const int cr = (kr < kvalid ? kr : 0) / 32;  // this lane's piece within the run
#pragma unroll
            for (int t = 0; t < NT; t++) {
              const uint8_t *p = lsc + 16 * t * RB + cr * 16 * SP + r * SP;
              lsv[ii][t] = SP == 2 ? (uint32_t)*reinterpret_cast<const uint16_t *>(p) : (uint32_t)*p;
            }
          }
        }
      }
    }
    // fp8-block: raised wave priority over the step's MFMAs, as in mma_run_mx.  Measured on MI355X,
    // T = 64 slice 256: fp8-block 80.6 -> 79.4 us per step; NVFP4 62.2 -> 63.0, bf16 137.0 ->
    // 139.2 and q4_0 63.6 -> 71.0 us, whose dequantization is vector work inside the block.
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ii = 0; ii < NPF; ii++) {
      const int i = i0 + ii;
      if (i >= COUNT) break;
      const bool v0 = 128 * i + (FP4 ? 32 : 16) * g < kvalid;  // first (FP4: only) half of the lane's K
      const bool v1 = 128 * i + 64 + 16 * g < kvalid;          // FP8 second half
      frag8 av[4];
#pragma unroll
      for (int q = 0; q < 4; q++) av[q].q = ar[ii].q[q];
      if constexpr (Q4) {
        if (128 * i >= kvalid) continue;  // wave-uniform: a whole step past the range
        bool qv[4];  // wave-uniform: block q of the step lies inside the range
#pragma unroll
        for (int q = 0; q < 4; q++) qv[q] = !QMASK || (128 * i + 32 * q < kvalid && kw0 + 128 * i + 32 * q >= kphase);
        frag8 neg;  // bf16 -136 in every slot
        neg.q = make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u);
        f32x4_t ns[4];
#pragma unroll
        for (int q = 0; q < 4; q++) ns[q] = mfma_bf16(av[q], neg, zero4());
#pragma unroll
        for (int t = 0; t < NT; t++) {
          const uint32_t dw[4] = {c0[ii][t].x, c0[ii][t].y, c0[ii][t].z, c0[ii][t].w};
          const float d[4] = {f16_to_f32(qsv[ii][t].x), f16_to_f32(qsv[ii][t].x >> 16), f16_to_f32(qsv[ii][t].y),
                              f16_to_f32(qsv[ii][t].y >> 16)};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            if (!qv[q]) continue;
            frag8 bq;
            q4x8_to_bf16_biased(dw[q], bq);
            const f32x4_t tmp = mfma_bf16(av[q], bq, ns[q]);
#pragma unroll
            for (int j = 0; j < 4; j++) acc[t][j] += d[q] * tmp[j];
          }
        }
        continue;
      }
#pragma unroll
      for (int t = 0; t < NT; t++) {
        frag8 bv[4];
        if constexpr (FMT == MOE_FMT_NVFP4) {
          decode_nvfp4(c0[ii][t], lsv[ii][t] & 0xFFu, (lsv[ii][t] >> 8) & 0xFFu, bv);
        } else if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
          decode_mxfp4(c0[ii][t], lsv[ii][t] & 0xFFu, bv);
        } else if constexpr (BF16) {
          bv[0].q = c0[ii][t];
          bv[1].q = c1[ii][t];
          bv[2].q = c2[ii][t];
          bv[3].q = c3[ii][t];
        } else {
          fp8x8_to_bf16(c0[ii][t].x, c0[ii][t].y, bv[0]);
          fp8x8_to_bf16(c0[ii][t].z, c0[ii][t].w, bv[1]);
          fp8x8_to_bf16(c1[ii][t].x, c1[ii][t].y, bv[2]);
          fp8x8_to_bf16(c1[ii][t].z, c1[ii][t].w, bv[3]);
        }
        if constexpr (FP4) {
          if (!v0) zero_frags(bv);
        } else if constexpr (BF16) {  // kvalid is a multiple of 32: per MFMA slot
#pragma unroll
          for (int q = 0; q < 4; q++)
            if (128 * i + 32 * q >= kvalid) bv[q].q = make_uint4(0, 0, 0, 0);
        } else {
          if (!v0) bv[0].q = bv[1].q = make_uint4(0, 0, 0, 0);
          if (!v1) bv[2].q = bv[3].q = make_uint4(0, 0, 0, 0);
        }
        if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
          f32x4_t tmp = zero4();
#pragma unroll
          for (int q = 0; q < 4; q++) tmp = mfma_bf16(av[q], bv[q], tmp);
#pragma unroll
          for (int j = 0; j < 4; j++) acc[t][j] += bs[ii][t] * tmp[j];
        } else {
#pragma unroll
          for (int q = 0; q < 4; q++) acc[t] = mfma_bf16(av[q], bv[q], acc[t]);
        }
      }
    }
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) __builtin_amdgcn_s_setprio(0);
  }
}

// An activation matrix [rows, K] carried as two e4m3 planes (hi, lo) with an e8m0 scale per
// 32-element block of each row: q holds plane 0 then plane 1, s the scales likewise.
struct ActMX {
  rsrc_t q, s;
  uint32_t qplane, splane;  // bytes per plane
  uint32_t K;               // row width in elements
};

// The MXFP4 counterpart of mma_run: same chunk mapping, grouping (2 chunks per group) and
// weight layout, but each chunk is two scaled MFMAs (hi and lo plane of A) on the raw FP4
// codes.  Within a chunk, lane group g holds A's K [16g, 16g+16) and [64+16g, +16) and B's
// K [32g, 32g+32) (the instruction's operand layout), so both operands cover the same 128
// K indices.  Positions at or past kvalid contribute zero: their A bytes and B codes are
// replaced by zeros and their scales by 1, so stale workspace bytes never reach the MFMA.
//   a_q, a_s: byte offsets of this lane's row in the planes and in the scales (or
//             0x80000000 for a padding row, which reads zeros without a memory request)
//   lsc: as in mma_run (required when RB = 4 * COUNT is a multiple of 16)
template <int NT, int COUNT, bool NTW = false>
__device__ __forceinline__ void mma_run_mx(const ActMX &A, uint32_t a_q, uint32_t a_s,
                                           const WMat<MOE_FMT_MXFP4_E8M0> &m, const uint32_t (&rows)[NT],
                                           int b_k0, int kw0, int kvalid, int g, f32x4_t (&acc)[NT],
                                           uint8_t *lsc = nullptr) {
  constexpr int FMT = MOE_FMT_MXFP4_E8M0;
  const uint32_t K = (uint32_t)m.K;
  const int lane = lane_id(), r = lane & 15;
  constexpr int RB = 4 * COUNT;  // staged scale bytes per lane (one e8m0 per 32 K)
  constexpr int SQ = RB / 16;
  static_assert(NT % 4 == 0, "whole tiles per 16-lane group when staging scale runs");
  constexpr int TPG = NT / 4;  // tiles whose scale runs one 16-lane group stages
  uint4 stg[TPG][SQ > 0 ? SQ : 1];
  if constexpr (SQ > 0) {
#pragma unroll
    for (int u = 0; u < TPG; u++) {  // lanes 16t..16t+15 fetch the runs of tiles t, t + 4, ...
      const uint32_t run = (rows[(lane >> 4) + 4 * u] & ~15u) * (K / 32) + ((b_k0 + kw0) / 32) * 16;
#pragma unroll
      for (int q = 0; q < SQ; q++) stg[u][q] = buf_load16(m.scales, run + r * RB + 16 * q);
    }
  }
  const bool asal = ((A.K / 32) % 4 == 0) && ((kw0 / 32) % 4 == 0);
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i0 = 0; i0 < COUNT; i0 += 2) {
    const int kg = kw0 + (128 * i0 < kvalid ? 128 * i0 : 0);
    uint32_t lsv[2][NT];
    if constexpr (SQ == 0) {
#pragma unroll
      for (int ii = 0; ii < 2; ii++) {
        const int kr = 128 * (i0 + ii) + 32 * g;
        const uint32_t pc = (uint32_t)(b_k0 + kw0 + (kr < kvalid ? kr : 0)) / 32;
#pragma unroll
        for (int t = 0; t < NT; t++) lsv[ii][t] = buf_load1(m.scales, scale_tile_off<FMT>(rows[t], K) + pc * 16);
      }
    }
    const uint4 ash = load_scale_span<FMT>(A.s, a_s + kg / 32, asal);
    const uint4 asl = load_scale_span<FMT>(A.s, A.splane + a_s + kg / 32, asal);
    uint4 ah[2][2], al[2][2], c[2][NT];
#pragma unroll
    for (int ii = 0; ii < 2; ii++) {
      const int i = i0 + ii;
      if (i >= COUNT) break;
      const int kc = kw0 + (128 * i < kvalid ? 128 * i : 0);
      ah[ii][0] = buf_load16(A.q, a_q + kc + 16 * g);
      ah[ii][1] = buf_load16(A.q, a_q + kc + 64 + 16 * g);
      al[ii][0] = buf_load16(A.q, A.qplane + a_q + kc + 16 * g);
      al[ii][1] = buf_load16(A.q, A.qplane + a_q + kc + 64 + 16 * g);
      const int kr = 128 * i + 32 * g;
      const uint32_t pc = (uint32_t)(b_k0 + kw0 + (kr < kvalid ? kr : 0)) / 32;
#pragma unroll
      for (int t = 0; t < NT; t++) c[ii][t] = buf_load16w<NTW>(m.codes, code_tile_off<FMT>(rows[t], K) + pc * 256);
    }
    if constexpr (SQ > 0) {  // B scale bytes from the wave's LDS region (staged once per run)
      {
        if (i0 == 0) {
#pragma unroll
          for (int u = 0; u < TPG; u++)
#pragma unroll
            for (int q = 0; q < SQ; q++) *reinterpret_cast<uint4 *>(lsc + (lane + 64 * u) * RB + 16 * q) = stg[u][q];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
#pragma unroll
      for (int ii = 0; ii < 2; ii++) {
        const int kr = 128 * (i0 + ii) + 32 * g;
        const int cr = (kr < kvalid ? kr : 0) / 32;
#pragma unroll
        for (int t = 0; t < NT; t++) lsv[ii][t] = lsc[16 * t * RB + cr * 16 + r];
      }
    }
    // Raised wave priority over the scaled MFMAs: at two or three waves per SIMD, the wave whose
    // operands have arrived issues its matrix ops ahead of the other waves' loads and address
    // math.  Measured on MI355X, DeepSeek-shaped layer slice 1024 (step / gate_up, us): T = 256
    // 366.6 / 208.5 -> 348.6 / 196.1, T = 16 141.2 / 78.2 -> 134.7 / 75.1, T = 1 33.9 -> 33.4.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ii = 0; ii < 2; ii++) {
      const int i = i0 + ii;
      if (i >= COUNT) break;
      const int rel = 128 * i;
      const bool vb = rel + 32 * g < kvalid;  // this lane group's 32-wide block (both scales)
      const bool v0 = rel + 16 * g < kvalid, v1 = rel + 64 + 16 * g < kvalid;
      const uint4 h0 = v0 ? ah[ii][0] : z, h1 = v1 ? ah[ii][1] : z;
      const uint4 l0 = v0 ? al[ii][0] : z, l1 = v1 ? al[ii][1] : z;
      const uint32_t sh = vb ? (span_scales<FMT>(ash, ii, g) & 0xFFu) : 127u;
      const uint32_t sl = vb ? (span_scales<FMT>(asl, ii, g) & 0xFFu) : 127u;
#pragma unroll
      for (int t = 0; t < NT; t++) {
        const uint4 cbv = vb ? c[ii][t] : z;
        const uint32_t sbv = vb ? (lsv[ii][t] & 0xFFu) : 127u;
        acc[t] = mfma_scale_e4m3_e2m1(h0, h1, cbv, sh, sbv, acc[t]);
        acc[t] = mfma_scale_e4m3_e2m1(l0, l1, cbv, sl, sbv, acc[t]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

// ---------------------------------------------------------------------------- gate_up

// Workgroup = KW waves on one 16-row block and GC slice columns [c0, c0+GC): tiles
// 0..GT-1 are gate rows lo+c0+16t+[0,16), tiles GT..2GT-1 the matching up rows I+....  The
// first kwaves waves split K into contiguous ranges; their partial sums are added in wave
// order through LDS, then wave t < GT applies the SwiGLU epilogue of tile t.  Every column
// group of a row block reads the block's activation rows again.  Where those reads rival the
// weight bytes (MXFP4 with several pairs per expert: an e4m3 activation pair per 4-bit
// weight, re-read by 32 column groups at Il = 1024), GC = 64 halves them; its 8 tiles run at
// 2 waves per SIMD (195 VGPRs).  Measured on MI355X, DeepSeek-V4-Flash-shaped layer, slice
// 1024: T = 256 gate_up 232 -> 221 us; at T = 16 the halved workgroup count cost 1.7 us, so
// the launcher takes GC = 64 only from 4 pairs per expert on average.
constexpr int kMinWaves = 3;  // waves per SIMD the expert kernels are compiled for

// Routing of the one token of a whole-layer call, done by every routed gate_up workgroup
// (NTH threads) in place of reading an alignment.  The logits are the router's split-K
// partials summed in split order from +0, plus the bias: the float operations of the top-k
// kernels, so the same values.  Order: the key (logit descending, index ascending; NaN as
// -inf, -0 as +0: rank_key).  Thread x holds the keys of experts x + NTH q; each wave takes
// the k largest of its experts by k rounds of a wave maximum (select_topk's rounds), and wave
// 0 ranks the waves' candidates: the k of rank < k are the picks, in rank order, which is the
// order the top-k kernels select them in.  The softmax weights repeat select_topk's
// arithmetic on the same values.  For T = 1 and 16-row blocks the alignment is one block per
// pick in expert order: pick number sb in that order is this workgroup's expert (returned in
// e_out, its pair index in pair_out).  The writer workgroup also stores the logits, ids and
// weights moe_route gives and every array moe_align gives for them.
// scr: 4 E + 8 k NTH/64 + 1280 bytes of LDS, 8-byte aligned.
template <int NTH>
__device__ __forceinline__ void route_one_token(const GateUpArgs &a, int sb, bool writer, uint8_t *scr, int &e_out,
                                                int &pair_out) {
  constexpr int NW = NTH / 64, NQ = (1024 + NTH - 1) / NTH;  // waves; keys per thread for E <= 1024
  const int E = a.E, k = a.k, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t *cand = reinterpret_cast<uint64_t *>(scr);            // [NW][k] each wave's k largest
  uint64_t *pkey = cand + NW * k;                                // [64] keys of the picks by rank
  int32_t *pexp = reinterpret_cast<int32_t *>(pkey + 64);        // [64] their experts
  int32_t *ord_e = pexp + 64, *ord_j = ord_e + 64;               // [64] picks in expert order: expert, rank
  float *lg = reinterpret_cast<float *>(ord_j + 64);             // [E]
  uint64_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; q++) {
    const int e = tid + NTH * q;
    key[q] = 0;  // below every expert's key
    if (e < E) {
      float v[16];  // at most 16 splits, all loads in flight together
#pragma unroll
      for (int u = 0; u < 16; u++) v[u] = u < a.r_ks ? a.r_part[(size_t)u * E + e] : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < 16; u++)
        if (u < a.r_ks) sum += v[u];
      sum += a.r_bias ? a.r_bias[e] : 0.f;
      lg[e] = sum;
      key[q] = rank_key(sum != sum ? -INFINITY : sum, e);
      if (writer && a.r_logits) a.r_logits[e] = sum;
    }
  }
  // descending order of the thread's keys (odd-even transposition)
#pragma unroll
  for (int pass = 0; pass < NQ; pass++)
#pragma unroll
    for (int q = pass & 1; q + 1 < NQ; q += 2)
      if (key[q] < key[q + 1]) {
        const uint64_t t = key[q];
        key[q] = key[q + 1];
        key[q + 1] = t;
      }
  // this wave's k largest: the largest head score, the lowest expert among the heads holding it
  // (ties only), then the winner's lane shifts; an exhausted wave yields 0
  for (int j = 0; j < k; j++) {
    const uint32_t hv = (uint32_t)(key[0] >> 32);
    const uint32_t m = wave_max_u32(hv);
    const uint64_t cb = __ballot(hv == m);
    int wl = __ffsll((unsigned long long)cb) - 1;
    if (__popcll(cb) > 1) {
      const uint32_t iv = hv == m ? (uint32_t)key_index(key[0]) : 0xFFFFFFFFu;
      wl = __ffsll((unsigned long long)__ballot(iv == wave_min_u32(iv))) - 1;
    }
    const uint32_t klo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], wl);
    if (lane == 0) cand[wave * k + j] = m ? ((uint64_t)m << 32) | klo : 0;
    if (lane == wl) {
#pragma unroll
      for (int q = 0; q + 1 < NQ; q++) key[q] = key[q + 1];
      key[NQ - 1] = 0;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int C = NW * k;  // candidates; distinct experts, and at least k of them are real
    for (int c = lane; c < C; c += 64) {
      const uint64_t me = cand[c];
      int rank = 0;
      for (int i = 0; i < C; i++) rank += cand[i] > me ? 1 : 0;
      if (me && rank < k) {
        pkey[rank] = me;
        pexp[rank] = key_index(me);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float top = key_value(pkey[0]);
    const float mine = lane < k ? key_value(pkey[lane]) : 0.f;
    float z;
    if (a.r_renorm) {
      z = lane < k ? expf(mine - top) : 0.f;
    } else {
      z = 0.f;
      for (int e = lane; e < E; e += 64) z += expf(lg[e] - top);
    }
    z = wave_sum_f32(z);
    if (writer && lane < k) {
      a.r_ids[lane] = pexp[lane];
      a.r_w[lane] = expf(mine - top) / z;
    }
    if (lane < k) {  // place in expert order (the picks are distinct experts)
      const int ej = pexp[lane];
      int rb = 0;
      for (int j = 0; j < k; j++) rb += pexp[j] < ej ? 1 : 0;
      ord_e[rb] = ej;
      ord_j[rb] = lane;
    }
  }
  __syncthreads();
  e_out = ord_e[sb];
  pair_out = ord_j[sb];
  if (writer) {  // moe_align's output for these picks: P = k pairs, sentinel k, 16-row blocks
    for (int p = tid; p < a.cap; p += NTH) a.al_sorted[p] = (p & 15) == 0 && (p >> 4) < k ? ord_j[p >> 4] : k;
    for (int b = tid; b < a.cap / 16; b += NTH) a.al_block[b] = b < k ? ord_e[b] : -1;
    for (int e = tid; e <= E; e += NTH) {
      int below = 0, hit = 0;
      for (int j = 0; j < k; j++) {
        below += ord_e[j] < e ? 1 : 0;
        hit |= ord_e[j] == e ? 1 : 0;
      }
      a.al_offsets[e] = 16 * below;
      if (e < E) a.al_counts[e] = hit;
    }
    if (tid == 0) a.al_total[0] = 16 * k;
  }
  __syncthreads();  // every read of scr done before the caller reuses it
}

// KW = waves per workgroup, all splitting K: 4, or 8 when few pairs leave most of the chip
// idle (each wave then covers half the K range, one round trip fewer).  ROUTE1: the
// whole-layer call for one token (route_one_token in place of the alignment's reads).
template <int FMT, int COUNT, int KW, int GC, bool NTW, bool ROUTE1 = false>
__global__ __launch_bounds__(64 * KW, GC == 64 ? 2 : kMinWaves) void k_gate_up(GateUpArgs a) {
  constexpr int GT = GC / 16;
  static_assert(GT <= KW, "one wave per gate tile in the epilogue");
  __shared__ __attribute__((aligned(16))) float red[KW][2 * GT][4][64];  // [wave][tile][j][lane]
  __shared__ float hbuf[16][GC + 1];         // MXFP4: the block's h before the plane split
  // FP4: per wave, the scale bytes of the workgroup's 2*GC weight rows over one run
  __shared__ __attribute__((aligned(16))) uint8_t lsc[(FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_MXFP4_E8M0 || FMT == MOE_FMT_Q4_0) ? KW * 2 * GC * (128 * COUNT / (FMT == MOE_FMT_MXFP4_E8M0 ? 32 : 16)) : 16];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int sb = a.cols_fastest ? blockIdx.y : blockIdx.x;
  const int c0 = (a.cols_fastest ? blockIdx.x : blockIdx.y) * GC;
  const bool is_shared = sb >= a.n_routed_sub;
  int p0, e, tok;
  const uint8_t *codes;
  const uint8_t *scales;
  const float *glob;
  if (!is_shared) {
    p0 = sb * 16;
    if constexpr (ROUTE1) {  // one token: block sb holds pick sb (in expert order) in row 0
      if (sb >= a.k) return;   // uniform over the workgroup
      static_assert(sizeof(red) >= 4 * 1024 + 8 * KW * 64 + 1280, "routing scratch for E <= 1024, k <= 64");
      int e1, j1;
      route_one_token<64 * KW>(a, sb, sb == 0 && c0 == 0, reinterpret_cast<uint8_t *>(&red[0][0][0][0]), e1, j1);
      e = __builtin_amdgcn_readfirstlane(e1);
      tok = r == 0 ? 0 : -1;
    } else {
      // three independent loads in flight together (p0 < cap indexes both arrays)
      const int tp = a.total_padded[0], eb = a.block_expert[p0 / a.block_m], f = a.sorted_ids[p0 + r];
      if (p0 >= __builtin_amdgcn_readfirstlane(tp)) return;  // uniform over the workgroup
      e = __builtin_amdgcn_readfirstlane(eb);
      if (e < 0) return;
      tok = f < a.T * a.k ? f / a.k : -1;
    }
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
  const int ntile = min(GT, (a.Il - c0) / 16);  // gate tiles inside the slice (Il % 32 == 0)
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, 2 * I, H);
  uint32_t rows[2 * GT];  // rows inside this expert's [2I, H] matrix
#pragma unroll
  for (int t = 0; t < GT; t++) {
    rows[t] = a.lo + c0 + 16 * (t < ntile ? t : 0) + r;
    rows[GT + t] = rows[t] + I;
  }
  float gsc[GT], usc[GT];  // per-row globals, loaded early
#pragma unroll
  for (int t = 0; t < GT; t++) {
    gsc[t] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + rows[t]] : 1.f;
    usc[t] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + rows[GT + t]] : 1.f;
  }
  // FP4 and Q4_0 scales are staged per wave when a run's scale bytes per tile are whole
  // 16-byte pieces (runs of at least 2 steps for NVFP4 and Q4_0, 4 for MXFP4); otherwise
  // lanes load theirs
  uint8_t *wsc = nullptr;
  if constexpr (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_MXFP4_E8M0 || FMT == MOE_FMT_Q4_0) {
    constexpr int sdiv = FMT == MOE_FMT_MXFP4_E8M0 ? 32 : 16;  // elements per scale byte
    constexpr int RB = 128 * COUNT / sdiv;
    if (RB % 16 == 0) wsc = &lsc[wave * 2 * GC * RB];
  }
  f32x4_t acc[2 * GT];
#pragma unroll
  for (int t = 0; t < 2 * GT; t++) acc[t] = zero4();
  // K split: wave w < a.kwaves takes [w*kw, (w+1)*kw), kw = 128 * a.ksteps
  // in runs of COUNT steps.  Padding rows point past the
  // activation buffer: they read zeros without a memory request.
  const int kw = 128 * a.ksteps;
  if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    const uint32_t T = (uint32_t)a.T;
    const ActMX A{make_rsrc(a.xq, 2 * T * H), make_rsrc(a.xs, 2 * T * (H / 32)), T * H, T * (H / 32), (uint32_t)H};
    const uint32_t aq = tok >= 0 ? (uint32_t)tok * H : 0x80000000u;
    const uint32_t as = tok >= 0 ? (uint32_t)tok * (H / 32) : 0x80000000u;
    if (wave < a.kwaves)
      for (int kk = 0; kk < kw; kk += 128 * COUNT)  // runs of COUNT steps; the tail is masked
        mma_run_mx<2 * GT, COUNT, NTW>(A, aq, as, m, rows, 0, wave * kw + kk, kw - kk, g, acc, wsc);
  } else {
    const rsrc_t ra = make_rsrc(a.x, (uint32_t)a.T * H * 2);
    const uint32_t a_row = tok >= 0 ? (uint32_t)tok * H * 2 : 0x80000000u;
    if (wave < a.kwaves) {
      for (int kk = 0; kk < kw; kk += 128 * COUNT)
        mma_run<FMT, 2 * GT, COUNT, false, NTW>(ra, a_row, m, rows, 0, wave * kw + kk, kw - kk, g, acc, wsc);
    }
  }
#pragma unroll
  for (int t = 0; t < 2 * GT; t++)
#pragma unroll
    for (int j = 0; j < 4; j++) red[wave][t][j][lane] = acc[t][j];
  __syncthreads();
  if (wave < ntile) {
    const int t = wave;  // gate tile t, up tile GT + t
#pragma unroll
    for (int j = 0; j < 4; j++) {
      float gv = 0.f, uv = 0.f;
#pragma unroll
      for (int w = 0; w < KW; w++) {
        gv += red[w][t][j][lane];
        uv += red[w][GT + t][j][lane];
      }
      gv *= gsc[t];
      uv *= usc[t];
      const float hv = gv / (1.f + __expf(-gv)) * uv;
      if constexpr (FMT == MOE_FMT_MXFP4_E8M0)
        hbuf[4 * g + j][16 * t + r] = hv;
      else
        a.h[(size_t)(p0 + 4 * g + j) * a.Il + c0 + 16 * t + r] = bf16_bits(hv);
    }
  }
  if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    // h rows of this block, each 32-column block of [c0, c0 + GC) one e8m0 block: 16 lanes per
    // (row, block), whole waves per block (a block past the slice is skipped by whole rows)
    __syncthreads();
    for (int item = threadIdx.x; item < 16 * 16 * (GC / 32); item += 64 * KW) {
      const int blk = item >> 8, row = (item >> 4) & 15, cp = 32 * blk + (item & 15) * 2;
      if (c0 + 32 * blk >= a.Il) break;  // uniform over the wave
      const float v[2] = {hbuf[row][cp], hbuf[row][cp + 1]};
      uint32_t qh[1], ql[1], s1, s2;
      mx8_split<2>(v, [](float x) { return row16_max(x); }, qh, ql, s1, s2);
      // a row without a token (all 16 lanes of the row) is never read: its planes are not written.
      // Measured on MI355X, DeepSeek-shaped layer: T = 256 369.9 -> 366.0 us, T = 16 145.1 -> 140.8
      // us per step (about half of the 16-row blocks' rows are padding there).  The bf16 h rows of
      // the other formats are still all written: skipping them there changed the decode kernels'
      // register allocation and measured slower for NVFP4 (T = 64 61.9 -> 62.7 us).
      if (__shfl(tok, row) < 0) continue;
      const size_t Il = (size_t)a.Il, hplane = (size_t)a.h_rows * Il, splane = (size_t)a.h_rows * (Il / 32);
      const size_t o = (size_t)(p0 + row) * Il + c0 + cp;
      *reinterpret_cast<uint16_t *>(a.hq + o) = (uint16_t)qh[0];
      *reinterpret_cast<uint16_t *>(a.hq + hplane + o) = (uint16_t)ql[0];
      if ((item & 15) == 0) {
        const size_t so = (size_t)(p0 + row) * (Il / 32) + (c0 + 32 * blk) / 32;
        a.hs[so] = (uint8_t)s1;
        a.hs[splane + so] = (uint8_t)s2;
      }
    }
  }
}

// ---------------------------------------------------------------------------- down

// Wave w owns hidden columns [n0, n0 + 16*DNT), n0 = group*64*DNT + 16*DNT*w: DNT MFMA
// tiles sharing one A fragment (a row block of h); K = the slice width Il.
constexpr int DNT = 4;

// Bytes of the per-wave LDS region down_wave stages FP4 / Q4_0 scale runs in (16 otherwise).
template <int FMT, int COUNT>
constexpr int down_lsc_bytes() {
  return (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_MXFP4_E8M0 || FMT == MOE_FMT_Q4_0)
             ? 16 * DNT * (128 * COUNT / (FMT == MOE_FMT_MXFP4_E8M0 ? 32 : 16))
             : 16;
}

// One wave's down tile: the 16 rows of sub-block sb (routed below a.n_routed_sub, then the
// shared expert's) against hidden columns [n0, n0 + 16 DNT), K = the slice.  Returns false when
// the sub-block holds no rows in use (past total_padded or no expert); otherwise acc[t][j] is
// row 4g + j, column n0 + 16 t + r of the unweighted pair rows, before the per-row global
// (dglob[t]), dst[j] the Y row of row 4g + j (-1: padding) and ntile the tiles inside H.
// lsc: this wave's down_lsc_bytes<FMT, COUNT>() bytes of LDS.
template <int FMT, int COUNT, bool NTW>
__device__ __forceinline__ bool down_wave(const DownArgs &a, int sb, int n0, uint8_t *lsc, f32x4_t (&acc)[DNT],
                                          int (&dst)[4], float (&dglob)[DNT], int &ntile) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const bool is_shared = sb >= a.n_routed_sub;
  int p0, e;
  const uint8_t *codes;
  const uint8_t *scales;
  const float *glob;
  int f0 = 0;  // pair of this lane's row (routed blocks)
  if (!is_shared) {
    p0 = sb * 16;
    // independent loads in flight together (p0 < cap indexes both arrays)
    const int tp = a.total_padded[0], eb = a.block_expert[p0 / a.block_m];
    f0 = a.sorted_ids[p0 + r];
    if (p0 >= __builtin_amdgcn_readfirstlane(tp)) return false;
    e = __builtin_amdgcn_readfirstlane(eb);
    if (e < 0) return false;
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
  ntile = min(DNT, (H - n0) / 16);
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, H, I);
  // FP4 and Q4_0 scales are staged per wave when a run's scale bytes per tile are whole
  // 16-byte pieces (runs of at least 2 steps for NVFP4 and Q4_0, 4 for MXFP4); otherwise
  // lanes load theirs
  uint8_t *wsc = nullptr;
  if constexpr (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_MXFP4_E8M0 || FMT == MOE_FMT_Q4_0) {
    constexpr int sdiv = FMT == MOE_FMT_MXFP4_E8M0 ? 32 : 16;  // elements per scale byte
    constexpr int RB = 128 * COUNT / sdiv;
    if (RB % 16 == 0) wsc = lsc;
  }
  uint32_t rows[DNT];  // rows inside this expert's [H, I] matrix
#pragma unroll
  for (int t = 0; t < DNT; t++) rows[t] = n0 + 16 * (t < ntile ? t : 0) + r;
#pragma unroll
  for (int t = 0; t < DNT; t++) acc[t] = zero4();
  // destination rows: lane r of every lane group already holds the pair of row r (f0), and
  // this lane's result rows are 4g + j, so they come from a cross-lane shuffle, not a load
  const int P = a.T * a.k;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (!is_shared) {
      const int f = __shfl(f0, 4 * g + j);
      dst[j] = f < P ? f : -1;
    } else {
      const int t = p0 + 4 * g + j - a.cap;
      dst[j] = t < a.T ? P + t : -1;
    }
  }
#pragma unroll
  for (int t = 0; t < DNT; t++) dglob[t] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * H + n0 + 16 * t + r] : 1.f;
  // padding rows (no pair / past T) point past h: they read zeros without a memory request
  const bool real = is_shared ? (p0 - a.cap + r < a.T) : (f0 < P);
  if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    const uint32_t hr = (uint32_t)a.h_rows, ul = (uint32_t)Il;
    const ActMX A{make_rsrc(a.hq, 2 * hr * ul), make_rsrc(a.hs, 2 * hr * (ul / 32)), hr * ul, hr * (ul / 32), ul};
    const uint32_t aq = real ? (uint32_t)(p0 + r) * ul : 0x80000000u;
    const uint32_t as = real ? (uint32_t)(p0 + r) * (ul / 32) : 0x80000000u;
    for (int kw0 = 0; kw0 < Il; kw0 += 128 * COUNT)  // runs of COUNT steps; the tail is masked
      mma_run_mx<DNT, COUNT, NTW>(A, aq, as, m, rows, a.lo, kw0, Il - kw0, g, acc, wsc);
  } else {
    const rsrc_t ra = make_rsrc(a.h, (uint32_t)a.h_rows * Il * 2);
    const uint32_t a_row = real ? (uint32_t)(p0 + r) * Il * 2 : 0x80000000u;
    // Q4_0 steps cover 128-element pieces of the row from its start: a slice starting at a
    // multiple of 32 inside one starts kph elements into its first step
    constexpr bool Q4 = FMT == MOE_FMT_Q4_0;
    const int kph = Q4 ? a.lo & 127 : 0;
    for (int kw0 = 0; kw0 < Il + kph; kw0 += 128 * COUNT)
      mma_run<FMT, DNT, COUNT, Q4, NTW>(ra, a_row, m, rows, a.lo - kph, kw0, Il + kph - kw0, g, acc, wsc, kph);
  }
  return true;
}

// Row pitch (floats) of a wave's 16 x 64 output tile in LDS: 68 puts the four row groups a
// result register spans (rows 4 apart) two by two in different bank halves, and keeps rows
// 16-byte aligned.
constexpr int kYPitch = 16 * DNT + 4;

// The pair rows leave through LDS for MXFP4 only.  Measured on MI355X (whole step, same box):
// DeepSeek-shaped layer T = 256 371.6 -> 369.7 us, T = 16 145.6 -> 144.7 us; NVFP4 T = 64
// 62.2 -> 62.9 us (its 2-step instance crosses 128 registers), fp8-block and q4_0 unchanged.
template <int FMT>
constexpr bool kDownStagedY = FMT == MOE_FMT_MXFP4_E8M0;

// Grid position of a down workgroup -> (16-row sub-block, column group).  With the column
// group fastest (grid (ncol, nsub)) the column groups of one sub-block all run on one XCD
// (workgroups are dealt to the 8 XCDs by linear index mod 8), so that sub-block's h rows are
// fetched into one L2 instead of all eight; sub-blocks past the last whole group of 8 keep the
// plain order.  Measured on MI355X (two pairs of runs, same box): DeepSeek-shaped MXFP4 layer
// T = 256, slice 1024: down 122.7 / 123.3 -> 118.6 / 117.9 us; NVFP4 T = 64, slice 512: down
// 32.6 -> 31.3 us.  The same order for gate_up measured slower (194.7 -> 199.4 us), so gate_up
// keeps the plain order.
__device__ __forceinline__ void down_tile(int cols_fastest, int &sb, int &cg) {
  if (!cols_fastest) {
    sb = blockIdx.x;
    cg = blockIdx.y;
    return;
  }
  const int ncol = gridDim.x, L = blockIdx.x + ncol * blockIdx.y;
  if (L >= (int)(gridDim.y & ~7u) * ncol) {
    sb = blockIdx.y;
    cg = blockIdx.x;
    return;
  }
  const int slot = L >> 3;
  sb = 8 * (slot / ncol) + (L & 7);
  cg = slot - (slot / ncol) * ncol;
}

template <int FMT, int COUNT, bool NTW>
__global__ __launch_bounds__(256, kMinWaves) void k_down(DownArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lsc[4 * down_lsc_bytes<FMT, COUNT>()];
  __shared__ __attribute__((aligned(16))) float ytile[kDownStagedY<FMT> ? 4 : 1][16][kYPitch];  // per wave: its rows
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  int sb, cg;
  down_tile(a.cols_fastest, sb, cg);
  const int n0 = cg * 64 * DNT + wave * 16 * DNT;  // first output column
  if (n0 >= a.H) return;
  f32x4_t acc[DNT];
  int dst[4], ntile;
  float dglob[DNT];
  if (!down_wave<FMT, COUNT, NTW>(a, sb, n0, &lsc[wave * down_lsc_bytes<FMT, COUNT>()], acc, dst, dglob, ntile))
    return;
  const int H = a.H;
  if constexpr (!kDownStagedY<FMT>) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (dst[j] < 0) continue;
#pragma unroll
      for (int t = 0; t < DNT; t++) {
        if (t >= ntile) break;
        a.Y[(size_t)dst[j] * H + n0 + 16 * t + r] = acc[t][j] * dglob[t];
      }
    }
    return;
  }
  // The pair rows through LDS: register j of lane (r, g) is row 4g + j, column 16t + r, so the
  // direct stores above write 64-byte pieces of four rows; here each store writes 16 bytes a
  // lane, 16 lanes per row, whole 256-byte row pieces of 4 rows.
  float(*yt)[kYPitch] = ytile[wave];
#pragma unroll
  for (int t = 0; t < DNT; t++)
#pragma unroll
    for (int j = 0; j < 4; j++) yt[4 * g + j][16 * t + r] = acc[t][j] * dglob[t];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c4 = 4 * r;  // this lane's 4 columns of a row
#pragma unroll
  for (int u = 0; u < 4; u++) {
    // row 4u + g: the lanes of row group u hold its destination as their dst[g]
    int d = -1;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int v = __shfl(dst[j], 16 * u);
      d = g == j ? v : d;
    }
    if (d >= 0 && c4 < 16 * ntile)
      *reinterpret_cast<float4 *>(&a.Y[(size_t)d * H + n0 + c4]) =
          *reinterpret_cast<const float4 *>(&yt[4 * u + g][c4]);
  }
}

// One token (T = 1): down and combine in one kernel.  A workgroup of 16 waves owns hidden
// columns [64 x, 64 x + 64); wave w takes sub-block w (the routed ones, one pair each at
// most, then the shared expert's at n_routed_sub), so every row the token's output sums is
// in this workgroup.  The waves leave their rows (unweighted, after the per-row global, as
// the Y rows) in LDS under the row's pair index (the shared row after the k pairs), and one
// thread per column sums them as k_combine does: the k pairs in order, weighted, then the
// shared row.  A row nobody writes (an id outside [0, E)) counts as zero.
template <int FMT, int COUNT, bool NTW>
__global__ __launch_bounds__(1024) void k_down_t1(DownArgs a, const float *__restrict__ topk_w, void *__restrict__ out,
                                                  int out_bf16) {
  __shared__ __attribute__((aligned(16))) uint8_t lsc[16 * down_lsc_bytes<FMT, COUNT>()];
  __shared__ float rowv[17][64];  // [pair (k <= 15), then the shared row][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15;
  const int n0 = blockIdx.x * 64, k = a.k;
  for (int i = tid; i < 17 * 64; i += 1024) (&rowv[0][0])[i] = 0.f;
  __syncthreads();
  const int nsub = a.n_routed_sub + (a.sdn ? 1 : 0);
  if (wave < nsub) {
    f32x4_t acc[DNT];
    int dst[4], ntile;
    float dglob[DNT];
    if (down_wave<FMT, COUNT, NTW>(a, wave, n0, &lsc[wave * down_lsc_bytes<FMT, COUNT>()], acc, dst, dglob, ntile)) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (dst[j] < 0) continue;  // dst: pair f < k, or k + 0 for the shared row
#pragma unroll
        for (int t = 0; t < DNT; t++)
          if (t < ntile) rowv[dst[j]][16 * t + r] = acc[t][j] * dglob[t];
      }
    }
  }
  __syncthreads();
  const int n = n0 + tid;
  if (tid >= 64 || n >= a.H) return;
  float s = 0.f;
  for (int j = 0; j < k; j++) s += topk_w[j] * rowv[j][tid];
  if (a.sdn) s += 1.f * rowv[k][tid];
  if (out_bf16)
    reinterpret_cast<uint16_t *>(out)[n] = bf16_bits(s);
  else
    reinterpret_cast<float *>(out)[n] = s;
}

// ---------------------------------------------------------------------------- combine

// out[t] = sum_j w[t*k + j] Y[t*k + j] + Y[T*k + t] (shared, weight 1), in this order, in
// fp32.  Y rows are fp32 (streaming kernels, a thread owns 4 consecutive columns) or bf16
// (prefill GEMMs, 8 columns: one 16-byte load per row); H % 128 == 0.
template <bool YBF16>
__global__ __launch_bounds__(256) void k_combine(const void *__restrict__ Yv, const float *__restrict__ w, int T,
                                                 int k, int H, int has_shared, void *__restrict__ out,
                                                 int out_bf16) {
  constexpr int NC = YBF16 ? 8 : 4;  // columns per thread
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * NC;
  if (n >= H) return;
  const int nrows = k + (has_shared ? 1 : 0);  // the token's k pair rows, then its shared row
  float acc[NC];
#pragma unroll
  for (int c = 0; c < NC; c++) acc[c] = 0.f;
  // rows in flight: 16 for the fp32 rows of the streaming kernels (k <= 15 plus the shared row
  // in one round trip, measured faster at decode), 8 for the bf16 rows of the prefill GEMMs
  constexpr int NB = YBF16 ? 8 : 16;
  for (int j0 = 0; j0 < nrows; j0 += NB) {
    float v[NB][NC], wj[NB];
#pragma unroll
    for (int u = 0; u < NB; u++) {
      const int j = j0 + u;
      const size_t row = j < k ? (size_t)t * k + j : (size_t)T * k + t;
      wj[u] = j < k ? w[row] : 1.f;  // row < T * k for routed rows
      if (j < nrows) {
        if constexpr (YBF16) {
          const uint4 q = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(Yv) + row * H + n);
          const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int c = 0; c < 4; c++) {
            v[u][2 * c] = __uint_as_float(d[c] << 16);
            v[u][2 * c + 1] = __uint_as_float(d[c] & 0xFFFF0000u);
          }
        } else {
          const float4 q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(Yv) + row * H + n);
          v[u][0] = q.x;
          v[u][1] = q.y;
          v[u][2] = q.z;
          v[u][3] = q.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NB; u++)
      if (j0 + u < nrows)
#pragma unroll
        for (int c = 0; c < NC; c++) acc[c] += wj[u] * v[u][c];
  }
  if (out_bf16) {
    uint32_t pk[NC / 2];
#pragma unroll
    for (int c = 0; c < NC / 2; c++) pk[c] = (uint32_t)bf16_bits(acc[2 * c]) | ((uint32_t)bf16_bits(acc[2 * c + 1]) << 16);
    uint16_t *o = reinterpret_cast<uint16_t *>(out) + (size_t)t * H + n;
    if constexpr (NC == 8)
      *reinterpret_cast<uint4 *>(o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    else
      *reinterpret_cast<uint2 *>(o) = make_uint2(pk[0], pk[1]);
  } else {
    float *o = reinterpret_cast<float *>(out) + (size_t)t * H + n;
#pragma unroll
    for (int c = 0; c < NC; c += 4) *reinterpret_cast<float4 *>(o + c) = make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]);
  }
}

// ---------------------------------------------------------------------------- launchers

// Step count of a K run as a template argument: 1, 2, 4 or 8 (runs are masked past K).
// Longer K ranges loop over runs; fp8-block, MXFP4 and bf16 keep runs at 4 steps or fewer,
// past which their per-step operand registers no longer fit the occupancy target.
static int count_class(int fmt, int steps) {
  const int c = steps <= 1 ? 1 : steps <= 2 ? 2 : steps <= 4 ? 4 : 8;
  return fmt == MOE_FMT_NVFP4 ? c : (c < 4 ? c : 4);
}

template <int FMT, int KW, int GC, bool NTW>
static void launch_gate_up_nt(const GateUpArgs &a, dim3 grid, hipStream_t s) {
  const dim3 block(64 * KW);
  if constexpr (KW == 8 && GC == 32 && !NTW) {  // the one-token whole-layer call (route1_launchable)
    if (a.route1) {
      switch (count_class(FMT, a.ksteps)) {
        case 1: hipLaunchKernelGGL((k_gate_up<FMT, 1, KW, GC, NTW, true>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_gate_up<FMT, 2, KW, GC, NTW, true>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_gate_up<FMT, 4, KW, GC, NTW, true>), grid, block, 0, s, a); break;
        default:
          if constexpr (FMT == MOE_FMT_NVFP4) hipLaunchKernelGGL((k_gate_up<FMT, 8, KW, GC, NTW, true>), grid, block, 0, s, a);
          break;
      }
      return;
    }
  }
  switch (count_class(FMT, a.ksteps)) {
    case 1: hipLaunchKernelGGL((k_gate_up<FMT, 1, KW, GC, NTW>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_gate_up<FMT, 2, KW, GC, NTW>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_gate_up<FMT, 4, KW, GC, NTW>), grid, block, 0, s, a); break;
    default:
      if constexpr (FMT == MOE_FMT_NVFP4) hipLaunchKernelGGL((k_gate_up<FMT, 8, KW, GC, NTW>), grid, block, 0, s, a);
      break;
  }
}

template <int FMT, int KW, int GC>
static void launch_gate_up_kw(const GateUpArgs &a, dim3 grid, hipStream_t s) {
  // the non-temporal hint on weight loads only where it measured faster (gate_up: bf16 and
  // MXFP4 weights, from 128 pairs)
  if constexpr (FMT == MOE_FMT_MXFP4_E8M0 || FMT == MOE_FMT_BF16) {
    if (a.nt_weights) {
      launch_gate_up_nt<FMT, KW, GC, true>(a, grid, s);
      return;
    }
  }
  launch_gate_up_nt<FMT, KW, GC, false>(a, grid, s);
}

template <int FMT, int GC>
static void launch_gate_up_gc(const GateUpArgs &a, int n_shared_sub, hipStream_t s) {
  const int nsub = a.n_routed_sub + n_shared_sub, ncol = (a.Il + GC - 1) / GC;
  const dim3 grid = a.cols_fastest ? dim3(ncol, nsub) : dim3(nsub, ncol);
  if constexpr (GC == 32) {
    if (a.kwaves > 4) {
      launch_gate_up_kw<FMT, 8, GC>(a, grid, s);
      return;
    }
  }
  launch_gate_up_kw<FMT, 4, GC>(a, grid, s);
}

template <int FMT>
static void launch_gate_up_grid(const GateUpArgs &a, int n_shared_sub, hipStream_t s) {
  // 64 slice columns per workgroup for MXFP4 with at least 4 pairs per expert on average
  // (the 8-wave K split, chosen only for few pairs, keeps 32)
  if constexpr (FMT == MOE_FMT_MXFP4_E8M0) {
    if ((long long)a.T * a.k >= 4LL * a.E && a.kwaves <= 4) {
      launch_gate_up_gc<FMT, 64>(a, n_shared_sub, s);
      return;
    }
  }
  launch_gate_up_gc<FMT, 32>(a, n_shared_sub, s);
}


template <int FMT>
static void launch_down_fmt(const DownArgs &a, dim3 grid, hipStream_t s) {
  // runs of at most 4 steps (down loops over runs; longer ones exceed the register budget);
  // Q4_0 steps start at multiples of 128 of the row, so a slice may touch one more
  const int kph = FMT == MOE_FMT_Q4_0 ? a.lo & 127 : 0;
  switch (count_class(MOE_FMT_FP8_BLOCK128, (a.Il + kph + 127) / 128)) {
    case 1:
      if (a.nt_weights) hipLaunchKernelGGL((k_down<FMT, 1, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_down<FMT, 1, false>), grid, dim3(256), 0, s, a);
      break;
    case 2:
      if (a.nt_weights) hipLaunchKernelGGL((k_down<FMT, 2, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_down<FMT, 2, false>), grid, dim3(256), 0, s, a);
      break;
    default:
      if (a.nt_weights) hipLaunchKernelGGL((k_down<FMT, 4, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((k_down<FMT, 4, false>), grid, dim3(256), 0, s, a);
      break;
  }
}

template <int FMT>
static void launch_down_t1_fmt(const DownArgs &a, const float *topk_w, void *out, int out_bf16, hipStream_t s) {
  const dim3 grid((a.H + 63) / 64), block(1024);
  const int kph = FMT == MOE_FMT_Q4_0 ? a.lo & 127 : 0;
  switch (count_class(MOE_FMT_FP8_BLOCK128, (a.Il + kph + 127) / 128)) {
    case 1: hipLaunchKernelGGL((k_down_t1<FMT, 1, false>), grid, block, 0, s, a, topk_w, out, out_bf16); break;
    case 2: hipLaunchKernelGGL((k_down_t1<FMT, 2, false>), grid, block, 0, s, a, topk_w, out, out_bf16); break;
    default: hipLaunchKernelGGL((k_down_t1<FMT, 4, false>), grid, block, 0, s, a, topk_w, out, out_bf16); break;
  }
}

// The MXFP4 instantiations (expert_mxfp4.hip).
void launch_gate_up_mxfp4(const GateUpArgs &a, int n_shared_sub, hipStream_t s);
void launch_down_mxfp4(const DownArgs &a, dim3 grid, hipStream_t s);
void launch_down_t1_mxfp4(const DownArgs &a, const float *topk_w, void *out, int out_bf16, hipStream_t s);

}  // namespace qmoe
