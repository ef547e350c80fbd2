// expert_tiled.hip -- the expert GEMMs for many tokens per expert (prefill), gfx950.
//
// Same computation as expert.hip (gate rows [lo,hi), up rows [I+lo, I+hi), down columns
// [lo,hi) of one rank's slice: FreeToken issue #62 "What it touches" item 1; SwiGLU expert
// linear in the intermediate index: issue #520 section 4), tiled for reuse instead of
// streaming: a workgroup owns a 128-row block of the aligned pair list (one expert) and 128
// weight rows, and walks K in stages of 64.  Per stage the activation tile (gathered token
// rows of x, or rows of h) and the weight tile are staged in LDS, the weight tile
// dequantized to bf16 once per workgroup; 4 waves then run 2 x 2 blocks of 64 x 64 outputs
// on v_mfma_f32_16x16x32_bf16.  LDS is double buffered: the global loads of stage s+1 are
// in flight while stage s multiplies, and one barrier per stage separates the buffers.
//
//   NVFP4      e2m1 * e4m3 group scale, exact in bf16; the per-row fp32 global is applied
//              in the epilogue (W4A16).
//   FP8_BLOCK  e4m3 -> bf16 exact; each 128-wide K block's partial product is scaled by
//              its fp32 weight_scale_inv and added to the accumulator (W8A16).
#include "device_common.h"
#include "launch.h"

namespace qmoe {
namespace {

constexpr int TM = 128;       // pair rows per tile = one align block of 128
constexpr int TW = 128;       // weight rows per tile
constexpr int TK = 64;        // K per stage
constexpr int LDP = TK + 8;   // LDS row pitch in bf16 elements (144 B: 16-row reads hit distinct banks)

struct TileLDS {
  uint16_t a[2][TM][LDP];
  uint16_t b[2][TW][LDP];
};

// ---------------------------------------------------------------- stage loads and stores

// Activation tile: a thread moves 4 pieces of 16 B; piece q is row 32*wave + 8*q + lane/8,
// columns [8*(lane%8), +8) of the stage (each row's 128 B are read by 8 adjacent lanes).
struct ATile {
  uint4 v[4];
};

__device__ __forceinline__ void a_fetch(rsrc_t ra, const uint32_t (&row_off)[4], int k0, int seg, ATile &t) {
#pragma unroll
  for (int q = 0; q < 4; q++) t.v[q] = buf_load16(ra, row_off[q] + (uint32_t)(k0 + 8 * seg) * 2);
}

__device__ __forceinline__ void a_store(uint16_t (*la)[LDP], const ATile &t, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 4; q++)
    *reinterpret_cast<uint4 *>(&la[32 * wave + 8 * q + (lane >> 3)][8 * (lane & 7)]) = t.v[q];
}

// Weight tile: a thread owns tile row tid/2 and the 32-wide K half tid%2 of the stage.
struct BTile {
  uint4 c0, c1;  // codes: 16 B (FP4) or 32 B (FP8)
  uint32_t sc;   // NVFP4: the two e4m3 group scales
};

template <int FMT>
__device__ __forceinline__ void b_fetch(const WMat<FMT> &m, uint32_t row, int k, BTile &t) {
  const uint32_t K = (uint32_t)m.K;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    t.c0 = buf_load16(m.codes, row * (K / 2) + k / 2);
    t.sc = buf_load2(m.scales, row * (K / 16) + k / 16);
  } else {
    t.c0 = buf_load16(m.codes, row * K + k);
    t.c1 = buf_load16(m.codes, row * K + k + 16);
  }
}

template <int FMT>
__device__ __forceinline__ void b_store(uint16_t *dst, const BTile &t, bool valid) {
  frag8 f[4];
  if constexpr (FMT == MOE_FMT_NVFP4) {
    const float s0 = e4m3_to_f32(t.sc & 0xFFu), s1 = e4m3_to_f32((t.sc >> 8) & 0xFFu);
    fp4x8_mul_to_bf16(t.c0.x, s0, f[0]);
    fp4x8_mul_to_bf16(t.c0.y, s0, f[1]);
    fp4x8_mul_to_bf16(t.c0.z, s1, f[2]);
    fp4x8_mul_to_bf16(t.c0.w, s1, f[3]);
  } else {
    fp8x8_to_bf16(t.c0.x, t.c0.y, f[0]);
    fp8x8_to_bf16(t.c0.z, t.c0.w, f[1]);
    fp8x8_to_bf16(t.c1.x, t.c1.y, f[2]);
    fp8x8_to_bf16(t.c1.z, t.c1.w, f[3]);
  }
  if (!valid) zero_frags(f);
#pragma unroll
  for (int q = 0; q < 4; q++) *reinterpret_cast<uint4 *>(dst + 8 * q) = f[q].q;
}

// ---------------------------------------------------------------- the MFMA stage

// acc[i][j] += A rows (a_row0 + 16 i) x weight rows brow[j], over the stage's 64 K.
__device__ __forceinline__ void mma_stage(const uint16_t (*la)[LDP], const uint16_t (*lb)[LDP], int a_row0,
                                          const int (&brow)[4], int lane, f32x4_t (&acc)[4][4]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < TK; kk += 32) {
    frag8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; i++) a[i].q = *reinterpret_cast<const uint4 *>(&la[a_row0 + 16 * i + r][kk + 8 * g]);
#pragma unroll
    for (int j = 0; j < 4; j++) b[j].q = *reinterpret_cast<const uint4 *>(&lb[brow[j] + r][kk + 8 * g]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
  }
}

// FP8 block scales: acc += s_j * part over one 128-wide K block, then part = 0.
__device__ __forceinline__ void fold_block(f32x4_t (&acc)[4][4], f32x4_t (&part)[4][4], const float (&s)[4]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int q = 0; q < 4; q++) acc[i][j][q] += s[j] * part[i][j][q];
      part[i][j] = zero4();
    }
}

// The K loop shared by both GEMMs.  Thread roles: activation pieces (4 rows given by
// a_off, byte offsets of the rows' K origin, 0x80000000 for rows that read zeros) and the
// weight tile row `wrow` of matrix m (half `bhalf` of each stage, zeroed unless wvalid).
// K runs over [0, nK*TK) relative to the weight column b_k0; weight K halves at or past
// kvalid load zeros.  FP8: scale(kb, j) gives the weight_scale_inv of col tile j, K block kb.
template <int FMT, typename ScaleFn>
__device__ __forceinline__ void tiled_k_loop(TileLDS &lds, rsrc_t ra, const uint32_t (&a_off)[4], const WMat<FMT> &m,
                                             uint32_t wrow, bool wvalid, int b_k0, int nK, int kvalid,
                                             const int (&brow)[4], ScaleFn scale, f32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane & 7, brr = tid >> 1, bhalf = tid & 1;
  const int a_row0 = (wave >> 1) * 64;
  f32x4_t part[4][4];
  if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) part[i][j] = zero4();
  }
  ATile at;
  BTile bt;
  a_fetch(ra, a_off, 0, seg, at);
  b_fetch<FMT>(m, wrow, b_k0 + 32 * bhalf, bt);
  a_store(lds.a[0], at, wave, lane);
  b_store<FMT>(&lds.b[0][brr][32 * bhalf], bt, wvalid && 32 * bhalf < kvalid);
  __syncthreads();
  for (int s = 0; s < nK; s++) {
    const int cur = s & 1;
    const bool more = s + 1 < nK;
    const int kn = (s + 1) * TK + 32 * bhalf;  // next stage's weight K (relative)
    if (more) {
      a_fetch(ra, a_off, (s + 1) * TK, seg, at);
      b_fetch<FMT>(m, wrow, b_k0 + (kn < kvalid ? kn : 0), bt);
    }
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
      mma_stage(lds.a[cur], lds.b[cur], a_row0, brow, lane, part);
      if (s & 1) {
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; j++) sc[j] = scale(s >> 1, j);
        fold_block(acc, part, sc);
      }
    } else {
      mma_stage(lds.a[cur], lds.b[cur], a_row0, brow, lane, acc);
    }
    if (more) {
      a_store(lds.a[cur ^ 1], at, wave, lane);
      b_store<FMT>(&lds.b[cur ^ 1][brr][32 * bhalf], bt, wvalid && kn < kvalid);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = zero4();
}

}  // namespace

// ---------------------------------------------------------------- gate_up + SwiGLU

// Tile (blockIdx.x, blockIdx.y): pair rows [p0, p0 + 128) of one expert (shared tiles
// follow the routed ones) and slice columns [c0, c0 + 64): weight tile rows 0..63 are the
// gate rows lo+c0+[0,64), rows 64..127 the up rows I+lo+c0+[0,64).  Wave (wm, wn) owns
// rows 64 wm + [0,64) and the gate/up column pairs c0 + 32 wn + [0,32), so SwiGLU is local.
template <int FMT>
__global__ __launch_bounds__(256, 2) void k_gate_up_tiled(GateUpArgs a) {
  __shared__ TileLDS lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int n_routed = a.cap / TM;
  const bool is_shared = (int)blockIdx.x >= n_routed;
  const int c0 = blockIdx.y * 64;
  int p0, e;
  const uint8_t *codes, *scales;
  const float *glob;
  if (!is_shared) {
    p0 = blockIdx.x * TM;
    if (p0 >= __builtin_amdgcn_readfirstlane(a.total_padded[0])) return;
    e = __builtin_amdgcn_readfirstlane(a.block_expert[p0 / a.block_m]);
    if (e < 0) return;
    codes = a.gu;
    scales = a.gus;
    glob = a.gug;
  } else {
    p0 = a.cap + (blockIdx.x - n_routed) * TM;
    e = 0;
    codes = a.sgu;
    scales = a.sgus;
    glob = a.sgug;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, 2 * I, H);
  const rsrc_t ra = make_rsrc(a.x, (uint32_t)T * H * 2);
  uint32_t a_off[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int p = p0 + 32 * wave + 8 * q + (lane >> 3);
    int tok;
    if (!is_shared) {
      const int f = a.sorted_ids[p];
      tok = f < P ? f / a.k : -1;
    } else {
      tok = p - a.cap < T ? p - a.cap : -1;
    }
    a_off[q] = tok >= 0 ? (uint32_t)tok * H * 2 : 0x80000000u;
  }
  const int brr = tid >> 1;
  const int bc = c0 + (brr & 63);  // slice column of this thread's weight row
  const bool wvalid = bc < Il;
  const uint32_t wrow = (uint32_t)((brr < 64 ? 0 : I) + a.lo + (wvalid ? bc : c0));
  const int brow[4] = {32 * wn, 32 * wn + 16, 64 + 32 * wn, 64 + 32 * wn + 16};
  f32x4_t acc[4][4];
  zero_acc(acc);
  auto scale = [&](int kb, int j) {
    const int wr = (j < 2 ? 0 : I) + a.lo + c0 + 32 * wn + 16 * (j & 1);
    return buf_load_f32(m.scales, (uint32_t)((wr / 128) * (H / 128) + kb) * 4);
  };
  tiled_k_loop<FMT>(lds, ra, a_off, m, wrow, wvalid, 0, H / TK, H, brow, scale, acc);
  // epilogue: per-row globals (NVFP4), SwiGLU, h in bf16
  float gg[2], ug[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int col = c0 + 32 * wn + 16 * j + r;
    const int cc = col < Il ? col : c0;
    gg[j] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + a.lo + cc] : 1.f;
    ug[j] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + I + a.lo + cc] : 1.f;
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const size_t row = (size_t)(p0 + 64 * wm + 16 * i + 4 * g + jj);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int col = c0 + 32 * wn + 16 * j + r;
        if (col >= Il) continue;
        const float gv = acc[i][j][jj] * gg[j], uv = acc[i][j + 2][jj] * ug[j];
        a.h[row * Il + col] = bf16_bits(gv / (1.f + __expf(-gv)) * uv);
      }
    }
}

// ---------------------------------------------------------------- down

// Tile (blockIdx.x, blockIdx.y): h rows [p0, p0 + 128) and hidden columns [n0, n0 + 128);
// K = the slice [lo, hi).  Wave (wm, wn) owns rows 64 wm + [0,64), columns 64 wn + [0,64).
template <int FMT>
__global__ __launch_bounds__(256, 2) void k_down_tiled(DownArgs a) {
  __shared__ TileLDS lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int n_routed = a.cap / TM;
  const bool is_shared = (int)blockIdx.x >= n_routed;
  const int n0 = blockIdx.y * TW;
  int p0, e;
  const uint8_t *codes, *scales;
  const float *glob;
  if (!is_shared) {
    p0 = blockIdx.x * TM;
    if (p0 >= __builtin_amdgcn_readfirstlane(a.total_padded[0])) return;
    e = __builtin_amdgcn_readfirstlane(a.block_expert[p0 / a.block_m]);
    if (e < 0) return;
    codes = a.dn;
    scales = a.dns;
    glob = a.dng;
  } else {
    p0 = a.cap + (blockIdx.x - n_routed) * TM;
    e = 0;
    codes = a.sdn;
    scales = a.sdns;
    glob = a.sdng;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, H, I);
  const rsrc_t ra = make_rsrc(a.h, (uint32_t)a.h_rows * Il * 2);
  uint32_t a_off[4];
#pragma unroll
  for (int q = 0; q < 4; q++) a_off[q] = (uint32_t)(p0 + 32 * wave + 8 * q + (lane >> 3)) * Il * 2;
  const uint32_t wrow = (uint32_t)(n0 + (tid >> 1));
  const int brow[4] = {64 * wn, 64 * wn + 16, 64 * wn + 32, 64 * wn + 48};
  f32x4_t acc[4][4];
  zero_acc(acc);
  auto scale = [&](int kb, int j) {
    const int wr = n0 + 64 * wn + 16 * j;
    return buf_load_f32(m.scales, (uint32_t)((wr / 128) * (I / 128) + a.lo / 128 + kb) * 4);
  };
  tiled_k_loop<FMT>(lds, ra, a_off, m, wrow, true, a.lo, (Il + TK - 1) / TK, Il, brow, scale, acc);
  float dg[4];
#pragma unroll
  for (int j = 0; j < 4; j++) dg[j] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * H + n0 + 64 * wn + 16 * j + r] : 1.f;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int p = p0 + 64 * wm + 16 * i + 4 * g + jj;
      int dst;
      float wgt;
      if (!is_shared) {
        const int f = a.sorted_ids[p];
        dst = f < P ? f : -1;
        wgt = f < P ? a.topk_w[f] : 0.f;
      } else {
        dst = p - a.cap < T ? P + (p - a.cap) : -1;
        wgt = 1.f;
      }
      if (dst < 0) continue;
#pragma unroll
      for (int j = 0; j < 4; j++) a.Y[(size_t)dst * H + n0 + 64 * wn + 16 * j + r] = wgt * acc[i][j][jj] * dg[j];
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_gate_up_tiled(int fmt, const GateUpArgs &a, int n_shared_tiles, hipStream_t s) {
  const dim3 grid(a.cap / TM + n_shared_tiles, (a.Il + 63) / 64);
  if (fmt == MOE_FMT_NVFP4)
    hipLaunchKernelGGL(k_gate_up_tiled<MOE_FMT_NVFP4>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_gate_up_tiled<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_tiled(int fmt, const DownArgs &a, int n_shared_tiles, hipStream_t s) {
  const dim3 grid(a.cap / TM + n_shared_tiles, a.H / TW);
  if (fmt == MOE_FMT_NVFP4)
    hipLaunchKernelGGL(k_down_tiled<MOE_FMT_NVFP4>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_down_tiled<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qmoe
