// expert_tiled.hip -- fp8-block and bf16 expert GEMMs for many tokens per expert (prefill),
// and the router GEMM for many tokens, gfx950.  (NVFP4 prefill runs in expert_wide.hip.)
//
// Same computation as expert.hip (gate rows [lo,hi), up rows [I+lo, I+hi), down columns
// [lo,hi) of one rank's slice: FreeToken issue #62 "What it touches" item 1; SwiGLU expert
// linear in the intermediate index: issue #520 section 4), tiled for reuse instead of
// streaming: a workgroup owns a 128-row block of the aligned pair list (one expert) and 128
// weight rows, and walks K in stages of 64 (gate_up) or 32 (down).  Per stage the activation tile (gathered token
// rows of x, or rows of h) and the weight tile are staged in LDS, the weight tile
// dequantized to bf16 once per workgroup; 4 waves then run 2 x 2 blocks of 64 x 64 outputs
// on v_mfma_f32_16x16x32_bf16.  LDS is double buffered: the global loads of stage s+1 are
// in flight while stage s multiplies, and one barrier per stage separates the buffers.
//
//   BF16       used as stored.
//   FP8_BLOCK  e4m3 -> bf16 exact; each 128-wide K block's partial product is scaled by
//              its fp32 weight_scale_inv and added to the accumulator (W8A16).
#include "device_common.h"
#include "launch.h"

namespace qmoe {
namespace {

constexpr int TM = 128;  // pair rows per tile = one align block of 128
constexpr int TW = 128;  // weight rows per tile

// K per stage TK is 64 (gate_up: K = H is long) or 32 (down: K = the slice, short, where
// the smaller LDS footprint lets more workgroups share a CU).  Derived sizes:
template <int TK> struct Stage {
  static constexpr int CPR = TK / 8;    // 16-byte chunks per LDS row (bf16)
  static constexpr int NQ = CPR / 2;    // activation chunks each thread stages per stage
  static constexpr int RPI = 64 / CPR;  // tile rows one wave instruction covers when staging
  static constexpr int WK = TK / 2;     // weights per thread per stage (half a tile row)
};

// LDS tiles are stored XOR-swizzled: K chunk c (elements [8c, 8c+8)) of tile row R sits at
// chunk c ^ (R & 7) of its 128-byte row (TK 64) or c ^ ((R >> 1) & 3) of its 64-byte row
// (TK 32).  The MFMA operand reads (16 rows x one chunk per lane group) and the stores
// then run at full LDS bandwidth on gfx950, which a plain or padded pitch does not reach
// for 16-row reads.
template <int TK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return TK == 64 ? 8 * (chunk ^ (row & 7)) : 8 * (chunk ^ ((row >> 1) & 3));
}

template <int TK>
struct TileLDS {
  uint16_t a[2][TM][TK];
  uint16_t b[2][TW][TK];
};

// ---------------------------------------------------------------- stage loads and stores

// Activation tile: thread chunk q covers row 32*wave + RPI*q + lane/CPR, K chunk lane%CPR
// (adjacent lanes read one row's TK*2 bytes).
template <int TK>
__device__ __forceinline__ int a_row_of(int wave, int lane, int q) {
  return 32 * wave + Stage<TK>::RPI * q + lane / Stage<TK>::CPR;
}

template <int TK>
struct ATile {
  uint4 v[Stage<TK>::NQ];
};

template <int TK>
__device__ __forceinline__ void a_fetch(rsrc_t ra, const uint32_t (&row_off)[Stage<TK>::NQ], int k0, int lane,
                                        ATile<TK> &t) {
#pragma unroll
  for (int q = 0; q < Stage<TK>::NQ; q++)
    t.v[q] = buf_load16(ra, row_off[q] + (uint32_t)(k0 + 8 * (lane % Stage<TK>::CPR)) * 2);
}

template <int TK>
__device__ __forceinline__ void a_store(uint16_t (*la)[TK], const ATile<TK> &t, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Stage<TK>::NQ; q++) {
    const int row = a_row_of<TK>(wave, lane, q);
    *reinterpret_cast<uint4 *>(&la[row][swz<TK>(row, lane % Stage<TK>::CPR)]) = t.v[q];
  }
}

// Plain bf16 weights (the router): no scales, no dequantization.
constexpr int kFmtBf16 = 0;

// Weight tile: thread tid stages tile row b_row_of(tid) and part b_half_of(tid) of every
// stage (WK weights).  The quantized weights are in the tile-16 layout (MOE_LAYOUT_TILE16:
// 16-row tiles stored piece-major, a piece = 16 code bytes), and a 32-thread group covers
// one tile: threads 0-15 its rows' part 0, threads 16-31 the same rows' part 1, two
// adjacent 256-byte pieces (one 512-byte run).  The row-major bf16 router weights pair the
// threads of a row instead.
template <int FMT, int TK>
constexpr bool kPairMap = FMT == kFmtBf16;

template <int FMT, int TK>
__device__ __forceinline__ int b_row_of(int tid) {
  return kPairMap<FMT, TK> ? tid >> 1 : 16 * (tid >> 5) + (tid & 15);
}

template <int FMT, int TK>
__device__ __forceinline__ int b_half_of(int tid) {
  return kPairMap<FMT, TK> ? tid & 1 : (tid >> 4) & 1;
}

struct BTile {
  uint4 c0, c1, c2, c3;  // codes: WK bytes (FP8) or 2*WK bytes (bf16)
};

// Loads part `half` of the stage starting at K offset ks (a multiple of TK) of matrix row `row`:
//   FP8   TK 64: pieces ks/16 + half and ks/16 + half + 2 (16 elements each)
//   FP8   TK 32: piece ks/16 + half
//   BF16 (tile-16 bank) TK 64: pieces ks/8 + 4 half + {0..3};  TK 32: ks/8 + 2 half + {0,1}
//   bf16 router (row-major): elements [ks + TK/2 half, +TK/2) of the row
template <int FMT, int TK>
__device__ __forceinline__ void b_fetch(const WMat<FMT> &m, uint32_t row, int ks, int half, BTile &t) {
  const uint32_t K = (uint32_t)m.K;
  if constexpr (FMT == MOE_FMT_BF16) {
    const uint32_t cb = (row & ~15u) * (2 * K) + (row & 15u) * 16;
    const uint32_t pc = (uint32_t)ks / 8 + (TK / 16) * half;
    t.c0 = buf_load16(m.codes, cb + pc * 256);
    t.c1 = buf_load16(m.codes, cb + (pc + 1) * 256);
    if constexpr (TK == 64) {
      t.c2 = buf_load16(m.codes, cb + (pc + 2) * 256);
      t.c3 = buf_load16(m.codes, cb + (pc + 3) * 256);
    }
  } else if constexpr (FMT == kFmtBf16) {
    const uint32_t o = (row * K + ks + (TK / 2) * half) * 2;
    t.c0 = buf_load16(m.codes, o);
    t.c1 = buf_load16(m.codes, o + 16);
    if constexpr (TK == 64) {
      t.c2 = buf_load16(m.codes, o + 32);
      t.c3 = buf_load16(m.codes, o + 48);
    }
  } else {
    const uint32_t cb = (row & ~15u) * K + (row & 15u) * 16;
    const uint32_t pc = (uint32_t)ks / 16 + half;
    t.c0 = buf_load16(m.codes, cb + pc * 256);
    if constexpr (TK == 64) t.c1 = buf_load16(m.codes, cb + (pc + 2) * 256);
  }
}

// Dequantizes and stores this thread's WK weights of tile row `row` (the 8-element K chunks
// b_fetch's part `half` covers).
template <int FMT, int TK>
__device__ __forceinline__ void b_store(uint16_t *rowp, int row, int half, const BTile &t, bool valid) {
  constexpr int NC = Stage<TK>::WK / 8;
  frag8 f[NC];
  if constexpr (FMT == kFmtBf16 || FMT == MOE_FMT_BF16) {
    f[0].q = t.c0;
    f[1].q = t.c1;
    if constexpr (NC == 4) {
      f[2].q = t.c2;
      f[3].q = t.c3;
    }
  } else {
    fp8x8_to_bf16(t.c0.x, t.c0.y, f[0]);
    fp8x8_to_bf16(t.c0.z, t.c0.w, f[1]);
    if constexpr (NC == 4) {
      fp8x8_to_bf16(t.c1.x, t.c1.y, f[2]);
      fp8x8_to_bf16(t.c1.z, t.c1.w, f[3]);
    }
  }
  if (!valid)
#pragma unroll
    for (int q = 0; q < NC; q++) f[q].q = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < NC; q++) {
    // FP8 TK 64 holds pieces half and half + 2: chunks 2 half + {0,1} and 4 + 2 half + {0,1}
    const int c = (FMT == MOE_FMT_FP8_BLOCK128 && TK == 64) ? (q < 2 ? 2 * half + q : 2 + 2 * half + q) : NC * half + q;
    *reinterpret_cast<uint4 *>(rowp + swz<TK>(row, c)) = f[q].q;
  }
}

// ---------------------------------------------------------------- the MFMA stage

// acc[i][j] += A rows (a_row0 + 16 i) x weight rows brow[j], over the stage's K.
template <int TK>
__device__ __forceinline__ void mma_stage(const uint16_t (*la)[TK], const uint16_t (*lb)[TK], int a_row0,
                                          const int (&brow)[4], int lane, f32x4_t (&acc)[4][4]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < TK; kk += 32) {
    frag8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      a[i].q = *reinterpret_cast<const uint4 *>(&la[a_row0 + 16 * i + r][swz<TK>(r, kk / 8 + g)]);
#pragma unroll
    for (int j = 0; j < 4; j++) b[j].q = *reinterpret_cast<const uint4 *>(&lb[brow[j] + r][swz<TK>(r, kk / 8 + g)]);
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

// The K loop shared by both GEMMs.  Thread roles: activation chunks (NQ rows given by
// a_off, byte offsets of the rows' K origin, 0x80000000 for rows that read zeros) and the
// weight tile row `wrow` of matrix m (part b_half_of(tid) of each stage, zeroed unless
// wvalid).  K runs over [0, nK*TK) relative to the weight column b_k0; stages at or past
// kvalid (a multiple of TK in every caller) load clamped offsets and store zeros.
// FP8: scale(kb, j) gives the weight_scale_inv of col tile j, K block kb.
template <int FMT, int TK, typename ScaleFn>
__device__ __forceinline__ void tiled_k_loop(TileLDS<TK> &lds, rsrc_t ra, const uint32_t (&a_off)[Stage<TK>::NQ],
                                             const WMat<FMT> &m,
                                             uint32_t wrow, bool wvalid, int b_k0, int nK, int kvalid,
                                             const int (&brow)[4], ScaleFn scale, f32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int brr = b_row_of<FMT, TK>(tid), bhalf = b_half_of<FMT, TK>(tid);
  const int a_row0 = (wave >> 1) * 64;
  f32x4_t part[4][4];
  if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) part[i][j] = zero4();
  }
  // Loads run two stages ahead of the multiply: register set s%2 receives stage s+2 while
  // stage s multiplies out of LDS buffer s%2 and stage s+1 (in registers since the
  // previous stage) is stored to LDS buffer (s+1)%2.
  ATile<TK> at[2];
  BTile bt[2];
  auto fetch = [&](int st, ATile<TK> &ta, BTile &tb) {  // weight loads first: oldest in the queue
    const int kb = st * TK;
    b_fetch<FMT, TK>(m, wrow, b_k0 + (kb < kvalid ? kb : 0), bhalf, tb);
    a_fetch<TK>(ra, a_off, st * TK, lane, ta);
  };
  auto store = [&](int st, const ATile<TK> &ta, const BTile &tb) {
    a_store<TK>(lds.a[st & 1], ta, wave, lane);
    b_store<FMT, TK>(lds.b[st & 1][brr], brr, bhalf, tb, wvalid && st * TK + (TK / 2) * bhalf < kvalid);
  };
  // Fetches are unconditional (stages past the end reload the last one, unused) so that
  // every path has the same loads in flight and the compiler's waits stay partial.
  fetch(0, at[0], bt[0]);
  fetch(nK > 1 ? 1 : 0, at[1], bt[1]);
  store(0, at[0], bt[0]);
  __syncthreads();
  auto stage = [&](int st, ATile<TK> &ta_free, BTile &tb_free, const ATile<TK> &ta_next, const BTile &tb_next) {
    fetch(st + 2 < nK ? st + 2 : nK - 1, ta_free, tb_free);
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
      mma_stage<TK>(lds.a[st & 1], lds.b[st & 1], a_row0, brow, lane, part);
      constexpr int SPB = 128 / TK;  // stages per 128-wide scale block
      if (st % SPB == SPB - 1) {
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; j++) sc[j] = scale(st / SPB, j);
        fold_block(acc, part, sc);
      }
    } else {
      mma_stage<TK>(lds.a[st & 1], lds.b[st & 1], a_row0, brow, lane, acc);
    }
    // unconditional (after the last stage it fills the idle buffer, which nobody reads) so
    // that every path through the loop leaves the same loads in flight
    store(st + 1, ta_next, tb_next);
    __syncthreads();
  };
  int st = 0;
  for (; st + 1 < nK; st += 2) {
    stage(st, at[0], bt[0], at[1], bt[1]);
    stage(st + 1, at[1], bt[1], at[0], bt[0]);
  }
  if (st < nK) stage(st, at[0], bt[0], at[1], bt[1]);  // odd stage count: the last one, peeled
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
  constexpr int TK = 64;
  __shared__ TileLDS<TK> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int n_routed = a.cap / TM;
  const bool is_shared = (int)blockIdx.x >= n_routed;
  const int c0 = blockIdx.y * 64;
  int p0, e;
  const uint8_t *codes, *scales;
  if (!is_shared) {
    p0 = blockIdx.x * TM;
    const int tp = a.total_padded[0], eb = a.block_expert[p0 / a.block_m];  // both in flight (p0 < cap)
    if (p0 >= __builtin_amdgcn_readfirstlane(tp)) return;
    e = __builtin_amdgcn_readfirstlane(eb);
    if (e < 0) return;
    codes = a.gu;
    scales = a.gus;
  } else {
    p0 = a.cap + (blockIdx.x - n_routed) * TM;
    e = 0;
    codes = a.sgu;
    scales = a.sgus;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, 2 * I, H);
  const rsrc_t ra = make_rsrc(a.x, (uint32_t)T * H * 2);
  uint32_t a_off[Stage<TK>::NQ];
#pragma unroll
  for (int q = 0; q < Stage<TK>::NQ; q++) {
    const int p = p0 + a_row_of<TK>(wave, lane, q);
    int tok;
    if (!is_shared) {
      const int f = a.sorted_ids[p];
      tok = f < P ? f / a.k : -1;
    } else {
      tok = p - a.cap < T ? p - a.cap : -1;
    }
    a_off[q] = tok >= 0 ? (uint32_t)tok * H * 2 : 0x80000000u;
  }
  const int brr = b_row_of<FMT, TK>(tid);
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
  tiled_k_loop<FMT, TK>(lds, ra, a_off, m, wrow, wvalid, 0, H / TK, H, brow, scale, acc);
  // epilogue: SwiGLU, h in bf16
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const size_t row = (size_t)(p0 + 64 * wm + 16 * i + 4 * g + jj);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int col = c0 + 32 * wn + 16 * j + r;
        if (col >= Il) continue;
        const float gv = acc[i][j][jj], uv = acc[i][j + 2][jj];
        a.h[row * Il + col] = bf16_bits(gv / (1.f + __expf(-gv)) * uv);
      }
    }
}

// ---------------------------------------------------------------- down

// Tile (blockIdx.x, blockIdx.y): h rows [p0, p0 + 128) and hidden columns [n0, n0 + 128);
// K = the slice [lo, hi).  Wave (wm, wn) owns rows 64 wm + [0,64), columns 64 wn + [0,64).
// The per-pair rows go to Y in bf16: at prefill sizes Y is the largest stream of the layer
// (pairs x H), and the combine weights and sums its rows in fp32.
template <int FMT>
__global__ __launch_bounds__(256, 2) void k_down_tiled(DownArgs a) {
  constexpr int TK = 32;
  __shared__ TileLDS<TK> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int n_routed = a.cap / TM;
  const bool is_shared = (int)blockIdx.x >= n_routed;
  const int n0 = blockIdx.y * TW;
  int p0, e;
  const uint8_t *codes, *scales;
  if (!is_shared) {
    p0 = blockIdx.x * TM;
    const int tp = a.total_padded[0], eb = a.block_expert[p0 / a.block_m];  // both in flight (p0 < cap)
    if (p0 >= __builtin_amdgcn_readfirstlane(tp)) return;
    e = __builtin_amdgcn_readfirstlane(eb);
    if (e < 0) return;
    codes = a.dn;
    scales = a.dns;
  } else {
    p0 = a.cap + (blockIdx.x - n_routed) * TM;
    e = 0;
    codes = a.sdn;
    scales = a.sdns;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, H, I);
  const rsrc_t ra = make_rsrc(a.h, (uint32_t)a.h_rows * Il * 2);
  uint32_t a_off[Stage<TK>::NQ];
#pragma unroll
  for (int q = 0; q < Stage<TK>::NQ; q++) a_off[q] = (uint32_t)(p0 + a_row_of<TK>(wave, lane, q)) * Il * 2;
  const uint32_t wrow = (uint32_t)(n0 + b_row_of<FMT, TK>(tid));
  const int brow[4] = {64 * wn, 64 * wn + 16, 64 * wn + 32, 64 * wn + 48};
  f32x4_t acc[4][4];
  zero_acc(acc);
  auto scale = [&](int kb, int j) {
    const int wr = n0 + 64 * wn + 16 * j;
    return buf_load_f32(m.scales, (uint32_t)((wr / 128) * (I / 128) + a.lo / 128 + kb) * 4);
  };
  tiled_k_loop<FMT, TK>(lds, ra, a_off, m, wrow, true, a.lo, (Il + TK - 1) / TK, Il, brow, scale, acc);
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int p = p0 + 64 * wm + 16 * i + 4 * g + jj;
      int dst;
      if (!is_shared) {
        const int f = a.sorted_ids[p];
        dst = f < P ? f : -1;
      } else {
        dst = p - a.cap < T ? P + (p - a.cap) : -1;
      }
      if (dst < 0) continue;
      uint16_t *yrow = reinterpret_cast<uint16_t *>(a.Y) + (size_t)dst * H + n0 + 64 * wn + r;
#pragma unroll
      for (int j = 0; j < 4; j++) yrow[16 * j] = bf16_bits(acc[i][j][jj]);
    }
}

// ---------------------------------------------------------------- router

// logits (or split-K partials) of many tokens: tile (blockIdx.x, blockIdx.y, blockIdx.z) =
// tokens [t0, t0 + 128) x experts [e0, e0 + 128) over K = [kbeg, kbeg + kchunk) of H; wave
// (wm, wn) owns tokens 64 wm + [0,64) and experts 64 wn + [0,64).  The bias is added here
// only without a K split (the top-k kernel adds it after summing the partials otherwise).
__global__ __launch_bounds__(256, 2) void k_router_tiled(const uint16_t *__restrict__ x, int T, int H,
                                                         const uint16_t *__restrict__ w, int E,
                                                         const float *__restrict__ bias, int kchunk,
                                                         float *__restrict__ part) {
  constexpr int TK = 64;
  __shared__ TileLDS<TK> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TW, kbeg = blockIdx.z * kchunk;
  const rsrc_t ra = make_rsrc(x, (uint32_t)T * H * 2);
  uint32_t a_off[Stage<TK>::NQ];
#pragma unroll
  for (int q = 0; q < Stage<TK>::NQ; q++) {
    const int t = t0 + a_row_of<TK>(wave, lane, q);
    a_off[q] = t < T ? (uint32_t)(t * H + kbeg) * 2 : 0x80000000u;
  }
  WMat<kFmtBf16> m;
  m.codes = m.scales = make_rsrc(w, (uint32_t)E * H * 2);
  m.K = H;
  const int ew = e0 + b_row_of<kFmtBf16, TK>(tid);
  const bool wvalid = ew < E;
  const int brow[4] = {64 * wn, 64 * wn + 16, 64 * wn + 32, 64 * wn + 48};
  f32x4_t acc[4][4];
  zero_acc(acc);
  auto noscale = [](int, int) { return 1.f; };
  tiled_k_loop<kFmtBf16, TK>(lds, ra, a_off, m, (uint32_t)(wvalid ? ew : 0), wvalid, kbeg, kchunk / TK, kchunk, brow,
                             noscale, acc);
  float* dst = part + (size_t)blockIdx.z * T * E;
  const bool add_bias = bias && gridDim.z == 1;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = e0 + 64 * wn + 16 * j + r;
    if (e >= E) continue;
    const float bv = add_bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int t = t0 + 64 * wm + 16 * i + 4 * g + jj;
        if (t < T) dst[(size_t)t * E + e] = acc[i][j][jj] + bv;
      }
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_router_tiled(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int ks,
                               float *part, hipStream_t s) {
  const dim3 grid((T + TM - 1) / TM, (E + TW - 1) / TW, ks);
  hipLaunchKernelGGL(k_router_tiled, grid, dim3(256), 0, s, x, T, H, w, E, bias, H / ks, part);
  return hipGetLastError();
}


hipError_t launch_gate_up_tiled(int fmt, const GateUpArgs &a, int n_shared_tiles, hipStream_t s) {
  const dim3 grid(a.cap / TM + n_shared_tiles, (a.Il + 63) / 64);
  if (fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_BF16 || fmt == MOE_FMT_FP8_BLOCK128) return launch_gate_up_wide(fmt, a, n_shared_tiles, s);
  hipLaunchKernelGGL(k_gate_up_tiled<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_tiled(int fmt, const DownArgs &a, int n_shared_tiles, hipStream_t s) {
  const dim3 grid(a.cap / TM + n_shared_tiles, a.H / TW);
  if (fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_BF16 || fmt == MOE_FMT_FP8_BLOCK128) return launch_down_wide(fmt, a, n_shared_tiles, s);
  hipLaunchKernelGGL(k_down_tiled<MOE_FMT_FP8_BLOCK128>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qmoe
