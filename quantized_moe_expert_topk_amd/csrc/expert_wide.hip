// expert_wide.hip -- NVFP4, fp8-block and bf16 expert GEMMs for many tokens per expert
// (prefill), gfx950.
//
// Same computation as the streaming kernels of expert.hip (gate rows [lo,hi), up rows
// [I+lo, I+hi), down columns [lo,hi) of one rank's slice: FreeToken issue #62 "What it
// touches" item 1; SwiGLU expert linear in the intermediate index: issue #520 section 4;
// NVFP4 W4A16 with the e4m3 group scale exact in bf16 and the per-row fp32 global applied
// to the fp32 result: issue #520 section 2; fp8-block weights with one fp32 scale per 128 x 128
// block: PR #637 "Implementation notes").
//
// Work split: a workgroup owns a 128-row block of the aligned pair list (one expert) and 256
// weight rows; each of its 4 waves owns all 128 rows x 64 weight rows, 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (the 32x32 form keeps the matrix core near its peak with one wave
// per SIMD, which the register budget here allows).  Only the activation tile goes through
// LDS (gathered x rows or h rows, 128 x 128 bf16 per K stage, double buffered, one barrier
// per stage).  The weights are read straight into registers in operand order: lane l of a
// wave holds weight row l % 32 of a 32-row tile and the contiguous K half
// [64 h, 64 h + 64) of each 128-wide stage (h = l / 32), i.e. two 16-byte code pieces of the
// tile-16 layout, and MFMA c of the stage takes K [64 h + 8 c, +8) from both operands.  Each
// wave dequantizes only its own 64 rows; per stage it runs 64 MFMAs against 4 KB of codes.
// bf16 weights (no dequantization, 2 bytes per weight) take 64-wide K stages instead, so that
// two stages of a lane's weights still fit its registers: lane l then holds K [32 h, 32 h + 32)
// of each stage, four 16-byte pieces.  fp8-block weights (1 byte each, but 128-wide activation
// stages would not fit beside them) take 64-wide stages too, two 16-byte pieces of 16 e4m3 per
// lane, converted exactly to bf16; two stages make one 128 x 128 scale block of each 32-row
// column tile.  The block scale cannot go into the bf16 operand exactly and a second set of
// accumulators does not fit, so each tile's accumulators are held in units of the current
// block's scale: entering a block with scale s' multiplies them by s / s' (s the previous
// block's), and the epilogue multiplies by the last scale.
//
// K loop: stage s multiplies from LDS buffer s%2 and weight register set s%2.  Meanwhile the
// activation loads of stage s+1 (issued as stage s starts, stored to the other LDS buffer as it
// ends) and the weight loads of stage s+1 (issued during stage s-1) are in flight; the weight
// loads of stage s+2 go out once set s%2 is consumed.
//
// Workgroup order: the dispatcher assigns workgroup L to XCD L mod 8.  The row blocks in use
// (the routed ones below total_padded, then the shared expert's) are dealt to the XCDs in
// turn, and the column groups of a row block, which share its activation rows, run back to
// back on the same XCD.  (Giving each XCD a contiguous run of row blocks instead, so that
// consecutive blocks of one expert share its weights in L2, measured slower.)
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace qmoe {
namespace {

constexpr int WM = 128;          // pair rows per workgroup (one align block of 128)
constexpr int WCOLS = 256;       // weight rows per workgroup (64 per wave)

// K per stage: 128 for NVFP4 (4 KB of codes per wave), 64 for bf16 (8 KB) and fp8-block (4 KB).
template <int FMT>
constexpr int kWideK = FMT == MOE_FMT_NVFP4 ? 128 : 64;

// Output tile of one wave after the K loop: 128 rows x 64 bf16, rows padded to 72 so that
// the two row groups a 32x32 result register covers (rows 4 apart) fall in different banks.
constexpr int OPITCH = 72;

struct __attribute__((aligned(16))) WideLDS {
  union {
    uint16_t a[2 * WM * 128];        // K loop: activation tiles, 2 x [128][WK] (32 or 16 KB each)
    uint16_t o[4][WM][OPITCH];       // epilogue: each wave's output tile, 4 x 18 KB
  };
  int32_t dst[WM];  // down: destination row of each pair row (-1: none)
};

// K chunk c (elements [8c, 8c+8)) of tile row R is stored XOR-swizzled so that a fragment read
// (16 consecutive rows, one chunk index per 16 lanes) and a row store touch every bank once:
// 256-byte rows (WK 128) at chunk c ^ (R & 15); 128-byte rows (WK 64, two rows per 256 bytes of
// banks) at chunk c ^ ((R >> 1) & 7).
template <int WK>
__device__ __forceinline__ int wswz(int R, int c) {
  return WK == 128 ? 8 * (c ^ (R & 15)) : 8 * (c ^ ((R >> 1) & 7));
}

// A thread's share of one activation stage: chunk tid % CPR of rows tid / CPR + RSTEP q.
template <int WK>
struct AStage {
  static constexpr int CPR = WK / 8, NQ = WM * CPR / 256, RSTEP = 256 / CPR;
  uint4 v[NQ];
};

// A lane's weights of one stage.  NVFP4: [column tile][piece] codes (32 e2m1 each) and the
// pieces' two e4m3 group scales; fp8-block: [column tile][piece] 16 e4m3 each and the tile's
// block scale; bf16: [column tile][piece] 8 bf16 each.
template <int FMT>
struct BStage {
  static constexpr int NP = FMT == MOE_FMT_BF16 ? 4 : 2;
  uint4 c[2][NP];
  uint32_t s[2][2];
  float bs[2];
};

// The pipelined K loop.  a_off: byte offsets of the K origin of the thread's 8 activation
// rows (0x80000000: a row that reads zeros).  cb/sb: tile-16 code and scale offsets of this
// lane's weight row in each of the wave's two 32-row column tiles (fp8-block: sb is the
// offset of the tile's row of block scales).  K runs over nK stages from weight column b_k0;
// positions at or past kvalid (a multiple of 32) contribute zero (TAIL: kvalid may end inside
// a stage; otherwise it is nK * WK).  fp8-block: post[ct] receives the scale the
// accumulators of column tile ct are left in units of (0 while every block scale was 0);
// b_k0 is a multiple of 128, so even stages start a scale block.
// AFFINE: the activation rows are consecutive, a_off[q] = a_off[0] + q * a_stride (down, whose
// h rows are; only a_off[0] is read, which keeps 7 registers free).
// WALK: the workgroup walks ncgs column groups of its row block in one pipeline.  Stage s of
// the walk is stage s % nK of column group s / nK; boff(cgl, cb, sb) gives the weight offsets of
// local column group cgl (cb/sb are then unused), and after the last stage of every group but
// the last, epi(cgl) stores that group's results from acc (post: fp8-block as above) and clears
// acc, between two barriers: its LDS tile overlaps the activation buffers.  Meanwhile the
// weight loads of the next two stages and the activation loads of the next stage (the first
// of the next group: the same rows) stay in flight.  The caller stores the last group after
// the loop, as without WALK.  fp8-block needs nK even (scale blocks start on even stages).
struct NoBOff {
  __device__ void operator()(int, uint32_t (&)[2], uint32_t (&)[2]) const {}
};
struct NoEpi {
  __device__ void operator()(int) const {}
};

// Wave priority over a stage's MFMA block: with two workgroups on a CU, the wave that holds
// its operands in registers issues its matrix ops ahead of the other workgroup's loads and
// address math, so the matrix core idles less.  Measured on MI355X (gate_up / down, us):
// fp8-block T = 4096, slice 256: 112.9 / 82.2 -> 103.5 / 81.6; bf16 T = 8192, full I:
// 459 / 306 -> 453 / 289.  NVFP4 runs without it: its in-register decode of the weights is
// vector work inside that block, and the raised priority slowed it (332 / 208 -> 337 / 214).
template <int FMT>
constexpr bool kWidePrio = FMT == MOE_FMT_FP8_BLOCK128 || FMT == MOE_FMT_BF16;

template <int FMT, bool TAIL, bool AFFINE, bool WALK = false, class BOff = NoBOff, class Epi = NoEpi>
__device__ __forceinline__ void wide_k_loop(WideLDS &lds, rsrc_t ra,
                                            const uint32_t (&a_off)[AStage<kWideK<FMT>>::NQ], uint32_t a_stride,
                                            const WMat<FMT> &m, const uint32_t (&cb)[2], const uint32_t (&sb)[2],
                                            int b_k0, int nK, int kvalid, f32x16_t (&acc)[4][2],
                                            float (&post)[2], int ncgs = 1, BOff boff = {}, Epi epi = {}) {
  constexpr int WK = kWideK<FMT>;
  using AS = AStage<WK>;
  using BS = BStage<FMT>;
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int ac = tid % AS::CPR;  // the activation chunk this thread stages
  AS at;
  BS bt[2];
  float scur[2] = {0.f, 0.f};  // fp8-block: the scale the accumulators are in units of
  uint32_t zm[2] = {~0u, ~0u};  // fp8-block: all ones while the current block's scale is nonzero
  auto abuf = [&](int st) { return &lds.a[(st & 1) * WM * WK]; };  // [WM][WK]
  auto fetch_a = [&](int st, AS &t) {
    const int k = st * WK + 8 * ac;
    const uint32_t kk = (uint32_t)(k < kvalid ? k : 0);
#pragma unroll
    for (int q = 0; q < AS::NQ; q++) t.v[q] = buf_load16(ra, (AFFINE ? a_off[0] + q * a_stride : a_off[q]) + kk * 2);
  };
  auto fetch_b_at = [&](int st, const uint32_t (&cb)[2], const uint32_t (&sb)[2], BS &t) {
    if constexpr (FMT == MOE_FMT_BF16) {  // pieces of 8: K [32 h + 8 p, +8) of the stage
      const int k = st * WK + 32 * h;
      const uint32_t pc = (uint32_t)(b_k0 + (k < kvalid ? k : 0)) / 8;
#pragma unroll
      for (int p = 0; p < 4; p++)
#pragma unroll
        for (int ct = 0; ct < 2; ct++) t.c[ct][p] = buf_load16(m.codes, cb[ct] + (pc + p) * 256);
    } else if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {  // pieces of 16: K [32 h + 16 p, +16)
      const int k = st * WK;
      const uint32_t kk = (uint32_t)(b_k0 + (k < kvalid ? k : 0));
      const uint32_t pc = kk / 16 + 2 * h;
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int ct = 0; ct < 2; ct++) t.c[ct][p] = buf_load16(m.codes, cb[ct] + (pc + p) * 256);
#pragma unroll
      for (int ct = 0; ct < 2; ct++) t.bs[ct] = buf_load_f32(m.scales, sb[ct] + kk / 128 * 4);
    } else {  // pieces of 32: K [64 h + 32 p, +32) of the stage
#pragma unroll
      for (int p = 0; p < 2; p++) {
        const int k = st * WK + 64 * h + 32 * p;
        const uint32_t pc = (uint32_t)(b_k0 + (k < kvalid ? k : 0)) / 32;
#pragma unroll
        for (int ct = 0; ct < 2; ct++) {
          t.c[ct][p] = buf_load16(m.codes, cb[ct] + pc * 256);
          t.s[ct][p] = buf_load2(m.scales, sb[ct] + pc * 32);
        }
      }
    }
  };
  // walk stage s: weights of stage s % nK of local column group s / nK (clamped to the last
  // group past the walk: unused loads at in-bounds offsets)
  auto fetch_b = [&](int s, BS &t) {
    if constexpr (WALK) {
      const int cgl = min(s / nK, ncgs - 1);
      uint32_t cbx[2], sbx[2];
      boff(cgl, cbx, sbx);
      fetch_b_at(s - cgl * nK, cbx, sbx, t);
    } else {
      fetch_b_at(s, cb, sb, t);
    }
  };
  // the activation tile of stage st (K position) into LDS buffer s % 2
  auto store_a = [&](int s, int st, const AS &t) {
    const bool ok = !TAIL || st * WK + 8 * ac < kvalid;
    uint16_t *b = abuf(s);
#pragma unroll
    for (int q = 0; q < AS::NQ; q++) {
      const int R = tid / AS::CPR + AS::RSTEP * q;
      *reinterpret_cast<uint4 *>(b + R * WK + wswz<WK>(R, ac)) = ok ? t.v[q] : make_uint4(0, 0, 0, 0);
    }
  };
  // MFMA c of a stage takes K [(WK / 2) h + 8 c, +8) in this lane.
  auto read_a = [&](int s, int c, frag8 (&f)[4]) {
    const uint16_t *b = abuf(s);
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
      f[mi].q = *reinterpret_cast<const uint4 *>(b + (32 * mi + r32) * WK + wswz<WK>(r32, (WK / 16) * h + c));
  };
  // fp8-block: a zero block scale clears the codes (zm), so that its block adds nothing
  auto dec_b = [&](int st, int c, const BS &t, frag8 (&f)[2]) {
    if constexpr (FMT == MOE_FMT_BF16) {
      const bool bvalid = !TAIL || st * WK + 32 * h < kvalid;
#pragma unroll
      for (int ct = 0; ct < 2; ct++) f[ct].q = bvalid ? t.c[ct][c] : make_uint4(0, 0, 0, 0);
    } else if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
      const int p = c >> 1;
      const bool bvalid = !TAIL || st * WK + 32 * h + 16 * p < kvalid;
#pragma unroll
      for (int ct = 0; ct < 2; ct++) {
        const uint4 &cv = t.c[ct][p];
        fp8x8_to_bf16(((c & 1) ? cv.z : cv.x) & zm[ct], ((c & 1) ? cv.w : cv.y) & zm[ct], f[ct]);
        if (!bvalid) f[ct].q = make_uint4(0, 0, 0, 0);
      }
    } else {
      const int p = c >> 2, d = c & 3;
      const bool bvalid = !TAIL || st * WK + 64 * h + 32 * p < kvalid;
#pragma unroll
      for (int ct = 0; ct < 2; ct++) {
        const uint4 &cv = t.c[ct][p];
        const uint32_t code = d == 0 ? cv.x : d == 1 ? cv.y : d == 2 ? cv.z : cv.w;
        fp4x8_mul_to_bf16(code, e4m3_to_f32(t.s[ct][p] >> (8 * (d >> 1))), f[ct]);
        if (!bvalid) f[ct].q = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // first: the stage starts an fp8 scale block (std::true_type or std::false_type)
  // walk stage s (LDS buffer s % 2) at K stage st
  auto compute = [&](int s, int st, const BS &t, auto first) {
    if constexpr (FMT == MOE_FMT_FP8_BLOCK128 && decltype(first)::value) {
#pragma unroll
      for (int ct = 0; ct < 2; ct++) {
        const float sn = t.bs[ct];
        const bool nz = sn != 0.f;
        const float r = nz ? scur[ct] / sn : 1.f;
        scur[ct] = nz ? sn : scur[ct];
        zm[ct] = nz ? ~0u : 0u;
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
#pragma unroll
          for (int j = 0; j < 16; j++) acc[mi][ct][j] *= r;
      }
    }
    if constexpr (kWidePrio<FMT>) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < WK / 16; c++) {
      frag8 af[4], bf[2];
      read_a(s, c, af);
      dec_b(st, c, t, bf);
#pragma unroll
      for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int ct = 0; ct < 2; ct++) acc[mi][ct] = mfma32_bf16(af[mi], bf[ct], acc[mi][ct]);
    }
    if constexpr (kWidePrio<FMT>) __builtin_amdgcn_s_setprio(0);
  };
  fetch_a(0, at);
  fetch_b(0, bt[0]);
  fetch_b(1, bt[1]);
  store_a(0, 0, at);
  __syncthreads();
  // Fetches past the last stage reload clamped offsets (unused) and the store after the
  // last stage fills the idle buffer with zeros, so every path keeps the same loads in flight.
  if constexpr (!WALK) {
    auto stage = [&](int st, BS &b_cur, auto first) {
      fetch_a(st + 1, at);
      compute(st, st, b_cur, first);
      fetch_b(st + 2, b_cur);
      store_a(st + 1, st + 1, at);
      __syncthreads();
    };
    int st = 0;
    for (; st + 1 < nK; st += 2) {
      stage(st, bt[0], std::true_type{});
      stage(st + 1, bt[1], std::false_type{});
    }
    if (st < nK) stage(st, bt[0], std::true_type{});
  } else {
    const int S = ncgs * nK;
    auto stage = [&](int s, int st, BS &b_cur, auto first) __attribute__((always_inline)) {
      const int stn = st + 1 == nK ? 0 : st + 1;
      fetch_a(stn, at);
      compute(s, st, b_cur, first);
      fetch_b(s + 2, b_cur);
      if (stn == 0 && s + 1 < S) {  // a column group ends and another follows
        __syncthreads();
        if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
          post[0] = scur[0];
          post[1] = scur[1];
        }
        epi(s / nK);
        __syncthreads();
      }
      store_a(s + 1, stn, at);
      __syncthreads();
      return stn;
    };
    int s = 0, st = 0;
    for (; s + 1 < S; s += 2) {
      st = stage(s, st, bt[0], std::true_type{});
      st = stage(s + 1, st, bt[1], std::false_type{});
    }
    if (s < S) stage(s, st, bt[0], std::true_type{});
  }
  if constexpr (FMT == MOE_FMT_FP8_BLOCK128) {
    post[0] = scur[0];
    post[1] = scur[1];
  }
}

// Grid position -> (row block index idx among those in use, column group cg); see the
// workgroup order above.  Positions idx < n_used are routed row block idx; the next ones are
// the shared expert's row blocks; the rest have no work.  The kernels load the routed block's
// expert and pair ids at idx (clamped) together with total_padded, before they know which
// case holds: one dependent round trip fewer before the first activation and weight loads.
__device__ __forceinline__ void wide_position(int ncg, int &idx, int &cg) {
  const int L = blockIdx.x, j = L >> 3;
  idx = (j / ncg) * 8 + (L & 7);
  cg = j % ncg;
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int mi = 0; mi < 4; mi++)
#pragma unroll
    for (int ct = 0; ct < 2; ct++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[mi][ct][j] = 0.f;
}

// Row of the 32-row tile that register j of this lane holds.
__device__ __forceinline__ int d_row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

}  // namespace

// gate_up + SwiGLU.  Column group cg covers slice columns [c0, c0 + 128): wave w owns gate
// rows lo + c0 + 32 w + [0, 32) (column tile 0) and the matching up rows I + ... (column
// tile 1), so SwiGLU stays in registers.
template <int FMT>
__global__ __launch_bounds__(256, 2) void k_gate_up_wide(GateUpArgs a, int n_rb, int ncg) {
  constexpr int WK = kWideK<FMT>;
  using AS = AStage<WK>;
  __shared__ WideLDS lds;
  const int n_routed = a.cap / WM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int idx, cg;
  wide_position(ncg, idx, cg);
  const int ridx = max(0, min(idx, n_routed - 1));  // the routed row block idx would be
  const int tp = a.total_padded[0];
  const int eb = a.block_expert[ridx * WM / a.block_m];
  int sf[AS::NQ];  // pair ids of this thread's rows of that block
#pragma unroll
  for (int q = 0; q < AS::NQ; q++) sf[q] = a.sorted_ids[ridx * WM + tid / AS::CPR + AS::RSTEP * q];
  // all of them in flight before the first wait (left alone, the compiler moves the loads
  // whose values only the routed path uses below the exit test)
  asm volatile("" ::"s"(tp), "s"(eb));
#pragma unroll
  for (int q = 0; q < AS::NQ; q++) asm volatile("" ::"v"(sf[q]));
  const int n_used = __builtin_amdgcn_readfirstlane(tp) / WM;
  if (idx >= n_used + (n_rb - n_routed)) return;
  const bool is_shared = idx >= n_used;
  const int rb = is_shared ? n_routed + (idx - n_used) : idx;
  const int c0 = cg * (WCOLS / 2);
  int p0, e;
  const uint8_t *codes, *scales;
  const float *glob;
  if (!is_shared) {
    p0 = rb * WM;
    e = __builtin_amdgcn_readfirstlane(eb);
    if (e < 0) return;
    codes = a.gu;
    scales = a.gus;
    glob = a.gug;
  } else {
    p0 = a.cap + (rb - n_routed) * WM;
    e = 0;
    codes = a.sgu;
    scales = a.sgus;
    glob = a.sgug;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, 2 * I, H);
  const rsrc_t ra = make_rsrc(a.x, (uint32_t)T * H * 2);
  uint32_t a_off[AS::NQ];
#pragma unroll
  for (int q = 0; q < AS::NQ; q++) {
    const int p = p0 + tid / AS::CPR + AS::RSTEP * q;
    int tok;
    if (!is_shared) {
      const int f = sf[q];
      tok = f < P ? f / a.k : -1;
    } else {
      tok = p - a.cap < T ? p - a.cap : -1;
    }
    a_off[q] = tok >= 0 ? (uint32_t)tok * H * 2 : 0x80000000u;
  }
  const int col = c0 + 32 * wave + (lane & 31);  // this lane's slice column (B operand and D)
  const int cc = col < Il ? col : (lane & 31);   // columns past the slice read row lane%32 (unused)
  uint32_t cb[2], sb[2];
#pragma unroll
  for (int ct = 0; ct < 2; ct++) {
    const uint32_t row = (uint32_t)((ct == 0 ? 0 : I) + a.lo + cc);
    cb[ct] = (row & ~15u) * (uint32_t)(FMT == MOE_FMT_BF16 ? 2 * H : FMT == MOE_FMT_FP8_BLOCK128 ? H : H / 2) +
             (row & 15u) * 16;
    sb[ct] = FMT == MOE_FMT_FP8_BLOCK128 ? row / 128 * (uint32_t)(H / 128) * 4
                                         : (row & ~15u) * (uint32_t)(H / 16) + (row & 15u) * 2;
  }
  float post[2] = {FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + a.lo + cc] : 1.f,
                   FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * 2 * I + I + a.lo + cc] : 1.f};
  f32x16_t acc[4][2];
  zero_acc(acc);
  wide_k_loop<FMT, false, false>(lds, ra, a_off, 0, m, cb, sb, 0, H / WK, H, acc, post);
  // h through LDS (the K loop ended with a barrier): each wave's 128 x 32 block, then rows
  // leave as 16-byte chunks (4 lanes per 64-byte row segment)
  uint16_t (*o)[OPITCH] = lds.o[wave];
#pragma unroll
  for (int mi = 0; mi < 4; mi++)
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float gv = acc[mi][0][j] * post[0], uv = acc[mi][1][j] * post[1];
      o[32 * mi + d_row(lane, j)][lane & 31] = bf16_bits(gv / (1.f + __expf(-gv)) * uv);
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int ch = lane & 3, c8 = c0 + 32 * wave + 8 * ch;  // this lane's 8 columns
  if (c8 < Il) {
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const int R = (lane >> 2) + 16 * q;
      *reinterpret_cast<uint4 *>(a.h + (size_t)(p0 + R) * Il + c8) = *reinterpret_cast<const uint4 *>(&o[R][8 * ch]);
    }
  }
}

// down.  Column group cg covers hidden columns [cg * 256, +256): wave w owns 64 w + [0, 64)
// of them (two 32-column tiles); K = the slice.  The pair rows go to Y in bf16 (the combine
// weights and sums them in fp32), as in the other prefill kernels.  K is only the slice width
// (2 to 8 stages), so for fp8-block a workgroup walks cgw consecutive column groups of its row
// block in one pipeline (chunk ch of the grid: groups [ch cgw, ch cgw + cgw) past H clipped):
// the metadata loads, the pipeline fill and the workgroup launch are paid once per walk, and
// each group's stores overlap the next group's first weight loads.  Measured on MI355X, fp8-block
// layer T = 4096, slice 256: 88.9 -> 82.4 us with walks of 2 groups (4: 93.9, 8: 99.7).  NVFP4
// and bf16 keep one group per workgroup: their walk spills registers at the 256-register budget
// and measured slower (NVFP4 prefill T = 8192, full I: 205 -> 222 us at 2 groups).
template <int FMT>
constexpr bool kDownWalk = FMT == MOE_FMT_FP8_BLOCK128;

template <int FMT>
__global__ __launch_bounds__(256, 2) void k_down_wide(DownArgs a, int n_rb, int nch, int cgw) {
  constexpr int WK = kWideK<FMT>;
  using AS = AStage<WK>;
  __shared__ WideLDS lds;
  const int n_routed = a.cap / WM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int idx, ch;
  wide_position(nch, idx, ch);
  const int ridx = max(0, min(idx, n_routed - 1));  // the routed row block idx would be
  const int tp = a.total_padded[0];
  const int eb = a.block_expert[ridx * WM / a.block_m];
  const int sd = tid < WM ? a.sorted_ids[ridx * WM + tid] : 0;  // pair id of row tid of that block
  asm volatile("" ::"s"(tp), "s"(eb), "v"(sd));  // all in flight before the first wait (see gate_up)
  const int n_used = __builtin_amdgcn_readfirstlane(tp) / WM;
  if (idx >= n_used + (n_rb - n_routed)) return;
  const bool is_shared = idx >= n_used;
  const int rb = is_shared ? n_routed + (idx - n_used) : idx;
  int p0, e;
  const uint8_t *codes, *scales;
  const float *glob;
  if (!is_shared) {
    p0 = rb * WM;
    e = __builtin_amdgcn_readfirstlane(eb);
    if (e < 0) return;
    codes = a.dn;
    scales = a.dns;
    glob = a.dng;
  } else {
    p0 = a.cap + (rb - n_routed) * WM;
    e = 0;
    codes = a.sdn;
    scales = a.sdns;
    glob = a.sdng;
  }
  const int T = a.T, H = a.H, I = a.I, Il = a.Il, P = a.T * a.k;
  const int cg0 = ch * cgw, ncgs = min(cgw, (H + WCOLS - 1) / WCOLS - cg0);  // this walk's column groups
  const WMat<FMT> m = weight_matrix<FMT>(codes, scales, e, H, I);
  const rsrc_t ra = make_rsrc(a.h, (uint32_t)a.h_rows * Il * 2);
  uint32_t a_off[AS::NQ] = {(uint32_t)(p0 + tid / AS::CPR) * Il * 2};  // rows RSTEP apart
  const uint32_t a_stride = (uint32_t)AS::RSTEP * Il * 2;
  // weight row of tile ct of local column group cgl (columns past H read row lane % 32, unused)
  auto wrow = [&](int cgl, int ct) __attribute__((always_inline)) {
    const int n = (cg0 + cgl) * WCOLS + 64 * wave + 32 * ct + (lane & 31);
    return (uint32_t)(n < H ? n : (lane & 31));
  };
  auto boff = [&](int cgl, uint32_t (&cb)[2], uint32_t (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < 2; ct++) {
      const uint32_t row = wrow(cgl, ct);
      cb[ct] = (row & ~15u) * (uint32_t)(FMT == MOE_FMT_BF16 ? 2 * I : FMT == MOE_FMT_FP8_BLOCK128 ? I : I / 2) +
               (row & 15u) * 16;
      sb[ct] = FMT == MOE_FMT_FP8_BLOCK128 ? row / 128 * (uint32_t)(I / 128) * 4
                                           : (row & ~15u) * (uint32_t)(I / 16) + (row & 15u) * 2;
    }
  };
  uint32_t cb[2], sb[2];
  boff(0, cb, sb);
  float dg[2];  // NVFP4: the per-row globals of the current column group; the loop's post
#pragma unroll
  for (int ct = 0; ct < 2; ct++) dg[ct] = FMT == MOE_FMT_NVFP4 ? glob[(size_t)e * H + wrow(0, ct)] : 1.f;
  if (tid < WM) {  // destination of each pair row, read back in every epilogue
    const int p = p0 + tid;
    if (!is_shared) {
      lds.dst[tid] = sd < P ? sd : -1;
    } else {
      lds.dst[tid] = p - a.cap < T ? P + (p - a.cap) : -1;
    }
  }
  f32x16_t acc[4][2];
  zero_acc(acc);
  // pair rows of local column group cgl through LDS (called after a barrier, which also
  // published dst): each wave's 128 x 64 block, then 16-byte chunks (8 lanes per 128-byte row)
  auto store_rows = [&](int cgl) __attribute__((always_inline)) {
    uint16_t (*o)[OPITCH] = lds.o[wave];
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int R = 32 * mi + d_row(lane, j);
#pragma unroll
        for (int ct = 0; ct < 2; ct++) o[R][32 * ct + (lane & 31)] = bf16_bits(acc[mi][ct][j] * dg[ct]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int ch8 = lane & 7, n8 = (cg0 + cgl) * WCOLS + 64 * wave + 8 * ch8;  // this lane's 8 columns
    if (n8 < H) {
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const int R = (lane >> 3) + 8 * q;
        const int d = lds.dst[R];
        if (d >= 0)
          *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.Y) + (size_t)d * H + n8) =
              *reinterpret_cast<const uint4 *>(&o[R][8 * ch8]);
      }
    }
  };
  // between column groups: store the finished one, clear acc, load the next group's globals
  auto epi = [&](int cgl) __attribute__((always_inline)) {
    store_rows(cgl);
    zero_acc(acc);
    if constexpr (FMT == MOE_FMT_NVFP4) {
#pragma unroll
      for (int ct = 0; ct < 2; ct++) dg[ct] = glob[(size_t)e * H + wrow(cgl + 1, ct)];
    }
  };
  constexpr bool W = kDownWalk<FMT>;
  if (Il % WK == 0)
    wide_k_loop<FMT, false, true, W>(lds, ra, a_off, a_stride, m, cb, sb, a.lo, Il / WK, Il, acc, dg, ncgs, boff, epi);
  else
    wide_k_loop<FMT, true, true, W>(lds, ra, a_off, a_stride, m, cb, sb, a.lo, (Il + WK - 1) / WK, Il, acc, dg, ncgs,
                                    boff, epi);
  store_rows(ncgs - 1);  // the K loop ended with a barrier
}

hipError_t launch_gate_up_wide(int fmt, const GateUpArgs &a, int n_shared_tiles, hipStream_t s) {
  const int n_rb = a.cap / WM + n_shared_tiles, ncg = (a.Il + WCOLS / 2 - 1) / (WCOLS / 2);
  const int grid = (n_rb + 7) / 8 * 8 * ncg;
  if (fmt == MOE_FMT_BF16)
    hipLaunchKernelGGL(k_gate_up_wide<MOE_FMT_BF16>, dim3(grid), dim3(256), 0, s, a, n_rb, ncg);
  else if (fmt == MOE_FMT_FP8_BLOCK128)
    hipLaunchKernelGGL(k_gate_up_wide<MOE_FMT_FP8_BLOCK128>, dim3(grid), dim3(256), 0, s, a, n_rb, ncg);
  else if (fmt == MOE_FMT_NVFP4)
    hipLaunchKernelGGL(k_gate_up_wide<MOE_FMT_NVFP4>, dim3(grid), dim3(256), 0, s, a, n_rb, ncg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_down_wide(int fmt, const DownArgs &a, int n_shared_tiles, hipStream_t s) {
  const int n_rb = a.cap / WM + n_shared_tiles, ncg = (a.H + WCOLS - 1) / WCOLS;
  const int cgw = fmt == MOE_FMT_FP8_BLOCK128 ? (ncg < 2 ? ncg : 2) : 1;  // column groups per workgroup
  const int nch = (ncg + cgw - 1) / cgw;
  const int grid = (n_rb + 7) / 8 * 8 * nch;
  if (fmt == MOE_FMT_BF16)
    hipLaunchKernelGGL(k_down_wide<MOE_FMT_BF16>, dim3(grid), dim3(256), 0, s, a, n_rb, nch, cgw);
  else if (fmt == MOE_FMT_FP8_BLOCK128)
    hipLaunchKernelGGL(k_down_wide<MOE_FMT_FP8_BLOCK128>, dim3(grid), dim3(256), 0, s, a, n_rb, nch, cgw);
  else if (fmt == MOE_FMT_NVFP4)
    hipLaunchKernelGGL(k_down_wide<MOE_FMT_NVFP4>, dim3(grid), dim3(256), 0, s, a, n_rb, nch, cgw);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qmoe
