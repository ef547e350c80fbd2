// router_tiled.hip -- the router GEMM for many tokens (logits = x W_r^T (+ bias); routing
// rule: issue #62, second comment), gfx950.
//
// A workgroup owns 128 tokens x 128 experts and walks K (the hidden dimension, or one split-K
// range of it) in stages of 64.  Per stage the token tile (bf16 rows of x) and the router
// weight tile (bf16 rows of W_r) are staged in LDS; 4 waves then run 2 x 2 blocks of 64 x 64
// outputs on v_mfma_f32_16x16x32_bf16.  LDS is double buffered: the global loads run two
// stages ahead in registers, and one barrier per stage separates the buffers.
#include "device_common.h"
#include "launch.h"

namespace qmoe {
namespace {

constexpr int TM = 128;  // tokens per tile
constexpr int TW = 128;  // experts per tile
constexpr int TK = 64;   // K per stage
constexpr int CPR = TK / 8;    // 16-byte chunks per LDS row
constexpr int NQ = CPR / 2;    // token-row chunks each thread stages per stage
constexpr int RPI = 64 / CPR;  // tile rows one wave instruction covers when staging

// K chunk c (elements [8c, 8c+8)) of tile row R sits at chunk c ^ (R & 7) of its 128-byte
// row, so that the MFMA operand reads (16 rows x one chunk per 16 lanes) and the stores run
// at full LDS bandwidth; a plain or padded pitch does not reach it for 16-row reads.
__device__ __forceinline__ int swz(int row, int chunk) { return 8 * (chunk ^ (row & 7)); }

struct TileLDS {
  uint16_t a[2][TM][TK];
  uint16_t b[2][TW][TK];
};

// Token tile: thread chunk q covers row 32 wave + RPI q + lane / CPR, K chunk lane % CPR
// (adjacent lanes read one row's 128 bytes).
__device__ __forceinline__ int a_row_of(int wave, int lane, int q) { return 32 * wave + RPI * q + lane / CPR; }

// Weight tile: thread tid stages row tid / 2, K half tid % 2 (32 weights, 64 bytes).
struct ATile {
  uint4 v[NQ];
};
struct BTile {
  uint4 c[4];
};

__device__ __forceinline__ void a_fetch(rsrc_t ra, const uint32_t (&row_off)[NQ], int k0, int lane, ATile &t) {
#pragma unroll
  for (int q = 0; q < NQ; q++) t.v[q] = buf_load16(ra, row_off[q] + (uint32_t)(k0 + 8 * (lane % CPR)) * 2);
}

__device__ __forceinline__ void a_store(uint16_t (*la)[TK], const ATile &t, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < NQ; q++) {
    const int row = a_row_of(wave, lane, q);
    *reinterpret_cast<uint4 *>(&la[row][swz(row, lane % CPR)]) = t.v[q];
  }
}

// Elements [ks + 32 half, +32) of weight row `row` (row-major [E][K]).
__device__ __forceinline__ void b_fetch(rsrc_t w, uint32_t K, uint32_t row, int ks, int half, BTile &t) {
  const uint32_t o = (row * K + ks + 32 * half) * 2;
#pragma unroll
  for (int q = 0; q < 4; q++) t.c[q] = buf_load16(w, o + 16 * q);
}

__device__ __forceinline__ void b_store(uint16_t *rowp, int row, int half, const BTile &t, bool valid) {
#pragma unroll
  for (int q = 0; q < 4; q++)
    *reinterpret_cast<uint4 *>(rowp + swz(row, 4 * half + q)) = valid ? t.c[q] : make_uint4(0, 0, 0, 0);
}

// acc[i][j] += token rows (a_row0 + 16 i) x expert rows brow[j], over the stage's K.
__device__ __forceinline__ void mma_stage(const uint16_t (*la)[TK], const uint16_t (*lb)[TK], int a_row0,
                                          const int (&brow)[4], int lane, f32x4_t (&acc)[4][4]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < TK; kk += 32) {
    frag8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      a[i].q = *reinterpret_cast<const uint4 *>(&la[a_row0 + 16 * i + r][swz(r, kk / 8 + g)]);
#pragma unroll
    for (int j = 0; j < 4; j++) b[j].q = *reinterpret_cast<const uint4 *>(&lb[brow[j] + r][swz(r, kk / 8 + g)]);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
  }
}

}  // namespace

// logits (or split-K partials) of many tokens: tile (blockIdx.x, blockIdx.y, blockIdx.z) =
// tokens [t0, t0 + 128) x experts [e0, e0 + 128) over K = [kbeg, kbeg + kchunk) of H; wave
// (wm, wn) owns tokens 64 wm + [0,64) and experts 64 wn + [0,64).  The bias is added here
// only without a K split (the top-k kernel adds it after summing the partials otherwise).
__global__ __launch_bounds__(256, 2) void k_router_tiled(const uint16_t *__restrict__ x, int T, int H,
                                                         const uint16_t *__restrict__ w, int E,
                                                         const float *__restrict__ bias, int kchunk,
                                                         float *__restrict__ part) {
  __shared__ TileLDS lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4, wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TW, kbeg = blockIdx.z * kchunk;
  const rsrc_t ra = make_rsrc(x, (uint32_t)T * H * 2);
  const rsrc_t rw = make_rsrc(w, (uint32_t)E * H * 2);
  uint32_t a_off[NQ];
#pragma unroll
  for (int q = 0; q < NQ; q++) {
    const int t = t0 + a_row_of(wave, lane, q);
    a_off[q] = t < T ? (uint32_t)(t * H + kbeg) * 2 : 0x80000000u;
  }
  const int brr = tid >> 1, bhalf = tid & 1;
  const int ew = e0 + brr;
  const bool wvalid = ew < E;
  const uint32_t wrow = (uint32_t)(wvalid ? ew : 0);
  const int brow[4] = {64 * wn, 64 * wn + 16, 64 * wn + 32, 64 * wn + 48};
  const int a_row0 = wm * 64, nK = kchunk / TK;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = zero4();
  ATile at[2];
  BTile bt[2];
  auto fetch = [&](int st, ATile &ta, BTile &tb) {  // weight loads first: oldest in the queue
    b_fetch(rw, (uint32_t)H, wrow, kbeg + st * TK, bhalf, tb);
    a_fetch(ra, a_off, st * TK, lane, ta);
  };
  auto store = [&](int st, const ATile &ta, const BTile &tb) {
    a_store(lds.a[st & 1], ta, wave, lane);
    b_store(lds.b[st & 1][brr], brr, bhalf, tb, wvalid);
  };
  // Fetches are unconditional (stages past the end reload the last one, unused) so that
  // every path has the same loads in flight and the compiler's waits stay partial.
  fetch(0, at[0], bt[0]);
  fetch(nK > 1 ? 1 : 0, at[1], bt[1]);
  store(0, at[0], bt[0]);
  __syncthreads();
  auto stage = [&](int st, ATile &ta_free, BTile &tb_free, const ATile &ta_next, const BTile &tb_next) {
    fetch(st + 2 < nK ? st + 2 : nK - 1, ta_free, tb_free);
    mma_stage(lds.a[st & 1], lds.b[st & 1], a_row0, brow, lane, acc);
    // after the last stage this fills the idle buffer, which nobody reads
    store(st + 1, ta_next, tb_next);
    __syncthreads();
  };
  int st = 0;
  for (; st + 1 < nK; st += 2) {
    stage(st, at[0], bt[0], at[1], bt[1]);
    stage(st + 1, at[1], bt[1], at[0], bt[0]);
  }
  if (st < nK) stage(st, at[0], bt[0], at[1], bt[1]);  // odd stage count: the last one, peeled
  float *dst = part + (size_t)blockIdx.z * T * E;
  const bool add_bias = bias && gridDim.z == 1;
  static_assert(sizeof(TileLDS) >= sizeof(float) * TM * TW, "the output tile fits the stage buffers");
  if (E % 4 == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0) {
    // The tile leaves through LDS (the stage buffers, 64 KB = 128 x 128 fp32; the K loop ended
    // with a barrier) as 16-byte pieces of whole rows, 32 lanes per row of 128 experts, instead of
    // 64-byte pieces of four rows per store (the path below, for other E or an unaligned part).
    // Measured on MI355X, E = 256, 16.8 MB of partials: T = 8192 27.0 -> 20.6 us, T = 4096
    // 21.0 -> 14.5 us (a timing copy without any stores: 19.9 and 13.0 us).
    float(*ot)[TW] = reinterpret_cast<float(*)[TW]>(&lds);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++) ot[64 * wm + 16 * i + 4 * g + jj][64 * wn + 16 * j + r] = acc[i][j][jj];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TM * TW / 4 / 256; q++) {
      const int c = tid + 256 * q, row = c / (TW / 4), e = e0 + 4 * (c % (TW / 4)), t = t0 + row;
      if (t < T && e < E) {
        float4 v = *reinterpret_cast<const float4 *>(&ot[row][e - e0]);
        if (add_bias) {
          v.x += bias[e];
          v.y += bias[e + 1];
          v.z += bias[e + 2];
          v.w += bias[e + 3];
        }
        *reinterpret_cast<float4 *>(&dst[(size_t)t * E + e]) = v;
      }
    }
    return;
  }
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

hipError_t launch_router_tiled(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int ks,
                               float *part, hipStream_t s) {
  const dim3 grid((T + TM - 1) / TM, (E + TW - 1) / TW, ks);
  hipLaunchKernelGGL(k_router_tiled, grid, dim3(256), 0, s, x, T, H, w, E, bias, H / ks, part);
  return hipGetLastError();
}

}  // namespace qmoe
