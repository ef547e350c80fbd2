// launch.h -- internal interface between the host-side ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

struct GateUpArgs {
  const uint16_t *x;  // [T, H] bf16
  int T, H, k;
  const uint8_t *gu;  // routed bank gate_up codes (all experts)
  const uint8_t *gus; // routed gate_up scales
  const float *gug;   // routed gate_up globals (NVFP4) or null
  const uint8_t *sgu, *sgus;  // shared bank (1 expert) or null
  const float *sgug;
  int E, I;
  const int32_t *sorted_ids, *block_expert, *total_padded;
  int block_m, cap, n_routed_sub;  // routed 16-row sub-blocks launched (<= cap / 16, see abi.cpp)
  int lo, Il;
  int kwaves, ksteps;  // K split of gate_up: kwaves waves x ksteps steps of 128 (H = 128*kwaves*ksteps)
  int cols_fastest;    // streaming kernels: grid x is the column group (else the 16-row sub-block)
  int nt_weights;      // streaming kernels: non-temporal weight loads (many pairs)
  uint16_t *h;  // [h_rows, Il] bf16 (NVFP4, fp8-block)
  int h_rows;   // cap + 16 * n_shared_sub
  // MXFP4: x and h as two e4m3 planes with e8m0 scales per 32 (plane 1 follows plane 0)
  const uint8_t *xq, *xs;  // [2][T][H], [2][T][H/32]
  uint8_t *hq, *hs;        // [2][h_rows][Il], [2][h_rows][Il/32]
  // Whole-layer call for one token (route1 != 0): the routed workgroups rank the router's
  // logits themselves instead of reading an alignment; workgroup 0 writes the routing and the
  // alignment outputs (the same arrays as sorted_ids, block_expert and total_padded above).
  int route1;
  const float *r_part;  // [r_ks][E] split-K partial logits, or the logits with the bias (r_ks == 1)
  const float *r_bias;  // [E] added after the partials, or NULL
  int r_ks;            // splits in r_part
  int r_renorm;
  float *r_logits;      // [E] output, or NULL
  int32_t *r_ids;       // [k] output
  float *r_w;           // [k] output
  int32_t *al_sorted, *al_block, *al_counts, *al_offsets, *al_total;
};

struct DownArgs {
  const uint16_t *h;
  const uint8_t *hq, *hs;  // MXFP4 (see GateUpArgs)
  int h_rows;  // rows of h (cap + shared rows)
  int T, H, k;
  const uint8_t *dn, *dns;
  const float *dng;
  const uint8_t *sdn, *sdns;
  const float *sdng;
  int E, I;
  const int32_t *sorted_ids, *block_expert, *total_padded;
  int block_m, cap, n_routed_sub;
  int lo, Il;
  int cols_fastest;  // as in GateUpArgs; k_down then keeps the column groups of a sub-block on one XCD
  int nt_weights;    // as in GateUpArgs
  float *Y;  // [T * k + T_shared, H] unweighted pair rows: fp32 (streaming kernels) or bf16 (prefill GEMMs)
};

// Host side of the ABI (abi.cpp): record the detail text of a failing call (returns code),
// and run every argument check of moe_expert_forward, giving the workspace bytes it needs.
int set_last_error(int code, const char *msg);
int forward_workspace_need(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                           const float *topk_w, const moe_align_out *al, int lo, int hi, void *out, int out_dtype,
                           size_t *need);

int router_ksplit(int T, int E, int H);
size_t router_workspace_bytes(int T, int E, int H);
// MXFP4 activation planes of x (ActMX layout: q [2][T][H] e4m3, s [2][T][H/32] e8m0) for the
// router GEMM to write alongside the logits, where router_writes_planes(T).
struct XPlanes {
  uint8_t *q, *s;
};
bool router_writes_planes(int T);
// The router GEMM of launch_route alone: split-K partials into partial when it splits K
// (*ks > 1), else the logits with the bias added into logits; xp: also the planes, or NULL.
hipError_t launch_router(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias,
                         float *logits, float *partial, int *ks, const XPlanes *xp, hipStream_t s);
hipError_t launch_route(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int k,
                        int renormalize, float *logits, int32_t *ids, float *wts, float *partial,
                        hipStream_t s);
hipError_t launch_router_tiled(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int ks,
                               float *part, hipStream_t s);
hipError_t launch_topk(const float *logits, int T, int E, const float *bias, int k, int renormalize,
                       int32_t *ids, float *wts, hipStream_t s);
hipError_t launch_align(const int32_t *ids, int T, int k, int E, int BM, int cap, int32_t *sorted_ids,
                        int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded,
                        int32_t *hist, hipStream_t s);
// route + align: one router GEMV and one top-k + align workgroup when route_align_fused(T, E, k),
// else launch_route then launch_align.  partial and hist as for those two.
bool route_align_fused(int T, int E, int k);
hipError_t launch_route_align(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int k,
                              int renormalize, float *logits, int32_t *ids, float *wts, float *partial, int BM,
                              int cap, int32_t *sorted_ids, int32_t *block_expert, int32_t *counts,
                              int32_t *offsets, int32_t *total_padded, int32_t *hist, hipStream_t s,
                              const XPlanes *xp = nullptr);
hipError_t launch_gate_up(int fmt, const GateUpArgs &a, int n_shared_sub, hipStream_t s);
hipError_t launch_down(int fmt, const DownArgs &a, int n_shared_sub, hipStream_t s);
// One token: down and the combine in one launch (16 waves per 64 hidden columns, one per
// sub-block) when down_t1_fused(fmt, a, has_shared); writes out directly.
bool down_t1_fused(int fmt, const DownArgs &a, int has_shared);
hipError_t launch_down_t1(int fmt, const DownArgs &a, const float *topk_w, void *out, int out_bf16, hipStream_t s);
// Prefill GEMMs for align blocks of 128 rows (NVFP4, FP8_BLOCK128, BF16) with only the
// activation tile in LDS (128 pair rows x 256 weight rows per workgroup); the shared expert's
// rows are ceil(T/128) row blocks after the routed ones.
hipError_t launch_gate_up_wide(int fmt, const GateUpArgs &a, int n_shared_tiles, hipStream_t s);
hipError_t launch_down_wide(int fmt, const DownArgs &a, int n_shared_tiles, hipStream_t s);
// moe_pack_bank: [rows, pitch] bytes -> 16-row tiles stored piece-major in units of `unit`
// (16, 8, 2 or 1) bytes.
hipError_t launch_pack_tile16(const void *src, void *dst, size_t rows, uint32_t pitch, int unit, hipStream_t s);
// Same destination order from E column-major matrices: src[e] is [pitch, N] bytes (row n of
// the destination = column n of the source), unit 16 or 1.
hipError_t launch_pack_tile16_t(const void *src, void *dst, size_t E, size_t N, uint32_t pitch, int unit,
                                hipStream_t s);
// Q4_0 codes [rows, pitch] -> the tile-16 piece order with the nibbles regrouped per piece.
hipError_t launch_pack_q4_0(const void *src, void *dst, size_t rows, uint32_t pitch, hipStream_t s);
hipError_t launch_act_mx8(const uint16_t *x, int rows, int K, uint8_t *q, uint8_t *sc, hipStream_t s);
// Y rows (unweighted) in fp32 (streaming kernels) or bf16 (prefill GEMMs); the combine applies
// the routing weights topk_w [T * k].
hipError_t launch_combine(const void *Y, bool y_bf16, const float *topk_w, int T, int k, int H, int has_shared,
                          void *out, int out_bf16, hipStream_t s);

}  // namespace qmoe
