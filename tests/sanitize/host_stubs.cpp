// host_stubs.cpp -- host stand-ins for what the C ABI's host code (csrc/abi.cpp) calls outside
// itself, so that abi.cpp can be built with AddressSanitizer and UndefinedBehaviorSanitizer
// as plain host C++ and driven on a machine without a GPU (tests/test_host_sanitizers.py):
//   - the four HIP runtime calls abi.cpp makes: a device 0 that reports gfx950, an error
//     string, and an asynchronous copy that only counts (the pointers are not host memory);
//   - the kernel launchers declared in launch.h: each checks the invariants the kernels
//     rely on for the arguments the ABI built (sizes, capacities, offsets inside the
//     workspace) and counts the launch.
// Nothing here computes the layer; the GPU tests do that.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.h"

namespace {
int g_launches = 0;
int g_bad = 0;
size_t g_ws_bytes = 0;  // the workspace the driver passed (0: unknown)

void expect(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "stub: invariant failed: %s\n", what);
    g_bad++;
  }
}

// The expert kernels index the workspace from its base with 32-bit offsets below 2 GiB.
void expect_inside(const void *base, const void *p, size_t bytes, const char *what) {
  if (!g_ws_bytes || !p) return;
  const char *b = static_cast<const char *>(base), *q = static_cast<const char *>(p);
  expect(q >= b && (size_t)(q - b) + bytes <= g_ws_bytes, what);
}
const void *g_ws_base = nullptr;
const void *g_rws_base = nullptr;  // the route workspace the driver passed (NULL: unknown)
size_t g_rws_bytes = 0;
}  // namespace

extern "C" {
int stub_launches(void) { return g_launches; }
int stub_failures(void) { return g_bad; }
void stub_set_workspace(const void *base, size_t bytes) {
  g_ws_base = base;
  g_ws_bytes = bytes;
}
void stub_set_route_workspace(const void *base, size_t bytes) {
  g_rws_base = base;
  g_rws_bytes = bytes;
}

hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int) {
  std::memset(prop, 0, sizeof *prop);
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub error"; }
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) {
  expect(dst && src && n, "copy arguments");
  g_launches++;
  return hipSuccess;
}
}

namespace qmoe {

size_t router_workspace_bytes(int T, int E, int H) {
  expect(T > 0 && E > 0 && H > 0, "router sizes");
  return (size_t)16 * T * E * sizeof(float);
}

bool router_writes_planes(int T) { return T < 1024; }

hipError_t launch_router(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *, float *logits,
                         float *partial, int *ks, const XPlanes *xp, hipStream_t) {
  if (xp) expect_inside(g_ws_base, xp->q, (size_t)2 * T * H, "planes inside the workspace");
  expect(x && w && logits && T > 0 && H % 128 == 0 && E >= 1, "router args");
  *ks = 2;  // the one-token path with split-K partials
  expect(partial != nullptr, "router partials");
  if (g_rws_base)
    expect(partial == g_rws_base && (size_t)2 * T * E * 4 <= g_rws_bytes, "router partials inside the route workspace");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_route(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *, int k, int,
                        float *logits, int32_t *ids, float *wts, float *, hipStream_t) {
  expect(x && w && logits && ids && wts && T > 0 && H % 128 == 0 && k >= 1 && k <= E && k <= 64, "route args");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_topk(const float *logits, int T, int E, const float *, int k, int, int32_t *ids, float *wts,
                       hipStream_t) {
  expect(logits && ids && wts && T > 0 && k >= 1 && k <= E, "top-k args");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_align(const int32_t *ids, int T, int k, int E, int BM, int cap, int32_t *sorted_ids,
                        int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded, int32_t *,
                        hipStream_t) {
  expect(ids && sorted_ids && block_expert && counts && offsets && total_padded, "align pointers");
  expect(T > 0 && k > 0 && E > 0 && BM % 16 == 0 && cap % BM == 0 && (long long)cap >= (long long)T * k, "align sizes");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_route_align(const uint16_t *x, int T, int H, const uint16_t *w, int E, const float *bias, int k,
                              int renormalize, float *logits, int32_t *ids, float *wts, float *partial, int BM,
                              int cap, int32_t *sorted_ids, int32_t *block_expert, int32_t *counts,
                              int32_t *offsets, int32_t *total_padded, int32_t *hist, hipStream_t s,
                              const XPlanes *xp) {
  if (xp) expect(T < 1024 && xp->q && xp->s, "planes only from the split-K router");
  const hipError_t e = launch_route(x, T, H, w, E, bias, k, renormalize, logits, ids, wts, partial, s);
  if (e != hipSuccess) return e;
  return launch_align(ids, T, k, E, BM, cap, sorted_ids, block_expert, counts, offsets, total_padded, hist, s);
}

static void check_expert_args(int T, int k, int E, int I, int lo, int Il, int block_m, int cap, int n_routed_sub) {
  expect(T > 0 && k >= 1 && k <= E, "expert T, k");
  expect(lo >= 0 && Il > 0 && lo + Il <= I && lo % 32 == 0 && Il % 32 == 0, "expert slice");
  expect(block_m % 16 == 0 && cap % block_m == 0, "expert capacity");
  expect(n_routed_sub >= 0 && n_routed_sub <= cap / 16, "routed sub-blocks");
}

hipError_t launch_gate_up(int, const GateUpArgs &a, int n_shared_sub, hipStream_t) {
  check_expert_args(a.T, a.k, a.E, a.I, a.lo, a.Il, a.block_m, a.cap, a.n_routed_sub);
  expect(a.kwaves * a.ksteps * 128 == a.H, "gate_up K split");
  if (a.route1) {  // the one-token whole-layer path: every routing pointer set, 8 waves, 16-row blocks
    expect(a.T == 1 && a.block_m == 16 && a.kwaves == 8 && a.k <= 64 && a.E <= 1024, "one-token routing shape");
    expect(a.r_part && a.r_ks >= 1 && a.r_ids && a.r_w && a.al_sorted && a.al_block && a.al_counts &&
               a.al_offsets && a.al_total,
           "one-token routing pointers");
    expect(a.n_routed_sub >= a.k, "a routed sub-block per pick");
  }
  expect(a.h_rows >= a.cap + 16 * n_shared_sub, "intermediate rows");
  expect_inside(g_ws_base, a.h, (size_t)a.cap * a.Il * 2, "intermediate inside the workspace");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_gate_up_wide(int, const GateUpArgs &a, int n_shared_tiles, hipStream_t) {
  check_expert_args(a.T, a.k, a.E, a.I, a.lo, a.Il, a.block_m, a.cap, a.n_routed_sub);
  expect(a.block_m % 128 == 0 && a.h_rows >= a.cap + 128 * n_shared_tiles, "prefill rows");
  expect_inside(g_ws_base, a.h, (size_t)a.h_rows * a.Il * 2, "intermediate inside the workspace");
  g_launches++;
  return hipSuccess;
}

static void check_down(const DownArgs &a) {
  check_expert_args(a.T, a.k, a.E, a.I, a.lo, a.Il, a.block_m, a.cap, a.n_routed_sub);
  expect_inside(g_ws_base, a.Y, (size_t)a.T * a.k * a.H * 2, "pair rows inside the workspace");
}

hipError_t launch_down(int, const DownArgs &a, int, hipStream_t) {
  check_down(a);
  g_launches++;
  return hipSuccess;
}

hipError_t launch_down_wide(int, const DownArgs &a, int, hipStream_t) {
  check_down(a);
  expect(a.block_m % 128 == 0, "prefill block");
  g_launches++;
  return hipSuccess;
}

bool down_t1_fused(int, const DownArgs &a, int has_shared) {
  return a.T == 1 && a.k <= 15 && a.n_routed_sub + (has_shared ? 1 : 0) <= 16;
}

hipError_t launch_down_t1(int, const DownArgs &a, const float *topk_w, void *out, int, hipStream_t) {
  check_down(a);
  expect(a.T == 1 && topk_w && out, "one-token down");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_act_mx8(const uint16_t *x, int rows, int K, uint8_t *q, uint8_t *sc, hipStream_t) {
  expect(x && q && sc && rows > 0 && K % 32 == 0, "activation split");
  expect_inside(g_ws_base, q, (size_t)2 * rows * K, "planes inside the workspace");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_combine(const void *Y, bool, const float *topk_w, int T, int k, int H, int, void *out, int,
                          hipStream_t) {
  expect(Y && topk_w && out && T > 0 && k > 0 && H % 128 == 0, "combine args");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_pack_tile16(const void *src, void *dst, size_t rows, uint32_t pitch, int unit, hipStream_t) {
  expect(src && dst && rows % 16 == 0 && pitch % unit == 0, "tile-16 pack");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_pack_tile16_t(const void *src, void *dst, size_t E, size_t N, uint32_t pitch, int unit,
                                hipStream_t) {
  expect(src && dst && E > 0 && N % 16 == 0 && pitch > 0 && (unit == 16 || unit == 1), "transposed pack");
  g_launches++;
  return hipSuccess;
}

hipError_t launch_pack_q4_0(const void *src, void *dst, size_t rows, uint32_t pitch, hipStream_t) {
  expect(src && dst && rows % 16 == 0 && pitch % 16 == 0, "q4_0 pack");
  g_launches++;
  return hipSuccess;
}

}  // namespace qmoe
