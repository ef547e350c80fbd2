// abi.cpp -- host side of the C ABI declared in include/qmoe.h: argument and layout checks
// (all before anything is enqueued), workspace sizing, and kernel dispatch on the
// caller's stream.  No call allocates device memory or synchronises with the host.
#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <string>

#include "launch.h"
#include "qmoe.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

// Per-device "is this a gfx950" cache: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipGetDeviceProperties failed");
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(MOE_ERR_UNSUPPORTED, "this library runs on gfx950 (MI355X) only");
  return MOE_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int format_block(int fmt) {
  switch (fmt) {
    case MOE_FMT_NVFP4: return 16;
    case MOE_FMT_FP8_BLOCK128: return 128;
    case MOE_FMT_MXFP4_E8M0: return 32;
    case MOE_FMT_BF16: return 1;
    case MOE_FMT_Q4_0: return 32;
    default: return 0;
  }
}

const char *format_name(int fmt) {
  switch (fmt) {
    case MOE_FMT_NVFP4: return "NVFP4";
    case MOE_FMT_FP8_BLOCK128: return "FP8_BLOCK128";
    case MOE_FMT_MXFP4_E8M0: return "MXFP4_E8M0";
    case MOE_FMT_BF16: return "BF16";
    case MOE_FMT_Q4_0: return "Q4_0";
    default: return "unknown";
  }
}

// Grid order of the streaming kernels: column groups fastest (neighbouring workgroups read
// adjacent pieces of one expert's slice) when the slice is wide and the pairs many; 16-row
// sub-blocks fastest otherwise.  Measured on MI355X: T*k = 512 at Il = 512 and T*k = 2048 at
// Il = 1024 are faster column-first, T*k = 512 at Il = 256 and T*k <= 128 are not.  The
// sub-blocks then index grid y, limited to 65535.
bool cols_fastest(int T, int k, int Il, int n_sub) {
  return Il >= 512 && (long long)T * k >= 512 && n_sub <= 65535;
}

// Streaming kernels load the expert weights with the non-temporal hint from 128 pairs on: the
// weights are read once, and the hint keeps them from evicting the reused activation rows
// (measured on MI355X, T = 64: fp8-block step 90.6 -> 82.4 us, bf16 151.9 -> 138.7 us; the
// DeepSeek-V4-Flash-shaped MXFP4 layer at T = 256 392 -> 378 us).  With few pairs the loads
// are latency-bound and the hint measured slower (T = 1: 24.5 -> 25.6 us).  gate_up takes it
// only for MXFP4 and bf16 weights (NVFP4 and q4_0 gate_up measured 0.7-1.5 us slower with it);
// down only where one slice row of its weight holds at least 256 bytes (4-bit codes over a
// 256-wide slice measured 1.5 us slower with it, over a 512-wide slice 2-5 us faster).
bool nt_weights(int T, int k) { return (long long)T * k >= 128; }

bool nt_down_weights(int fmt, int T, int k, int Il) {
  const int bits = fmt == MOE_FMT_BF16 ? 16 : fmt == MOE_FMT_FP8_BLOCK128 ? 8 : 4;
  return nt_weights(T, k) && (long long)Il * bits >= 256 * 8;
}

// gate_up K split: H = 128 * kwaves * ksteps with kwaves <= 4 and ksteps <= 8 (kwaves as
// large as possible).  Returns false if H has no such factorisation.
bool gate_up_ksplit(int H, int *kwaves, int *ksteps) {
  const int n = H / 128;
  for (int w = 4; w >= 1; w--)
    if (n % w == 0 && n / w <= 8) {
      *kwaves = w;
      *ksteps = n / w;
      return true;
    }
  return false;
}

int check_bank(const moe_bank *b, const char *name) {
  if (!b) return fail(MOE_ERR_INVALID_ARG, "%s bank is NULL", name);
  const int blk = format_block(b->fmt);
  if (!blk) return fail(MOE_ERR_INVALID_ARG, "%s bank: unknown format %d", name, b->fmt);
  if (b->E < 1 || b->H < 1 || b->I < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s bank: E=%d H=%d I=%d must be positive", name, b->E, b->H, b->I);
  if (b->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s bank: E=%d > 1024", name, b->E);
  if (!b->gate_up || !b->down || (b->fmt != MOE_FMT_BF16 && (!b->gate_up_scale || !b->down_scale)))
    return fail(MOE_ERR_INVALID_ARG, "%s bank: NULL weight or scale pointer", name);
  if (b->fmt == MOE_FMT_NVFP4 && (!b->gate_up_global || !b->down_global))
    return fail(MOE_ERR_INVALID_ARG, "%s bank: NVFP4 needs gate_up_global and down_global", name);
  if (b->I % blk)
    return fail(MOE_ERR_ALIGNMENT, "%s bank: I=%d is not a multiple of the %s block %d", name, b->I,
                format_name(b->fmt), blk);
  int kw, ks;
  if (b->H % 128 || !gate_up_ksplit(b->H, &kw, &ks))
    return fail(MOE_ERR_UNSUPPORTED, "%s bank: H=%d must be 128 * w * s with w <= 4 and s <= 8", name, b->H);
  if (b->I % 32)
    return fail(MOE_ERR_UNSUPPORTED, "%s bank: I=%d must be a multiple of 32 (row pitch of 16-byte loads)",
                name, b->I);
  if (b->fmt == MOE_FMT_Q4_0 && b->I % 128)
    return fail(MOE_ERR_UNSUPPORTED, "%s bank: Q4_0 needs I=%d to be a multiple of 128 (4 blocks per piece row)",
                name, b->I);
  if (b->layout != MOE_LAYOUT_TILE16)
    return fail(MOE_ERR_UNSUPPORTED, "%s bank: layout %d; the expert kernels read MOE_LAYOUT_TILE16 banks "
                "(reorder once with moe_pack_bank)", name, b->layout);
  return MOE_OK;
}

// Bytes of each array of a bank (codes and scales of gate_up and down, NVFP4 globals).
struct BankSizes {
  size_t gu, gus, gug, dn, dns, dng;
  uint32_t gu_pitch, gus_pitch, dn_pitch, dns_pitch;  // bytes per row (codes, FP4 scales)
  int unit;  // reordered scale bytes per unit: NVFP4 2, MXFP4 1 (per 32 elements), Q4_0 8 (per 128)
};

BankSizes bank_sizes(const moe_bank *b) {
  BankSizes z{};
  const size_t E = (size_t)b->E, H = (size_t)b->H, I = (size_t)b->I;
  const bool fp8 = b->fmt == MOE_FMT_FP8_BLOCK128, bf16 = b->fmt == MOE_FMT_BF16;
  z.gu_pitch = (uint32_t)(bf16 ? 2 * H : fp8 ? H : H / 2);
  z.dn_pitch = (uint32_t)(bf16 ? 2 * I : fp8 ? I : I / 2);
  z.gu = E * 2 * I * z.gu_pitch;
  z.dn = E * H * z.dn_pitch;
  if (bf16) {
    z.gus = z.dns = 0;
  } else if (fp8) {
    z.gus = E * (2 * I / 128) * (H / 128) * 4;
    z.dns = E * (H / 128) * (I / 128) * 4;
  } else {  // per-row scales: NVFP4 one byte per 16, MXFP4 one byte per 32, Q4_0 fp16 per 32
    const size_t sdiv = b->fmt == MOE_FMT_NVFP4 ? 16 : b->fmt == MOE_FMT_Q4_0 ? 16 : 32;
    z.unit = b->fmt == MOE_FMT_NVFP4 ? 2 : b->fmt == MOE_FMT_Q4_0 ? 8 : 1;
    z.gus_pitch = (uint32_t)(H / sdiv);
    z.dns_pitch = (uint32_t)(I / sdiv);
    z.gus = E * 2 * I * z.gus_pitch;
    z.dns = E * H * z.dns_pitch;
  }
  if (b->fmt == MOE_FMT_NVFP4) {
    z.gug = E * 2 * I * 4;
    z.dng = E * H * 4;
  }
  return z;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_slice(const moe_bank *b, int lo, int hi) {
  const int blk = format_block(b->fmt);
  if (!(0 <= lo && lo < hi && hi <= b->I))
    return fail(MOE_ERR_ALIGNMENT, "slice [%d, %d) is not a non-empty range inside [0, I=%d)", lo, hi, b->I);
  if (lo % blk || hi % blk)
    return fail(MOE_ERR_ALIGNMENT, "slice [%d, %d) is not on the %s block boundary (%d)", lo, hi,
                format_name(b->fmt), blk);
  if (lo % 32 || hi % 32)
    return fail(MOE_ERR_UNSUPPORTED, "slice [%d, %d): the kernels need lo and hi multiples of 32", lo, hi);
  return MOE_OK;
}

int check_align_out(const moe_align_out *al, int T, int k, int E) {
  if (!al) return fail(MOE_ERR_INVALID_ARG, "align descriptor is NULL");
  if (al->block_m < 16 || al->block_m > 256 || al->block_m % 16)
    return fail(MOE_ERR_UNSUPPORTED, "block_m=%d must be a multiple of 16 in [16, 256]", al->block_m);
  const int32_t need = moe_align_capacity(T, k, E, al->block_m);
  if (need < 0) return fail(MOE_ERR_INVALID_ARG, "bad sizes for the alignment capacity");
  if (al->capacity < need || al->capacity % al->block_m)
    return fail(MOE_ERR_INVALID_ARG, "capacity=%d must be a multiple of block_m and >= %d", al->capacity, need);
  if (!al->sorted_ids || !al->block_expert || !al->counts || !al->offsets || !al->total_padded)
    return fail(MOE_ERR_INVALID_ARG, "align descriptor has a NULL array");
  return MOE_OK;
}

struct FwdPlan {
  int Il, n_routed_sub, n_shared_sub, n_shared_tiles, shared_rows, h_rows, P, Psh;
  bool tiled;  // 128-row align blocks (NVFP4, FP8_BLOCK128, BF16): the prefill GEMMs
  // workspace layout: [h][x planes (MXFP4)][Y]; MXFP4 h is [hq][hs], x is [xq][xs]
  size_t hs_off, xq_off, xs_off, y_off, y_bytes, total;
};

// 16-row sub-blocks the streaming kernels launch for the routed pairs: all of the capacity's,
// or fewer when no routing can fill them.  Expert e's run takes ceil(c_e / BM) blocks of BM
// rows, so the runs in use hold at most P/16 + min(E, P) * BM/16 sub-blocks (P = T*k pairs);
// sub-blocks past total_padded exit at once, but their workgroups still cost launch slots
// (at T = 1, E = 256, BM = 16: 9 sub-blocks instead of 257).
int routed_sub_blocks(int T, int k, int E, int BM, int cap) {
  const long long P = (long long)T * k;
  const long long bound = (P + 15) / 16 + std::min<long long>(E, P) * (BM / 16);
  return (int)std::min<long long>(cap / 16, bound);
}

FwdPlan plan_forward(const moe_bank *routed, const moe_bank *shared, int T, int k, int cap, int BM, int lo, int hi) {
  FwdPlan p;
  p.Il = hi - lo;
  p.n_routed_sub = routed_sub_blocks(T, k, routed->E, BM, cap);
  p.n_shared_sub = shared ? (T + 15) / 16 : 0;
  p.n_shared_tiles = shared ? (T + 127) / 128 : 0;
  p.shared_rows = p.n_shared_tiles * 128;  // room for whole 128-row tiles
  p.h_rows = cap + p.shared_rows;
  p.tiled = false;
  p.P = T * k;
  p.Psh = shared ? T : 0;
  const size_t rows = (size_t)p.h_rows, Il = (size_t)p.Il, H = (size_t)routed->H;
  if (routed->fmt == MOE_FMT_MXFP4_E8M0) {
    p.hs_off = align_up(2 * rows * Il, 256);
    p.xq_off = p.hs_off + align_up(2 * rows * (Il / 32), 256);
    p.xs_off = p.xq_off + align_up(2 * (size_t)T * H, 256);
    p.y_off = p.xs_off + align_up(2 * (size_t)T * (H / 32), 256);
  } else {
    p.hs_off = p.xq_off = p.xs_off = 0;
    p.y_off = align_up(rows * Il * 2, 256);
  }
  p.y_bytes = align_up((size_t)(p.P + p.Psh) * H * 4, 256);
  p.total = p.y_off + p.y_bytes;
  return p;
}

// Checks shared by the forward entry points; fills *plan.
int check_forward(const moe_bank *routed, const moe_bank *shared, int T, int k, const moe_align_out *al,
                  int lo, int hi, size_t workspace_bytes, const void *workspace, FwdPlan *plan) {
  int rc = check_bank(routed, "routed");
  if (rc) return rc;
  if (shared) {
    rc = check_bank(shared, "shared");
    if (rc) return rc;
    if (shared->E != 1 || shared->fmt != routed->fmt || shared->H != routed->H || shared->I != routed->I)
      return fail(MOE_ERR_INVALID_ARG,
                  "shared bank must be one expert of the routed bank's format, H and I (E=%d fmt=%d H=%d I=%d)",
                  shared->E, shared->fmt, shared->H, shared->I);
  }
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (k < 1 || k > routed->E) return fail(MOE_ERR_INVALID_ARG, "k=%d must be in [1, E=%d]", k, routed->E);
  rc = check_slice(routed, lo, hi);
  if (rc) return rc;
  rc = check_align_out(al, T, k, routed->E);
  if (rc) return rc;
  if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "T*k too large");
  // kernels address x, the intermediate and each expert's matrices with 32-bit offsets
  const long long Il = hi - lo, rows = (long long)al->capacity + 128LL * ((T + 127) / 128);
  if ((long long)T * routed->H * 2 >= (1LL << 31) || rows * Il * 2 >= (1LL << 31) ||
      2LL * routed->I * routed->H >= (1LL << 31))
    return fail(MOE_ERR_UNSUPPORTED, "tensor exceeds 2 GiB (32-bit buffer offsets)");
  *plan = plan_forward(routed, shared, T, k, al->capacity, al->block_m, lo, hi);
  plan->tiled = al->block_m % 128 == 0 && routed->fmt != MOE_FMT_MXFP4_E8M0 && routed->fmt != MOE_FMT_Q4_0;
  if (workspace_bytes < plan->total)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, plan->total);
  if (!workspace && plan->total) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  return MOE_OK;
}

// Every host-side check of moe_expert_forward's arguments.
int check_forward_call(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                       const float *topk_w, const moe_align_out *al, int lo, int hi, void *out, int out_dtype,
                       size_t workspace_bytes, const void *workspace, FwdPlan *plan) {
  int rc = check_forward(routed, shared, T, k, al, lo, hi, workspace_bytes, workspace, plan);
  if (rc) return rc;
  if (T > 0 && (!x_bf16 || !topk_w || !out)) return fail(MOE_ERR_INVALID_ARG, "x, topk_w or out is NULL");
  if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16)
    return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d", out_dtype);
  return MOE_OK;
}

qmoe::GateUpArgs gate_up_args(const moe_bank *routed, const moe_bank *shared, const void *x, int T, int k,
                              const moe_align_out *al, int lo, const FwdPlan &p, void *workspace) {
  qmoe::GateUpArgs a{};  // the one-token routing fields stay zero (route1 off)
  a.x = static_cast<const uint16_t *>(x);
  a.T = T;
  a.H = routed->H;
  a.k = k;
  a.gu = static_cast<const uint8_t *>(routed->gate_up);
  a.gus = static_cast<const uint8_t *>(routed->gate_up_scale);
  a.gug = routed->gate_up_global;
  a.sgu = shared ? static_cast<const uint8_t *>(shared->gate_up) : nullptr;
  a.sgus = shared ? static_cast<const uint8_t *>(shared->gate_up_scale) : nullptr;
  a.sgug = shared ? shared->gate_up_global : nullptr;
  a.E = routed->E;
  a.I = routed->I;
  a.sorted_ids = al->sorted_ids;
  a.block_expert = al->block_expert;
  a.total_padded = al->total_padded;
  a.block_m = al->block_m;
  a.cap = al->capacity;
  a.n_routed_sub = p.n_routed_sub;
  a.lo = lo;
  a.Il = p.Il;
  gate_up_ksplit(routed->H, &a.kwaves, &a.ksteps);
  // Few pairs: at most about one wave per SIMD would be busy, so split K over 8 waves
  // per workgroup (half the K range, one round trip fewer per wave) when H allows it.
  // The bound on the busy 16-row blocks is the pair count (or E), plus the shared blocks.
  // Q4_0 (cheap dequantization) also gains at decode-sized batches (T = 64, H = 2048:
  // gate_up 32.0 -> 28.8 us on MI355X), where NVFP4 loses (27.1 -> 37.1 us).
  const long long blocks = std::min<long long>((long long)T * k, routed->E) + p.n_shared_sub;
  const long long kw8_limit = routed->fmt == MOE_FMT_Q4_0 ? 16384 : 2048;
  if (!p.tiled && (routed->H / 128) % 8 == 0 && blocks * (p.Il / 32) * 4 < kw8_limit) {
    a.kwaves = 8;
    a.ksteps = routed->H / 1024;
  }
  a.cols_fastest = cols_fastest(T, k, p.Il, p.n_routed_sub + p.n_shared_sub);
  a.nt_weights = nt_weights(T, k);
  char *ws = static_cast<char *>(workspace);
  a.h = reinterpret_cast<uint16_t *>(ws);
  a.h_rows = p.h_rows;
  a.hq = reinterpret_cast<uint8_t *>(ws);
  a.hs = reinterpret_cast<uint8_t *>(ws + p.hs_off);
  a.xq = reinterpret_cast<const uint8_t *>(ws + p.xq_off);
  a.xs = reinterpret_cast<const uint8_t *>(ws + p.xs_off);
  return a;
}

qmoe::DownArgs down_args(const moe_bank *routed, const moe_bank *shared, int T, int k, const moe_align_out *al,
                         int lo, const FwdPlan &p, void *workspace) {
  qmoe::DownArgs a;
  const char *ws = static_cast<const char *>(workspace);
  a.h = reinterpret_cast<const uint16_t *>(ws);
  a.hq = reinterpret_cast<const uint8_t *>(ws);
  a.hs = reinterpret_cast<const uint8_t *>(ws + p.hs_off);
  a.h_rows = p.h_rows;
  a.T = T;
  a.H = routed->H;
  a.k = k;
  a.dn = static_cast<const uint8_t *>(routed->down);
  a.dns = static_cast<const uint8_t *>(routed->down_scale);
  a.dng = routed->down_global;
  a.sdn = shared ? static_cast<const uint8_t *>(shared->down) : nullptr;
  a.sdns = shared ? static_cast<const uint8_t *>(shared->down_scale) : nullptr;
  a.sdng = shared ? shared->down_global : nullptr;
  a.E = routed->E;
  a.I = routed->I;
  a.sorted_ids = al->sorted_ids;
  a.block_expert = al->block_expert;
  a.total_padded = al->total_padded;
  a.block_m = al->block_m;
  a.cap = al->capacity;
  a.n_routed_sub = p.n_routed_sub;
  a.lo = lo;
  a.Il = p.Il;
  a.cols_fastest = cols_fastest(T, k, p.Il, p.n_routed_sub + p.n_shared_sub);
  a.nt_weights = nt_down_weights(routed->fmt, T, k, p.Il);
  a.Y = reinterpret_cast<float *>(static_cast<char *>(workspace) + p.y_off);
  return a;
}

// gate_up for prepared arguments: MXFP4's activation planes (unless the router GEMM already
// wrote them: planes_ready), then the gate_up kernel.
int launch_gate_up_args(const moe_bank *routed, const qmoe::GateUpArgs &a, int T, const FwdPlan &p,
                        void *workspace, hipStream_t s, bool planes_ready = false) {
  if (routed->fmt == MOE_FMT_MXFP4_E8M0 && !planes_ready) {
    char *ws = static_cast<char *>(workspace);
    const int rc = hip_status(qmoe::launch_act_mx8(a.x, T, routed->H, reinterpret_cast<uint8_t *>(ws + p.xq_off),
                                                   reinterpret_cast<uint8_t *>(ws + p.xs_off), s),
                              "activation split launch");
    if (rc) return rc;
  }
  if (p.tiled) return hip_status(qmoe::launch_gate_up_wide(routed->fmt, a, p.n_shared_tiles, s), "gate_up launch");
  return hip_status(qmoe::launch_gate_up(routed->fmt, a, p.n_shared_sub, s), "gate_up launch");
}

int run_gate_up(const moe_bank *routed, const moe_bank *shared, const void *x, int T, int k,
                const moe_align_out *al, int lo, const FwdPlan &p, void *workspace, hipStream_t s) {
  const qmoe::GateUpArgs a = gate_up_args(routed, shared, x, T, k, al, lo, p, workspace);
  return launch_gate_up_args(routed, a, T, p, workspace, s);
}

// moe_layer_forward's one-token path: one token on 16-row blocks, gate_up on the launch shape
// its routing variant is built for (8 waves splitting K, which the launcher pairs with 32
// slice columns, and cached weight loads).
bool route1_path(const qmoe::GateUpArgs &a, const FwdPlan &p, int T, int block_m) {
  return T == 1 && block_m == 16 && !p.tiled && a.kwaves == 8 && !a.nt_weights;
}

int run_down(const moe_bank *routed, const moe_bank *shared, int T, int k, const float *topk_w,
             const moe_align_out *al, int lo, const FwdPlan &p, void *out, int out_dtype, void *workspace,
             hipStream_t s) {
  qmoe::DownArgs a = down_args(routed, shared, T, k, al, lo, p, workspace);
  if (!p.tiled && qmoe::down_t1_fused(routed->fmt, a, shared != nullptr))
    return hip_status(qmoe::launch_down_t1(routed->fmt, a, topk_w, out, out_dtype == MOE_OUT_BF16, s), "down launch");
  int rc = p.tiled ? hip_status(qmoe::launch_down_wide(routed->fmt, a, p.n_shared_tiles, s), "down launch")
                   : hip_status(qmoe::launch_down(routed->fmt, a, p.n_shared_sub, s), "down launch");
  if (rc) return rc;
  return hip_status(qmoe::launch_combine(a.Y, p.tiled, topk_w, T, k, routed->H, shared != nullptr, out,
                                         out_dtype == MOE_OUT_BF16, s),
                    "combine launch");
}

}  // namespace

namespace qmoe {

int set_last_error(int code, const char *msg) { return fail(code, "%s", msg); }

int forward_workspace_need(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                           const float *topk_w, const moe_align_out *al, int lo, int hi, void *out, int out_dtype,
                           size_t *need) {
  FwdPlan p;
  static const char probe = 0;  // a non-NULL workspace: only the size is asked for here
  const int rc = check_forward_call(routed, shared, x_bf16, T, k, topk_w, al, lo, hi, out, out_dtype, SIZE_MAX,
                                    &probe, &p);
  if (rc) return rc;
  *need = p.total;
  return MOE_OK;
}

}  // namespace qmoe

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_ALIGNMENT: return "slice not aligned to the format block";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or device";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_align_capacity(int T, int k, int E, int block_m) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return -1;
  const long long need = (long long)T * k + (long long)E * (block_m - 1);
  const long long cap = (need + block_m - 1) / block_m * block_m;
  return cap > 0x7fffffffLL ? -1 : (int32_t)cap;
}

int32_t moe_choose_block_m(int T, int k, int E, int fmt) {
  if (T < 0 || k < 1 || E < 1) return fail(MOE_ERR_INVALID_ARG, "moe_choose_block_m: T=%d k=%d E=%d", T, k, E);
  // pairs per expert on average, compared as T*k against multiples of E (no rounding)
  const long long pairs = (long long)T * k, e = E;
  const bool wide = fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_FP8_BLOCK128 || fmt == MOE_FMT_BF16;
  if (wide && pairs >= 32 * e) return 128;
  if (pairs <= 16 * e) return 16;
  if (pairs <= 64 * e) return 32;
  return 64;
}

size_t moe_align_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k < 1 || E < 1) return 0;
  const long long P = (long long)T * k;
  return (size_t)((P + 1023) / 1024) * (size_t)E * sizeof(int32_t);
}

size_t moe_workspace_bytes(const moe_bank *routed, const moe_bank *shared, int T, int k, int block_m,
                           int slice_lo, int slice_hi) {
  if (!routed || T < 0 || k < 1 || slice_hi <= slice_lo || block_m < 16) return 0;
  const int32_t cap = moe_align_capacity(T, k, routed->E, block_m);
  if (cap < 0) return 0;
  return plan_forward(routed, shared, T, k, cap, block_m, slice_lo, slice_hi).total;
}

size_t moe_route_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H < 128 || E < 1) return 0;
  return qmoe::router_workspace_bytes(T, E, H);
}

size_t moe_route_align_workspace_bytes(int T, int H, int E, int k) {
  // the router's partials, then (256-byte aligned) the align histograms
  return (moe_route_workspace_bytes(T, H, E) + 255) / 256 * 256 + moe_align_workspace_bytes(T, k, E);
}

}  // extern "C"

namespace {

int check_route(const void *x_bf16, int T, int H, const void *w_router_bf16, int E, int k, const float *logits,
                const int32_t *topk_ids, const float *topk_w) {
  if (!w_router_bf16 || (T > 0 && (!x_bf16 || !logits || !topk_ids || !topk_w)))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: NULL required pointer");
  if (T < 0 || H < 1 || E < 1) return fail(MOE_ERR_INVALID_ARG, "moe_route: T=%d H=%d E=%d", T, H, E);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route: k=%d must be in [1, E=%d]", k, E);
  if (E > 1024 || k > 64) return fail(MOE_ERR_UNSUPPORTED, "moe_route: needs E <= 1024 and k <= 64");
  if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_route: H=%d must be a multiple of 128", H);
  if (T > 16 * 65535) return fail(MOE_ERR_UNSUPPORTED, "moe_route: T=%d too large", T);
  if ((long long)T * H * 2 >= (1LL << 31) || (long long)E * H * 2 >= (1LL << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_route: x or the router weight exceeds 2 GiB (32-bit buffer offsets)");
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_route(const void *x_bf16, int T, int H, const void *w_router_bf16, int E, const float *bias, int k,
              int renormalize, float *logits, int32_t *topk_ids, float *topk_w, void *workspace,
              size_t workspace_bytes, void *stream) {
  int rc0 = check_route(x_bf16, T, H, w_router_bf16, E, k, logits, topk_ids, topk_w);
  if (rc0) return rc0;
  const size_t need = moe_route_workspace_bytes(T, H, E);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu", workspace_bytes, need);
  if (need && !workspace) return fail(MOE_ERR_INVALID_ARG, "moe_route: workspace is NULL");
  int rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  return hip_status(qmoe::launch_route(static_cast<const uint16_t *>(x_bf16), T, H,
                                       static_cast<const uint16_t *>(w_router_bf16), E, bias, k, renormalize, logits,
                                       topk_ids, topk_w, static_cast<float *>(workspace),
                                       static_cast<hipStream_t>(stream)),
                    "route launch");
}

int moe_route_from_logits(const float *logits, int T, int E, const float *bias, int k, int renormalize,
                          int32_t *topk_ids, float *topk_w, void *stream) {
  if (T > 0 && (!logits || !topk_ids || !topk_w))
    return fail(MOE_ERR_INVALID_ARG, "moe_route_from_logits: NULL pointer");
  if (T < 0 || E < 1) return fail(MOE_ERR_INVALID_ARG, "moe_route_from_logits: T=%d E=%d", T, E);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route_from_logits: k=%d must be in [1, E=%d]", k, E);
  if (E > 1024 || k > 64) return fail(MOE_ERR_UNSUPPORTED, "moe_route_from_logits: needs E <= 1024 and k <= 64");
  int rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  return hip_status(qmoe::launch_topk(logits, T, E, bias, k, renormalize, topk_ids, topk_w,
                                      static_cast<hipStream_t>(stream)),
                    "topk launch");
}

int moe_align(const int32_t *topk_ids, int T, int k, int E, const moe_align_out *out, void *workspace,
              size_t workspace_bytes, void *stream) {
  if (!topk_ids && T > 0) return fail(MOE_ERR_INVALID_ARG, "moe_align: topk_ids is NULL");
  if (T < 0 || k < 1 || E < 1) return fail(MOE_ERR_INVALID_ARG, "moe_align: T=%d k=%d E=%d", T, k, E);
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_align: E=%d > 1024", E);
  if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "moe_align: T*k too large");
  int rc = check_align_out(out, T, k, E);
  if (rc) return rc;
  const size_t need = moe_align_workspace_bytes(T, k, E);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_align: workspace %zu < %zu", workspace_bytes, need);
  if (need && !workspace) return fail(MOE_ERR_INVALID_ARG, "moe_align: workspace is NULL");
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  return hip_status(qmoe::launch_align(topk_ids, T, k, E, out->block_m, out->capacity, out->sorted_ids,
                                       out->block_expert, out->counts, out->offsets, out->total_padded,
                                       static_cast<int32_t *>(workspace), static_cast<hipStream_t>(stream)),
                    "align launch");
}

int moe_route_align(const void *x_bf16, int T, int H, const void *w_router_bf16, int E, const float *bias, int k,
                    int renormalize, float *logits, int32_t *topk_ids, float *topk_w, const moe_align_out *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_route(x_bf16, T, H, w_router_bf16, E, k, logits, topk_ids, topk_w);
  if (rc) return rc;
  if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "moe_route_align: T*k too large");
  rc = check_align_out(out, T, k, E);
  if (rc) return rc;
  const size_t need = moe_route_align_workspace_bytes(T, H, E, k);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_route_align: workspace %zu < %zu", workspace_bytes, need);
  if (need && !workspace) return fail(MOE_ERR_INVALID_ARG, "moe_route_align: workspace is NULL");
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  char *ws = static_cast<char *>(workspace);
  const size_t hist_off = (moe_route_workspace_bytes(T, H, E) + 255) / 256 * 256;
  return hip_status(qmoe::launch_route_align(static_cast<const uint16_t *>(x_bf16), T, H,
                                             static_cast<const uint16_t *>(w_router_bf16), E, bias, k, renormalize,
                                             logits, topk_ids, topk_w, reinterpret_cast<float *>(ws), out->block_m,
                                             out->capacity, out->sorted_ids, out->block_expert, out->counts,
                                             out->offsets, out->total_padded, reinterpret_cast<int32_t *>(ws + hist_off),
                                             static_cast<hipStream_t>(stream)),
                    "route_align launch");
}

int moe_pack_bank(const moe_bank *src, const moe_bank *dst, void *stream) {
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: NULL bank");
  if (!format_block(src->fmt)) return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: unknown format %d", src->fmt);
  const bool transposed = src->layout == MOE_LAYOUT_MXFP4_T;
  if ((src->layout != MOE_LAYOUT_ROWS && !transposed) || dst->layout != MOE_LAYOUT_TILE16)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: src layout must be ROWS or MXFP4_T (%d) and dst TILE16 (%d)",
                src->layout, dst->layout);
  if (transposed && src->fmt != MOE_FMT_MXFP4_E8M0)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: the transposed layout is for MXFP4 banks");
  if (dst->fmt != src->fmt || dst->E != src->E || dst->H != src->H || dst->I != src->I)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: src and dst differ in fmt, E, H or I");
  if (src->E < 1 || src->H < 1 || src->I < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: E=%d H=%d I=%d must be positive", src->E, src->H, src->I);
  // elements per 16-byte piece (Q4_0: a piece row of 4 pieces covers 4 whole blocks)
  const int piece = src->fmt == MOE_FMT_BF16 ? 8 : src->fmt == MOE_FMT_FP8_BLOCK128 ? 16
                    : src->fmt == MOE_FMT_Q4_0 ? 128 : 32;
  if (src->H % piece || src->I % piece || src->H % 128 || (src->fmt == MOE_FMT_FP8_BLOCK128 && src->I % 128))
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_bank: H=%d and I=%d need whole %d-element pieces per row", src->H,
                src->I, piece);
  if ((long long)src->E * 2 * src->I * src->H > (1LL << 40))
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_bank: bank too large");
  const moe_bank *b[2] = {src, dst};
  for (const moe_bank *x : b) {
    if (!x->gate_up || !x->down || (x->fmt != MOE_FMT_BF16 && (!x->gate_up_scale || !x->down_scale)))
      return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: NULL weight or scale pointer");
    if (x->fmt == MOE_FMT_NVFP4 && (!x->gate_up_global || !x->down_global))
      return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: NVFP4 needs gate_up_global and down_global");
    if ((reinterpret_cast<uintptr_t>(x->gate_up) | reinterpret_cast<uintptr_t>(x->down)) % 16)
      return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: weight codes must be 16-byte aligned");
  }
  const BankSizes z = bank_sizes(src);
  // fp4: per-row scales that are reordered with the codes (NVFP4, MXFP4, Q4_0)
  const bool fp8 = src->fmt == MOE_FMT_FP8_BLOCK128, fp4 = !fp8 && src->fmt != MOE_FMT_BF16;
  const bool q4 = src->fmt == MOE_FMT_Q4_0;
  if (overlap(src->gate_up, z.gu, dst->gate_up, z.gu) || overlap(src->down, z.dn, dst->down, z.dn) ||
      (fp4 && (overlap(src->gate_up_scale, z.gus, dst->gate_up_scale, z.gus) ||
                overlap(src->down_scale, z.dns, dst->down_scale, z.dns))))
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_bank: dst codes or scales overlap src");
  int rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t E = (size_t)src->E, H = (size_t)src->H, I = (size_t)src->I;
  if (transposed) {  // gather each matrix's columns: codes [K/2, N] and scales [K/32, N] per expert
    const struct { const void *from; const void *to; size_t N; uint32_t pitch; int unit; } t[4] = {
        {src->gate_up, dst->gate_up, 2 * I, z.gu_pitch, 16}, {src->down, dst->down, H, z.dn_pitch, 16},
        {src->gate_up_scale, dst->gate_up_scale, 2 * I, z.gus_pitch, 1},
        {src->down_scale, dst->down_scale, H, z.dns_pitch, 1}};
    for (const auto &m : t) {
      rc = hip_status(qmoe::launch_pack_tile16_t(m.from, const_cast<void *>(m.to), E, m.N, m.pitch, m.unit, s),
                      "pack launch");
      if (rc) return rc;
    }
    return ok();
  }
  if (q4) {  // codes: nibble order changes too
    rc = hip_status(qmoe::launch_pack_q4_0(src->gate_up, const_cast<void *>(dst->gate_up), E * 2 * I, z.gu_pitch, s),
                    "pack launch");
    if (rc) return rc;
    rc = hip_status(qmoe::launch_pack_q4_0(src->down, const_cast<void *>(dst->down), E * H, z.dn_pitch, s),
                    "pack launch");
  } else {
    rc = hip_status(qmoe::launch_pack_tile16(src->gate_up, const_cast<void *>(dst->gate_up), E * 2 * I,
                                             z.gu_pitch, 16, s), "pack launch");
    if (rc) return rc;
    rc = hip_status(qmoe::launch_pack_tile16(src->down, const_cast<void *>(dst->down), E * H, z.dn_pitch, 16, s),
                    "pack launch");
  }
  if (rc) return rc;
  if (fp4) {
    rc = hip_status(qmoe::launch_pack_tile16(src->gate_up_scale, const_cast<void *>(dst->gate_up_scale), E * 2 * I,
                                             z.gus_pitch, z.unit, s), "pack launch");
    if (rc) return rc;
    rc = hip_status(qmoe::launch_pack_tile16(src->down_scale, const_cast<void *>(dst->down_scale), E * H,
                                             z.dns_pitch, z.unit, s), "pack launch");
    if (rc) return rc;
  }
  // order-free arrays: plain copies when dst has its own storage
  const struct { const void *from; const void *to; size_t n; } same[4] = {
      {fp8 ? src->gate_up_scale : nullptr, dst->gate_up_scale, z.gus},
      {fp8 ? src->down_scale : nullptr, dst->down_scale, z.dns},
      {src->gate_up_global, dst->gate_up_global, z.gug},
      {src->down_global, dst->down_global, z.dng}};
  for (const auto &c : same) {
    if (!c.from || !c.to || c.from == c.to || !c.n) continue;
    rc = hip_status(hipMemcpyAsync(const_cast<void *>(c.to), c.from, c.n, hipMemcpyDeviceToDevice, s), "pack copy");
    if (rc) return rc;
  }
  return ok();
}

int moe_expert_gate_up(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                       const moe_align_out *al, int slice_lo, int slice_hi, void *workspace, size_t workspace_bytes,
                       void *stream) {
  FwdPlan p;
  int rc = check_forward(routed, shared, T, k, al, slice_lo, slice_hi, workspace_bytes, workspace, &p);
  if (rc) return rc;
  if (!x_bf16 && T > 0) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  return run_gate_up(routed, shared, x_bf16, T, k, al, slice_lo, p, workspace, static_cast<hipStream_t>(stream));
}

int moe_expert_down(const moe_bank *routed, const moe_bank *shared, int T, int k, const float *topk_w,
                    const moe_align_out *al, int slice_lo, int slice_hi, void *out, int out_dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
  FwdPlan p;
  int rc = check_forward(routed, shared, T, k, al, slice_lo, slice_hi, workspace_bytes, workspace, &p);
  if (rc) return rc;
  if (T > 0 && (!topk_w || !out)) return fail(MOE_ERR_INVALID_ARG, "topk_w or out is NULL");
  if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16)
    return fail(MOE_ERR_INVALID_ARG, "out_dtype=%d", out_dtype);
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  return run_down(routed, shared, T, k, topk_w, al, slice_lo, p, out, out_dtype, workspace,
                  static_cast<hipStream_t>(stream));
}

int moe_layer_forward(const void *x_bf16, int T, const void *w_router_bf16, const float *bias, int k,
                      int renormalize, const moe_bank *routed, const moe_bank *shared, int slice_lo, int slice_hi,
                      float *logits, int32_t *topk_ids, float *topk_w, const moe_align_out *al, void *out,
                      int out_dtype, void *route_workspace, size_t route_workspace_bytes, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!routed) return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward: routed bank is NULL");
  const int H = routed->H, E = routed->E;
  int rc = check_route(x_bf16, T, H, w_router_bf16, E, k, logits, topk_ids, topk_w);
  if (rc) return rc;
  FwdPlan p;
  rc = check_forward_call(routed, shared, x_bf16, T, k, topk_w, al, slice_lo, slice_hi, out, out_dtype,
                          workspace_bytes, workspace, &p);
  if (rc) return rc;
  const size_t rneed = moe_route_align_workspace_bytes(T, H, E, k);
  if (route_workspace_bytes < rneed)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_forward: route workspace %zu < %zu", route_workspace_bytes, rneed);
  if (rneed && !route_workspace) return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward: route workspace is NULL");
  // gate_up reads the router's partials while it writes the expert workspace (one token), and the
  // router writes MXFP4's planes into it beside its partials: the two must not share bytes
  if (rneed && p.total && overlap(route_workspace, rneed, workspace, p.total))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward: route workspace and workspace overlap");
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  qmoe::GateUpArgs a = gate_up_args(routed, shared, x_bf16, T, k, al, slice_lo, p, workspace);
  // MXFP4: the split-K router GEMM, which reads x anyway, also writes its activation planes
  char *ws = static_cast<char *>(workspace);
  const qmoe::XPlanes planes{reinterpret_cast<uint8_t *>(ws + p.xq_off), reinterpret_cast<uint8_t *>(ws + p.xs_off)};
  const bool mx_planes = routed->fmt == MOE_FMT_MXFP4_E8M0 && qmoe::router_writes_planes(T);
  const qmoe::XPlanes *xp = mx_planes ? &planes : nullptr;
  char *rws = static_cast<char *>(route_workspace);
  float *part = reinterpret_cast<float *>(rws);
  if (!route1_path(a, p, T, al->block_m)) {  // the kernels of the two calls
    const size_t hist_off = (moe_route_workspace_bytes(T, H, E) + 255) / 256 * 256;
    rc = hip_status(qmoe::launch_route_align(static_cast<const uint16_t *>(x_bf16), T, H,
                                             static_cast<const uint16_t *>(w_router_bf16), E, bias, k, renormalize,
                                             logits, topk_ids, topk_w, part, al->block_m, al->capacity,
                                             al->sorted_ids, al->block_expert, al->counts, al->offsets,
                                             al->total_padded, reinterpret_cast<int32_t *>(rws + hist_off), s, xp),
                    "route_align launch");
    if (rc) return rc;
    rc = launch_gate_up_args(routed, a, T, p, workspace, s, mx_planes);
    if (rc) return rc;
    return run_down(routed, shared, T, k, topk_w, al, slice_lo, p, out, out_dtype, workspace, s);
  }
  // one token: the router GEMM, then gate_up ranks its logits in every routed workgroup and
  // writes the routing and the alignment, which down reads
  int ks = 1;
  rc = hip_status(qmoe::launch_router(static_cast<const uint16_t *>(x_bf16), T, H,
                                      static_cast<const uint16_t *>(w_router_bf16), E, bias, logits, part, &ks, xp, s),
                  "router launch");
  if (rc) return rc;
  a.route1 = 1;
  a.r_part = ks > 1 ? part : logits;  // one split: the router added the bias into the logits
  a.r_bias = ks > 1 ? bias : nullptr;
  a.r_ks = ks;
  a.r_renorm = renormalize;
  a.r_logits = ks > 1 ? logits : nullptr;
  a.r_ids = topk_ids;
  a.r_w = topk_w;
  a.al_sorted = al->sorted_ids;
  a.al_block = al->block_expert;
  a.al_counts = al->counts;
  a.al_offsets = al->offsets;
  a.al_total = al->total_padded;
  rc = launch_gate_up_args(routed, a, T, p, workspace, s, mx_planes);
  if (rc) return rc;
  return run_down(routed, shared, T, k, topk_w, al, slice_lo, p, out, out_dtype, workspace, s);
}

int moe_expert_forward(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                       const float *topk_w, const moe_align_out *al, int slice_lo, int slice_hi, void *out,
                       int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  FwdPlan p;
  int rc = check_forward_call(routed, shared, x_bf16, T, k, topk_w, al, slice_lo, slice_hi, out, out_dtype,
                              workspace_bytes, workspace, &p);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  if (T == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = run_gate_up(routed, shared, x_bf16, T, k, al, slice_lo, p, workspace, s);
  if (rc) return rc;
  return run_down(routed, shared, T, k, topk_w, al, slice_lo, p, out, out_dtype, workspace, s);
}

}  // extern "C"
