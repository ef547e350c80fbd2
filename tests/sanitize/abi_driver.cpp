// abi_driver.cpp -- drives every entry point of the C ABI (include/qmoe.h) through its host code
// (csrc/abi.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer and linked against
// the host stand-ins of host_stubs.cpp instead of the HIP runtime and the kernels
// (tests/test_host_sanitizers.py).  Device pointers are fake addresses that the host code must
// never dereference.  Each call's return code is checked against the one the header documents:
// valid calls reach the (stubbed) launches, invalid ones are rejected before any launch.
// Exit status 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "qmoe.h"

extern "C" int stub_launches(void);
extern "C" int stub_failures(void);
extern "C" void stub_set_workspace(const void *base, size_t bytes);
extern "C" void stub_set_route_workspace(const void *base, size_t bytes);

namespace {

int failures = 0;

void expect_rc(int got, int want, const char *what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL: %s: status %d (%s), expected %d; last error: %s\n", what, got,
                 moe_status_string(got), want, moe_last_error());
    failures++;
  }
}

void expect(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    failures++;
  }
}

// A fake device address: never dereferenced by host code.
void *dev(uintptr_t region) { return reinterpret_cast<void *>(region << 32); }

moe_bank bank(int fmt, int E, int H, int I, int layout = MOE_LAYOUT_TILE16) {
  moe_bank b;
  std::memset(&b, 0, sizeof b);
  b.fmt = fmt;
  b.E = E;
  b.H = H;
  b.I = I;
  b.gate_up = dev(0x10);
  b.down = dev(0x11);
  if (fmt != MOE_FMT_BF16) {
    b.gate_up_scale = dev(0x12);
    b.down_scale = dev(0x13);
  }
  if (fmt == MOE_FMT_NVFP4) {
    b.gate_up_global = static_cast<const float *>(dev(0x14));
    b.down_global = static_cast<const float *>(dev(0x15));
  }
  b.layout = layout;
  return b;
}

moe_align_out align_desc(int T, int k, int E, int bm) {
  moe_align_out a;
  a.sorted_ids = static_cast<int32_t *>(dev(0x20));
  a.block_expert = static_cast<int32_t *>(dev(0x21));
  a.counts = static_cast<int32_t *>(dev(0x22));
  a.offsets = static_cast<int32_t *>(dev(0x23));
  a.total_padded = static_cast<int32_t *>(dev(0x24));
  a.block_m = bm;
  a.capacity = moe_align_capacity(T, k, E, bm);
  return a;
}

void routing() {
  const int T = 37, H = 256, E = 64, k = 6;
  void *x = dev(0x30), *wr = dev(0x31), *ws = dev(0x32);
  float *logits = static_cast<float *>(dev(0x33)), *tw = static_cast<float *>(dev(0x34));
  int32_t *ids = static_cast<int32_t *>(dev(0x35));
  const size_t rws = moe_route_workspace_bytes(T, H, E);
  int before = stub_launches();
  expect_rc(moe_route(x, T, H, wr, E, nullptr, k, 1, logits, ids, tw, ws, rws, nullptr), MOE_OK, "route");
  expect(stub_launches() > before, "route launches");
  expect_rc(moe_route(x, T, 100, wr, E, nullptr, k, 1, logits, ids, tw, ws, rws, nullptr), MOE_ERR_UNSUPPORTED,
            "route with H not a multiple of 128");
  expect_rc(moe_route(x, T, H, wr, E, nullptr, 0, 1, logits, ids, tw, ws, rws, nullptr), MOE_ERR_INVALID_ARG,
            "route with k = 0");
  expect_rc(moe_route(x, T, H, wr, 2000, nullptr, k, 1, logits, ids, tw, ws, rws, nullptr), MOE_ERR_UNSUPPORTED,
            "route with E > 1024");
  expect_rc(moe_route(nullptr, T, H, wr, E, nullptr, k, 1, logits, ids, tw, ws, rws, nullptr), MOE_ERR_INVALID_ARG,
            "route without x");
  before = stub_launches();
  expect_rc(moe_route(x, 0, H, wr, E, nullptr, k, 1, logits, ids, tw, ws, rws, nullptr), MOE_OK, "route T = 0");
  expect(stub_launches() == before, "route T = 0 enqueues nothing");
  expect_rc(moe_route_from_logits(logits, T, E, nullptr, k, 1, ids, tw, nullptr), MOE_OK, "route from logits");
  expect_rc(moe_route_from_logits(logits, T, E, nullptr, E + 1, 1, ids, tw, nullptr), MOE_ERR_INVALID_ARG,
            "route from logits with k > E");

  for (int bm : {16, 32, 64, 128, 256}) {
    moe_align_out al = align_desc(T, k, E, bm);
    const size_t aws = moe_align_workspace_bytes(T, k, E);
    expect_rc(moe_align(ids, T, k, E, &al, ws, aws, nullptr), MOE_OK, "align");
    const size_t raws = moe_route_align_workspace_bytes(T, H, E, k);
    expect_rc(moe_route_align(x, T, H, wr, E, nullptr, k, 1, logits, ids, tw, &al, ws, raws, nullptr), MOE_OK,
              "route_align");
    expect_rc(moe_route_align(x, T, H, wr, E, nullptr, k, 1, logits, ids, tw, &al, ws, raws - 1, nullptr),
              MOE_ERR_WORKSPACE, "route_align with a short workspace");
    al.capacity -= bm;
    expect_rc(moe_align(ids, T, k, E, &al, ws, aws, nullptr), MOE_ERR_INVALID_ARG, "align below capacity");
  }
  moe_align_out bad = align_desc(T, k, E, 16);
  bad.block_m = 24;
  expect_rc(moe_align(ids, T, k, E, &bad, ws, 1 << 20, nullptr), MOE_ERR_UNSUPPORTED, "align with block_m 24");
  expect(moe_align_capacity(-1, 8, 256, 16) < 0 && moe_align_capacity(1 << 30, 64, 1024, 256) < 0,
         "capacity rejects bad and overflowing sizes");
  expect(moe_choose_block_m(8192, 8, 256, MOE_FMT_NVFP4) == 128 && moe_choose_block_m(1, 8, 256, 0) == 16 &&
             moe_choose_block_m(-1, 8, 256, 0) == MOE_ERR_INVALID_ARG,
         "block-size policy");
}

void expert_layer(int fmt) {
  const int E = 16, H = fmt == MOE_FMT_FP8_BLOCK128 ? 256 : 128, I = 256;
  moe_bank routed = bank(fmt, E, H, I), shared = bank(fmt, 1, H, I);
  void *x = dev(0x40), *out = dev(0x41), *ws = dev(0x42);
  float *tw = static_cast<float *>(dev(0x43));
  const int lo_step = fmt == MOE_FMT_FP8_BLOCK128 ? 128 : 32;
  for (int T : {1, 2, 9, 300}) {
    const int k = T == 1 ? 4 : 3;
    for (int bm : {16, 64, 128}) {
      moe_align_out al = align_desc(T, k, E, bm);
      for (int lo = 0; lo < I; lo += lo_step) {
        const int hi = lo + lo_step < I ? I : lo + lo_step;
        const size_t need = moe_workspace_bytes(&routed, &shared, T, k, bm, lo, hi);
        expect(need > 0, "workspace bytes of a valid call");
        stub_set_workspace(ws, need);
        const int before = stub_launches();
        for (int od : {MOE_OUT_F32, MOE_OUT_BF16})
          expect_rc(moe_expert_forward(&routed, &shared, x, T, k, tw, &al, lo, hi, out, od, ws, need, nullptr),
                    MOE_OK, "expert forward");
        expect(stub_launches() > before, "expert forward launches");
        expect_rc(moe_expert_gate_up(&routed, nullptr, x, T, k, &al, lo, hi, ws, need, nullptr), MOE_OK,
                  "gate_up alone");
        expect_rc(moe_expert_down(&routed, nullptr, T, k, tw, &al, lo, hi, out, MOE_OUT_F32, ws, need, nullptr),
                  MOE_OK, "down alone");
        expect_rc(moe_expert_forward(&routed, &shared, x, T, k, tw, &al, lo, hi, out, MOE_OUT_F32, ws, need - 1,
                                     nullptr),
                  MOE_ERR_WORKSPACE, "expert forward with a short workspace");
      }
      stub_set_workspace(nullptr, 0);
      const size_t big = (size_t)1 << 40;
      expect(moe_expert_forward(&routed, &shared, x, T, k, tw, &al, 0, I + 32, out, 0, ws, big, nullptr) != MOE_OK,
             "slice past I");
      expect(moe_expert_forward(&routed, &shared, x, T, k, tw, &al, 8, 8, out, 0, ws, big, nullptr) != MOE_OK,
             "empty slice");
      expect(moe_expert_forward(&routed, &shared, x, T, k, tw, &al, 0, I, out, 7, ws, big, nullptr) ==
                 MOE_ERR_INVALID_ARG,
             "bad output type");
      expect(moe_expert_forward(&routed, &shared, x, T, E + 1, tw, &al, 0, I, out, 0, ws, big, nullptr) != MOE_OK,
             "k > E");
      moe_bank rows = bank(fmt, E, H, I, MOE_LAYOUT_ROWS);
      expect_rc(moe_expert_forward(&rows, nullptr, x, T, k, tw, &al, 0, I, out, 0, ws, big, nullptr),
                MOE_ERR_UNSUPPORTED, "row-major bank");
      moe_bank other = bank(fmt == MOE_FMT_NVFP4 ? MOE_FMT_MXFP4_E8M0 : MOE_FMT_NVFP4, 1, H, I);
      expect(moe_expert_forward(&routed, &other, x, T, k, tw, &al, 0, I, out, 0, ws, big, nullptr) ==
                 MOE_ERR_INVALID_ARG,
             "shared bank of another format");
      expect_rc(moe_expert_forward(&routed, &shared, x, 0, k, tw, &al, 0, I, out, 0, ws, big, nullptr), MOE_OK,
                "T = 0");
    }
  }
}

// moe_layer_forward: the one-token path (H = 1024 gives gate_up's 8-wave K split) and the
// two calls' path, for every format, with the workspaces exact and one byte short.
void layer_call(int fmt) {
  const int E = 16, H = 1024, I = 256;
  moe_bank routed = bank(fmt, E, H, I), shared = bank(fmt, 1, H, I);
  void *x = dev(0x60), *wr = dev(0x61), *out = dev(0x62), *ws = dev(0x63), *rws = dev(0x64);
  float *lg = static_cast<float *>(dev(0x65)), *tw = static_cast<float *>(dev(0x66));
  int32_t *ids = static_cast<int32_t *>(dev(0x67));
  const int lo = 0, hi = fmt == MOE_FMT_FP8_BLOCK128 ? 128 : 64;
  for (int T : {1, 3}) {
    const int k = 4;
    moe_align_out al = align_desc(T, k, E, 16);
    const size_t need = moe_workspace_bytes(&routed, &shared, T, k, 16, lo, hi);
    const size_t rneed = moe_route_align_workspace_bytes(T, H, E, k);
    stub_set_workspace(ws, need);
    stub_set_route_workspace(rws, rneed);
    const int before = stub_launches();
    expect_rc(moe_layer_forward(x, T, wr, nullptr, k, 1, &routed, &shared, lo, hi, lg, ids, tw, &al, out,
                                MOE_OUT_F32, rws, rneed, ws, need, nullptr),
              MOE_OK, "layer forward");
    expect(stub_launches() > before, "layer forward launches");
    stub_set_workspace(nullptr, 0);
    stub_set_route_workspace(nullptr, 0);
    expect_rc(moe_layer_forward(x, T, wr, nullptr, k, 1, &routed, &shared, lo, hi, lg, ids, tw, &al, out,
                                MOE_OUT_F32, rws, rneed - 1, ws, need, nullptr),
              MOE_ERR_WORKSPACE, "layer forward with a short route workspace");
    expect_rc(moe_layer_forward(x, T, wr, nullptr, k, 1, &routed, &shared, lo, hi, lg, ids, tw, &al, out,
                                MOE_OUT_F32, rws, rneed, ws, need - 1, nullptr),
              MOE_ERR_WORKSPACE, "layer forward with a short workspace");
    expect_rc(moe_layer_forward(x, T, nullptr, nullptr, k, 1, &routed, &shared, lo, hi, lg, ids, tw, &al, out,
                                MOE_OUT_F32, rws, rneed, ws, need, nullptr),
              MOE_ERR_INVALID_ARG, "layer forward without a router weight");
  }
}

void packing(int fmt) {
  const int E = 4, H = fmt == MOE_FMT_FP8_BLOCK128 ? 256 : 128, I = 128;
  moe_bank src = bank(fmt, E, H, I, MOE_LAYOUT_ROWS), dst = bank(fmt, E, H, I, MOE_LAYOUT_TILE16);
  dst.gate_up = dev(0x50);
  dst.down = dev(0x51);
  if (dst.gate_up_scale) dst.gate_up_scale = dev(0x52);
  if (dst.down_scale) dst.down_scale = dev(0x53);
  if (dst.gate_up_global) dst.gate_up_global = static_cast<const float *>(dev(0x54));
  if (dst.down_global) dst.down_global = static_cast<const float *>(dev(0x55));
  const int before = stub_launches();
  expect_rc(moe_pack_bank(&src, &dst, nullptr), MOE_OK, "pack");
  expect(stub_launches() > before, "pack launches");
  expect_rc(moe_pack_bank(&src, &src, nullptr), MOE_ERR_INVALID_ARG, "pack in place");
  expect_rc(moe_pack_bank(nullptr, &dst, nullptr), MOE_ERR_INVALID_ARG, "pack without source");
  moe_bank wrong = dst;
  wrong.H = H + 128;
  expect(moe_pack_bank(&src, &wrong, nullptr) != MOE_OK, "pack into another shape");
  if (fmt == MOE_FMT_MXFP4_E8M0) {
    moe_bank t = bank(fmt, E, H, I, MOE_LAYOUT_MXFP4_T);
    expect_rc(moe_pack_bank(&t, &dst, nullptr), MOE_OK, "pack transposed MXFP4");
  }
}

}  // namespace

int main() {
  for (int s = -6; s <= 1; s++) expect(moe_status_string(s) && *moe_status_string(s), "status text");
  routing();
  for (int fmt : {MOE_FMT_NVFP4, MOE_FMT_FP8_BLOCK128, MOE_FMT_MXFP4_E8M0, MOE_FMT_BF16, MOE_FMT_Q4_0}) {
    expert_layer(fmt);
    layer_call(fmt);
    packing(fmt);
  }
  if (stub_failures()) {
    std::fprintf(stderr, "%d kernel-argument invariant(s) failed\n", stub_failures());
    failures++;
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi driver ok (%d stub launches)\n", stub_launches());
  return 0;
}
