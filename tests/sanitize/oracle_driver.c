/* oracle_driver.c -- runs the fp64 oracle (oracle/oracle.c) and the synthetic input generators
 * (synth/synth.c) over small layers of every expert format, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).  It checks only what a memory or
 * arithmetic fault would break: every output is written and finite, the routing picks valid
 * experts, and the alignment places every pair once.  Parity itself is the other tests' job.
 * Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* generator entry points (synth/synth.c) */
void synth_bf16_normal(uint64_t seed, uint32_t tag, uint32_t index, double sigma, int64_t n, uint16_t *out);
void synth_nvfp4_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols, double sigma,
                        uint8_t *codes, uint8_t *scales, float *global);
void synth_fp8blk_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols, double sigma,
                         uint8_t *codes, float *scale_inv);
void synth_mxfp4_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols, double sigma,
                        uint8_t *codes, uint8_t *scales);
void synth_q4_0_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols, double sigma,
                       uint8_t *codes, uint16_t *d);
void synth_zipf_bias(uint64_t seed, uint32_t tag, int E, double s, float *bias);

static int failures = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, "FAIL: " __VA_ARGS__);  \
      fprintf(stderr, "\n");                  \
      failures++;                             \
    }                                         \
  } while (0)

typedef struct {
  oracle_bank b;
  void *mem[6];
} owned_bank;

static void *xalloc(size_t n) {
  void *p = calloc(n ? n : 1, 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

/* One bank of E experts of format fmt, every matrix drawn from its own stream. */
static owned_bank make_bank(int fmt, int E, int H, int I, uint64_t seed) {
  owned_bank o;
  memset(&o, 0, sizeof o);
  o.b.fmt = fmt;
  o.b.E = E;
  o.b.H = H;
  o.b.I = I;
  const size_t gu = (size_t)2 * I * H, dn = (size_t)H * I;
  uint8_t *guc, *dnc;
  switch (fmt) {
    case ORACLE_NVFP4: {
      guc = xalloc(E * gu / 2);
      uint8_t *gus = xalloc(E * gu / 16);
      float *gug = xalloc(sizeof(float) * E * 2 * I);
      dnc = xalloc(E * dn / 2);
      uint8_t *dns = xalloc(E * dn / 16);
      float *dng = xalloc(sizeof(float) * E * H);
      for (int e = 0; e < E; e++) {
        synth_nvfp4_matrix(seed, 1, e, 2 * I, H, 0.02, guc + e * gu / 2, gus + e * gu / 16, gug + (size_t)e * 2 * I);
        synth_nvfp4_matrix(seed, 2, e, H, I, 0.02, dnc + e * dn / 2, dns + e * dn / 16, dng + (size_t)e * H);
      }
      o.b.gate_up_scale = gus;
      o.b.gate_up_global = gug;
      o.b.down_scale = dns;
      o.b.down_global = dng;
      o.mem[2] = gus;
      o.mem[3] = gug;
      o.mem[4] = dns;
      o.mem[5] = dng;
      break;
    }
    case ORACLE_FP8BLK: {
      guc = xalloc(E * gu);
      float *gus = xalloc(sizeof(float) * E * (2 * I / 128) * (H / 128));
      dnc = xalloc(E * dn);
      float *dns = xalloc(sizeof(float) * E * (H / 128) * (I / 128));
      for (int e = 0; e < E; e++) {
        synth_fp8blk_matrix(seed, 1, e, 2 * I, H, 0.02, guc + e * gu, gus + (size_t)e * (2 * I / 128) * (H / 128));
        synth_fp8blk_matrix(seed, 2, e, H, I, 0.02, dnc + e * dn, dns + (size_t)e * (H / 128) * (I / 128));
      }
      o.b.gate_up_scale = gus;
      o.b.down_scale = dns;
      o.mem[2] = gus;
      o.mem[4] = dns;
      break;
    }
    case ORACLE_MXFP4: {
      guc = xalloc(E * gu / 2);
      uint8_t *gus = xalloc(E * gu / 32);
      dnc = xalloc(E * dn / 2);
      uint8_t *dns = xalloc(E * dn / 32);
      for (int e = 0; e < E; e++) {
        synth_mxfp4_matrix(seed, 1, e, 2 * I, H, 0.02, guc + e * gu / 2, gus + e * gu / 32);
        synth_mxfp4_matrix(seed, 2, e, H, I, 0.02, dnc + e * dn / 2, dns + e * dn / 32);
      }
      o.b.gate_up_scale = gus;
      o.b.down_scale = dns;
      o.mem[2] = gus;
      o.mem[4] = dns;
      break;
    }
    case ORACLE_BF16: {
      uint16_t *g = xalloc(2 * E * gu), *d = xalloc(2 * E * dn);
      for (int e = 0; e < E; e++) {
        synth_bf16_normal(seed, 1, e, 0.02, (int64_t)gu, g + e * gu);
        synth_bf16_normal(seed, 2, e, 0.02, (int64_t)dn, d + e * dn);
      }
      guc = (uint8_t *)g;
      dnc = (uint8_t *)d;
      break;
    }
    default: { /* Q4_0 */
      guc = xalloc(E * gu / 2);
      uint16_t *gus = xalloc(2 * E * gu / 32);
      dnc = xalloc(E * dn / 2);
      uint16_t *dns = xalloc(2 * E * dn / 32);
      for (int e = 0; e < E; e++) {
        synth_q4_0_matrix(seed, 1, e, 2 * I, H, 0.02, guc + e * gu / 2, gus + e * gu / 32);
        synth_q4_0_matrix(seed, 2, e, H, I, 0.02, dnc + e * dn / 2, dns + e * dn / 32);
      }
      o.b.gate_up_scale = gus;
      o.b.down_scale = dns;
      o.mem[2] = gus;
      o.mem[4] = dns;
      break;
    }
  }
  o.b.gate_up = guc;
  o.b.down = dnc;
  o.mem[0] = guc;
  o.mem[1] = dnc;
  return o;
}

static void free_bank(owned_bank *o) {
  for (int i = 0; i < 6; i++) free(o->mem[i]);
}

/* route -> align -> expert forward (full I and two slices) for one layer */
static void run_layer(int fmt, int T, int E, int k, int H, int I, int with_shared, int with_bias, uint64_t seed) {
  owned_bank routed = make_bank(fmt, E, H, I, seed), shared;
  if (with_shared) shared = make_bank(fmt, 1, H, I, seed + 17);
  uint16_t *x = xalloc(2 * (size_t)T * H), *wr = xalloc(2 * (size_t)E * H);
  synth_bf16_normal(seed, 3, 0, 1.0, (int64_t)T * H, x);
  synth_bf16_normal(seed, 4, 0, 0.02, (int64_t)E * H, wr);
  float *bias = NULL;
  if (with_bias) {
    bias = xalloc(sizeof(float) * E);
    synth_zipf_bias(seed, 5, E, 1.1, bias);
  }
  double *logits = xalloc(sizeof(double) * (size_t)T * E), *w = xalloc(sizeof(double) * (size_t)T * k);
  double *gap = xalloc(sizeof(double) * (size_t)T);
  int32_t *ids = xalloc(sizeof(int32_t) * (size_t)T * k);
  CHECK(oracle_route(x, T, H, wr, E, bias, k, 1, logits, ids, w, gap) == 0, "oracle_route fmt %d", fmt);
  for (int i = 0; i < T * k; i++) CHECK(ids[i] >= 0 && ids[i] < E, "route id %d out of range", ids[i]);
  for (int i = 0; i < T * k; i++) CHECK(isfinite(w[i]) && w[i] >= 0, "route weight");
  for (int BM = 16; BM <= 128; BM *= 2) {
    const int32_t cap = oracle_align_capacity(T, k, E, BM);
    CHECK(cap > 0 && cap % BM == 0, "capacity %d for BM %d", cap, BM);
    int32_t *sorted = xalloc(sizeof(int32_t) * cap), *blk = xalloc(sizeof(int32_t) * (cap / BM));
    int32_t *counts = xalloc(sizeof(int32_t) * E), *offs = xalloc(sizeof(int32_t) * (E + 1)), tp = -1;
    CHECK(oracle_align(ids, T, k, E, BM, sorted, blk, counts, offs, &tp) == 0, "oracle_align BM %d", BM);
    int *seen = xalloc(sizeof(int) * (size_t)T * k);
    for (int p = 0; p < cap; p++)
      if (sorted[p] < T * k) {
        CHECK(sorted[p] >= 0, "sorted id");
        if (sorted[p] >= 0) seen[sorted[p]]++;
      }
    for (int f = 0; f < T * k; f++) CHECK(seen[f] == 1, "pair %d placed %d times", f, seen[f]);
    CHECK(tp >= 0 && tp <= cap && offs[E] == tp, "total_padded");
    free(seen);
    free(sorted);
    free(blk);
    free(counts);
    free(offs);
  }
  const int cuts[3][2] = {{0, I}, {0, I / 2}, {I / 2, I}};
  double *out = xalloc(sizeof(double) * (size_t)T * H);
  for (int c = 0; c < 3; c++) {
    for (size_t i = 0; i < (size_t)T * H; i++) out[i] = NAN;
    CHECK(oracle_expert_forward(&routed.b, with_shared ? &shared.b : NULL, x, T, k, ids, w, cuts[c][0], cuts[c][1],
                                out) == 0,
          "oracle_expert_forward fmt %d slice [%d,%d)", fmt, cuts[c][0], cuts[c][1]);
    for (size_t i = 0; i < (size_t)T * H; i++) CHECK(isfinite(out[i]), "forward output %zu not finite", i);
  }
  double *dq = xalloc(sizeof(double) * (size_t)2 * I * H);
  oracle_dequant_gate_up(&routed.b, E - 1, dq);
  oracle_dequant_down(&routed.b, 0, dq);
  for (size_t i = 0; i < (size_t)H * I; i++) CHECK(isfinite(dq[i]), "dequant");
  free(dq);
  free(out);
  free(x);
  free(wr);
  free(bias);
  free(logits);
  free(w);
  free(gap);
  free(ids);
  free_bank(&routed);
  if (with_shared) free_bank(&shared);
}

int main(void) {
  for (unsigned c = 0; c < 16; c++) CHECK(oracle_e2m1(c) == oracle_e2m1(c), "e2m1");
  for (unsigned b = 0; b < 256; b++) {
    (void)oracle_e4m3fn(b);
    (void)oracle_e8m0(b);
  }
  for (unsigned b = 0; b < 65536; b += 7) {
    (void)oracle_bf16(b);
    (void)oracle_f16(b);
  }
  const int fmts[5] = {ORACLE_NVFP4, ORACLE_FP8BLK, ORACLE_MXFP4, ORACLE_BF16, ORACLE_Q4_0};
  for (int i = 0; i < 5; i++) {
    const int f = fmts[i];
    const int H = f == ORACLE_FP8BLK ? 256 : 128, I = f == ORACLE_FP8BLK ? 256 : 128;
    run_layer(f, 5, 8, 2, H, I, 1, 1, 100 + i);    /* ragged T, shared expert, bias */
    run_layer(f, 1, 4, 4, H, I, 0, 0, 200 + i);    /* one token, k = E */
    run_layer(f, 33, 16, 3, H, I, 1, 0, 300 + i);  /* several tiles of pairs */
  }
  /* degenerate routing inputs: no tokens, k = E = 1 */
  int32_t ids0[1] = {0};
  const int32_t cap1 = oracle_align_capacity(1, 1, 1, 16);
  int32_t *s1 = xalloc(sizeof(int32_t) * cap1), b1[1], c1[1], o1[2], t1 = 0;
  CHECK(oracle_align(ids0, 1, 1, 1, 16, s1, b1, c1, o1, &t1) == 0 && t1 == 16, "align k = E = 1");
  free(s1);
  CHECK(oracle_align_capacity(0, 8, 256, 16) >= 0, "capacity at T = 0");
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
