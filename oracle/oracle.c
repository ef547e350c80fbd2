/*
 * oracle.c -- plain, slow, fp64 CPU reference of one quantized MoE expert layer on a
 * slice [lo, hi) of the expert intermediate dimension.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * What it computes (FreeToken pages):
 *   - SwiGLU expert y = (silu(x Wg^T) * (x Wu^T)) Wd^T, linear in the intermediate index,
 *     so a slice [lo,hi) of I gives a hidden-width partial sum (issue #520, section 4
 *     "Expert sharding").
 *   - gate_up is [2I, H] with gate rows [0, I) and up rows [I, 2I); a slice reads gate
 *     rows [lo,hi) and up rows [I+lo, I+hi); down is [H, I] and a slice reads columns
 *     [lo,hi) (issue #62, "What it touches" item 1).
 *   - Companion scales follow their weight's axis; the NVFP4 per-output-row global is
 *     [N] (PR #637, "Implementation notes"); fp8-block weights carry a 128x128
 *     weight_scale_inv; DeepSeek-V4 FP4 experts carry 32-element scale blocks (PR #70,
 *     "Checkpoint loading").  NVFP4 groups are 16 elements (issue #520 section 2).
 *   - The router is replicated; top-k with norm_topk_prob renormalisation (issue #62,
 *     second comment; PR #70 ownership table).
 *   - The shared SwiGLU expert runs on the same slice and is added to the routed partial
 *     before the single reduction (PR #70 ownership table and the paragraph after it).
 *   - NVFP4 runs as W4A16: weights are dequantized and multiplied against 16-bit
 *     activations (issue #520 section 2).  Here that product is exact in fp64.
 *
 * Readings where the pages are silent (each listed with its reason in the design notes):
 *   low nibble = even K index; W = e2m1 * e4m3(scale) * global (NVFP4),
 *   W = e4m3 * scale_inv (fp8-block), W = e2m1 * 2^(e8m0-127) (MXFP4); scale group
 *   index c/16, c/32, (r/128, c/128) from the matrix origin; softmax routing with the
 *   expert order (logit descending, index ascending) and the decision taken on
 *   fp32-rounded logits; moe_align = stable counting sort by expert, each group padded
 *   to a multiple of the block size with the sentinel T*k; plain silu(g)*u.
 *
 * Format constants of this file (independent of any other module):
 *   ORACLE_NVFP4 = 1, ORACLE_FP8BLK = 2, ORACLE_MXFP4 = 3.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------ decode tables */

/* e2m1 (OCP Microscaling Formats v1.0, FP4 E2M1): 1 sign, 2 exponent (bias 1), 1 mantissa.
 * The 16 values written out: codes 0..7 are the magnitudes, 8..15 their negatives. */
static const double E2M1_VALUES[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double oracle_e2m1(unsigned code) { return E2M1_VALUES[code & 15u]; }

/* e4m3fn (OCP 8-bit floating point, E4M3): bias 7, no infinities, S.1111.111 = NaN,
 * subnormals (m/8) * 2^-6. */
double oracle_e4m3fn(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u) v = ((double)m / 8.0) * ldexp(1.0, -6);
  else v = (1.0 + (double)m / 8.0) * ldexp(1.0, (int)e - 7);
  return s ? -v : v;
}

/* e8m0 (OCP Microscaling v1.0 scale): 2^(b-127); 0xFF = NaN. */
double oracle_e8m0(unsigned b) {
  b &= 255u;
  if (b == 255u) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16(unsigned bits) {
  uint32_t u = (uint32_t)(bits & 0xFFFFu) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0 = subnormal. */
double oracle_f16(unsigned bits) {
  const unsigned E = (bits >> 10) & 31u, f = bits & 1023u;
  double v;
  if (E == 31u) v = f ? NAN : INFINITY;
  else if (E == 0u) v = ldexp((double)f, -24);
  else v = ldexp(1.0 + (double)f / 1024.0, (int)E - 15);
  return (bits & 0x8000u) ? -v : v;
}

/* q4_0 code of element c of a row (32-element blocks of 16 bytes; byte j holds element j in
 * its low nibble and element j + 16 in its high nibble). */
static inline unsigned q4_0_code(const uint8_t *row, int c) {
  const uint8_t b = row[16 * (c / 32) + (c % 32) % 16];
  return (c % 32) < 16 ? (unsigned)(b & 15u) : (unsigned)(b >> 4);
}

static inline unsigned nibble(const uint8_t *row, int c) {
  uint8_t b = row[c >> 1];
  return (c & 1) ? (unsigned)(b >> 4) : (unsigned)(b & 15u); /* even index in the low nibble */
}

/* ------------------------------------------------------------------ dequantization */

/* Element (r, c) of expert e's gate_up matrix [2I, H] (r = output row, c = K index). */
double oracle_weight_gate_up(const oracle_bank *b, int e, int r, int c) {
  const int H = b->H, I = b->I;
  if (b->fmt == ORACLE_NVFP4) {
    const uint8_t *codes = b->gate_up + ((size_t)e * 2 * I + r) * (size_t)(H / 2);
    const uint8_t *sc = (const uint8_t *)b->gate_up_scale + ((size_t)e * 2 * I + r) * (size_t)(H / 16);
    return oracle_e2m1(nibble(codes, c)) * oracle_e4m3fn(sc[c / 16]) *
           (double)b->gate_up_global[(size_t)e * 2 * I + r];
  }
  if (b->fmt == ORACLE_FP8BLK) {
    const uint8_t code = b->gate_up[((size_t)e * 2 * I + r) * (size_t)H + c];
    const float *si = (const float *)b->gate_up_scale + (size_t)e * (2 * I / 128) * (H / 128);
    return oracle_e4m3fn(code) * (double)si[(r / 128) * (H / 128) + c / 128];
  }
  if (b->fmt == ORACLE_BF16) /* unquantized bf16 stacked experts (issue #62 "Suggested staging" 1) */
    return oracle_bf16(((const uint16_t *)b->gate_up)[((size_t)e * 2 * I + r) * (size_t)H + c]);
  if (b->fmt == ORACLE_Q4_0) { /* 32-element blocks (issue #62 "What it touches" item 2) */
    const uint8_t *codes = b->gate_up + ((size_t)e * 2 * I + r) * (size_t)(H / 2);
    const uint16_t *d = (const uint16_t *)b->gate_up_scale + ((size_t)e * 2 * I + r) * (size_t)(H / 32);
    return ((double)q4_0_code(codes, c) - 8.0) * oracle_f16(d[c / 32]);
  }
  /* MXFP4 */
  const uint8_t *codes = b->gate_up + ((size_t)e * 2 * I + r) * (size_t)(H / 2);
  const uint8_t *sc = (const uint8_t *)b->gate_up_scale + ((size_t)e * 2 * I + r) * (size_t)(H / 32);
  return oracle_e2m1(nibble(codes, c)) * oracle_e8m0(sc[c / 32]);
}

/* Element (n, i) of expert e's down matrix [H, I] (n = output row, i = K index). */
double oracle_weight_down(const oracle_bank *b, int e, int n, int i) {
  const int H = b->H, I = b->I;
  if (b->fmt == ORACLE_NVFP4) {
    const uint8_t *codes = b->down + ((size_t)e * H + n) * (size_t)(I / 2);
    const uint8_t *sc = (const uint8_t *)b->down_scale + ((size_t)e * H + n) * (size_t)(I / 16);
    return oracle_e2m1(nibble(codes, i)) * oracle_e4m3fn(sc[i / 16]) *
           (double)b->down_global[(size_t)e * H + n];
  }
  if (b->fmt == ORACLE_FP8BLK) {
    const uint8_t code = b->down[((size_t)e * H + n) * (size_t)I + i];
    const float *si = (const float *)b->down_scale + (size_t)e * (H / 128) * (I / 128);
    return oracle_e4m3fn(code) * (double)si[(n / 128) * (I / 128) + i / 128];
  }
  if (b->fmt == ORACLE_BF16)
    return oracle_bf16(((const uint16_t *)b->down)[((size_t)e * H + n) * (size_t)I + i]);
  if (b->fmt == ORACLE_Q4_0) {
    const uint8_t *codes = b->down + ((size_t)e * H + n) * (size_t)(I / 2);
    const uint16_t *d = (const uint16_t *)b->down_scale + ((size_t)e * H + n) * (size_t)(I / 32);
    return ((double)q4_0_code(codes, i) - 8.0) * oracle_f16(d[i / 32]);
  }
  const uint8_t *codes = b->down + ((size_t)e * H + n) * (size_t)(I / 2);
  const uint8_t *sc = (const uint8_t *)b->down_scale + ((size_t)e * H + n) * (size_t)(I / 32);
  return oracle_e2m1(nibble(codes, i)) * oracle_e8m0(sc[i / 32]);
}

/* ------------------------------------------------------------------ routing */

/* logits[t, e] = sum_h x[t,h] * Wr[e,h] + bias[e], in fp64. */
void oracle_router_logits(const uint16_t *x, int T, int H, const uint16_t *Wr, int E,
                          const float *bias, double *logits) {
#pragma omp parallel for schedule(static) if ((long)T * E * H > (1L << 22))
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int h = 0; h < H; h++)
        acc += oracle_bf16(x[(size_t)t * H + h]) * oracle_bf16(Wr[(size_t)e * H + h]);
      logits[(size_t)t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

/* Expert a ranks before expert b: larger score first, lower index on equal scores. */
static int ranks_before(const double *s, int a, int b) {
  return s[a] > s[b] || (s[a] == s[b] && a < b);
}

/* Top-k of each row of `score` [T, E] plus softmax weights.
 * Selection: the k experts that rank first under (score descending, index ascending),
 * written in that order.  Weights: softmax over the k selected scores when renormalize
 * (norm_topk_prob), else the full softmax probability of each selected expert.
 * gap[t] (optional): score of the k-th minus score of the (k+1)-th expert (inf if k==E). */
int oracle_topk(const double *score, int T, int E, int k, int renormalize, int32_t *ids,
                double *w, double *gap) {
  if (k < 1 || k > E || T < 0) return -1;
  int *order = (int *)malloc(sizeof(int) * (size_t)E);
  for (int t = 0; t < T; t++) {
    const double *s = score + (size_t)t * E;
    /* selection by repeated scan: the j-th pick is the best expert not yet picked */
    char *taken = (char *)calloc((size_t)E, 1);
    for (int j = 0; j < k + 1 && j < E; j++) {
      int best = -1;
      for (int e = 0; e < E; e++)
        if (!taken[e] && (best < 0 || ranks_before(s, e, best))) best = e;
      order[j] = best;
      taken[best] = 1;
    }
    free(taken);
    double mx = s[order[0]], z = 0.0;
    if (renormalize) {
      for (int j = 0; j < k; j++) z += exp(s[order[j]] - mx);
    } else {
      for (int e = 0; e < E; e++) z += exp(s[e] - mx);
    }
    for (int j = 0; j < k; j++) {
      ids[(size_t)t * k + j] = order[j];
      w[(size_t)t * k + j] = exp(s[order[j]] - mx) / z;
    }
    if (gap) gap[t] = (k < E) ? s[order[k - 1]] - s[order[k]] : INFINITY;
  }
  free(order);
  return 0;
}

/* Full route: fp64 logits, rounded to fp32 (the precision the GPU kernel decides in),
 * then top-k and softmax weights on the rounded values.  logits_out (optional) receives
 * the unrounded fp64 logits. */
int oracle_route(const uint16_t *x, int T, int H, const uint16_t *Wr, int E, const float *bias,
                 int k, int renormalize, double *logits_out, int32_t *ids, double *w, double *gap) {
  double *lg = (double *)malloc(sizeof(double) * (size_t)T * E + 8);
  oracle_router_logits(x, T, H, Wr, E, bias, lg);
  if (logits_out) memcpy(logits_out, lg, sizeof(double) * (size_t)T * E);
  for (size_t i = 0; i < (size_t)T * E; i++) lg[i] = (double)(float)lg[i];
  int rc = oracle_topk(lg, T, E, k, renormalize, ids, w, gap);
  free(lg);
  return rc;
}

/* ------------------------------------------------------------------ alignment */

int32_t oracle_align_capacity(int T, int k, int E, int BM) {
  long need = (long)T * k + (long)E * (BM - 1);
  return (int32_t)(((need + BM - 1) / BM) * BM);
}

/* Stable counting sort of the T*k flat pairs f = t*k + j by expert id, each expert's run
 * padded to a multiple of BM with the sentinel T*k.
 *   counts[e]        number of pairs routed to e
 *   offsets[e]       start of e's run; offsets[E] = total_padded
 *   sorted_ids[cap]  pair indices, ascending f within each expert; sentinel elsewhere
 *   block_expert[cap/BM]  expert of each BM-row block, -1 past total_padded */
int oracle_align(const int32_t *ids, int T, int k, int E, int BM, int32_t *sorted_ids,
                 int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded) {
  if (T < 0 || k < 1 || E < 1 || BM < 1) return -1;
  const int P = T * k;
  const int cap = oracle_align_capacity(T, k, E, BM);
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int f = 0; f < P; f++) {
    if (ids[f] < 0 || ids[f] >= E) return -2;
    counts[ids[f]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + ((counts[e] + BM - 1) / BM) * BM;
  *total_padded = offsets[E];
  for (int p = 0; p < cap; p++) sorted_ids[p] = P;
  for (int e = 0; e < E; e++) {
    int pos = offsets[e];
    for (int f = 0; f < P; f++)
      if (ids[f] == e) sorted_ids[pos++] = f;
  }
  for (int bk = 0; bk < cap / BM; bk++) block_expert[bk] = -1;
  for (int e = 0; e < E; e++)
    for (int bk = offsets[e] / BM; bk < offsets[e + 1] / BM; bk++) block_expert[bk] = e;
  return 0;
}

/* ------------------------------------------------------------------ expert layer */

/* y[n] (n in [0,H)) of expert e for token row xt, over intermediate slice [lo,hi):
 *   g_i = xt . Wg[i],  u_i = xt . Wu[I+i],  a_i = silu(g_i) * u_i,  y_n = sum_i a_i Wd[n,i].
 * Wgu/Wd are expert e's dequantized slice: Wgu[2*Il, H] (gate rows then up rows),
 * Wd[H, Il]. */
static void swiglu_expert(const double *xt, const double *Wgu, const double *Wd, int H, int Il,
                          double *a, double *y) {
  for (int i = 0; i < Il; i++) {
    double g = 0.0, u = 0.0;
    const double *wg = Wgu + (size_t)i * H, *wu = Wgu + (size_t)(Il + i) * H;
    for (int h = 0; h < H; h++) {
      g += xt[h] * wg[h];
      u += xt[h] * wu[h];
    }
    a[i] = g / (1.0 + exp(-g)) * u;
  }
  for (int n = 0; n < H; n++) {
    double acc = 0.0;
    const double *wd = Wd + (size_t)n * Il;
    for (int i = 0; i < Il; i++) acc += a[i] * wd[i];
    y[n] = acc;
  }
}

static void dequant_slice(const oracle_bank *b, int e, int lo, int hi, double *Wgu, double *Wd) {
  const int H = b->H, I = b->I, Il = hi - lo;
  for (int i = 0; i < Il; i++)
    for (int h = 0; h < H; h++) {
      Wgu[(size_t)i * H + h] = oracle_weight_gate_up(b, e, lo + i, h);        /* gate row lo+i */
      Wgu[(size_t)(Il + i) * H + h] = oracle_weight_gate_up(b, e, I + lo + i, h); /* up row I+lo+i */
    }
  for (int n = 0; n < H; n++)
    for (int i = 0; i < Il; i++) Wd[(size_t)n * Il + i] = oracle_weight_down(b, e, n, lo + i);
}

/* out[t, n] = sum_j w[t,j] * y_{ids[t,j]}(x_t)[n]  (+ shared expert's y(x_t)[n], weight 1)
 * over the slice [lo, hi).  out is [T, H] fp64, overwritten.  Per output element the sum
 * is taken in the fixed order j = 0..k-1, then the shared term, whatever the threading. */
int oracle_expert_forward(const oracle_bank *routed, const oracle_bank *shared, const uint16_t *x,
                          int T, int k, const int32_t *ids, const double *w, int lo, int hi,
                          double *out) {
  if (!routed || T < 0 || k < 1 || lo < 0 || hi <= lo || hi > routed->I) return -1;
  if (shared && (shared->E != 1 || shared->H != routed->H || hi > shared->I)) return -1;
  const int H = routed->H, E = routed->E, Il = hi - lo, P = T * k;
  for (int f = 0; f < P; f++)
    if (ids[f] < 0 || ids[f] >= E) return -2;
  double *xd = (double *)malloc(sizeof(double) * (size_t)T * H + 8);
  for (size_t i = 0; i < (size_t)T * H; i++) xd[i] = oracle_bf16(x[i]);
  double *Y = (double *)calloc((size_t)(P + T) * H + 8, sizeof(double)); /* per pair, then shared */
  const int nexp = E + (shared ? 1 : 0);
#pragma omp parallel
  {
    double *Wgu = (double *)malloc(sizeof(double) * (size_t)2 * Il * H);
    double *Wd = (double *)malloc(sizeof(double) * (size_t)H * Il);
    double *a = (double *)malloc(sizeof(double) * (size_t)Il);
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < nexp; e++) {
      const int is_shared = (e == E);
      int used = is_shared;
      for (int f = 0; f < P && !used; f++) used = (ids[f] == e);
      if (!used) continue; /* experts with no tokens are never read */
      dequant_slice(is_shared ? shared : routed, is_shared ? 0 : e, lo, hi, Wgu, Wd);
      if (is_shared) {
        for (int t = 0; t < T; t++)
          swiglu_expert(xd + (size_t)t * H, Wgu, Wd, H, Il, a, Y + (size_t)(P + t) * H);
      } else {
        for (int f = 0; f < P; f++)
          if (ids[f] == e) swiglu_expert(xd + (size_t)(f / k) * H, Wgu, Wd, H, Il, a, Y + (size_t)f * H);
      }
    }
    free(Wgu);
    free(Wd);
    free(a);
  }
  for (int t = 0; t < T; t++)
    for (int n = 0; n < H; n++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++) acc += w[(size_t)t * k + j] * Y[(size_t)(t * k + j) * H + n];
      if (shared) acc += Y[(size_t)(P + t) * H + n];
      out[(size_t)t * H + n] = acc;
    }
  free(Y);
  free(xd);
  return 0;
}

/* Whole dequantized matrices of expert e (full I): gate_up [2I, H] and down [H, I]. */
void oracle_dequant_gate_up(const oracle_bank *b, int e, double *out) {
  for (int r = 0; r < 2 * b->I; r++)
    for (int c = 0; c < b->H; c++) out[(size_t)r * b->H + c] = oracle_weight_gate_up(b, e, r, c);
}

void oracle_dequant_down(const oracle_bank *b, int e, double *out) {
  for (int n = 0; n < b->H; n++)
    for (int i = 0; i < b->I; i++) out[(size_t)n * b->I + i] = oracle_weight_down(b, e, n, i);
}

/* Threads the OpenMP loops above use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
