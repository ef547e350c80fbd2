/*
 * synth.c -- seeded synthetic inputs for the quantized MoE expert layer.
 *
 * This module only PRODUCES inputs: activations, router weights, router bias and
 * quantized expert banks.  It computes none of the layer (no routing, no alignment,
 * no GEMM, no SwiGLU).  Both the CPU oracle and the GPU library consume the bytes it
 * writes; it shares no code with either of them.
 *
 * Random numbers: SplitMix64 (S. Vigna, "Further scramblings of Marsaglia's xorshift
 * generators", the splitmix64.c reference) used as a counter-based generator: output i
 * of a stream with key K is mix(K + (i+1)*0x9E3779B97F4A7C15).  Normals come from the
 * Box-Muller transform of two consecutive uniforms.  Streams are keyed by
 * (seed, tensor tag, index) so any expert of any bank can be generated alone and the
 * full-I and I-sliced runs see identical bytes.
 *
 * Quantizers (the encoders the weight formats imply; the decoders live separately in the
 * oracle and in the GPU kernels):
 *   NVFP4     : per-row fp32 global G = amax_row/(6*448); per 16-element group along K an
 *               e4m3fn scale s = RNE((amax_g/6)/G); codes RNE_e2m1(w/(s*G)), saturating.
 *   fp8-block : per 128x128 block scale_inv = amax/448 (fp32); codes RNE_e4m3(w/scale_inv).
 *   MXFP4     : per 32-element group along K an e8m0 exponent floor(log2 amax) - 2
 *               (OCP Microscaling v1.0, emax of e2m1 = 2); codes RNE_e2m1(w/2^x), saturating.
 * Packed FP4: two codes per byte, the even K index in the low nibble.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for (seed, tag, index). */
uint64_t synth_key(uint64_t seed, uint32_t tag, uint32_t index) {
  uint64_t k = sm64_mix(seed + GAMMA);
  k = sm64_mix(k ^ (((uint64_t)tag << 32) | (uint64_t)index));
  return k;
}

static inline uint64_t sm64_at(uint64_t key, uint64_t i) { return sm64_mix(key + (i + 1) * GAMMA); }

/* Uniform in (0,1): 53 random bits, offset by half a step so log() never sees 0. */
static inline double u01(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1.0p-53; }

/* Standard normal number i of stream `key` (Box-Muller; even i -> cos, odd i -> sin). */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = u01(sm64_at(key, 2 * p));
  double u2 = u01(sm64_at(key, 2 * p + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* Fill out[0..n) with sigma * N(0,1) numbers start..start+n of stream (seed, tag, index). */
void synth_normal_f64(uint64_t seed, uint32_t tag, uint32_t index, int64_t start, int64_t n,
                      double sigma, double *out) {
  uint64_t key = synth_key(seed, tag, index);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = sigma * normal_at(key, (uint64_t)(start + i));
}

/* Uniform doubles in (0,1), numbers start..start+n of stream (seed, tag, index). */
void synth_uniform_f64(uint64_t seed, uint32_t tag, uint32_t index, int64_t start, int64_t n,
                       double *out) {
  uint64_t key = synth_key(seed, tag, index);
  for (int64_t i = 0; i < n; i++) out[i] = u01(sm64_at(key, (uint64_t)(start + i)));
}

/* fp64 -> fp32 (C cast, round to nearest even) -> bf16 (round to nearest even). */
static inline uint16_t to_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* bf16 tensor of n elements drawn from N(0, sigma^2). */
void synth_bf16_normal(uint64_t seed, uint32_t tag, uint32_t index, double sigma, int64_t n,
                       uint16_t *out) {
  uint64_t key = synth_key(seed, tag, index);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = to_bf16(sigma * normal_at(key, (uint64_t)i));
}

/* ---------------- encoders (round to nearest, ties to even) ---------------- */

/* |v| -> e2m1 magnitude code 0..7 for the grid {0,.5,1,1.5,2,3,4,6}, saturating at 6.
 * Midpoints that tie go to the even code. */
static inline uint8_t enc_e2m1_mag(double a) {
  return (uint8_t)((a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) +
                   (a > 5.0));
}
static inline uint8_t enc_e2m1(double v) {
  uint8_t m = enc_e2m1_mag(fabs(v));
  return (v < 0 && m) ? (uint8_t)(m | 8) : m;
}

/* fp64 -> OCP e4m3fn code, saturating at 448 (0x7E). */
static uint8_t enc_e4m3(double v) {
  double a = fabs(v);
  uint8_t code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < 0x1.0p-6) {
    code = (uint8_t)nearbyint(a * 512.0); /* subnormal step 2^-9; 8 lands on 0x08 = 2^-6 */
  } else {
    int ex;
    double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5,1) */
    int e = ex - 1;           /* a = (2f) * 2^e */
    int m = (int)nearbyint((2.0 * f - 1.0) * 8.0);
    if (m == 8) { e += 1; m = 0; }
    if (e > 8 || (e == 8 && m == 7)) code = 0x7E;
    else code = (uint8_t)(((e + 7) << 3) | m);
  }
  return (v < 0 && code) ? (uint8_t)(code | 0x80) : code;
}

/* Encoder-side inverse of enc_e4m3 (needed to form the residual w/(s*G)). */
static double val_e4m3(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp((double)m, -9);
  return (b & 0x80) ? -v : v;
}

/* ---------------- quantized matrices [rows, cols], K = cols ---------------- */

/* NVFP4: codes [rows, cols/2], scales [rows, cols/16] e4m3fn, global [rows] fp32. */
void synth_nvfp4_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols,
                        double sigma, uint8_t *codes, uint8_t *scales, float *global) {
  uint64_t key = synth_key(seed, tag, index);
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
    for (int r = 0; r < rows; r++) {
      double amax = 0.0;
      for (int c = 0; c < cols; c++) {
        w[c] = sigma * normal_at(key, (uint64_t)r * (uint64_t)cols + (uint64_t)c);
        if (fabs(w[c]) > amax) amax = fabs(w[c]);
      }
      float G = amax > 0.0 ? (float)(amax / (6.0 * 448.0)) : 1.0f;
      global[r] = G;
      uint8_t *crow = codes + (size_t)r * (cols / 2);
      uint8_t *srow = scales + (size_t)r * (cols / 16);
      for (int g = 0; g < cols / 16; g++) {
        double ga = 0.0;
        for (int c = 0; c < 16; c++) {
          double a = fabs(w[g * 16 + c]);
          if (a > ga) ga = a;
        }
        uint8_t s = enc_e4m3((ga / 6.0) / (double)G);
        srow[g] = s;
        double step = val_e4m3(s) * (double)G;
        for (int c = 0; c < 16; c += 2) {
          uint8_t lo = step > 0.0 ? enc_e2m1(w[g * 16 + c] / step) : 0;
          uint8_t hi = step > 0.0 ? enc_e2m1(w[g * 16 + c + 1] / step) : 0;
          crow[(g * 16 + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
    free(w);
  }
}

/* fp8-block: codes [rows, cols] e4m3fn, scale_inv [rows/128, cols/128] fp32. */
void synth_fp8blk_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols,
                         double sigma, uint8_t *codes, float *scale_inv) {
  uint64_t key = synth_key(seed, tag, index);
  int rb = rows / 128, cb = cols / 128;
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * 128 * (size_t)cols);
#pragma omp for schedule(static)
    for (int br = 0; br < rb; br++) {
      for (int r = 0; r < 128; r++)
        for (int c = 0; c < cols; c++)
          w[(size_t)r * cols + c] =
              sigma * normal_at(key, (uint64_t)(br * 128 + r) * (uint64_t)cols + (uint64_t)c);
      for (int bc = 0; bc < cb; bc++) {
        double amax = 0.0;
        for (int r = 0; r < 128; r++)
          for (int c = 0; c < 128; c++) {
            double a = fabs(w[(size_t)r * cols + bc * 128 + c]);
            if (a > amax) amax = a;
          }
        float si = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
        scale_inv[(size_t)br * cb + bc] = si;
        for (int r = 0; r < 128; r++)
          for (int c = 0; c < 128; c++)
            codes[(size_t)(br * 128 + r) * cols + bc * 128 + c] =
                enc_e4m3(w[(size_t)r * cols + bc * 128 + c] / (double)si);
      }
    }
    free(w);
  }
}

/* MXFP4: codes [rows, cols/2], scales [rows, cols/32] e8m0. */
void synth_mxfp4_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols,
                        double sigma, uint8_t *codes, uint8_t *scales) {
  uint64_t key = synth_key(seed, tag, index);
#pragma omp parallel
  {
    double w[32];
#pragma omp for schedule(static)
    for (int r = 0; r < rows; r++) {
      uint8_t *crow = codes + (size_t)r * (cols / 2);
      uint8_t *srow = scales + (size_t)r * (cols / 32);
      for (int g = 0; g < cols / 32; g++) {
        double amax = 0.0;
        for (int c = 0; c < 32; c++) {
          w[c] = sigma * normal_at(key, (uint64_t)r * (uint64_t)cols + (uint64_t)(g * 32 + c));
          if (fabs(w[c]) > amax) amax = fabs(w[c]);
        }
        int x = 0;
        if (amax > 0.0) {
          int ex;
          frexp(amax, &ex); /* amax in [2^(ex-1), 2^ex) */
          x = (ex - 1) - 2;
        }
        if (x < -127) x = -127;
        if (x > 127) x = 127;
        srow[g] = (uint8_t)(x + 127);
        double step = ldexp(1.0, x);
        for (int c = 0; c < 32; c += 2) {
          uint8_t lo = enc_e2m1(w[c] / step), hi = enc_e2m1(w[c + 1] / step);
          crow[(g * 32 + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
  }
}

/* Per-expert router bias with Zipf(s) popularity: expert e gets rank pi(e)+1 of a seeded
 * permutation pi and bias ln p_rank, p_r = r^-s / sum_{r'=1..E} r'^-s. */
/* IEEE binary16 bits of v, round to nearest even (subnormals included; |v| >= 65520 -> inf). */
static uint16_t to_f16(double v) {
  const uint16_t sign = v < 0.0 ? 0x8000u : 0u;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  int e;
  const double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  int E = e + 14;                 /* biased exponent of a normal result */
  if (E >= 1) {
    long f = lrint((2.0 * m - 1.0) * 1024.0);
    if (f == 1024) {
      f = 0;
      E += 1;
    }
    if (E >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (E << 10) | f);
  }
  return (uint16_t)(sign | lrint(a * 16777216.0)); /* subnormal: units of 2^-24 (1024 -> smallest normal) */
}

static double val_f16(uint16_t b) {
  const int E = (b >> 10) & 31, f = b & 1023;
  const double v = E == 0 ? ldexp((double)f, -24) : ldexp(1.0 + f / 1024.0, E - 15);
  return (b & 0x8000u) ? -v : v;
}

/* q4_0 (llama.cpp's 32-element blocks): per block, the element of largest magnitude m sets
 * d = m / -8 (stored as fp16), codes q = clamp(floor(v / d + 8.5), 0, 15), so w = (q - 8) d;
 * byte j of a block holds element j in its low nibble and element j + 16 in its high nibble.
 * codes [rows, cols/2], d [rows, cols/32] fp16 bits. */
void synth_q4_0_matrix(uint64_t seed, uint32_t tag, uint32_t index, int rows, int cols, double sigma,
                       uint8_t *codes, uint16_t *d) {
  uint64_t key = synth_key(seed, tag, index);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; r++) {
    double w[32];
    for (int b = 0; b < cols / 32; b++) {
      double m = 0.0;
      for (int c = 0; c < 32; c++) {
        w[c] = sigma * normal_at(key, (uint64_t)r * (uint64_t)cols + (uint64_t)(32 * b + c));
        if (fabs(w[c]) > fabs(m)) m = w[c];
      }
      const uint16_t db = to_f16(m / -8.0);
      d[(size_t)r * (cols / 32) + b] = db;
      const double dv = val_f16(db), id = dv != 0.0 ? 1.0 / dv : 0.0;
      uint8_t *blk = codes + (size_t)r * (cols / 2) + 16 * b;
      for (int j = 0; j < 16; j++) {
        int q0 = (int)floor(w[j] * id + 8.5), q1 = (int)floor(w[j + 16] * id + 8.5);
        q0 = q0 < 0 ? 0 : q0 > 15 ? 15 : q0;
        q1 = q1 < 0 ? 0 : q1 > 15 ? 15 : q1;
        blk[j] = (uint8_t)(q0 | (q1 << 4));
      }
    }
  }
}

void synth_zipf_bias(uint64_t seed, uint32_t tag, int E, double s, float *bias) {
  int *perm = (int *)malloc(sizeof(int) * (size_t)E);
  for (int e = 0; e < E; e++) perm[e] = e;
  uint64_t key = synth_key(seed, tag, 0);
  for (int e = E - 1; e > 0; e--) { /* Fisher-Yates */
    int j = (int)(u01(sm64_at(key, (uint64_t)e)) * (double)(e + 1));
    if (j > e) j = e;
    int t = perm[e]; perm[e] = perm[j]; perm[j] = t;
  }
  double z = 0.0;
  for (int r = 1; r <= E; r++) z += pow((double)r, -s);
  for (int e = 0; e < E; e++) bias[e] = (float)log(pow((double)(perm[e] + 1), -s) / z);
  free(perm);
}

/* Random int32 values in [0, n) (for align inputs that do not come from routing). */
void synth_randint(uint64_t seed, uint32_t tag, uint32_t index, int64_t count, int32_t n,
                   int32_t *out) {
  uint64_t key = synth_key(seed, tag, index);
  for (int64_t i = 0; i < count; i++) {
    int32_t v = (int32_t)(u01(sm64_at(key, (uint64_t)i)) * (double)n);
    out[i] = v < n ? v : n - 1;
  }
}
