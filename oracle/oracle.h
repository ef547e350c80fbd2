/* oracle.h -- declarations of the fp64 CPU oracle (test infrastructure only; the GPU
 * library never includes this header). */
#ifndef QMOE_ORACLE_H
#define QMOE_ORACLE_H

#include <stdint.h>

#define ORACLE_NVFP4 1
#define ORACLE_FP8BLK 2
#define ORACLE_MXFP4 3
#define ORACLE_BF16 4
#define ORACLE_Q4_0 5

/* One bank of E experts in the full-I layout (expert-major, row-major per matrix).
 *   NVFP4 : gate_up u8 [E,2I,H/2], gate_up_scale e4m3 [E,2I,H/16], gate_up_global f32 [E,2I],
 *           down u8 [E,H,I/2], down_scale e4m3 [E,H,I/16], down_global f32 [E,H]
 *   FP8BLK: gate_up e4m3 [E,2I,H], gate_up_scale f32 [E,2I/128,H/128],
 *           down e4m3 [E,H,I], down_scale f32 [E,H/128,I/128]
 *   MXFP4 : gate_up u8 [E,2I,H/2], gate_up_scale e8m0 [E,2I,H/32],
 *           down u8 [E,H,I/2], down_scale e8m0 [E,H,I/32]
 *   BF16  : gate_up bf16 bits [E,2I,H], down bf16 bits [E,H,I] (passed through the u8 pointers);
 *           no scales or globals
 *   Q4_0  : gate_up u8 [E,2I,H/2], gate_up_scale fp16 bits [E,2I,H/32], down u8 [E,H,I/2],
 *           down_scale fp16 bits [E,H,I/32]; 32-element blocks, byte j of a block holds
 *           element j (low nibble) and j+16 (high nibble); w = (q - 8) * d */
typedef struct {
  int fmt, E, H, I;
  const uint8_t *gate_up;
  const void *gate_up_scale;
  const float *gate_up_global;
  const uint8_t *down;
  const void *down_scale;
  const float *down_global;
} oracle_bank;

double oracle_e2m1(unsigned code);
double oracle_e4m3fn(unsigned b);
double oracle_e8m0(unsigned b);
double oracle_bf16(unsigned bits);
double oracle_f16(unsigned bits);
double oracle_weight_gate_up(const oracle_bank *b, int e, int r, int c);
double oracle_weight_down(const oracle_bank *b, int e, int n, int i);
void oracle_router_logits(const uint16_t *x, int T, int H, const uint16_t *Wr, int E,
                          const float *bias, double *logits);
int oracle_topk(const double *score, int T, int E, int k, int renormalize, int32_t *ids,
                double *w, double *gap);
int oracle_route(const uint16_t *x, int T, int H, const uint16_t *Wr, int E, const float *bias,
                 int k, int renormalize, double *logits_out, int32_t *ids, double *w, double *gap);
int32_t oracle_align_capacity(int T, int k, int E, int BM);
int oracle_align(const int32_t *ids, int T, int k, int E, int BM, int32_t *sorted_ids,
                 int32_t *block_expert, int32_t *counts, int32_t *offsets, int32_t *total_padded);
int oracle_expert_forward(const oracle_bank *routed, const oracle_bank *shared, const uint16_t *x,
                          int T, int k, const int32_t *ids, const double *w, int lo, int hi,
                          double *out);
void oracle_dequant_gate_up(const oracle_bank *b, int e, double *out);
void oracle_dequant_down(const oracle_bank *b, int e, double *out);
int oracle_num_threads(void);

#endif
