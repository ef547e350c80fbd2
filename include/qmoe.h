/*
 * qmoe.h -- C ABI of an MI355X (gfx950) library that computes one quantized
 * Mixture-of-Experts layer on a slice [slice_lo, slice_hi) of the expert intermediate
 * dimension I: top-k routing, token->expert alignment, the gate_up grouped GEMM with a
 * SwiGLU epilogue, the down projection to hidden-width partial sums, and the
 * routing-weighted combine with the shared expert.
 *
 * Source of the operation: the FreeToken pages (issue #520 "[TP=2] Quantized MoE expert
 * parallelism ...", issue #62 "Offloaded MoE ignores tensor parallelism ...", PR #637
 * "tensor-parallel weight sharding", PR #70 "tensor-parallel DeepSeek-V4 runtime").
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers, except the two descriptor structs
 *     (moe_bank, moe_align_out), which live in host memory and hold device pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call only
 *     enqueues work on that stream and returns; nothing synchronises with the host, no
 *     device memory is allocated or freed, and grid sizes depend on host arguments only
 *     (never on device-side counts), so a sequence of calls can be captured in a HIP graph.
 *     The expert-layer calls are dense in and dense out with static shapes, as the pages'
 *     fused kernels are (issue #62, second comment; issue #62 "Why not expert parallelism").
 *   - The caller owns every buffer.  The library keeps no pointer after a call returns and
 *     never aliases one argument through another (the pages clone every shard so that no
 *     view pins its parent: issue #520 section 4 ".clone()", PR #70 "Checkpoint loading").
 *   - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  All argument checks run on
 *     the host before anything is enqueued ("fail with a targeted configuration error
 *     before any layer is built", PR #70 "Checkpoint loading"; "does not silently pad",
 *     PR #70 "Scope and non-goals").  moe_last_error() returns this thread's detail text.
 *   - T == 0 (no tokens) is a successful no-op once the other arguments check out; arrays
 *     whose size is proportional to T may then be NULL.
 *   - The library runs on gfx950 only; any other device gives MOE_ERR_UNSUPPORTED.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null required pointer, T < 0, k < 1, k > E, bad sizes   */
#define MOE_ERR_ALIGNMENT (-2)   /* slice not on the format's block boundary, or !(0<=lo<hi<=I) */
#define MOE_ERR_UNSUPPORTED (-3) /* shape the kernels do not cover, or device not gfx950     */
#define MOE_ERR_WORKSPACE (-4)   /* workspace smaller than the *_workspace_bytes() figure    */
#define MOE_ERR_HIP (-5)         /* a HIP runtime call or launch failed                      */

/* ------------------------------------------------------------------ expert banks */

/* Weight formats.
 *   MOE_FMT_NVFP4: packed e2m1 codes, one e4m3fn scale per 16 consecutive K elements, and
 *     an fp32 global per output row; W = e2m1 * e4m3(scale) * global, computed as W4A16
 *     (weights dequantized, multiplied against bf16 activations: issue #520 section 2).
 *   MOE_FMT_FP8_BLOCK128: e4m3fn codes with an fp32 weight_scale_inv per 128x128 block;
 *     W = e4m3 * scale_inv (PR #637 "Implementation notes"; PR #70 "Checkpoint loading").
 *   MOE_FMT_MXFP4_E8M0: packed e2m1 codes with an e8m0 scale per 32 consecutive K
 *     elements; W = e2m1 * 2^(e8m0 - 127) (the DeepSeek-V4 routed FP4 experts' 32-element
 *     scale blocks, PR #70 "Checkpoint loading"; issue #62 "What it touches" item 2).
 *   MOE_FMT_BF16: unquantized bf16 stacked experts, the first format the pages stage through
 *     the same slicing (issue #62 "Suggested staging" item 1; PR #637 "What is sharded": bf16
 *     stacked experts are split like the quantized ones); no scales or globals.
 *   MOE_FMT_Q4_0: 4-bit codes in 32-element blocks with an fp16 scale d per block (issue #62
 *     "What it touches" item 2 and "Suggested staging" item 3), in llama.cpp's q4_0 order:
 *     byte j of a block's 16 holds element j (low nibble) and element j + 16 (high nibble);
 *     W = (q - 8) * d.  Slices are on the block, multiples of 32; a packed bank's I must
 *     be a multiple of 128 (one 16-byte piece of each of 4 blocks per 128 elements).
 * Packed FP4 stores two codes per byte, the even K index in the low nibble. */
typedef enum {
  MOE_FMT_NVFP4 = 1,
  MOE_FMT_FP8_BLOCK128 = 2,
  MOE_FMT_MXFP4_E8M0 = 3,
  MOE_FMT_BF16 = 4,
  MOE_FMT_Q4_0 = 5
} moe_format;

/* Byte order of a bank's weight codes and FP4 scales (moe_bank.layout).
 *   MOE_LAYOUT_ROWS    row-major, as stored by the checkpoint (the shapes below).
 *   MOE_LAYOUT_TILE16  the order the expert kernels read, made by moe_pack_bank: every
 *     group of 16 consecutive rows of a matrix (rows of all experts counted together) is
 *     stored piece-major.  For codes the piece is 16 bytes (32 FP4, 16 FP8 or 8 BF16 elements):
 *     byte b of row r sits at (r/16)*16*P + (b/16)*256 + (r%16)*16 + b%16, P = bytes per
 *     row.  FP4 scales use the scale bytes of one 32-element piece as their unit
 *     (NVFP4 2 bytes, MXFP4 1): byte j of row r sits at
 *     (r/16)*16*S + (j/u)*16*u + (r%16)*u + j%u, S = scale bytes per row, u = unit.
 *     Sizes are unchanged; FP8_BLOCK128 scales and the NVFP4 globals keep their order.
 *     Q4_0 differs: its 16-byte piece (s, g) of a row holds, for each of the 4 blocks of the
 *     128-element step s, the 8 elements [8g, 8g+8) of that block as one dword, element 2i in
 *     bits [4i, 4i+4) and element 2i+1 in bits [16+4i, 20+4i); its scale unit is the 8 bytes
 *     of one step's 4 scales.
 *     One wave load is then one contiguous 1 KB run that is already in the matrix-core
 *     operand order (16 rows x 64 bytes), and any slice of rows or columns on a
 *     multiple of 32 elements stays addressable. */
#define MOE_LAYOUT_ROWS 0
#define MOE_LAYOUT_TILE16 1
/* MOE_LAYOUT_MXFP4_T  MXFP4 as some checkpoints store it, transposed (issue #62 "What it
 *     touches" item 3: blocks_t [K/2, N], sliced along N, the scales sliced differently):
 *     every expert matrix W [N, K] is stored as codes [K/2, N] (byte b of column n holds
 *     elements 2b, 2b+1 of row n, the even one in the low nibble) and e8m0 scales [K/32, N];
 *     gate_up has N = 2I (gate columns [0, I), up [I, 2I)) and K = H, down N = H and K = I.
 *     A rank's slice of such a bank is a column range of gate_up (two ranges) and a row
 *     range of down.  Accepted as moe_pack_bank's source only. */
#define MOE_LAYOUT_MXFP4_T 2

/* One bank of E experts, full-I layout, expert-major and row-major per matrix
 * (issue #520 patch, nvfp4.py layout()/pack(); issue #62 "What it touches" item 1):
 *   gate_up        [E, 2I, H] weights: gate rows [0, I), up rows [I, 2I); K = H.
 *                  NVFP4/MXFP4/Q4_0: u8 [E, 2I, H/2]; FP8_BLOCK128: u8 e4m3 [E, 2I, H];
 *                  BF16: bf16 [E, 2I, H].
 *   gate_up_scale  NVFP4: u8 e4m3 [E, 2I, H/16]; FP8_BLOCK128: f32 [E, 2I/128, H/128];
 *                  MXFP4: u8 e8m0 [E, 2I, H/32]; Q4_0: fp16 [E, 2I, H/32];
 *                  BF16: unused (NULL allowed).
 *   gate_up_global NVFP4 only: f32 [E, 2I] (per output row); NULL otherwise.
 *   down           [E, H, I] weights; K = I.  NVFP4/MXFP4/Q4_0: u8 [E, H, I/2];
 *                  FP8_BLOCK128: u8 e4m3 [E, H, I]; BF16: bf16 [E, H, I].
 *   down_scale     NVFP4: u8 e4m3 [E, H, I/16]; FP8_BLOCK128: f32 [E, H/128, I/128];
 *                  MXFP4: u8 e8m0 [E, H, I/32]; Q4_0: fp16 [E, H, I/32];
 *                  BF16: unused (NULL allowed).
 *   down_global    NVFP4 only: f32 [E, H]; NULL otherwise.
 * A rank that stores only its own slice passes that storage as a bank with I = hi - lo
 * and the slice [0, I) (PR #70: TP=1 is the identity layout).
 * `layout` is MOE_LAYOUT_ROWS or MOE_LAYOUT_TILE16 (the order of gate_up, down and their
 * FP4 scales); moe_expert_forward reads TILE16 banks only. */
typedef struct {
  int32_t fmt; /* moe_format */
  int32_t E, H, I;
  const void *gate_up;
  const void *gate_up_scale;
  const float *gate_up_global;
  const void *down;
  const void *down_scale;
  const float *down_global;
  int32_t layout; /* MOE_LAYOUT_* */
} moe_bank;

/* moe_pack_bank -- reorders a MOE_LAYOUT_ROWS (or, for MXFP4, MOE_LAYOUT_MXFP4_T) bank into
 * MOE_LAYOUT_TILE16 storage, once, when the weights are loaded (a pure permutation of bytes:
 * values and formats unchanged).
 *   src   a ROWS bank, or an MXFP4 bank in MOE_LAYOUT_MXFP4_T (device pointers).
 *   dst   a TILE16 bank of the same fmt, E, H and I whose gate_up, gate_up_scale, down and
 *         down_scale point at device buffers of the same sizes as src's, not overlapping
 *         them; dst's FP8_BLOCK128 scales and NVFP4 globals, when they are other buffers
 *         than src's, receive a plain copy.  The caller owns both banks' storage.
 * Requires 16 | 2I, 16 | H and whole 16-byte code pieces per row (H and I multiples of 32
 * for the FP4 formats, of 16 for FP8, of 8 for BF16, of 128 for Q4_0).  Enqueued on `stream`; no host
 * synchronisation. */
int moe_pack_bank(const moe_bank *src, const moe_bank *dst, void *stream);

/* ------------------------------------------------------------------ routing */

/* moe_route -- replicated router and top-k selection (issue #62 second comment:
 * norm_topk_prob defaults to True and the router is replicated; PR #70 ownership table:
 * every rank must make the same expert selection).
 *   x_bf16        [T, H] bf16 tokens.
 *   w_router_bf16 [E, H] bf16 router weight.
 *   bias          [E] f32 added to every token's logits, or NULL.
 *   logits        [T, E] f32 output: logits[t,e] = sum_h x[t,h] W[e,h] + bias[e]
 *                 (fp32 accumulation of exact bf16 products, summed in a fixed order).
 *   topk_ids      [T, k] int32 output: the k experts ranking first under
 *                 (logit descending, expert index ascending), in that order.
 *   topk_w        [T, k] f32 output: softmax over the k selected logits when renormalize
 *                 != 0, else the full softmax probability of each selected expert.
 *   workspace     >= moe_route_workspace_bytes(T, H, E) bytes (split-K partial logits of
 *                 small batches; 0 bytes, and NULL allowed, for large ones).
 * Requires 1 <= k <= min(E, 64), E <= 1024 and H % 128 == 0.  Deterministic. */
size_t moe_route_workspace_bytes(int T, int H, int E);
int moe_route(const void *x_bf16, int T, int H, const void *w_router_bf16, int E,
              const float *bias, int k, int renormalize, float *logits, int32_t *topk_ids,
              float *topk_w, void *workspace, size_t workspace_bytes, void *stream);

/* moe_route_from_logits -- the selection step of moe_route on caller-supplied f32 logits
 * [T, E] (plus bias[e] if non-NULL, added in f32 before selection).  Same outputs and
 * rules as moe_route. */
int moe_route_from_logits(const float *logits, int T, int E, const float *bias, int k,
                          int renormalize, int32_t *topk_ids, float *topk_w, void *stream);

/* ------------------------------------------------------------------ alignment */

/* Output of moe_align: the T*k flat pairs f = t*k + j stably sorted by expert, every
 * expert's run padded to a multiple of block_m with the sentinel T*k.  The pages name this
 * step (moe_align, PR #637 "Notes") without defining it; this is the definition.
 *   sorted_ids   [capacity] int32: pair indices, ascending f within each expert; sentinel
 *                T*k in padding slots and from total_padded to capacity.
 *   block_expert [capacity / block_m] int32: expert of each block_m-row block; -1 past
 *                total_padded.
 *   counts       [E] int32: pairs routed to each expert.
 *   offsets      [E + 1] int32: start of each expert's run; offsets[E] = total_padded.
 *   total_padded [1] int32.
 *   block_m      rows per block: a multiple of 16 in [16, 256].
 *   capacity     must be >= moe_align_capacity(T, k, E, block_m). */
typedef struct {
  int32_t *sorted_ids;
  int32_t *block_expert;
  int32_t *counts;
  int32_t *offsets;
  int32_t *total_padded;
  int32_t block_m;
  int32_t capacity;
} moe_align_out;

/* Rows needed for any routing: T*k + E*(block_m - 1), rounded up to block_m. */
int32_t moe_align_capacity(int T, int k, int E, int block_m);

/* moe_choose_block_m -- the align block size that selects the expert kernels best suited to
 * T tokens routed k ways over E experts of format fmt (a moe_format, or 0 if not known yet).
 * With m = T*k/E pairs per expert on average: 128 (the prefill GEMMs, which reuse each weight
 * tile across 128 pair rows) when m >= 32 and fmt is NVFP4, FP8_BLOCK128 or BF16; otherwise
 * the streaming kernels with 16 (m <= 16), 32 (m <= 64) or 64 rows.  A pure function of its
 * arguments, so every rank picks the same kernels.  Returns MOE_ERR_INVALID_ARG for T < 0,
 * k < 1 or E < 1.  Pass the result to moe_align_capacity / moe_align and, through the align
 * descriptor, to moe_expert_forward. */
int32_t moe_choose_block_m(int T, int k, int E, int fmt);

/* Device workspace moe_align needs (per-chunk expert histograms). */
size_t moe_align_workspace_bytes(int T, int k, int E);

/* moe_align -- stable counting sort of topk_ids [T, k] (int32 in [0, E)).  Every output
 * array in *out is fully written.  Deterministic: the result does not depend on
 * scheduling.  Requires E <= 1024.  An id outside [0, E) is a caller error whose pairs
 * are dropped (they appear nowhere in sorted_ids). */
int moe_align(const int32_t *topk_ids, int T, int k, int E, const moe_align_out *out,
              void *workspace, size_t workspace_bytes, void *stream);

/* moe_route_align -- moe_route followed by moe_align on its topk_ids, in one call, for the
 * decode step: same arguments, outputs and requirements as the two calls (the route
 * arguments, then the align descriptor *out, whose every array is fully written), and
 * results identical to them bit for bit.  For 1 <= T <= 8, E <= 512 and T*k <= 1024 the
 * top-k selection and the counting sort run in one workgroup with the picks kept on chip
 * (one kernel launch fewer than the two calls); otherwise it enqueues exactly what the two
 * calls enqueue.
 *   workspace  >= moe_route_align_workspace_bytes(T, H, E, k) bytes: the router's split-K
 *              partials, then, 256-byte aligned, the alignment histograms.
 * T == 0 enqueues nothing (as moe_route and moe_align). */
size_t moe_route_align_workspace_bytes(int T, int H, int E, int k);
int moe_route_align(const void *x_bf16, int T, int H, const void *w_router_bf16, int E,
                    const float *bias, int k, int renormalize, float *logits, int32_t *topk_ids,
                    float *topk_w, const moe_align_out *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------------------------ expert layer */

/* Device workspace moe_expert_forward needs for (routed, shared, T, k, block_m, slice):
 * with rows = capacity + 128*ceil(T/128) if shared else capacity, Il = hi - lo, and each
 * term rounded up to 256 bytes,
 *   NVFP4, FP8_BLOCK128, BF16, Q4_0:  rows*Il*2  +  (T*k + T_shared)*H*4
 *   MXFP4:  2*rows*Il + 2*rows*Il/32 + 2*T*H + 2*T*H/32  +  (T*k + T_shared)*H*4
 * (the intermediate activation, MXFP4's activation planes, and per-pair partial rows).
 * Returns 0 for arguments moe_expert_forward would reject as invalid. */
size_t moe_workspace_bytes(const moe_bank *routed, const moe_bank *shared, int T, int k,
                           int block_m, int slice_lo, int slice_hi);

#define MOE_OUT_F32 0
#define MOE_OUT_BF16 1

/* moe_expert_forward -- the quantized expert layer on the slice [slice_lo, slice_hi) of I,
 * producing this rank's hidden-width partial sum (issue #520 section 4 "Expert sharding":
 * the MoE output is sum_i silu(gate_i) up_i down_i, linear in the intermediate index).
 *   For every pair f = t*k + j routed to expert e = topk_ids[t, j] (given through `al`):
 *     g_i = x_t . Wg_e[i],  u_i = x_t . Wu_e[I + i]    for i in [lo, hi)  (gate rows
 *       [lo, hi), up rows [I+lo, I+hi): issue #62 "What it touches" item 1)
 *     a_i = silu(g_i) * u_i, rounded to bf16 (the A16 activation of the down GEMM)
 *   MXFP4 runs on the native scaled FP4 MFMA, whose activation operand is 8-bit at most:
 *   x and a are carried as two e4m3 planes, hi = e4m3(v/X1)*X1 and lo = e4m3((v-hi)/X2)*X2,
 *   with e8m0 X1, X2 per 32 elements (about bf16's 8 significant bits), so its results
 *   equal the W4A16 ones to within the documented tolerance, not bit for bit.
 *     y_n = sum_{i in [lo,hi)} a_i Wd_e[n, i]       for n in [0, H)  (down columns)
 *   out[t, :] = sum_j topk_w[t, j] * y(pair t*k+j)  +  shared(x_t)
 *   where the shared expert (weight 1, same slice) is added to the routed partial before
 *   any reduction across ranks (PR #70 ownership table and the paragraph after it).
 * Companion scales are sliced with their weight's axis; the NVFP4 per-row globals of
 * gate_up follow its rows and down_global is used whole (PR #637 "Implementation notes").
 *   routed      E-expert bank; shared: NULL or a 1-expert bank of the same format, H and I;
 *               both in MOE_LAYOUT_TILE16 (moe_pack_bank), else MOE_ERR_UNSUPPORTED.
 *               This is where the call departs from taking banks exactly as the pages store
 *               them: the shapes, the gate/up row ranges, the down column range and the
 *               companion-scale slicing are the pages' (issue #62 "What it touches" item 1,
 *               PR #637 "Implementation notes"), but the bytes of each 16-row tile must have
 *               been reordered once, at load, by moe_pack_bank (a permutation; a rank's slice
 *               stays a pointer range).  Row-major bytes would cost the streaming kernels
 *               about a fifth of their read rate (16 different rows per wave load).
 *   x_bf16      [T, H] bf16; topk_w [T, k] f32; al: the moe_align output for these ids.
 *   slice_lo/hi multiples of the format block (NVFP4 16, MXFP4 32, FP8_BLOCK128 128, BF16 1,
 *               Q4_0 32), with 0 <= lo < hi <= I (issue #62 "What it touches" item 2; PR #70
 *               div_tp(..., multiple_of=128)).  The kernels additionally need lo and hi to
 *               be multiples of 32, else MOE_ERR_UNSUPPORTED.
 *   out         [T, H] f32 (out_dtype MOE_OUT_F32) or bf16 (MOE_OUT_BF16), overwritten.
 *   workspace   >= moe_workspace_bytes(...) bytes of device memory.
 * A token one of whose ids lay outside [0, E) (a caller error: moe_align drops such pairs)
 * gets an undefined output row; every other token's row is unaffected.
 * Experts that received no tokens are never read.  The align block size picks the kernels
 * (moe_choose_block_m gives the library's choice):
 * al->block_m a multiple of 128 runs NVFP4, FP8_BLOCK128 and BF16 on prefill GEMMs that reuse
 * each weight across 128 pair rows (for many tokens per expert); other block sizes,
 * and MXFP4 and Q4_0, run the streaming kernels that read each selected weight byte once per
 * 16-row block (for few tokens per expert).  Both compute the same result, except that the
 * prefill GEMMs round each pair row y to bf16 before the fp32 weighted sum (the pair rows
 * are the layer's largest stream at many tokens; the streaming kernels keep them in fp32). */
int moe_expert_forward(const moe_bank *routed, const moe_bank *shared, const void *x_bf16,
                       int T, int k, const float *topk_w, const moe_align_out *al,
                       int slice_lo, int slice_hi, void *out, int out_dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/* moe_expert_forward_static -- moe_expert_forward on a workspace the library owns, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, kernels and results as
 * moe_expert_forward, without workspace and workspace_bytes: the workspace is a fixed
 * MOE_STATIC_SCRATCH_BYTES device array inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating library routine).
 *   Limit: a call whose moe_workspace_bytes(...) exceeds MOE_STATIC_SCRATCH_BYTES returns
 *   MOE_ERR_WORKSPACE before anything is enqueued (64 MiB holds, e.g., the Qwen3.6-shaped
 *   NVFP4 decode layer at T = 64 and the DeepSeek-V4-Flash-shaped MXFP4 layer at T = 256 on
 *   a 1024-wide slice; prefill batches need moe_expert_forward and a caller workspace).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps what the previous
 *   call left there (no part of it needs to start at zero).  Calls that overlap in time on
 *   one GPU (two streams, two threads, two graphs replayed concurrently) race on it and give
 *   undefined results; order them on one stream.
 *   The first call on a device looks up the array's device address for that device
 *   (hipGetSymbolAddress); make that first call outside graph capture. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_expert_forward_static(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T, int k,
                              const float *topk_w, const moe_align_out *al, int slice_lo, int slice_hi,
                              void *out, int out_dtype, void *stream);

/* The two halves of moe_expert_forward, for callers that time or schedule them apart.
 * Both take the same arguments and the same workspace; moe_expert_down reads what
 * moe_expert_gate_up left in the workspace for the same (routed, shared, x, al, slice). */
int moe_expert_gate_up(const moe_bank *routed, const moe_bank *shared, const void *x_bf16,
                       int T, int k, const moe_align_out *al, int slice_lo, int slice_hi,
                       void *workspace, size_t workspace_bytes, void *stream);
int moe_expert_down(const moe_bank *routed, const moe_bank *shared, int T, int k,
                    const float *topk_w, const moe_align_out *al, int slice_lo, int slice_hi,
                    void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                    void *stream);

/* moe_layer_forward -- the whole layer in one call: moe_route_align (router GEMM, top-k,
 * alignment), then moe_expert_forward on the slice [slice_lo, slice_hi) (gate_up + SwiGLU,
 * down, the weighted combine with the shared expert).  The same arguments, requirements and
 * checks as those two calls (H and E are routed->H and routed->E; the router arguments as in
 * moe_route; *al receives the alignment), and the same outputs bit for bit: logits, topk_ids
 * and topk_w, every array of *al, and out.
 *   route_workspace >= moe_route_align_workspace_bytes(T, H, E, k) bytes;
 *   workspace       >= moe_workspace_bytes(routed, shared, T, k, al->block_m, lo, hi) bytes;
 *   the two must not overlap (kernels of the call use both at once), else MOE_ERR_INVALID_ARG.
 * For one token (T = 1) on 16-row blocks, when the gate_up launch takes 8 waves per
 * workgroup, the top-k and the alignment run inside the gate_up kernel: each routed
 * workgroup sums the router's partial logits and ranks them itself, and the first writes the
 * routing and alignment outputs, so the decode step of one token is the router, gate_up and
 * down kernels (plus MXFP4's activation split), one launch and one kernel boundary fewer
 * than the two calls.  Otherwise it enqueues exactly what the two calls enqueue.  T == 0
 * enqueues nothing. */
int moe_layer_forward(const void *x_bf16, int T, const void *w_router_bf16, const float *bias, int k,
                      int renormalize, const moe_bank *routed, const moe_bank *shared, int slice_lo,
                      int slice_hi, float *logits, int32_t *topk_ids, float *topk_w, const moe_align_out *al,
                      void *out, int out_dtype, void *route_workspace, size_t route_workspace_bytes,
                      void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ diagnostics */

const char *moe_status_string(int status); /* static text for a status code */
const char *moe_last_error(void);          /* this thread's detail text for the last error */

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
