/*
 * e4b.h — C ABI of a fused Mixture-of-Experts layer on 4-bit expert weights, for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, on one GPU, the expert part of a MoE layer whose fused expert
 * stacks gate_up_proj [E, 2I, H] and down_proj [E, H, I] (rows = output features,
 * columns = input features, the transformers-v5 layout described in the experts4bit-qlora
 * 0.35.0 project description) are stored as 4-bit codes:
 *
 *   NF4   — 16-entry NormalFloat codebook, one float32 absmax per 64 consecutive weights
 *           of a row, two codes per byte (bitsandbytes pull request #1984, Summary and
 *           Design; grouped-nf4-gemm 0.25.0 project description, opening section and
 *           "Try it on CPU right now" example 1).
 *   MXFP4 — OCP e2m1 codes with one e8m0 scale byte per 32 consecutive weights of a row
 *           (grouped-nf4-gemm 0.25.0 project description, opening section and "Try it on
 *           CPU right now" example 2).
 *
 * The forward multiplies directly on the packed bytes: codes are decoded in registers
 * and scaled per block, products accumulate in fp32, and only the final output is
 * rounded to bf16 (grouped-nf4-gemm 0.25.0 project description, opening section).  No
 * dequantised copy of a weight is ever written.  Beside the forward: the input gradient of
 * the grouped product on the same packed stacks (e4b_grouped_dgrad), and an int4-b32
 * routed decode GEMV with exact integer block sums (e4b_pack_int4_b32, e4b_gemv_int4_b32).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major and dense.
 *     The library allocates and frees nothing; between calls it keeps only a per-device
 *     cache of the architecture check and CU count (and, once a call needs it, the raised
 *     dynamic-LDS limit of the int4 GEMV kernel).  Calls on different streams may run
 *     concurrently if their buffers do not overlap.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work
 *     and return; results are visible after the caller synchronises the stream.
 *   - Arguments are validated on the host before anything is enqueued.  A failed check
 *     returns a negative e4b_status and enqueues nothing.  There is no fallback path:
 *     either the gfx950 kernels run or the call fails.
 *   - Every pointer must be 16-byte aligned.  bf16 values are passed as uint16_t bits.
 *   - Faults inside kernels surface at the caller's next synchronisation; launch
 *     failures return E4B_ERR_HIP.
 *
 * Operand ranges of the forward and the dgrad.  The matrix products take fp16 operands with
 * fp32 accumulation (bf16 inputs are converted exactly where they fit).  The stated output
 * tolerance holds while every operand is an fp16 normal number:
 *   x, g    bf16 activations / gradients: |v| <= 65504.  Larger values become +-inf in fp16
 *           and the output shows inf or NaN; |v| < 2^-14 is carried as an fp16 subnormal
 *           (absolute error <= 2^-25).
 *   NF4     decoded weight = fp16(C[code]) * fp16(absmax * 2^8), product sums scaled by 2^-8
 *           (both exact): every nonzero decoded weight is an fp16 normal (relative error
 *           <= 2^-11 per rounding, two roundings) for 2^-18 <= absmax <= 255.  Larger absmax
 *           overflows; smaller absmax decodes to fp16 subnormals (absolute error <= 2^-33 per
 *           weight).
 *   MXFP4   decoded weight = e2m1 * 2^e, exact in fp16 for scale exponents e = byte - 127 in
 *           [-23, 13]; above 13 large codes overflow, below -23 small codes are rounded.
 *   h       the activation between the two products is stored as fp16: |h| <= 65504 (larger
 *           becomes inf); below 2^-14 it is an fp16 subnormal (absolute error <= 2^-25).
 * These ranges are not checked on the device: a check would need a device-to-host read,
 * which the asynchronous calls never make.
 */
#ifndef E4B_H_
#define E4B_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum e4b_status {
  E4B_OK = 0,
  E4B_ERR_ARG = -1,         /* NULL pointer, non-positive size, bad flag or format */
  E4B_ERR_SHAPE = -2,       /* a dimension breaks a block or tiling constraint */
  E4B_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  E4B_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the queried size */
  E4B_ERR_UNSUPPORTED = -5, /* current device is not gfx950 */
  E4B_ERR_OVERFLOW = -6,    /* a count does not fit the index types (T*k >= 2^31, ...) */
  E4B_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed */
  E4B_ERR_TOO_LARGE = -8    /* more workspace than e4b_moe_forward_noalloc's fixed scratch */
} e4b_status;

typedef enum e4b_fmt { E4B_FMT_NF4 = 0, E4B_FMT_MXFP4 = 1 } e4b_fmt;

/* e4b_route_permute flags */
#define E4B_ROUTE_RENORMALIZE 0x1 /* softmax over the chosen k logits (default reading) */

/* e4b_moe_args.flags: execution path (bits 0-1).  AUTO picks the small-M streaming path
 * when the mean routed rows per expert T*k/E is below 16, the MFMA tile path otherwise
 * (128-row tiles below a mean of 512 rows, 256-row tiles from there).  The choice depends only on host-known sizes; no device value is read back. */
#define E4B_PATH_AUTO 0x0
#define E4B_PATH_GEMM 0x1 /* MFMA grouped GEMM, 128- or 256-row tiles (an expert's last <= 1/4
                           * tile of rows goes to 16-row tiles of the streaming kernel) */
#define E4B_PATH_GEMV 0x2 /* small-M streaming path: 16-row tiles, each expert's weights streamed
                           * once per 16 routed rows */
#define E4B_PATH_MASK 0x3
/* e4b_moe_args.flags bits 2-3: row-tile override for the MFMA path (0 = chosen from the
 * sizes): 32 rows (1 wave), 128 rows (4 waves), 256 rows (4 waves).  An override selects
 * the MFMA path under E4B_PATH_AUTO; with E4B_PATH_GEMV it is E4B_ERR_ARG. */
#define E4B_TILE_AUTO 0x0
#define E4B_TILE_32 0x4
#define E4B_TILE_128 0x8
#define E4B_TILE_256 0xC
#define E4B_TILE_MASK 0xC
/* e4b_moe_args.flags bits 4-5: expert variant of the MXFP4 model family with per-expert
 * biases and a clamped GLU (experts4bit-qlora 0.35.0 project description, Scope; the pages
 * give no formula, so the family's own definition is taken).  Any format may use them.
 *   E4B_ACT_CLAMPED_GLU  h = min(G,7) * sigmoid(1.702 * min(G,7)) * (clamp(U,-7,7) + 1)
 *                        instead of h = silu(G) * U
 *   E4B_GU_INTERLEAVED   gate_up rows interleaved: row 2j is gate j, row 2j+1 is up j
 *                        (default: rows 0..I-1 gate, I..2I-1 up) */
#define E4B_ACT_CLAMPED_GLU 0x10
#define E4B_GU_INTERLEAVED 0x20
/* e4b_moe_args.flags bits 6-7: the route of an MXFP4 gate_up on MFMA tiles (0 = the library's
 * default).  E4B_MXFP4_SCALED: the block-scaled fp8 x fp4 matrix instruction of gfx950 takes the
 * released e2m1 bytes and e8m0 scales as they are, and the bf16 activations exactly as two fp8
 * e4m3 parts under an e8m0 scale per 32 (two instructions per product; remainders below 2^-9 of
 * a block's largest activation rounded to 2^-10 of it).  E4B_MXFP4_FP16: weights decoded to
 * fp16 in registers, fp16 matrix instruction.  Both: E4B_ERR_ARG.  Ignored for NF4 and for the
 * streaming path. */
#define E4B_MXFP4_SCALED 0x40
#define E4B_MXFP4_FP16 0x80
#define E4B_MXFP4_ROUTE_MASK 0xC0
/* e4b_moe_args.flags bit 8: how the down GEMM's results reach the token rows (the weighted
 * combine among the grouped-nf4-gemm 0.25.0 glue kernels, project description opening
 * section).  Clear (the default, deterministic): the down GEMM writes one float32 row per
 * routed slot ([T*k, H] in the workspace) and a last pass sums each token's k rows in slot
 * order, so repeated calls give identical bits.  E4B_COMBINE_ATOMIC, on the MFMA tile path:
 * the down GEMM adds topk_w * (its product) straight into a float32 [T, H] accumulator
 * (out_f32 when given, else the workspace) with device-scope float32 atomic adds, and the
 * last pass only rounds it to bf16; no per-slot rows are written.  The order of a token's k
 * additions then depends on scheduling, so the last bits of out and out_f32 may differ from
 * call to call (each result stays within the same error bound).  On the streaming path
 * (E4B_PATH_GEMV, or AUTO choosing it) the flag is accepted and the combine stays the
 * deterministic one. */
#define E4B_COMBINE_ATOMIC 0x100

/*
 * e4b_pack_nf4 — quantise bf16 expert stacks to NF4.
 *   w       [E, N, K] bf16 (uint16 bits).  K % 64 == 0.
 *   packed  [E, N, K/2] uint8 out.  Byte p of a row holds codes of elements 2p (high
 *           nibble) and 2p+1 (low nibble).
 *   absmax  [E, N, K/64] float32 out: max |w| over each 64-block.
 * Per block: n = w / absmax (float32, correctly rounded); code = index of the nearest
 * codebook value, an exact tie taking the lower code; an all-zero block gets absmax 0
 * and code 7 (zero).  Defined by the pages cited above (per-expert blockwise absmax,
 * [N, K] -> [N, K/2] uint8 + [N, K/64] float32).  Bit-exact and deterministic.
 */
int e4b_pack_nf4(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                 uint8_t* packed, float* absmax, void* stream);

/*
 * e4b_pack_mxfp4 — quantise bf16 expert stacks to MXFP4 (OCP MX v1.0 conversion).
 *   w       [E, N, K] bf16 bits.  K % 32 == 0.
 *   blocks  [E, N, K/32, 16] uint8 out.  Byte p of a block holds element 2p in the low
 *           nibble and 2p+1 in the high nibble (released-checkpoint order).
 *   scales  [E, N, K/32] uint8 out: e8m0 byte = shared exponent + 127, where the shared
 *           exponent is floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an
 *           all-zero block).  Elements are w / 2^exponent rounded to the nearest e2m1
 *           value (ties to even, saturating at 6), sign kept.  Bit-exact.
 */
int e4b_pack_mxfp4(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                   uint8_t* blocks, uint8_t* scales, void* stream);

/* Workspace bytes e4b_route_permute needs for (T, E, k). */
int e4b_route_workspace_bytes(int64_t T, int64_t E, int32_t k, size_t* bytes);

/*
 * e4b_route_permute — top-k routing and the expert-major slot order (the router
 * epilogue among the grouped-nf4-gemm 0.25.0 glue kernels, project description opening
 * section).
 *   logits          [T, E] float32, finite.
 *   k               1 <= k <= E, k <= 64.  E <= 1024.  T*k < 2^31.
 *   topk_ids        [T, k] int32 out: per token the k largest logits in descending
 *                   order, equal logits ordered by the lower expert index.
 *   topk_w          [T, k] float32 out: softmax over the chosen k logits (flag
 *                   E4B_ROUTE_RENORMALIZE), or the full softmax probabilities of the
 *                   chosen experts (flag clear).
 *   expert_offsets  [E+1] int32 out: exclusive prefix sum of per-expert slot counts.
 *   sorted_slots    [T*k] int32 out: slot ids s = t*k + j ordered by expert, then token.
 *   ws, ws_bytes    device workspace of at least e4b_route_workspace_bytes().
 * ids, offsets and slots are bit-exact and deterministic.
 */
int e4b_route_permute(const float* logits, int64_t T, int64_t E, int32_t k, int32_t flags,
                      int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                      int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream);

/* Arguments of e4b_moe_forward.  Sizes: H % 64 == 0, I % 64 == 0 (both formats); T*H,
 * T*k*I and I*H below 2^31 (E4B_ERR_OVERFLOW otherwise). */
typedef struct e4b_moe_args {
  int32_t fmt;            /* e4b_fmt */
  int32_t k;              /* experts per token, as given to e4b_route_permute */
  int64_t E, H, I, T;
  const uint16_t* x;      /* [T, H] bf16 bits; |x| <= 65504 (see "Operand ranges") */
  const uint8_t* w_gu;    /* NF4 [E, 2I, H/2]  | MXFP4 [E, 2I, H/32, 16]; rows 0..I-1 gate, I..2I-1 up */
  const void* s_gu;       /* NF4 float [E, 2I, H/64] | MXFP4 uint8 [E, 2I, H/32] */
  const uint8_t* w_dn;    /* NF4 [E, H, I/2]   | MXFP4 [E, H, I/32, 16] */
  const void* s_dn;       /* NF4 float [E, H, I/64]  | MXFP4 uint8 [E, H, I/32] */
  const float* topk_w;    /* [T, k] routing weights from e4b_route_permute */
  const int32_t* expert_offsets; /* [E+1] from e4b_route_permute */
  const int32_t* sorted_slots;   /* [T*k] from e4b_route_permute */
  uint16_t* out;          /* [T, H] bf16 out: RNE of the fp32 result */
  float* out_f32;         /* [T, H] float32 out, or NULL: the value `out` is rounded from */
  void* ws;               /* device workspace of at least e4b_moe_workspace_bytes() */
  size_t ws_bytes;
  int32_t flags;          /* E4B_PATH_* | E4B_TILE_* | E4B_ACT_* | E4B_GU_* | E4B_MXFP4_* |
                           * E4B_COMBINE_ATOMIC */
  int32_t reserved;       /* must be 0 */
  /* NULL, or 6 hipEvent_t the call records on `stream` around its 5 stages (x conversion,
   * tile map, gate_up GEMM, down GEMM, combine), so a caller can time each kernel on the
   * stream it runs on.  Events are created and owned by the caller. */
  void* const* stage_events;
  /* NULL, or [E, 2I] float32 bias added to each gate_up product (same row order as w_gu),
   * and NULL, or [E, H] float32 bias added to each down product before the weighted sum. */
  const float* b_gu;
  const float* b_dn;
} e4b_moe_args;

/* Workspace bytes e4b_moe_forward needs for the sizes, format and flags in `a`. */
int e4b_moe_workspace_bytes(const e4b_moe_args* a, size_t* bytes);

/*
 * e4b_moe_forward — the MoE expert layer on packed weights.
 * For every token t: out[t] = sum_j topk_w[t,j] * down_e( silu(gate_e(x_t)) * up_e(x_t) )
 * with e = the expert of slot t*k+j (bitsandbytes pull request #1984, Design: per-expert
 * SwiGLU MLP; grouped-nf4-gemm 0.25.0, opening section: one launch over all active
 * experts, table decode, block scaling, fp32 accumulation, bf16 epilogue).
 * Matrix products use fp16 operands (x converted exactly from bf16; decoded weights and
 * the SwiGLU activation rounded to fp16) with fp32 accumulation; the combine is fp32 in
 * a fixed order, so results are deterministic run to run.
 */
int e4b_moe_forward(const e4b_moe_args* a, void* stream);

/*
 * e4b_moe_forward_noalloc — e4b_moe_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * same kernels and results; the workspace is a fixed scratch array the library holds in
 * device memory, one copy per GPU it runs on, until the process ends
 * (e4b_noalloc_scratch_bytes() bytes, 64 MiB: decode-sized batches, e.g. up to T = 64 tokens
 * of a 128-expert top-8 layer with H = 2048, I = 768).
 *   a->ws must be NULL and a->ws_bytes 0 (E4B_ERR_ARG otherwise).  A call whose workspace
 *   (e4b_moe_workspace_bytes) exceeds the scratch returns E4B_ERR_TOO_LARGE and enqueues
 *   nothing.  The call allocates nothing (no hipMalloc, no library allocation); the caller
 *   passes every input and output.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap on one GPU (on
 *   different streams without ordering between them, or from several host threads) race and
 *   must be serialised by the caller.  The scratch keeps the last call's contents; nothing in
 *   it needs to start at zero.
 */
int e4b_moe_forward_noalloc(const e4b_moe_args* a, void* stream);

/* Bytes of the scratch e4b_moe_forward_noalloc uses (a compile-time constant). */
size_t e4b_noalloc_scratch_bytes(void);

/* Arguments of e4b_moe_decode_step.  Sizes: 1 <= T <= 8, T*k <= 64, T*H <= 32768, E <= 1024,
 * H % 64 == 0, I % 64 == 0, I*H < 2^31. */
typedef struct e4b_decode_args {
  int32_t fmt;            /* e4b_fmt */
  int32_t k;              /* experts per token */
  int64_t E, H, I, T;
  int32_t route_flags;    /* E4B_ROUTE_RENORMALIZE or 0, as for e4b_route_permute */
  int32_t flags;          /* E4B_ACT_CLAMPED_GLU | E4B_GU_INTERLEAVED, as for e4b_moe_forward */
  const float* logits;    /* [T, E] float32 router logits */
  const uint16_t* x;      /* [T, H] bf16 bits; |x| <= 65504 */
  const uint8_t* w_gu;    /* packed gate_up stack, as for e4b_moe_forward */
  const void* s_gu;
  const uint8_t* w_dn;    /* packed down stack */
  const void* s_dn;
  const float* b_gu;      /* NULL or [E, 2I] float32 */
  const float* b_dn;      /* NULL or [E, H] float32 */
  int32_t* topk_ids;      /* NULL or [T, k] out: as e4b_route_permute */
  float* topk_w;          /* NULL or [T, k] out (both or neither of topk_ids / topk_w) */
  int32_t* expert_offsets; /* NULL or [E+1] out */
  int32_t* sorted_slots;  /* NULL or [T*k] out */
  uint16_t* out;          /* [T, H] bf16 out: RNE of the fp32 result */
  float* out_f32;         /* NULL or [T, H] float32 out */
  int32_t* status;        /* NULL or one int32 out: 0, or 1 if the grid barrier gave up waiting
                           * (then `out` is not valid) */
  int32_t spin_limit;     /* polls of the grid barrier before it gives up; 0 = the default
                           * (about a million polls, under a second); negative = do not
                           * wait (for tests of the give-up path) */
  int32_t reserved;       /* must be 0 */
  void* ws;               /* device workspace of at least e4b_decode_workspace_bytes(), zero-filled
                           * before the first call with it (e.g. at allocation): its head holds
                           * the kernel's counters, which every call leaves zero again */
  size_t ws_bytes;
} e4b_decode_args;

/* Workspace bytes e4b_moe_decode_step needs for the sizes in `a`. */
int e4b_decode_workspace_bytes(const e4b_decode_args* a, size_t* bytes);

/*
 * e4b_moe_decode_step — one decode step for a few tokens in a single launch: the router
 * epilogue of e4b_route_permute (bit-identical ids, weights, offsets and slots), the grouped
 * gate_up products with the activation, the down products and the weighted combine of
 * e4b_moe_forward (the same fp16-operand / fp32-accumulation numerics, the same tolerance),
 * fused so that the step costs one kernel launch (grouped-nf4-gemm 0.25.0 project
 * description, "What is measured", limit 1: at decode the fused path loses to a CUDA-graphed
 * baseline, its launches costing more than its bytes; the opening section names the router
 * epilogue among the decode glue kernels).  The kernel's workgroups meet once at a grid
 * barrier (between the gate_up and the down products); the grid never exceeds what the device
 * holds at once.  Calls sharing a workspace must not overlap; calls with distinct workspaces
 * may run concurrently.  The result is deterministic run to run.
 */
int e4b_moe_decode_step(const e4b_decode_args* a, void* stream);

/* Arguments of e4b_grouped_dgrad. */
typedef struct e4b_dgrad_args {
  int32_t fmt;            /* e4b_fmt */
  int32_t reserved;       /* must be 0 */
  int64_t E, N, K;        /* packed stack [E, N, K] (as packed by e4b_pack_*); N % 64 == 0, K % 64 == 0 */
  int64_t S;              /* grouped rows: expert_offsets[E] */
  const uint16_t* g;      /* [S, N] bf16 bits, rows grouped by expert; values in fp16 range */
  const uint8_t* w;       /* NF4 [E, N, K/2] | MXFP4 [E, N, K/32, 16] */
  const void* s;          /* NF4 float [E, N, K/64] | MXFP4 uint8 [E, N, K/32] */
  const int32_t* expert_offsets; /* [E+1]: rows of expert e are offsets[e] .. offsets[e+1]-1 */
  float* out_f32;         /* [S, K] float32 out */
  uint16_t* out;          /* [S, K] bf16 out (RNE of out_f32), or NULL */
  void* ws;               /* device workspace of at least e4b_dgrad_workspace_bytes() */
  size_t ws_bytes;
} e4b_dgrad_args;

/* Workspace bytes e4b_grouped_dgrad needs for the sizes in `a`. */
int e4b_dgrad_workspace_bytes(const e4b_dgrad_args* a, size_t* bytes);

/*
 * e4b_grouped_dgrad — the input gradient of the grouped expert product on the packed
 * stacks (Cerin Amroth "ML systems" index, Ownership: the grouped packed GEMM and its dgrad):
 * out[p, :] = g[p, :] @ W_e for every row p of expert e's block, W_e the decoded [N, K]
 * weight.  For gate_up (N = 2I, K = H) g is the gradient of the gate/up products and out
 * the gradient of x's grouped copies; for down (N = H, K = I) g is the gradient of y.
 * fp16 operands (g converted exactly from bf16, weights decoded to fp16) with fp32
 * accumulation; deterministic.  Synchronous errors as e4b_moe_forward.
 */
int e4b_grouped_dgrad(const e4b_dgrad_args* a, void* stream);

/*
 * e4b_pack_int4_b32 — round-to-nearest int4-b32 packing of bf16 stacks (grouped-nf4-gemm
 * 0.25.0 project description, opening section: the int4-b32 decode GEMV and its packer; the
 * pages give no conversion rule, the one below is the plain round-to-nearest reading; the
 * calibrated GPTQ packer needs calibration data and is not provided).
 *   w       [E, N, K] bf16 bits.  K % 32 == 0.
 *   packed  [E, N, K/2] uint8 out: signed 4-bit codes q in [-8, 7], two's complement; byte p
 *           of a row holds element 2p in the low nibble and 2p+1 in the high nibble.
 *   scales  [E, N, K/32] fp16 bits out: s = fp16(absmax / 7) of each 32-block (float32
 *           division, correctly rounded, then round-to-nearest-even to fp16).
 * q = clamp(rint(w / s), -8, 7) with the float32 division by the stored scale; an all-zero
 * block (or one whose scale rounds to 0) gets s = 0 and q = 0.  Weight = s * q.  Bit-exact.
 */
int e4b_pack_int4_b32(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                      uint8_t* packed, uint16_t* scales, void* stream);

/*
 * e4b_quantize_act_int8 — the per-token int8 activations the int4-b32 GEMV multiplies
 * (exact integer accumulation needs integer activations; the pages give no rule, one
 * float32 scale per token is taken).
 *   x   [T, K] bf16 bits.  K % 32 == 0.
 *   q   [T, K] int8 out: clamp(rint(x / s), -127, 127) (float32 division, correctly rounded).
 *   s   [T] float32 out: absmax of the row / 127 (correctly rounded); an all-zero row gets s = 0
 *       and q = 0.  Bit-exact.
 */
int e4b_quantize_act_int8(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* s,
                          void* stream);

/* Arguments of e4b_gemv_int4_b32. */
typedef struct e4b_int4_gemv_args {
  int64_t E, N, K;        /* int4-b32 stack [E, N, K]; N % 16 == 0, K % 128 == 0, K <= 8192 */
  int64_t T;              /* tokens */
  int32_t k;              /* routed experts per token: 1 <= k <= E, k <= 64 */
  int32_t reserved;       /* must be 0 */
  const uint16_t* x;      /* [T, K] bf16 bits */
  const uint8_t* w;       /* [E, N, K/2] as packed by e4b_pack_int4_b32 */
  const uint16_t* s;      /* [E, N, K/32] fp16 bits */
  const int32_t* expert_offsets; /* [E+1], from e4b_route_permute */
  const int32_t* sorted_slots;   /* [T*k], from e4b_route_permute */
  float* out_f32;         /* [T*k, N] float32 out, rows in sorted order */
  void* ws;               /* device workspace of at least e4b_int4_gemv_workspace_bytes() */
  size_t ws_bytes;
} e4b_int4_gemv_args;

/* Workspace bytes e4b_gemv_int4_b32 needs for the sizes in `a`. */
int e4b_int4_gemv_workspace_bytes(const e4b_int4_gemv_args* a, size_t* bytes);

/*
 * e4b_gemv_int4_b32 — the routed decode GEMV on int4-b32 weights with exact integer
 * accumulation (Cerin Amroth "ML systems" index, Solutions: a single-token int4 decode GEMV
 * over routed MoE experts).  For every sorted row p of expert e (token t = sorted_slots[p] / k):
 *   out_f32[p, n] = s_x[t] * sum_b s[e, n, b] * I_b,
 * I_b = sum over the 32 k of block b of q[e, n, k] * q_x[t, k], an exact int32 sum, with q_x,
 * s_x the activations of e4b_quantize_act_int8, recomputed inside the call: into the workspace
 * by a quantiser launch, or, for 1-3 tokens and at most 4096 experts, by each workgroup of the
 * GEMV for its own token rows (the same arithmetic, so the same codes; one launch).  The
 * block terms are summed in float32 in a fixed order: deterministic.  A dense layer is the
 * case E = 1, k = 1.  Synchronous errors as e4b_moe_forward.
 */
int e4b_gemv_int4_b32(const e4b_int4_gemv_args* a, void* stream);

/*
 * e4b_stream_probe — a plain streaming read (mode 0) or copy (mode 1) of `bytes` bytes, the
 * memory ceiling the layer's HBM rates are read against on the same device (grouped-nf4-gemm
 * 0.25.0 project description, "See it on your own hardware first": a ratio is shown beside
 * its instrument's own reference).  Not part of the layer.
 *   src   device buffer of `bytes` bytes (a multiple of 16), read once with 16-byte loads.
 *   dst   mode 1: device buffer of `bytes` bytes, written with the copy.  mode 0: NULL, or a
 *         4-byte word the read kernel never writes in practice (its loads feed a value it
 *         stores only on an impossible match).
 */
int e4b_stream_probe(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream);

/* Static description of a status code. */
const char* e4b_status_string(int status);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int e4b_version(void);

#ifdef __cplusplus
}
#endif

#endif /* E4B_H_ */
