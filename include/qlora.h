/*
 * qlora.h -- C ABI of the MI355X (gfx950) NF4 / QLoRA linear library.
 *
 * What the library computes (the pages it follows are named per call):
 *   - NF4 quantization of a frozen fp32 weight: one absmax per 64 consecutive
 *     weights, nearest of 16 normal-quantile levels per weight, and double
 *     quantization of the absmax values to 8 bits with one fp32 scale per 256
 *     blocks (ultralytics glossary "QLoRA", "Como funciona a QLoRA": NF4 and
 *     double-quantization bullets; paperclase lesson "QLoRA", Partes 1-3).
 *   - dequantization of that weight to bfloat16 (same pages; paperclase
 *     Parte 2, w_hat = NF4[c] * absmax).
 *   - the QLoRA linear, forward h = W_hat x + (alpha/r) B A x and backward
 *     (dX through W_hat and the LoRA path; gradients for A and B only)
 *     (paperclase "QLoRA", Parte 4, "El gradiente atraviesa la base de 4
 *     bits").
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major data on
 *     the current HIP device, 16-byte aligned.  The caller owns every buffer,
 *     including the workspace; the library allocates no device memory and
 *     keeps no pointer after returning.  Its only global state is a
 *     per-device cache of the architecture check (thread-safe).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Each call checks
 *     its arguments on the host, enqueues its kernels on `stream` and
 *     returns; nothing is synchronised.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Return value: QLORA_OK (0) or a negative qlora_status.  A call that
 *     fails validation enqueues nothing and leaves every output untouched.
 *     Validation happens before any HIP call, so it can be exercised on a
 *     machine without a GPU.  No call aborts or throws.
 *   - Outputs must not alias inputs (not checked).
 *   - bfloat16 values are passed as raw 16-bit patterns (qlora_bf16).
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qlora_bf16;   /* raw bfloat16 bits */
typedef void* qlora_stream;    /* hipStream_t */

enum qlora_status {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,      /* a required pointer is NULL */
  QLORA_ERR_SHAPE = -2,     /* a size is negative, not a multiple of 64, or out of range
                               (linear calls: a bf16 operand of 2^31 bytes or more) */
  QLORA_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
  QLORA_ERR_WORKSPACE = -4, /* workspace missing or smaller than qlora_workspace_bytes() */
  QLORA_ERR_LAUNCH = -5,    /* a kernel launch failed (hipGetLastError) */
  QLORA_ERR_DEVICE = -6,    /* no HIP device, or the current device is not gfx950 */
  QLORA_ERR_VALUE = -7      /* a scalar argument is not finite */
};

/* Block and group sizes of the format (fixed). */
#define QLORA_NF4_BLOCK 64      /* weights per absmax block */
#define QLORA_NF4_GROUP 256     /* blocks per double-quantization scale */
#define QLORA_MAX_RANK 256      /* largest LoRA rank r accepted */

/* qlora_nf4_weight.flags: the weight's format.  0 is the double-quantized
 * format; QLORA_NF4_ABSMAX_FP32 the 4.5-bit one (an exact fp32 absmax per
 * block, as nf4_quantize_nodq writes it).  All other bits are reserved and
 * must be 0. */
#define QLORA_NF4_ABSMAX_FP32 0x1u
#define QLORA_NF4_FLAGS_KNOWN 0x1u

/*
 * A frozen NF4 weight W_hat [rows = out_features, cols = in_features].
 * Blocks are 64 consecutive weights of the row-major flattening, so with
 * cols % 64 == 0 a block never crosses a row; double-quantization groups are
 * 256 consecutive blocks of the same flattening and may cross rows.
 *   codes        [rows*cols/2]  packed 4-bit codes; element 2i in bits 0-3,
 *                               element 2i+1 in bits 4-7 of byte i
 *   flags        the format (QLORA_NF4_ABSMAX_FP32 or 0; other bits reserved,
 *                a set reserved bit is QLORA_ERR_VALUE)
 * flags = 0, double-quantized (4 + 8/64 + 32/16384 bits per weight):
 *   absmax_q     [rows*cols/64] 8-bit double-quantized absmax, one per block
 *   absmax_scale [ceil(rows*cols/16384)] fp32 scale per group of 256 blocks
 * flags = QLORA_NF4_ABSMAX_FP32 (4 + 32/64 = 4.5 bits per weight, paperclase
 * "QLoRA", Parte 3, "Bits por parametro"):
 *   absmax_q     unused (may be NULL)
 *   absmax_scale [rows*cols/64] the exact fp32 absmax of each block
 * Code c selects level L[c] of the 16-entry codebook (nf4_codebook), with
 * L ascending and L[7] = +0.0.  The linear calls accept both formats: the
 * 4.5-bit one runs the dequantize-then-bf16-GEMM route at every token count
 * (its W_hat is expanded into the workspace, see qlora_workspace_bytes_flags);
 * qlora_merge takes the double-quantized format only.
 */
typedef struct {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_scale;
  int64_t rows;
  int64_t cols;
  uint32_t flags;
} qlora_nf4_weight;

/*
 * Sizes in bytes of the three NF4 buffers for `numel` weights
 * (numel >= 0, numel % 64 == 0): codes numel/2, absmax_q numel/64,
 * absmax_scale 4*ceil(numel/16384).  That is 4 + 8/64 + 32/16384 bits per
 * weight, the double-quantization budget of paperclase "QLoRA", Parte 3,
 * "Bits por parametro".  Host only; any output pointer may be NULL.
 * Errors: QLORA_ERR_SHAPE.
 */
int nf4_storage_bytes(int64_t numel, size_t* codes_bytes, size_t* absmax_q_bytes,
                      size_t* scale_bytes);

/*
 * nf4_quantize -- Q1..Q4: fp32 weight -> NF4 codes + double-quantized absmax.
 * Follows ultralytics glossary "QLoRA", "Como funciona a QLoRA" (one absmax
 * per 64 weights, nearest of the 16 quantile levels, absmax values quantized
 * to 8 bits in blocks of 256) and paperclase "QLoRA", Parte 4 (codes by argmin
 * of the distance to the levels; two codes per byte).  Per block b of 64
 * weights: a_b = max |w|; per weight x = fl32(w / a_b) and code = the first
 * index j minimising |fl32(x - L[j])|.  Per group g of 256 blocks:
 * s_g = max a_b, q_b = round_half_even(fl32(fl32(a_b / s_g) * 255)).  A zero
 * block gets codes 7 and q 0; a zero group gets s 0.  The last group may be
 * partial.  The codes use the exact fp32 a_b.
 *   w            [numel] fp32, finite (non-finite input: outputs unspecified)
 *   numel        >= 0, multiple of 64, at most 2^36; 0 is a no-op
 *   codes        [numel/2] out;  absmax_q [numel/64] out;
 *   absmax_scale [ceil(numel/16384)] out
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
int nf4_quantize(const float* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                 float* absmax_scale, qlora_stream stream);

/*
 * nf4_dequantize -- D1: NF4 storage -> bfloat16 weight.
 * a_hat_b = fl32(fl32(q_b / 255) * s_g);  w_hat = bf16_rne(fl32(L[c] * a_hat_b))
 * (paperclase "QLoRA", Parte 2: w_hat = NF4[c] * absmax; ultralytics "QLoRA":
 * weights are dequantized to bfloat16 right before the matmul).
 *   codes, absmax_q, absmax_scale as produced by nf4_quantize for numel
 *   (numel limits as for nf4_quantize)
 *   w_out [numel] bf16 out (row-major, same order as the quantized input)
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
int nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_scale,
                   int64_t numel, qlora_bf16* w_out, qlora_stream stream);

/*
 * nf4_quantize_nodq / nf4_dequantize_nodq -- the same format without double
 * quantization: one exact fp32 absmax per 64-weight block, 4 + 32/64 = 4.5
 * bits per weight (paperclase "QLoRA", Parte 3, "Bits por parametro": 4 bits
 * plus the absmax; ultralytics glossary "QLoRA": the NF4 construction and
 * its mean-squared-error comparison use exact block absmax values).
 * Codes exactly as nf4_quantize (they use the exact absmax in both formats);
 * w_hat = bf16_rne(fl32(L[c] * a_b)).
 *   codes  [numel/2];  absmax [numel/64] fp32 (out of quantize, in of dequantize)
 *   numel  >= 0, multiple of 64, at most 2^36 (0 is a no-op)
 * A qlora_nf4_weight with flags = QLORA_NF4_ABSMAX_FP32 and absmax_scale =
 * this absmax array describes such a weight to the linear calls.
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
int nf4_quantize_nodq(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                      qlora_stream stream);
int nf4_dequantize_nodq(const uint8_t* codes, const float* absmax, int64_t numel, qlora_bf16* w_out,
                        qlora_stream stream);

/*
 * Workspace bytes needed by qlora_linear_fwd (backward = 0) or
 * qlora_linear_bwd (backward = 1) for T tokens, in/out features and rank r.
 * Returns 0 for invalid shapes and at least 256 otherwise.  Host only.
 *
 * The workspace is scratch for intermediate products: padded LoRA factors,
 * fp32 partial sums (the rank-r reductions, the token slices of dA and dB,
 * and, below one workgroup per CU, the split-K ranges of a GEMM: at most
 * 32 MiB), the transposed dequantized weight of the backward from T = 17 on
 * or with dropout, and, from T = 512 on, the forward's dequantized weight
 * (2 * out * in bytes each; both calls also run without that weight in the
 * smaller workspaces of qlora_workspace_bytes_fwd_min / _bwd_min).  Up to
 * T = 16 without dropout the backward keeps no dequantized weight: it holds
 * fp32 row-split partials of dX (splits * T * in * 4 bytes, splits <=
 * ceil(512 / (in / 64))) and the rank-r reductions' partials (T * r * 4 bytes
 * per 128 columns / rows).  It needs no initialisation and keeps nothing
 * between calls.  The small-token forward (T <= 16 and r <= 64) uses it only
 * for U = X A^T (n * T * r fp32 values), computed once up front when r > 16
 * or the projections have more than 4096 output rows together; with r <= 16
 * and at most 4096 rows ws may be NULL.  Calls that overlap in time
 * (different streams) must not share a workspace.
 */
size_t qlora_workspace_bytes(int64_t T, int64_t in_features, int64_t out_features, int64_t r,
                             int backward);

/*
 * Workspace bytes for a weight of the given format (qlora_nf4_weight.flags),
 * for n projections sharing X (out_features[0..n-1], 1 <= n <= 8; n = 1 for
 * the single-projection calls), with (dropout = 1) or without LoRA dropout
 * (dropout needs n = 1).  With flags = 0 the result equals the functions
 * above; with QLORA_NF4_ABSMAX_FP32 the forward also holds the expanded W_hat
 * (2 * sum(out) * in bytes) at every T.  Returns 0 for invalid arguments
 * (including reserved flag bits).  Host only.
 */
size_t qlora_workspace_bytes_flags(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                   int64_t r, int backward, int dropout, uint32_t flags);

/*
 * The smallest workspace a backward call accepts (single, multi or dropout
 * form, for a weight of the given format; arguments as in
 * qlora_workspace_bytes_flags with backward = 1): the layout without the
 * expanded W_hat^T, whose dX GEMM dequantizes the weight tiles while it stages
 * them (paperclase "QLoRA", Parte 4: the dequantized weight is built, used
 * and discarded; ultralytics glossary "QLoRA", "Compromissos": the memory
 * saved is paid for in time).  Equal to the full size where no such route
 * exists (T <= 16 without dropout, where the backward never expands W_hat^T;
 * the 4.5-bit format, which always expands it).  Returns 0 for invalid
 * arguments.  Host only.
 */
size_t qlora_workspace_bytes_bwd_min(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                     int64_t r, int dropout, uint32_t flags);

/*
 * The smallest workspace a forward call accepts (single, multi or dropout
 * form; arguments as in qlora_workspace_bytes_flags with backward = 0): the
 * layout without the expanded W_hat, where the GEMM dequantizes each weight
 * tile while it stages it.  Equal to the full size where no such route exists
 * (below 512 tokens, where the forward never expands W_hat; the 4.5-bit
 * format, which always expands it).  Returns 0 for invalid arguments.  Host
 * only.
 */
size_t qlora_workspace_bytes_fwd_min(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                     int64_t r, int dropout, uint32_t flags);

/*
 * qlora_linear_fwd -- F1 + F2: Y = X W_hat^T + (alpha/r) (X A^T) B^T.
 * paperclase "QLoRA", Parte 4, h = W_hat x + (alpha/r) B A x, with
 * W_hat = dq(codes, absmax) as nf4_dequantize defines it.  Where W_hat lives
 * depends on T and the workspace: up to 16 tokens it is rebuilt in registers
 * right before the matrix cores use it; from 17 to 511 tokens it is rebuilt
 * while each weight tile is staged into on-chip memory; from 512 tokens on it
 * is expanded once into the workspace (2 * out * in bytes) and read back by
 * the GEMM when ws_bytes >= qlora_workspace_bytes(T, in, out, r, 0) (the
 * faster route there), and otherwise rebuilt in the staging as below 512
 * (any ws_bytes >= qlora_workspace_bytes_fwd_min; Y is the same bit for bit).
 * bf16 inputs, fp32 accumulation, one rounding of Y to bf16 at the end.
 *   W   NF4 weight [out, in]; in % 64 == 0, out % 64 == 0
 *   X   [T, in] bf16;  T >= 0 (0 is a no-op; X and Y may then be NULL)
 *   A   [r, in] bf16;  B [out, r] bf16;  1 <= r <= 256;  alpha finite
 *   Y   [T, out] bf16 out
 *   ws  workspace of ws_bytes >= qlora_workspace_bytes_fwd_min(T, in, &out, 1, r, 0, flags)
 * Size limit (all linear calls, also multi / dropout / merge): X, Y, dY, dX
 * and the dequantized weight [out, in] in bf16 must each be smaller than
 * 2^31 bytes (QLORA_ERR_SHAPE otherwise); larger token batches are split
 * into several calls.
 * Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, DEVICE, LAUNCH.
 */
int qlora_linear_fwd(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* Y, void* ws, size_t ws_bytes, qlora_stream stream);

/*
 * qlora_linear_fwd_noalloc -- qlora_linear_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and arguments
 * without a workspace.  It uses the library's own scratch instead: a static
 * device array of qlora_noalloc_scratch_bytes() bytes (16 MiB), one copy per
 * GPU, held until the process ends; the call itself allocates nothing.
 *   The call takes the route the scratch holds: from 512 tokens on W_hat is
 *   expanded into it when the whole layout fits, else each weight tile is
 *   dequantized in the GEMM's staging (as qlora_linear_fwd with a smaller
 *   workspace; Y is the same bit for bit).  Calls whose smallest workspace
 *   (qlora_workspace_bytes_fwd_min) exceeds the scratch -- very large
 *   token counts or ranks -- are refused with QLORA_ERR_WORKSPACE before any
 *   HIP call.  The small-token path (T <= 16) needs at most T x r x 4 bytes
 *   and always fits.
 *   Every call on one GPU shares that GPU's scratch (it needs no
 *   initialisation and keeps nothing between calls): calls that overlap in
 *   time on one GPU (different streams, or different host threads without
 *   ordering) race on it and must not be issued.
 * Errors: as qlora_linear_fwd, plus WORKSPACE as above and DEVICE if the
 * scratch cannot be located on the current device.
 */
size_t qlora_noalloc_scratch_bytes(void);
int qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                             const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                             qlora_bf16* Y, qlora_stream stream);

/*
 * Multi-projection forms: n (1..8) projections that share the input X and
 * the rank r / alpha, e.g. q|k|v or gate|up (coddykit "LoRA y QLoRA": the
 * adapters go on several target modules of the same layer; ultralytics
 * glossary "QLoRA": adapters on every linear).  One pass computes
 * X A_i^T for all i, one GEMM launch covers all projections (their outputs
 * side by side), and the backward's dX is one GEMM over the concatenated
 * outputs, rounded once:
 *   Y  [T, N] bf16,  N = sum_i out_i; projection i owns columns
 *                    [sum_{j<i} out_j, sum_{j<=i} out_j) of Y (and of dY)
 *   dX [T, in] = sum_i (dY_i W_hat_i + s (dY_i B_i) A_i), one rounding
 *   dA[i] [r, in], dB[i] [out_i, r] fp32, overwritten
 *   W[i]  NF4 weights, all with the same cols = in and the same flags;  A[i], B[i] as above
 * Arguments and errors otherwise as for the single-projection calls; the
 * workspace is sized by qlora_workspace_bytes_multi (0 for invalid shapes,
 * n outside 1..8 or a NULL out_features).  n = 1 is exactly the
 * single-projection call.
 */
size_t qlora_workspace_bytes_multi(int64_t T, int64_t in_features, const int64_t* out_features,
                                   int n, int64_t r, int backward);
int qlora_linear_fwd_multi(const qlora_nf4_weight* W, int n, const qlora_bf16* X, int64_t T,
                           const qlora_bf16* const* A, const qlora_bf16* const* B, int64_t r,
                           float alpha, qlora_bf16* Y, void* ws, size_t ws_bytes,
                           qlora_stream stream);
int qlora_linear_bwd_multi(const qlora_nf4_weight* W, int n, const qlora_bf16* X,
                           const qlora_bf16* dY, int64_t T, const qlora_bf16* const* A,
                           const qlora_bf16* const* B, int64_t r, float alpha, qlora_bf16* dX,
                           float* const* dA, float* const* dB, void* ws, size_t ws_bytes,
                           qlora_stream stream);

/*
 * qlora_linear_bwd -- B1..B3 for the forward above, with s = alpha/r:
 *   dX = dY W_hat + s (dY B) A        [T, in]  bf16 (one rounding)
 *   dA = s (dY B)^T X                 [r, in]  fp32
 *   dB = s dY^T (X A^T)               [out, r] fp32
 * paperclase "QLoRA", Parte 4: dL/dx = (W_hat + (alpha/r) B A)^T dL/dh; no
 * gradient for W_hat (the codes are not parameters); A and B are the only
 * trained tensors.  dA and dB are overwritten, not accumulated.  From
 * T = 17 on (or with dropout) they are sums over token slices (a count fixed
 * by the shape) written to the workspace and added in a fixed order, and the
 * dX product takes one of two routes, chosen by ws_bytes:
 *   ws_bytes >= qlora_workspace_bytes(T, in, out, r, 1): W_hat^T is expanded
 *     into the workspace (2 * out * in bytes) and read by a bf16 GEMM (the
 *     faster route);
 *   qlora_workspace_bytes_bwd_min(...) <= ws_bytes < that: the GEMM reads
 *     the codes and dequantizes each weight tile, transposed, while staging
 *     it into on-chip memory, so W_hat^T is never stored and the workspace
 *     holds only the rank-r products (megabytes).
 * Both routes give the same dX, dA and dB bit for bit.  Up to T = 16 without
 * dropout the backward streams the codes once, W_hat existing only in LDS
 * tiles, sums fp32 row-split partials of dX in a fixed order (one rounding)
 * and writes each element of dA and dB once; both size functions give the
 * same size there.  Y, dX, dA and dB are reproducible bit for bit.
 *   dY [T, out] bf16; other arguments as in qlora_linear_fwd;
 *   ws of ws_bytes >= qlora_workspace_bytes_bwd_min(T, in, &out, 1, r, 0, flags)
 * T == 0 writes zeros to dA and dB and nothing else (X, dY, dX may be NULL).
 * Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, DEVICE, LAUNCH.
 */
int qlora_linear_bwd(const qlora_nf4_weight* W, const qlora_bf16* X, const qlora_bf16* dY,
                     int64_t T, const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                     qlora_stream stream);

/*
 * LoRA dropout (training).  coddykit "LoRA y QLoRA" configures the adapter
 * with lora_dropout = 0.05; reading taken here (as in the PEFT layer the page
 * configures): dropout acts on the adapter's input only,
 *   X~ = keep o X / (1 - p),   Y = X W_hat^T + s (X~ A^T) B^T,
 * and the backward of that forward:
 *   dX = dY W_hat + (keep / (1 - p)) o (s (dY B) A)   (one bf16 rounding)
 *   dA = s (dY B)^T X~,   dB = s dY^T (X~ A^T).
 * The mask is drawn by the caller and passed in (the library has no random
 * number generator): keep [T, in / 8] bytes, row-major, bit k % 8 of byte
 * keep[t * in/8 + k / 8] set = element (t, k) kept; any alignment.  The
 * forward and backward of one step must get the same mask.  0 <= p < 1
 * (p = 0 with every bit set equals the plain linear up to summation order).
 * Single projection only.  These calls always take the general (workspace)
 * path, also for T <= 16:
 *   ws of ws_bytes >= qlora_workspace_bytes_dropout(T, in, out, r, backward)
 * (0 for invalid shapes, at least 256 otherwise; host only).
 * T == 0: the forward does nothing, the backward writes zeros to dA and dB.
 * Errors: NULL (keep NULL with T > 0, or as the plain calls), VALUE (p not in
 * [0, 1) or alpha not finite), SHAPE, ALIGN, WORKSPACE, DEVICE, LAUNCH.
 */
size_t qlora_workspace_bytes_dropout(int64_t T, int64_t in_features, int64_t out_features, int64_t r,
                                     int backward);
int qlora_linear_fwd_dropout(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                             const uint8_t* keep, float p, const qlora_bf16* A, const qlora_bf16* B,
                             int64_t r, float alpha, qlora_bf16* Y, void* ws, size_t ws_bytes,
                             qlora_stream stream);
int qlora_linear_bwd_dropout(const qlora_nf4_weight* W, const qlora_bf16* X, const qlora_bf16* dY,
                             int64_t T, const uint8_t* keep, float p, const qlora_bf16* A,
                             const qlora_bf16* B, int64_t r, float alpha, qlora_bf16* dX, float* dA,
                             float* dB, void* ws, size_t ws_bytes, qlora_stream stream);

/*
 * Workspace bytes needed by qlora_merge: 0 for invalid shapes, at least 256
 * otherwise.  Host only.  Scratch only; needs no initialisation.
 */
size_t qlora_merge_workspace_bytes(int64_t in_features, int64_t out_features, int64_t r);

/*
 * qlora_merge -- folds the adapter into the frozen weight for serving:
 *   W_out = bf16(W_hat + (alpha/r) B A)          [out, in] bf16
 * (coddykit "LoRA y QLoRA": the adapter is merged into the base with
 * merge_and_unload; ultralytics glossary "QLoRA", "Compromissos": the 4-bit
 * base must be dequantized to 16 bits first).  Per element:
 * bf16_rne(fma(s, sum_j B[m][j] A[j][n], w_hat)) with w_hat exactly as
 * nf4_dequantize produces it, the rank-r sum accumulated in fp32 and added,
 * scaled, with one fp32 rounding; then one bf16 rounding.
 *   W      NF4 weight [out, in]; in % 64 == 0, out % 64 == 0
 *   A      [r, in] bf16;  B [out, r] bf16;  1 <= r <= 256;  alpha finite
 *   W_out  [out, in] bf16 out (row-major)
 *   ws     workspace of ws_bytes >= qlora_merge_workspace_bytes(in, out, r)
 *          (zero-padded copies of B and A^T; for r <= 64 with r % 8 == 0 the
 *          kernel reads A and B as they are and leaves ws untouched)
 * Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, DEVICE, LAUNCH.
 */
int qlora_merge(const qlora_nf4_weight* W, const qlora_bf16* A, const qlora_bf16* B, int64_t r,
                float alpha, qlora_bf16* W_out, void* ws, size_t ws_bytes, qlora_stream stream);

/* Host copy of the 16 fp32 levels the kernels use (ascending, L[7] = +0.0). */
void nf4_codebook(float out[16]);

/*
 * Host copy of the 15 fp32 code thresholds the quantize kernel uses:
 * code(x) = number of j with x > t[j], for x = fl32(w / a).  Exposed so the
 * threshold rule can be checked exhaustively against the argmin definition
 * on the CPU.
 */
void nf4_code_thresholds(float out[15]);

/*
 * Host copy of the bucket table the quantize kernel looks codes up in.  The
 * kernel works on X = fl32(16 w / a) = 16 x; for k = floor(X) in -16..16,
 * entry k + 16 holds base[k + 16], the number of scaled thresholds 16 t[j]
 * below k, and thr[k + 16], the one scaled threshold in [k, k + 1) (+inf if
 * none); code = base + (X > thr), which equals the rule above.  Exposed so
 * that equality can be checked exhaustively on the CPU.
 */
void nf4_code_buckets(float thr[33], uint32_t base[33]);

/* Static description of a status code. */
const char* qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
