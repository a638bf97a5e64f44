/*
 * qlora_nf4.h — C ABI of the MI355X (gfx950) NF4 + LoRA linear-layer library.
 *
 * The operations are those of QLoRA as described by
 *   [MC] "QLoRA: Efficient Finetuning of Quantized LLMs" (Michał Chromiak's blog),
 *   [TT] "QLoRA in LLMs" (TensorTonic),
 *   [GO] "QLoRA: the paper that put large-model fine-tuning on a desk" (Good Omens).
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or retains them.  Where an entry point needs temporary
 *    device memory the caller passes a workspace sized by qlora_workspace_size().
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work and returns without synchronizing; all of a call's work is
 *    ordered on `stream`.  Calls on different streams are safe when their
 *    buffers (workspaces included) are disjoint.
 *  - bf16 tensors are passed as uint16_t bit patterns (bfloat16: 1 sign, 8
 *    exponent, 7 fraction bits).  All matrices are row-major.
 *  - Pointers must be 16-byte aligned unless stated otherwise.
 *  - Errors: arguments are validated before anything is enqueued; on
 *    QLORA_ERR_INVALID_VALUE or QLORA_ERR_UNSUPPORTED nothing is launched and
 *    no output is touched.  A failed kernel launch returns QLORA_ERR_LAUNCH
 *    (kernels of the same call already enqueued before it still run).  The
 *    library takes each launch's status from the launch call itself: it never
 *    reads or clears the calling thread's HIP last-error state, so an error
 *    left there by the caller's own earlier work stays for the caller to see.
 *    No exception crosses the ABI.  Non-finite inputs give unspecified (but
 *    memory-safe) results.
 *  - Thread safety: the library holds no shared mutable state after its
 *    one-time initialisation of the NF4 tables (done under a lock on first
 *    use); the timing hook's events are per thread.
 */
#ifndef QLORA_NF4_H_
#define QLORA_NF4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_VALUE = 1, /* bad pointer, size, alignment, rank or workspace */
  QLORA_ERR_UNSUPPORTED = 2,   /* valid request outside what this build supports */
  QLORA_ERR_LAUNCH = 3,        /* the HIP runtime rejected a kernel launch */
  QLORA_ERR_INTERNAL = 4       /* the NF4 tables could not be built */
} qlora_status_t;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype_t;

/*
 * 4-bit codebooks.  A code is the index of its value in an ascending 16-entry
 * table (qlora_codebook_levels), chosen as the nearest value to
 * fp32(w / absmax), ties to the lower one.
 *  NF4   the NormalFloat values ([MC] "1. NormalFloat", [TT] §5), code 7 = 0.
 *  INT4  the symmetric absmax integer grid of [TT] §2 at 4 bits: q/7 for
 *        q = -8..7 at code q + 8 (q = -8 is never produced).
 *  FP4   the E2M1 values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and negatives, divided
 *        by 6, at codes 1..15 (code 0, -1.5, is never produced); the pages
 *        compare NF4 with FP4 ([MC] "What the experiments establish") but fix
 *        no FP4 layout, so this one is a reading.
 */
typedef enum { QLORA_CB_NF4 = 0, QLORA_CB_INT4 = 1, QLORA_CB_FP4 = 2 } qlora_codebook_t;

/* Workspace queries (qlora_workspace_size `op`). */
typedef enum {
  QLORA_OP_DOUBLE_QUANT = 0, /* a = number of block scales */
  QLORA_OP_LINEAR_FWD = 1,   /* a = M tokens, b = h, c = o */
  QLORA_OP_LINEAR_BWD = 2    /* a = M tokens, b = h, c = o */
} qlora_op_t;

#define QLORA_BLOCK 64      /* weights per first-level scale ([MC] "2. Double quantization") */
#define QLORA_CHUNK 256     /* first-level scales per second-level scale ([MC] "A worked memory budget") */
#define QLORA_MAX_RANK 128  /* largest LoRA rank r accepted */

/*
 * One frozen NF4 weight with double-quantized scales.  Logical shape h x o
 * (the pages' W: h inputs, o outputs, [MC] "The algebra").  Stored in
 * PyTorch's Linear.weight order [o][h]: row n holds output n's h weights, so
 * each 64-weight block runs along h.  Produced by qlora_quantize on the [o][h]
 * buffer followed by qlora_double_quant.  This struct is a host object (48
 * bytes on LP64: four pointers, then h at offset 32 and o at offset 40); the
 * pointers in it are device pointers.  Weights encoded with another codebook
 * (qlora_quantize_cb) use the same struct with the `_cb` entry points, which
 * take the codebook as an argument.
 */
typedef struct {
  const uint8_t *codes;   /* h*o/2 bytes: two 4-bit codes per byte, first in the high nibble */
  const int8_t *qabsmax;  /* h*o/64 int8 block scales (mean-centred) */
  const float *scale2;    /* ceil(h*o/64/256) float32 steps, one per 256 block scales */
  const float *mean;      /* 1 float32: the mean of the float32 block scales */
  int64_t h;              /* input width, a positive multiple of 64, at most 2^20 */
  int64_t o;              /* output width, a positive multiple of 64, at most 2^20 */
} qlora_nf4_weight_t;

/*
 * qlora_quantize — blockwise NF4 quantization ([MC] "1. NormalFloat";
 * [TT] §2 "Choose a scale, then round", §3, §5).
 *  w       n weights, float32 or bf16 (w_dtype), any 1-D buffer.
 *  codes   out, ceil(n/2) bytes: code of element 2k in the high nibble of byte k.
 *  absmax  out, ceil(n/64) float32: the largest magnitude of each 64-block.
 * Each weight is divided by its block's largest magnitude (IEEE float32
 * division) and mapped to the nearest of the 16 NF4 levels, ties to the lower
 * level.  A short last block is zero-padded; an odd n pads the last low nibble
 * with code 7 (the zero level); an all-zero block gets code 7 everywhere.
 * Alignment: w 16 bytes; codes and absmax 4 bytes.
 */
qlora_status_t qlora_quantize(const void *w, qlora_dtype_t w_dtype, int64_t n, uint8_t *codes,
                              float *absmax, void *stream);

/*
 * qlora_double_quant — quantization of the block scales ([MC] "2. Double
 * quantization"; [TT] §6; [GO] "Idea two").
 *  absmax   nblocks float32 block scales (from qlora_quantize), all >= 0.
 *  qabsmax  out, nblocks int8.
 *  scale2   out, ceil(nblocks/256) float32 steps.
 *  mean     out, 1 float32 (device).
 *  workspace/ws_bytes  device scratch of at least
 *           qlora_workspace_size(QLORA_OP_DOUBLE_QUANT, nblocks, ...) bytes;
 *           its contents on entry do not matter.
 * mean = the exact mean of all scales rounded once to float32 (independent of
 * summation order).  Each chunk j of 256 consecutive centred scales
 * c = fp32(a - mean) gets step s2_j = fp32(max|c| / 127) and codes
 * q = rint(fp32(c / s2_j)) in [-127, 127] ([TT] §2's symmetric int8 scheme;
 * step 0 gives codes 0).  Requires 1 <= nblocks < 2^32.
 * Alignment: absmax 16 bytes, workspace 256 bytes, qabsmax, scale2 and mean 4.
 */
qlora_status_t qlora_double_quant(const float *absmax, int64_t nblocks, int8_t *qabsmax, float *scale2,
                                  float *mean, void *workspace, size_t ws_bytes, void *stream);

/*
 * qlora_double_quant_noalloc — qlora_double_quant without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as qlora_double_quant minus workspace/ws_bytes; it
 * allocates nothing and calls no allocating routine.  Its partial sums live in
 * a 48 KB static array the library keeps on each GPU it runs on until the
 * process ends; every accepted size (1 <= nblocks < 2^32) fits in it, since the
 * partial-sum pass never uses more than 512 slots.  The first call on a device
 * looks the array's address up once (hipGetSymbolAddress).  `stream` must
 * belong to the current device (QLORA_ERR_INVALID_VALUE otherwise).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU (on
 * different streams) race and give wrong results; calls ordered on one stream
 * are safe.
 */
qlora_status_t qlora_double_quant_noalloc(const float *absmax, int64_t nblocks, int8_t *qabsmax, float *scale2,
                                          float *mean, void *stream);

/*
 * qlora_dequantize — rebuild n weights ([MC] "1. NormalFloat": codes are
 * dequantized to BF16 for computation; [GO] "The core move").
 *  a_hat = fp32(fp32(qabsmax * scale2) + mean)      (no fused multiply-add)
 *  w_hat = fp32(level[code] * a_hat)                 (out_dtype QLORA_F32)
 *        = bf16 round-to-nearest-even of that value  (out_dtype QLORA_BF16)
 *  out   n float32 or bf16 values.
 * Alignment: codes and out 16 bytes; scale2 and mean 4 bytes; qabsmax any.
 */
qlora_status_t qlora_dequantize(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                                const float *mean, int64_t n, void *out, qlora_dtype_t out_dtype,
                                void *stream);

/*
 * Codebook variants of the codec: the same storage, encoder and scales with
 * the levels of `codebook` (qlora_quantize / qlora_dequantize are the
 * QLORA_CB_NF4 cases).  Arguments, layouts and alignment as above.
 */
qlora_status_t qlora_quantize_cb(const void *w, qlora_dtype_t w_dtype, int64_t n, qlora_codebook_t codebook,
                                 uint8_t *codes, float *absmax, void *stream);
qlora_status_t qlora_dequantize_cb(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                                   const float *mean, int64_t n, qlora_codebook_t codebook, void *out,
                                   qlora_dtype_t out_dtype, void *stream);

/*
 * qlora_dequantize_nodq — reconstruction without double quantization: the
 * float32 block scales from quantization are used as stored,
 * w_hat = fp32(level[code] * absmax[block]) ([MC] "2. Double quantization"
 * is an addition on top of blockwise quantization).  absmax 4-byte aligned.
 */
qlora_status_t qlora_dequantize_nodq(const uint8_t *codes, const float *absmax, int64_t n,
                                     qlora_codebook_t codebook, void *out, qlora_dtype_t out_dtype,
                                     void *stream);

/* The 16 float32 values of a codebook, ascending (index = code). */
qlora_status_t qlora_codebook_levels(qlora_codebook_t codebook, float *levels);

/*
 * qlora_linear_fwd — Y = X·W_hat + s·(X·L1)·L2 ([MC] "The algebra", Eq. 3;
 * [TT] §3), with W_hat the bf16 dequantization of W computed on the fly.
 *  X   [M][h] bf16.     L1 [h][r] bf16.    L2 [r][o] bf16.
 *  Y   out [M][o] bf16.
 *  T   out [M][r] bf16 = X·L1 (float32 accumulation, rounded once), kept for
 *      the backward pass.
 *  r = 0 means no adapter: L1, L2 and T may be NULL.  1 <= M, 0 <= r <= 128.
 *  workspace: qlora_workspace_size(QLORA_OP_LINEAR_FWD, M, h, o, r) bytes.
 * Products accumulate in float32 on bf16 operands; outputs round once to bf16.
 */
qlora_status_t qlora_linear_fwd(const qlora_nf4_weight_t *W, const uint16_t *X, int64_t M,
                                const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                                uint16_t *Y, uint16_t *T, void *workspace, size_t ws_bytes,
                                void *stream);

/*
 * qlora_linear_bwd — gradients through the frozen dequantized weight into the
 * adapters ([MC] Figure 1 and "One training step"; [TT] §4; [GO] "The core
 * move": no gradient ever updates the 4-bit weights, so there is no dW).
 *  With U = dY·L2^T:
 *   dX  = dY·W_hat^T + s·U·L1^T   out [M][h] bf16
 *   dL1 = s·X^T·U                 out [h][r] float32
 *   dL2 = s·T^T·dY                out [r][o] float32
 *  T is the forward's saved [M][r] bf16 product X·L1.  r = 0: only dX is
 *  computed and X, T, L1, L2, dL1, dL2 may be NULL.
 *  workspace: qlora_workspace_size(QLORA_OP_LINEAR_BWD, M, h, o, r) bytes.
 *  The token sum behind dL1 and dL2 is split into chunks whose operand rows
 *  stay below 2^31 bytes each; a shape that would need more than 65535 such
 *  chunks (only for M in the hundreds of millions on the widest layers)
 *  returns QLORA_ERR_UNSUPPORTED.
 */
qlora_status_t qlora_linear_bwd(const qlora_nf4_weight_t *W, const uint16_t *X, const uint16_t *T,
                                const uint16_t *dY, int64_t M, const uint16_t *L1, const uint16_t *L2,
                                int32_t r, float s, uint16_t *dX, float *dL1, float *dL2,
                                void *workspace, size_t ws_bytes, void *stream);

/*
 * The linear layer on a weight encoded with another codebook
 * (qlora_quantize_cb): arguments, layouts and errors as qlora_linear_fwd and
 * qlora_linear_bwd, the codes decoded with the levels of `codebook`
 * (qlora_linear_fwd / qlora_linear_bwd are the QLORA_CB_NF4 cases).
 */
qlora_status_t qlora_linear_fwd_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *X,
                                   int64_t M, const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                                   uint16_t *Y, uint16_t *T, void *workspace, size_t ws_bytes, void *stream);
qlora_status_t qlora_linear_bwd_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *X,
                                   const uint16_t *T, const uint16_t *dY, int64_t M, const uint16_t *L1,
                                   const uint16_t *L2, int32_t r, float s, uint16_t *dX, float *dL1, float *dL2,
                                   void *workspace, size_t ws_bytes, void *stream);

/*
 * qlora_merge_adapter — merge a trained adapter into the frozen base
 * ([TT] §11 "Saving, Loading, and Merging QLoRA Adapters": dequantize the base
 * to a wider precision and add the LoRA update; [GO] "What it added up to").
 *  W' = W_hat + s·L1·L2 in W's [o][h] storage: entry (n, k) =
 *       fp32(w_hat + fp32(s * P)),  P = sum_q L1[k][q] * L2[q][n]
 *  where w_hat is qlora_dequantize's float32 value and P comes from bf16
 *  products with float32 accumulation (summation order unspecified).
 *  L1 [h][r] bf16, L2 [r][o] bf16, 16-byte aligned (may be NULL when r = 0),
 *       0 <= r <= 128.
 *  out  [o][h] float32 or bf16 (round to nearest even of the float32 value);
 *       16-byte aligned.
 */
qlora_status_t qlora_merge_adapter(const qlora_nf4_weight_t *W, const uint16_t *L1, const uint16_t *L2,
                                   int32_t r, float s, void *out, qlora_dtype_t out_dtype, void *stream);

/*
 * qlora_merge_requantize — the merge followed by NF4 re-quantization in one
 * pass ([TT] §11: merging and quantizing again adds a second quantization
 * error).  codes_out (h*o/2 bytes) and absmax_out (h*o/64 float32) are what
 * qlora_quantize returns for the float32 merged weight qlora_merge_adapter
 * computes; follow with qlora_double_quant(absmax_out, ...) to obtain the new
 * weight's int8 scales.  codes_out 8-byte and absmax_out 4-byte aligned; they must not
 * alias W's buffers.
 */
qlora_status_t qlora_merge_requantize(const qlora_nf4_weight_t *W, const uint16_t *L1, const uint16_t *L2,
                                      int32_t r, float s, uint8_t *codes_out, float *absmax_out, void *stream);

/*
 * The merge and the merge with re-quantization for a weight encoded with
 * another codebook: W_hat uses the levels of `codebook` and the re-encoding
 * uses the same codebook.  Otherwise as qlora_merge_adapter and
 * qlora_merge_requantize (the QLORA_CB_NF4 cases).
 */
qlora_status_t qlora_merge_adapter_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *L1,
                                      const uint16_t *L2, int32_t r, float s, void *out, qlora_dtype_t out_dtype,
                                      void *stream);
qlora_status_t qlora_merge_requantize_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *L1,
                                         const uint16_t *L2, int32_t r, float s, uint8_t *codes_out,
                                         float *absmax_out, void *stream);

/*
 * qlora_adamw_step — one optimizer step on adapter parameters ([TT] §4 "One
 * QLoRA Training Step, End to End": only the adapters are updated; the update
 * itself is not written out on the pages, so this is AdamW with decoupled
 * weight decay, Loshchilov and Hutter).  Elementwise over n float32 values:
 *   p <- p * (1 - lr*wd)
 *   m <- beta1*m + (1 - beta1)*g          v <- beta2*v + (1 - beta2)*g*g
 *   p <- p - lr/(1 - beta1^t) * m / (sqrt(v)/sqrt(1 - beta2^t) + eps)
 *  param      float32 master values, updated in place (e.g. L1 then L2, flat)
 *  grad       float32 gradients (qlora_linear_bwd's dL1 / dL2)
 *  exp_avg, exp_avg_sq   float32 first / second moments, updated in place;
 *             start at 0 before step 1.  Like param and grad they may live in
 *             device memory or in pinned host memory allocated with
 *             hipHostMalloc (optimizer state kept in CPU RAM, [TT] §7 "Paged
 *             Optimizers"; the kernel then reads and writes it over the link).
 *  step       t, 1-based.   0 <= beta1, beta2 < 1;  eps > 0;  lr, wd >= 0.
 *  param_bf16 optional (may be NULL): receives bf16(p) (round to nearest even),
 *             the copy the linear layer consumes.
 *  param, grad, exp_avg, exp_avg_sq 16-byte aligned, param_bf16 8-byte aligned;
 *  no two of the arrays may overlap.
 */
qlora_status_t qlora_adamw_step(float *param, const float *grad, float *exp_avg, float *exp_avg_sq, int64_t n,
                                int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                                uint16_t *param_bf16, void *stream);

/*
 * Block glue: the elementwise steps between the NF4 linears of a transformer
 * block.  [MC] "A closer look: Design choices and memory costs" puts adapters
 * on every linear of the block, attention and feed-forward; the feed-forward of
 * the LLaMA models the pages name is gated, its gate and up projections G and
 * U meeting in H = SiLU(G) * U with SiLU(g) = g / (1 + exp(-g)) before the down
 * projection.  All tensors are n bf16 values in any matching shape, 16-byte
 * aligned; arithmetic is float32, each output rounded once to nearest even.
 * Outputs must not overlap the inputs (qlora_grad_sum excepted, see there).
 *
 * qlora_silu_gate_fwd  H = SiLU(G) * U.
 * qlora_silu_gate_bwd  for the upstream gradient dH:
 *                        dU = dH * SiLU(G)
 *                        dG = dH * U * sigmoid(G) * (1 + G * (1 - sigmoid(G)))
 *                      dG and dU must be different buffers.
 * qlora_grad_sum       out = parts[0] + ... + parts[k-1], summed in that order:
 *                      the gradient of an input that several linears read (the
 *                      block input feeds q, k, v, gate and up).  `parts` is a
 *                      HOST array of k device pointers, 1 <= k <= 8; `out` may
 *                      be one of them (exactly, not a partial overlap).
 */
qlora_status_t qlora_silu_gate_fwd(const uint16_t *G, const uint16_t *U, int64_t n, uint16_t *H, void *stream);
qlora_status_t qlora_silu_gate_bwd(const uint16_t *G, const uint16_t *U, const uint16_t *dH, int64_t n, uint16_t *dG,
                                   uint16_t *dU, void *stream);
qlora_status_t qlora_grad_sum(const uint16_t *const *parts, int32_t k, int64_t n, uint16_t *out, void *stream);

/* Workspace bytes an entry point needs (always a multiple of 256; may be 0). */
qlora_status_t qlora_workspace_size(qlora_op_t op, int64_t a, int64_t b, int64_t c, int32_t r,
                                    size_t *bytes);

/*
 * Timing hook for benchmarks and profilers.  `kernel` 0 = the forward fused
 * dequant-GEMM, 1 = the dX kernel of qlora_linear_bwd (the fused dequant-GEMM,
 * or for M <= 16 the few-token dX kernel), 2 = the few-token forward
 * (M <= 16).  When `start`/`stop` (hipEvent_t handles) are non-NULL, every
 * later launch of that kernel by the calling thread records `start` just
 * before and `stop` just after itself on the call's stream.  NULL/NULL turns
 * the hook off.  Per thread; the library only records, never synchronizes.
 * Events created with hipEventDisableSystemFence disturb the timed stream
 * least (a default event's system-scope fence stalls it for microseconds).
 */
qlora_status_t qlora_set_timing_events(int32_t kernel, void *start, void *stop);

/*
 * Stream probe, a measurement helper rather than a step of the method: the
 * plain HBM streaming rate for the byte mix of a bandwidth-bound kernel, the
 * ceiling its own rate is compared with.  Moves `n_tiles` tiles; tile t reads
 * the 1024 * rd contiguous bytes of `src` at byte 1024 * rd * t and writes the
 * 1024 * wr contiguous bytes of `dst` at byte 1024 * wr * t, with fully
 * coalesced 16-byte accesses.  Launch shape: `blocks` workgroups of 256
 * threads (0: min(ceil(n_tiles / 8), 8192); at most 2^20), each wave taking
 * `depth` tiles (1, 2, 4 or 8) per pass with all their loads issued first; a
 * caller takes the best rate over a sweep of shapes as the ceiling.
 *   (rd, wr) = (1, 0)  read only (the few-token forward's weight stream);
 *              (4, 1)  four bytes read per byte written (quantization of bf16
 *                      weights reads 2 and writes 0.52 bytes per weight);
 *              (1, 4)  the reverse (dequantization to bf16).
 *  src: n_tiles * 1024 * rd bytes; dst: n_tiles * 1024 * wr bytes, or 16 bytes
 *  when wr = 0 (it may receive one store).  Both 16-byte aligned.  The values
 *  written are a function of those read and otherwise unspecified.
 *  QLORA_ERR_INVALID_VALUE for any other (rd, wr) or depth, blocks out of
 *  range, NULL or misaligned pointers, or n_tiles < 1.
 */
qlora_status_t qlora_stream_probe(int32_t rd, int32_t wr, int32_t depth, int32_t blocks, const void *src, void *dst,
                                  int64_t n_tiles, void *stream);

/* Static description of a status code (never NULL). */
const char *qlora_status_string(qlora_status_t status);

/* Host copy of the 16 float32 NF4 levels the kernels use, ascending
 * (code 0 = -1, code 7 = 0, code 15 = +1).  Returns QLORA_ERR_INTERNAL if the
 * tables could not be built. */
qlora_status_t qlora_nf4_levels(float out[16]);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H_ */
