/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) library for the frozen-NF4
 * linear layer with a LoRA adapter.
 *
 * The method (sources named by page title and section):
 *   - "QLoRA — 650億パラメータのモデルをGPU 1枚で微調整する" (ta-paperlens),
 *     sections 量子化を1段落で, NF4, 二重量子化, 勾配は実際どこへ行くのか;
 *   - LLM book chapter 26 "LoRA/QLoRA" (waylandz), 26.2.1-26.2.4, 26.6.3;
 *   - Ultralytics glossary "QLoRA", "So funktioniert QLoRA" and its code example.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer (memory of the current HIP device)
 *     unless a comment says "host".  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream); every call only enqueues work on it and
 *     returns without synchronising.
 *   - The caller allocates and owns all memory, including workspaces.  The
 *     library never allocates, frees or keeps a pointer after returning.
 *   - 16-bit tensors are passed as uint16_t bit patterns, row-major.  They
 *     are bf16 unless the weight they go with has compute_dtype
 *     QLORA_COMPUTE_FP16, in which case every "bf16" below reads "fp16"
 *     (IEEE binary16) and every rounding to it is to nearest even.
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-OK status nothing has been enqueued.  Errors of already enqueued
 *     kernels surface at the caller's next synchronisation.
 *   - Inputs must be finite (NaN/Inf are outside the contract).
 *   - Calls keep no state between them (apart from the per-thread timing
 *     events of qlora_set_timing_events) and may be made from several host
 *     threads.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_NF4_FORMAT_VERSION 1
#define QLORA_NF4_BLOCKSIZE 64       /* weights per absmax block               */
#define QLORA_NF4_DQ_BLOCKSIZE 256   /* block constants per second-level scale */
#define QLORA_NF4_DQ_OFF 0           /* dq_blocksize of a weight without double quantisation */
#define QLORA_MAX_RANK 128

/* quant_type: the 4-bit codebook */
#define QLORA_QUANT_NF4 0            /* normal-quantile levels with an exact 0 */
#define QLORA_QUANT_INT4 1           /* evenly spaced levels -1 + 2i/15        */
/* compute_dtype: the 16-bit type of activations, adapters and dequantised weights */
#define QLORA_COMPUTE_BF16 0
#define QLORA_COMPUTE_FP16 1

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,       /* a required pointer is NULL                       */
  QLORA_ERR_SHAPE = 2,      /* a size is out of range (see each entry point)    */
  QLORA_ERR_ALIGN = 3,      /* a device pointer is not 16-byte aligned          */
  QLORA_ERR_WORKSPACE = 4,  /* workspace smaller than the matching *_workspace() */
  QLORA_ERR_DEVICE = 5,     /* the current device is not a gfx950 GPU           */
  QLORA_ERR_HIP = 6,        /* a HIP runtime call failed; see qlora_last_hip_error */
  QLORA_ERR_FORMAT = 7,     /* weight descriptor has a wrong version/blocksize,
                               an unknown variant, or a variant the call does not take */
  QLORA_ERR_SCRATCH = 8     /* qlora_linear_fwd_noalloc: the call needs more workspace
                               than its fixed device array holds */
} qlora_status;

/*
 * Packed NF4 weight with double-quantised block constants (host struct that
 * holds device pointers; caller-owned).  The layout below is the default
 * format (quant_type NF4, double quantisation on, compute dtype bf16); the
 * variants follow it.
 *
 * W is [rows = out_features, cols = in_features] row-major, rows % 16 == 0,
 * cols % 64 == 0.
 * Block b covers elements [64 b, 64 b + 64) of the row-major flattening, so a
 * block never crosses a row.  n = rows * cols, n_b = n / 64,
 * n_g = ceil(n_b / 256).
 *   codes         [n / 2]  NF4 codes, element 2i in the low nibble of byte i
 *                          (ta-paperlens NF4 section; waylandz 26.6.3: half a
 *                          byte per weight).
 *   absmax_code   [n_b]    OCP FP8 E4M3 bit pattern of the centred, group-scaled
 *                          block constant (ta-paperlens 二重量子化).
 *   absmax_scale  [n_g]    float32 s2_g: largest |c_b - mu| in group g.
 *   absmax_offset [1]      float32 mu: mean of all block constants.
 * Decoded block constant: c'_b = RN32(RN32(e4m3(code_b) * 2^-8 * s2_g) + mu);
 * dequantised weight: bf16_RNE(RN32(q[code] * c'_b)).
 * Storage: n/2 + n_b + 4 n_g + 4 bytes = 4 + 8/64 + 32/16384 bits per weight
 * plus 32 bits per tensor (ta-paperlens 二重量子化: about 4.127 bits).
 *
 * Variants (the config knobs bnb_4bit_use_double_quant and
 * bnb_4bit_compute_dtype of ta-paperlens コードで見る, and the comparison
 * codebook of the Ultralytics code example):
 *   dq_blocksize QLORA_NF4_DQ_OFF: no double quantisation; absmax_scale holds
 *     the n_b float32 block constants c_b themselves and absmax_code,
 *     absmax_offset are unused (may be NULL): 4 + 32/64 = 4.5 bits per weight
 *     (ta-paperlens 二重量子化).
 *   quant_type QLORA_QUANT_INT4: levels -1 + 2i/15 rounded to float32 (no
 *     exact 0; a zero quotient takes level 7); quantise, dequantise and
 *     merge only -- the linear entry points return QLORA_ERR_FORMAT.
 *   compute_dtype QLORA_COMPUTE_FP16: every 16-bit tensor of the calls that
 *     take this weight (dequantised or merged weight, X, A, B, Y, U, dY, dX)
 *     is IEEE binary16; roundings are to nearest even (ta-paperlens 落とし穴:
 *     FP16 where the GPU has no BF16; waylandz 26.6.4 uses float16).
 */
typedef struct {
  int32_t format_version;   /* QLORA_NF4_FORMAT_VERSION */
  int32_t blocksize;        /* QLORA_NF4_BLOCKSIZE      */
  int32_t dq_blocksize;     /* QLORA_NF4_DQ_BLOCKSIZE, or QLORA_NF4_DQ_OFF */
  int16_t quant_type;       /* QLORA_QUANT_NF4 (0) or QLORA_QUANT_INT4 */
  int16_t compute_dtype;    /* QLORA_COMPUTE_BF16 (0) or QLORA_COMPUTE_FP16 */
  int64_t rows;
  int64_t cols;
  uint8_t *codes;
  uint8_t *absmax_code;
  float *absmax_scale;
  float *absmax_offset;
} qlora_nf4_weight;

/* Fill a descriptor's header fields for a [rows, cols] weight in the default
 * format (host call; pointers are left untouched).  Returns QLORA_ERR_SHAPE
 * unless rows >= 16, rows % 16 == 0, cols >= 64, cols % 64 == 0 and
 * rows * cols < 2^44; QLORA_ERR_NULL if w is NULL. */
qlora_status qlora_nf4_weight_init(qlora_nf4_weight *w, int64_t rows, int64_t cols);

/* The same for a variant: quant_type QLORA_QUANT_*, double_quant 0 or 1,
 * compute_dtype QLORA_COMPUTE_*.  QLORA_ERR_FORMAT for an unknown value. */
qlora_status qlora_nf4_weight_init_ex(qlora_nf4_weight *w, int64_t rows, int64_t cols,
                                      int quant_type, int double_quant, int compute_dtype);

/* Byte sizes of the four device buffers of the weight a descriptor describes
 * (any format; 0 for a buffer the format does not use).  Any output pointer
 * may be NULL.  Errors as check of the descriptor's header fields. */
qlora_status qlora_nf4_weight_buffer_sizes(const qlora_nf4_weight *w, size_t *codes_bytes,
                                           size_t *absmax_code_bytes,
                                           size_t *absmax_scale_bytes,
                                           size_t *absmax_offset_bytes);

/* Byte sizes of the four device buffers of a [rows, cols] weight (host call).
 * Any output pointer may be NULL.  Returns QLORA_ERR_SHAPE on a bad shape. */
qlora_status qlora_nf4_buffer_sizes(int64_t rows, int64_t cols, size_t *codes_bytes,
                                    size_t *absmax_code_bytes, size_t *absmax_scale_bytes,
                                    size_t *absmax_offset_bytes);

/* Workspace bytes qlora_nf4_quantize needs: the float32 block constants and
 * one float64 partial sum per group (0 on a bad shape).  A weight without
 * double quantisation needs none (ws may then be NULL). */
size_t qlora_nf4_quantize_workspace(int64_t rows, int64_t cols);

/*
 * Blockwise NF4 quantisation plus double quantisation of a float32 weight.
 * (ta-paperlens 量子化を1段落で, NF4, 二重量子化; Ultralytics code example.)
 *   W    [rows, cols] float32, read only.
 *   out  host descriptor initialised by qlora_nf4_weight_init for the same
 *        shape; its four device buffers are written.
 *   ws   device workspace of at least qlora_nf4_quantize_workspace() bytes.
 * Per block: c = max |w|; code = nearest NF4 level to RN32(w / c), ties to the
 * lower index; an all-zero block gets the zero level.  Then mu = mean of all
 * c (fixed pairwise float64 tree), d = RN32(c - mu), s2 = max |d| per group of
 * 256 blocks, code8 = E4M3 round-to-nearest-even of RN32(d / s2) * 256
 * (0x00 when s2 == 0).  Without double quantisation c itself is stored.
 * With quant_type INT4 the levels are the evenly spaced ones.
 */
qlora_status qlora_nf4_quantize(const float *W, const qlora_nf4_weight *out, void *ws,
                                size_t ws_bytes, void *stream);

/*
 * Dequantise a packed weight to bf16 [rows, cols] (W_bf16 written; fp16 for
 * a weight whose compute_dtype is QLORA_COMPUTE_FP16): round16(RN32(q[code] *
 * c)) with c the decoded or, without double quantisation, the stored
 * constant.
 * (ta-paperlens 量子化を1段落で: restore by lookup and multiply; the bf16
 * values are bit-identical to those the fused linear kernels use.)
 */
qlora_status qlora_nf4_dequantize(const qlora_nf4_weight *w, uint16_t *W_bf16, void *stream);

/*
 * Fold the adapter into the dequantised base (the deployment step):
 *   W_merged = bf16( w_hat + s * (B A) ),  s = alpha / r,
 * with w_hat the bf16 weight qlora_nf4_dequantize gives, B A accumulated in
 * float32, s * (B A) rounded to float32, added to w_hat in float32 and the
 * sum rounded once to bf16 (round to nearest, ties to even).
 * (waylandz LLM book 26.2: merge once, W + (alpha/r) B A, then inference has
 * no adapter cost; ta-paperlens 落とし穴 and Ultralytics QLoRA, Kompromisse:
 * the merge is done on the base dequantised to 16 bit; quantising the merged
 * weight again is qlora_nf4_quantize of its float32 values.)
 *   w         packed weight, read only (never written).
 *   A         [r, cols] bf16, B [rows, r] bf16, read only, 16-byte aligned.
 *   r         16 .. 128, a multiple of 16; alpha finite.
 *   W_merged  [rows, cols] bf16, written, 16-byte aligned.
 * No workspace.  Errors: QLORA_ERR_NULL, QLORA_ERR_ALIGN, QLORA_ERR_SHAPE
 * (bad descriptor, rank or alpha), QLORA_ERR_DEVICE, QLORA_ERR_HIP.
 */
qlora_status qlora_nf4_merge(const qlora_nf4_weight *w, const uint16_t *A, const uint16_t *B,
                             int32_t r, float alpha, uint16_t *W_merged, void *stream);

/*
 * One AdamW step on n adapter parameters (A and B of a linear, in one or
 * several calls), float32 master parameters and moments:
 *   p1 = p * (1 - lr wd);  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   p  = p1 - lr / (1 - b1^step) * m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * (ta-paperlens ページ化オプティマイザ and waylandz 26.6.4: Adam's two moments
 * per trainable parameter in 32 bit, only for A and B; Adam with decoupled
 * weight decay, bias-corrected, in the form PyTorch's AdamW documents.)
 * The constants are computed on the host in float64 (b^step by binary
 * exponentiation) and rounded once to float32; each element operation is
 * one float32 rounding in the order above, no fused multiply-add.
 *   param, exp_avg, exp_avg_sq  [n] float32, read and written in place.
 *   grad        [n] float32 (dA or dB of qlora_linear_bwd), read only.
 *   param_bf16  [n] bf16 copy for the next forward (bf16_RNE of the new
 *               param), written; may be NULL.
 *   step        1-based step count; hyperparameters as in PyTorch's AdamW.
 * All pointers 16-byte aligned.  Errors: QLORA_ERR_NULL, QLORA_ERR_ALIGN,
 * QLORA_ERR_SHAPE (n < 1, step < 1, lr < 0, eps <= 0, weight_decay < 0, a
 * beta outside [0, 1), any non-finite value), QLORA_ERR_DEVICE, QLORA_ERR_HIP.
 * (The pages' paging of these states to host memory is not done: the states
 * of a 65B model's adapters fit in HBM many times over.)
 */
qlora_status qlora_adamw_step(float *param, float *exp_avg, float *exp_avg_sq,
                              const float *grad, uint16_t *param_bf16, int64_t n, int64_t step,
                              double lr, double beta1, double beta2, double eps,
                              double weight_decay, void *stream);

/* The same step with the 16-bit copy in the compute dtype of the weights the
 * adapters serve: compute_dtype QLORA_COMPUTE_BF16 (as qlora_adamw_step) or
 * QLORA_COMPUTE_FP16 (param16 then receives binary16, nearest even;
 * ta-paperlens 落とし穴).  QLORA_ERR_FORMAT for another compute_dtype. */
qlora_status qlora_adamw_step16(float *param, float *exp_avg, float *exp_avg_sq,
                                const float *grad, uint16_t *param16, int compute_dtype,
                                int64_t n, int64_t step, double lr, double beta1, double beta2,
                                double eps, double weight_decay, void *stream);

/* Workspace bytes for qlora_linear_fwd (is_bwd = 0) or qlora_linear_bwd
 * (is_bwd = 1) at T tokens, a [rows, cols] weight and rank r (0 on bad args;
 * also 0 for T = 0, which needs no workspace).  The size depends on the
 * once-per-call dequantisation policy below, read at the time of the query. */
size_t qlora_linear_workspace(int64_t T, int64_t rows, int64_t cols, int32_t r, int is_bwd);

/*
 * Once-per-call dequantisation policy of the linear layer (process-wide).
 * Every matmul dequantises the blocks it needs to 16 bit (ta-paperlens
 * 勾配は実際どこへ行くのか; Ultralytics "So funktioniert QLoRA": dequantise
 * right before the matmul): for T >= min_tokens (default 2048) the forward
 * and the backward of qlora_linear_* dequantise the whole weight once per
 * call into their workspace (2 bytes a weight) and the GEMM streams that
 * copy; below it (and always in qlora_linear_fwd_noalloc) the GEMM decodes
 * each weight tile into LDS for every tile of 256 tokens.  Both give the
 * same bits.  qlora_set_pre_dequant_min_tokens returns the previous value,
 * or -1 (and changes nothing) for min_tokens < 0; INT64_MAX turns the
 * once-per-call pass off.  Workspace sizes follow the policy at the time of
 * the query: a call whose policy changed since leaves QLORA_ERR_WORKSPACE
 * if its workspace became too small.  The value is one atomic word: a change
 * made while other threads size or make calls is safe, each of them sees the
 * old or the new value.
 */
int64_t qlora_set_pre_dequant_min_tokens(int64_t min_tokens);
int64_t qlora_pre_dequant_min_tokens(void);

/*
 * Forward of the frozen-NF4 linear layer with a LoRA adapter:
 *   Y = X dequant(W)^T + (alpha / r) (X A^T) B^T
 * (ta-paperlens 勾配は実際どこへ行くのか: h = dequant(W_NF4) x + B A x with bf16
 * compute; waylandz 26.2.4: the adapter term is scaled by alpha / r).
 *   X      [T, cols] bf16        A [r, cols] bf16        B [rows, r] bf16
 *   Y      [T, rows] bf16 (written)
 *   U_save [T, r] bf16 (written; X A^T for the backward) or NULL
 * T >= 0, r % 16 == 0, 16 <= r <= 128; T * rows and T * cols below 2^30,
 * rows * cols below 2^32, rows and cols at most 2^22 (QLORA_ERR_SHAPE
 * otherwise).  T = 0 (an empty batch) writes nothing; X, Y, U_save and ws
 * may then be NULL.  Accumulation is float32 on bf16 MFMA; the packed weight is
 * only read.  For T <= 64 (generation-sized batches, ta-paperlens 落とし穴)
 * the call takes the skinny path, which streams the packed weight once and
 * forms X A^T in the same pass.  From T = qlora_pre_dequant_min_tokens()
 * on (2048 by default) it dequantises the weight once into the workspace (2
 * bytes a weight, fewer than 2^30 weights and at most 2^20 columns) and the
 * GEMM fetches that copy; in between the GEMM decodes the packed weight tile
 * by tile.  Both give the same bits; the workspace size reflects the path.
 */
qlora_status qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t T,
                              const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                              uint16_t *Y, uint16_t *U_save, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * qlora_linear_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (bit for bit) and errors as qlora_linear_fwd,
 * without a workspace argument: the workspace is a fixed array of
 * qlora_linear_fwd_noalloc_max_scratch() bytes (32 MiB) that the library
 * holds in device memory on every GPU it runs on, until the process ends.
 * The call allocates and frees nothing.  Its GEMM always decodes the packed
 * weight tile by tile (no 16-bit copy of the weight), and it drops the
 * K-split of the GEMM's last tiles when that split's partials would not fit.
 * QLORA_ERR_SCRATCH (before any device work) when even that workspace exceeds
 * the array.  All calls on one GPU share its array: calls that overlap on one GPU
 * (on two streams at once) race; calls ordered on one stream do not.  The
 * first call on a device resolves the array's address (hipGetSymbolAddress),
 * which a caller under graph capture should do once before capturing.
 */
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t T,
                                      const uint16_t *A, const uint16_t *B, int32_t r,
                                      float alpha, uint16_t *Y, uint16_t *U_save, void *stream);
size_t qlora_linear_fwd_noalloc_max_scratch(void);

/*
 * Backward of the same layer for an upstream gradient dY; there is no
 * gradient for W (ta-paperlens 勾配は実際どこへ行くのか: the input gradient
 * passes through dequant(W)^T, only A and B are trained, W is never written).
 *   G  = dY B
 *   dX = dY dequant(W) + s G A              [T, cols] bf16 (written)
 *   dA = s G^T X                            [r, cols] float32 (written)
 *   dB = s dY^T U                           [rows, r] float32 (written)
 * with s = alpha / r and U = X A^T: U_saved (the forward's U_save) when not
 * NULL, else recomputed.  Same shape rules as the forward; for T = 0 dA and
 * dB are set to 0 (sums over no tokens) and X, dY, U_saved, dX and ws may
 * be NULL.  As in the forward, from T = qlora_pre_dequant_min_tokens() on
 * the weight is dequantised once into the workspace for the dX GEMM.
 */
qlora_status qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY,
                              int64_t T, const uint16_t *A, const uint16_t *B, int32_t r,
                              float alpha, const uint16_t *U_saved, uint16_t *dX, float *dA,
                              float *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * lora_dropout: dropout on the adapter's input (ta-paperlens コードで見る and
 * 現場ではこう使う, waylandz 26.4.2 / 26.5.1 / 26.6.4: LoraConfig sets
 * lora_dropout, 0.05 in every example).  The frozen path sees X unchanged;
 * the adapter sees D(X) = keep * X / (1 - p).
 *
 * Keep decisions come from Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC11): element (t, k) of
 * X [T, cols] is kept iff word (t mod 4) of the generator at counter
 * (k, t / 4, offset low 32 bits, offset high 32 bits) with key (seed low 32
 * bits, seed high 32 bits) is at least floor(p * 2^32).  A call with the
 * same seed and offset reproduces the mask; use a distinct offset per layer
 * and step.
 *
 * Packed mask ("keep", qlora_dropout_mask_bytes(T, cols) bytes): the bit of
 * element (t, k) is bit (t mod 4) of the low nibble (k even) or high nibble
 * (k odd) of byte (t / 4) * (cols / 2) + k / 2; bits of tokens past T are 0.
 */
typedef struct {
  double p;          /* drop probability, 0 <= p < 1                          */
  uint64_t seed;     /* generator key                                         */
  uint64_t offset;   /* generator counter words 2 and 3                       */
} qlora_dropout;

/* Bytes of the packed keep mask of T tokens x cols features (0 on bad args,
 * and for T = 0). */
size_t qlora_dropout_mask_bytes(int64_t T, int64_t cols);

/*
 * Draw the keep mask of X [T, cols] into `keep` (written, 4-byte aligned)
 * and, when X is given, the dropped input X_dropped [T, cols] bf16 (x where
 * kept, +0 elsewhere; the 1 / (1 - p) scale is not applied).  X and
 * X_dropped are both NULL or both set (16-byte aligned).  cols % 64 == 0,
 * T >= 0, T * cols below 2^30; T = 0 does nothing (any pointers).  Errors: QLORA_ERR_NULL, QLORA_ERR_ALIGN,
 * QLORA_ERR_SHAPE (sizes, or p outside [0, 1)), QLORA_ERR_DEVICE,
 * QLORA_ERR_HIP.
 */
qlora_status qlora_dropout_mask(const qlora_dropout *d, int64_t T, int64_t cols,
                                const uint16_t *X, uint16_t *X_dropped, uint8_t *keep,
                                void *stream);

/* Workspace bytes for qlora_linear_fwd_dropout (is_bwd = 0) or
 * qlora_linear_bwd_dropout (is_bwd = 1) (0 on bad args, and for T = 0). */
size_t qlora_linear_workspace_dropout(int64_t T, int64_t rows, int64_t cols, int32_t r,
                                      int is_bwd);

/*
 * Forward with lora_dropout:
 *   Y = X dequant(W)^T + s (D(X) A^T) B^T,   s = alpha / r.
 *   U_save     [T, r] bf16, D(X) A^T (what dB needs), written, or NULL.
 *   keep_save  the packed keep mask, written (16-byte aligned), or NULL (then it lives in the
 *              workspace only); pass it to the backward to skip the redraw.
 *   X_dropped_save  [T, cols] 16-bit, written with the dropped input (x where
 *              kept, +0 elsewhere; 1 / (1 - p) not applied; 16-byte aligned), or
 *              NULL.  Passing it to the backward spares the backward the pass
 *              that re-forms it from X and the mask (T * cols * 2 bytes kept per
 *              layer, as autograd keeps a dropout's output).
 * Every token count takes the general path (the skinny path of
 * qlora_linear_fwd serves inference, which has no dropout).  p = 0 gives
 * the same bits as qlora_linear_fwd's general path.  Other arguments,
 * shape rules and errors as qlora_linear_fwd, plus QLORA_ERR_NULL for a NULL
 * d and QLORA_ERR_SHAPE for p outside [0, 1).
 */
qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight *w, const uint16_t *X, int64_t T,
                                      const uint16_t *A, const uint16_t *B, int32_t r,
                                      float alpha, const qlora_dropout *d, uint16_t *Y,
                                      uint16_t *U_save, uint8_t *keep_save,
                                      uint16_t *X_dropped_save, void *ws, size_t ws_bytes,
                                      void *stream);

/*
 * Backward with lora_dropout (no dW):
 *   G  = dY B
 *   dX = dY dequant(W) + keep * (s G A) / (1 - p)
 *   dA = s G^T D(X)
 *   dB = s dY^T U,   U = D(X) A^T: U_saved if not NULL, else recomputed.
 * keep_saved: the forward's keep_save (read), or NULL to redraw the mask
 * from d (the same seed and offset as the forward).  X_dropped_saved: the
 * forward's X_dropped_save (read), or NULL to form D(X) again from X and
 * the mask; when given, X is not read and may be NULL.  Other arguments as
 * qlora_linear_bwd.
 */
qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight *w, const uint16_t *X,
                                      const uint16_t *dY, int64_t T, const uint16_t *A,
                                      const uint16_t *B, int32_t r, float alpha,
                                      const qlora_dropout *d, const uint8_t *keep_saved,
                                      const uint16_t *X_dropped_saved, const uint16_t *U_saved,
                                      uint16_t *dX, float *dA, float *dB, void *ws,
                                      size_t ws_bytes, void *stream);

/*
 * Measurement aid.  On the calling host thread, until changed, every later
 * call that launches kernel group `which` records `start_event` on the
 * caller's stream right before that group and `stop_event` right after it
 * (hipEvent_t handles passed as void*, created by the caller; NULL, NULL
 * turns it off).  Groups: QLORA_TIMING_FWD_GEMM (the fused forward GEMM,
 * or for T <= 64 the two kernels of the skinny forward),
 * QLORA_TIMING_DX_GEMM (the fused backward-dX GEMM), QLORA_TIMING_QUANTIZE
 * (the three quantisation kernels), QLORA_TIMING_DEQUANT, QLORA_TIMING_MERGE,
 * QLORA_TIMING_ADAMW, QLORA_TIMING_DROPOUT (the mask kernel).  Returns
 * QLORA_ERR_SHAPE for an unknown group.
 */
#define QLORA_TIMING_FWD_GEMM 0
#define QLORA_TIMING_DX_GEMM 1
#define QLORA_TIMING_QUANTIZE 2
#define QLORA_TIMING_DEQUANT 3
#define QLORA_TIMING_MERGE 4
#define QLORA_TIMING_ADAMW 5
#define QLORA_TIMING_DROPOUT 6
qlora_status qlora_set_timing_events(int which, void *start_event, void *stop_event);

/* Static English text for a status code (never NULL). */
const char *qlora_status_string(qlora_status s);

/* hipError_t value of the last QLORA_ERR_HIP on the calling host thread. */
int qlora_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
