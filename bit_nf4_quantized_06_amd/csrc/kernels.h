// Internal launcher interface between the C ABI (abi.cpp) and the gfx950
// kernels.  Every launcher only enqueues work on `stream` and returns the
// launch status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qlora {

// --- bulk path (quantize.hip) ---------------------------------------------
// qt: codebook (0 NF4, 1 evenly spaced INT4); dq: double quantisation
// (otherwise s2 holds the n_b float32 block constants and code8, mu, cblk,
// gpart are unused); f16: fp16 output instead of bf16.
hipError_t launch_quantize(const float* W, int64_t n_b, uint8_t* codes, uint8_t* code8,
                           float* s2, float* mu, float* cblk, double* gpart, int qt, bool dq,
                           hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* code8, const float* s2,
                             const float* mu, int64_t n, uint16_t* out, int qt, bool dq, bool f16,
                             hipStream_t stream);

// --- fused dequant GEMMs (gemm.hip) ---------------------------------------
// out[T, out_len] = act[T, red_len] * Wop + lora_l[T, r] * lora_r[out_len, r]^T
// where Wop = dequant(W)^T (forward: red = cols, out = rows) or dequant(W)
// (backward dX: red = rows, out = cols).
struct GemmArgs {
  const uint16_t* act;     // [T, red_len] bf16
  const uint8_t* codes;    // packed weight [rows, cols]
  const uint8_t* code8;
  const float* s2;
  const float* mu;
  int64_t rows, cols;
  const uint16_t* lora_l;  // [T, r] bf16, already multiplied by alpha / r
  const uint16_t* lora_r;  // [out_len, r] bf16
  int32_t r;
  uint16_t* out;           // [T, out_len] bf16
  int64_t T;
  // backward dX only: packed lora_dropout keep mask of [T, cols] (one nibble
  // per 4 tokens x 1 feature), applied to the seed lora_l * lora_r^T; NULL
  // for none
  const uint8_t* keep;
  bool dq;                 // double-quantised constants (else s2 = float32 c per block)
  bool f16;                // fp16 compute (else bf16)
  // the weight already dequantised to 16 bit, [rows, cols] (then codes,
  // code8, s2, mu are not read), or NULL: dequantise in the kernel
  const uint16_t* wdq;
  // K-split of the last tiles: tiles from split_from on run as two units
  // each, one per half of the reduction; both store their float32 partial
  // (part: [tile - split_from][2][65536]) and count in (cnt: [tile -
  // split_from], zero at launch); the second to arrive adds the other's and
  // writes the tile.  split_from = the tile count: no split.
  int split_from;
  float* part;
  uint32_t* cnt;
};
hipError_t launch_qlora_fwd_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_qlora_dx_gemm(const GemmArgs& a, hipStream_t stream);

// lora_dropout (dropout.hip): draw (generate) or read the packed keep mask
// of [T, cols] and, when X is set, write Xd = X where kept, +0 elsewhere.
struct DropoutArgs {
  const uint16_t* X;       // [T, cols] bf16 or NULL
  uint16_t* Xd;            // [T, cols] bf16 (with X)
  uint8_t* keep;           // [ceil(T/4), cols/2] bytes: written or read
  int64_t T, cols;
  uint32_t thr;            // floor(p 2^32)
  uint32_t key0, key1;     // generator key (seed)
  uint32_t ctr2, ctr3;     // counter words 2, 3 (offset)
  bool generate;
};
hipError_t launch_dropout(const DropoutArgs& a, hipStream_t stream);

// Skinny forward for T <= kGemvMaxTokens (gemv.hip): split partials of
// X dequant(W)^T (P) and of U = X A^T (PU), then
// Y = bf16(sum_s P + bf16(scale U) B^T) and U_save = bf16(U).
struct GemvArgs {
  const uint16_t* X;       // [T, cols] bf16
  const uint8_t* codes;    // packed weight [rows, cols]
  const uint8_t* code8;
  const float* s2;
  const float* mu;
  int64_t rows, cols, T;
  const uint16_t* A;       // [r, cols] bf16
  const uint16_t* B;       // [rows, r] bf16
  int32_t r;
  float scale;             // alpha / r
  uint16_t* Y;             // [T, rows] bf16
  uint16_t* U_save;        // [T, r] bf16 or NULL
  float* P;                // [splits][T][rows]
  float* PU;               // [splits][T][r]
  int32_t splits;
  bool dq;                 // double-quantised constants (else s2 = float32 c per block)
  bool f16;                // fp16 compute (else bf16)
};
hipError_t launch_qlora_gemv(const GemvArgs& a, hipStream_t stream);

// --- adapter optimizer step (adamw.hip) -------------------------------------
// float32 constants of one step (computed on the host from float64 values).
struct AdamwArgs {
  float* p;
  float* m;
  float* v;
  const float* g;
  uint16_t* p_bf16;         // 16-bit copy (bf16, or fp16 with f16), may be NULL
  bool f16;
  int64_t n;
  float decay, b1, omb1, b2, omb2, step_size, bc2_sqrt, eps;
};
hipError_t launch_adamw(const AdamwArgs& a, hipStream_t stream);

// --- adapter merge (merge.hip) ----------------------------------------------
// out = bf16(w_hat + scale * (B A)), B [rows, r], A [r, cols], out [rows, cols].
struct MergeArgs {
  const uint8_t* codes;
  const uint8_t* code8;
  const float* s2;
  const float* mu;
  int64_t rows, cols;
  const uint16_t* A;
  const uint16_t* B;
  int32_t r;
  float scale;
  uint16_t* out;
  int qt;                  // codebook (0 NF4, 1 evenly spaced INT4)
  bool dq;                 // double-quantised constants (else s2 = float32 c per block)
  bool f16;                // fp16 (else bf16) A, B, base and result
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// --- LoRA side products (lora.hip) ----------------------------------------
// Split-reduction partials P[s][t][p] = sum_{k in chunk s} L[t][k] R(p, k),
// L [T, red] bf16, P float32 [S][T][r]; R is [r, red] (R(p, k) = R[p][k]) or,
// with r_by_rows, [red, r] (R(p, k) = R[k][p]), read in place.
int lora_proj_splits(int64_t T, int64_t red, int32_t r);
hipError_t launch_lora_proj_partial(const uint16_t* L, const uint16_t* R, bool r_by_rows,
                                    int64_t T, int64_t red, int32_t r, int splits, float* P,
                                    bool f16, hipStream_t stream);
// bf16 transposes: out[c][r'] = in[r'][c] for an [R, C] input; out has row
// stride ld_out and is zero for R <= r' < ld_out.
struct TransposeJob {
  const uint16_t* in;
  int64_t R, C;
  uint16_t* out;
  int64_t ld_out;
};
struct TransposeJobs {
  TransposeJob job[3];
  int tiles[3];   // filled by the launcher
  int n;
};
// v = sum_s P[s] (fixed order s = 0, 1, ...).  Each output may be NULL:
// out_rm[t][p] = bf16(scale_rm * v), out_sc[t][p] = bf16(scale * v),
// out_tr[p][t] = bf16(scale_rm * v) with row stride ld_tr and zeros for
// T <= t < ld_tr.  The same launch runs the transposes of `tj` (tj.n may
// be 0).
struct ProjReduce {
  const float* P;
  int64_t T;
  int32_t r;
  int32_t splits;
  uint16_t* out_rm;
  uint16_t* out_sc;
  float scale;
  float scale_rm;          // 1 except under lora_dropout (1 / (1 - p))
  uint16_t* out_tr;
  int64_t ld_tr;
  bool f16;                // outputs fp16 (else bf16)
  // also zeroed by this launch: the arrival counters of the fused GEMM that
  // follows it (NULL / 0: none)
  uint32_t* zero_cnt;
  int n_zero;
  // also run by this launch: the linear layer's once-per-call dequantisation
  // of its NF4 weight to 16 bit (the type of f16) into dq_out [rows, cols]
  // (NULL: none); dq_words = rows * cols / 8; constants as in the
  // descriptor, double-quantised (dq_dq) or float32
  const uint8_t* dq_codes = nullptr;
  const uint8_t* dq_code8 = nullptr;
  const float* dq_s2 = nullptr;
  const float* dq_mu = nullptr;
  int64_t dq_words = 0;
  bool dq_dq = false;
  uint16_t* dq_out = nullptr;
};
hipError_t launch_lora_proj_reduce(const ProjReduce& a, TransposeJobs tj, hipStream_t stream);

// Adapter-gradient partials and their reduction, up to two problems per
// launch: P[s] = sum_{t in chunk s} S[t][p] L[t][q] with S [T, r] and L [T, Q]
// bf16 (token-major), stored [r, Q] (transposed == 0) or [Q, r]
// (transposed != 0); then out = scale * sum_s P[s] in the same layout.
struct GradJob {
  const uint16_t* S;
  const uint16_t* L;
  int64_t Q;
  float* P;
  float* out;
  int transposed;
};
struct GradJobs {
  GradJob job[2];
  int n;
};
int lora_grad_splits(int64_t T, int64_t Q);
hipError_t launch_lora_grad_partial(GradJobs jobs, int64_t T, int32_t r, int splits, bool f16,
                                    hipStream_t stream);
hipError_t launch_lora_grad_reduce(GradJobs jobs, int32_t r, int splits, float scale,
                                   hipStream_t stream);

// n float32 zeros at p (n % 4 == 0, p 16-byte aligned).
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);

}  // namespace qlora
