// Host-side shape/pointer validation and workspace layout shared by the
// entry points (abi.cpp) and the host-only validation unit (validate.cpp).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qlora_nf4.h"

namespace qlora {

constexpr size_t kWsAlign = 256;

// Token counts up to this use the skinny forward (gemv.hip).
constexpr int64_t kGemvMaxTokens = 64;
int gemv_splits(int64_t rows, int64_t cols);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WeightDims {
  int64_t rows, cols, n, n_b, n_g;
  int qt;      // codebook: QLORA_QUANT_NF4 / QLORA_QUANT_INT4
  bool dq;     // double-quantised constants (else float32 constants)
  bool f16;    // compute dtype fp16 (else bf16)
};

// Shape rules of a packed weight: rows >= 1, rows % 16 == 0, cols >= 64,
// cols % 64 == 0, and n = rows * cols below 2^44.
qlora_status check_weight_shape(int64_t rows, int64_t cols, WeightDims* d);
qlora_status check_descriptor(const qlora_nf4_weight* w, WeightDims* d);
bool aligned16(const void* p);

// Workspace layout of the quantizer.
struct QuantWs {
  size_t cblk_off, gpart_off, total;
};
QuantWs quant_ws_layout(const WeightDims& d);

// Workspace layout of the linear forward / backward.
struct LinearWs {
  int s_proj_x;     // split count of X A^T over cols
  int s_proj_dy;    // split count of dY B over rows
  int s_grad;       // split count of G^T X and U^T dY over tokens
  int s_gemv;       // split count of the skinny forward (0: fused GEMM path)
  size_t proj_off, u_off, gemv_off, gemv_u_off, at_off, g_off, gn_off, un_off, grad_off, grad_b_off;
  size_t xd_off, keep_off;   // lora_dropout: dropped input [T, cols] bf16 and the packed mask
  size_t total;
};
// With dropout the forward always takes the general path and the layout
// adds the dropped input and the keep mask.
LinearWs linear_ws_layout(int64_t T, const WeightDims& d, int32_t r, bool bwd,
                          bool dropout = false);

bool linear_dims_ok(int64_t T, int64_t rows, int64_t cols);

// lora_dropout: shape rule of a [T, cols] input (cols % 64 == 0, T * cols
// bf16 below 2 GiB), bytes of its packed keep mask, and the kernel constants
// of a qlora_dropout (QLORA_ERR_NULL / QLORA_ERR_SHAPE for a NULL pointer or
// p outside [0, 1)).
bool dropout_dims_ok(int64_t T, int64_t cols);
size_t dropout_mask_bytes(int64_t T, int64_t cols);
struct DropoutConsts {
  uint32_t thr, key0, key1, ctr2, ctr3;
  float inv_keep;   // RN32(1 / (1 - p))
};
qlora_status dropout_consts(const qlora_dropout* d, DropoutConsts* k);

// Step constants of qlora_adamw_step (float64 arithmetic, one rounding to
// float32 each); false on invalid hyperparameters.
struct AdamwConsts {
  float decay, b1, omb1, b2, omb2, step_size, bc2_sqrt, eps;
};
bool adamw_constants(int64_t step, double lr, double beta1, double beta2, double eps,
                     double weight_decay, AdamwConsts* k);

qlora_status check_linear_args(const qlora_nf4_weight* w, int64_t T, int32_t r, float alpha,
                               WeightDims* d);

}  // namespace qlora
