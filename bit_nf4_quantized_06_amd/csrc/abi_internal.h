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
  size_t proj_off, u_off, gemv_off, gemv_u_off, at_off, g_off, gn_off, un_off, grad_off, grad_b_off, total;
};
LinearWs linear_ws_layout(int64_t T, const WeightDims& d, int32_t r, bool bwd);

bool linear_dims_ok(int64_t T, int64_t rows, int64_t cols);

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
