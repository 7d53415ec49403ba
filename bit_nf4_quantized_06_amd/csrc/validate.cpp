// Host-only argument validation and workspace layouts of the C ABI.  Pure
// C++ with no HIP calls, so every error path can be exercised without a GPU.
#include <math.h>
#include <string.h>

#include <atomic>

#include "abi_internal.h"

namespace qlora {

// Split count of the rank-r projections: about 512 workgroups of 4 waves
// (two per CU), each split at least two 128-wide iterations long, and the
// float32 partials (S T r) at most a quarter of the bytes of L (T red bf16).
int lora_proj_splits(int64_t T, int64_t red, int32_t r) {
  const int64_t tiles = (T + 127) / 128;
  // about one workgroup per CU: measured on the 7B block at 8192 tokens,
  // half that many splits ran the step 0.8% faster than two per CU (longer
  // reduction runs per workgroup, half the partials to reduce), a quarter
  // 1.2% slower, one split 6% slower
  int64_t s = (256 + tiles - 1) / tiles;
  int64_t max_s = (red + 255) / 256;
  const int64_t by_bytes = red / (8 * (int64_t)(r > 0 ? r : 1));
  if (max_s > by_bytes) max_s = by_bytes;
  if (s > max_s) s = max_s;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

// Split count of the adapter gradients: about 256 workgroups of 4 waves
// (one per CU) while keeping the float32 partial buffers small.
int lora_grad_splits(int64_t T, int64_t Q) {
  const int64_t qb = (Q + 127) / 128;
  int64_t s = (256 + qb - 1) / qb;
  const int64_t max_s = (T + 255) / 256;
  if (s > max_s) s = max_s;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return (int)s;
}

// Split count of the skinny forward: about 1536 workgroups (6 per CU), each
// wave keeping at least 2 blocks of the reduction (measured best on the
// 8192 x 8192, 22016 x 8192 and 8192 x 22016 shapes at 16 tokens).
int gemv_splits(int64_t rows, int64_t cols) {
  const int64_t tiles = (rows + 63) / 64;
  const int64_t kblocks = cols / 64;
  int64_t s = (1536 + tiles - 1) / tiles;
  int64_t max_s = kblocks / 8;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

qlora_status check_weight_shape(int64_t rows, int64_t cols, WeightDims* d) {
  if (rows < 1 || cols < 64 || (cols % 64) != 0 || (rows % 16) != 0) return QLORA_ERR_SHAPE;
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return QLORA_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n >= (int64_t(1) << 44)) return QLORA_ERR_SHAPE;
  if (d) {
    d->rows = rows;
    d->cols = cols;
    d->n = n;
    d->n_b = n / 64;
    d->n_g = (d->n_b + 255) / 256;
  }
  return QLORA_OK;
}

// The linear-layer kernels address the packed codes and each bf16 activation
// or gradient tensor with 32-bit buffer offsets: every one of them must stay
// below 2 GiB.
bool linear_dims_ok(int64_t T, int64_t rows, int64_t cols) {
  const int64_t kMaxDim = int64_t(1) << 22;
  const int64_t kMaxElems16 = (int64_t(1) << 30) - 64;   // bf16 elements below 2 GiB
  if (T < 0 || rows > kMaxDim || cols > kMaxDim) return false;   // T = 0: an empty batch
  if (rows * cols > 2 * kMaxElems16) return false;      // packed codes below 2 GiB
  if (T > kMaxElems16 / cols || T > kMaxElems16 / rows) return false;
  return true;
}

bool dropout_dims_ok(int64_t T, int64_t cols) {
  const int64_t kMaxElems16 = (int64_t(1) << 30) - 64;
  if (T < 0 || cols < 64 || (cols % 64) != 0 || cols > (int64_t(1) << 22)) return false;
  return T <= kMaxElems16 / cols;
}

size_t dropout_mask_bytes(int64_t T, int64_t cols) {
  return (size_t)((T + 3) / 4) * (size_t)(cols / 2);
}

qlora_status dropout_consts(const qlora_dropout* d, DropoutConsts* k) {
  if (!d) return QLORA_ERR_NULL;
  const double p = d->p;
  if (!(p >= 0.0 && p < 1.0)) return QLORA_ERR_SHAPE;   // also rejects NaN
  // p * 2^32 is exact in float64 and below 2^32, so its floor fits 32 bits
  k->thr = (uint32_t)floor(p * 4294967296.0);
  k->key0 = (uint32_t)(d->seed & 0xFFFFFFFFu);
  k->key1 = (uint32_t)(d->seed >> 32);
  k->ctr2 = (uint32_t)(d->offset & 0xFFFFFFFFu);
  k->ctr3 = (uint32_t)(d->offset >> 32);
  k->inv_keep = (float)(1.0 / (1.0 - p));
  return QLORA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Header fields only: version, block sizes and variant codes.
static qlora_status check_format(const qlora_nf4_weight* w) {
  if (w->format_version != QLORA_NF4_FORMAT_VERSION || w->blocksize != QLORA_NF4_BLOCKSIZE ||
      (w->dq_blocksize != QLORA_NF4_DQ_BLOCKSIZE && w->dq_blocksize != QLORA_NF4_DQ_OFF) ||
      (w->quant_type != QLORA_QUANT_NF4 && w->quant_type != QLORA_QUANT_INT4) ||
      (w->compute_dtype != QLORA_COMPUTE_BF16 && w->compute_dtype != QLORA_COMPUTE_FP16))
    return QLORA_ERR_FORMAT;
  return QLORA_OK;
}

qlora_status check_descriptor(const qlora_nf4_weight* w, WeightDims* d) {
  if (!w) return QLORA_ERR_NULL;
  qlora_status s = check_format(w);
  if (s != QLORA_OK) return s;
  s = check_weight_shape(w->rows, w->cols, d);
  if (s != QLORA_OK) return s;
  const bool dq = w->dq_blocksize == QLORA_NF4_DQ_BLOCKSIZE;
  if (d) {
    d->qt = w->quant_type;
    d->dq = dq;
    d->f16 = w->compute_dtype == QLORA_COMPUTE_FP16;
  }
  if (!w->codes || !w->absmax_scale || (dq && (!w->absmax_code || !w->absmax_offset)))
    return QLORA_ERR_NULL;
  if (!aligned16(w->codes) || !aligned16(w->absmax_scale) ||
      (dq && (!aligned16(w->absmax_code) || !aligned16(w->absmax_offset))))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

QuantWs quant_ws_layout(const WeightDims& d) {
  QuantWs q;
  q.cblk_off = 0;
  q.gpart_off = align_up(sizeof(float) * (size_t)d.n_b, kWsAlign);
  q.total = q.gpart_off + align_up(sizeof(double) * (size_t)d.n_g, kWsAlign);
  return q;
}

int gemm_split_from(int64_t T, int64_t out_len, int64_t red_len) {
  const int64_t tiles = ((T + kGemmTileTokens - 1) / kGemmTileTokens) *
                        ((out_len + kGemmTileOut - 1) / kGemmTileOut);
  const int64_t rem = tiles % kGemmCUs;
  const int64_t nsteps = (red_len + 63) / 64;
  // at least one full round before it, a last round at most half full, and
  // at least 8 reduction steps in each half
  if (tiles <= kGemmCUs || rem == 0 || 2 * rem > kGemmCUs || nsteps < 16) return (int)tiles;
  return (int)(tiles - rem);
}

namespace {
std::atomic<int64_t> g_pre_dq_min_tokens{kPreDqMinTokens};
}  // namespace

int64_t pre_dq_min_tokens() { return g_pre_dq_min_tokens.load(std::memory_order_relaxed); }

bool pre_dq_fits(const WeightDims& d) {
  return d.n < ((int64_t)1 << 30) && d.cols <= ((int64_t)1 << 20);
}

LinearWs linear_ws_layout(int64_t T, const WeightDims& d, int32_t r, bool bwd, bool dropout,
                          bool gemm_split, bool pre_dq) {
  LinearWs L;
  memset(&L, 0, sizeof(L));
  L.s_proj_x = lora_proj_splits(T, d.cols, r);
  L.s_proj_dy = lora_proj_splits(T, d.rows, r);
  L.s_grad = lora_grad_splits(T, d.cols > d.rows ? d.cols : d.rows);
  L.s_gemv = (!bwd && !dropout && T <= kGemvMaxTokens) ? gemv_splits(d.rows, d.cols) : 0;
  size_t off = 0;
  const int s_proj = bwd ? (L.s_proj_x > L.s_proj_dy ? L.s_proj_x : L.s_proj_dy) : L.s_proj_x;
  L.proj_off = off;
  off += align_up(sizeof(float) * (size_t)s_proj * (size_t)T * (size_t)r, kWsAlign);
  L.u_off = off;
  off += align_up(2 * (size_t)T * (size_t)r, kWsAlign);
  L.gemv_off = off;
  off += align_up(sizeof(float) * (size_t)L.s_gemv * (size_t)T * (size_t)d.rows, kWsAlign);
  L.gemv_u_off = off;
  off += align_up(sizeof(float) * (size_t)L.s_gemv * (size_t)T * (size_t)r, kWsAlign);
  if (bwd) {
    L.at_off = off;
    off += align_up(2 * (size_t)d.cols * (size_t)r, kWsAlign);
    L.g_off = off;
    off += align_up(2 * (size_t)T * (size_t)r, kWsAlign);
    L.gn_off = off;
    off += align_up(2 * (size_t)T * (size_t)r, kWsAlign);
    L.un_off = off;
    off += align_up(2 * (size_t)T * (size_t)r, kWsAlign);
    L.grad_off = off;
    off += align_up(sizeof(float) * (size_t)L.s_grad * (size_t)r * (size_t)d.cols, kWsAlign);
    L.grad_b_off = off;
    off += align_up(sizeof(float) * (size_t)L.s_grad * (size_t)r * (size_t)d.rows, kWsAlign);
  }
  if (dropout) {
    L.xd_off = off;
    off += align_up(2 * (size_t)T * (size_t)d.cols, kWsAlign);
    L.keep_off = off;
    off += align_up(dropout_mask_bytes(T, d.cols), kWsAlign);
  }
  if (L.s_gemv == 0) {
    const int64_t out_len = bwd ? d.cols : d.rows;
    const int64_t red_len = bwd ? d.rows : d.cols;
    L.gemm_tiles = (int)(((T + kGemmTileTokens - 1) / kGemmTileTokens) *
                         ((out_len + kGemmTileOut - 1) / kGemmTileOut));
    L.gemm_split = gemm_split ? gemm_split_from(T, out_len, red_len) : L.gemm_tiles;
    const size_t n_split = (size_t)(L.gemm_tiles - L.gemm_split);
    if (n_split > 0) {
      L.split_part_off = off;
      off += align_up(sizeof(float) * n_split * 2 * 65536, kWsAlign);
      L.split_cnt_off = off;
      off += align_up(sizeof(uint32_t) * n_split, kWsAlign);
    }
    L.pre_dq = pre_dq && T >= pre_dq_min_tokens() && pre_dq_fits(d);
    if (L.pre_dq) {
      L.wdq_off = off;
      off += align_up(2 * (size_t)d.n, kWsAlign);
    }
  }
  L.total = off;
  return L;
}

// x^t for an integer t >= 0 by binary exponentiation in float64 (a fixed
// sequence of IEEE multiplications, so any implementation gets the same bits).
static double power_by_squaring(double x, int64_t t) {
  double r = 1.0;
  while (t) {
    if (t & 1) r *= x;
    x *= x;
    t >>= 1;
  }
  return r;
}

bool adamw_constants(int64_t step, double lr, double beta1, double beta2, double eps,
                     double weight_decay, AdamwConsts* k) {
  if (step < 1 || !isfinite(lr) || lr < 0.0 || !isfinite(eps) || eps <= 0.0 ||
      !isfinite(weight_decay) || weight_decay < 0.0 || !(beta1 >= 0.0 && beta1 < 1.0) ||
      !(beta2 >= 0.0 && beta2 < 1.0))
    return false;
  k->decay = (float)(1.0 - lr * weight_decay);
  k->b1 = (float)beta1;
  k->omb1 = (float)(1.0 - beta1);
  k->b2 = (float)beta2;
  k->omb2 = (float)(1.0 - beta2);
  k->step_size = (float)(lr / (1.0 - power_by_squaring(beta1, step)));
  k->bc2_sqrt = (float)sqrt(1.0 - power_by_squaring(beta2, step));
  k->eps = (float)eps;
  return true;
}

qlora_status check_linear_args(const qlora_nf4_weight* w, int64_t T, int32_t r, float alpha,
                               WeightDims* d) {
  const qlora_status s = check_descriptor(w, d);
  if (s != QLORA_OK) return s;
  if (d->qt != QLORA_QUANT_NF4) return QLORA_ERR_FORMAT;   // linear kernels: NF4 levels
  if (!linear_dims_ok(T, d->rows, d->cols)) return QLORA_ERR_SHAPE;
  if (r < 16 || r > QLORA_MAX_RANK || (r % 16) != 0) return QLORA_ERR_SHAPE;
  if (!isfinite(alpha)) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

}  // namespace qlora

extern "C" {

qlora_status qlora_nf4_weight_init(qlora_nf4_weight* w, int64_t rows, int64_t cols) {
  if (!w) return QLORA_ERR_NULL;
  const qlora_status s = qlora::check_weight_shape(rows, cols, nullptr);
  if (s != QLORA_OK) return s;
  w->format_version = QLORA_NF4_FORMAT_VERSION;
  w->blocksize = QLORA_NF4_BLOCKSIZE;
  w->dq_blocksize = QLORA_NF4_DQ_BLOCKSIZE;
  w->quant_type = QLORA_QUANT_NF4;
  w->compute_dtype = QLORA_COMPUTE_BF16;
  w->rows = rows;
  w->cols = cols;
  return QLORA_OK;
}

qlora_status qlora_nf4_weight_init_ex(qlora_nf4_weight* w, int64_t rows, int64_t cols,
                                      int quant_type, int double_quant, int compute_dtype) {
  if (!w) return QLORA_ERR_NULL;
  if ((quant_type != QLORA_QUANT_NF4 && quant_type != QLORA_QUANT_INT4) ||
      (double_quant != 0 && double_quant != 1) ||
      (compute_dtype != QLORA_COMPUTE_BF16 && compute_dtype != QLORA_COMPUTE_FP16))
    return QLORA_ERR_FORMAT;
  const qlora_status s = qlora_nf4_weight_init(w, rows, cols);
  if (s != QLORA_OK) return s;
  w->dq_blocksize = double_quant ? QLORA_NF4_DQ_BLOCKSIZE : QLORA_NF4_DQ_OFF;
  w->quant_type = (int16_t)quant_type;
  w->compute_dtype = (int16_t)compute_dtype;
  return QLORA_OK;
}

qlora_status qlora_nf4_weight_buffer_sizes(const qlora_nf4_weight* w, size_t* codes_bytes,
                                           size_t* absmax_code_bytes,
                                           size_t* absmax_scale_bytes,
                                           size_t* absmax_offset_bytes) {
  if (!w) return QLORA_ERR_NULL;
  qlora_status s = qlora::check_format(w);
  if (s != QLORA_OK) return s;
  qlora::WeightDims d;
  s = qlora::check_weight_shape(w->rows, w->cols, &d);
  if (s != QLORA_OK) return s;
  const bool dq = w->dq_blocksize == QLORA_NF4_DQ_BLOCKSIZE;
  if (codes_bytes) *codes_bytes = (size_t)(d.n / 2);
  if (absmax_code_bytes) *absmax_code_bytes = dq ? (size_t)d.n_b : 0;
  if (absmax_scale_bytes) *absmax_scale_bytes = sizeof(float) * (size_t)(dq ? d.n_g : d.n_b);
  if (absmax_offset_bytes) *absmax_offset_bytes = dq ? sizeof(float) : 0;
  return QLORA_OK;
}

qlora_status qlora_nf4_buffer_sizes(int64_t rows, int64_t cols, size_t* codes_bytes,
                                    size_t* absmax_code_bytes, size_t* absmax_scale_bytes,
                                    size_t* absmax_offset_bytes) {
  qlora::WeightDims d;
  const qlora_status s = qlora::check_weight_shape(rows, cols, &d);
  if (s != QLORA_OK) return s;
  if (codes_bytes) *codes_bytes = (size_t)(d.n / 2);
  if (absmax_code_bytes) *absmax_code_bytes = (size_t)d.n_b;
  if (absmax_scale_bytes) *absmax_scale_bytes = sizeof(float) * (size_t)d.n_g;
  if (absmax_offset_bytes) *absmax_offset_bytes = sizeof(float);
  return QLORA_OK;
}

size_t qlora_nf4_quantize_workspace(int64_t rows, int64_t cols) {
  qlora::WeightDims d;
  if (qlora::check_weight_shape(rows, cols, &d) != QLORA_OK) return 0;
  return qlora::quant_ws_layout(d).total;
}

size_t qlora_linear_workspace(int64_t T, int64_t rows, int64_t cols, int32_t r, int is_bwd) {
  qlora::WeightDims d;
  if (qlora::check_weight_shape(rows, cols, &d) != QLORA_OK) return 0;
  if (!qlora::linear_dims_ok(T, rows, cols)) return 0;
  if (r < 16 || r > QLORA_MAX_RANK || (r % 16) != 0) return 0;
  if (T == 0) return 0;   // an empty batch uses no workspace
  return qlora::linear_ws_layout(T, d, r, is_bwd != 0).total;
}

int64_t qlora_set_pre_dequant_min_tokens(int64_t min_tokens) {
  if (min_tokens < 0) return -1;
  return qlora::g_pre_dq_min_tokens.exchange(min_tokens, std::memory_order_relaxed);
}

int64_t qlora_pre_dequant_min_tokens(void) { return qlora::pre_dq_min_tokens(); }

size_t qlora_dropout_mask_bytes(int64_t T, int64_t cols) {
  if (!qlora::dropout_dims_ok(T, cols)) return 0;
  return qlora::dropout_mask_bytes(T, cols);
}

size_t qlora_linear_workspace_dropout(int64_t T, int64_t rows, int64_t cols, int32_t r,
                                      int is_bwd) {
  qlora::WeightDims d;
  if (qlora::check_weight_shape(rows, cols, &d) != QLORA_OK) return 0;
  if (!qlora::linear_dims_ok(T, rows, cols)) return 0;
  if (r < 16 || r > QLORA_MAX_RANK || (r % 16) != 0) return 0;
  if (T == 0) return 0;   // an empty batch uses no workspace
  return qlora::linear_ws_layout(T, d, r, is_bwd != 0, true).total;
}

const char* qlora_status_string(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "a size is out of range";
    case QLORA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_DEVICE: return "the current device is not a gfx950 GPU";
    case QLORA_ERR_HIP: return "a HIP runtime call failed";
    case QLORA_ERR_FORMAT: return "weight descriptor has a wrong format version or block size";
    case QLORA_ERR_SCRATCH:
      return "the call needs more workspace than qlora_linear_fwd_noalloc's fixed device array "
             "(qlora_linear_fwd_noalloc_max_scratch bytes); use qlora_linear_fwd with a workspace";
  }
  return "unknown status";
}

}  // extern "C"
