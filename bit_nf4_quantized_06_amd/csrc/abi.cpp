// C ABI entry points: validate on the host, then enqueue the gfx950 kernels on
// the caller's stream.  No allocation, no synchronisation, no retained state
// other than a per-device "is gfx950" cache.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <string.h>

#include <atomic>

#include "abi_internal.h"
#include "kernels.h"
#include "qlora_nf4.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

qlora_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return QLORA_ERR_HIP;
}

qlora_status check_device_impl() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? QLORA_OK : QLORA_ERR_DEVICE;
}

struct TimingPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local TimingPair g_timing[7];

// Run `launch` between the caller's timing events of group `which` (if set).
template <typename F>
hipError_t timed(int which, hipStream_t st, F&& launch) {
  const TimingPair& tp = g_timing[which];
  if (tp.start) {
    const hipError_t e = hipEventRecord(tp.start, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e == hipSuccess && tp.stop) e = hipEventRecord(tp.stop, st);
  return e;
}

template <typename T>
T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

namespace qlora {

void set_last_hip_error(int e) { g_last_hip_error = e; }

qlora_status check_device() { return check_device_impl(); }

}  // namespace qlora

namespace {

using namespace qlora;

// The once-per-call dequantisation of w into wdq, run by the projection's
// reduce launch.
void set_dequant(ProjReduce& pr, const qlora_nf4_weight* w, const WeightDims& d, uint16_t* wdq) {
  pr.dq_codes = w->codes;
  pr.dq_code8 = w->absmax_code;
  pr.dq_s2 = w->absmax_scale;
  pr.dq_mu = w->absmax_offset;
  pr.dq_words = d.n / 8;
  pr.dq_dq = d.dq;
  pr.dq_out = wdq;
}

// General forward path: U = inv (Xa A^T) by split reduction (U_save =
// bf16(U), Us = bf16(s U)), then Y = X dequant(W)^T + Us B^T in the fused
// GEMM.  Xa is X, or under lora_dropout the dropped input (inv = 1 / (1-p)).
hipError_t enqueue_fwd_general(const qlora_nf4_weight* w, const WeightDims& d, const uint16_t* X,
                               const uint16_t* Xa, int64_t T, const uint16_t* A,
                               const uint16_t* B, int32_t r, float scale, float inv,
                               uint16_t* Y, uint16_t* U_save, void* ws, const LinearWs& L,
                               hipStream_t st) {
  uint16_t* Us = ws_ptr<uint16_t>(ws, L.u_off);     // [T, r] bf16(s * U)
  float* P = ws_ptr<float>(ws, L.proj_off);
  const int n_split = L.gemm_tiles - L.gemm_split;
  uint32_t* cnt = n_split > 0 ? ws_ptr<uint32_t>(ws, L.split_cnt_off) : nullptr;
  uint16_t* wdq = L.pre_dq ? ws_ptr<uint16_t>(ws, L.wdq_off) : nullptr;
  hipError_t e = launch_lora_proj_partial(Xa, A, false, T, d.cols, r, L.s_proj_x, P, d.f16, st);
  if (e == hipSuccess) {
    TransposeJobs none;
    none.n = 0;
    // the reduction also zeroes the GEMM's arrival counters and runs the
    // once-per-call dequantisation
    ProjReduce pr{P, T, r, L.s_proj_x, U_save, Us, scale * inv, inv, nullptr, 0, d.f16, cnt,
                  n_split};
    if (wdq) set_dequant(pr, w, d, wdq);
    e = launch_lora_proj_reduce(pr, none, st);
  }
  if (e == hipSuccess) {
    GemmArgs g;
    g.act = X;
    g.codes = w->codes;
    g.code8 = w->absmax_code;
    g.s2 = w->absmax_scale;
    g.mu = w->absmax_offset;
    g.rows = d.rows;
    g.cols = d.cols;
    g.lora_l = Us;
    g.lora_r = B;
    g.r = r;
    g.out = Y;
    g.T = T;
    g.keep = nullptr;
    g.dq = d.dq;
    g.f16 = d.f16;
    g.wdq = wdq;
    g.split_from = L.gemm_split;
    g.part = n_split > 0 ? ws_ptr<float>(ws, L.split_part_off) : nullptr;
    g.cnt = cnt;
    e = timed(QLORA_TIMING_FWD_GEMM, st, [&] { return launch_qlora_fwd_gemm(g, st); });
  }
  return e;
}

// Backward: G = dY B (Gn = bf16(inv G), Gs = bf16(s inv G)), the A^T
// transpose, U if not saved, dX = dY dequant(W) + keep * (Gs A) in the fused
// GEMM, then dA = s Gn^T Xa and dB = s dY^T U.  Without dropout Xa = X,
// inv = 1 and keep = NULL.
hipError_t enqueue_bwd(const qlora_nf4_weight* w, const WeightDims& d, const uint16_t* Xa,
                       const uint16_t* dY, int64_t T, const uint16_t* A, const uint16_t* B,
                       int32_t r, float scale, float inv, const uint8_t* keep,
                       const uint16_t* U_saved, uint16_t* dX, float* dA, float* dB, void* ws,
                       const LinearWs& L, hipStream_t st) {
  uint16_t* At = ws_ptr<uint16_t>(ws, L.at_off);    // [cols, r]
  uint16_t* Gs = ws_ptr<uint16_t>(ws, L.g_off);     // [T, r] bf16(s inv dY B)
  uint16_t* Gn = ws_ptr<uint16_t>(ws, L.gn_off);    // [T, r] bf16(inv dY B)
  uint16_t* Un = ws_ptr<uint16_t>(ws, L.un_off);    // [T, r] bf16(inv Xa A^T) if not given
  float* P = ws_ptr<float>(ws, L.proj_off);
  const int n_split = L.gemm_tiles - L.gemm_split;
  uint32_t* cnt = n_split > 0 ? ws_ptr<uint32_t>(ws, L.split_cnt_off) : nullptr;
  uint16_t* wdq = L.pre_dq ? ws_ptr<uint16_t>(ws, L.wdq_off) : nullptr;

  // G = dY B (B read in place as [rows, r]); its reduction writes the dX
  // seed's left operand and dA's, transposes A for the dX seed in the same
  // launch, zeroes the dX GEMM's arrival counters and runs the once-per-call
  // dequantisation
  hipError_t e = launch_lora_proj_partial(dY, B, true, T, d.rows, r, L.s_proj_dy, P, d.f16, st);
  if (e == hipSuccess) {
    TransposeJobs tj;
    tj.n = 1;
    tj.job[0] = TransposeJob{A, r, d.cols, At, r};
    ProjReduce pr{P, T, r, L.s_proj_dy, Gn, Gs, scale * inv, inv, nullptr, 0, d.f16, cnt, n_split};
    if (wdq) set_dequant(pr, w, d, wdq);
    e = launch_lora_proj_reduce(pr, tj, st);
  }
  // U for dB when the forward's U was not kept: recompute inv Xa A^T
  const uint16_t* U = U_saved;
  if (e == hipSuccess && !U_saved) {
    e = launch_lora_proj_partial(Xa, A, false, T, d.cols, r, L.s_proj_x, P, d.f16, st);
    if (e == hipSuccess) {
      TransposeJobs none;
      none.n = 0;
      e = launch_lora_proj_reduce(
          ProjReduce{P, T, r, L.s_proj_x, Un, nullptr, 0.0f, inv, nullptr, 0, d.f16}, none, st);
    }
    U = Un;
  }
  if (e == hipSuccess) {
    GemmArgs g;
    g.act = dY;
    g.codes = w->codes;
    g.code8 = w->absmax_code;
    g.s2 = w->absmax_scale;
    g.mu = w->absmax_offset;
    g.rows = d.rows;
    g.cols = d.cols;
    g.lora_l = Gs;
    g.lora_r = At;
    g.r = r;
    g.out = dX;
    g.T = T;
    g.keep = keep;
    g.dq = d.dq;
    g.f16 = d.f16;
    g.wdq = wdq;
    g.split_from = L.gemm_split;
    g.part = n_split > 0 ? ws_ptr<float>(ws, L.split_part_off) : nullptr;
    g.cnt = cnt;
    e = timed(QLORA_TIMING_DX_GEMM, st, [&] { return launch_qlora_dx_gemm(g, st); });
  }
  // dA = s Gn^T Xa and dB = s dY^T U: partials of both in one launch, then
  // one fixed-order reduction
  if (e == hipSuccess) {
    GradJobs gj;
    gj.n = 2;
    gj.job[0] = GradJob{Gn, Xa, d.cols, ws_ptr<float>(ws, L.grad_off), dA, 0};
    gj.job[1] = GradJob{U, dY, d.rows, ws_ptr<float>(ws, L.grad_b_off), dB, 1};
    e = launch_lora_grad_partial(gj, T, r, L.s_grad, d.f16, st);
    if (e == hipSuccess) e = launch_lora_grad_reduce(gj, r, L.s_grad, scale, st);
  }
  return e;
}

hipError_t enqueue_dropout(const DropoutConsts& k, int64_t T, int64_t cols, const uint16_t* X,
                           uint16_t* Xd, uint8_t* keep, bool generate, hipStream_t st) {
  DropoutArgs a;
  a.X = X;
  a.Xd = Xd;
  a.keep = keep;
  a.T = T;
  a.cols = cols;
  a.thr = k.thr;
  a.key0 = k.key0;
  a.key1 = k.key1;
  a.ctr2 = k.ctr2;
  a.ctr3 = k.ctr3;
  a.generate = generate;
  return timed(QLORA_TIMING_DROPOUT, st, [&] { return launch_dropout(a, st); });
}

}  // namespace

extern "C" {

int qlora_last_hip_error(void) { return g_last_hip_error; }

qlora_status qlora_set_timing_events(int which, void* start_event, void* stop_event) {
  if (which < 0 || which > QLORA_TIMING_DROPOUT) return QLORA_ERR_SHAPE;
  g_timing[which].start = static_cast<hipEvent_t>(start_event);
  g_timing[which].stop = static_cast<hipEvent_t>(stop_event);
  return QLORA_OK;
}

qlora_status qlora_nf4_quantize(const float* W, const qlora_nf4_weight* out, void* ws,
                                size_t ws_bytes, void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_descriptor(out, &d);
  if (s != QLORA_OK) return s;
  // without double quantisation the constants go straight to absmax_scale:
  // no workspace
  if (!W || (d.dq && !ws)) return QLORA_ERR_NULL;
  if (!aligned16(W) || (ws && !aligned16(ws))) return QLORA_ERR_ALIGN;
  const QuantWs L = quant_ws_layout(d);
  if (d.dq && ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(QLORA_TIMING_QUANTIZE, st, [&] {
    return launch_quantize(W, d.n_b, out->codes, out->absmax_code, out->absmax_scale,
                           out->absmax_offset, d.dq ? ws_ptr<float>(ws, L.cblk_off) : nullptr,
                           d.dq ? ws_ptr<double>(ws, L.gpart_off) : nullptr, d.qt, d.dq, st);
  });
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_nf4_dequantize(const qlora_nf4_weight* w, uint16_t* W_bf16, void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_descriptor(w, &d);
  if (s != QLORA_OK) return s;
  if (!W_bf16) return QLORA_ERR_NULL;
  if (!aligned16(W_bf16)) return QLORA_ERR_ALIGN;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(QLORA_TIMING_DEQUANT, st, [&] {
    return launch_dequantize(w->codes, w->absmax_code, w->absmax_scale, w->absmax_offset, d.n,
                             W_bf16, d.qt, d.dq, d.f16, st);
  });
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_nf4_merge(const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B,
                             int32_t r, float alpha, uint16_t* W_merged, void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_descriptor(w, &d);
  if (s != QLORA_OK) return s;
  if (!A || !B || !W_merged) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_merged)) return QLORA_ERR_ALIGN;
  if (r < 16 || r > QLORA_MAX_RANK || (r % 16) != 0 || !isfinite(alpha)) return QLORA_ERR_SHAPE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MergeArgs m;
  m.codes = w->codes;
  m.code8 = w->absmax_code;
  m.s2 = w->absmax_scale;
  m.mu = w->absmax_offset;
  m.rows = d.rows;
  m.cols = d.cols;
  m.A = A;
  m.B = B;
  m.r = r;
  m.scale = alpha / (float)r;
  m.out = W_merged;
  m.qt = d.qt;
  m.dq = d.dq;
  m.f16 = d.f16;
  const hipError_t e = timed(QLORA_TIMING_MERGE, st, [&] { return launch_merge(m, st); });
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_adamw_step(float* param, float* exp_avg, float* exp_avg_sq,
                              const float* grad, uint16_t* param_bf16, int64_t n, int64_t step,
                              double lr, double beta1, double beta2, double eps,
                              double weight_decay, void* stream) {
  return qlora_adamw_step16(param, exp_avg, exp_avg_sq, grad, param_bf16, QLORA_COMPUTE_BF16, n,
                            step, lr, beta1, beta2, eps, weight_decay, stream);
}

qlora_status qlora_adamw_step16(float* param, float* exp_avg, float* exp_avg_sq,
                                const float* grad, uint16_t* param16, int compute_dtype,
                                int64_t n, int64_t step, double lr, double beta1, double beta2,
                                double eps, double weight_decay, void* stream) {
  using namespace qlora;
  uint16_t* param_bf16 = param16;
  if (compute_dtype != QLORA_COMPUTE_BF16 && compute_dtype != QLORA_COMPUTE_FP16)
    return QLORA_ERR_FORMAT;
  if (!param || !exp_avg || !exp_avg_sq || !grad) return QLORA_ERR_NULL;
  if (!aligned16(param) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) || !aligned16(grad) ||
      (param_bf16 && !aligned16(param_bf16)))
    return QLORA_ERR_ALIGN;
  AdamwConsts k;
  if (n < 1 || !adamw_constants(step, lr, beta1, beta2, eps, weight_decay, &k))
    return QLORA_ERR_SHAPE;
  const qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AdamwArgs a;
  a.p = param;
  a.m = exp_avg;
  a.v = exp_avg_sq;
  a.g = grad;
  a.p_bf16 = param_bf16;
  a.f16 = compute_dtype == QLORA_COMPUTE_FP16;
  a.n = n;
  a.decay = k.decay;
  a.b1 = k.b1;
  a.omb1 = k.omb1;
  a.b2 = k.b2;
  a.omb2 = k.omb2;
  a.step_size = k.step_size;
  a.bc2_sqrt = k.bc2_sqrt;
  a.eps = k.eps;
  const hipError_t e = timed(QLORA_TIMING_ADAMW, st, [&] { return launch_adamw(a, st); });
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

namespace qlora {
namespace {

// T = 0, an empty token batch: nothing is read; the forward writes nothing,
// the backward writes dA = 0 and dB = 0 (sums over no tokens).  Only the
// adapter and gradient pointers are checked; activation pointers and the
// workspace may be NULL.
qlora_status empty_batch(const WeightDims& d, int32_t r, const uint16_t* A, const uint16_t* B,
                         float* dA, float* dB, bool bwd, hipStream_t st) {
  if (!A || !B || (bwd && (!dA || !dB))) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || (bwd && (!aligned16(dA) || !aligned16(dB))))
    return QLORA_ERR_ALIGN;
  const qlora_status s = check_device();
  if (s != QLORA_OK || !bwd) return s;
  hipError_t e = launch_zero_f32(dA, (int64_t)r * d.cols, st);
  if (e == hipSuccess) e = launch_zero_f32(dB, d.rows * (int64_t)r, st);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

}  // namespace
}  // namespace qlora

qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t T,
                              const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                              uint16_t* Y, uint16_t* U_save, void* ws, size_t ws_bytes,
                              void* stream) {
  return qlora::linear_fwd_impl(w, X, T, A, B, r, alpha, Y, U_save, ws, ws_bytes, stream, true,
                                true);
}

}  // extern "C"

qlora_status qlora::linear_fwd_impl(const qlora_nf4_weight* w, const uint16_t* X, int64_t T,
                                    const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                                    uint16_t* Y, uint16_t* U_save, void* ws, size_t ws_bytes,
                                    void* stream, bool gemm_split, bool pre_dq) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_linear_args(w, T, r, alpha, &d);
  if (s != QLORA_OK) return s;
  if (T == 0)
    return empty_batch(d, r, A, B, nullptr, nullptr, false, static_cast<hipStream_t>(stream));
  if (!X || !A || !B || !Y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(ws) ||
      (U_save && !aligned16(U_save)))
    return QLORA_ERR_ALIGN;
  const LinearWs L = linear_ws_layout(T, d, r, false, false, gemm_split, pre_dq);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);

  const float scale = alpha / (float)r;
  if (L.s_gemv > 0) {
    // few tokens: U = X A^T and X dequant(W)^T in one streaming pass
    GemvArgs ga;
    ga.X = X;
    ga.codes = w->codes;
    ga.code8 = w->absmax_code;
    ga.s2 = w->absmax_scale;
    ga.mu = w->absmax_offset;
    ga.rows = d.rows;
    ga.cols = d.cols;
    ga.T = T;
    ga.A = A;
    ga.B = B;
    ga.r = r;
    ga.scale = scale;
    ga.Y = Y;
    ga.U_save = U_save;
    ga.P = ws_ptr<float>(ws, L.gemv_off);
    ga.PU = ws_ptr<float>(ws, L.gemv_u_off);
    ga.splits = L.s_gemv;
    ga.dq = d.dq;
    ga.f16 = d.f16;
    const hipError_t e =
        timed(QLORA_TIMING_FWD_GEMM, st, [&] { return launch_qlora_gemv(ga, st); });
    return e == hipSuccess ? QLORA_OK : hip_fail(e);
  }
  const hipError_t e =
      enqueue_fwd_general(w, d, X, X, T, A, B, r, scale, 1.0f, Y, U_save, ws, L, st);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

extern "C" {

qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                              int64_t T, const uint16_t* A, const uint16_t* B, int32_t r,
                              float alpha, const uint16_t* U_saved, uint16_t* dX, float* dA,
                              float* dB, void* ws, size_t ws_bytes, void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_linear_args(w, T, r, alpha, &d);
  if (s != QLORA_OK) return s;
  if (T == 0) return empty_batch(d, r, A, B, dA, dB, true, static_cast<hipStream_t>(stream));
  if (!X || !dY || !A || !B || !dX || !dA || !dB || !ws) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dX) ||
      !aligned16(dA) || !aligned16(dB) || !aligned16(ws) || (U_saved && !aligned16(U_saved)))
    return QLORA_ERR_ALIGN;
  const LinearWs L = linear_ws_layout(T, d, r, true);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = enqueue_bwd(w, d, X, dY, T, A, B, r, alpha / (float)r, 1.0f, nullptr,
                                   U_saved, dX, dA, dB, ws, L, st);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_dropout_mask(const qlora_dropout* dp, int64_t T, int64_t cols,
                                const uint16_t* X, uint16_t* X_dropped, uint8_t* keep,
                                void* stream) {
  using namespace qlora;
  DropoutConsts k;
  qlora_status s = dropout_consts(dp, &k);
  if (s != QLORA_OK) return s;
  if (!dropout_dims_ok(T, cols)) return QLORA_ERR_SHAPE;
  if (T == 0) return QLORA_OK;   // an empty mask
  if (!keep || (X == nullptr) != (X_dropped == nullptr)) return QLORA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(keep) & 3u) != 0 || (X && !aligned16(X)) ||
      (X_dropped && !aligned16(X_dropped)))
    return QLORA_ERR_ALIGN;
  s = check_device();
  if (s != QLORA_OK) return s;
  const hipError_t e =
      enqueue_dropout(k, T, cols, X, X_dropped, keep, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* X, int64_t T,
                                      const uint16_t* A, const uint16_t* B, int32_t r,
                                      float alpha, const qlora_dropout* dp, uint16_t* Y,
                                      uint16_t* U_save, uint8_t* keep_save,
                                      uint16_t* X_dropped_save, void* ws, size_t ws_bytes,
                                      void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_linear_args(w, T, r, alpha, &d);
  if (s != QLORA_OK) return s;
  DropoutConsts k;
  s = dropout_consts(dp, &k);
  if (s != QLORA_OK) return s;
  if (T == 0)
    return empty_batch(d, r, A, B, nullptr, nullptr, false, static_cast<hipStream_t>(stream));
  if (!X || !A || !B || !Y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(ws) ||
      (U_save && !aligned16(U_save)) || (keep_save && !aligned16(keep_save)) ||
      (X_dropped_save && !aligned16(X_dropped_save)))
    return QLORA_ERR_ALIGN;
  const LinearWs L = linear_ws_layout(T, d, r, false, true);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* Xd = X_dropped_save ? X_dropped_save : ws_ptr<uint16_t>(ws, L.xd_off);
  uint8_t* keep = keep_save ? keep_save : ws_ptr<uint8_t>(ws, L.keep_off);
  hipError_t e = enqueue_dropout(k, T, d.cols, X, Xd, keep, true, st);
  if (e == hipSuccess)
    e = enqueue_fwd_general(w, d, X, Xd, T, A, B, r, alpha / (float)r, k.inv_keep, Y, U_save,
                            ws, L, st);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* X,
                                      const uint16_t* dY, int64_t T, const uint16_t* A,
                                      const uint16_t* B, int32_t r, float alpha,
                                      const qlora_dropout* dp, const uint8_t* keep_saved,
                                      const uint16_t* X_dropped_saved, const uint16_t* U_saved,
                                      uint16_t* dX, float* dA, float* dB, void* ws,
                                      size_t ws_bytes, void* stream) {
  using namespace qlora;
  WeightDims d;
  qlora_status s = check_linear_args(w, T, r, alpha, &d);
  if (s != QLORA_OK) return s;
  DropoutConsts k;
  s = dropout_consts(dp, &k);
  if (s != QLORA_OK) return s;
  if (T == 0) return empty_batch(d, r, A, B, dA, dB, true, static_cast<hipStream_t>(stream));
  // X is not read when the forward's dropped input is given
  if ((!X && !X_dropped_saved) || !dY || !A || !B || !dX || !dA || !dB || !ws)
    return QLORA_ERR_NULL;
  if ((X && !aligned16(X)) || !aligned16(dY) || !aligned16(A) || !aligned16(B) ||
      !aligned16(dX) || !aligned16(dA) || !aligned16(dB) || !aligned16(ws) ||
      (U_saved && !aligned16(U_saved)) || (keep_saved && !aligned16(keep_saved)) ||
      (X_dropped_saved && !aligned16(X_dropped_saved)))
    return QLORA_ERR_ALIGN;
  const LinearWs L = linear_ws_layout(T, d, r, true, true);
  if (ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // with a saved mask the kernel only reads it (the pointer is not written)
  uint8_t* keep = keep_saved ? const_cast<uint8_t*>(keep_saved) : ws_ptr<uint8_t>(ws, L.keep_off);
  const uint16_t* Xa = X_dropped_saved;
  hipError_t e = hipSuccess;
  if (X_dropped_saved) {
    // the dropped input is given: only a missing mask is redrawn (bits only)
    if (!keep_saved) e = enqueue_dropout(k, T, d.cols, nullptr, nullptr, keep, true, st);
  } else {
    uint16_t* Xd = ws_ptr<uint16_t>(ws, L.xd_off);
    e = enqueue_dropout(k, T, d.cols, X, Xd, keep, keep_saved == nullptr, st);
    Xa = Xd;
  }
  if (e == hipSuccess)
    e = enqueue_bwd(w, d, Xa, dY, T, A, B, r, alpha / (float)r, k.inv_keep, keep, U_saved, dX,
                    dA, dB, ws, L, st);
  return e == hipSuccess ? QLORA_OK : hip_fail(e);
}

}  // extern "C"
