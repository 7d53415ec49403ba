// AdamW step on the adapter parameters (gfx950), float32 master parameters and
// moments, plus the bf16 copy the next forward reads:
//
//   p1 = p * decay;  m1 = b1 m + (1-b1) g;  v1 = b2 v + (1-b2) (g g);
//   p2 = p1 - step_size * (m1 / (sqrt(v1) / sqrt(bc2) + eps))
//
// (the copy is fp16 for fp16 compute, ta-paperlens 落とし穴)
// (ta-paperlens ページ化オプティマイザ and waylandz 26.6.4: Adam's two moments
// per trainable parameter are kept in 32 bit, and only A and B have them;
// Adam with decoupled weight decay, bias-corrected, in the form PyTorch's
// AdamW documents.)  Every operation is one IEEE float32 rounding in the
// order written (no contraction into FMA; division is the correctly rounded
// sequence and the square root is corrected to the rounded value), so results
// are reproducible bit for bit.
// The step constants come from the host, computed in float64.
//
// Bound by HBM: 28 bytes per element move (p, m, v, g in; p, m, v out) plus
// 2 for the bf16 copy.  Each thread handles 4 consecutive elements with
// 16-byte accesses, grid-stride; the n % 4 tail is done by the first threads.
#include "device_common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Correctly rounded float32 square root of x >= 0.  v_sqrt_f32 is within 1
// ulp; of its estimate s and the two neighbours s-, s+, the rounded root is
// s- when x <= s- * s and s+ when x > s * s+ (those products sit a quarter
// ulp^2 below the squared midpoints, and no float32 x falls in between), the
// signs read off the exact residuals of two FMAs, both with the estimate s.  Inputs below 2^-96 are scaled by 2^32
// first and the root by 2^-16 after (exact powers of two).
__device__ __forceinline__ float sqrt_rn(float x) {
  const bool tiny = x < 0x1p-96f;
  const float xs = tiny ? x * 0x1p+32f : x;
  const float s = __builtin_amdgcn_sqrtf(xs);
  const float sd = __uint_as_float(__float_as_uint(s) - 1u);
  const float su = __uint_as_float(__float_as_uint(s) + 1u);
  float r = __builtin_fmaf(-sd, s, xs) <= 0.0f ? sd : s;
  r = __builtin_fmaf(-su, s, xs) > 0.0f ? su : r;
  r = tiny ? r * 0x1p-16f : r;
  return xs == 0.0f ? xs : r;
}

__device__ __forceinline__ void adamw_one(const AdamwArgs& a, float& p, float& m, float& v,
                                          float g) {
  const float p1 = __fmul_rn(p, a.decay);
  m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.omb1, g));
  v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(a.omb2, __fmul_rn(g, g)));
  const float den = __fadd_rn(__fdiv_rn(sqrt_rn(v), a.bc2_sqrt), a.eps);
  p = __fsub_rn(p1, __fmul_rn(a.step_size, __fdiv_rn(m, den)));
}

}  // namespace

__global__ __launch_bounds__(256) void adamw_kernel(AdamwArgs a) {
  const int64_t n4 = a.n >> 2;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    f32x4_t p = reinterpret_cast<const f32x4_t*>(a.p)[i];
    f32x4_t m = reinterpret_cast<const f32x4_t*>(a.m)[i];
    f32x4_t v = reinterpret_cast<const f32x4_t*>(a.v)[i];
    const f32x4_t g = reinterpret_cast<const f32x4_t*>(a.g)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = p[e], me = m[e], ve = v[e];
      adamw_one(a, pe, me, ve, g[e]);
      p[e] = pe;
      m[e] = me;
      v[e] = ve;
    }
    reinterpret_cast<f32x4_t*>(a.p)[i] = p;
    reinterpret_cast<f32x4_t*>(a.m)[i] = m;
    reinterpret_cast<f32x4_t*>(a.v)[i] = v;
    if (a.p_bf16)
      reinterpret_cast<uint2*>(a.p_bf16)[i] =
          a.f16 ? uint2{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])}
                : uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
  if (blockIdx.x == 0 && threadIdx.x < (a.n & 3)) {
    const int64_t j = 4 * n4 + threadIdx.x;
    float pe = a.p[j], me = a.m[j], ve = a.v[j];
    adamw_one(a, pe, me, ve, a.g[j]);
    a.p[j] = pe;
    a.m[j] = me;
    a.v[j] = ve;
    if (a.p_bf16)
      a.p_bf16[j] = (uint16_t)((a.f16 ? pack_f16x2(pe, 0.0f) : pack_bf16x2(pe, 0.0f)) & 0xFFFFu);
  }
}

hipError_t launch_adamw(const AdamwArgs& a, hipStream_t stream) {
  int64_t blocks = ((a.n >> 2) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlora
