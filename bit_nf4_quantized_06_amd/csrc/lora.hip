// LoRA side products of the adapter path (gfx950):
//   U  = X A^T          and  G  = dY B                (rank-r projections)
//   dA = s G^T X        and  dB = s dY^T U            (adapter gradients)
// (ta-paperlens 勾配は実際どこへ行くのか: only A and B receive gradients;
//  waylandz 26.2.1/26.2.4: B is [out, r], A is [r, in], scale alpha / r.)
//
// These kernels stream one large activation-shaped operand (X or dY) against
// a small rank-r one, so they are bound by HBM bandwidth.  Each wave keeps
// 8-16 loads of 1 KB in flight (unrolled loops, buffer loads whose
// out-of-range reads return 0 instead of branches).  Reductions are split
// into fixed chunks whose float32 partial sums are added in a fixed order by
// a second kernel: every result is run-to-run deterministic (no
// floating-point atomics).
#include "device_common.h"
#include "kernels.h"

namespace qlora {

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset that reads as 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0ull : bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// P[s][t][p] = sum_{k in chunk s} L[t][k] R[p][k]   (L [T, red], R [r, red])
// Workgroup = 4 waves over 128 rows of L; a wave owns 32 rows (two MFMA
// 16x16x32 row groups) and all r = 16 NJ columns, and walks its reduction
// chunk 128 at a time with all 8 L loads and 4 NJ R loads issued first.
// ---------------------------------------------------------------------------
template <int NJ>
__global__ __launch_bounds__(256) void lora_proj_partial_kernel(
    const uint16_t* __restrict__ L, const uint16_t* __restrict__ R, int64_t T, int64_t red,
    int64_t chunk, float* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 128 + wave * 32;
  const int64_t kb = (int64_t)blockIdx.y * chunk;
  const int64_t ke = kb + chunk < red ? kb + chunk : red;
  const __amdgpu_buffer_rsrc_t lr = rsrc(L, (uint64_t)T * red * 2);
  const __amdgpu_buffer_rsrc_t rr = rsrc(R, (uint64_t)(16 * NJ) * red * 2);
  const int kl = 8 * (lane >> 4);
  f32x4_t acc[2][NJ];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[g][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t k = kb; k < ke; k += 128) {
    u32x4_t a[4][2], b[4][NJ];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t kk = k + 32 * u + kl;
      const bool ok = kk < ke;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int64_t row = m0 + 16 * g + (lane & 15);
        a[u][g] = bload16(lr, ok && row < T ? (uint32_t)((row * red + kk) * 2) : kOOB);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        b[u][j] = bload16(rr, ok ? (uint32_t)(((int64_t)(16 * j + (lane & 15)) * red + kk) * 2)
                                 : kOOB);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[g][j] = mfma16(a[u][g], b[u][j], acc[g][j]);
  }
  float* out = P + (int64_t)blockIdx.y * T * (16 * NJ);
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = m0 + 16 * g + 4 * (lane >> 4) + e;
        if (t < T) out[t * (16 * NJ) + 16 * j + (lane & 15)] = acc[g][j][e];
      }
}

static int64_t proj_chunk(int64_t red, int splits) {
  int64_t c = (red + splits - 1) / splits;
  return (c + 127) / 128 * 128;
}

hipError_t launch_lora_proj_partial(const uint16_t* L, const uint16_t* R, int64_t T,
                                    int64_t red, int32_t r, int splits, float* P,
                                    hipStream_t stream) {
  const int64_t chunk = proj_chunk(red, splits);
  const dim3 grid((unsigned)((T + 127) / 128), (unsigned)splits);
  switch (r >> 4) {
#define QLORA_PROJ_CASE(NJ)                                                                   \
  case NJ:                                                                                    \
    hipLaunchKernelGGL(lora_proj_partial_kernel<NJ>, grid, dim3(256), 0, stream, L, R, T, red, \
                       chunk, P);                                                             \
    break;
    QLORA_PROJ_CASE(1) QLORA_PROJ_CASE(2) QLORA_PROJ_CASE(3) QLORA_PROJ_CASE(4)
    QLORA_PROJ_CASE(5) QLORA_PROJ_CASE(6) QLORA_PROJ_CASE(7) QLORA_PROJ_CASE(8)
#undef QLORA_PROJ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Fixed-order sum of the split partials.  Writes any of: out_rm[t][p] =
// bf16(v), out_sc[t][p] = bf16(scale * v) (the pre-scaled operand the fused
// GEMM seeds its accumulators with), out_tr[p][t] = bf16(v) with row stride
// ld_tr and zeros for T <= t < ld_tr.
// 64 outputs (t, p) per workgroup; wave q adds splits q, q + 4, q + 8, ...
// (loads issued 8 at a time), then the four wave sums are added in order q =
// 0..3: a fixed order for any launch.
__global__ __launch_bounds__(256) void lora_proj_reduce_kernel(
    const float* __restrict__ P, int64_t T, int r, int splits, uint16_t* __restrict__ out_rm,
    uint16_t* __restrict__ out_sc, float scale, uint16_t* __restrict__ out_tr, int64_t ld_tr,
    int64_t rows_total) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  const bool live = i < rows_total * r;
  const int64_t t = live ? i / r : 0;
  const int p = live ? (int)(i - t * r) : 0;
  float v = 0.0f;
  if (live && t < T) {
    const float* src = P + t * r + p;
    const int64_t stride = T * r;
    int s = q;
    for (; s + 28 < splits; s += 32) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = src[(int64_t)(s + 4 * j) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) v += x[j];
    }
    for (; s < splits; s += 4) v += src[(int64_t)s * stride];
  }
  part[q][lane] = v;
  __syncthreads();
  if (q != 0 || !live) return;
  v = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  const uint16_t b = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  if (t < T) {
    if (out_rm) out_rm[t * r + p] = b;
    if (out_sc) out_sc[t * r + p] = (uint16_t)(pack_bf16x2(v * scale, 0.0f) & 0xFFFFu);
  }
  if (out_tr) out_tr[(int64_t)p * ld_tr + t] = b;
}

hipError_t launch_lora_proj_reduce(const float* P, int64_t T, int32_t r, int splits,
                                   uint16_t* out_rm, uint16_t* out_sc, float scale,
                                   uint16_t* out_tr, int64_t ld_tr, hipStream_t stream) {
  const int64_t rows_total = out_tr ? ld_tr : T;
  const int64_t n = rows_total * r;
  hipLaunchKernelGGL(lora_proj_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0,
                     stream, P, T, r, splits, out_rm, out_sc, scale, out_tr, ld_tr, rows_total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Up to three bf16 transposes in one launch: out[c][r'] = in[r'][c] for an
// [R, C] input; out has row stride ld_out and is zero for R <= r' < ld_out.
// 32 x 32 tiles through shared memory; workgroups are assigned to jobs by
// the tile counts of the jobs before them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposeJobs jobs) {
  __shared__ uint16_t tile[32][33];
  int b = blockIdx.x;
  int jdx = 0;
  while (jdx < jobs.n - 1 && b >= jobs.tiles[jdx]) {
    b -= jobs.tiles[jdx];
    ++jdx;
  }
  const TransposeJob& jb = jobs.job[jdx];
  const int64_t tiles_c = (jb.C + 31) / 32;
  const int64_t c0 = (int64_t)(b % tiles_c) * 32;
  const int64_t r0 = (int64_t)(b / tiles_c) * 32;
  const int tx = threadIdx.x & 31;
  const int ty = threadIdx.x >> 5;   // 0..7
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t rr = r0 + ty + 8 * k;
    const int64_t cc = c0 + tx;
    tile[ty + 8 * k][tx] = (rr < jb.R && cc < jb.C) ? jb.in[rr * jb.C + cc] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t cc = c0 + ty + 8 * k;
    const int64_t rr = r0 + tx;
    if (cc < jb.C && rr < jb.ld_out) jb.out[cc * jb.ld_out + rr] = tile[tx][ty + 8 * k];
  }
}

hipError_t launch_transposes(TransposeJobs jobs, hipStream_t stream) {
  int total = 0;
  for (int i = 0; i < jobs.n; ++i) {
    const TransposeJob& j = jobs.job[i];
    jobs.tiles[i] = (int)(((j.C + 31) / 32) * ((j.ld_out + 31) / 32));
    total += jobs.tiles[i];
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)total), dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// C[s][p][q] = sum_{t in chunk s} St[p][t] L[t][q], for up to two problems at
// once (blockIdx.z): the dA partials (St = G^T, L = X) and the dB^T partials
// (St = U^T, L = dY).  Workgroup = 4 waves over the same 128 columns q; the
// waves take interleaved 64-token slices of the chunk and their partials are
// added in a fixed order through shared memory.  The B operand needs 8
// consecutive tokens of one column per lane while L is token-major: each lane
// loads an 8 x 8 tile (8 rows, 16 B each; 16 lanes cover 256 contiguous bytes
// of a row) and transposes it in registers, which yields operands for 8
// columns q = q0 + 8 (lane % 16) + v, v = 0..7 (one MFMA per v).
// ---------------------------------------------------------------------------
template <int NP>
__global__ __launch_bounds__(256) void lora_grad_partial_kernel(GradJobs jobs, int64_t T,
                                                               int64_t chunk) {
  __shared__ f32x4_t red_buf[NP * 8 * 64];
  const GradJob& jb = jobs.job[blockIdx.z];
  const int64_t Q = jb.Q;
  const int64_t q0 = (int64_t)blockIdx.x * 128;
  if (q0 >= Q) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tb = (int64_t)blockIdx.y * chunk;
  const int64_t te = tb + chunk < T ? tb + chunk : T;
  const int64_t qc = q0 + 8 * (lane & 15);
  const __amdgpu_buffer_rsrc_t lr = rsrc(jb.L, (uint64_t)T * Q * 2);
  const __amdgpu_buffer_rsrc_t sr = rsrc(jb.St, (uint64_t)(16 * NP) * jb.ld_st * 2);
  f32x4_t acc[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[p][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = tb + 64 * wave; t0 < te; t0 += 256) {
    u32x4_t in[2][8];
    u32x4_t sa[2][NP];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t tl = t0 + 32 * h + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        in[h][i] = bload16(lr, (tl + i < te && qc < Q) ? (uint32_t)(((tl + i) * Q + qc) * 2) : kOOB);
#pragma unroll
      for (int p = 0; p < NP; ++p)
        sa[h][p] = bload16(sr, (uint32_t)(((int64_t)(16 * p + (lane & 15)) * jb.ld_st + tl) * 2));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t bop[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bop[2 * c][d] = perm(in[h][2 * d + 1][c], in[h][2 * d][c], 0x05040100u);
          bop[2 * c + 1][d] = perm(in[h][2 * d + 1][c], in[h][2 * d][c], 0x07060302u);
        }
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[p][v] = mfma16(sa[h][p], bop[v], acc[p][v]);
    }
  }
  // fixed-order sum of the 4 waves: ((w0 + w1) + w2) + w3
  for (int w = 1; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 8; ++v) red_buf[(p * 8 + v) * 64 + lane] = acc[p][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[p][v] += red_buf[(p * 8 + v) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave == 0 && qc < Q) {
    float* out = jb.P + (int64_t)blockIdx.y * (16 * NP) * Q;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pr = 16 * p + 4 * (lane >> 4) + e;
        f32x4_t lo = f32x4_t{acc[p][0][e], acc[p][1][e], acc[p][2][e], acc[p][3][e]};
        f32x4_t hi = f32x4_t{acc[p][4][e], acc[p][5][e], acc[p][6][e], acc[p][7][e]};
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(out + (int64_t)pr * Q + qc);
        dst[0] = lo;
        dst[1] = hi;
      }
    }
  }
}

hipError_t launch_lora_grad_partial(GradJobs jobs, int64_t T, int32_t r, int splits,
                                    hipStream_t stream) {
  int64_t chunk = (T + splits - 1) / splits;
  chunk = (chunk + 255) / 256 * 256;
  int64_t qmax = 0;
  for (int i = 0; i < jobs.n; ++i) qmax = jobs.job[i].Q > qmax ? jobs.job[i].Q : qmax;
  const dim3 grid((unsigned)((qmax + 127) / 128), (unsigned)splits, (unsigned)jobs.n);
  switch (r >> 4) {
#define QLORA_GRAD_CASE(NP)                                                                  \
  case NP:                                                                                   \
    hipLaunchKernelGGL(lora_grad_partial_kernel<NP>, grid, dim3(256), 0, stream, jobs, T,    \
                       chunk);                                                               \
    break;
    QLORA_GRAD_CASE(1) QLORA_GRAD_CASE(2) QLORA_GRAD_CASE(3) QLORA_GRAD_CASE(4)
    QLORA_GRAD_CASE(5) QLORA_GRAD_CASE(6) QLORA_GRAD_CASE(7) QLORA_GRAD_CASE(8)
#undef QLORA_GRAD_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// out = scale * sum_s P[s] for each job: transposed == 0 -> out[p][q] ([r, Q]),
// transposed != 0 -> out[q][p] ([Q, r]).  All jobs in one launch.
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(GradJobs jobs, int r, int splits,
                                                               float scale) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int jdx = 0;
  while (jdx < jobs.n && i >= (int64_t)r * jobs.job[jdx].Q) {
    i -= (int64_t)r * jobs.job[jdx].Q;
    ++jdx;
  }
  if (jdx >= jobs.n) return;
  const GradJob& jb = jobs.job[jdx];
  const int64_t Q = jb.Q;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += jb.P[(int64_t)s * r * Q + i];
  v *= scale;
  if (!jb.transposed) {
    jb.out[i] = v;
  } else {
    const int64_t p = i / Q;
    const int64_t q = i - p * Q;
    jb.out[q * r + p] = v;
  }
}

hipError_t launch_lora_grad_reduce(GradJobs jobs, int32_t r, int splits, float scale,
                                   hipStream_t stream) {
  int64_t n = 0;
  for (int i = 0; i < jobs.n; ++i) n += (int64_t)r * jobs.job[i].Q;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, jobs, r, splits, scale);
  return hipGetLastError();
}

}  // namespace qlora
