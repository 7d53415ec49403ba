// LoRA side products of the adapter path (gfx950):
//   U  = X A^T          and  G  = dY B                (rank-r projections)
//   dA = s G^T X        and  dB = s dY^T U            (adapter gradients)
// (ta-paperlens 勾配は実際どこへ行くのか: only A and B receive gradients;
//  waylandz 26.2.1/26.2.4: B is [out, r], A is [r, in], scale alpha / r.)
//
// All reductions are split into fixed chunks whose float32 partial sums are
// added in a fixed order by a second kernel: results are run-to-run
// deterministic (no floating-point atomics).
#include "device_common.h"
#include "kernels.h"

namespace qlora {

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// ---------------------------------------------------------------------------
// P[s][t][p] = sum_{k in chunk s} L[t][k] R[p][k].  Workgroup = 4 waves, a
// wave owns 16 rows of L and all r columns; MFMA 16x16x32 with L rows as the
// A operand and rows of R as the B operand (both reduction-contiguous).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lora_proj_partial_kernel(
    const uint16_t* __restrict__ L, const uint16_t* __restrict__ R, int64_t T, int64_t red,
    int r, int64_t chunk, float* __restrict__ P) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int64_t kb = (int64_t)blockIdx.y * chunk;
  const int64_t ke = kb + chunk < red ? kb + chunk : red;
  const int nj = r >> 4;
  const int64_t row = m0 + (lane & 15);
  const bool row_ok = row < T;
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t k = kb; k < ke; k += 32) {
    const int64_t kk = k + 8 * (lane >> 4);
    const bool k_ok = kk < ke;
    u32x4_t a = u32x4_t{0u, 0u, 0u, 0u};
    if (row_ok && k_ok) a = load16(L + row * red + kk);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < nj) {
        u32x4_t b = u32x4_t{0u, 0u, 0u, 0u};
        if (k_ok) b = load16(R + (int64_t)(16 * j + (lane & 15)) * red + kk);
        acc[j] = mfma16(a, b, acc[j]);
      }
    }
  }
  float* out = P + (int64_t)blockIdx.y * T * r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < nj) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = m0 + 4 * (lane >> 4) + e;
        if (t < T) out[t * r + 16 * j + (lane & 15)] = acc[j][e];
      }
    }
  }
}

static int64_t proj_chunk(int64_t red, int splits) {
  int64_t c = (red + splits - 1) / splits;
  return (c + 63) / 64 * 64;
}

hipError_t launch_lora_proj_partial(const uint16_t* L, const uint16_t* R, int64_t T,
                                    int64_t red, int32_t r, int splits, float* P,
                                    hipStream_t stream) {
  const int64_t chunk = proj_chunk(red, splits);
  dim3 grid((unsigned)((T + 63) / 64), (unsigned)splits);
  hipLaunchKernelGGL(lora_proj_partial_kernel, grid, dim3(256), 0, stream, L, R, T, red, r,
                     chunk, P);
  return hipGetLastError();
}

// Fixed-order sum of the split partials.  Writes any of: out_rm[t][p] =
// bf16(v), out_sc[t][p] = bf16(scale * v) (the pre-scaled operand the fused
// GEMM seeds its accumulators with), out_tr[p][t] = bf16(v) with row stride
// ld_tr and zeros for T <= t < ld_tr.
__global__ __launch_bounds__(256) void lora_proj_reduce_kernel(
    const float* __restrict__ P, int64_t T, int r, int splits, uint16_t* __restrict__ out_rm,
    uint16_t* __restrict__ out_sc, float scale, uint16_t* __restrict__ out_tr, int64_t ld_tr,
    int64_t rows_total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows_total * r) return;
  const int64_t t = i / r;
  const int p = (int)(i - t * r);
  float v = 0.0f;
  if (t < T) {
    for (int s = 0; s < splits; ++s) v += P[((int64_t)s * T + t) * r + p];
  }
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
  hipLaunchKernelGGL(lora_proj_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, P, T, r, splits, out_rm, out_sc, scale, out_tr, ld_tr, rows_total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// out[c][r'] = in[r'][c], 32x32 tiles through shared memory; rows R..ld_out-1
// of the input side are written as zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int64_t R, int64_t C,
                                                             uint16_t* __restrict__ out,
                                                             int64_t ld_out) {
  __shared__ uint16_t tile[32][33];
  const int tx = threadIdx.x & 31;
  const int ty = threadIdx.x >> 5;   // 0..7
  const int64_t c0 = (int64_t)blockIdx.x * 32;
  const int64_t r0 = (int64_t)blockIdx.y * 32;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t rr = r0 + ty + 8 * k;
    const int64_t cc = c0 + tx;
    tile[ty + 8 * k][tx] = (rr < R && cc < C) ? in[rr * C + cc] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t cc = c0 + ty + 8 * k;
    const int64_t rr = r0 + tx;
    if (cc < C && rr < ld_out) out[cc * ld_out + rr] = tile[tx][ty + 8 * k];
  }
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t R, int64_t C, uint16_t* out,
                                 int64_t ld_out, hipStream_t stream) {
  dim3 grid((unsigned)((C + 31) / 32), (unsigned)((ld_out + 31) / 32));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, in, R, C, out, ld_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// C[s][p][q] = sum_{t in chunk s} St[p][t] L[t][q].
// Workgroup = 4 waves over the same 128 columns q; the waves take interleaved
// 32-token slices of the chunk and their partials are added in a fixed order
// through shared memory.  The B operand needs 8 consecutive tokens of one
// column per lane while L is token-major: each lane loads an 8 x 8 tile
// (8 rows, 16 B each; 16 lanes cover 256 contiguous bytes of a row) and
// transposes it in registers, which yields operands for 8 columns
// q = q0 + 8 * (lane % 16) + v, v = 0..7 (one MFMA per v).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lora_grad_partial_kernel(
    const uint16_t* __restrict__ St, int64_t ld_st, const uint16_t* __restrict__ L, int64_t T,
    int64_t Q, int r, int64_t chunk, float* __restrict__ P) {
  __shared__ f32x4_t red_buf[8 * 8 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t q0 = (int64_t)blockIdx.x * 128;
  const int64_t tb = (int64_t)blockIdx.y * chunk;
  const int64_t te = tb + chunk < T ? tb + chunk : T;
  const int np = r >> 4;
  const int64_t qc = q0 + 8 * (lane & 15);
  const bool q_ok = qc < Q;
  f32x4_t acc[8][8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[p][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = tb + 32 * wave; t0 < te; t0 += 128) {
    const int64_t tl = t0 + 8 * (lane >> 4);
    u32x4_t in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      in[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (q_ok && tl + i < te) in[i] = load16(L + (tl + i) * Q + qc);
    }
    u32x4_t bop[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        bop[2 * c][d] = perm(in[2 * d + 1][c], in[2 * d][c], 0x05040100u);
        bop[2 * c + 1][d] = perm(in[2 * d + 1][c], in[2 * d][c], 0x07060302u);
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p < np) {
        const u32x4_t a = load16(St + (int64_t)(16 * p + (lane & 15)) * ld_st + tl);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[p][v] = mfma16(a, bop[v], acc[p][v]);
      }
    }
  }
  // fixed-order sum of the 4 waves: ((w0 + w1) + w2) + w3
  for (int w = 1; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
        if (p < np)
#pragma unroll
          for (int v = 0; v < 8; ++v) red_buf[(p * 8 + v) * 64 + lane] = acc[p][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
        if (p < np)
#pragma unroll
          for (int v = 0; v < 8; ++v) acc[p][v] += red_buf[(p * 8 + v) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave == 0 && q_ok) {
    float* out = P + (int64_t)blockIdx.y * r * Q;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p < np) {
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
}

hipError_t launch_lora_grad_partial(const uint16_t* St, int64_t ld_st, const uint16_t* L,
                                    int64_t T, int64_t Q, int32_t r, int splits, float* P,
                                    hipStream_t stream) {
  int64_t chunk = (T + splits - 1) / splits;
  chunk = (chunk + 127) / 128 * 128;
  dim3 grid((unsigned)((Q + 127) / 128), (unsigned)splits);
  hipLaunchKernelGGL(lora_grad_partial_kernel, grid, dim3(256), 0, stream, St, ld_st, L, T, Q, r,
                     chunk, P);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(const float* __restrict__ P,
                                                               int r, int64_t Q, int splits,
                                                               float scale, int transposed,
                                                               float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)r * Q) return;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += P[(int64_t)s * r * Q + i];
  v *= scale;
  if (!transposed) {
    out[i] = v;
  } else {
    const int64_t p = i / Q;
    const int64_t q = i - p * Q;
    out[q * r + p] = v;
  }
}

hipError_t launch_lora_grad_reduce(const float* P, int32_t r, int64_t Q, int splits, float scale,
                                   int transposed, float* out, hipStream_t stream) {
  const int64_t n = (int64_t)r * Q;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, P, r, Q, splits, scale, transposed, out);
  return hipGetLastError();
}

}  // namespace qlora
