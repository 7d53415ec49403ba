// Fused NF4-dequant GEMMs of the QLoRA linear layer (gfx950, bf16 MFMA).
//
//   forward:      Y  = X  dequant(W)^T + s (X A^T) B^T
//   backward dX:  dX = dY dequant(W)   + s (dY B)  A
// ta-paperlens 勾配は実際どこへ行くのか: each matmul dequantises the NF4 blocks it
// needs to bf16, uses them and drops them; the input gradient goes through
// dequant(W)^T; W is never written.  Ultralytics "So funktioniert QLoRA":
// dequantise right before the matmul and add the LoRA path.
//
// Kernel shape: a workgroup of 4 waves computes a 256 (tokens) x 256 (output
// columns) tile with float32 accumulators, stepping the reduction by 64 (one
// NF4 block per weight row in the forward).  Per step:
//   * the activation tile (256 x 64 bf16) is staged global -> registers ->
//     LDS, 16-byte chunks XOR-swizzled by row to keep ds_read_b128 conflict
//     free;
//   * the weight tile is dequantised once per workgroup straight into LDS:
//     each thread builds the 16-entry bf16 table q[k] * c' of one block and
//     translates its packed nibbles with v_perm byte lookups.  The forward
//     keeps W's [out, in] layout; the backward writes the tile transposed so
//     both MFMA operands are reduction-contiguous;
//   * each wave runs 8 x 8 MFMA 16x16x32 bf16 per 32-wide slice on its
//     128 x 128 sub-tile.
// LDS is double buffered: the global loads and dequantisation of step k+1
// are issued around the MFMAs of step k, with one barrier per step.
// The rank-r LoRA product seeds the accumulators (s * L R^T computed first by
// MFMA over r), so the epilogue is a single rounding to bf16.
#include "device_common.h"
#include "kernels.h"

namespace qlora {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;

// element offset of 16-byte chunk `chunk` (8 bf16) of tile row `row`
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <bool kBwd>
__global__ __launch_bounds__(256, 1) void qlora_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t red_len = kBwd ? g.rows : g.cols;
  const int64_t out_len = kBwd ? g.cols : g.rows;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t nsteps = (red_len + BK - 1) / BK;
  const int64_t kblocks = g.cols / 64;
  const float mu = g.mu[0];

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- LoRA term: acc = s * lora_l[rows] . lora_r[cols]^T over r --------
  {
    const int r = g.r;
    for (int p0 = 0; p0 < r; p0 += 32) {
      const int p = p0 + 8 * (lane >> 4);
      const bool p_ok = p < r;
      u32x4_t af[8], bf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + 128 * wm + 16 * i + (lane & 15);
        af[i] = (p_ok && row < g.T) ? ld16(g.lora_l + row * r + p) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t col = n0 + 128 * wn + 16 * j + (lane & 15);
        bf[j] = (p_ok && col < out_len) ? ld16(g.lora_r + col * r + p) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] *= g.scale;
  }

  // ---- staging registers ---------------------------------------------------
  u32x4_t a_reg[8];
  u32x4_t c_reg[2];
  float cp_reg = 0.0f;
  bool w_ok = false;

  auto load_step = [&](int64_t step) {
    const int64_t kbase = step * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int64_t t = m0 + row;
      const int64_t k = kbase + (tid & 7) * 8;
      a_reg[i] = (t < g.T && k < red_len) ? ld16(g.act + t * red_len + k)
                                          : u32x4_t{0u, 0u, 0u, 0u};
    }
    int64_t n, kc;
    if (!kBwd) {
      n = n0 + tid;
      kc = kbase;
    } else {
      n = kbase + (tid & 63);
      kc = n0 + 64 * (tid >> 6);
    }
    w_ok = n < g.rows && kc < g.cols;
    if (w_ok) {
      const u32x4_t* cptr = reinterpret_cast<const u32x4_t*>(g.codes + ((n * g.cols + kc) >> 1));
      c_reg[0] = cptr[0];
      c_reg[1] = cptr[1];
      const int64_t blk = n * kblocks + (kc >> 6);
      cp_reg = block_constant(g.code8[blk], g.s2[blk >> 8], mu);
    }
  };

  auto store_step = [&](int buf) {
    uint16_t* as = As[buf];
    uint16_t* bs = Bs[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4_t*>(as + swz(row, tid & 7)) = a_reg[i];
    }
    const Nf4Lut lut = make_lut(cp_reg);
    if (!kBwd) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        u32x4_t o = u32x4_t{0u, 0u, 0u, 0u};
        if (w_ok) {
          uint32_t d[4];
          dequant8(lut, c_reg[w >> 2][w & 3], d);
          o = u32x4_t{d[0], d[1], d[2], d[3]};
        }
        *reinterpret_cast<u32x4_t*>(bs + swz(tid, w)) = o;
      }
    } else {
      const int nl = tid & 63;
      const int rbase = 64 * (tid >> 6);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t d[4] = {0u, 0u, 0u, 0u};
        if (w_ok) dequant8(lut, c_reg[w >> 2][w & 3], d);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + 8 * w + 2 * e;
          bs[swz(row, nl >> 3) + (nl & 7)] = (uint16_t)(d[e] & 0xFFFFu);
          bs[swz(row + 1, nl >> 3) + (nl & 7)] = (uint16_t)(d[e] >> 16);
        }
      }
    }
  };

  auto compute = [&](int buf) {
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kchunk = s * 4 + (lane >> 4);
      u32x4_t af[8], bf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(as + swz(128 * wm + 16 * i + (lane & 15), kchunk));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bf[j] = *reinterpret_cast<const u32x4_t*>(bs + swz(128 * wn + 16 * j + (lane & 15), kchunk));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
    }
  };

  load_step(0);
  store_step(0);
  __syncthreads();
  for (int64_t step = 0; step < nsteps; ++step) {
    const int cur = (int)(step & 1);
    const bool more = step + 1 < nsteps;
    if (more) load_step(step + 1);
    compute(cur);
    if (more) store_step(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: round to bf16 -------------------------------------------
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = n0 + 128 * wn + 16 * j + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + 128 * wm + 16 * i + 4 * (lane >> 4) + e;
        if (row < g.T && col < out_len)
          g.out[row * out_len + col] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
      }
    }
  }
}

hipError_t launch_qlora_fwd_gemm(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.rows + BN - 1) / BN), (unsigned)((a.T + BM - 1) / BM));
  hipLaunchKernelGGL(qlora_gemm_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qlora_dx_gemm(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.cols + BN - 1) / BN), (unsigned)((a.T + BM - 1) / BM));
  hipLaunchKernelGGL(qlora_gemm_kernel<true>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qlora
