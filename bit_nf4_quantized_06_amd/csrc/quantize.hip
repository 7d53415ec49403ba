// Bulk kernels: blockwise NF4 quantisation, double quantisation of the block
// constants, and dequantisation to bf16 (gfx950).  Variants: the evenly
// spaced INT4 codebook (Ultralytics glossary "QLoRA", code example), no double
// quantisation (float32 constants stored as they are, ta-paperlens 二重量子化:
// 4.5 bits per weight) and fp16 output (ta-paperlens 落とし穴).
//
// Method: ta-paperlens "QLoRA — 650億パラメータ…", sections 量子化を1段落で
// (absmax per block of 64, nearest level, restore by lookup and multiply),
// NF4 (16 normal-quantile levels with an exact 0 and ends at +-1) and
// 二重量子化 (constants grouped by 256, stored as 8-bit floats with one float32
// per group, after subtracting their mean); Ultralytics glossary "QLoRA"
// (levels construction, blocks of 64, blocks of 256).
#include "device_common.h"
#include "kernels.h"

namespace qlora {

typedef double f64x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Quantise: one workgroup per group of 256 blocks (16384 weights, 64 KB of
// float32).  A wave owns 64 consecutive blocks, all loaded up front; per
// iteration 8 lanes share a block: lane s holds the 16-byte chunks s and
// s + 8 of the block's 256 bytes, so each load instruction covers whole
// 128-byte lines.
// The block absmax is an 8-lane xor butterfly.  The quotient RN32(w / c) is
// computed as Markstein's corrected product with the correctly rounded
// reciprocal of c's significand (one IEEE division per block); with
// y = RN(1/c) and q0 = RN(w y) within an ulp, the residual w - q0 c is exact
// and q0 + residual * y rounds to RN(w / c).  Scaling both w and c by 2^-e
// (e = exponent of c) keeps y normal for any finite c, denormals included.
// Lane s holds elements 4s .. 4s+3 and 32 + 4s .. 32 + 4s + 3; a neighbour
// exchange (DPP) assembles the 8-element code words: even lanes store words
// 0..3, odd lanes words 4..7.
// ---------------------------------------------------------------------------

// Nearest-level code by bins.  [-1, 1] is cut into 32 bins of width 1/16,
// bin b covering [b/16 - 1, (b+1)/16 - 1).  Each holds at most one decision
// threshold of either codebook (neighbouring NF4 thresholds are at least
// 0.08 apart, INT4's 2/15), so the code of a quotient r in bin b is the
// number of thresholds below the bin's lower edge plus (r > the bin's
// threshold; +inf for a bin without one), ties going to the lower level as
// the comparison is strict.  b = floor(fma(r, 16, 16)) (|r| <= 1, so 0 <=
// b <= 32, clamped to 31): 16 r is exact and the one rounding can only lift
// r into the next bin, and only within 2^-24 of that bin's lower edge, where
// the next bin's count plus its comparison give the same code as long as no
// threshold lies in between -- NF4's thresholds lie at least 1.6e-3 from an
// edge, and INT4's threshold at exactly 0 is itself an edge, compared
// against r.  (Checked on the host against the plain threshold count for
// both codebooks on 2.0e6 quotients each: random, every float32 within 200
// ulps of each threshold and edge, +-1, +-0, +-2^-149.)  The table, one
// 8-byte entry per bin, lives in LDS: the 32 entries cover the 64 banks once,
// so lanes reading different bins never conflict.  This replaces a 4-step
// binary search of compares and selects: 600 -> 349 vector instructions in
// the NF4 kernel body, 15-22% less time.
struct CodeBin {
  float thr;
  uint32_t base;
};

template <int kQT>
struct CodeBins {
  CodeBin b[32];
  constexpr CodeBins() : b{} {
    for (int i = 0; i < 32; ++i) {
      const float lo = (float)i / 16.0f - 1.0f;
      const float hi = (float)(i + 1) / 16.0f - 1.0f;
      uint32_t base = 0u;
      float t = __builtin_huge_valf();
      for (int k = 0; k < 15; ++k) {
        const float x = kQT ? kINT4Thr[k] : kNF4Thr[k];   // 0: NF4, 1: evenly spaced INT4
        if (x < lo)
          ++base;
        else if (x < hi)
          t = x;
      }
      b[i] = CodeBin{t, base};
    }
  }
};

template <int kQT>
__device__ constexpr CodeBins<kQT> kCodeBins{};

__device__ __forceinline__ uint32_t code_of(float r, const uint2* bins) {
  uint32_t bi = __float2uint_rz(fmaf(r, 16.0f, 16.0f));
  bi = bi < 31u ? bi : 31u;
  const uint2 e = bins[bi];
  return e.y + (r > __uint_as_float(e.x) ? 1u : 0u);
}

// kDQ: also the group's float64 partial sum of the constants (the mean's
// tree); cblk is then the workspace copy of the constants, otherwise the
// stored float32 constants themselves.
template <int kQT, bool kDQ>
__global__ __launch_bounds__(256) void nf4_quantize_blocks_kernel(
    const float* __restrict__ W, int64_t n_b, uint32_t* __restrict__ codes,
    float* __restrict__ cblk, double* __restrict__ gpart) {
  __shared__ double wsum[4];
  __shared__ uint2 bins[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < 32)
    bins[tid] = make_uint2(__float_as_uint(kCodeBins<kQT>.b[tid].thr), kCodeBins<kQT>.b[tid].base);
  __syncthreads();

  const int64_t blk0 = (int64_t)blockIdx.x * kGroup + wave * 64;
  const int sub = lane & 7;
  const bool odd = sub & 1;
  float c_keep = 0.0f;
  // All 16 of the lane's loads (the wave's 64 blocks, 16 KB) go out before
  // any block is coded: 256 bytes per lane in flight, as a plain read stream
  // needs to approach the HBM rate.  Non-temporal buffer loads over the
  // wave's blocks; blocks past the end read as 0.
  f32x4_t x[8][2];
  {
    const int64_t nb_here = n_b - blk0 < 64 ? (n_b - blk0 > 0 ? n_b - blk0 : 0) : 64;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(W + blk0 * kBlock), 0, (int)(nb_here * kBlock * 4), 0x00020000);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = (uint32_t)((it * 8 + (lane >> 3)) * kBlock * 4 + (sub + 8 * h) * 16);
        x[it][h] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 2));
      }
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int64_t b = blk0 + it * 8 + (lane >> 3);
    const bool valid = b < n_b;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = x[it][0][e];       // elements 4s .. 4s+3
      v[4 + e] = x[it][1][e];   // elements 32 + 4s ..
    }
    float m = fabsf(v[0]);
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));

    uint32_t h0, h1;                         // codes of v[0..3], v[4..7]
    if (m == 0.0f) {
      h0 = h1 = 0x7777u;                     // all-zero block: the zero level
    } else {
      int ex;
      const float cm = frexpf(m, &ex);       // m = cm * 2^ex, cm in [0.5, 1)
      const float y = __fdiv_rn(1.0f, cm);
      uint32_t hh[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wm = ldexpf(v[e], -ex);
        const float q0 = wm * y;
        const float rem = fmaf(-q0, cm, wm);
        float r = fmaf(rem, y, q0);
        if (kQT == 1 && fabsf(wm) < 0x1p-126f) {
          // the scaling may have rounded a tiny w (c >= 1); the quotient is
          // then below 2^-125, where the only decision is the evenly spaced
          // codebook's threshold at 0: IEEE w / c is 0 exactly when
          // |w| 2^150 <= c (an exact scaling; inf above 2^-22 is right too)
          const bool nz = ldexpf(fabsf(v[e]), 150) > m;
          r = copysignf(nz ? 0x1p-149f : 0.0f, v[e]);
        }
        hh[e >> 2] |= code_of(r, bins) << (4 * (e & 3));
      }
      h0 = hh[0];
      h1 = hh[1];
    }
    // even lane 2p: word p = h0 | (h0 of lane 2p+1) << 16
    // odd lane 2p+1: word 4 + p = (h1 of lane 2p) | h1 << 16
    const uint32_t send = odd ? h0 : h1;
    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    const uint32_t word = odd ? (got | (h1 << 16)) : (h0 | (got << 16));
    if (valid) codes[b * 8 + (odd ? 4 : 0) + (sub >> 1)] = word;
    if (sub == it) c_keep = m;   // lane l keeps block (l & 7) * 8 + (l >> 3)
  }
  // lane j <- block j of this wave
  const float c = __shfl(c_keep, (lane & 7) * 8 + (lane >> 3));
  const int64_t bj = blk0 + lane;
  if (bj < n_b) cblk[bj] = c;
  if (kDQ) {
    // pairwise float64 tree over the wave's 64 consecutive blocks (padding = 0)
    double s = (bj < n_b) ? (double)c : 0.0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) s += __shfl_down(s, d);
    if (lane == 0) wsum[wave] = s;
    __syncthreads();
    if (tid == 0) gpart[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
}

// ---------------------------------------------------------------------------
// Mean of the block constants: perfect binary float64 tree over the group
// partials (which are its level-8 nodes), zero-padded to a power of two.
// One workgroup of 16 waves.  A wave load takes 128 consecutive leaves
// (16 bytes per lane, 1 KB contiguous); the lane adds its pair and five
// shuffle levels fold the 64 pair sums, so lane 0 holds that 128-leaf
// subtree.  Wave w owns an aligned run of R = max(S / 16, 1) such subtrees
// (S = subtrees in the padded tree), folded 8 at a time and then like a
// binary counter; the 16 run sums are folded last.  Every step adds the two
// children of one node of the same tree.
// ---------------------------------------------------------------------------
// R / 8 < 2^16 (n < 2^44 weights): at most 17 levels of pending subtrees.
constexpr int kMeanLevels = 17;
constexpr int kMeanChunk = 8;   // 128-leaf subtrees per load batch
constexpr int kEncGroupsPerWave = 2;

__device__ __forceinline__ double mean_tree_run(const double* __restrict__ gpart, int64_t n_g,
                                                int64_t R, int wave, int lane) {
  // pending[l]: sum of the last complete subtree of kMeanChunk * 2^l
  // 128-leaf subtrees still waiting for its right sibling (lane 0's value
  // is the one that counts; the levels are unrolled selects, so every index
  // is a constant and the pending sums stay in registers)
  double pending[kMeanLevels];
#pragma unroll
  for (int l = 0; l < kMeanLevels; ++l) pending[l] = 0.0;
  double run = 0.0;
  const int64_t s0 = (int64_t)wave * R;   // first subtree of this wave's run
  for (int64_t i0 = 0; i0 < R; i0 += kMeanChunk) {
    double v[kMeanChunk];
#pragma unroll
    for (int j = 0; j < kMeanChunk; ++j) {
      const int64_t idx = (s0 + i0 + j) * 128 + 2 * lane;
      double lo = 0.0, hi = 0.0;
      if (i0 + j < R) {
        if (idx + 1 < n_g) {
          const f64x2_t x = *reinterpret_cast<const f64x2_t*>(gpart + idx);
          lo = x[0];
          hi = x[1];
        } else if (idx < n_g) {
          lo = gpart[idx];
        }
      }
      v[j] = lo + hi;
    }
#pragma unroll
    for (int j = 0; j < kMeanChunk; ++j)
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) v[j] += __shfl_down(v[j], d);
#pragma unroll
    for (int w = 1; w < kMeanChunk; w <<= 1)
#pragma unroll
      for (int j = 0; j < kMeanChunk; j += 2 * w) v[j] = v[j] + v[j + w];
    double acc = v[0];
    const int64_t k = i0 / kMeanChunk;   // chunk index inside the run
    // the carry runs up through the set low bits of k, merging each pending
    // left sibling, and parks the sum at the first clear bit
    bool carry = true;
#pragma unroll
    for (int l = 0; l < kMeanLevels; ++l) {
      const bool bit = (k >> l) & 1;
      const double merged = pending[l] + acc;
      pending[l] = (carry && !bit) ? acc : pending[l];
      acc = (carry && bit) ? merged : acc;
      carry = carry && bit;
    }
    run = acc;   // after the last chunk (all bits of k set): the run's sum
  }
  return run;
}

__global__ __launch_bounds__(1024) void dq_mean_kernel(const double* __restrict__ gpart,
                                                       int64_t n_g, int64_t n_b, int64_t R,
                                                       float* __restrict__ mu_out) {
  __shared__ double sh[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const double run = mean_tree_run(gpart, n_g, R, wave, lane);
  if (lane == 0) sh[wave] = run;
  __syncthreads();
  if (threadIdx.x < 64) {
    double u = lane < 16 ? sh[lane] : 0.0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) u += __shfl_down(u, d);
    if (lane == 0) mu_out[0] = (float)(u / (double)n_b);
  }
}

// ---------------------------------------------------------------------------
// Double-quantisation codes: one wave per group of 256 blocks, lane l holds
// blocks 4l .. 4l + 3 of it (one 16-byte load, one 4-byte store of codes);
// each wave takes two groups, both loaded before either is encoded.
// d = RN32(c - mu); s2 = max |d| over the group; code8 = E4M3_RNE(RN32(d / s2)
// * 256).  n_b is a multiple of 16, so a lane's 4 blocks are all in or out.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ cblk,
                                                        const float* __restrict__ mu_p,
                                                        int64_t n_b, int64_t n_g,
                                                        uint32_t* __restrict__ code8,
                                                        float* __restrict__ s2_out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const float mu = mu_p[0];
  f32x4_t c[kEncGroupsPerWave];
#pragma unroll
  for (int k = 0; k < kEncGroupsPerWave; ++k) {
    const int64_t b0 = (wave * kEncGroupsPerWave + k) * kGroup + 4 * lane;
    c[k] = b0 < n_b ? *reinterpret_cast<const f32x4_t*>(cblk + b0) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int k = 0; k < kEncGroupsPerWave; ++k) {
    const int64_t g = wave * kEncGroupsPerWave + k;
    const int64_t b0 = g * kGroup + 4 * lane;
    const bool valid = b0 < n_b;
    float d[4];
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d[e] = valid ? __fsub_rn(c[k][e], mu) : 0.0f;
      a = fmaxf(a, fabsf(d[e]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    const float s2 = a;
    if (lane == 0 && g < n_g) s2_out[g] = s2;
    if (valid) {
      uint32_t word = 0u;
      if (s2 > 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          word |= e4m3_encode_rne(__fdiv_rn(d[e], s2) * 256.0f) << (8 * e);
      }
      code8[b0 >> 2] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantise to bf16 (or fp16): one chunk of 1024 words per workgroup
// (dequant_chunk), levels of codebook qt from an LDS table.
// ---------------------------------------------------------------------------
template <bool kDQ, bool kF16>
__global__ __launch_bounds__(256) void nf4_dequant_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ s2, const float* __restrict__ mu_p, int64_t n_words, int qt,
    u32x4_t* __restrict__ out) {
  __shared__ float q[16];
  if (threadIdx.x < 16) q[threadIdx.x] = qt ? kINT4[threadIdx.x] : kNF4[threadIdx.x];
  __syncthreads();
  dequant_chunk<kDQ, kF16>(codes, code8, s2, kDQ ? mu_p[0] : 0.0f, n_words, blockIdx.x, q, out);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const float* W, int64_t n_b, uint8_t* codes, uint8_t* code8,
                           float* s2, float* mu, float* cblk, double* gpart, int qt, bool dq,
                           hipStream_t stream) {
  const int64_t n_g = (n_b + kGroup - 1) / kGroup;
  uint32_t* cw = reinterpret_cast<uint32_t*>(codes);
  if (!dq) {
    // the float32 constants are the stored state (s2 holds n_b of them)
    if (qt)
      hipLaunchKernelGGL((nf4_quantize_blocks_kernel<1, false>), dim3((unsigned)n_g), dim3(256),
                         0, stream, W, n_b, cw, s2, nullptr);
    else
      hipLaunchKernelGGL((nf4_quantize_blocks_kernel<0, false>), dim3((unsigned)n_g), dim3(256),
                         0, stream, W, n_b, cw, s2, nullptr);
    return hipGetLastError();
  }
  if (qt)
    hipLaunchKernelGGL((nf4_quantize_blocks_kernel<1, true>), dim3((unsigned)n_g), dim3(256), 0,
                       stream, W, n_b, cw, cblk, gpart);
  else
    hipLaunchKernelGGL((nf4_quantize_blocks_kernel<0, true>), dim3((unsigned)n_g), dim3(256), 0,
                       stream, W, n_b, cw, cblk, gpart);
  int64_t pow2 = 1;
  while (pow2 < n_g) pow2 <<= 1;
  const int64_t subtrees = pow2 > 128 ? pow2 / 128 : 1;
  const int64_t run = subtrees > 16 ? subtrees / 16 : 1;
  hipLaunchKernelGGL(dq_mean_kernel, dim3(1), dim3(1024), 0, stream, gpart, n_g, n_b, run, mu);
  const int64_t enc_waves = (n_g + kEncGroupsPerWave - 1) / kEncGroupsPerWave;
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)((enc_waves + 3) / 4)), dim3(256), 0, stream,
                     cblk, mu, n_b, n_g, reinterpret_cast<uint32_t*>(code8), s2);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* code8, const float* s2,
                             const float* mu, int64_t n, uint16_t* out, int qt, bool dq, bool f16,
                             hipStream_t stream) {
  const int64_t n_words = n / 8;
  const dim3 grid((unsigned)((n_words + 1023) / 1024));
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  u32x4_t* o = reinterpret_cast<u32x4_t*>(out);
  if (dq && !f16)
    hipLaunchKernelGGL((nf4_dequant_kernel<true, false>), grid, dim3(256), 0, stream, cw, code8,
                       s2, mu, n_words, qt, o);
  else if (dq)
    hipLaunchKernelGGL((nf4_dequant_kernel<true, true>), grid, dim3(256), 0, stream, cw, code8,
                       s2, mu, n_words, qt, o);
  else if (!f16)
    hipLaunchKernelGGL((nf4_dequant_kernel<false, false>), grid, dim3(256), 0, stream, cw, code8,
                       s2, mu, n_words, qt, o);
  else
    hipLaunchKernelGGL((nf4_dequant_kernel<false, true>), grid, dim3(256), 0, stream, cw, code8,
                       s2, mu, n_words, qt, o);
  return hipGetLastError();
}

}  // namespace qlora
