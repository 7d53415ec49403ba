// lora_dropout keep mask and dropped adapter input (gfx950).
//
// (ta-paperlens コードで見る, waylandz 26.4.2 / 26.5.1 / 26.6.4: the adapter
// config sets lora_dropout; the dropout acts on the adapter's input.)  The
// keep decisions come from Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC11): element (t, k) of
// X [T, cols] is kept iff word (t mod 4) of the generator at counter
// (k, t / 4, ctr2, ctr3) under key (key0, key1) is >= thr = floor(p 2^32).
// One call serves the four tokens of a quad at one feature, and the packed
// mask keeps exactly that grouping: one nibble per (quad, feature), bit
// (t mod 4), low nibble for even k.  Bits of tokens past T are 0.
//
// A thread owns one token quad and 8 consecutive features: 8 generator calls
// make one 32-bit mask word (nibble e = feature 8j + e), then the four rows'
// 16-byte pieces of X are masked and stored.  A wave covers 512 consecutive
// features, so each row access is 1 KB contiguous and each mask store 256 B.
// 4 bytes per element move (X read, X_dropped written) plus 1/8 byte of
// mask, and the generator costs 10 rounds of two 32x32->64-bit products per
// 4 elements: on 4096 x 4096 the generator alone (mask only) takes about
// 11 us, the HBM traffic about 9 us; the kernel runs at 15 us.  (A looped
// variant that prefetches the next unit's rows during the generator was
// measured no faster.)
#include "device_common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Philox-4x32 with 10 rounds: a round multiplies counter words 0 and 2 by
// the round multipliers into 64-bit products and forms
// (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key
// advances by the two Weyl increments before every round but the first.
__device__ __forceinline__ void philox4x32_10(uint32_t& x0, uint32_t& x1, uint32_t& x2,
                                              uint32_t& x3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one v_mad_u64_u32 per product and one three-input xor (bitop3 with
    // truth table 0x96) per new word: 703 instructions for 8 calls instead
    // of 966 with separate high and low multiplies and two-input xors
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    x0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x1, k0, 0x96);
    x1 = (uint32_t)p1;
    x2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x3, k1, 0x96);
    x3 = (uint32_t)p0;
  }
}

}  // namespace

template <bool kGenerate>
__global__ __launch_bounds__(256) void dropout_kernel(DropoutArgs a, uint32_t chunks_per_quad,
                                                      uint32_t total) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= total) return;
  const uint32_t q = i / chunks_per_quad;
  const uint32_t j = i - q * chunks_per_quad;
  const int64_t t0 = 4 * (int64_t)q;
  const int64_t valid = a.T - t0;   // >= 1 tokens of this quad lie inside X

  // the X rows first, so their loads are in flight during the generator
  u32x4_t x[4];
  if (a.X) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = u < valid ? t0 + u : t0;
      x[u] = *reinterpret_cast<const u32x4_t*>(a.X + t * a.cols + 8 * (int64_t)j);
    }
  }

  uint32_t* word = reinterpret_cast<uint32_t*>(a.keep + (int64_t)q * (a.cols >> 1)) + j;
  uint32_t m;
  if (kGenerate) {
    m = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t c0 = 8u * j + (uint32_t)e, c1 = q, c2 = a.ctr2, c3 = a.ctr3;
      philox4x32_10(c0, c1, c2, c3, a.key0, a.key1);
      const uint32_t nib = (uint32_t)(c0 >= a.thr) | ((uint32_t)(c1 >= a.thr) << 1) |
                           ((uint32_t)(c2 >= a.thr) << 2) | ((uint32_t)(c3 >= a.thr) << 3);
      m |= nib << (4 * e);
    }
    if (valid < 4) m &= 0x11111111u * ((1u << valid) - 1u);
    *word = m;
  } else {
    m = *word;
  }

  if (a.X) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < valid) {
        const uint32_t bits = (m >> u) & 0x11111111u;   // feature 8j + e at bit 4e
        u32x4_t y;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = ((bits >> (8 * w)) & 1u) * 0x0000FFFFu;
          const uint32_t hi = ((bits >> (8 * w + 4)) & 1u) * 0xFFFF0000u;
          y[w] = x[u][w] & (lo | hi);
        }
        *reinterpret_cast<u32x4_t*>(a.Xd + (t0 + u) * a.cols + 8 * (int64_t)j) = y;
      }
    }
  }
}

hipError_t launch_dropout(const DropoutArgs& a, hipStream_t stream) {
  const uint32_t cpq = (uint32_t)(a.cols >> 3);
  const uint32_t total = (uint32_t)(((a.T + 3) >> 2) * (int64_t)cpq);
  const unsigned blocks = (total + 255u) / 256u;
  if (a.generate)
    hipLaunchKernelGGL(dropout_kernel<true>, dim3(blocks), dim3(256), 0, stream, a, cpq, total);
  else
    hipLaunchKernelGGL(dropout_kernel<false>, dim3(blocks), dim3(256), 0, stream, a, cpq, total);
  return hipGetLastError();
}

}  // namespace qlora
