// Device helpers shared by the gfx950 kernels of the NF4 + LoRA linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kBlock = 64;      // weights per absmax block
constexpr int kGroup = 256;     // blocks per second-level constant

// NF4 levels, ascending: standard-normal quantiles at evenly spaced
// probabilities (8 above 0.5, 7 mirrored below, plus an exact 0), divided by
// the largest (Ultralytics glossary "QLoRA", code example under
// "So funktioniert QLoRA"; ta-paperlens NF4 section).  Evaluated in high
// precision and rounded once to float32.
__device__ constexpr float kNF4[16] = {
    -0x1.000000p+0f, -0x1.647366p-1f, -0x1.0cd660p-1f, -0x1.946540p-2f,
    -0x1.234498p-2f, -0x1.7a6a7ep-3f, -0x1.74f0d6p-4f, 0.0f,
    0x1.45f606p-4f,  0x1.4995c2p-3f,  0x1.f809b8p-3f,  0x1.5a0670p-2f,
    0x1.c3496ep-2f,  0x1.200f54p-1f,  0x1.722762p-1f,  0x1.000000p+0f};

// Decision thresholds of the nearest-level rule.  T[k] is the largest float32
// not above the exact midpoint of levels k and k+1, so for a float32 quotient
// r:  r lies above that midpoint  <=>  r > T[k].  Exact midpoints therefore
// stay with the lower level (ties to the lower index).
__device__ constexpr float kNF4Thr[15] = {
    -0x1.b239b4p-1f, -0x1.38a4e4p-1f, -0x1.d70900p-2f, -0x1.5bd4ecp-2f,
    -0x1.e079d8p-3f, -0x1.1a7176p-3f, -0x1.74f0d6p-5f, 0x1.45f606p-5f,
    0x1.ec90c4p-4f,  0x1.a0cfbcp-3f,  0x1.2b05a6p-2f,  0x1.8ea7eep-2f,
    0x1.00da04p-1f,  0x1.491b5ap-1f,  0x1.b913b0p-1f};

// The evenly spaced 4-bit comparison codebook, -1 + 2i/15 rounded once to
// float32 (Ultralytics glossary "QLoRA", code example: 16 evenly spaced
// levels from -1 to 1, no exact 0), and its decision thresholds (largest
// float32 not above the exact midpoint of neighbouring levels; the middle
// one is exactly 0, so a zero quotient takes the lower level 7).
__device__ constexpr float kINT4[16] = {
    -0x1.000000p+0f, -0x1.bbbbbcp-1f, -0x1.777778p-1f, -0x1.333334p-1f,
    -0x1.dddddep-2f, -0x1.555556p-2f, -0x1.99999ap-3f, -0x1.111112p-4f,
    0x1.111112p-4f,  0x1.99999ap-3f,  0x1.555556p-2f,  0x1.dddddep-2f,
    0x1.333334p-1f,  0x1.777778p-1f,  0x1.bbbbbcp-1f,  0x1.000000p+0f};
__device__ constexpr float kINT4Thr[15] = {
    -0x1.dddddep-1f, -0x1.99999ap-1f, -0x1.555556p-1f, -0x1.111112p-1f,
    -0x1.99999ap-2f, -0x1.111112p-2f, -0x1.111112p-3f, 0.0f,
    0x1.111110p-3f,  0x1.111110p-2f,  0x1.99999ap-2f,  0x1.111110p-1f,
    0x1.555556p-1f,  0x1.99999ap-1f,  0x1.dddddep-1f};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// two float32 to binary16, round to nearest even (subnormals kept).  The
// empty asm makes both inputs opaque: otherwise the compiler fuses the
// multiply or add that produced them into a mixed-precision FMA (v_fma_mix),
// which rounds the exact result once to binary16 -- different from rounding
// to float32 first wherever the float32 value is a binary16 tie.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  asm("" : "+v"(lo), "+v"(hi));
  f16x2_t v;
  v.x = (_Float16)lo;
  v.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// the 16-bit compute type of a kernel instance: bfloat16 or binary16
template <bool kF16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
  return kF16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// float32 value of the 16-bit pattern in the low half of v
template <bool kF16>
__device__ __forceinline__ float lo16_to_f32(uint32_t v) {
  if (kF16) return (float)__builtin_bit_cast(f16x2_t, v).x;
  return __uint_as_float(v << 16);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// OCP FP8 E4M3 value of a bit pattern (low byte of `code`), times 2^-8, as
// float32.  v_cvt_f32_fp8 decodes the OCP format exactly on gfx950 (every
// finite pattern; the quantiser never emits the NaN patterns 0x7F / 0xFF);
// the scaling by 2^-8 is exact for every finite pattern.
__device__ __forceinline__ float e4m3_decode_scaled(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0) * 0x1p-8f;
}

// OCP FP8 E4M3 bit pattern nearest to x, ties to even; |x| <= 256 assumed
// (no saturation path).  Sign bit copied (so -0 gives 0x80).
__device__ __forceinline__ uint32_t e4m3_encode_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 31) << 7;
  const float a = fabsf(x);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);      // subnormal: units of 2^-9
  } else {
    const uint32_t ua = __float_as_uint(a);
    mag = (((ua >> 23) - 120u) << 3) | ((ua >> 20) & 7u);
    const uint32_t rest = ua & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (mag & 1u))) mag += 1u;
  }
  return sign | mag;
}

// Block constant of a weight: with double quantisation decoded from the
// 8-bit code, the group scale and the mean (below); without it the float32
// constant itself, which kernels load into the group-scale slot (byte offset
// 4 blk instead of 4 (blk / 256)).
template <bool kDQ>
__device__ __forceinline__ uint32_t scale_offset(int64_t blk) {
  return kDQ ? (uint32_t)((blk >> 8) * 4) : (uint32_t)(blk * 4);
}

// Decoded block constant c' = RN32(RN32(e4m3(code8) * 2^-8 * s2) + mu), no FMA.
__device__ __forceinline__ float block_constant(uint32_t code8, float s2, float mu) {
  return __fadd_rn(__fmul_rn(e4m3_decode_scaled(code8), s2), mu);
}

// c' of a block, or +0 for a block outside the weight (a mask, not a branch,
// so the surrounding straight-line schedule is kept).
__device__ __forceinline__ float block_constant_or_zero(bool ok, uint32_t code8, float s2,
                                                        float mu) {
  const float v = block_constant(code8, s2, mu);
  return __uint_as_float(__float_as_uint(v) & (ok ? 0xFFFFFFFFu : 0u));
}

template <bool kDQ>
__device__ __forceinline__ float weight_constant_or_zero(bool ok, uint32_t code8, float s2_or_c,
                                                         float mu) {
  if (kDQ) return block_constant_or_zero(ok, code8, s2_or_c, mu);
  return __uint_as_float(__float_as_uint(s2_or_c) & (ok ? 0xFFFFFFFFu : 0u));
}

// Dequantise chunk `chunk` of a packed weight to 16 bit: 1024 words of 8
// codes, each of the 256 threads handling 4 words one wave-stride apart so
// that every load (4 B a lane) and store (16 B a lane) of a wave is
// contiguous.  The level comes from the table q (16 floats, in LDS), is
// multiplied by the block constant (decoded, or the stored float32 one
// without double quantisation) in float32 and rounded once to the 16-bit
// compute type.  Shared by the standalone dequantiser and the linear layer's
// once-per-call pass.
template <bool kDQ, bool kF16>
__device__ __forceinline__ void dequant_chunk(const uint32_t* __restrict__ codes,
                                              const uint8_t* __restrict__ code8,
                                              const float* __restrict__ s2, float mu,
                                              int64_t n_words, int64_t chunk, const float* q,
                                              u32x4_t* __restrict__ out) {
  const int64_t base = chunk * (256 * 4) + threadIdx.x;
  uint32_t w[4];
  float cp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + j * 256;
    w[j] = 0u;
    cp[j] = 0.0f;
    if (i < n_words) {
      w[j] = __builtin_nontemporal_load(codes + i);
      const int64_t blk = i >> 3;
      cp[j] = kDQ ? block_constant(code8[blk], s2[blk >> 8], mu) : s2[blk];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + j * 256;
    if (i < n_words) {
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __fmul_rn(q[(w[j] >> (8 * e)) & 15u], cp[j]);
        const float b = __fmul_rn(q[(w[j] >> (8 * e + 4)) & 15u], cp[j]);
        o[e] = pack16x2<kF16>(a, b);
      }
      __builtin_nontemporal_store(o, out + i);
    }
  }
}

// 16-entry bf16 lookup table of one block, q[k] * c' rounded once to bf16,
// split into byte planes for v_perm lookups:
//   lo[i] byte j = low byte of entry 4i+j, hi[i] byte j = high byte.
struct Nf4Lut {
  uint32_t lo[4];
  uint32_t hi[4];
};

template <bool kF16>
__device__ __forceinline__ Nf4Lut make_lut(float cprime) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    p[j] = pack16x2<kF16>(__fmul_rn(kNF4[2 * j], cprime), __fmul_rn(kNF4[2 * j + 1], cprime));
  Nf4Lut t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = perm(p[2 * i + 1], p[2 * i], 0x06040200u);
    t.hi[i] = perm(p[2 * i + 1], p[2 * i], 0x07050301u);
  }
  return t;
}

// Look up 4 codes held one per byte (values 0..15): returns the low bytes and
// the high bytes of the 4 bf16 entries.
__device__ __forceinline__ void lut4(const Nf4Lut& t, uint32_t s, uint32_t& rlo, uint32_t& rhi) {
  const uint32_t s3 = s & 0x07070707u;
  const uint32_t sel = ((s >> 1) & 0x04040404u) | 0x03020100u;   // byte j: j or 4+j by bit 3
  const uint32_t alo = perm(t.lo[1], t.lo[0], s3);
  const uint32_t blo = perm(t.lo[3], t.lo[2], s3);
  const uint32_t ahi = perm(t.hi[1], t.hi[0], s3);
  const uint32_t bhi = perm(t.hi[3], t.hi[2], s3);
  rlo = perm(blo, alo, sel);
  rhi = perm(bhi, ahi, sel);
}

// Dequantise 8 codes (one 32-bit word, element e in bits 4e..4e+3) to 8 bf16
// in natural order: out[j] holds elements 2j (low half) and 2j+1 (high half).
__device__ __forceinline__ void dequant8(const Nf4Lut& t, uint32_t w, uint32_t out[4]) {
  uint32_t elo, ehi, olo, ohi;
  lut4(t, w & 0x0F0F0F0Fu, elo, ehi);           // elements 0,2,4,6
  lut4(t, (w >> 4) & 0x0F0F0F0Fu, olo, ohi);    // elements 1,3,5,7
  const uint32_t la = perm(olo, elo, 0x05010400u);   // low bytes of e0..e3
  const uint32_t lb = perm(olo, elo, 0x07030602u);   // low bytes of e4..e7
  const uint32_t ha = perm(ohi, ehi, 0x05010400u);
  const uint32_t hb = perm(ohi, ehi, 0x07030602u);
  out[0] = perm(ha, la, 0x05010400u);
  out[1] = perm(ha, la, 0x07030602u);
  out[2] = perm(hb, lb, 0x05010400u);
  out[3] = perm(hb, lb, 0x07030602u);
}

template <bool kF16 = false>
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef float f32x16v_t __attribute__((ext_vector_type(16)));

template <bool kF16 = false>
__device__ __forceinline__ f32x16v_t mfma32x32(const u32x4_t& a, const u32x4_t& b,
                                               const f32x16v_t& c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                   __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

}  // namespace qlora
