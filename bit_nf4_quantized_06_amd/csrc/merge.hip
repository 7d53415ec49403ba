// Merge of the LoRA adapter into the dequantised base (gfx950):
//
//   W_merged[n][k] = bf16( w_hat[n][k] + s * (B A)[n][k] ),  s = alpha / r,
//
// w_hat the bf16 dequantised weight, B [rows, r] and A [r, cols] bf16, the
// product accumulated in float32, scaled and added in float32, rounded once
// to bf16.  (Variants: fp16 in place of bf16 throughout, float32 block
// constants without double quantisation, the evenly spaced INT4 codebook.)  (waylandz LLM book 26.2: at inference the adapter is folded into
// the weight once, W + (alpha/r) B A; ta-paperlens 落とし穴 and the
// Ultralytics QLoRA page, Kompromisse: the merge is done on the base
// dequantised to 16 bit, and the result may be quantised again.)
//
// Bound by HBM: per weight it reads half a byte of codes and writes two bytes
// of bf16; the rank-r product (r multiply-adds per weight) runs on MFMA.
//
// Workgroup = 4 waves over 256 columns and a group of 256 rows, walked 32
// rows at a time.  The 256-column slice of A stays in LDS for the whole
// group (row stride padded by 16 bytes); each wave forms (B A) for the 32
// rows x its 64 columns with MFMA 32x32x16, B fragments straight from
// memory (8 consecutive r of one row), A fragments through ds_read_b64_tr_b16
// (8 consecutive r of one column).  s * (B A) goes to LDS in float32, laid
// out per consumer thread (36 floats, 16-byte aligned, 9 distinct 16-byte
// bank groups per 16 threads); then each thread decodes four 8-weight
// chunks of one row, 64 columns apart, adds its 32 values and writes four
// 16-byte pieces: 8 neighbouring threads fill whole 128-byte lines with each
// store (16-byte pieces at a 64-byte stride, as a thread-contiguous layout
// gives, measured 25% slower, twice as slow with non-temporal stores).  The codes, block
// constant inputs and B fragments of the next pass are loaded while the
// current one runs.
#include "device_common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kMergeCols = 256;   // columns per workgroup
constexpr int kMergeRows = 256;   // rows per workgroup
constexpr int kTileRows = 32;     // rows per pass
constexpr int kASlice = 264;      // A slice row stride in elements (256 + 8)
constexpr int kDStride = 36;      // floats per consumer thread in the delta buffer

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <bool kF16>
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b,
                                           const f32x16_t& c) {
  return mfma32x32<kF16>(a, b, c);
}

__device__ __forceinline__ u32x4_t ld_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo);
  const uint2 h = __builtin_bit_cast(uint2, hi);
  return u32x4_t{l.x, l.y, h.x, h.y};
}

// float32 value of x rounded to the 16-bit compute type (nearest even)
template <bool kF16>
__device__ __forceinline__ float round16(float x) {
  return lo16_to_f32<kF16>(pack16x2<kF16>(x, 0.0f));
}

}  // namespace

// Loads of one 32-row pass: this thread's codes and block-constant inputs
// (consumer role) and its B fragments (MFMA role).  The consumer thread owns
// four 8-column chunks of one row, 64 columns apart (columns kb + 64 w +
// [0, 8), w = 0..3), i.e. one chunk in each of four consecutive blocks: 8
// neighbouring threads then write whole 128-byte lines with each store, the
// four 8-bit constant codes are one 4-byte load and the group scale is
// shared.  Row and column indices are clamped into the weight, so every
// load is unconditional (no branch, no serialising wait); values of clamped
// rows or chunks are never stored.  (The four blocks need not start at a
// multiple of 4 nor lie in one group of 256, so each has its own loads.)
template <int NP>
struct MergePass {
  uint32_t cw[4];           // 8 codes of chunk w
  uint32_t c8[4];           // 8-bit constant code of chunk w's block
  float s2[4];              // group scale of chunk w's block
  u32x4_t bf[NP];
};

struct MergeCtx {
  const uint16_t* as;
  float* dl;
  const float* q;
  const float* dmine;
  float mu;
  int crow, l32, lhi, wave, prow, acol[2];
  int64_t kb;               // first column of chunk 0
  int64_t kclamp[4];        // chunk w's first column, clamped into the weight
  bool wok[4];              // chunk w lies inside the weight
};

// kDQ false: s2[w] receives chunk w's block constant itself (float32, one
// per block) and there is no 8-bit code.
template <int NP, bool kDQ>
__device__ __forceinline__ void merge_load(const MergeArgs& a, const MergeCtx& c, int64_t n0,
                                           MergePass<NP>& m) {
  const int64_t last = a.rows - 1;
  const int64_t n = n0 + c.crow < last ? n0 + c.crow : last;
  const int64_t rowe = n * a.cols;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int64_t e0 = rowe + c.kclamp[w];
    m.cw[w] = *reinterpret_cast<const uint32_t*>(a.codes + e0 / 2);
    if (kDQ) {
      m.c8[w] = a.code8[e0 >> 6];
      m.s2[w] = a.s2[e0 >> 14];
    } else {
      m.c8[w] = 0u;
      m.s2[w] = a.s2[e0 >> 6];
    }
  }
  const int64_t bn = n0 + c.l32 < last ? n0 + c.l32 : last;
#pragma unroll
  for (int j = 0; j < NP; ++j)
    m.bf[j] = *reinterpret_cast<const u32x4_t*>(a.B + bn * (16 * NP) + 16 * j + 8 * c.lhi);
}

// One 32-row pass from `cur`; the loads of the pass after it go to `nxt`
// first.  The two register sets alternate between passes (no copy, so
// nothing waits for the loads or for the previous pass's stores).
template <int NP, bool kDQ, bool kF16>
__device__ __forceinline__ void merge_pass(const MergeArgs& a, const MergeCtx& c, int64_t n0,
                                           const MergePass<NP>& cur, MergePass<NP>& nxt) {
  merge_load<NP, kDQ>(a, c, n0 + kTileRows, nxt);
  f32x16_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* p = c.as + (16 * j + c.prow) * kASlice + c.acol[t];
      acc[t] = mfma32<kF16>(cur.bf[j], ld_tr_pair(p, p + 4 * kASlice), acc[t]);
    }
  }
  // acc[t][e] = (B A)[row 8 (e / 4) + 4 lhi + e % 4][column 64 wave + 32 t + l32];
  // column col belongs to consumer thread 8 row + (col / 8) % 8, element
  // 8 (col / 64) + col % 8 of its 32
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int col = 64 * c.wave + 32 * t + c.l32;
    const int slot = (col >> 3) & 7;
    const int elem = 8 * (col >> 6) + (col & 7);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * c.lhi + (e & 3);
      c.dl[(row * 8 + slot) * kDStride + elem] = __fmul_rn(acc[t][e], a.scale);
    }
  }
  __syncthreads();
  u32x4_t d4[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) d4[j] = *reinterpret_cast<const u32x4_t*>(c.dmine + 4 * j);
  const int64_t n = n0 + c.crow;
  const bool row_ok = n < a.rows;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float cp = kDQ ? block_constant(cur.c8[w], cur.s2[w], c.mu) : cur.s2[w];
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 8 * w + 2 * e;   // element index within the 32
      const float lo = round16<kF16>(__fmul_rn(c.q[(cur.cw[w] >> (8 * e)) & 15u], cp));
      const float hi = round16<kF16>(__fmul_rn(c.q[(cur.cw[w] >> (8 * e + 4)) & 15u], cp));
      const float dlo = __uint_as_float(d4[i >> 2][i & 3]);
      const float dhi = __uint_as_float(d4[(i + 1) >> 2][(i + 1) & 3]);
      o[e] = pack16x2<kF16>(__fadd_rn(lo, dlo), __fadd_rn(hi, dhi));
    }
    if (row_ok && c.wok[w])
      *reinterpret_cast<u32x4_t*>(a.out + n * a.cols + c.kb + 64 * w) = o;
  }
  __syncthreads();   // the delta buffer is rewritten by the next pass
}

template <int NP, bool kDQ, bool kF16>
__global__ __launch_bounds__(256) void nf4_merge_kernel(MergeArgs a) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int R = 16 * NP;
  __shared__ __attribute__((aligned(16))) uint16_t as[R * kASlice];
  __shared__ __attribute__((aligned(16))) float dl[256 * kDStride];
  __shared__ float q[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  MergeCtx c;
  c.as = as;
  c.dl = dl;
  c.q = q;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.l32 = lane & 31;
  c.lhi = lane >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * kMergeCols;
  const int64_t nb = (int64_t)blockIdx.y * kMergeRows;
  const int64_t ne = nb + kMergeRows < a.rows ? nb + kMergeRows : a.rows;
  if (tid < 16) q[tid] = a.qt ? kINT4[tid] : kNF4[tid];
  // the A slice; columns past the weight read a clamped column, and only
  // feed columns that are never stored
  for (int i = tid; i < R * 32; i += 256) {
    const int p = i >> 5;
    const int ch = i & 31;
    const int64_t k = k0 + 8 * ch < a.cols ? k0 + 8 * ch : a.cols - 8;
    *reinterpret_cast<u32x4_t*>(as + p * kASlice + 8 * ch) =
        *reinterpret_cast<const u32x4_t*>(a.A + (int64_t)p * a.cols + k);
  }
  c.mu = kDQ ? a.mu[0] : 0.0f;
  // consumer role: row crow of the pass, chunks at columns kb + 64 w
  c.crow = tid >> 3;
  c.kb = k0 + 8 * (tid & 7);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    c.wok[w] = k0 + 64 * w < a.cols;
    c.kclamp[w] = (c.wok[w] ? k0 + 64 * w : a.cols - 64) + 8 * (tid & 7);
  }
  c.dmine = dl + tid * kDStride;
  // MFMA role: 32 rows x columns 64 wave + 32 t + [0, 32)
  c.prow = 8 * c.lhi + ((lane & 15) >> 2);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    c.acol[t] = 64 * c.wave + 32 * t + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  MergePass<NP> p0, p1;
  merge_load<NP, kDQ>(a, c, nb, p0);
  __syncthreads();   // A slice and table visible
  if (ne - nb == kMergeRows) {
    // a whole row group: straight-line passes, so the waits before each
    // pass count exactly the loads and stores issued since its own loads
#pragma unroll
    for (int i = 0; i < kMergeRows / kTileRows; i += 2) {
      merge_pass<NP, kDQ, kF16>(a, c, nb + i * kTileRows, p0, p1);
      merge_pass<NP, kDQ, kF16>(a, c, nb + (i + 1) * kTileRows, p1, p0);
    }
  } else {
    for (int64_t n0 = nb; n0 < ne; n0 += 2 * kTileRows) {
      merge_pass<NP, kDQ, kF16>(a, c, n0, p0, p1);
      if (n0 + kTileRows >= ne) break;
      merge_pass<NP, kDQ, kF16>(a, c, n0 + kTileRows, p1, p0);
    }
  }
#endif
}

template <bool kDQ, bool kF16>
static hipError_t merge_dispatch(const MergeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.cols + kMergeCols - 1) / kMergeCols),
                  (unsigned)((a.rows + kMergeRows - 1) / kMergeRows));
  switch (a.r >> 4) {
#define QLORA_MERGE_CASE(NP)                                                                  \
  case NP:                                                                                    \
    hipLaunchKernelGGL((nf4_merge_kernel<NP, kDQ, kF16>), grid, dim3(256), 0, stream, a);     \
    break;
    QLORA_MERGE_CASE(1) QLORA_MERGE_CASE(2) QLORA_MERGE_CASE(3) QLORA_MERGE_CASE(4)
    QLORA_MERGE_CASE(5) QLORA_MERGE_CASE(6) QLORA_MERGE_CASE(7) QLORA_MERGE_CASE(8)
#undef QLORA_MERGE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.dq && !a.f16) return merge_dispatch<true, false>(a, stream);
  if (a.dq) return merge_dispatch<true, true>(a, stream);
  if (!a.f16) return merge_dispatch<false, false>(a, stream);
  return merge_dispatch<false, true>(a, stream);
}

}  // namespace qlora
