// Merge of the LoRA adapter into the dequantised base (gfx950):
//
//   W_merged[n][k] = bf16( w_hat[n][k] + s * (B A)[n][k] ),  s = alpha / r,
//
// w_hat the bf16 dequantised weight, B [rows, r] and A [r, cols] bf16, the
// product accumulated in float32, scaled and added in float32, rounded once
// to bf16.  (Variants: fp16 in place of bf16 throughout, float32 block
// constants without double quantisation, the evenly spaced INT4 codebook.)
// (waylandz LLM book 26.2: at inference the adapter is folded into the
// weight once, W + (alpha/r) B A; ta-paperlens 落とし穴 and the Ultralytics
// QLoRA page, Kompromisse: the merge is done on the base dequantised to 16
// bit, and the result may be quantised again.)
//
// Bound by HBM: per weight it reads half a byte of codes and writes two bytes
// of bf16; the rank-r product (r multiply-adds per weight) runs on MFMA.
//
// Workgroup = 8 waves over a tile of 256 columns x 256 rows; wave w owns
// the 32-row block w.  Every load of the workgroup goes out at its start --
// the tile's 256-column slice of A (for LDS, row stride 576 bytes, so the
// transposed fragment reads below hit 64 distinct banks per 32 lanes), then
// each wave's B fragments, codes and block-constant inputs -- so the A
// slice's wait before the one workgroup barrier leaves the row loads in
// flight.  The codes arrive as whole 128-byte lines (8 lanes a row) and are
// redistributed through the wave's LDS tile.  All of a row block's loads
// complete before its first store, so no wait on a load ever waits on a
// store.
//
// A wave walks its 8 column sub-tiles of 32.  A sub-tile is one MFMA
// 32x32x16 chain over r with the A fragment first (8 consecutive r of one
// column, ds_read_b64_tr_b16) and the B fragment second (8 consecutive r of
// one row), so the float32 product lands with one weight row per lane pair:
// lane l and l + 32 hold row l % 32, columns 4 h + 8 g + [0, 4) (h = l / 32,
// g = 0..3).  Two v_permlane32_swap per accumulator quad regroup it so that
// lane l holds columns [0, 16) and lane l + 32 columns [16, 32) of its row:
// 16 consecutive weights of one block.  The block's 16-entry table q[k] * c'
// (rounded to 16 bit) is built by the lane pair in registers, 8 entries each,
// and looked up with byte permutes straight into float32 patterns; the next
// sub-tile's MFMA chain is issued before this one's VALU work.  The rounded
// results of two sub-tiles (32 rows x 64 columns) pass through the wave's
// LDS tile (16-byte chunks XOR-swizzled by row) and leave in whole 128-byte
// rows, 8 lanes a row: stores that cover a quarter line each ran 30% slower.
//
// Tiles are numbered so that the tiles one XCD receives (dispatch is
// round-robin over the 8 XCDs) walk down the rows of one column slice: the
// A slice is fetched once per XCD and column slice, and B (rows x r) stays
// in each XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kMergeCols = 256;   // columns per workgroup tile
constexpr int kMergeRows = 256;   // rows per workgroup tile
constexpr int kASlice = 288;      // A slice row stride in elements (256 + 32)
constexpr int kMergeWaves = 8;    // one 32-row block per wave

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ u32x4_t ld_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo);
  const uint2 h = __builtin_bit_cast(uint2, hi);
  return u32x4_t{l.x, l.y, h.x, h.y};
}

// Table of one row's block: the 16 entries q[k] * c' (float32 product, one
// rounding to the 16-bit type, as the bulk dequantiser) as byte planes for
// v_perm lookups.  Lanes l and l + 32 hold the same row and block: lane half
// h forms entries 8h .. 8h+7 (kq = those levels) and the halves are
// exchanged with v_permlane32_swap.
template <bool kF16>
__device__ __forceinline__ Nf4Lut merge_lut(float cp, const float kq[8]) {
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pack16x2<kF16>(__fmul_rn(kq[2 * j], cp), __fmul_rn(kq[2 * j + 1], cp));
  const uint32_t lo_a = perm(p[1], p[0], 0x06040200u);
  const uint32_t lo_b = perm(p[3], p[2], 0x06040200u);
  const uint32_t hi_a = perm(p[1], p[0], 0x07050301u);
  const uint32_t hi_b = perm(p[3], p[2], 0x07050301u);
  // permlane32_swap(x, x): first result = lower half's x in every lane,
  // second = upper half's x in every lane
  const auto sa = __builtin_amdgcn_permlane32_swap(lo_a, lo_a, false, false);
  const auto sb = __builtin_amdgcn_permlane32_swap(lo_b, lo_b, false, false);
  const auto sc = __builtin_amdgcn_permlane32_swap(hi_a, hi_a, false, false);
  const auto sd = __builtin_amdgcn_permlane32_swap(hi_b, hi_b, false, false);
  Nf4Lut t;
  t.lo[0] = sa[0];
  t.lo[1] = sb[0];
  t.lo[2] = sa[1];
  t.lo[3] = sb[1];
  t.hi[0] = sc[0];
  t.hi[1] = sd[0];
  t.hi[2] = sc[1];
  t.hi[3] = sd[1];
  return t;
}

// The 8 codes of word w (element i in bits 4i..4i+3) as the float32 values
// of their 16-bit table entries.  bf16: the entry's two bytes become the
// upper half of the float32 pattern (v_perm selector 0x0C gives a zero
// byte); fp16: the 16-bit pattern is converted.
template <bool kF16>
__device__ __forceinline__ void dequant8_f32(const Nf4Lut& t, uint32_t w, float out[8]) {
  uint32_t elo, ehi, olo, ohi;
  lut4(t, w & 0x0F0F0F0Fu, elo, ehi);           // elements 0, 2, 4, 6
  lut4(t, (w >> 4) & 0x0F0F0F0Fu, olo, ohi);    // elements 1, 3, 5, 7
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!kF16) {
      const uint32_t sel = ((4u + j) << 24) | ((uint32_t)j << 16) | 0x0C0Cu;
      out[2 * j] = __uint_as_float(perm(ehi, elo, sel));
      out[2 * j + 1] = __uint_as_float(perm(ohi, olo, sel));
    } else {
      const uint32_t sel = 0x0C0C0000u | ((4u + j) << 8) | (uint32_t)j;
      out[2 * j] = lo16_to_f32<true>(perm(ehi, elo, sel));
      out[2 * j + 1] = lo16_to_f32<true>(perm(ohi, olo, sel));
    }
  }
}

// Block-constant inputs of one lane's row for the tile's 4 blocks (256
// columns).  Row and column are clamped into the weight, so every load is
// unconditional; values of clamped rows or blocks are never stored.
struct MergeConsts {
  uint32_t c8[4];   // 8-bit constant code of block b
  float s2[4];      // its group scale (float32 block constant without DQ)
};

// With double quantisation the tile's 4 blocks of a row are consecutive
// blocks blk0 .. blk0 + 3: their 8-bit codes are 4 consecutive bytes, read
// as the (at most) two aligned words that hold them, and they span at most
// two groups, so two scale loads serve all four (4 loads instead of 8).  The
// code array is 16-byte aligned and n_b (rows a multiple of 16) a multiple
// of 16, so every aligned word below n_b lies inside it; blocks past the row
// read the next row's bytes and feed only columns that are never stored.
template <bool kDQ>
__device__ __forceinline__ void merge_const_loads(const MergeArgs& a, int64_t nc, int64_t k0,
                                                  MergeConsts& m) {
  if (kDQ) {
    const int64_t n_b = (a.rows * a.cols) >> 6;
    const int64_t blk0 = (nc * a.cols + k0) >> 6;
    const int64_t w0 = blk0 & ~(int64_t)3;
    const int64_t w1 = w0 + 4 < n_b ? w0 + 4 : w0;
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(a.code8 + w0);
    const uint32_t hi = *reinterpret_cast<const uint32_t*>(a.code8 + w1);
    const uint32_t bytes = __builtin_amdgcn_alignbyte(hi, lo, (uint32_t)(blk0 & 3));
    const int64_t g0 = blk0 >> 8;
    const int64_t g1 = (blk0 + 3 < n_b ? blk0 + 3 : n_b - 1) >> 8;
    const float s2a = a.s2[g0];
    const float s2b = a.s2[g1];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      m.c8[b] = (bytes >> (8 * b)) & 0xFFu;
      m.s2[b] = ((blk0 + b) >> 8) == g0 ? s2a : s2b;
    }
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int64_t col = k0 + 64 * b;
      col = col < a.cols ? col : a.cols - 64;
      m.c8[b] = 0u;
      m.s2[b] = a.s2[(nc * a.cols + col) >> 6];
    }
  }
}

// Byte offset of the 8-byte code piece (chunk c = tile columns 32 c .. +32,
// half h) of row `row` in a wave's staging tile of a row block's codes
// (32 rows x 128 bytes): chunks XOR-swizzled by row bits 1..3 and halves by
// row bit 4, so 32 lanes reading one chunk of 32 rows hit 64 distinct banks
// and 8 lanes writing one row's 8 chunks hit distinct banks.
__device__ __forceinline__ int code_slot(int row, int c, int h) {
  return row * 128 + ((c ^ ((row >> 1) & 7)) << 4) + ((h ^ ((row >> 4) & 1)) << 3);
}

}  // namespace

// Loads of one wave's 32-row block: B fragments, the codes as whole lines
// (chunk c = tile columns 32 c .. +32 of rows 8 it + lane / 8) and the block
// constant inputs.  Rows and columns are clamped into the weight; values of
// clamped rows and columns are never stored.
template <int NP>
struct MergeRowIn {
  u32x4_t bf[NP];
  u32x4_t cc[4];
  MergeConsts m;
};

template <int NP, bool kDQ>
__device__ __forceinline__ void merge_row_issue(const MergeArgs& a, int64_t n0, int64_t k0,
                                                int lane, MergeRowIn<NP>& in) {
  const int l32 = lane & 31, lhi = lane >> 5;
  const int64_t n = n0 + l32;
  const int64_t nc = n < a.rows ? n : a.rows - 1;
#pragma unroll
  for (int j = 0; j < NP; ++j)
    in.bf[j] = *reinterpret_cast<const u32x4_t*>(a.B + nc * (16 * NP) + 16 * j + 8 * lhi);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int64_t gn = n0 + 8 * it + (lane >> 3);
    gn = gn < a.rows ? gn : a.rows - 1;
    int64_t col = k0 + 32 * (lane & 7);
    col = col < a.cols ? col : a.cols - 32;
    in.cc[it] = *reinterpret_cast<const u32x4_t*>(a.codes + ((gn * a.cols + col) >> 1));
  }
  merge_const_loads<kDQ>(a, nc, k0, in.m);
}

// One 32-row block: the 8 sub-tiles of 32 columns, each an MFMA chain over r
// for s * (B A), the table lookups and the add, out through the wave's
// staging tile.
template <int NP, bool kDQ, bool kF16>
__device__ __forceinline__ void merge_row_process(const MergeArgs& a, const uint16_t* as,
                                                  uint16_t* stg, int64_t n0, int64_t k0,
                                                  int lane, float mu, const float kq[8],
                                                  const MergeRowIn<NP>& in) {
  const int l32 = lane & 31, lhi = lane >> 5;
  // A fragment of sub-tile s, slice j: rows 16 j + prow (+4), column 32 s + acol
  const int prow = 8 * lhi + ((lane & 15) >> 2);
  const int acol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // the codes through the staging tile into 8 bytes per lane and sub-tile
  // (the wave reads only what it wrote, and its LDS operations complete in
  // order: no barrier); rows 16..31 (it >= 2) store their halves swapped
  uint2 cw[8];
  {
    unsigned char* sb = reinterpret_cast<unsigned char*>(stg);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = 8 * it + (lane >> 3);
      const u32x4_t v = in.cc[it];
      const u32x4_t w = it >= 2 ? u32x4_t{v[2], v[3], v[0], v[1]} : v;
      *reinterpret_cast<u32x4_t*>(sb + code_slot(row, lane & 7, 0) - (((row >> 4) & 1) << 3)) = w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      cw[st] = *reinterpret_cast<const uint2*>(sb + code_slot(l32, st, lhi));
  }
  float cps[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    cps[b] = kDQ ? block_constant(in.m.c8[b], in.m.s2[b], mu) : in.m.s2[b];
  // forced here: every load of the row block completes before its first
  // store, so no later wait on a load also waits on stores
  asm volatile("" ::"v"(cps[0]), "v"(cps[1]), "v"(cps[2]), "v"(cps[3]));
  auto product = [&](int st) {
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const uint16_t* p = as + (16 * j + prow) * kASlice + 32 * st + acol;
      acc = mfma32x32<kF16>(ld_tr_pair(p, p + 4 * kASlice), in.bf[j], acc);
    }
    return acc;
  };
  f32x16_t acc_next = product(0);
  Nf4Lut lut;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    // the next sub-tile's MFMAs run while this one's VALU work issues
    const f32x16_t acc = acc_next;
    if (s < 7) acc_next = product(s + 1);
    // acc[4 g + e]: row l32, column 8 g + 4 lhi + e.  After the swaps v[i]
    // is column 16 lhi + i.
    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]),
                                                      __float_as_uint(acc[8 + e]), false, false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[4 + e]),
                                                      __float_as_uint(acc[12 + e]), false, false);
      v[e] = __uint_as_float(x[0]);
      v[4 + e] = __uint_as_float(x[1]);
      v[8 + e] = __uint_as_float(y[0]);
      v[12 + e] = __uint_as_float(y[1]);
    }
    // sub-tiles 2b and 2b + 1 of a row share block b
    if ((s & 1) == 0) lut = merge_lut<kF16>(cps[s >> 1], kq);
    const uint32_t words[2] = {cw[s].x, cw[s].y};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float base[8];
      dequant8_f32<kF16>(lut, words[w], base);
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * w + 2 * e;
        o[e] = pack16x2<kF16>(__fadd_rn(base[2 * e], __fmul_rn(v[i], a.scale)),
                              __fadd_rn(base[2 * e + 1], __fmul_rn(v[i + 1], a.scale)));
      }
      // 16-byte chunk 4 (s & 1) + 2 lhi + w of this row in the staging tile
      const int ch = 4 * (s & 1) + 2 * lhi + w;
      *reinterpret_cast<u32x4_t*>(stg + l32 * 64 + ((ch ^ (l32 & 7)) << 3)) = o;
    }
    if (s & 1) {
      // the pair of sub-tiles (64 columns) back out in whole 128-byte rows:
      // 8 lanes per row, 8 rows per store
      const int ch = lane & 7;
      const int64_t col = k0 + 32 * (s - 1) + 8 * ch;
      u32x4_t o[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = 8 * it + (lane >> 3);
        o[it] = *reinterpret_cast<const u32x4_t*>(stg + row * 64 + ((ch ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int64_t gn = n0 + 8 * it + (lane >> 3);
        if (gn < a.rows && col < a.cols)
          *reinterpret_cast<u32x4_t*>(a.out + gn * a.cols + col) = o[it];
      }
    }
  }
}

template <int NP, bool kDQ, bool kF16>
__global__ __launch_bounds__(64 * kMergeWaves) void nf4_merge_kernel(MergeArgs a, int n_ct, int n_rt) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int R = 16 * NP;
  __shared__ __attribute__((aligned(16))) uint16_t as[R * kASlice];
  __shared__ __attribute__((aligned(16))) uint16_t stage[kMergeWaves][32 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* stg = stage[wave];   // this wave's 32 x 64 staging tile

  // tile: XCD-major, then down the rows of one column slice
  const int pid = blockIdx.x;
  const int total = n_ct * n_rt;
  const int xcd = pid & 7;
  const int base = total >> 3, rem = total & 7;
  const int qi = __builtin_amdgcn_readfirstlane(xcd * base + (xcd < rem ? xcd : rem) + (pid >> 3));
  const int ct = qi / n_rt;
  const int rt = qi - ct * n_rt;
  const int64_t k0 = (int64_t)ct * kMergeCols;
  const int64_t nb = (int64_t)rt * kMergeRows;

  // the A slice first (columns past the weight read a clamped column and
  // only feed sub-tiles that are never stored), then the row block's loads:
  // the A slice's wait leaves them in flight
  // levels 8 lhi .. 8 lhi + 7 of the codebook (uniform loads of both halves,
  // so no vector load of them waits behind the row loads)
  float kq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float lo = a.qt ? kINT4[j] : kNF4[j];
    const float hi = a.qt ? kINT4[8 + j] : kNF4[8 + j];
    kq[j] = (lane >> 5) ? hi : lo;
  }
  constexpr int kAIters = R * 32 / (64 * kMergeWaves);
  u32x4_t av[kAIters];
#pragma unroll
  for (int t = 0; t < kAIters; ++t) {
    const int i = tid + t * 64 * kMergeWaves;
    const int64_t k = k0 + 8 * (i & 31) < a.cols ? k0 + 8 * (i & 31) : a.cols - 8;
    av[t] = *reinterpret_cast<const u32x4_t*>(a.A + (int64_t)(i >> 5) * a.cols + k);
  }
  MergeRowIn<NP> in0;
  merge_row_issue<NP, kDQ>(a, nb + 32 * wave, k0, lane, in0);
#pragma unroll
  for (int t = 0; t < kAIters; ++t) {
    const int i = tid + t * 64 * kMergeWaves;
    *reinterpret_cast<u32x4_t*>(as + (i >> 5) * kASlice + 8 * (i & 31)) = av[t];
  }
  const float mu = kDQ ? a.mu[0] : 0.0f;
  __syncthreads();   // A slice visible
  if (nb + 32 * wave < a.rows)
    merge_row_process<NP, kDQ, kF16>(a, as, stg, nb + 32 * wave, k0, lane, mu, kq, in0);
#endif
}

template <bool kDQ, bool kF16>
static hipError_t merge_dispatch(const MergeArgs& a, hipStream_t stream) {
  const int n_ct = (int)((a.cols + kMergeCols - 1) / kMergeCols);
  const int n_rt = (int)((a.rows + kMergeRows - 1) / kMergeRows);
  const dim3 grid((unsigned)n_ct * (unsigned)n_rt);
  switch (a.r >> 4) {
#define QLORA_MERGE_CASE(NP)                                                                  \
  case NP:                                                                                    \
    hipLaunchKernelGGL((nf4_merge_kernel<NP, kDQ, kF16>), grid, dim3(64 * kMergeWaves), 0, stream, a,      \
                       n_ct, n_rt);                                                           \
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
