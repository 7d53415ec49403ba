// Skinny forward of the QLoRA linear layer for few tokens (T <= 64):
//   Y = X dequant(W)^T + s (X A^T) B^T,   U = X A^T.
// ta-paperlens 落とし穴: the 4-bit format pays off in generation with small
// batches, which is bound by how many weight bytes are read.  Here every
// weight meets at most 64 tokens, so the kernels are built to read the packed
// weight once (0.516 B per weight with its constants) and to dequantise each
// weight exactly once, in registers.  Two launches:
//
// 1. qlora_gemv_partial_kernel.  A workgroup of 4 waves owns 64 output rows
//    and one split of the reduction; the waves take the 64-wide blocks of that
//    split in turn (wave w: blocks w, w+4, ...), so together they stream 128
//    contiguous bytes of every weight row.  The row tiles past the weight's
//    rows are the r rows of the LoRA factor A, read as plain bf16: U = X A^T
//    is formed by the same launch as X dequant(W)^T.
//    Each wave computes C[token][row] for 32 (or 64) tokens x 64 rows with
//    MFMA 32x32x16: the weight is the B operand (lane l holds row l % 32 of a
//    32-row group and half l / 32 of the block: 32 codes = 16 bytes), the
//    activations are the A operand (lane l: token l % 32, same half).  Inside
//    one MFMA the pairing of reduction indices with operand slots is free as
//    long as both operands agree, so the weights are produced in the order
//    the byte lookups give them -- elements (0,2,4,6,1,3,5,7) of each code
//    word -- and the activations are permuted to that order (4 byte permutes
//    per 8 activations, shared by both row groups).
//    Dequantisation: c' is decoded from the 8-bit code (hardware FP8
//    conversion) and the group's scale and offset; the 16-entry bf16 table
//    q[k] * c' (float32 product, one rounding, as the bulk dequantiser) is
//    built half by half -- the two lanes that share a row each form 8
//    entries and exchange them with v_permlane32_swap -- and nibbles are
//    translated with byte permutes.  The four waves' float32 tiles are added
//    in LDS in a fixed order and stored as one split partial.
// 2. qlora_gemv_finish_kernel.  U = sum of the A-tile partials (fixed order),
//    stored as bf16 and, scaled by s, kept in LDS as bf16; the LoRA term
//    (s U) B^T comes from MFMA 32x32x16 and Y = bf16(sum_s P + LoRA).  B and
//    the first batch of W partials are requested before U's partials, so
//    the kernel waits for one round trip where it waited for three.
#include "abi_internal.h"
#include "device_common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr uint32_t kOOBv = 0x80000000u;   // offset past every descriptor range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_v(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0ull : bytes),
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <bool kF16>
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b,
                                           const f32x16_t& c) {
  return mfma32x32<kF16>(a, b, c);
}

// 8 codes of one word (element i in bits 4i..4i+3) to bf16, slot order
// (e0,e2 | e4,e6 | e1,e3 | e5,e7).
__device__ __forceinline__ u32x4_t dequant8_eo(const Nf4Lut& t, uint32_t w) {
  uint32_t elo, ehi, olo, ohi;
  lut4(t, w & 0x0F0F0F0Fu, elo, ehi);
  lut4(t, (w >> 4) & 0x0F0F0F0Fu, olo, ohi);
  u32x4_t o;
  o[0] = perm(ehi, elo, 0x05010400u);
  o[1] = perm(ehi, elo, 0x07030602u);
  o[2] = perm(ohi, olo, 0x05010400u);
  o[3] = perm(ohi, olo, 0x07030602u);
  return o;
}

// 8 consecutive bf16 values to the same slot order.
__device__ __forceinline__ u32x4_t act_eo(const u32x4_t& d) {
  u32x4_t o;
  o[0] = perm(d[1], d[0], 0x05040100u);
  o[1] = perm(d[3], d[2], 0x05040100u);
  o[2] = perm(d[1], d[0], 0x07060302u);
  o[3] = perm(d[3], d[2], 0x07060302u);
  return o;
}

// Table of one row's block, lanes l and l + 32 holding the same c': lane half
// h forms entries 8h .. 8h+7 (kq = the levels 8h .. 8h+7) as byte planes and
// the halves are exchanged.
template <bool kF16>
__device__ __forceinline__ Nf4Lut make_lut_pair(float cp, const float kq[8]) {
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pack16x2<kF16>(__fmul_rn(kq[2 * j], cp), __fmul_rn(kq[2 * j + 1], cp));
  const uint32_t lo_a = perm(p[1], p[0], 0x06040200u);
  const uint32_t lo_b = perm(p[3], p[2], 0x06040200u);
  const uint32_t hi_a = perm(p[1], p[0], 0x07050301u);
  const uint32_t hi_b = perm(p[3], p[2], 0x07050301u);
  // permlane32_swap(x, x): first result = lower half's x in every lane,
  // second = upper half's x in every lane.
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

template <int TG, bool kLora>
struct GemvStage {
  u32x4_t w[2][kLora ? 4 : 1];   // NF4: 16 code bytes per row group; A: 32 bf16
  // block-constant inputs of row group `half` (lanes l and l + 32 hold the
  // same row of each group, so each half loads one group's and the two
  // halves exchange them)
  uint32_t c8;
  float s2;
  u32x4_t x[TG][4];              // 32 activations per token group
};

// acc[tg][ng] += X[tokens of tg][k] * Wrow[ng][k] over the blocks st0 + wave,
// st0 + wave + 4, ... below st1.
template <int TG, bool kLora, bool kDQ, bool kF16>
__device__ __forceinline__ void gemv_tile(const GemvArgs& g, int64_t n0, int64_t st0,
                                          int64_t st1, int wave, int lane,
                                          f32x16_t (&acc)[TG][2]) {
  const int half = lane >> 5;
  const int64_t K = g.cols;
  const int64_t kblocks = K >> 6;
  const int64_t nrows = kLora ? g.r : g.rows;
  const __amdgpu_buffer_rsrc_t xr = rsrc_v(g.X, (uint64_t)g.T * K * 2);
  const __amdgpu_buffer_rsrc_t wr =
      kLora ? rsrc_v(g.A, (uint64_t)g.r * K * 2) : rsrc_v(g.codes, (uint64_t)(g.rows * K) >> 1);
  const __amdgpu_buffer_rsrc_t c8r = rsrc_v(g.code8, (uint64_t)(g.rows * kblocks));
  // without double quantisation the group-scale slot holds each block's
  // float32 constant and there is no 8-bit code to load
  const __amdgpu_buffer_rsrc_t s2r =
      rsrc_v(g.s2, kDQ ? (uint64_t)((g.rows * kblocks + 255) >> 8) * 4
                       : (uint64_t)(g.rows * kblocks) * 4);
  const float mu = (kLora || !kDQ) ? 0.0f : g.mu[0];

  bool row_ok[2];
  int64_t row[2];
#pragma unroll
  for (int ng = 0; ng < 2; ++ng) {
    row[ng] = n0 + 32 * ng + (lane & 31);
    row_ok[ng] = row[ng] < nrows;
  }
  bool tok_ok[TG];
  int64_t xbase[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int64_t t = 32 * tg + (lane & 31);
    tok_ok[tg] = t < g.T;
    xbase[tg] = (t * K + 32 * half) * 2;
  }
  float kq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kq[j] = half ? kNF4[8 + j] : kNF4[j];

  auto load = [&](int64_t st, bool ok, GemvStage<TG, kLora>& s) {
#pragma unroll
    for (int ng = 0; ng < 2; ++ng) {
      const bool v = ok && row_ok[ng];
      if (kLora) {
        const uint32_t off = v ? (uint32_t)((row[ng] * K + st * 64 + 32 * half) * 2) : kOOBv;
#pragma unroll
        for (int q = 0; q < (kLora ? 4 : 1); ++q) s.w[ng][q] = load16(wr, off + 16 * q);
      } else {
        const int64_t blk = row[ng] * kblocks + st;
        s.w[ng][0] = load16(wr, v ? (uint32_t)(blk * 32 + 16 * half) : kOOBv);
      }
    }
    if (!kLora) {
      const bool v = ok && row_ok[half];
      const int64_t blk = row[half] * kblocks + st;
      if (kDQ)
        s.c8 = __builtin_amdgcn_raw_buffer_load_b8(c8r, v ? (uint32_t)blk : kOOBv, 0, 0);
      else
        s.c8 = 0u;
      s.s2 = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(s2r, v ? scale_offset<kDQ>(blk) : kOOBv,
                                                      0, 0));
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const uint32_t off = (ok && tok_ok[tg]) ? (uint32_t)(xbase[tg] + st * 128) : kOOBv;
#pragma unroll
      for (int q = 0; q < 4; ++q) s.x[tg][q] = load16(xr, off + 16 * q);
    }
  };

  GemvStage<TG, kLora> cur, nxt;
  int64_t st = st0 + wave;
  load(st, st < st1, cur);
  for (; st < st1; st += 4) {
    load(st + 4, st + 4 < st1, nxt);
    // priority 1 while this block is dequantised and multiplied, 0 while
    // the wave waits for the next one's loads: a wave whose data has
    // arrived issues ahead of one still waiting (-2.5% on the 65B decode
    // block, same bits)
    __builtin_amdgcn_s_setprio(1);
    u32x4_t a[TG][4];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[tg][q] = act_eo(cur.x[tg][q]);
    // the block-constant inputs of both row groups: [0] from the lower
    // half's lanes, [1] from the upper half's
    uint32_t c8[2] = {0u, 0u};
    float s2v[2] = {0.0f, 0.0f};
    if (!kLora) {
      const auto cx = __builtin_amdgcn_permlane32_swap(cur.c8, cur.c8, false, false);
      const auto sx = __builtin_amdgcn_permlane32_swap(__float_as_uint(cur.s2),
                                                       __float_as_uint(cur.s2), false, false);
      c8[0] = cx[0];
      c8[1] = cx[1];
      s2v[0] = __uint_as_float(sx[0]);
      s2v[1] = __uint_as_float(sx[1]);
    }
#pragma unroll
    for (int ng = 0; ng < 2; ++ng) {
      if (kLora) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4_t b = act_eo(cur.w[ng][kLora ? q : 0]);
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) acc[tg][ng] = mfma32<kF16>(a[tg][q], b, acc[tg][ng]);
        }
      } else {
        const float cp = weight_constant_or_zero<kDQ>(row_ok[ng], c8[ng], s2v[ng], mu);
        const Nf4Lut lt = make_lut_pair<kF16>(cp, kq);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4_t b = dequant8_eo(lt, cur.w[ng][0][q]);
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) acc[tg][ng] = mfma32<kF16>(a[tg][q], b, acc[tg][ng]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    cur = nxt;
  }
}

}  // namespace

// Grid: (w_tiles + LoRA tiles, splits); TG = token groups of 32.
template <int TG, bool kDQ, bool kF16>
__global__ __launch_bounds__(256) void qlora_gemv_partial_kernel(GemvArgs g, int w_tiles,
                                                                 int steps_per) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) float red[3 * TG * 2 * 16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t kblocks = g.cols >> 6;
  const bool lora = (int)blockIdx.x >= w_tiles;
  const int64_t n0 = (int64_t)(lora ? (int)blockIdx.x - w_tiles : (int)blockIdx.x) * 64;
  const int64_t nrows = lora ? g.r : g.rows;
  const int64_t st0 = (int64_t)blockIdx.y * steps_per;
  const int64_t st1 = st0 + steps_per < kblocks ? st0 + steps_per : kblocks;

  f32x16_t acc[TG][2];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int ng = 0; ng < 2; ++ng)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tg][ng][e] = 0.0f;
  if (lora)
    gemv_tile<TG, true, kDQ, kF16>(g, n0, st0, st1, wave, lane, acc);
  else
    gemv_tile<TG, false, kDQ, kF16>(g, n0, st0, st1, wave, lane, acc);

  // ---- fixed-order sum of the four waves' tiles, one split partial -------
  if (wave > 0) {
    float* dst = red + (wave - 1) * (TG * 2 * 16 * 64);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int ng = 0; ng < 2; ++ng)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[((tg * 2 + ng) * 16 + e) * 64 + lane] = acc[tg][ng][e];
  }
  __syncthreads();
  if (wave == 0) {
    float* out = (lora ? g.PU : g.P) + (int64_t)blockIdx.y * g.T * nrows;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int ng = 0; ng < 2; ++ng) {
        const int64_t n = n0 + 32 * ng + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int idx = ((tg * 2 + ng) * 16 + e) * 64 + lane;
          float v = acc[tg][ng][e];
          v += red[idx];
          v += red[TG * 2 * 16 * 64 + idx];
          v += red[2 * TG * 2 * 16 * 64 + idx];
          const int64_t t = 32 * tg + 8 * (e >> 2) + 4 * half + (e & 3);
          if (t < g.T && n < nrows) out[t * nrows + n] = v;
        }
      }
  }
#endif
}

// Grid: ceil(rows / 128); wave w owns rows 128 blockIdx.x + 32 w .. + 31.
// kHalf (T <= 16): only MFMA output rows 0..15 hold tokens, so only the
// accumulator entries e < 8 are loaded and stored.  The LoRA operand B and
// the first kBatch split partials are requested before U is reduced, so the
// three independent load chains share one round trip.
template <int TG, bool kF16, bool kHalf>
__global__ __launch_bounds__(256) void qlora_gemv_finish_kernel(GemvArgs g) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kE = kHalf ? 8 : 16;                          // accumulator entries in use
  // splits per batch of W-partial and U-partial loads (16 at once with
  // T <= 16 measured 1% slower on the 65B decode block than 8)
  constexpr int kBatch = kHalf ? 8 : (TG == 1 ? 4 : 1);
  constexpr int kUBatch = 8;
  __shared__ __attribute__((aligned(16))) uint16_t us[64 * 128];   // bf16(s U) [t][p]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t N = g.rows, T = g.T;
  const int r = g.r;
  const int splits = g.splits;
  const int64_t n = (int64_t)blockIdx.x * 128 + 32 * wave + (lane & 31);

  // ---- requests that do not depend on U: B fragments, first partials -----
  const __amdgpu_buffer_rsrc_t br = rsrc_v(g.B, (uint64_t)N * r * 2);
  u32x4_t bfr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    bfr[j] = 16 * j < r ? load16(br, n < N ? (uint32_t)((n * r + 16 * j + 8 * half) * 2) : kOOBv)
                        : u32x4_t{0u, 0u, 0u, 0u};
  // rows past T are read from row T - 1 (loads stay unconditional) and
  // never stored; rows past N read row N - 1
  const int64_t nc = n < N ? n : N - 1;
  int64_t off[TG][kE];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t t = 32 * tg + 8 * (e >> 2) + 4 * half + (e & 3);
      off[tg][e] = (t < T ? t : T - 1) * N + nc;
    }
  float v[TG][kE];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int e = 0; e < kE; ++e) v[tg][e] = 0.0f;
  auto load_batch = [&](int s0, float (&x)[kBatch][TG][kE]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sc = s0 + i < splits ? s0 + i : splits - 1;
      const float* ps = g.P + (int64_t)sc * T * N;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int e = 0; e < kE; ++e) x[i][tg][e] = ps[off[tg][e]];
    }
  };
  // splits past the end read the last split and add 0 (the same sums, in
  // split order, as one pass over all splits)
  auto add_batch = [&](int s0, const float (&x)[kBatch][TG][kE]) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int e = 0; e < kE; ++e) v[tg][e] += s0 + i < splits ? x[i][tg][e] : 0.0f;
  };
  float x0[kBatch][TG][kE];
  load_batch(0, x0);

  // ---- U = sum over splits of the A-tile partials (fixed order) -----------
  // 4 entries per thread and round, kUBatch splits per batch of loads;
  // splits past the end read the last split and add 0.
  const int64_t TR = T * r;
  for (int64_t e0 = 0; e0 < TR; e0 += 1024) {
    int64_t ei[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ei[j] = e0 + tid + 256 * j;
      if (ei[j] >= TR) ei[j] = TR - 1;
    }
    float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < splits; s0 += kUBatch) {
      float x[kUBatch][4];
#pragma unroll
      for (int i = 0; i < kUBatch; ++i) {
        const int sc = s0 + i < splits ? s0 + i : splits - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[i][j] = g.PU[(int64_t)sc * TR + ei[j]];
      }
#pragma unroll
      for (int i = 0; i < kUBatch; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] += s0 + i < splits ? x[i][j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e = e0 + tid + 256 * j;
      if (e < TR) {
        us[e] = (uint16_t)(pack16x2<kF16>(u[j] * g.scale, 0.0f) & 0xFFFFu);
        if (blockIdx.x == 0 && g.U_save)
          g.U_save[e] = (uint16_t)(pack16x2<kF16>(u[j], 0.0f) & 0xFFFFu);
      }
    }
  }
  __syncthreads();

  // ---- LoRA term (s U) B^T by MFMA -------------------------------------------
  f32x16_t acc[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[tg][e] = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (16 * j < r) {
      const int p = 16 * j + 8 * half;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        // token rows past T read stale table entries; they only reach output
        // rows that are never stored
        const int t = 32 * tg + (lane & 31);
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(us + t * r + p);
        acc[tg] = mfma32<kF16>(a, bfr[j], acc[tg]);
      }
    }
  }

  // ---- the W partials, then Y = bf16(sum_s P + LoRA) -------------------------
  add_batch(0, x0);
  for (int s0 = kBatch; s0 < splits; s0 += kBatch) {
    float x[kBatch][TG][kE];
    load_batch(s0, x);
    add_batch(s0, x);
  }
  if (n >= N) return;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t t = 32 * tg + 8 * (e >> 2) + 4 * half + (e & 3);
      if (t < T) g.Y[t * N + n] = (uint16_t)(pack16x2<kF16>(v[tg][e] + acc[tg][e], 0.0f) & 0xFFFFu);
    }
#endif
}

template <int TG, bool kDQ, bool kF16>
static hipError_t gemv_launch(const GemvArgs& a, dim3 grid, dim3 fgrid, int w_tiles, int per,
                              hipStream_t stream) {
  hipLaunchKernelGGL((qlora_gemv_partial_kernel<TG, kDQ, kF16>), grid, dim3(256), 0, stream, a,
                     w_tiles, per);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool half_rows = false;
  if constexpr (TG == 1) half_rows = a.T <= 16;
  if constexpr (TG == 1) {
    if (half_rows)
      hipLaunchKernelGGL((qlora_gemv_finish_kernel<1, kF16, true>), fgrid, dim3(256), 0, stream,
                         a);
  }
  if (!half_rows)
    hipLaunchKernelGGL((qlora_gemv_finish_kernel<TG, kF16, false>), fgrid, dim3(256), 0, stream,
                       a);
  return hipGetLastError();
}

hipError_t launch_qlora_gemv(const GemvArgs& a, hipStream_t stream) {
  const int64_t kblocks = a.cols / 64;
  if (a.T < 1 || a.T > kGemvMaxTokens || a.splits < 1 || a.splits > kblocks || a.r < 16 ||
      a.r > 128)
    return hipErrorInvalidValue;
  const int per = (int)((kblocks + a.splits - 1) / a.splits);
  const int w_tiles = (int)((a.rows + 63) / 64);
  const int l_tiles = (a.r + 63) / 64;
  const dim3 grid((unsigned)(w_tiles + l_tiles), (unsigned)a.splits);
  const dim3 fgrid((unsigned)((a.rows + 127) / 128));
  if (a.T <= 32) {
    if (a.dq && !a.f16) return gemv_launch<1, true, false>(a, grid, fgrid, w_tiles, per, stream);
    if (a.dq) return gemv_launch<1, true, true>(a, grid, fgrid, w_tiles, per, stream);
    if (!a.f16) return gemv_launch<1, false, false>(a, grid, fgrid, w_tiles, per, stream);
    return gemv_launch<1, false, true>(a, grid, fgrid, w_tiles, per, stream);
  }
  if (a.dq && !a.f16) return gemv_launch<2, true, false>(a, grid, fgrid, w_tiles, per, stream);
  if (a.dq) return gemv_launch<2, true, true>(a, grid, fgrid, w_tiles, per, stream);
  if (!a.f16) return gemv_launch<2, false, false>(a, grid, fgrid, w_tiles, per, stream);
  return gemv_launch<2, false, true>(a, grid, fgrid, w_tiles, per, stream);
}

}  // namespace qlora
