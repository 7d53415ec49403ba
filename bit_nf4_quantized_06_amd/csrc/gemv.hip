// Skinny forward of the QLoRA linear layer for few tokens (T <= 64):
//   Y = X dequant(W)^T + (s X A^T) B^T.
// ta-paperlens 落とし穴: the 4-bit format pays off in generation with small
// batches, which is bound by how many weight bytes are read.  Here every
// weight meets at most 64 tokens, so the kernel is built to read the packed
// weight once (0.516 B per weight with its constants) and to dequantise each
// weight exactly once, in registers.
//
// Mapping.  A workgroup of 4 waves owns 64 weight rows and one split of the
// reduction; the waves take the 64-wide NF4 blocks of that split in turn
// (wave w: blocks w, w+4, ...), so together they stream 128 contiguous bytes
// of every row.  Each wave computes C[token][row] for 32 (or 64) tokens x 64
// rows with MFMA 32x32x16: the weight is the B operand (lane l holds row
// l % 32 of the row group and half l / 32 of the block, i.e. 32 codes = 16
// bytes), the activations are the A operand (lane l holds token l % 32, the
// same half of the block).  Inside one MFMA the pairing of reduction indices
// with operand slots is free as long as both operands agree, so the weights
// are produced in the order the byte lookups give them -- elements
// (0,2,4,6,1,3,5,7) of each code word -- and the activations are permuted
// to that order instead (4 byte permutes per 8 activations, shared by both
// row groups).
//
// Dequantisation: for its row and block a lane decodes c' from the 8-bit code
// and the group's scale and offset, forms the 16-entry bf16 table q[k] * c'
// (float32 product, one rounding, as the bulk dequantiser) and translates
// nibbles with byte permutes; no dequantised tile is stored anywhere.
//
// The LoRA term (s U) B^T seeds the accumulators of the first split (one
// more MFMA chain).  The four waves' float32 partial tiles are summed in LDS
// in a fixed order and written as one split partial; a finishing kernel adds
// the splits in order and rounds once to bf16 (a single split is rounded and
// stored directly).
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

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b,
                                           const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
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

// 8 consecutive bf16 activations to the same slot order.
__device__ __forceinline__ u32x4_t act_eo(const u32x4_t& d) {
  u32x4_t o;
  o[0] = perm(d[1], d[0], 0x05040100u);
  o[1] = perm(d[3], d[2], 0x05040100u);
  o[2] = perm(d[1], d[0], 0x07060302u);
  o[3] = perm(d[3], d[2], 0x07060302u);
  return o;
}

template <int TG>
struct GemvStage {
  u32x4_t code[2];       // 16 bytes of codes per row group
  u32x4_t x[TG][4];      // 32 activations per token group
  uint32_t c8[2];
  float s2[2];
};

}  // namespace

// TG = token groups of 32 (T <= 32 TG).  Grid: (ceil(rows / 64), splits).
template <int TG>
__global__ __launch_bounds__(256) void qlora_gemv_partial_kernel(GemmArgs g, int steps_per,
                                                                 float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) float red[3 * TG * 2 * 16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int64_t N = g.rows, K = g.cols;
  const int64_t kblocks = K >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t st0 = (int64_t)blockIdx.y * steps_per;
  const int64_t st1 = st0 + steps_per < kblocks ? st0 + steps_per : kblocks;
  const float mu = g.mu[0];

  const __amdgpu_buffer_rsrc_t xr = rsrc_v(g.act, (uint64_t)g.T * K * 2);
  const __amdgpu_buffer_rsrc_t cr = rsrc_v(g.codes, (uint64_t)(N * K) >> 1);
  const __amdgpu_buffer_rsrc_t c8r = rsrc_v(g.code8, (uint64_t)(N * kblocks));
  const __amdgpu_buffer_rsrc_t s2r = rsrc_v(g.s2, (uint64_t)((N * kblocks + 255) >> 8) * 4);

  bool row_ok[2];
  int64_t row[2];
#pragma unroll
  for (int ng = 0; ng < 2; ++ng) {
    row[ng] = n0 + 32 * ng + (lane & 31);
    row_ok[ng] = row[ng] < N;
  }
  bool tok_ok[TG];
  int64_t xbase[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int64_t t = 32 * tg + (lane & 31);
    tok_ok[tg] = t < g.T;
    xbase[tg] = (t * K + 32 * half) * 2;
  }

  auto load = [&](int64_t st, bool ok, GemvStage<TG>& s) {
#pragma unroll
    for (int ng = 0; ng < 2; ++ng) {
      const bool v = ok && row_ok[ng];
      const int64_t blk = row[ng] * kblocks + st;
      s.code[ng] = load16(cr, v ? (uint32_t)(blk * 32 + 16 * half) : kOOBv);
      s.c8[ng] = __builtin_amdgcn_raw_buffer_load_b8(c8r, v ? (uint32_t)blk : kOOBv, 0, 0);
      s.s2[ng] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(s2r, v ? (uint32_t)((blk >> 8) * 4) : kOOBv,
                                                      0, 0));
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const uint32_t off = (ok && tok_ok[tg]) ? (uint32_t)(xbase[tg] + st * 128) : kOOBv;
#pragma unroll
      for (int q = 0; q < 4; ++q) s.x[tg][q] = load16(xr, off + 16 * q);
    }
  };

  f32x16_t acc[TG][2];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int ng = 0; ng < 2; ++ng)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tg][ng][e] = 0.0f;

  // The first split's wave 0 starts from the LoRA term (s U) B^T of its
  // tile (U pre-scaled), so every output gets it exactly once.
  if (blockIdx.y == 0 && wave == 0) {
    const __amdgpu_buffer_rsrc_t ur = rsrc_v(g.lora_l, (uint64_t)g.T * g.r * 2);
    const __amdgpu_buffer_rsrc_t br = rsrc_v(g.lora_r, (uint64_t)N * g.r * 2);
    for (int p0 = 0; p0 < g.r; p0 += 16) {
      const int p = p0 + 8 * half;
#pragma unroll
      for (int ng = 0; ng < 2; ++ng) {
        const u32x4_t bv = load16(br, row_ok[ng] ? (uint32_t)((row[ng] * g.r + p) * 2) : kOOBv);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          const u32x4_t av = load16(
              ur, tok_ok[tg] ? (uint32_t)(((32 * tg + (lane & 31)) * g.r + p) * 2) : kOOBv);
          acc[tg][ng] = mfma32(av, bv, acc[tg][ng]);
        }
      }
    }
  }

  GemvStage<TG> cur, nxt;
  int64_t st = st0 + wave;
  load(st, st < st1, cur);
  for (; st < st1; st += 4) {
    load(st + 4, st + 4 < st1, nxt);
    u32x4_t a[TG][4];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[tg][q] = act_eo(cur.x[tg][q]);
#pragma unroll
    for (int ng = 0; ng < 2; ++ng) {
      const float cp = row_ok[ng] ? block_constant(cur.c8[ng], cur.s2[ng], mu) : 0.0f;
      const Nf4Lut lt = make_lut(cp);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t b = dequant8_eo(lt, cur.code[ng][q]);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[tg][ng] = mfma32(a[tg][q], b, acc[tg][ng]);
      }
    }
    cur = nxt;
  }

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
    const bool direct = gridDim.y == 1;
    float* out = P + (int64_t)blockIdx.y * g.T * N;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int ng = 0; ng < 2; ++ng)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int idx = ((tg * 2 + ng) * 16 + e) * 64 + lane;
          float v = acc[tg][ng][e];
          v += red[idx];
          v += red[TG * 2 * 16 * 64 + idx];
          v += red[2 * TG * 2 * 16 * 64 + idx];
          const int64_t t = 32 * tg + 8 * (e >> 2) + 4 * half + (e & 3);
          if (t < g.T && row_ok[ng]) {
            if (direct)
              g.out[t * N + row[ng]] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
            else
              out[t * N + row[ng]] = v;
          }
        }
  }
}

// Y = bf16(sum_s P[s]) over the flattened [T, rows] outputs, 4 per thread,
// splits added in order.
__global__ __launch_bounds__(256) void qlora_gemv_finish_kernel(int64_t n4, int splits,
                                                                const float* __restrict__ P,
                                                                uint16_t* __restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(P);
  f32x4_t v = p4[i];
  for (int s = 1; s < splits; ++s) {
    const f32x4_t w = p4[(int64_t)s * n4 + i];
    v[0] += w[0];
    v[1] += w[1];
    v[2] += w[2];
    v[3] += w[3];
  }
  uint2 o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  reinterpret_cast<uint2*>(Y)[i] = o;
}

hipError_t launch_qlora_gemv(const GemmArgs& a, float* P, int splits, hipStream_t stream) {
  const int64_t kblocks = a.cols / 64;
  if (a.T < 1 || a.T > kGemvMaxTokens || splits < 1 || splits > kblocks) return hipErrorInvalidValue;
  const int per = (int)((kblocks + splits - 1) / splits);
  const dim3 grid((unsigned)((a.rows + 63) / 64), (unsigned)splits);
  if (a.T <= 32)
    hipLaunchKernelGGL(qlora_gemv_partial_kernel<1>, grid, dim3(256), 0, stream, a, per, P);
  else
    hipLaunchKernelGGL(qlora_gemv_partial_kernel<2>, grid, dim3(256), 0, stream, a, per, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n4 = a.T * a.rows / 4;
  hipLaunchKernelGGL(qlora_gemv_finish_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                     stream, n4, splits, P, a.out);
  return hipGetLastError();
}

}  // namespace qlora
