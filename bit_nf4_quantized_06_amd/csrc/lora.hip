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
// P[s][t][p] = sum_{k in chunk s} L[t][k] R(p, k), L [T, red] bf16 and R the
// rank-r operand, stored either [r, red] (R(p, k) = R[p][k], the forward's
// A) or [red, r] (kRT: R(p, k) = R[k][p], the backward's B, read in place).
//
// Workgroup = 4 waves over 128 tokens; wave w owns tokens 32 w .. 32 w + 31
// (two MFMA 16x16x32 row groups) and all r columns, and walks the split's
// reduction chunk 128 at a time.  The 128-wide slice of R is shared by the
// four waves: it goes straight into LDS by buffer loads (no registers), one
// of three stages; the L operand goes to registers, three buffers.  Both
// run two iterations ahead, so every wave keeps 16 L loads of 1 KB in
// flight.  The stage and buffer indices are compile-time constants (the
// loop is unrolled by 3), so the DMA into one stage never makes the compiler
// wait before reading another.
//
// R stage layouts (bf16 elements):
//   [r, red] source: r rows x 16 chunks of 8, chunk' = chunk ^ (row & 15),
//       so the 16 rows one fragment read touches land in 16 distinct chunks;
//   [red, r] source: 128 rows x r, exactly as in memory (the rows of one
//       slice are contiguous); fragments come from ds_read_b64_tr_b16, which
//       hands each lane 4 consecutive rows of one column.
// ---------------------------------------------------------------------------
template <int NJ, bool kRT>
struct ProjCtx {
  __amdgpu_buffer_rsrc_t lr, rr;
  uint32_t x_off[2];        // per row group: lane's L byte offset at k = 0
  bool x_ok[2];             // token row inside L
  int64_t kb, ke;           // this split's reduction range
  int64_t red;
  uint32_t r_off[NJ];       // kRT == false: lane's R offset at k = 0 per DMA
  int r_row[NJ];            // kRT == false: R row of that DMA lane
  int r_chunk[NJ];          // kRT == false: logical chunk of that DMA lane
  uint32_t rt_byte[NJ];     // kRT: byte of the slice this DMA lane fetches
  int wave, lane;
};

template <int NJ, bool kRT>
__device__ __forceinline__ void proj_load_x(const ProjCtx<NJ, kRT>& c, int it, u32x4_t (&x)[4][2]) {
  const int64_t k0 = c.kb + (int64_t)it * 128 + 8 * (c.lane >> 4);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t k = k0 + 32 * u;
    const bool kin = k < c.ke;
#pragma unroll
    for (int g = 0; g < 2; ++g)
      x[u][g] = bload16(c.lr, kin && c.x_ok[g] ? c.x_off[g] + (uint32_t)(k * 2) : kOOB);
  }
}

template <int NJ, bool kRT>
__device__ __forceinline__ void proj_load_r(const ProjCtx<NJ, kRT>& c, int it, uint16_t* stage) {
  const int64_t k0 = c.kb + (int64_t)it * 128;
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int q = c.wave * NJ + i;   // 1 KB piece of the 4 NJ KB stage
    uint32_t off;
    if (!kRT) {
      const int64_t k = k0 + 8 * c.r_chunk[i];
      off = k < c.ke ? c.r_off[i] + (uint32_t)(k * 2) : kOOB;
    } else {
      const int64_t row = k0 + (int64_t)(c.rt_byte[i] / (32 * NJ));
      off = row < c.ke ? (uint32_t)(k0 * 32 * NJ) + c.rt_byte[i] : kOOB;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rr, (lds_void_t*)(stage + q * 512), 16, off, 0, 0,
                                             0);
  }
}

// B-operand fragment (16 columns p, 32 reduction indices) j of slice u
template <int NJ, bool kRT>
__device__ __forceinline__ u32x4_t proj_frag(const ProjCtx<NJ, kRT>& c, const uint16_t* stage,
                                             int u, int j) {
  if (!kRT) {
    const int p = 16 * j + (c.lane & 15);
    const int ch = (4 * u + (c.lane >> 4)) ^ (p & 15);
    return *reinterpret_cast<const u32x4_t*>(stage + p * 128 + 8 * ch);
  } else {
    const int row = 32 * u + 8 * (c.lane >> 4) + ((c.lane & 15) >> 2);
    const int col = 16 * j + 4 * (c.lane & 3);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(stage + row * (16 * NJ) + col));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(stage + (row + 4) * (16 * NJ) + col));
    const uint2 l = __builtin_bit_cast(uint2, lo);
    const uint2 h = __builtin_bit_cast(uint2, hi);
    return u32x4_t{l.x, l.y, h.x, h.y};
  }
}

// One 128-wide iteration on R stage SI and L buffer SI.  kMore: also issue
// L(it + 2) and R(it + 2).  Vector-memory issue order is pinned by
// scheduling barriers, so the wait before the workgroup barrier can count
// the loads issued after this wave's share of R(it): in the unrolled loop
// L(it + 1), R(it + 1) and L(it + 2); in the two iterations after it, which
// issue nothing, L(it + 1) and R(it + 1) for the first and none for the
// second (kTail = 1, 2).
template <int NJ, bool kRT, bool kF16, int SI, bool kMore, int kTail>
__device__ __forceinline__ void proj_iter(const ProjCtx<NJ, kRT>& c, int it, uint16_t* const (&st)[3],
                                          u32x4_t (&xb)[3][4][2], f32x4_t (&acc)[2][NJ]) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (kMore) proj_load_x(c, it + 2, xb[(SI + 2) % 3]);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int N = kMore ? 16 + NJ : (kTail == 1 ? 8 + NJ : 0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");
  if (kMore) proj_load_r(c, it + 2, st[(SI + 2) % 3]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4_t rf[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) rf[j] = proj_frag(c, st[SI], u, j);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[g][j] = mfma16<kF16>(xb[SI][u][g], rf[j], acc[g][j]);
  }
  __builtin_amdgcn_sched_barrier(0);
#endif
}

template <int NJ, bool kRT, bool kF16>
__global__ __launch_bounds__(256) void lora_proj_partial_kernel(
    const uint16_t* __restrict__ L, const uint16_t* __restrict__ R, int64_t T, int64_t red,
    int64_t chunk, float* __restrict__ P) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kStage = 16 * NJ * 128;   // bf16 elements
  __shared__ __attribute__((aligned(1024))) uint16_t s0[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[kStage];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[kStage];
  uint16_t* const st[3] = {s0, s1, s2};
  ProjCtx<NJ, kRT> c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.red = red;
  const int64_t m0 = (int64_t)blockIdx.x * 128 + 32 * c.wave;
  c.kb = (int64_t)blockIdx.y * chunk;
  c.ke = c.kb + chunk < red ? c.kb + chunk : red;
  const int nit = c.ke > c.kb ? (int)((c.ke - c.kb + 127) / 128) : 0;
  c.lr = rsrc(L, (uint64_t)T * red * 2);
  c.rr = rsrc(R, (uint64_t)(16 * NJ) * red * 2);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int64_t t = m0 + 16 * g + (c.lane & 15);
    c.x_ok[g] = t < T;
    c.x_off[g] = c.x_ok[g] ? (uint32_t)(t * red * 2) : 0u;
  }
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int q = c.wave * NJ + i;
    if (!kRT) {
      // piece q = rows 4 q .. 4 q + 3 of the stage, lane -> (row, physical chunk)
      const int row = 4 * q + (c.lane >> 4);
      const int ch = (c.lane & 15) ^ (row & 15);
      c.r_row[i] = row;
      c.r_chunk[i] = ch;
      c.r_off[i] = (uint32_t)((int64_t)row * red * 2);
    } else {
      c.rt_byte[i] = (uint32_t)(1024 * q + 16 * c.lane);
    }
  }
  f32x4_t acc[2][NJ];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[g][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nit > 0) {
    u32x4_t xb[3][4][2];
    // prologue in the steady-state issue order: X(0), R(0), X(1), R(1)
    proj_load_x(c, 0, xb[0]);
    __builtin_amdgcn_sched_barrier(0);
    proj_load_r(c, 0, s0);
    __builtin_amdgcn_sched_barrier(0);
    proj_load_x(c, 1, xb[1]);
    __builtin_amdgcn_sched_barrier(0);
    proj_load_r(c, 1, s1);
    __builtin_amdgcn_sched_barrier(0);
    // the unrolled body is one basic block (no early exits for the
    // compiler to sink the prefetches into); the last nit % 3 iterations
    // follow the loop
    const int nit3 = nit - nit % 3;
    for (int it = 0; it < nit3; it += 3) {
      proj_iter<NJ, kRT, kF16, 0, true, 0>(c, it, st, xb, acc);
      proj_iter<NJ, kRT, kF16, 1, true, 0>(c, it + 1, st, xb, acc);
      proj_iter<NJ, kRT, kF16, 2, true, 0>(c, it + 2, st, xb, acc);
    }
    if (nit3 < nit) proj_iter<NJ, kRT, kF16, 0, false, 1>(c, nit3, st, xb, acc);
    if (nit3 + 1 < nit) proj_iter<NJ, kRT, kF16, 1, false, 2>(c, nit3 + 1, st, xb, acc);
    // the loads issued past the end read nothing; let them land before exit
    __builtin_amdgcn_s_waitcnt((7 << 4) | (0xF << 8));
  }
  float* out = P + (int64_t)blockIdx.y * T * (16 * NJ);
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = m0 + 16 * g + 4 * (c.lane >> 4) + e;
        if (t < T) out[t * (16 * NJ) + 16 * j + (c.lane & 15)] = acc[g][j][e];
      }
#endif
}

static int64_t proj_chunk(int64_t red, int splits) {
  int64_t c = (red + splits - 1) / splits;
  return (c + 127) / 128 * 128;
}

template <bool kF16>
static hipError_t proj_partial_dispatch(const uint16_t* L, const uint16_t* R, bool r_by_rows,
                                        int64_t T, int64_t red, int32_t r, int splits, float* P,
                                        hipStream_t stream) {
  const int64_t chunk = proj_chunk(red, splits);
  const dim3 grid((unsigned)((T + 127) / 128), (unsigned)splits);
  switch ((r >> 4) * 2 + (r_by_rows ? 1 : 0)) {
#define QLORA_PROJ_CASE(NJ)                                                                   \
  case 2 * NJ:                                                                                \
    hipLaunchKernelGGL((lora_proj_partial_kernel<NJ, false, kF16>), grid, dim3(256), 0, stream, \
                       L, R, T, red, chunk, P);                                               \
    break;                                                                                    \
  case 2 * NJ + 1:                                                                            \
    hipLaunchKernelGGL((lora_proj_partial_kernel<NJ, true, kF16>), grid, dim3(256), 0, stream, \
                       L, R, T, red, chunk, P);                                               \
    break;
    QLORA_PROJ_CASE(1) QLORA_PROJ_CASE(2) QLORA_PROJ_CASE(3) QLORA_PROJ_CASE(4)
    QLORA_PROJ_CASE(5) QLORA_PROJ_CASE(6) QLORA_PROJ_CASE(7) QLORA_PROJ_CASE(8)
#undef QLORA_PROJ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lora_proj_partial(const uint16_t* L, const uint16_t* R, bool r_by_rows,
                                    int64_t T, int64_t red, int32_t r, int splits, float* P,
                                    bool f16, hipStream_t stream) {
  return f16 ? proj_partial_dispatch<true>(L, R, r_by_rows, T, red, r, splits, P, stream)
             : proj_partial_dispatch<false>(L, R, r_by_rows, T, red, r, splits, P, stream);
}

// ---------------------------------------------------------------------------
// Fixed-order sum of the split partials, v = P[0] + P[1] + ... + P[S-1], for
// four consecutive outputs (t, p .. p + 3) per thread (16-byte loads, 8
// splits in flight).  Writes any of: out_rm[t][p] = bf16(v), out_sc[t][p] =
// bf16(scale * v) (the pre-scaled operand the fused GEMM seeds its
// accumulators with), out_tr[p][t] = bf16(v) with row stride ld_tr and zeros
// for T <= t < ld_tr.  Workgroups past the reduction run the bf16 transposes
// of `tj` (32 x 32 tiles through LDS), so small layout changes the next
// kernels need ride along in the same launch.
// ---------------------------------------------------------------------------
__device__ void transpose_tile(const TransposeJobs& jobs, int b) {
  __shared__ uint16_t tile[32][33];
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

// One chunk (1024 words of 8 codes) of the once-per-call dequantisation.
__device__ void dequant_role(const ProjReduce& a, int64_t chunk) {
  __shared__ float q[16];
  if (threadIdx.x < 16) q[threadIdx.x] = kNF4[threadIdx.x];
  __syncthreads();
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(a.dq_codes);
  u32x4_t* out = reinterpret_cast<u32x4_t*>(a.dq_out);
  if (a.dq_dq) {
    const float mu = a.dq_mu[0];
    if (a.f16)
      dequant_chunk<true, true>(codes, a.dq_code8, a.dq_s2, mu, a.dq_words, chunk, q, out);
    else
      dequant_chunk<true, false>(codes, a.dq_code8, a.dq_s2, mu, a.dq_words, chunk, q, out);
  } else {
    if (a.f16)
      dequant_chunk<false, true>(codes, a.dq_code8, a.dq_s2, 0.0f, a.dq_words, chunk, q, out);
    else
      dequant_chunk<false, false>(codes, a.dq_code8, a.dq_s2, 0.0f, a.dq_words, chunk, q, out);
  }
}

// Workgroups [0, reduce_blocks): the split reduction; then `transpose_blocks`
// transpose tiles; then the dequantisation chunks (a.dq_out set).  The roles
// are independent, so one launch carries them all.
// Fixed-order sum src[0] + src[stride] + ... over `splits` float32 quads:
// loads go out 8 at a time (splits past the end re-read the last one), so up
// to 8 splits cost one memory round trip; the padding adds -0, which leaves
// every sum, signed zeros included, as the plain loop gives it.
__device__ __forceinline__ f32x4_t sum_splits(const f32x4_t* src, int64_t stride, int splits) {
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += 8) {
    f32x4_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sc = s0 + j < splits ? s0 + j : splits - 1;
      x[j] = src[(int64_t)sc * stride];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = s0 + j < splits;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += in ? x[j][e] : -0.0f;
    }
  }
  return v;
}

__global__ __launch_bounds__(256) void lora_proj_reduce_kernel(ProjReduce a, TransposeJobs tj,
                                                               unsigned reduce_blocks,
                                                               unsigned transpose_blocks) {
  if (blockIdx.x == 0 && (int)threadIdx.x < a.n_zero) a.zero_cnt[threadIdx.x] = 0u;
  if (blockIdx.x >= reduce_blocks + transpose_blocks) {
    dequant_role(a, (int64_t)(blockIdx.x - reduce_blocks - transpose_blocks));
    return;
  }
  if (blockIdx.x >= reduce_blocks) {
    transpose_tile(tj, (int)(blockIdx.x - reduce_blocks));
    return;
  }
  const int64_t rows_total = a.out_tr ? a.ld_tr : a.T;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= rows_total * a.r) return;
  const int64_t t = i / a.r;
  const int p = (int)(i - t * a.r);
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (t < a.T) v = sum_splits(reinterpret_cast<const f32x4_t*>(a.P + i), a.T * a.r / 4, a.splits);
  uint16_t b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    b[e] = (uint16_t)((a.f16 ? pack_f16x2(v[e] * a.scale_rm, 0.0f)
                             : pack_bf16x2(v[e] * a.scale_rm, 0.0f)) & 0xFFFFu);
  if (t < a.T) {
    if (a.out_rm)
      *reinterpret_cast<uint2*>(a.out_rm + i) =
          uint2{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
    if (a.out_sc)
      *reinterpret_cast<uint2*>(a.out_sc + i) =
          a.f16 ? uint2{pack_f16x2(v[0] * a.scale, v[1] * a.scale),
                        pack_f16x2(v[2] * a.scale, v[3] * a.scale)}
                : uint2{pack_bf16x2(v[0] * a.scale, v[1] * a.scale),
                        pack_bf16x2(v[2] * a.scale, v[3] * a.scale)};
  }
  if (a.out_tr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a.out_tr[(int64_t)(p + e) * a.ld_tr + t] = b[e];
  }
}

hipError_t launch_lora_proj_reduce(const ProjReduce& a, TransposeJobs tj, hipStream_t stream) {
  const int64_t rows_total = a.out_tr ? a.ld_tr : a.T;
  const unsigned nred = (unsigned)((rows_total * a.r / 4 + 255) / 256);
  int ttiles = 0;
  for (int i = 0; i < tj.n; ++i) {
    const TransposeJob& j = tj.job[i];
    tj.tiles[i] = (int)(((j.C + 31) / 32) * ((j.ld_out + 31) / 32));
    ttiles += tj.tiles[i];
  }
  const unsigned ndeq = a.dq_out ? (unsigned)((a.dq_words + 1023) / 1024) : 0u;
  hipLaunchKernelGGL(lora_proj_reduce_kernel, dim3(nred + (unsigned)ttiles + ndeq), dim3(256), 0,
                     stream, a, tj, nred, (unsigned)ttiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// C[s][p][q] = sum_{t in chunk s} S[t][p] L[t][q] for up to two problems per
// launch (blockIdx.z): the dA partials (S = G, L = X) and the dB partials
// (S = U, L = dY).  S [T, r] and L [T, Q] are bf16 in their natural
// token-major layout.  The reduction runs over tokens, so both MFMA operands
// need 8 consecutive tokens of one column per lane: every 64-token slice of
// L (128 columns) and of S goes straight into LDS by buffer loads, whole
// 256-byte row pieces at a time, and ds_read_b64_tr_b16 hands each lane 4
// consecutive rows of one column -- no register transposes.
//
// Workgroup = 4 waves over 128 columns q; wave w owns q0 + 32 w .. + 31 and
// all r rows p, so the four waves share each staged slice and need no
// reduction among themselves.  Three stages, loads two slices ahead.
// L stage: 64 rows x 16 chunks of 8, chunk' = chunk ^ f(row) with f(row) =
// 4 (row & 3) + 2 ((row >> 3) & 1), so the 4 rows x 2 chunks one 16-lane
// group of a transposed read touches, and the same for the next group, sit
// in 16 distinct chunks.  S stage: 64 rows x r, as in memory.
// Partials are written [p][q], or [q][p] for a transposed job (dB, kept as
// [Q, r]), so the reduction reads and writes contiguously in both cases.
// ---------------------------------------------------------------------------
template <int NP>
struct GradCtx {
  __amdgpu_buffer_rsrc_t lr, sr;
  uint32_t l_voff[4];   // L DMA i of this wave: byte offset at t = 0 (column part)
  int l_row[4];         // its row within the slice
  bool l_cok[4];        // its 8 columns lie inside Q (Q % 16 == 0: all or none)
  int64_t Q, tb, te;
  int wave, lane;
};

constexpr int kGradSD(int NP) { return (2 * NP + 3) / 4; }   // S DMAs per wave

template <int NP>
__device__ __forceinline__ void grad_load(const GradCtx<NP>& c, int it, uint16_t* lst,
                                          uint16_t* sst, uint16_t* dummy) {
  const int64_t t0 = c.tb + (int64_t)it * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + c.l_row[i];
    const uint32_t off = (t < c.te && c.l_cok[i]) ? (uint32_t)(t * c.Q * 2) + c.l_voff[i] : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.lr, (lds_void_t*)(lst + (4 * c.wave + i) * 512), 16,
                                             off, 0, 0, 0);
  }
  // the S slice is 64 rows x r = 2 NP pieces of 1 KB; pieces past it land
  // in a dummy area (their source is out of range: zeros)
#pragma unroll
  for (int i = 0; i < kGradSD(NP); ++i) {
    const int q = c.wave * kGradSD(NP) + i;
    const uint32_t byte = (uint32_t)(1024 * q + 16 * c.lane);
    const int64_t t = t0 + byte / (32 * NP);
    const bool real = q < 2 * NP;
    const uint32_t off = (real && t < c.te) ? (uint32_t)(t0 * 32 * NP) + byte : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.sr, (lds_void_t*)(real ? sst + q * 512 : dummy), 16,
                                             off, 0, 0, 0);
  }
}

__device__ __forceinline__ u32x4_t ld_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo);
  const uint2 h = __builtin_bit_cast(uint2, hi);
  return u32x4_t{l.x, l.y, h.x, h.y};
}

template <int NP, bool kF16, int SI>
__device__ __forceinline__ void grad_iter(const GradCtx<NP>& c, int it, uint16_t* const (&ls)[3],
                                          uint16_t* const (&ss)[3], uint16_t* dummy,
                                          f32x4_t (&acc)[NP][2]) {
#if defined(__HIP_DEVICE_COMPILE__)
  // slice it landed: the newer loads are slice it+1's (4 + kGradSD per wave)
  constexpr int N = 4 + kGradSD(NP);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");
  grad_load(c, it + 2, ls[(SI + 2) % 3], ss[(SI + 2) % 3], dummy);
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* L = ls[SI];
  const uint16_t* S = ss[SI];
  const int a = (c.lane & 15) >> 2;      // row within the 4-row group
  const int b = c.lane & 3;              // 4-column piece
  const int g = c.lane >> 4;             // 16-lane group: rows + 8 g
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int row = 32 * ks + 8 * g + a;
    u32x4_t lf[2], sf[NP];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      const int col = 32 * c.wave + 16 * cg + 4 * b;          // within the 128
      const int ch = col >> 3;
      const int f = 4 * (row & 3) + 2 * ((row >> 3) & 1);     // same for row + 4
      const int e0 = row * 128 + ((ch ^ f) << 3) + (col & 7);
      const int e1 = (row + 4) * 128 + ((ch ^ f) << 3) + (col & 7);
      lf[cg] = ld_tr_pair(L + e0, L + e1);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int col = 16 * j + 4 * b;
      sf[j] = ld_tr_pair(S + row * (16 * NP) + col, S + (row + 4) * (16 * NP) + col);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) acc[j][cg] = mfma16<kF16>(sf[j], lf[cg], acc[j][cg]);
  }
  __builtin_amdgcn_sched_barrier(0);
#endif
}

template <int NP, bool kF16>
__global__ __launch_bounds__(256) void lora_grad_partial_kernel(GradJobs jobs, int64_t T,
                                                               int64_t chunk) {
  // device pass only: the host pass needs just the signature (see the fused GEMM kernel)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint16_t l0[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t l1[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t l2[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t s0[64 * 16 * NP];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[64 * 16 * NP];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[64 * 16 * NP];
  __shared__ __attribute__((aligned(1024))) uint16_t dummy[512];
  uint16_t* const ls[3] = {l0, l1, l2};
  uint16_t* const ss[3] = {s0, s1, s2};
  const GradJob& jb = jobs.job[blockIdx.z];
  GradCtx<NP> c;
  c.Q = jb.Q;
  const int64_t q0 = (int64_t)blockIdx.x * 128;
  if (q0 >= c.Q) return;   // whole workgroup: before any barrier
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.tb = (int64_t)blockIdx.y * chunk;
  c.te = c.tb + chunk < T ? c.tb + chunk : T;
  const int nit = c.te > c.tb ? (int)((c.te - c.tb + 63) / 64) : 0;
  c.lr = rsrc(jb.L, (uint64_t)T * c.Q * 2);
  c.sr = rsrc(jb.S, (uint64_t)T * (16 * NP) * 2);
  {
    // L DMA i of wave w fills rows 4 (4 w + i) .. + 3: lane -> row + lane / 16,
    // physical chunk lane % 16, which holds logical chunk (lane % 16) ^ f(row)
    const int ph = c.lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (4 * c.wave + i) + (c.lane >> 4);
      const int f = 4 * (row & 3) + 2 * ((row >> 3) & 1);
      const int lc = ph ^ f;
      c.l_row[i] = row;
      c.l_voff[i] = (uint32_t)((q0 + 8 * lc) * 2);
      c.l_cok[i] = q0 + 8 * lc < c.Q;
    }
  }
  f32x4_t acc[NP][2];
#pragma unroll
  for (int j = 0; j < NP; ++j)
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) acc[j][cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nit > 0) {
    grad_load(c, 0, l0, s0, dummy);
    __builtin_amdgcn_sched_barrier(0);
    grad_load(c, 1, l1, s1, dummy);
    __builtin_amdgcn_sched_barrier(0);
    const int nit3 = nit - nit % 3;
    for (int it = 0; it < nit3; it += 3) {
      grad_iter<NP, kF16, 0>(c, it, ls, ss, dummy, acc);
      grad_iter<NP, kF16, 1>(c, it + 1, ls, ss, dummy, acc);
      grad_iter<NP, kF16, 2>(c, it + 2, ls, ss, dummy, acc);
    }
    if (nit3 < nit) grad_iter<NP, kF16, 0>(c, nit3, ls, ss, dummy, acc);
    if (nit3 + 1 < nit) grad_iter<NP, kF16, 1>(c, nit3 + 1, ls, ss, dummy, acc);
    // the loads issued past the end read nothing; let them land before exit
    __builtin_amdgcn_s_waitcnt((7 << 4) | (0xF << 8));
  }
  // acc[j][cg][e] = C[p = 16 j + 4 (lane / 16) + e][q = q0 + 32 w + 16 cg + lane % 16]
  float* out = jb.P + (int64_t)blockIdx.y * (16 * NP) * c.Q;
#pragma unroll
  for (int cg = 0; cg < 2; ++cg) {
    const int64_t q = q0 + 32 * c.wave + 16 * cg + (c.lane & 15);
    if (q >= c.Q) continue;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = 16 * j + 4 * (c.lane >> 4);
      if (jb.transposed) {
        *reinterpret_cast<f32x4_t*>(out + q * (16 * NP) + p) = acc[j][cg];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[(int64_t)(p + e) * c.Q + q] = acc[j][cg][e];
      }
    }
  }
#endif
}

static int64_t grad_chunk(int64_t T, int splits) {
  int64_t c = (T + splits - 1) / splits;
  return (c + 63) / 64 * 64;
}

hipError_t launch_lora_grad_partial(GradJobs jobs, int64_t T, int32_t r, int splits,
                                    bool f16, hipStream_t stream) {
  const int64_t chunk = grad_chunk(T, splits);
  int64_t qmax = 0;
  for (int i = 0; i < jobs.n; ++i) qmax = jobs.job[i].Q > qmax ? jobs.job[i].Q : qmax;
  const dim3 grid((unsigned)((qmax + 127) / 128), (unsigned)splits, (unsigned)jobs.n);
  switch (r >> 4) {
#define QLORA_GRAD_CASE(NP)                                                                  \
  case NP:                                                                                   \
    if (f16)                                                                                 \
      hipLaunchKernelGGL((lora_grad_partial_kernel<NP, true>), grid, dim3(256), 0, stream,   \
                         jobs, T, chunk);                                                    \
    else                                                                                     \
      hipLaunchKernelGGL((lora_grad_partial_kernel<NP, false>), grid, dim3(256), 0, stream,  \
                         jobs, T, chunk);                                                    \
    break;
    QLORA_GRAD_CASE(1) QLORA_GRAD_CASE(2) QLORA_GRAD_CASE(3) QLORA_GRAD_CASE(4)
    QLORA_GRAD_CASE(5) QLORA_GRAD_CASE(6) QLORA_GRAD_CASE(7) QLORA_GRAD_CASE(8)
#undef QLORA_GRAD_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// out[i] = scale * (P[0][i] + P[1][i] + ...) (fixed order) for each job; the
// partials already have the output's layout ([r, Q], or [Q, r] for a
// transposed job).  Four outputs per thread, 8 splits in flight; all jobs in
// one launch.
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(GradJobs jobs, int r, int splits,
                                                               float scale) {
  int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  // the job (at most two) by field-wise selects of the kernel arguments: no
  // dynamically indexed copy of the argument struct in memory
  const int64_t n0 = (int64_t)r * jobs.job[0].Q;
  const bool second = i >= n0;
  if (second) i -= n0;
  if (second && (jobs.n < 2 || i >= (int64_t)r * jobs.job[1].Q)) return;
  const int64_t Q = second ? jobs.job[1].Q : jobs.job[0].Q;
  const float* P = second ? jobs.job[1].P : jobs.job[0].P;
  float* out = second ? jobs.job[1].out : jobs.job[0].out;
  const f32x4_t v = sum_splits(reinterpret_cast<const f32x4_t*>(P + i), (int64_t)r * Q / 4, splits);
  *reinterpret_cast<f32x4_t*>(out + i) = v * scale;
}

hipError_t launch_lora_grad_reduce(GradJobs jobs, int32_t r, int splits, float scale,
                                   hipStream_t stream) {
  int64_t n = 0;
  for (int i = 0; i < jobs.n; ++i) n += (int64_t)r * jobs.job[i].Q;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0,
                     stream, jobs, r, splits, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// n float32 zeros (n % 4 == 0, 16-byte aligned): the adapter gradients of an
// empty token batch, written by a kernel rather than a memset so that a
// captured graph holds no memset node.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_f32_kernel(f32x4_t* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = (n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<f32x4_t*>(p), n4);
  return hipGetLastError();
}

}  // namespace qlora
