// Fused NF4-dequant GEMMs of the QLoRA linear layer (gfx950, bf16 MFMA).
//
//   forward:      Y  = X  dequant(W)^T + (s X A^T) B^T
//   backward dX:  dX = dY dequant(W)   + (s dY B)  A
// ta-paperlens 勾配は実際どこへ行くのか: each matmul dequantises the NF4 blocks it
// needs to bf16, uses them and drops them; the input gradient goes through
// dequant(W)^T; W is never written.  Ultralytics "So funktioniert QLoRA":
// dequantise right before the matmul and add the LoRA path.
//
// Kernel shape.  A workgroup of 4 waves (one per SIMD) computes a 256-token x
// 256-column output tile with float32 accumulators; each wave owns a
// 128 x 128 sub-tile held as 4 x 4 MFMA 32x32x16 blocks (256 AGPRs).  The
// reduction advances 64 per step, i.e. one NF4 block per weight row.
//
// Per step, both operands come from LDS (two stages of 64 KB each):
//   * activations (X or dY) 256 x 64 bf16: global -> registers -> LDS;
//   * the weight tile is dequantised once per workgroup straight into LDS.
//     Each thread owns one block of 64 weights: it builds the 16-entry bf16
//     table q[k] * c' (16 float32 products rounded once, as the bulk
//     dequantiser does) and translates its 32 bytes of nibbles with v_perm
//     byte lookups.  The tile keeps W's own row layout in both directions;
//     the backward reads its operand (reduction = W rows) with
//     ds_read_b64_tr_b16, which hands each lane 4 consecutive rows of one
//     column.
// The work of step k+1 (global loads issued one step ahead for activations
// and two steps ahead for the packed codes, dequantisation, LDS stores) is
// interleaved with the 64 MFMAs of step k; MFMA fragments are read one
// 16-wide slice ahead.  One barrier per step.
//
// LDS layouts (16-byte chunks XOR-swizzled so that every ds_read_b128,
// ds_read_b64_tr_b16 and ds_write_b128 pattern used here touches 16 distinct
// 16-byte bank groups per 256 bytes):
//   activation / forward weight tile: 256 rows x 8 chunks,
//       chunk' = chunk ^ ((row >> 1) & 7)
//   backward weight tile: 64 rows (W rows) x 32 chunks (256 W columns),
//       chunk' = chunk ^ (((row & 3) << 2) | ((row >> 2) & 3))
//
// Workgroups are numbered so that the 32 consecutive tiles a single XCD
// receives (dispatch is round-robin over the 8 XCDs) form a compact block
// of 4 token tiles x 8 column tiles, keeping their shared operand tiles in
// that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace qlora {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kStageElems = BM * BK;           // 16384 bf16 = 32 KB

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz_a(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}
__device__ __forceinline__ int swz_bt(int row, int chunk) {   // backward weight tile
  return row * BN + ((chunk ^ (((row & 3) << 2) | ((row >> 2) & 3))) << 3);
}

__device__ __forceinline__ u32x4_t ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x4_t ld_lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two ds_read_b64_tr_b16 -> one 8 x bf16 MFMA operand
__device__ __forceinline__ u32x4_t ld_lds_tr(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo);
  const uint2 h = __builtin_bit_cast(uint2, hi);
  return u32x4_t{l.x, l.y, h.x, h.y};
}

// tile index -> (token tile, column tile): XCD-major, then groups of 4 token tiles
__device__ __forceinline__ void tile_coords(int pid, int mt, int nt, int& tm, int& tn) {
  const int total = mt * nt;
  const int xcd = pid & 7;
  const int base = total >> 3;
  const int rem = total & 7;
  const int q = xcd * base + (xcd < rem ? xcd : rem) + (pid >> 3);
  constexpr int GM = 4;
  const int group = q / (GM * nt);
  const int first = group * GM;
  const int gm = (mt - first) < GM ? (mt - first) : GM;
  const int local = q - group * GM * nt;
  tm = first + local % gm;
  tn = local / gm;
}

template <bool kBwd>
__global__ __launch_bounds__(256, 1) void qlora_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];   // 128 KB
  uint16_t* const As0 = smem;
  uint16_t* const Bs0 = smem + 2 * kStageElems;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int64_t red_len = kBwd ? g.rows : g.cols;
  const int64_t out_len = kBwd ? g.cols : g.rows;
  const int mt = (int)((g.T + BM - 1) / BM);
  const int nt = (int)((out_len + BN - 1) / BN);
  int tm, tn;
  tile_coords(blockIdx.x, mt, nt, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int nsteps = (int)((red_len + BK - 1) / BK);
  const int64_t kblocks = g.cols >> 6;
  const float mu = g.mu[0];
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  f32x16_t acc[4][4];

  // ---- LoRA seed: acc = (s L) R^T over r (L is pre-scaled) -----------------
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  for (int p0 = 0; p0 < g.r; p0 += 16) {
    const int p = p0 + 8 * lhi;
    u32x4_t af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + 128 * wm + 32 * i + l32;
      af[i] = row < g.T ? ld_global16(g.lora_l + row * g.r + p) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + 128 * wn + 32 * j + l32;
      bf[j] = col < out_len ? ld_global16(g.lora_r + col * g.r + p) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
  }

  // ---- per-thread staging state -------------------------------------------
  // activation chunk i of this thread: tile row (tid >> 3) + 32 i, chunk tid & 7
  u32x4_t a_reg[8];
  // packed codes of this thread's weight block, for step k+1 (cur) and k+2 (nxt)
  u32x4_t c_cur[2], c_nxt[2];
  float cp_cur = 0.0f, cp_nxt = 0.0f;
  bool ok_cur = false, ok_nxt = false;

  // weight block owned by this thread at step `step`
  auto w_coords = [&](int step, int64_t& n, int64_t& kc) {
    if (!kBwd) {
      n = n0 + tid;
      kc = (int64_t)step * BK;
    } else {
      n = (int64_t)step * BK + (tid & 63);
      kc = n0 + 64 * (tid >> 6);
    }
  };
  auto load_codes = [&](int step, u32x4_t* c, float& cp, bool& ok) {
    int64_t n, kc;
    w_coords(step, n, kc);
    ok = step < nsteps && n < g.rows && kc < g.cols;
    if (ok) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(g.codes + ((n * g.cols + kc) >> 1));
      c[0] = p[0];
      c[1] = p[1];
      const int64_t blk = n * kblocks + (kc >> 6);
      cp = block_constant(g.code8[blk], g.s2[blk >> 8], mu);
    }
  };
  auto load_act = [&](int step) {
    const int64_t kbase = (int64_t)step * BK + (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = m0 + (tid >> 3) + 32 * i;
      a_reg[i] = (t < g.T && kbase < red_len) ? ld_global16(g.act + t * red_len + kbase)
                                              : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_act = [&](uint16_t* as, int i) {
    *reinterpret_cast<u32x4_t*>(as + swz_a((tid >> 3) + 32 * i, tid & 7)) = a_reg[i];
  };
  // dequantise word pair (2w, 2w+1) of the current block and store 16 weights
  auto store_w = [&](uint16_t* bs, const Nf4Lut& lut, int w) {
    uint32_t d0[4] = {0u, 0u, 0u, 0u}, d1[4] = {0u, 0u, 0u, 0u};
    if (ok_cur) {
      dequant8(lut, c_cur[w >> 1][(2 * w) & 3], d0);
      dequant8(lut, c_cur[w >> 1][(2 * w + 1) & 3], d1);
    }
    if (!kBwd) {
      *reinterpret_cast<u32x4_t*>(bs + swz_a(tid, 2 * w)) = u32x4_t{d0[0], d0[1], d0[2], d0[3]};
      *reinterpret_cast<u32x4_t*>(bs + swz_a(tid, 2 * w + 1)) = u32x4_t{d1[0], d1[1], d1[2], d1[3]};
    } else {
      const int row = tid & 63;
      const int chunk = 8 * (tid >> 6) + 2 * w;
      *reinterpret_cast<u32x4_t*>(bs + swz_bt(row, chunk)) = u32x4_t{d0[0], d0[1], d0[2], d0[3]};
      *reinterpret_cast<u32x4_t*>(bs + swz_bt(row, chunk + 1)) = u32x4_t{d1[0], d1[1], d1[2], d1[3]};
    }
  };
  // MFMA fragments of slice s from stage buffers (as, bs)
  auto load_frags = [&](const uint16_t* as, const uint16_t* bs, int s, u32x4_t* fa, u32x4_t* fb) {
    const int chunk = 2 * s + lhi;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = ld_lds16(as + swz_a(128 * wm + 32 * i + l32, chunk));
    if (!kBwd) {
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = ld_lds16(bs + swz_a(128 * wn + 32 * j + l32, chunk));
    } else {
      // rows 16 s + 8 lhi + 4 rr + (lane % 16) / 4, columns col0 .. col0 + 3
      const int rbase = 16 * s + 8 * lhi + ((lane & 15) >> 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col0 = 128 * wn + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int r0 = rbase, r1 = rbase + 4;
        fb[j] = ld_lds_tr(bs + swz_bt(r0, col0 >> 3) + (col0 & 7),
                          bs + swz_bt(r1, col0 >> 3) + (col0 & 7));
      }
    }
  };

  // ---- prologue: stage 0 in LDS, codes of step 1 in registers ---------------
  load_act(0);
  load_codes(0, c_cur, cp_cur, ok_cur);
  load_codes(1, c_nxt, cp_nxt, ok_nxt);
  {
#pragma unroll
    for (int i = 0; i < 8; ++i) store_act(As0, i);
    const Nf4Lut lut = make_lut(cp_cur);
#pragma unroll
    for (int w = 0; w < 4; ++w) store_w(Bs0, lut, w);
  }
  c_cur[0] = c_nxt[0];
  c_cur[1] = c_nxt[1];
  cp_cur = cp_nxt;
  ok_cur = ok_nxt;
  __syncthreads();

  u32x4_t fa[2][4], fb[2][4];
  load_frags(As0, Bs0, 0, fa[0], fb[0]);

  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const uint16_t* as = As0 + cur * kStageElems;
    const uint16_t* bs = Bs0 + cur * kStageElems;
    uint16_t* as_n = As0 + (cur ^ 1) * kStageElems;
    uint16_t* bs_n = Bs0 + (cur ^ 1) * kStageElems;
    const bool more = step + 1 < nsteps;
    if (more) load_act(step + 1);
    load_codes(step + 2, c_nxt, cp_nxt, ok_nxt);
    Nf4Lut lut;
    if (more) lut = make_lut(cp_cur);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int f = s & 1;
      if (s < 3) load_frags(as, bs, s + 1, fa[f ^ 1], fb[f ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[f][i], fb[f][j], acc[i][j]);
      if (more) {
        store_w(bs_n, lut, s);
        store_act(as_n, 2 * s);
        store_act(as_n, 2 * s + 1);
      }
    }
    c_cur[0] = c_nxt[0];
    c_cur[1] = c_nxt[1];
    cp_cur = cp_nxt;
    ok_cur = ok_nxt;
    __syncthreads();
    if (more) load_frags(as_n, bs_n, 0, fa[0], fb[0]);
  }

  // ---- epilogue: round to bf16 and store ------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + 128 * wn + 32 * j + l32;
      if (col < out_len) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * lhi + (e & 3);
          if (row < g.T)
            g.out[row * out_len + col] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

static unsigned num_tiles(int64_t T, int64_t out_len) {
  return (unsigned)(((T + BM - 1) / BM) * ((out_len + BN - 1) / BN));
}

hipError_t launch_qlora_fwd_gemm(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(qlora_gemm_kernel<false>, dim3(num_tiles(a.T, a.rows)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_qlora_dx_gemm(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(qlora_gemm_kernel<true>, dim3(num_tiles(a.T, a.cols)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace qlora
