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
// Operands, both read from LDS:
//   * activations (X or dY), 256 x 64 bf16 per step, are fetched straight
//     into LDS by buffer loads (no registers), two steps ahead, into a ring
//     of three 32 KB stages;
//   * the weight tile is dequantised once per workgroup into one of two
//     32 KB stages.  Each thread owns one block of 64 weights per step: its
//     32 bytes of packed codes arrive in registers two steps ahead; it builds
//     the 16-entry bf16 table q[k] * c' (16 float32 products rounded once,
//     as the bulk dequantiser does) and translates its nibbles with v_perm
//     byte lookups.  The tile keeps W's own row layout in both directions;
//     the backward reads its operand (reduction = W rows) with
//     ds_read_b64_tr_b16, which hands each lane 4 consecutive rows of one
//     column.
// All out-of-range rows and columns are handled by buffer-descriptor range
// checks (reads past the end return 0), so every 16-MFMA slice is a single
// basic block.  Within a slice the MFMAs are interleaved with the
// dequantisation VALU work, the LDS stores of the next stage and the
// fragment reads of the next slice (sched_group_barrier).  The one barrier
// per step sits before the last four MFMAs of the step, so the first
// fragments of the next step are read while they run.
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
constexpr int kAStages = 3;
constexpr int kBStages = 2;
constexpr uint32_t kOOB = 0x80000000u;         // buffer offset that reads as 0
constexpr int kVmemPerStep = 12;               // 8 activation DMAs + 4 code loads

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

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
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo);
  const uint2 h = __builtin_bit_cast(uint2, hi);
  return u32x4_t{l.x, l.y, h.x, h.y};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(n) lgkmcnt(0), then a workgroup barrier that is also a
// compiler memory barrier.  Outstanding LDS-DMA loads beyond the n newest
// are complete afterwards.
template <int N>
__device__ __forceinline__ void barrier_keep_vmem() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  asm volatile("s_barrier" ::: "memory");
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
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(kAStages + kBStages) * kStageElems];
  uint16_t* const As0 = smem;
  uint16_t* const Bs0 = smem + kAStages * kStageElems;

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

  // ---- LoRA seed: acc = (s L) R^T over r (L is pre-scaled) -----------------
  f32x16_t acc[4][4];
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

  // ---- buffer descriptors ---------------------------------------------------
  const int64_t rows_here = (g.T - m0) < BM ? (g.T - m0) : BM;
  const __amdgpu_buffer_rsrc_t act_rs =
      make_rsrc(g.act + m0 * red_len, (uint32_t)(rows_here * red_len * 2));
  const __amdgpu_buffer_rsrc_t codes_rs = make_rsrc(g.codes, (uint32_t)((g.rows * g.cols) >> 1));
  const __amdgpu_buffer_rsrc_t code8_rs = make_rsrc(g.code8, (uint32_t)(g.rows * kblocks));
  const __amdgpu_buffer_rsrc_t s2_rs =
      make_rsrc(g.s2, (uint32_t)(((g.rows * kblocks + 255) >> 8) * 4));

  // activation DMA of step `step` into stage (step % 3): wave w, load i covers
  // LDS bytes [(8 w + i) KB, +1 KB) of the stage, i.e. rows 8 (8 w + i) .. +8
  auto issue_act = [&](int step) {
    uint16_t* stage = As0 + (step % kAStages) * kStageElems;
    const int64_t k0 = (int64_t)step * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (wave * 8 + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      const int64_t k = k0 + 8 * c;
      const uint32_t off = (step < nsteps && k < red_len)
                               ? (uint32_t)((row * red_len + k) * 2) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_rs, (lds_void_t*)(stage + (wave * 8 + i) * 512),
                                               16, off, 0, 0, 0);
    }
  };

  // packed codes + block constant inputs of this thread's block at `step`
  struct CodeRegs {
    u32x4_t c0, c1;
    uint32_t code8;
    float s2;
    bool ok;
  };
  auto issue_codes = [&](int step, CodeRegs& r) {
    int64_t n, kc;
    if (!kBwd) {
      n = n0 + tid;
      kc = (int64_t)step * BK;
    } else {
      n = (int64_t)step * BK + (tid & 63);
      kc = n0 + 64 * (tid >> 6);
    }
    r.ok = step < nsteps && n < g.rows && kc < g.cols;
    const int64_t blk = n * kblocks + (kc >> 6);
    const uint32_t off = r.ok ? (uint32_t)((n * g.cols + kc) >> 1) : kOOB;
    const uint32_t off8 = r.ok ? (uint32_t)blk : kOOB;
    const uint32_t offs = r.ok ? (uint32_t)((blk >> 8) * 4) : kOOB;
    r.c0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(codes_rs, off, 0, 0));
    r.c1 = __builtin_bit_cast(u32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(codes_rs, off + 16, 0, 0));
    r.code8 = __builtin_amdgcn_raw_buffer_load_b8(code8_rs, off8, 0, 0);
    r.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(s2_rs, offs, 0, 0));
  };

  // dequantise words (2w, 2w+1) of `r` with `lut` into stage `bs`
  auto store_w = [&](uint16_t* bs, const Nf4Lut& lut, const CodeRegs& r, int w) {
    const u32x4_t& src = (w < 2) ? r.c0 : r.c1;
    uint32_t d0[4], d1[4];
    dequant8(lut, src[(2 * w) & 3], d0);
    dequant8(lut, src[(2 * w + 1) & 3], d1);
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
  auto lut_of = [&](const CodeRegs& r) {
    const float cp = r.ok ? block_constant(r.code8, r.s2, mu) : 0.0f;   // 0: invalid rows
    return make_lut(cp);
  };

  // MFMA fragments of slice s from stages (as, bs)
  auto load_frags = [&](const uint16_t* as, const uint16_t* bs, int s, u32x4_t* fa, u32x4_t* fb) {
    const int chunk = 2 * s + lhi;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = ld_lds16(as + swz_a(128 * wm + 32 * i + l32, chunk));
    if (!kBwd) {
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = ld_lds16(bs + swz_a(128 * wn + 32 * j + l32, chunk));
    } else {
      // rows 16 s + 8 lhi + 4 rr + (lane % 16) / 4, columns col0 .. col0 + 3
      const int r0 = 16 * s + 8 * lhi + ((lane & 15) >> 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col0 = 128 * wn + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        fb[j] = ld_lds_tr(bs + swz_bt(r0, col0 >> 3) + (col0 & 7),
                          bs + swz_bt(r0 + 4, col0 >> 3) + (col0 & 7));
      }
    }
  };

  // ---- prologue ------------------------------------------------------------
  CodeRegs cr_cur, cr_nxt;
  issue_act(0);
  issue_codes(0, cr_cur);
  issue_act(1);
  issue_codes(1, cr_nxt);
  {
    const Nf4Lut lut = lut_of(cr_cur);
#pragma unroll
    for (int w = 0; w < 4; ++w) store_w(Bs0, lut, cr_cur, w);
  }
  cr_cur = cr_nxt;
  barrier_keep_vmem<kVmemPerStep>();   // activation stage 0 complete

  u32x4_t fa[2][4], fb[2][4];
  load_frags(As0, Bs0, 0, fa[0], fb[0]);

  for (int step = 0; step < nsteps; ++step) {
    const uint16_t* as = As0 + (step % kAStages) * kStageElems;
    const uint16_t* bs = Bs0 + (step & 1) * kStageElems;
    const uint16_t* as_n = As0 + ((step + 1) % kAStages) * kStageElems;
    uint16_t* bs_n = Bs0 + ((step + 1) & 1) * kStageElems;

    issue_act(step + 2);
    issue_codes(step + 2, cr_nxt);
    const Nf4Lut lut = lut_of(cr_cur);

    // slices 0..2: 16 MFMAs each, interleaved with the next slice's fragment
    // reads and half of a word pair's dequantisation + stores
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int f = s & 1;
      load_frags(as, bs, s + 1, fa[f ^ 1], fb[f ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[f][i], fb[f][j], acc[i][j]);
      store_w(bs_n, lut, cr_cur, s);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // 5 VALU
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
      }
    }
    // slice 3: last word pair, then the barrier ahead of the final 4 MFMAs
    {
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[1][i], fb[1][j], acc[i][j]);
      store_w(bs_n, lut, cr_cur, 3);
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      barrier_keep_vmem<kVmemPerStep>();   // stage step+1 ready everywhere
      u32x4_t ga[4], gb[4];
      load_frags(as_n, bs_n, 0, ga, gb);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[3][j] = mfma32(fa[1][3], fb[1][j], acc[3][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[0][i] = ga[i];
        fb[0][i] = gb[i];
      }
    }
    cr_cur = cr_nxt;
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
