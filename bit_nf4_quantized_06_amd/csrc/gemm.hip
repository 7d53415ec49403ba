// Fused NF4-dequant GEMMs of the QLoRA linear layer (gfx950, bf16 MFMA).
//
//   forward:      Y  = X  dequant(W)^T + (s X A^T) B^T
//   backward dX:  dX = dY dequant(W)   + (s dY B)  A
// ta-paperlens 勾配は実際どこへ行くのか: each matmul dequantises the NF4 blocks it
// needs to bf16, uses them and drops them; the input gradient goes through
// dequant(W)^T; W is never written.  Ultralytics "So funktioniert QLoRA":
// dequantise right before the matmul and add the LoRA path.
//
// Kernel shape.  A workgroup of 8 waves computes a 256-token x 256-column
// output tile with float32 accumulators; the reduction advances 64 per step,
// i.e. one NF4 block per weight row.  Waves w and w + 4 share a SIMD and
// split one 128 x 128 quadrant into two 128 x 64 halves (4 x 2 MFMA
// 32x32x16 blocks, 128 AGPRs each).  With two waves per SIMD one wave's
// MFMAs keep the matrix core busy while the other waits on its loads, its
// LDS traffic or the dequantisation work; a single wave per SIMD cannot hide
// the VMEM issue stalls of the activation stream.
//
// Operands, both read from LDS:
//   * activations (X or dY), 256 x 64 bf16 per step, are fetched straight
//     into LDS by buffer loads (no registers), two steps ahead, into a ring
//     of three 32 KB stages (4 loads of 1 KB per wave and step);
//   * the weight tile is dequantised once per workgroup into one of two
//     32 KB stages.  Each pair of adjacent lanes owns one block of 64
//     weights per step, each lane 32 of them: its 16 bytes of packed codes
//     arrive in registers two steps ahead; it builds the 16-entry bf16 table
//     q[k] * c' (16 float32 products rounded once, as the bulk dequantiser
//     does) and translates its nibbles with v_perm byte lookups.  The tile
//     keeps W's own row layout in both directions; the backward reads its
//     operand (reduction = W rows) with ds_read_b64_tr_b16, which hands each
//     lane 4 consecutive rows of one column.
// From 2048 tokens on the library dequantises the whole weight once per call
// (kPreDq): the weight tile then arrives by DMA like the activations, into
// the same layout the decode writes, and the slices hold only MFMAs and
// fragment reads; tile, layouts, seed, split and epilogue are shared, so
// both paths give the same bits.
// Each tile starts from the LoRA product: the accumulators are seeded with
// (s L) R^T over the r adapter columns, whose 256 x 64 operand tiles arrive
// by DMA into the two stages the prologue leaves idle, issued ahead of the
// first stages' loads, so the seed waits for one memory round trip (loading
// its fragments from global memory 16 columns at a time took four, about
// 8 us of every round of tiles).
// All out-of-range rows and columns are handled by buffer-descriptor range
// checks (reads past the end return 0), so every 8-MFMA slice is a single
// basic block.  Within a slice the MFMAs are interleaved with the
// dequantisation VALU work, the LDS store of the next stage and the fragment
// reads of the next slice (sched_group_barrier).  The one barrier per step
// sits before the last two MFMAs of the step, so the first fragments of the
// next step are read while they run.
//
// LDS layouts (16-byte chunks XOR-swizzled).  The bank conflict counter
// shows 16-byte reads served 16 lanes (256 bytes) per cycle and 16-byte
// writes 8 lanes (128 bytes) per cycle; both layouts are conflict-free for
// every access below under those rules (measured: 0 conflict cycles):
//   activation / forward weight tile: 256 rows x 8 chunks (128 B a row),
//       chunk' = chunk ^ g(row), g(row) = ((row >> 1) & 7) ^ ((row & 1) << 1):
//       g takes all 8 values on the rows of one parity within 16 (fragment
//       reads: 16 rows, one chunk) and distinct low two bits on 4 aligned
//       rows (weight stores: 4 rows x 2 half-blocks);
//   backward weight tile: 64 rows (W rows) x 32 chunks (256 W columns),
//       chunk' = chunk ^ (((row & 3) << 2) | ((row & 3) ^ (((row >> 2) & 1) << 1))):
//       distinct bits 2-3 on 4 aligned rows (transposed reads), distinct
//       low bits on 4 aligned rows and on the 4 rows {r, r ^ 1, r + 4,
//       (r ^ 1) + 4} (weight stores).  The previous layouts, each tuned for
//       its reads alone, spent 19.5% (forward) and 42% (backward) of the
//       LDS cycles in bank conflicts; removing them took 1% and 3% off the
//       two GEMMs.
//
// Workgroups are numbered so that the 32 consecutive tiles a single XCD
// receives (dispatch is round-robin over the 8 XCDs) form a compact block
// of 4 token tiles x 8 column tiles, keeping their shared operand tiles in
// that XCD's L2.
#include "abi_internal.h"
#include "device_common.h"
#include "kernels.h"

namespace qlora {

constexpr int BM = kGemmTileTokens;   // 256 tokens per tile
constexpr int BN = kGemmTileOut;      // 256 outputs per tile
constexpr int BK = 64;
constexpr int kStageElems = BM * BK;           // 16384 bf16 = 32 KB
constexpr int kAStages = 3;
constexpr int kBStages = 2;
constexpr uint32_t kOOB = 0x80000000u;         // buffer offset that reads as 0
constexpr int kThreads = 512;                  // 8 waves
constexpr int kActLoads = 4;                   // activation DMAs per wave and step
// memory loads per reduction step of the in-LDS decode: the activation DMAs,
// the codes, the group scale (float32 block constant without double
// quantisation) and, with double quantisation, the 8-bit block code.  The
// explicit wait counts are built from this, so every one of these loads is
// issued and used (none may be dropped by the compiler as dead).
template <bool kDQ>
constexpr int vmem_per_step() { return kActLoads + (kDQ ? 3 : 2); }

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz_g(int row) {   // activation / forward weight tile
  return ((row >> 1) & 7) ^ ((row & 1) << 1);
}
__device__ __forceinline__ int swz_a(int row, int chunk) {
  return row * BK + ((chunk ^ swz_g(row)) << 3);
}
__device__ __forceinline__ int swz_bt_g(int row) {   // backward weight tile
  return ((row & 3) << 2) | ((row & 3) ^ (((row >> 2) & 1) << 1));
}
__device__ __forceinline__ int swz_bt(int row, int chunk) {
  return row * BN + ((chunk ^ swz_bt_g(row)) << 3);
}

__device__ __forceinline__ u32x4_t ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x4_t ld_lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <bool kF16>
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return mfma32x32<kF16>(a, b, c);
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

// Everything one workgroup needs across steps.  The five LDS stages are
// separate objects and every stage index is a compile-time constant (the
// step loop is unrolled by 6 = lcm(3, 2)), so the compiler can tell an
// activation DMA into one stage from LDS traffic on another and does not
// insert waits for outstanding DMA loads before unrelated LDS accesses.
template <bool kBwd>
struct GemmCtx {
  const GemmArgs& g;
  uint16_t* A[kAStages];
  uint16_t* B[kBStages];
  int tid, lane, wave, wm, wn, wg, l32, lhi, nsteps;
  int kstep0;               // first reduction step of this unit (K-split halves)
  int64_t m0, n0, red_len, kblocks;
  float mu;
  // buffer ranges (base, bytes) of the operands read with range checking
  const uint16_t* act_base;
  uint32_t act_bytes, codes_bytes, code8_bytes, s2_bytes;
  // weight already dequantised to 16 bit (kPreDq): its range and, in the
  // backward, the lane offsets of the step's four loads
  const uint16_t* w_base;
  uint32_t w_bytes;
  uint32_t w_voff[4];
  // per-lane byte offsets that do not change with the step
  uint32_t act_voff[2];     // activation DMA, even / odd 8-row block
  uint32_t code_voff;       // this lane's 16 code bytes at step 0
  int64_t blk0;             // this lane's block index at step 0
  bool w_row_ok;            // this lane's weight block lies inside W
  int wrow;                 // backward: W row of the block within the step
  // forward only (the backward keeps a whole table per lane: its transposed
  // fragments leave no registers for the split):
  float kq[kBwd ? 1 : 8];   // NF4 levels 8h .. 8h+7 of this lane's table half
  uint32_t code_flip;       // 0x88888888 on lanes holding the upper table half first
  // per-lane LDS element offsets inside a stage (loop invariant); the row
  // blocks i (+32 rows), column blocks j and, in the backward weight tile,
  // the slices (+16 rows) are constant additions folded into instruction
  // offsets
  int a_frag[4];            // activation fragment, slice s, row block 0
  int b_frag[4];            // forward: [s]; backward: [2 j + rr] for slice 0
  int w_store[4];           // dequantised chunk w of this lane's half block
};

struct CodeRegs {
  u32x4_t c;                // 32 codes: 4 words of 8
  uint32_t code8;
  float s2;
  bool ok;
};

// Activation DMA of step `step` into `stage`: wave w, load i fills LDS bytes
// [(4 w + i) KB, +1 KB) of the stage, i.e. tile rows 8 (4 w + i) .. +8.  The
// swizzle of a row only depends on the lane and on the parity of i, so each
// lane has two fixed byte offsets; the row block and the step enter through
// the scalar offset.  Columns past the end of the reduction (the last step
// of a backward whose weight has rows % 64 != 0) read real neighbouring
// data; the matching rows of the dequantised weight tile are exactly 0.
// Steps past the end read nothing (scalar offset beyond the range: zeros).
template <bool kBwd>
__device__ __forceinline__ void issue_act(const GemmCtx<kBwd>& c, uint16_t* stage, int step) {
  const uint32_t sbase = step < c.nsteps ? (uint32_t)((c.kstep0 + step) * BK * 2) : kOOB;
  const uint32_t row_bytes = (uint32_t)(c.red_len * 2);
#pragma unroll
  for (int i = 0; i < kActLoads; ++i) {
    const int blk8 = c.wave * kActLoads + i;
    const uint32_t soff = step < c.nsteps ? sbase + (uint32_t)(blk8 * 8) * row_bytes : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(c.act_base, c.act_bytes),
                                             (lds_void_t*)(stage + blk8 * 512), 16,
                                             c.act_voff[i & 1], soff, 0, 0);
  }
}

// Weight DMA of step `step` from a weight already dequantised to 16 bit, in
// the layout the in-kernel dequantisation writes.  Forward: the same tile
// shape as the activations (W rows n0 .. n0+255, 64 columns; load i of wave
// w fills W rows 8 (4 w + i) .. +8, the lane offsets are the activation
// ones).  Backward: W rows 64 step .. +64 by columns n0 .. n0+255 (512 B a
// row); load i of wave w fills tile rows 2 (4 w + i) and +1, lane l writes
// row 2 (4 w + i) + l / 32 at chunk position l % 32 and so fetches chunk
// (l % 32) ^ swz_bt_g(row), which only depends on i and l.  Rows past the
// end of W land past w_bytes and read 0 (range check), as do steps past the
// end.  The host takes this path only for fewer than 2^30 weights and at
// most 2^20 columns, so every offset stays below 2^31 + 2^29.  Loads I0 ..
// I1 - 1 of the wave's four.
template <int I0, int I1, bool kBwd>
__device__ __forceinline__ void issue_wdq(const GemmCtx<kBwd>& c, uint16_t* stage, int step) {
  const bool in = step < c.nsteps;
  const uint32_t ks = (uint32_t)(c.kstep0 + step);
  const uint32_t row_bytes = (uint32_t)(c.g.cols * 2);
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const int blk = c.wave * kActLoads + i;
    const uint32_t o = kBwd ? (ks * 64 + 2 * (uint32_t)blk) * row_bytes
                            : ks * (BK * 2) + 8 * (uint32_t)blk * row_bytes;
    const uint32_t soff = in ? o : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(c.w_base, c.w_bytes),
                                             (lds_void_t*)(stage + blk * 512), 16,
                                             kBwd ? c.w_voff[i] : c.act_voff[i & 1], soff, 0, 0);
  }
}

// packed codes and block-constant inputs of this lane's half block at `step`
// (kDQ false: the group-scale slot receives the block's float32 constant and
// there is no 8-bit code)
template <bool kBwd, bool kDQ>
__device__ __forceinline__ void issue_codes(const GemmCtx<kBwd>& c, int step, CodeRegs& r) {
  // forward: the block moves along the row (+32 B, +1 block per step);
  // backward: it moves down 64 rows (+64 rows of codes and constants)
  const bool in = step < c.nsteps;
  const int64_t ks = (int64_t)c.kstep0 + step;   // reduction step within the whole weight
  const int64_t dblk = kBwd ? ks * 64 * c.kblocks : ks;
  const uint32_t dcode = kBwd ? (uint32_t)(ks * 64 * (c.g.cols >> 1)) : (uint32_t)(ks * 32);
  const int64_t n_ok_rows = c.g.rows - (kBwd ? ks * 64 : 0);
  r.ok = in && c.w_row_ok && (!kBwd || c.wrow < n_ok_rows);
  const uint32_t scode = in ? dcode : kOOB;
  const int64_t blk = c.blk0 + dblk;
  r.c = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                        make_rsrc(c.g.codes, c.codes_bytes), c.code_voff, scode, 0));
  if constexpr (kDQ)
    r.code8 = __builtin_amdgcn_raw_buffer_load_b8(make_rsrc(c.g.code8, c.code8_bytes),
                                                  r.ok ? (uint32_t)blk : kOOB, 0, 0);
  else
    r.code8 = 0u;
  r.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       make_rsrc(c.g.s2, c.s2_bytes),
                                       r.ok ? scale_offset<kDQ>(blk) : kOOB, 0, 0));
}

// Table of this lane pair's block.  Forward: lane half h = lane & 1 forms
// entries 8h .. 8h+7 (kq = those levels) as byte planes, the neighbour lane
// supplies the other 8 (DPP quad_perm [1,0,3,2]); lanes with h = 1 hold the
// two halves swapped and flip bit 3 of their codes instead (code_flip).
// Backward: the whole table per lane.
template <bool kBwd, bool kDQ, bool kF16>
__device__ __forceinline__ Nf4Lut lut_of(const GemmCtx<kBwd>& c, const CodeRegs& r) {
  // 0: rows past the end
  const float cp = weight_constant_or_zero<kDQ>(r.ok, r.code8, r.s2, c.mu);
  if (kBwd) return make_lut<kF16>(cp);
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pack16x2<kF16>(__fmul_rn(c.kq[2 * j], cp), __fmul_rn(c.kq[2 * j + 1], cp));
  uint32_t own[4], nb[4];
  own[0] = perm(p[1], p[0], 0x06040200u);   // low bytes of own entries 0..3
  own[1] = perm(p[3], p[2], 0x06040200u);   // low bytes of own entries 4..7
  own[2] = perm(p[1], p[0], 0x07050301u);   // high bytes
  own[3] = perm(p[3], p[2], 0x07050301u);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    nb[q] = (uint32_t)__builtin_amdgcn_mov_dpp((int)own[q], 0xB1, 0xF, 0xF, false);
  Nf4Lut t;
  t.lo[0] = own[0];
  t.lo[1] = own[1];
  t.lo[2] = nb[0];
  t.lo[3] = nb[1];
  t.hi[0] = own[2];
  t.hi[1] = own[3];
  t.hi[2] = nb[2];
  t.hi[3] = nb[3];
  return t;
}

// dequantise word w of `r` (8 weights) into weight stage `bs`
template <bool kBwd>
__device__ __forceinline__ void store_w(const GemmCtx<kBwd>& c, uint16_t* bs, const Nf4Lut& lut,
                                        const CodeRegs& r, int w) {
  uint32_t d[4];
  dequant8(lut, kBwd ? r.c[w] : (r.c[w] ^ c.code_flip), d);
  *reinterpret_cast<u32x4_t*>(bs + c.w_store[w]) = u32x4_t{d[0], d[1], d[2], d[3]};
}

// MFMA fragments of slice s from stages (as, bs); the two weight fragments
// first: the slice's first MFMAs use both of them and the first activation
// fragment, so they can start after 3 of the 6 reads, which matters right
// after the step barrier, when every wave reads at once
template <bool kBwd>
__device__ __forceinline__ void load_frags(const GemmCtx<kBwd>& c, const uint16_t* as,
                                           const uint16_t* bs, int s, u32x4_t* fa, u32x4_t* fb) {
  if (!kBwd) {
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = ld_lds16(bs + c.b_frag[s] + 32 * j * BK);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = ld_lds_tr(bs + c.b_frag[2 * j] + 16 * s * BN, bs + c.b_frag[2 * j + 1] + 16 * s * BN);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = ld_lds16(as + c.a_frag[s] + 32 * i * BK);
}

// Interleave pattern of one 8-MFMA slice: each MFMA is followed by `V`
// VALU ops; the first NR also carry one LDS read (next slice's fragments),
// the first NM one VMEM load, and the last MFMA the LDS store (after MFMA 7
// rather than 5 or 3: -2 us and +7 us per attn_4096 step respectively
// against 5, measured in pairs).
template <int V, int NR, int NM>
__device__ __forceinline__ void slice_schedule() {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (q < NM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if (q == 7) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  }
}

// One reduction step on activation stage SA and weight stage SB.  On entry
// fa[0], fb[0] hold slice 0 of this step and `cur` the codes of step+1; on
// exit fa[0], fb[0] hold slice 0 of step+1 and `nxt` the codes of step+2
// (the caller swaps the two register sets for the next step: no copy, so
// nothing waits for the codes before they are used a step later).
template <bool kBwd, bool kDQ, bool kF16, int SA, int SB>
__device__ __forceinline__ void gemm_step(const GemmCtx<kBwd>& c, int step, f32x16_t (&acc)[4][2],
                                          u32x4_t (&fa)[2][4], u32x4_t (&fb)[2][2],
                                          CodeRegs& cur, CodeRegs& nxt) {
#if defined(__HIP_DEVICE_COMPILE__)   // device-only builtins; the host pass needs no body
  constexpr int kReads = kBwd ? 8 : 6;   // LDS read instructions per slice
  const uint16_t* as = c.A[SA];
  const uint16_t* bs = c.B[SB];
  uint16_t* as_next = c.A[(SA + 1) % kAStages];
  uint16_t* bs_next = c.B[(SB + 1) % kBStages];

  // Wave priority 1 through the step's slices, 0 from the barrier on: when
  // the two waves of a SIMD are in different phases, the one still working
  // through its MFMA slices issues first and the one waiting at (or just
  // past) the barrier yields.  Measured: -2 to -6 us per attn_4096 step in
  // three interleaved pairs; priority 3 was no different.
  __builtin_amdgcn_s_setprio(1);
  // slice 0: loads for step+2, the block table for step+1
  issue_act(c, c.A[(SA + 2) % kAStages], step + 2);
  issue_codes<kBwd, kDQ>(c, step + 2, nxt);
  const Nf4Lut lut = lut_of<kBwd, kDQ, kF16>(c, cur);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int f = s & 1;
    load_frags(c, as, bs, s + 1, fa[f ^ 1], fb[f ^ 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(fa[f][i], fb[f][j], acc[i][j]);
    store_w(c, bs_next, lut, cur, s);
    // 8 VALU ops per MFMA in the slice that also issues the step's memory
    // loads, 5 in the others (a sweep of 3..7 found 5..7 alike, about 2 us
    // per step ahead of 4, and 3 behind)
    if (s == 0)
      slice_schedule<8, kReads, vmem_per_step<kDQ>()>();
    else
      slice_schedule<5, kReads, 0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  // slice 3: 6 MFMAs with the last word, barrier, next step's first
  // fragments under the remaining 2 MFMAs
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(fa[1][i], fb[1][j], acc[i][j]);
  store_w(c, bs_next, lut, cur, 3);
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    if (q == 4) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  barrier_keep_vmem<vmem_per_step<kDQ>()>();   // stage step+1 complete and visible
  u32x4_t ga[4], gb[2];
  load_frags(c, as_next, bs_next, 0, ga, gb);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[3][j] = mfma32<kF16>(fa[1][3], fb[1][j], acc[3][j]);
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = ga[i];
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[0][j] = gb[j];
#endif
}

// One reduction step when the weight arrives dequantised (kPreDq): both
// operands come by DMA and the slices hold only MFMAs and their fragment
// reads.  Here the three-stage ring (A) holds the weight and the two-stage
// ring (B) the activations: a weight tile is shared by the 4 token tiles an
// XCD runs beside it, an activation tile by 8 column tiles, so weight loads
// miss the L2 more often and get the longer prefetch.  Slice 0 issues the
// activation tile of step+1 into the activation stage the previous step read
// (free since that step's barrier), slices 1 and 2 the weight tile of step+2
// (two loads each); the barrier, before the step's last four MFMAs, waits
// for all but the newest 4 loads (the weight tile of step+2).
template <int NR, int NM>
__device__ __forceinline__ void dma_slice_schedule() {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (q < NM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

template <bool kBwd, bool kF16, int SA, int SB>
__device__ __forceinline__ void gemm_step_dma(const GemmCtx<kBwd>& c, int step,
                                              f32x16_t (&acc)[4][2], u32x4_t (&fa)[2][4],
                                              u32x4_t (&fb)[2][2]) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kReads = kBwd ? 8 : 6;
  const uint16_t* ws = c.A[SA];
  const uint16_t* xs = c.B[SB];
  uint16_t* ws_next = c.A[(SA + 1) % kAStages];
  uint16_t* xs_next = c.B[(SB + 1) % kBStages];
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int f = s & 1;
    if (s == 0) issue_act(c, xs_next, step + 1);
    if (s == 1) issue_wdq<0, 2>(c, c.A[(SA + 2) % kAStages], step + 2);
    if (s == 2) issue_wdq<2, 4>(c, c.A[(SA + 2) % kAStages], step + 2);
    load_frags(c, xs, ws, s + 1, fa[f ^ 1], fb[f ^ 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(fa[f][i], fb[f][j], acc[i][j]);
    if (s == 0)
      dma_slice_schedule<kReads, kActLoads>();
    else
      dma_slice_schedule<kReads, 2>();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(fa[1][i], fb[1][j], acc[i][j]);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  barrier_keep_vmem<kActLoads>();   // stages of step+1 complete and visible
  u32x4_t ga[4], gb[2];
  load_frags(c, xs_next, ws_next, 0, ga, gb);
#pragma unroll
  for (int i = 2; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(fa[1][i], fb[1][j], acc[i][j]);
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = ga[i];
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[0][j] = gb[j];
#endif
}

template <bool kBwd, bool kDQ, bool kF16, bool kPreDq, int SA, int SB>
__device__ __forceinline__ void run_step(const GemmCtx<kBwd>& c, int step, f32x16_t (&acc)[4][2],
                                         u32x4_t (&fa)[2][4], u32x4_t (&fb)[2][2],
                                         CodeRegs& cur, CodeRegs& nxt) {
  if constexpr (kPreDq)
    gemm_step_dma<kBwd, kF16, SA, SB>(c, step, acc, fa, fb);
  else
    gemm_step<kBwd, kDQ, kF16, SA, SB>(c, step, acc, fa, fb, cur, nxt);
}

// kDrop (backward only): the seed is multiplied element-wise by the
// lora_dropout keep mask (g.keep) before the main loop.  kDQ: double-
// quantised block constants (else float32 constants); kF16: fp16 operands,
// tables and output (else bf16); kPreDq: the weight arrives dequantised to
// 16 bit (g.wdq, [rows, cols]) and is fetched by DMA like the activations
// (kDQ then unused).
template <bool kBwd, bool kDrop, bool kDQ, bool kF16, bool kPreDq>
__global__ __launch_bounds__(kThreads, 1) void qlora_gemm_kernel(GemmArgs g) {
  // The body is compiled in the device pass only: the host pass needs just
  // the kernel's signature, and it cannot instantiate the gfx950
  // buffer-resource helpers for more than one kernel with the same helper
  // arguments.
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t sa1[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t sa2[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t sb0[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t sb1[kStageElems];

  GemmCtx<kBwd> c{g, {sa0, sa1, sa2}, {sb0, sb1}};
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  // wave index through readfirstlane: provably uniform, so the DMA scalar
  // offsets and LDS bases derived from it stay in SGPRs
  c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  const int simd = c.wave & 3;   // waves w and w + 4 share a SIMD
  c.wm = simd >> 1;
  c.wn = simd & 1;
  c.wg = c.wave >> 2;            // which 64-column half of the quadrant
  c.l32 = c.lane & 31;
  c.lhi = c.lane >> 5;
  c.red_len = kBwd ? g.rows : g.cols;
  const int64_t out_len = kBwd ? g.cols : g.rows;
  const int mt = (int)((g.T + BM - 1) / BM);
  const int nt = (int)((out_len + BN - 1) / BN);
  // units past split_from are the two reduction halves of the tiles from
  // split_from on
  int q = blockIdx.x;
  int half = -1;
  if (q >= g.split_from) {
    const int u = q - g.split_from;
    q = g.split_from + (u >> 1);
    half = u & 1;
  }
  q = __builtin_amdgcn_readfirstlane(q);
  half = __builtin_amdgcn_readfirstlane(half);
  int tm, tn;
  tile_coords(q, mt, nt, tm, tn);
  // the divisions in tile_coords run on the vector unit; without this the
  // tile origin, and with it the activation descriptor, would sit in VGPRs
  // and every DMA would be wrapped in a waterfall loop
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  c.m0 = (int64_t)tm * BM;
  c.n0 = (int64_t)tn * BN;
  {
    const int all = (int)((c.red_len + BK - 1) / BK);
    const int first = all >> 1;
    c.kstep0 = half == 1 ? first : 0;
    c.nsteps = half < 0 ? all : (half == 0 ? first : all - first);
  }
  c.kblocks = g.cols >> 6;
  c.mu = kDQ ? g.mu[0] : 0.0f;
  const int64_t rows_here = (g.T - c.m0) < BM ? (g.T - c.m0) : BM;
  const int col0 = 128 * c.wn + 64 * c.wg;   // first output column of this wave in the tile
  {
    // activation DMA lane offsets (see issue_act): row-in-block = lane / 8,
    // swizzle g(row) with row bit 3 = parity of the load index
    const int rl = c.lane >> 3;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = 8 * par + rl;
      const int ch = (c.lane & 7) ^ swz_g(row);
      c.act_voff[par] = (uint32_t)((rl * c.red_len + 8 * ch) * 2);
    }
    // weight block of this lane pair: b = tid / 2, half h = tid % 2
    const int b = c.tid >> 1;
    const int h = c.tid & 1;
    if (!kBwd) {
#pragma unroll
      for (int j = 0; j < 8; ++j) c.kq[j] = h ? kNF4[8 + j] : kNF4[j];
    }
    c.code_flip = (!kBwd && h) ? 0x88888888u : 0u;
    int64_t n, kc;
    if (!kBwd) {
      n = c.n0 + b;              // W row
      kc = 32 * h;               // column within the step's block
      c.wrow = 0;
    } else {
      n = b & 63;                // W row within the step
      kc = c.n0 + 64 * (b >> 6) + 32 * h;
      c.wrow = b & 63;
    }
    c.w_row_ok = kBwd ? kc < g.cols : n < g.rows;   // backward rows are checked per step
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) c.a_frag[sl] = swz_a(128 * c.wm + c.l32, 2 * sl + c.lhi);
    if (!kBwd) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) c.b_frag[sl] = swz_a(col0 + c.l32, 2 * sl + c.lhi);
#pragma unroll
      for (int w = 0; w < 4; ++w) c.w_store[w] = swz_a(b, 4 * h + w);
    } else {
      // tr16 source lane: row 8 lhi + 4 rr + (lane % 16) / 4, columns cc .. cc + 3
      const int r0 = 8 * c.lhi + ((c.lane & 15) >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = col0 + 32 * j + 16 * ((c.lane >> 4) & 1) + 4 * (c.lane & 3);
        c.b_frag[2 * j] = swz_bt(r0, cc >> 3) + (cc & 7);
        c.b_frag[2 * j + 1] = swz_bt(r0 + 4, cc >> 3) + (cc & 7);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) c.w_store[w] = swz_bt(b & 63, 8 * (b >> 6) + 4 * h + w);
    }
    c.code_voff = c.w_row_ok ? (uint32_t)((n * g.cols + kc) >> 1) : kOOB;
    c.blk0 = n * (g.cols >> 6) + (kc >> 6);
  }
  if (kPreDq) {
    if (!kBwd) {
      const int64_t wr = (g.rows - c.n0) < BN ? (g.rows - c.n0) : BN;
      c.w_base = g.wdq + c.n0 * g.cols;
      c.w_bytes = __builtin_amdgcn_readfirstlane((uint32_t)(wr * g.cols * 2));
    } else {
      c.w_base = g.wdq + c.n0;
      c.w_bytes = __builtin_amdgcn_readfirstlane((uint32_t)((g.rows * g.cols - c.n0) * 2));
#pragma unroll
      for (int i = 0; i < kActLoads; ++i) {
        const int ch = (c.lane & 31) ^ swz_bt_g(2 * i + c.lhi);
        c.w_voff[i] = (uint32_t)((c.lhi * g.cols + 8 * ch) * 2);
      }
    }
  }
  c.act_base = g.act + c.m0 * c.red_len;
  c.act_bytes = (uint32_t)(rows_here * c.red_len * 2);
  c.codes_bytes = (uint32_t)((g.rows * g.cols) >> 1);
  c.code8_bytes = (uint32_t)(g.rows * c.kblocks);
  c.s2_bytes = kDQ ? (uint32_t)(((g.rows * c.kblocks + 255) >> 8) * 4)
                  : (uint32_t)(g.rows * c.kblocks * 4);
  const int l32 = c.l32, lhi = c.lhi, wm = c.wm;
  const int64_t m0 = c.m0, n0 = c.n0;

  // ---- LoRA seed operands: acc = (s L) R^T over r (L is pre-scaled).  The
  // 256 x 64 tiles of L (tokens m0 ..) and R (outputs n0 ..) for the first
  // 64 of the r columns go by DMA into the two stages the prologue leaves
  // idle (sa2, sb1), in the activation tile layout, ahead of the prologue's
  // own loads: the seed then costs one memory round trip instead of one per
  // 16 columns.  Rows past T or out_len lie past the range and read 0; the
  // columns past r of a row are never read.  (The second reduction half of
  // a split tile starts from zero and loads nothing.)
  const int seed_r = half == 1 ? 0 : g.r;
  uint16_t* const seed_l = sa2;
  uint16_t* const seed_rt = sb1;
  const int64_t outs_here = (out_len - c.n0) < BN ? (out_len - c.n0) : BN;
  uint32_t seed_voff[2];
  {
    const int rl = c.lane >> 3;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = 8 * par + rl;
      const int ch = (c.lane & 7) ^ swz_g(row);
      seed_voff[par] = (uint32_t)((rl * g.r + 8 * ch) * 2);
    }
  }
  const __amdgpu_buffer_rsrc_t l_rsrc =
      make_rsrc(g.lora_l + c.m0 * g.r, (uint32_t)(rows_here * g.r * 2));
  const __amdgpu_buffer_rsrc_t r_rsrc =
      make_rsrc(g.lora_r + c.n0 * g.r, (uint32_t)(outs_here * g.r * 2));
  auto issue_seed = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kActLoads; ++i) {
      const int blk8 = c.wave * kActLoads + i;
      const uint32_t soff = (uint32_t)((blk8 * 8 * g.r + c0) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(l_rsrc, (lds_void_t*)(seed_l + blk8 * 512), 16,
                                               seed_voff[i & 1], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_rsrc, (lds_void_t*)(seed_rt + blk8 * 512), 16,
                                               seed_voff[i & 1], soff, 0, 0);
    }
  };
  if (seed_r > 0) issue_seed(0);

  // ---- first loads: the stages of steps 0 and 1 (and the codes of both)
  CodeRegs ca, cb;   // codes of even / odd steps
  if (kPreDq) {
    // weight ring A, activation ring B (see gemm_step_dma)
    issue_wdq<0, kActLoads>(c, sa0, 0);
    issue_act(c, sb0, 0);
    issue_wdq<0, kActLoads>(c, sa1, 1);
  } else {
    issue_act(c, sa0, 0);
    issue_codes<kBwd, kDQ>(c, 0, ca);
    issue_act(c, sa1, 1);
    issue_codes<kBwd, kDQ>(c, 1, cb);
  }
  constexpr int kPrologueLoads = kPreDq ? 3 * kActLoads : 2 * vmem_per_step<kDQ>();

  // ---- LoRA seed -----------------------------------------------------------
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  {
    // forward-layout fragment offsets of R (the backward's weight fragments
    // use another layout)
    int rfrag[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) rfrag[sl] = swz_a(col0 + l32, 2 * sl + lhi);
    for (int c0 = 0; c0 < seed_r; c0 += BK) {
      if (c0 == 0) {
        barrier_keep_vmem<kPrologueLoads>();   // this wave's seed DMAs landed, and every wave's
      } else {
        __syncthreads();                       // every wave done reading the previous columns
        issue_seed(c0);
        barrier_keep_vmem<0>();
      }
      const int ns = (seed_r - c0) >= BK ? 4 : (seed_r - c0) >> 4;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (sl < ns) {
          u32x4_t af[4], bf[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) bf[j] = ld_lds16(seed_rt + rfrag[sl] + 32 * j * BK);
#pragma unroll
          for (int i = 0; i < 4; ++i) af[i] = ld_lds16(seed_l + c.a_frag[sl] + 32 * i * BK);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<kF16>(af[i], bf[j], acc[i][j]);
        }
      }
    }
  }
  if (kDrop && half != 1) {
    // the keep mask has one nibble per 4 tokens x 1 feature, exactly the 4
    // consecutive rows of one column a lane holds per accumulator group.
    // One batch of 8 byte loads per row block i (indices clamped, so the
    // batch issues back to back; clamped rows and columns are never
    // stored), applied before the next batch: few live registers beside
    // the accumulators.
    // (the lane indices pass through an empty asm so these index
    // expressions are not merged with the epilogue's, which would keep them
    // live across the main loop)
    int dl32 = l32, dlhi = lhi;
    asm volatile("" : "+v"(dl32), "+v"(dlhi));
    const int64_t quad_bytes = out_len >> 1;
    int64_t col_off[2];
    uint32_t col_shift[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int64_t col = n0 + col0 + 32 * j + dl32;
      col = col < out_len ? col : out_len - 1;
      col_off[j] = col >> 1;
      col_shift[j] = 4u * (uint32_t)(col & 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t nib[2][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int64_t row = m0 + 128 * wm + 32 * i + 8 * q + 4 * dlhi;
        row = row < g.T ? row : g.T - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          nib[j][q] = (uint32_t)g.keep[(row >> 2) * quad_bytes + col_off[j]] >> col_shift[j];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc[i][j][e] = ((nib[j][e >> 2] >> (e & 3)) & 1u) ? acc[i][j][e] : 0.0f;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- prologue: step 0's weight tile ----------------------------------------
  if (!kPreDq) {
    const Nf4Lut lut = lut_of<kBwd, kDQ, kF16>(c, ca);
#pragma unroll
    for (int w = 0; w < 4; ++w) store_w(c, sb0, lut, ca, w);
  }
  // activation stage 0 (and the DMA'd weight stage 0) complete
  barrier_keep_vmem<kPreDq ? kActLoads : vmem_per_step<kDQ>()>();

  u32x4_t fa[2][4], fb[2][2];
  if (kPreDq)
    load_frags(c, sb0, sa0, 0, fa[0], fb[0]);
  else
    load_frags(c, sa0, sb0, 0, fa[0], fb[0]);

  // whole groups of 6 steps (the stage cycle) in a loop without exits, so
  // each step's tail and the next step's head share one basic block; then
  // the last nsteps % 6 steps
  int step = 0;
  for (; step + 6 <= c.nsteps; step += 6) {
    run_step<kBwd, kDQ, kF16, kPreDq, 0, 0>(c, step, acc, fa, fb, cb, ca);
    run_step<kBwd, kDQ, kF16, kPreDq, 1, 1>(c, step + 1, acc, fa, fb, ca, cb);
    run_step<kBwd, kDQ, kF16, kPreDq, 2, 0>(c, step + 2, acc, fa, fb, cb, ca);
    run_step<kBwd, kDQ, kF16, kPreDq, 0, 1>(c, step + 3, acc, fa, fb, ca, cb);
    run_step<kBwd, kDQ, kF16, kPreDq, 1, 0>(c, step + 4, acc, fa, fb, cb, ca);
    run_step<kBwd, kDQ, kF16, kPreDq, 2, 1>(c, step + 5, acc, fa, fb, ca, cb);
  }
  if (step < c.nsteps) run_step<kBwd, kDQ, kF16, kPreDq, 0, 0>(c, step, acc, fa, fb, cb, ca);
  if (step + 1 < c.nsteps) run_step<kBwd, kDQ, kF16, kPreDq, 1, 1>(c, step + 1, acc, fa, fb, ca, cb);
  if (step + 2 < c.nsteps) run_step<kBwd, kDQ, kF16, kPreDq, 2, 0>(c, step + 2, acc, fa, fb, cb, ca);
  if (step + 3 < c.nsteps) run_step<kBwd, kDQ, kF16, kPreDq, 0, 1>(c, step + 3, acc, fa, fb, ca, cb);
  if (step + 4 < c.nsteps) run_step<kBwd, kDQ, kF16, kPreDq, 1, 0>(c, step + 4, acc, fa, fb, cb, ca);

  // ---- epilogue: round to 16 bit, stage the wave's 128 x 64 tile in LDS and
  // write whole 128-byte rows with 16-byte stores (16 stores per lane instead
  // of 128 two-byte ones; all workgroups reach this point together, so the
  // 33.5 MB of a 4096 x 4096 output drain as one tail).  The stages are free
  // once every DMA into them has landed, including the zero-filling ones
  // issued past the last step.  Wave w owns half (w % 2) of stage w / 2;
  // rows are 64 elements, their 8-column chunks XOR-swizzled by (row / 4) % 8
  // so that the two rows one write instruction touches fall in different
  // banks and each row still reads as 8 distinct 16-byte chunks.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (half >= 0) {
    // K-split tile: both halves store their float32 accumulators (device
    // scope, 16 bytes a lane, each store 1 KB contiguous) and count in; the
    // second to arrive adds the other's (float32 addition of two terms does
    // not depend on the order) and writes the tile.  Nothing waits for the
    // other half, so no schedule of the units can stall.  Visibility across
    // the XCDs (each has its own L2): the partials are stored and loaded with
    // the sc1 (device scope) cache-policy bit, which the memory system keeps
    // coherent across XCDs, and the arrival is a device-scope atomic issued
    // after every wave's stores have completed (wait, then barrier); the last
    // arriver loads only after its atomic has returned.  No L2-wide
    // write-back or invalidation is needed.
    // the arrival result goes through the weight stage the epilogue leaves idle
    uint32_t* sh_last = reinterpret_cast<uint32_t*>(sb1);
    const int su = q - g.split_from;
    // (the lane part of each offset in one register, the constant part in
    // the scalar offset)
    const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
        g.part + ((size_t)su * 2 + half) * 65536, 0, 65536 * 4, 0x00020000);
    const uint32_t voff = (uint32_t)c.tid * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint32_t soff = (uint32_t)(((2 * i + j) * 4 + e4) * kThreads * 16);
          const f32x4_t v = f32x4_t{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1],
                                    acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), mine, voff, soff,
                                                 16);
        }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores have completed
    __syncthreads();
    if (c.tid == 0)
      *sh_last = __hip_atomic_fetch_add(g.cnt + su, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == 1u ? 1u : 0u;
    __syncthreads();
    if (*sh_last == 0u) return;   // uniform: the other half writes the tile
    const __amdgpu_buffer_rsrc_t other = __builtin_amdgcn_make_buffer_rsrc(
        g.part + ((size_t)su * 2 + (half ^ 1)) * 65536, 0, 65536 * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint32_t soff = (uint32_t)(((2 * i + j) * 4 + e4) * kThreads * 16);
          const f32x4_t v = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(other, voff, soff, 16));
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][j][4 * e4 + k] += v[k];
        }
  }
  {
    uint16_t* stg = (c.wave >> 1) == 0 ? sa0 : (c.wave >> 1) == 1 ? sa1
                  : (c.wave >> 1) == 2 ? sa2 : sb0;
    stg += (c.wave & 1) * 8192;
    // the lane index re-derived behind an opaque copy, so that no address of
    // this epilogue is computed early and held live across the main loop
    int el = c.lane;
    asm volatile("" : "+v"(el));
    const int el32 = el & 31, elhi = el >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int lr = 32 * i + 8 * (e >> 2) + 4 * elhi + (e & 3);
          const int lc = 32 * j + el32;
          stg[lr * 64 + ((((lc >> 3) ^ ((lr >> 2) & 7)) << 3) | (lc & 7))] =
              (uint16_t)(pack16x2<kF16>(acc[i][j][e], 0.0f) & 0xFFFFu);
        }
    // the wave reads back only what it wrote (LDS operations of one wave
    // complete in order): no barrier
    const int ch = el & 7;
    const int64_t gcol = n0 + col0 + 8 * ch;   // out_len % 16 == 0: a chunk is all in or out
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 8 * it + (el >> 3);
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(stg + row * 64 + ((ch ^ ((row >> 2) & 7)) << 3));
      const int64_t grow = m0 + 128 * wm + row;
      if (grow < g.T && gcol < out_len)
        *reinterpret_cast<u32x4_t*>(g.out + grow * out_len + gcol) = v;
    }
  }
#endif
}

static unsigned num_tiles(int64_t T, int64_t out_len) {
  return (unsigned)(((T + BM - 1) / BM) * ((out_len + BN - 1) / BN));
}

template <bool kBwd, bool kDrop>
static void launch_fmt(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  if (a.wdq && !a.f16)
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, false, false, true>), grid,
                       dim3(kThreads), 0, stream, a);
  else if (a.wdq)
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, false, true, true>), grid, dim3(kThreads),
                       0, stream, a);
  else if (a.dq && !a.f16)
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, true, false, false>), grid,
                       dim3(kThreads), 0, stream, a);
  else if (a.dq)
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, true, true, false>), grid, dim3(kThreads),
                       0, stream, a);
  else if (!a.f16)
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, false, false, false>), grid,
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((qlora_gemm_kernel<kBwd, kDrop, false, true, false>), grid,
                       dim3(kThreads), 0, stream, a);
}

// one unit per tile, two per split tile
static unsigned num_units(const GemmArgs& a, int64_t out_len) {
  const unsigned tiles = num_tiles(a.T, out_len);
  const unsigned from = (unsigned)a.split_from < tiles ? (unsigned)a.split_from : tiles;
  return from + 2 * (tiles - from);
}

hipError_t launch_qlora_fwd_gemm(const GemmArgs& a, hipStream_t stream) {
  launch_fmt<false, false>(a, dim3(num_units(a, a.rows)), stream);
  return hipGetLastError();
}

hipError_t launch_qlora_dx_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.keep)
    launch_fmt<true, true>(a, dim3(num_units(a, a.cols)), stream);
  else
    launch_fmt<true, false>(a, dim3(num_units(a, a.cols)), stream);
  return hipGetLastError();
}

}  // namespace qlora
