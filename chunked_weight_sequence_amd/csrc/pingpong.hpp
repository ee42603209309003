// Eight-wave "ping-pong" matrix-core engine for 256 x 256 output tiles on gfx950.
//
// A 512-thread workgroup holds two groups of four waves; each SIMD runs one wave of each group.
// The K loop advances in 32-wide steps through an NS-stage LDS ring filled by direct
// global -> LDS copies (global_load_lds_dwordx4), and alternates two kinds of phases, separated
// by workgroup barriers:
//   memory phase   the wave issues its share of the copy for a later step and reads its operand
//                  fragments for the current step from LDS into registers;
//   compute phase  the wave issues its 32 products (v_mfma_f32_16x16x32_bf16) from registers.
// Group 1 runs one phase behind group 0, so while one wave of a SIMD computes, the other issues
// its memory work, and the SIMD's matrix core is fed from both. Each wave owns a 128 x 64 block
// of the tile (128 accumulator registers): wave w covers rows 128 ((w >> 1) & 1) and columns
// 64 ((w & 1) + 2 (w >> 2)); acc[i][j][e] is row 16 i + 4 (lane / 16) + e, column
// 16 j + lane % 16 of that block (pp_row, pp_col). (The 16 x 16 x 32 form runs the same
// products about 7% faster than 32 x 32 x 16 with identical results at the same register and
// LDS footprint.)
//
// Phases are numbered from 0 after the first barrier. Group 0 reads step u in phase 2u and
// computes it in 2u + 1; group 1 reads it in 2u + 1 and computes it in 2u + 2. Stage u % NS is
// last read in phase 2u + 1, so the copy for step u + NS - 1, which reuses the stage of step
// u - 1, is issued in the memory phase of step u, after the barrier that closed the last read
// of step u - 1. At the end of every odd phase 2u + 1 each wave waits for its own copies of step u + 1,
// and the barrier that follows makes all of them visible before anyone reads that step. Both
// groups execute the same number of barriers (one extra at the start for group 1, one extra at
// the end for group 0).
//
// Stage layout of a K-contiguous operand: rows r at r * 64 bytes (16 KB per operand); 16-byte
// chunk c of row r at slot c ^ ((r / 2) mod 4). A 16-byte LDS read is served 8 lanes at a time
// across 32 four-byte banks: the 8 lanes of a fragment read (8 consecutive rows, one chunk
// each) then fall on 8 distinct 4-bank groups (rows 2k and 2k + 1 start 16 banks apart and share
// a slot). A probe of SQ_LDS_BANK_CONFLICT measured no conflict cycles for this map, and about
// 3.7 per read for slot c ^ ((r / 4) mod 4), which is conflict-free only if 16 lanes were served
// at once across 64 banks.
#pragma once

#include <stdint.h>

#include "common.hpp"
#include "dma.hpp"

namespace ttt {
namespace {

constexpr int PP_T = 256;             // tile rows (A) and columns (B)
constexpr int PP_BK = 32;             // K per step
constexpr int PP_ROWB = PP_BK * 2;    // bytes per stage row
constexpr int PP_OPB = PP_T * PP_ROWB;  // bytes per operand per stage (16 KB)
constexpr int PP_STAGE = 2 * PP_OPB;  // 32 KB
constexpr int PP_RPI = 16;            // rows per copy instruction (64 lanes x 16 bytes)
constexpr int PP_IPW = PP_T / (PP_RPI * 8);  // copy instructions per wave per operand (2)
constexpr int PP_PER = 2 * PP_IPW;    // copy instructions per wave per step (A and B)

__device__ __forceinline__ constexpr int pp_sw(int r) { return (r >> 1) & 3; }

template <int NS>
struct alignas(16) PPSmem {
  char st[NS][PP_STAGE];
};

using PPAcc = f32x4[8][4];

// Position in the 256 x 256 tile of accumulator element acc[i][j][e] of this lane and wave.
__device__ __forceinline__ int pp_row(int wave, int lane, int i, int e) {
  return 128 * ((wave >> 1) & 1) + 16 * i + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int pp_col(int wave, int lane, int j) {
  return 64 * ((wave & 1) + 2 * (wave >> 2)) + 16 * j + (lane & 15);
}

__device__ __forceinline__ void pp_zero(PPAcc& acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;
}

// One operand of the tile: 256 rows of a matrix whose rows hold the contraction index. Row r of
// the tile is read from base + off[r] (bytes), element k of a row at + (k / 64) * kstride_b +
// (k % 64) * 2, so both plain row-major (kstride_b = 128) and K-blocked layouts work. The
// caller supplies the byte offset of each tile row through `row_off(r)`.
struct PPOp {
  uint32_t voff[PP_IPW];
  const char* base;
  long kstride_b;
  uint32_t lds_off;  // within a stage: 0 for A, PP_OPB for B
  template <class RowOff>
  __device__ __forceinline__ PPOp(const void* base_, long kstride_b_, uint32_t op_off, int wave,
                                  int lane, RowOff&& row_off)
      : base(static_cast<const char*>(base_)), kstride_b(kstride_b_),
        lds_off(op_off + uint32_t(wave) * 1024u) {
    const int lr = lane >> 2;
#pragma unroll
    for (int p = 0; p < PP_IPW; ++p) {
      const int r = (p * 8 + wave) * PP_RPI + lr;
      const int c = (lane & 3) ^ pp_sw(r);
      voff[p] = uint32_t(row_off(r) + c * 16);
    }
  }
  __device__ __forceinline__ void issue(uint32_t stage_lds, int k0) const {
    const char* sb = base + long(k0 >> 6) * kstride_b + (k0 & 63) * 2;
#pragma unroll
    for (int p = 0; p < PP_IPW; ++p)
      dma16(voff[p], sb, stage_lds + lds_off + uint32_t(p) * 8192u);
  }
};

// One operand whose 32-wide K steps are strided blocks: the 16-byte chunk c (K elements
// k0 + 8c .. + 7) of row r of the step starting at k0 sits at
//     base + (k0 / 32) * step_b + r * row_b + c * chunk_b,
// e.g. the K-blocked-by-32 layout [K/32][rows][32] (step_b = rows * 64, row_b = 64, chunk_b = 16),
// in which every step of a 256-row tile is one contiguous 16 KB block (the bf16 state snapshots
// are stored this way). The stage layout in LDS is the same as PPOp's; rows >= nrows re-read row
// nrows - 1.
struct PPOpS {
  uint32_t voff[PP_IPW];
  const char* base;
  long step_b;
  uint32_t lds_off;
  __device__ __forceinline__ PPOpS(const void* base_, long step_b_, int row_b, int chunk_b,
                                   uint32_t op_off, int wave, int lane, int nrows)
      : base(static_cast<const char*>(base_)), step_b(step_b_),
        lds_off(op_off + uint32_t(wave) * 1024u) {
    const int lr = lane >> 2;
#pragma unroll
    for (int p = 0; p < PP_IPW; ++p) {
      const int r = (p * 8 + wave) * PP_RPI + lr;
      const int c = (lane & 3) ^ pp_sw(r);
      voff[p] = uint32_t(min(r, nrows - 1) * row_b + c * chunk_b);
    }
  }
  __device__ __forceinline__ void issue(uint32_t stage_lds, int k0) const {
    const char* sb = base + long(k0 >> 5) * step_b;
#pragma unroll
    for (int p = 0; p < PP_IPW; ++p)
      dma16(voff[p], sb, stage_lds + lds_off + uint32_t(p) * 8192u);
  }
};

__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// wait until at most n of this wave's vector-memory operations are outstanding, n a multiple of
// PP_PER no larger than 3 * PP_PER (rounded down: a smaller count only waits longer)
__device__ __forceinline__ void pp_wait(int n) {
  if (n >= 3 * PP_PER) wait_vm<3 * PP_PER>();
  else if (n >= 2 * PP_PER) wait_vm<2 * PP_PER>();
  else if (n >= PP_PER) wait_vm<PP_PER>();
  else wait_vm<0>();
}

// The 32 products of one step: acc[i][j] += A block i (16 rows) x B block j (16 columns), K = 32.
__device__ __forceinline__ void pp_mma(PPAcc& acc, const uint4 (&fa)[8], const uint4 (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
}

template <int NS, class OpA = PPOp, class OpB = PPOp>
__device__ __forceinline__ void pp_segment(PPAcc& acc, const OpA& oa, const OpB& ob, int nk,
                                           PPSmem<NS>& sm, int wave, int lane) {
  static_assert(NS >= 2 && NS <= 5, "stage count");
  if (nk <= 0) return;
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = (wave & 1) + 2 * grp;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_u32(&sm.st[0][0]));
  // fragment offsets within a stage: lane l reads K chunk l / 16 of row l % 16 of every 16-row
  // block (A rows wm*128 + 16 i + l % 16, B rows wn*64 + 16 j + l % 16)
  const int r16 = lane & 15;
  const uint32_t slot = uint32_t(((lane >> 4) ^ pp_sw(r16)) * 16);  // pp_sw(16 i + r) = pp_sw(r)
  const uint32_t fa_off = uint32_t((wm * 128 + r16) * PP_ROWB) + slot;
  const uint32_t fb_off = uint32_t(PP_OPB + (wn * 64 + r16) * PP_ROWB) + slot;
  // prologue: the first NS steps
  const int pro = nk < NS ? nk : NS;
  for (int s = 0; s < pro; ++s) {
    oa.issue(lds0 + uint32_t(s * PP_STAGE), s * PP_BK);
    ob.issue(lds0 + uint32_t(s * PP_STAGE), s * PP_BK);
  }
  pp_wait(PP_PER * (pro - 1));
  pp_barrier();
  if (grp == 1) pp_barrier();
  for (int u = 0; u < nk; ++u) {
    // memory phase: the fragments of step u, then this wave's share of the copy for step
    // u + NS - 1 into the stage step u - 1 used (the fragment reads go first: they gate the
    // compute phase)
    const char* stage = &sm.st[u % NS][0];
    uint4 fa[8], fb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[i] = *reinterpret_cast<const uint4*>(stage + fa_off + i * 16 * PP_ROWB);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(stage + fb_off + j * 16 * PP_ROWB);
    if (u >= 1 && u + NS - 1 < nk) {
      const uint32_t st = lds0 + uint32_t(((u - 1) % NS) * PP_STAGE);
      oa.issue(st, (u + NS - 1) * PP_BK);
      ob.issue(st, (u + NS - 1) * PP_BK);
    }
    // copies of step u + 1 issued after the ones this wave still has in flight
    const int last = (u + NS - 1 < nk ? u + NS - 1 : nk - 1);
    const int after = (last - (u + 1)) > 0 ? PP_PER * (last - (u + 1)) : 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (grp == 1 && u + 1 < nk) pp_wait(after);
    pp_barrier();
    // compute phase
    pp_mma(acc, fa, fb);
    if (grp == 0 && u + 1 < nk) pp_wait(after);
    pp_barrier();
  }
  if (grp == 0) pp_barrier();
  wait_vm<0>();
}

// Epilogue through LDS for a tile whose columns are tokens and whose output is bf16, token-major
// (each token's RW tile values contiguous in memory). After the K loop the stage ring is free:
// the tile is staged there as 256 token rows of RW * 2 bytes (16-byte chunk c of row n at chunk
// c ^ (n mod RW / 8), so that the 16 lanes of one accumulator write, 16 consecutive tokens at
// the same chunk, fall on distinct banks), then stored as whole rows, 16 bytes a lane. A direct
// store from the accumulator writes 16 tokens x 8 bytes per instruction instead, and on a large
// output costs about twice as long.
template <int RW>
__device__ __forceinline__ void pp_stage_put(char* st, int n, int m, uint2 v) {
  constexpr int CPR = RW / 8;  // chunks per row
  const int c = m >> 3;
  *reinterpret_cast<uint2*>(st + n * (RW * 2) + ((c ^ (n & (CPR - 1))) << 4) + ((m >> 2) & 1) * 8) =
      v;
}
// store(n, c, v): row n, values 8 c .. 8 c + 7 of the row; called for every (n, c) of the tile
template <int RW, class Store>
__device__ __forceinline__ void pp_stage_drain(const char* st, int tid, Store&& store) {
  constexpr int CPR = RW / 8, RPP = 512 / CPR;  // chunks per row, rows per pass
#pragma unroll 4
  for (int pass = 0; pass < PP_T / RPP; ++pass) {
    const int n = pass * RPP + tid / CPR, c = tid % CPR;
    store(n, c, *reinterpret_cast<const uint4*>(st + n * (RW * 2) + ((c ^ (n & (CPR - 1))) << 4)));
  }
}
__device__ __forceinline__ void pp_store_nt(void* p, const uint4& v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

// One operand taken straight from a token-major matrix: element (k, m) at base + k * ldb + 2 m
// (k = token, m < 256 the tile's rows). A stage holds 32 token rows of 512 bytes; 16-byte chunk
// c of token row r sits at slot c ^ pp_swn(r), pp_swn(r) = 2 (r % 4) + 8 ((r / 8) % 2). The
// fragments are formed by transposing LDS reads (ds_read_b64_tr_b16): a 32-lane read pass covers
// token rows {0..3, 8..11} (+ 4, + 16) of one 16-column block, and under this slot map its 64
// eight-byte reads fall on the 64 banks once. Copy instruction p of wave w fills token rows
// 2 (8 p + w) and 2 (8 p + w) + 1. Token rows >= T re-read row T - 1 (the other operand is zero
// there); columns >= ncols re-read the last valid 8-column chunk (their products reach only
// accumulator rows that are never stored).
__device__ __forceinline__ constexpr int pp_swn(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }

struct PPOpN {
  uint32_t voff[PP_IPW];
  int lrow[PP_IPW], lchunk, cmax;
  const char* base;
  long ldb;  // bytes per token row
  int T;
  uint32_t lds_off;
  __device__ __forceinline__ PPOpN(const void* base_, long ldb_, int T_, int ncols, uint32_t op_off,
                                   int wave, int lane)
      : cmax(ncols / 8 - 1), base(static_cast<const char*>(base_)), ldb(ldb_), T(T_),
        lds_off(op_off + uint32_t(wave) * 1024u) {
    lchunk = lane & 31;
#pragma unroll
    for (int p = 0; p < PP_IPW; ++p) {
      const int r = (p * 8 + wave) * 2 + (lane >> 5);
      lrow[p] = r;
      voff[p] = uint32_t(long(r) * ldb + min(lchunk ^ pp_swn(r), cmax) * 16);
    }
  }
  __device__ __forceinline__ void issue(uint32_t stage_lds, int k0) const {
    const char* sb = base + long(k0) * ldb;
    if (k0 + PP_BK <= T) {
#pragma unroll
      for (int p = 0; p < PP_IPW; ++p)
        dma16(voff[p], sb, stage_lds + lds_off + uint32_t(p) * 8192u);
    } else {
#pragma unroll
      for (int p = 0; p < PP_IPW; ++p) {
        const int rr = min(k0 + lrow[p], T - 1) - k0;
        dma16(uint32_t(long(rr) * ldb + min(lchunk ^ pp_swn(lrow[p]), cmax) * 16), sb,
              stage_lds + lds_off + uint32_t(p) * 8192u);
      }
    }
  }
};

// The engine's loop with the A operand token-major (PPOpN, fragments formed by transposing LDS
// reads) and two hooks for a caller that also writes to memory while the stream runs:
//   pre(u)        at the start of step u's memory phase (the accumulator holds steps < u);
//   post(u, ops)  after the wave's copy share in step u's memory phase; it adds the number of
//                 vector-memory instructions it issues to `ops`.
// The copy waits then name the exact count of this wave's operations issued after the awaited
// copies (WL rounds it down to an immediate, which only waits longer).
template <int NS, class WL, class OpB, class Pre, class Post>
__device__ __forceinline__ void pp_stream(PPAcc& acc, const PPOpN& oa, const OpB& ob, int nk,
                                          PPSmem<NS>& sm, int wave, int lane, Pre&& pre,
                                          Post&& post) {
  static_assert(NS >= 2 && NS <= 5, "stage count");
  if (nk <= 0) return;
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = (wave & 1) + 2 * grp;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_u32(&sm.st[0][0]));
  // B fragments as in pp_segment. A fragments: lane l of 16-lane group g = l / 16, j = l % 16
  // reads 8 bytes (columns 4 (j % 4) .. + 3 of block i) of token rows 8 g + j / 4 (h = 0) and
  // + 4 (h = 1); after the transpose it holds column l % 16 of the block, tokens 8 g .. 8 g + 7,
  // the matrix-core operand layout. Block i is logical chunk wm*16 + 2 i + (j % 4) / 2, at slot
  // (that chunk) ^ pp_swn(row): the chunk's bits 1..3 carry i and pp_swn's bits 1..3 the row, so
  // block i sits at (block 0's slot) ^ 2 i.
  const int r16 = lane & 15;
  const uint32_t fb_off =
      uint32_t(PP_OPB + (wn * 64 + r16) * PP_ROWB + ((lane >> 4) ^ pp_sw(r16)) * 16);
  const int g = lane >> 4, j = lane & 15;
  const int row0 = 8 * g + (j >> 2);  // pp_swn(row0 + 4) = pp_swn(row0)
  const uint32_t arow = uint32_t(row0 * 512 + 8 * (j & 1));
  const uint32_t a_slot0 = uint32_t((wm * 16 + ((j & 3) >> 1)) ^ pp_swn(row0));
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  // this wave's operation count, and e[q] = the count right after the copies of step u + 1 + q
  // (constant indices only, so that the array stays in registers)
  int ops = 0, e0 = 0, e[NS - 1];
  const int pro = nk < NS ? nk : NS;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < pro) {
      oa.issue(lds0 + uint32_t(s * PP_STAGE), s * PP_BK);
      ob.issue(lds0 + uint32_t(s * PP_STAGE), s * PP_BK);
      ops += PP_PER;
    }
    if (s == 0) e0 = ops;
    else e[s - 1] = ops;
  }
  WL::wait(ops - e0);
  pp_barrier();
  if (grp == 1) pp_barrier();
  for (int u = 0; u < nk; ++u) {
    pre(u);
    const char* stage = &sm.st[u % NS][0];
    uint4 fa[8], fb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* p = stage + arow + ((a_slot0 ^ uint32_t(2 * i)) * 16);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 512));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      fa[i] = make_uint4(l2.x, l2.y, h2.x, h2.y);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      fb[jj] = *reinterpret_cast<const uint4*>(stage + fb_off + jj * 16 * PP_ROWB);
    if (u >= 1 && u + NS - 1 < nk) {
      const uint32_t st = lds0 + uint32_t(((u - 1) % NS) * PP_STAGE);
      oa.issue(st, (u + NS - 1) * PP_BK);
      ob.issue(st, (u + NS - 1) * PP_BK);
      ops += PP_PER;
      e[NS - 2] = ops;
    }
    post(u, ops);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (grp == 1 && u + 1 < nk) WL::wait(ops - e[0]);
    pp_barrier();
    pp_mma(acc, fa, fb);
    if (grp == 0 && u + 1 < nk) WL::wait(ops - e[0]);
    pp_barrier();
#pragma unroll
    for (int q = 0; q + 1 < NS - 1; ++q) e[q] = e[q + 1];
  }
  if (grp == 0) pp_barrier();
  wait_vm<0>();
}

}  // namespace
}  // namespace ttt
