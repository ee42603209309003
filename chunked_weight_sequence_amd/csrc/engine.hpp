// bf16 matrix-core GEMM engines for gfx950, shared by the scan and the target producer.
//
// Both compute acc += A[rows, k] B[cols, k]^T for one 256 (A rows) x BN (B rows) output tile per
// 256-thread workgroup (2 x 2 waves, v_mfma_f32_32x32x16_bf16), K in steps of 64:
//   * the register-staged engine (Rows, mma_segment): global -> registers -> double-buffered,
//     padded LDS; handles ragged shapes with masked loads;
//   * the direct-to-LDS engine (DOp, DOpN, DFrag, dma_segment): global -> LDS copies into an
//     NS-stage ring of unpadded, swizzled tiles, for shapes whose K steps are whole; DOpN reads
//     an A operand stored K-major (element (k, m) at base + k * ld + m) and forms fragments
//     with transposing LDS reads.
// The accumulator tile is written out through LDS (store_tile_raw) so that global stores are
// coalesced.
#pragma once

#include <stdint.h>

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "dma.hpp"

namespace ttt {
namespace {

constexpr int BM = 256, BK = 64, NTHR = 256;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row (16 bytes of padding)
constexpr int MT = BM / 64;    // 32-row blocks per wave along M (waves are 2x2)

template <int BN>
struct alignas(16) Smem {
  uint16_t a[2][BM * PITCH];
  uint16_t b[2][BN * PITCH];
};

template <int BN>
using Acc = f32x16[MT][BN / 64];

// Zero the bf16 elements of an 8-element chunk starting at k that fall outside [klo, khi).
__device__ __forceinline__ uint4 mask_k(uint4 v, int k, int klo, int khi) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e0 = k + 2 * q, e1 = e0 + 1;
    uint32_t m = 0;
    if (e0 >= klo && e0 < khi) m |= 0x0000FFFFu;
    if (e1 >= klo && e1 < khi) m |= 0xFFFF0000u;
    w[q] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// A [ROWS x BK] tile of a row-major bf16 matrix whose rows hold the contraction index, moved
// global -> registers -> LDS in 16-byte chunks (chunk = 8 consecutive K values of one row).
// FAST: every K step lies inside valid data (the K extent is a multiple of the step, or the
//   matrix is zero-padded past it), so loads are unconditional; rows >= nrows are clamped to the
//   last valid row: their products only reach accumulator rows/columns the epilogue never stores.
// otherwise: rows >= nrows and K positions outside [klo, khi) read as zero (masked copies).
// Element (row, k) sits at base + row * ld + (k / 64) * kstride + k % 64: kstride = 64 for a plain
// row-major matrix, rows * 64 for a K-blocked one ([K/64][rows][64], one K step per block).
template <int ROWS, bool FAST>
struct Rows {
  static constexpr int CPR = BK / 8;
  static constexpr int RPP = NTHR / CPR;
  static constexpr int PASSES = ROWS / RPP;
  const uint16_t* tb;  // this thread's chunk column in row 0
  int off[PASSES];     // element offset of this thread's row in pass p
  long kstride;        // elements between consecutive 64-wide K blocks
  int nrows, klo, khi, kc;
  uint4 r[PASSES];
  int kk[PASSES];      // K offset held in r[p] (masked variant)

  // c4stride (FAST only): 0, or the elements between the two 32-wide halves of a 64-wide K step
  // for an operand K-blocked by 32 ([K/32][rows][32], ld = 32, kstride = 64 * rows)
  __device__ __forceinline__ Rows(const uint16_t* base, long ld, int nrows_, int klo_, int khi_,
                                  int tid, long kstride_ = BK, long c4stride = 0)
      : kstride(kstride_), nrows(nrows_), klo(klo_), khi(khi_), kc(tid % CPR) {
    tb = base + (c4stride ? (kc >> 2) * c4stride + (kc & 3) * 8 : kc * 8);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = tid / CPR + p * RPP;
      off[p] = int((FAST ? min(row, nrows - 1) : row) * ld);
    }
  }
  __device__ __forceinline__ void load_pass(int p, int k0, int tid) {
    if constexpr (FAST) {  // k0 is a multiple of the step
      r[p] = *reinterpret_cast<const uint4*>(tb + off[p] + (k0 / BK) * kstride);
    } else {
      const int k = k0 + kc * 8, row = tid / CPR + p * RPP;
      kk[p] = k;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k + 8 > klo && k < khi && row < nrows)
        v = *reinterpret_cast<const uint4*>(tb - kc * 8 + off[p] + (k / BK) * kstride + k % BK);
      r[p] = v;
    }
  }
  __device__ __forceinline__ void store_pass(int p, uint16_t* s, int tid) const {
    uint4 v = r[p];
    if constexpr (!FAST) {
      const int k = kk[p];
      if (k < klo || k + 8 > khi) v = mask_k(v, k, klo, khi);
    }
    *reinterpret_cast<uint4*>(s + (tid / CPR + p * RPP) * PITCH + kc * 8) = v;
  }
  __device__ __forceinline__ void load(int k0, int tid) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) load_pass(p, k0, tid);
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) store_pass(p, s, tid);
  }
  __device__ __forceinline__ void load_half(int h, int k0, int tid) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      if (p % 2 == h) load_pass(p, k0, tid);
  }
  __device__ __forceinline__ void store_half(int h, uint16_t* s, int tid) const {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      if (p % 2 == h) store_pass(p, s, tid);
  }
};

template <int BN>
__device__ __forceinline__ void zero_acc(Acc<BN>& acc) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// Operand fragments of sub-step ks (16 K values) for this lane: MT blocks of A, NT blocks of B.
template <int BN>
__device__ __forceinline__ void read_frags(uint4 (&fa)[MT], uint4 (&fb)[BN / 64],
                                           const uint16_t* sa, const uint16_t* sb, int ks) {
#pragma unroll
  for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const uint4*>(sa + i * 32 * PITCH + ks * 16);
#pragma unroll
  for (int j = 0; j < BN / 64; ++j)
    fb[j] = *reinterpret_cast<const uint4*>(sb + j * 32 * PITCH + ks * 16);
}

// One sub-step (16 of the 64 K values of a step) with its share of the pipeline work:
//   - the fragments of the next sub-step (for the last sub-step: sub-step 0 of the next step,
//     from the other LDS buffer, which is complete after the barrier of sub-step 2);
//   - in sub-steps 0 and 1, half of the next step's tile into the idle LDS buffer and the global
//     loads that refill those registers for the step after;
//   - this sub-step's MT x NT products, interleaved one-for-one with the memory instructions.
template <int BN, int KS, bool STORE, bool LOAD, bool NEXT, class LA, class LB>
__device__ __forceinline__ void substep(Acc<BN>& acc, uint4 (&fa)[2][MT], uint4 (&fb)[2][BN / 64],
                                        LA& la, LB& lb, const uint16_t* sa, const uint16_t* sb,
                                        const uint16_t* sa_n, const uint16_t* sb_n, uint16_t* na,
                                        uint16_t* nb, int kload, int tid) {
  constexpr int NT = BN / 64;
  constexpr int CUR = KS & 1;
  constexpr bool READ = KS < 3 || NEXT;
  constexpr bool ST = STORE && KS < 2, LD = LOAD && KS < 2;
  constexpr int W = ST ? (LA::PASSES + LB::PASSES) / 2 : 0;
  constexpr int L = LD ? (LA::PASSES + LB::PASSES) / 2 : 0;
  constexpr int M = MT * NT;
  if constexpr (KS < 3) read_frags<BN>(fa[CUR ^ 1], fb[CUR ^ 1], sa, sb, KS + 1);
  else if constexpr (NEXT) read_frags<BN>(fa[0], fb[0], sa_n, sb_n, 0);
  if constexpr (ST) {
    la.store_half(KS, na, tid);
    lb.store_half(KS, nb, tid);
  }
  if constexpr (LD) {
    la.load_half(KS, kload, tid);
    lb.load_half(KS, kload, tid);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = mfma32x32x16(fa[CUR][i], fb[CUR][j], acc[i][j]);
  // instruction order: fragment reads, then MFMA / LDS store / MFMA / global load, ...
  if constexpr (READ) __builtin_amdgcn_sched_group_barrier(0x100, MT + NT, 0);
  constexpr int PAIRS = (W > L ? W : L) < M ? (W > L ? W : L) : M;
#pragma unroll
  for (int i = 0; i < PAIRS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < W) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (i < L) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if constexpr (M > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, M - PAIRS, 0);
  if constexpr (KS == 2 && NEXT) __syncthreads();
}

template <int BN, bool STORE, bool LOAD, bool NEXT, class LA, class LB>
__device__ __forceinline__ void kstep(Acc<BN>& acc, uint4 (&fa)[2][MT], uint4 (&fb)[2][BN / 64],
                                      LA& la, LB& lb, const uint16_t* sa, const uint16_t* sb,
                                      const uint16_t* sa_n, const uint16_t* sb_n, uint16_t* na,
                                      uint16_t* nb, int kload, int tid) {
  substep<BN, 0, STORE, LOAD, NEXT>(acc, fa, fb, la, lb, sa, sb, sa_n, sb_n, na, nb, kload, tid);
  substep<BN, 1, STORE, LOAD, NEXT>(acc, fa, fb, la, lb, sa, sb, sa_n, sb_n, na, nb, kload, tid);
  substep<BN, 2, STORE, LOAD, NEXT>(acc, fa, fb, la, lb, sa, sb, sa_n, sb_n, na, nb, kload, tid);
  substep<BN, 3, STORE, LOAD, NEXT>(acc, fa, fb, la, lb, sa, sb, sa_n, sb_n, na, nb, kload, tid);
}

// acc += A[rows, K] * B[cols, K]^T over the K steps starting at k_begin & ~7 that cover
// [k_begin, k_end). Step it's tile sits in LDS buffer it & 1; one barrier per step. After the
// products of step it, hook(it) runs (the next step's loads are already in flight).
struct NoHook {
  template <class... X>
  __device__ __forceinline__ void operator()(int, X&...) const {}
};

template <int BN, class LA, class LB, class Hook = NoHook>
__device__ __forceinline__ void mma_segment(Acc<BN>& acc, LA& la, LB& lb, int k_begin,
                                            int k_end, Smem<BN>& sm, int tid,
                                            Hook&& hook = Hook()) {
  constexpr int NT = BN / 64;
  const int k0 = k_begin & ~7;
  const int nk = k_end > k0 ? (k_end - k0 + BK - 1) / BK : 0;
  if (nk == 0) return;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int aoff = (wm * (BM / 2) + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const int boff = (wn * (BN / 2) + (lane & 31)) * PITCH + (lane >> 5) * 8;

  la.load(k0, tid);
  lb.load(k0, tid);
  la.store(sm.a[0], tid);
  lb.store(sm.b[0], tid);
  if (nk > 1) {
    la.load(k0 + BK, tid);
    lb.load(k0 + BK, tid);
  }
  __syncthreads();
  uint4 fa[2][MT], fb[2][NT];
  read_frags<BN>(fa[0], fb[0], sm.a[0] + aoff, sm.b[0] + boff, 0);
  int it = 0;
  for (; it + 2 < nk; ++it) {
    const int c = it & 1, n = c ^ 1;
    kstep<BN, true, true, true>(acc, fa, fb, la, lb, sm.a[c] + aoff, sm.b[c] + boff,
                                sm.a[n] + aoff, sm.b[n] + boff, sm.a[n], sm.b[n],
                                k0 + (it + 2) * BK, tid);
    hook(it);
  }
  if (it + 1 < nk) {
    const int c = it & 1, n = c ^ 1;
    kstep<BN, true, false, true>(acc, fa, fb, la, lb, sm.a[c] + aoff, sm.b[c] + boff,
                                 sm.a[n] + aoff, sm.b[n] + boff, sm.a[n], sm.b[n], 0, tid);
    hook(it);
    ++it;
  }
  {
    const int c = it & 1;
    kstep<BN, false, false, false>(acc, fa, fb, la, lb, sm.a[c] + aoff, sm.b[c] + boff, nullptr,
                                   nullptr, nullptr, nullptr, 0, tid);
    hook(it);
  }
  __syncthreads();  // the next segment or the epilogue reuses both buffers
}

// Epilogue: the accumulator tile (BM rows m x BN columns n) is staged through the idle LDS in
// passes of 64 columns, then handed back as f(n, m, v) with v = rows m .. m+3 of column n, where
// the 64 lanes of a wave take consecutive m of one column: every global access the caller makes
// is one contiguous 1 KB (fp32) or 512 B (bf16) run per wave instruction.
constexpr int STAGE_FLOATS = 64 * (BM + 4);  // epilogue staging: 64 columns of BM (+4) floats

// One 64-column pass of the accumulator into LDS: st[n * (BM + 4) + m] for the tile's columns
// pass*64 .. pass*64 + 63 (n relative to the pass) and all BM rows.
template <int BN>
__device__ __forceinline__ void stage_pass(const Acc<BN>& acc, float* st, int wave, int lane,
                                           int pass) {
  constexpr int SP = BM + 4;  // staged floats per column (padded)
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int j = 0; j < BN / 64; ++j) {
    const int n0 = wn * (BN / 2) + j * 32;
    if (n0 / 64 != pass) continue;
    const int n = n0 - pass * 64 + (lane & 31);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * (BM / 2) + i * 32 + 8 * q + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(st + n * SP + m) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]);
      }
  }
}

template <int BN, class Fn>
__device__ __forceinline__ void store_tile_raw(const Acc<BN>& acc, float* st, int tid, Fn&& f) {
  constexpr int SP = BM + 4;
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int pass = 0; pass < BN / 64; ++pass) {
    __syncthreads();  // the LDS is free: main loop or previous pass finished reading it
    stage_pass<BN>(acc, st, wave, lane, pass);
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int n = wave + 4 * r;
      f(pass * 64 + n, lane * 4, *reinterpret_cast<const float4*>(st + n * SP + lane * 4));
    }
  }
}

// As store_tile_raw, for epilogues that combine the tile's two row halves: f(n, m, lo, hi)
// receives rows m .. m+3 (lo) and m + BM/2 .. m + BM/2 + 3 (hi) of column n, m < BM/2; a
// half-wave covers one column.
template <int BN, class Fn>
__device__ __forceinline__ void store_tile_pairs(const Acc<BN>& acc, float* st, int tid, Fn&& f) {
  constexpr int SP = BM + 4;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = (lane & 31) * 4;
#pragma unroll
  for (int pass = 0; pass < BN / 64; ++pass) {
    __syncthreads();
    stage_pass<BN>(acc, st, wave, lane, pass);
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 8; ++r) {
      const int n = wave + 4 * (2 * r + (lane >> 5));
      const float* row = st + n * SP;
      f(pass * 64 + n, m, *reinterpret_cast<const float4*>(row + m),
        *reinterpret_cast<const float4*>(row + BM / 2 + m));
    }
  }
}

template <int BN, class Fn>
__device__ __forceinline__ void store_tile(const Acc<BN>& acc, Smem<BN>& sm, int tid, Fn&& f) {
  static_assert(STAGE_FLOATS * 4 <= sizeof(Smem<BN>), "staging buffer must fit in LDS");
  store_tile_raw<BN>(acc, reinterpret_cast<float*>(&sm), tid, f);
}

// =============================================================================================
// Direct-to-LDS engine (the unmasked shapes). Operand tiles go from global memory straight into
// LDS (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l), so no registers are spent
// on staging and the LDS holds NS K steps at once: the copy for step it + NS is issued as soon as
// step it's stage is released, NS - 1 steps before it is needed, which hides HBM latency behind
// that many steps of matrix-core work. Rows are unpadded (BKD bf16 each); 16-byte chunk c of
// row r sits at slot c ^ sw(r), sw(r) = (r / RPB) % CPR with RPB the rows per 256-byte line of
// the 64 LDS banks: the 16 lanes of one pass of a 16-byte fragment read (16 consecutive rows,
// one chunk each) then touch 16 distinct 4-bank groups. The vector-memory counter covers copies and stores alike and completes in
// order, so every wait names the exact number of this wave's operations issued after the copy
// it waits for (OpLog); any other memory instruction can only make a wait stricter.
template <int BKD_>
struct DC {
  static constexpr int BKD = BKD_;
  static constexpr int CPR = BKD / 8;   // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR;  // rows per 256-byte line (64 banks of 4 bytes)
  static constexpr int RPI = 64 / CPR;  // rows filled by one wave copy instruction (1 KB)
  static constexpr int KS = BKD / 16;   // matrix-core sub-steps per K step
  static constexpr int ROWB = BKD * 2;  // bytes per row
  static_assert(BKD == 32 || BKD == 64, "K step of the direct engine");
  __device__ static constexpr int sw(int r) { return (r / RPB) % CPR; }
};

template <int BN, int BKD, int NS>
struct alignas(16) SmemD {
  static constexpr int STAGE = (BM + BN) * BKD * 2;  // bytes: A rows, then B rows
  char st[NS][STAGE];
};

// The counts a plain segment waits with: k whole copy batches (PER operations each) after the
// awaited one, k = NS - 1 .. 0.
template <int PER, class Seq>
struct BatchWaits;
template <int PER, int... I>
struct BatchWaits<PER, std::integer_sequence<int, I...>> {
  using type = WaitList<(int(sizeof...(I)) - 1 - I) * PER...>;
};

// This wave's LDS reads are complete, then every wave meets: a stage read before this point may
// be overwritten after it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Count of this wave's vector-memory operations, and the count right after each of the copies
// for steps it+1 .. it+NS-1 (end[0] is the next step's).
template <int NS>
struct OpLog {
  int ops = 0;
  int end[NS - 1];
  __device__ __forceinline__ void shift(bool issued) {
#pragma unroll
    for (int q = 0; q + 1 < NS - 1; ++q) end[q] = end[q + 1];
    end[NS - 2] = issued ? ops : end[NS - 2];
  }
  __device__ __forceinline__ int after_next() const { return ops - end[0]; }
};

// One operand of a tile: ROWS rows holding the contraction index, element (row, k) at
// base + row * ld + (k / 64) * kstride + k % 64. Wave w's copy instruction p fills rows
// [(4p + w) RPI, +RPI) of the operand's block in a stage; rows >= nrows re-read the last valid
// row (their products reach only accumulator entries that are never stored).
template <int ROWS, int BKD>
struct DOp {
  using C = DC<BKD>;
  static constexpr int IPW = ROWS / (C::RPI * 4);
  static_assert(IPW >= 1 && ROWS % (C::RPI * 4) == 0, "rows per wave copy");
  uint32_t voff[IPW];
  const char* base;
  long kstride_b;
  uint32_t lds_off;
  __device__ __forceinline__ DOp(const uint16_t* base_, long ld, int nrows, long kstride,
                                 uint32_t lds_off_, int wave, int lane)
      : base(reinterpret_cast<const char*>(base_)), kstride_b(kstride * 2),
        lds_off(lds_off_ + uint32_t(wave) * 1024u) {
    const int lr = lane / C::CPR;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int r = (p * 4 + wave) * C::RPI + lr;  // row of the stage this lane fills
      const int c = (lane % C::CPR) ^ C::sw(r);
      const int row = min(r, nrows - 1);
      voff[p] = uint32_t(long(row) * ld * 2 + c * 16);
    }
  }
  template <int NSX>
  __device__ __forceinline__ void issue(uint32_t stage_lds, int k0, OpLog<NSX>& log) const {
    const char* sb = base + long(k0 / 64) * kstride_b + (k0 % 64) * 2;
#pragma unroll
    for (int p = 0; p < IPW; ++p) dma16(voff[p], sb, stage_lds + lds_off + uint32_t(p) * 4096u);
    log.ops += IPW;
  }
};

// The A operand taken straight from a token-major matrix (element (k, m) at base + k * ld + m,
// k = token, m < BM): each stage holds BKD token rows of BM bf16 (512 bytes), 16-byte chunk c
// of token row r at chunk c ^ 4 (r % 4): a transposing read pass (32 lanes: 4 token rows x 2
// column groups x 32 bytes) then covers one 256-byte line of the 64 banks once. Matrix-core fragments, which want 8 consecutive
// tokens of one m per lane, are then formed by transposing LDS reads (ds_read_b64_tr_b16).
// Token rows >= T re-read row T - 1 (the other operand is zero there); columns >= ncols re-read
// the last valid 8-column chunk (their products reach only accumulator rows never stored).
template <int BKD>
struct DOpN {
  static constexpr int RB = BM * 2;           // bytes per token row
  static constexpr int RPI = 1024 / RB;       // token rows per wave copy instruction
  static constexpr int LPR = 64 / RPI;        // lanes per token row
  static constexpr int IPW = BKD / (RPI * 4);
  static_assert(IPW >= 1 && BKD % (RPI * 4) == 0, "token rows per wave copy");
  uint32_t voff[IPW];
  int lrow[IPW], lchunk, cmax;
  const char* base;
  long ldb;  // bytes per token row of the matrix
  int T;
  uint32_t lds_off;
  __device__ __forceinline__ DOpN(const uint16_t* base_, long ld, int T_, int ncols,
                                  uint32_t lds_off_, int wave, int lane)
      : cmax(ncols / 8 - 1), base(reinterpret_cast<const char*>(base_)), ldb(ld * 2), T(T_),
        lds_off(lds_off_ + uint32_t(wave) * 1024u) {
    lchunk = lane % LPR;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int r = (p * 4 + wave) * RPI + lane / LPR;
      lrow[p] = r;
      voff[p] = uint32_t(long(r) * ldb + min(lchunk ^ (4 * (r % 4)), cmax) * 16);
    }
  }
  template <int NSX>
  __device__ __forceinline__ void issue(uint32_t stage_lds, int k0, OpLog<NSX>& log) const {
    const char* sb = base + long(k0) * ldb;
    if (k0 + BKD <= T) {
#pragma unroll
      for (int p = 0; p < IPW; ++p)
        dma16(voff[p], sb, stage_lds + lds_off + uint32_t(p) * 4096u);
    } else {
#pragma unroll
      for (int p = 0; p < IPW; ++p) {
        const int rr = min(k0 + lrow[p], T - 1) - k0;
        const uint32_t v =
            uint32_t(long(rr) * ldb + min(lchunk ^ (4 * (lrow[p] % 4)), cmax) * 16);
        dma16(v, sb, stage_lds + lds_off + uint32_t(p) * 4096u);
      }
    }
    log.ops += IPW;
  }
};

// Byte offsets within a stage of this lane's fragment chunks, per sub-step (block 0). With a
// natural (token-major) A operand, a lane of 16-lane group g = lane / 16, j = lane % 16 reads
// token rows 16 ks + 8 (g / 2) + 4 h + j / 4 (h = 0, 1: two transposing reads of 4 tokens) at
// columns wm*128 + 32 i + 16 (g % 2) + 4 (j % 4): afterwards lane l holds column l % 32, tokens
// 8 (l / 32) .. +7 of the sub-step, the matrix-core operand layout.
template <int BN, int BKD, bool AN = false>
struct DFrag {
  using C = DC<BKD>;
  uint32_t a[AN ? MT : C::KS], b[C::KS];
  uint32_t arow = 0;
  __device__ __forceinline__ DFrag(int wm, int wn, int lane) {
    const int m = lane & 31, kh = lane >> 5, sw = C::sw(m);  // sw(m + 32 i) = sw(m)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int slot = ((2 * ks + kh) ^ sw) * 16;
      if constexpr (!AN) a[ks] = uint32_t((wm * (BM / 2) + m) * C::ROWB + slot);
      b[ks] = uint32_t(BKD * BM * 2 + (wn * (BN / 2) + m) * C::ROWB + slot);
    }
    if constexpr (AN) {
      const int g = lane >> 4, j = lane & 15;
      arow = uint32_t((8 * (g >> 1) + (j >> 2)) * BM * 2 + 8 * (j & 1));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int c = wm * 16 + 4 * i + 2 * (g & 1) + ((j & 3) >> 1);
        a[i] = uint32_t((c ^ (4 * (j >> 2))) * 16);  // token row % 4 = j / 4
      }
    }
  }
};

template <int BN, int BKD, bool AN>
__device__ __forceinline__ void dread(uint4 (&fa)[MT], uint4 (&fb)[BN / 64], const char* stage,
                                      const DFrag<BN, BKD, AN>& fr, int ks) {
  constexpr int RB = DC<BKD>::ROWB;
  if constexpr (AN) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const char* p = stage + fr.arow + fr.a[i] + ks * 16 * BM * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * BM * 2));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      fa[i] = make_uint4(l2.x, l2.y, h2.x, h2.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i)
      fa[i] = *reinterpret_cast<const uint4*>(stage + fr.a[ks] + i * 32 * RB);
  }
#pragma unroll
  for (int j = 0; j < BN / 64; ++j)
    fb[j] = *reinterpret_cast<const uint4*>(stage + fr.b[ks] + j * 32 * RB);
}

template <int BN>
__device__ __forceinline__ void dmma(Acc<BN>& acc, const uint4 (&fa)[MT],
                                     const uint4 (&fb)[BN / 64]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
}

// acc += A[rows, k] B[cols, k]^T over K steps k0 = 0, BKD, ... < nk * BKD, through the direct
// engine. pre(it) runs before the first product of step it (the accumulator then holds steps
// < it exactly); post(it, log) runs once per step after step it + NS's copies are issued; a post
// hook that issues vector-memory operations adds them to log.ops.
struct NoPre {
  __device__ __forceinline__ void operator()(int) const {}
};
struct NoPost {
  template <class L>
  __device__ __forceinline__ void operator()(int, L&) const {}
};

template <int BN, int BKD, int NS, class WLX = void, class OA, class OB, class FR,
          class Pre = NoPre, class Post = NoPost>
__device__ __forceinline__ void dma_segment(Acc<BN>& acc, const OA& oa, const OB& ob, int nk,
                                            SmemD<BN, BKD, NS>& sm, const FR& fr,
                                            Pre&& pre = Pre(), Post&& hook = Post()) {
  using C = DC<BKD>;
  using WL = std::conditional_t<std::is_void_v<WLX>,
                                typename BatchWaits<OA::IPW + OB::IPW,
                                                    std::make_integer_sequence<int, NS>>::type,
                                WLX>;
  constexpr int ST = SmemD<BN, BKD, NS>::STAGE;
  if (nk <= 0) return;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_u32(&sm.st[0][0]));
  OpLog<NS> log;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < nk) {
      oa.issue(lds0 + uint32_t(s * ST), s * BKD, log);
      ob.issue(lds0 + uint32_t(s * ST), s * BKD, log);
    }
    if (s >= 1) log.end[s - 1] = log.ops;
  }
  WL::wait(log.ops - (OA::IPW + OB::IPW));  // step 0's copies have landed

  lds_barrier();
  uint4 fa[2][MT], fb[2][BN / 64];
  dread<BN, BKD>(fa[0], fb[0], &sm.st[0][0], fr, 0);
  for (int it = 0; it < nk; ++it) {
    const char* cur = &sm.st[it % NS][0];
    const char* nxt = &sm.st[(it + 1) % NS][0];
    const bool more = it + 1 < nk;
    pre(it);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int cb = ks & 1;
      if (ks + 1 < C::KS) {
        // this sub-step's products, with the next sub-step's fragments read ahead of them
        dread<BN, BKD>(fa[cb ^ 1], fb[cb ^ 1], cur, fr, ks + 1);
        dmma<BN>(acc, fa[cb], fb[cb]);
        __builtin_amdgcn_sched_group_barrier(0x100, MT + BN / 64, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT * (BN / 64), 0);
        if (ks == C::KS - 2 && more) {
          // step it + 1's copies have landed (this wave's, then everyone's); step it's stage is
          // free once every wave has finished reading it
          WL::wait(log.after_next());
          lds_barrier();
        }
      } else {
        if (more) {
          dread<BN, BKD>(fa[cb ^ 1], fb[cb ^ 1], nxt, fr, 0);
          if (it + NS < nk) {
            oa.issue(lds0 + uint32_t((it % NS) * ST), (it + NS) * BKD, log);
            ob.issue(lds0 + uint32_t((it % NS) * ST), (it + NS) * BKD, log);
          }
          log.shift(it + NS < nk);
          hook(it, log);
        }
        dmma<BN>(acc, fa[cb], fb[cb]);
      }
    }
    if (!more) hook(it, log);
  }
  wait_vm<0>();
  lds_barrier();  // the caller may reuse the stages
}

__device__ __forceinline__ uint2 pack4(float4 v) {
  return make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
}

// Blocks are dealt to the 8 XCDs round-robin (block id % 8). Give each XCD a contiguous range
// of logical tiles so tiles sharing operand panels meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / 8, full = per * 8;
  if (bid >= full) return bid;
  return (bid % 8) * per + bid / 8;
}

}  // namespace
}  // namespace ttt
