// In-Place TTT chunk scan on CDNA4 matrix cores (bf16 operands, fp32 accumulation, fp32 state).
//
// What is computed ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv 2604.06169):
// for each chunk i, O_i = Z_i W_i^T with the state from before chunk i's update (section 3), and
// W_{i+1} = W_i + eta * V_i^T Z_i (section 2). The deltas are additive (section 6), so the state
// a chunk sees is W_0 plus an exclusive prefix sum of earlier deltas.
//
// How it is scheduled on one GPU. Chunks are taken in groups of k (G = k*C tokens, about 1024).
// Inside a group the state is not re-materialised per chunk; instead, for a token t in chunk r of
// group g,
//     O_t = z_t W_g^T + eta * sum_{s in group, chunk(s) < chunk(t)} (z_t . z_s) v_s,
// the same exclusive prefix written with the intra-group part as a masked Z Z^T product. This
// trades a small amount of extra matrix work ((k-1) * C * (d_ff + d_model) flop per token) for
// a k-fold cut in state traffic (the fp32 state is about 100 MB at d_model 2560 x d_ff 9728).
// Phases, in launch order:
//   0 stage      token-major copies Zt [d_ff, Tp], Vt [d_model, Tp] so that every product below
//                reads operands with the contraction index contiguous;
//   1 corr       S_g = eta * mask(Z_g Z_g^T) blocks for all groups at once (bf16);
//   2 update     W_{g+1} = W_g + eta * Vt_g Zt_g^T, one launch per group (the only sequential
//                chain); each state is kept as a snapshot;
//   3 apply      O_g = Z_g W_g^T + S_g V_g for all groups in one launch;
//   2 (last)     the final group's update into W_final, issued after apply so that W_final
//                may alias W0.
// Every product is one kernel shape: a 256x256 output tile per 256-thread workgroup (2x2 waves,
// each 128x128 as 4x4 blocks of v_mfma_f32_32x32x16_bf16), K steps of 64 staged through
// double-buffered LDS from registers, and tiles mapped so that each XCD works on a contiguous
// range of logical tiles that share operand panels in its L2.
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row (16 bytes of padding)
constexpr int MT = BM / 64;    // 32x32 blocks per wave along M (waves are 2x2)
constexpr int NT = BN / 64;    // 32x32 blocks per wave along N

struct alignas(16) Smem {
  uint16_t a[2][BM * PITCH];
  uint16_t b[2][BN * PITCH];
};

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

// A [ROWS x BK] tile of a row-major bf16 matrix whose rows hold the contraction index.
// Rows >= nrows and K positions outside [klo, khi) read as zero. Reads are 16-byte chunks at
// K offsets that are multiples of 8, so ld and the base must keep rows 16-byte aligned.
template <int ROWS>
struct RowsBF16 {
  static constexpr int CPR = BK / 8;
  static constexpr int RPP = NTHR / CPR;
  static constexpr int PASSES = ROWS / RPP;
  const uint16_t* base;
  long ld;
  int nrows, klo, khi;
  uint4 r[PASSES];

  __device__ __forceinline__ void load(int k0, int tid) {
    const int kc = tid % CPR, rr = tid / CPR;
    const int k = k0 + kc * 8;
    const bool kin = (k + 8 > klo) && (k < khi);
    const bool kpart = (k < klo) || (k + 8 > khi);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rr + p * RPP;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kin && row < nrows) {
        v = *reinterpret_cast<const uint4*>(base + long(row) * ld + k);
        if (kpart) v = mask_k(v, k, klo, khi);
      }
      r[p] = v;
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
    const int kc = tid % CPR, rr = tid / CPR;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      *reinterpret_cast<uint4*>(s + (rr + p * RPP) * PITCH + kc * 8) = r[p];
  }
};

// The same tile read from an fp32 matrix and rounded to bf16 (nearest even) on the way to LDS.
template <int ROWS>
struct RowsF32 {
  static constexpr int CPR = BK / 8;
  static constexpr int RPP = NTHR / CPR;
  static constexpr int PASSES = ROWS / RPP;
  const float* base;
  long ld;
  int nrows, klo, khi;
  float4 lo[PASSES], hi[PASSES];
  bool part[PASSES];
  int kk;

  __device__ __forceinline__ void load(int k0, int tid) {
    const int kc = tid % CPR, rr = tid / CPR;
    const int k = k0 + kc * 8;
    kk = k;
    const bool kin = (k + 8 > klo) && (k < khi);
    const bool kpart = (k < klo) || (k + 8 > khi);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rr + p * RPP;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (kin && row < nrows) {
        const float4* src = reinterpret_cast<const float4*>(base + long(row) * ld + k);
        a = src[0];
        b = src[1];
      }
      lo[p] = a;
      hi[p] = b;
      part[p] = kin && kpart;
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
    const int kc = tid % CPR, rr = tid / CPR;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      uint4 v = make_uint4(pack2bf(lo[p].x, lo[p].y), pack2bf(lo[p].z, lo[p].w),
                           pack2bf(hi[p].x, hi[p].y), pack2bf(hi[p].z, hi[p].w));
      if (part[p]) v = mask_k(v, kk, klo, khi);
      *reinterpret_cast<uint4*>(s + (rr + p * RPP) * PITCH + kc * 8) = v;
    }
  }
};

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[MT][NT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// One K step (BK) of the 2x2-wave tile from LDS.
__device__ __forceinline__ void mma_step(f32x16 (&acc)[MT][NT], const uint16_t* sa,
                                         const uint16_t* sb, int wm, int wn, int lane) {
  const int r = lane & 31, kq = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < BK; ks += 16) {
    uint4 a[MT], b[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      a[i] = *reinterpret_cast<const uint4*>(sa + (wm * (BM / 2) + i * 32 + r) * PITCH + ks + kq);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      b[j] = *reinterpret_cast<const uint4*>(sb + (wn * (BN / 2) + j * 32 + r) * PITCH + ks + kq);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  }
}

// acc += A[rows, K] * B[cols, K]^T over K positions [k_begin, k_end): register prefetch of the
// next K step while the current one is multiplied out of LDS; one barrier per step.
template <class LA, class LB>
__device__ __forceinline__ void mma_segment(f32x16 (&acc)[MT][NT], LA& la, LB& lb, int k_begin,
                                            int k_end, Smem& sm, int tid) {
  const int k0 = k_begin & ~7;
  const int nk = k_end > k0 ? (k_end - k0 + BK - 1) / BK : 0;
  if (nk == 0) return;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  la.load(k0, tid);
  lb.load(k0, tid);
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    la.store(sm.a[buf], tid);
    lb.store(sm.b[buf], tid);
    __syncthreads();
    if (it + 1 < nk) {
      la.load(k0 + (it + 1) * BK, tid);
      lb.load(k0 + (it + 1) * BK, tid);
    }
    mma_step(acc, sm.a[buf], sm.b[buf], wm, wn, lane);
  }
  __syncthreads();  // the next segment (or tile) reuses both buffers
}

// Calls f(row, col, value) for every accumulator element of this lane (tile coordinates).
template <class Fn>
__device__ __forceinline__ void for_each_acc(const f32x16 (&acc)[MT][NT], int tid, Fn&& f) {
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = wn * (BN / 2) + j * 32 + (lane & 31);
        f(row, col, acc[i][j][e]);
      }
}

// Blocks are dealt to the 8 XCDs round-robin (block id % 8). Give each XCD a contiguous range
// of logical tiles so tiles sharing operand panels meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / 8, full = per * 8;
  if (bid >= full) return bid;
  return (bid % 8) * per + bid / 8;
}

// ---------------------------------------------------------------------------------------------
// Phase 0: out[b][c][t] = in[b][t][c] for t < T, zero for T <= t < Tp (N % 16 == 0).
__global__ __launch_bounds__(256) void k_stage(const uint16_t* __restrict__ in,
                                               uint16_t* __restrict__ out, int T, int Tp, int N,
                                               long in_b, long out_b) {
  __shared__ uint16_t tile[64][64 + 2];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z, tid = threadIdx.x;
  in += b * in_b;
  out += b * out_b;
  {
    const int r = tid >> 2, cq = (tid & 3) * 16, t = t0 + r;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (t < T && c0 + cq < N) {
      const uint4* p = reinterpret_cast<const uint4*>(in + long(t) * N + c0 + cq);
      v0 = p[0];
      v1 = p[1];
    }
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      tile[r][cq + 2 * q] = uint16_t(w[q] & 0xFFFFu);
      tile[r][cq + 2 * q + 1] = uint16_t(w[q] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = tid >> 2, tq = (tid & 3) * 16;
    if (c0 + c < N) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = uint32_t(tile[tq + 2 * q][c]) | (uint32_t(tile[tq + 2 * q + 1][c]) << 16);
      uint4* p = reinterpret_cast<uint4*>(out + long(c0 + c) * Tp + t0 + tq);
      p[0] = make_uint4(w[0], w[1], w[2], w[3]);
      p[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Phase 1: S_g[t - g0][s - sbase] = eta * (z_t . z_s) if g0 <= s and chunk(s) < chunk(t), else 0,
// for t in group g = [g0, g1) and s up to the chunk start of the tile's last row.
__global__ __launch_bounds__(NTHR, 1) void k_corr(const uint16_t* __restrict__ Z, long z_b,
                                                  uint16_t* __restrict__ S, long s_b, long s_g,
                                                  int Gp, int T, int F, int C, int G, int ntt,
                                                  int nst, float eta) {
  __shared__ Smem sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = ntt * nst;
  const int g = tile / per_g, rem = tile % per_g, tt = rem / nst, st = rem % nst;
  const int g0 = g * G, g1 = min(g0 + G, T);
  const int t_start = g0 + tt * BM;
  if (t_start >= g1) return;
  const int t_end = min(t_start + BM, g1);
  const int cs_last = ((t_end - 1) / C) * C;
  const int sbase = g0 & ~7;
  const int s_start = sbase + st * BN;
  if (!(s_start < cs_last && s_start + BN > g0)) return;
  const uint16_t* Zb = Z + b * z_b;
  RowsBF16<BM> la{Zb + long(t_start) * F, F, t_end - t_start, 0, F, {}};
  RowsBF16<BN> lb{Zb + long(s_start) * F, F, min(BN, T - s_start), 0, F, {}};
  f32x16 acc[MT][NT];
  zero_acc(acc);
  mma_segment(acc, la, lb, 0, F, sm, tid);
  uint16_t* Sg = S + b * s_b + g * s_g;
  for_each_acc(acc, tid, [&](int row, int col, float v) {
    const int t = t_start + row, s = s_start + col;
    if (t < t_end && s - sbase < Gp) {
      const bool keep = s >= g0 && (s / C) < (t / C);
      Sg[long(t - g0) * Gp + (s - sbase)] = f2bf(keep ? eta * v : 0.f);
    }
  });
}

// ---------------------------------------------------------------------------------------------
// Phase 2: Wout = Win + eta * Vt[:, t0:t1] Zt[:, t0:t1]^T  ([d_model, d_ff], fp32).
__global__ __launch_bounds__(NTHR, 1) void k_update(const uint16_t* __restrict__ Vt,
                                                    const uint16_t* __restrict__ Zt, long ldt,
                                                    long vt_b, long zt_b, const float* Win,
                                                    long win_b, float* Wout, long wout_b, int D,
                                                    int F, int t0, int t1, float eta,
                                                    int tiles_m) {
  __shared__ Smem sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  RowsBF16<BM> la{Vt + b * vt_b + long(m0) * ldt, ldt, min(BM, D - m0), t0, t1, {}};
  RowsBF16<BN> lb{Zt + b * zt_b + long(n0) * ldt, ldt, min(BN, F - n0), t0, t1, {}};
  f32x16 acc[MT][NT];
  zero_acc(acc);
  mma_segment(acc, la, lb, t0, t1, sm, tid);
  const float* wi = Win + b * win_b;
  float* wo = Wout + b * wout_b;
  for_each_acc(acc, tid, [&](int row, int col, float v) {
    const int d = m0 + row, f = n0 + col;
    if (d < D && f < F) {
      const size_t i = size_t(d) * F + f;
      wo[i] = wi[i] + eta * v;
    }
  });
}

// ---------------------------------------------------------------------------------------------
// Phase 3: O[t][d] = sum_f Z[t][f] W_g[d][f] + sum_s S_g[t][s] V[s][d] for every group g.
template <typename TOut>
__global__ __launch_bounds__(NTHR, 1) void k_apply(
    const uint16_t* __restrict__ Z, long z_b, const float* W0, long w0_b, const float* Wsnap,
    long snap_g, long snap_b, const uint16_t* S, long s_b, long s_g, int Gp,
    const uint16_t* __restrict__ Vt, long ldt, long vt_b, TOut* __restrict__ O, long o_b, int T,
    int F, int D, int C, int G, int ntt, int ntd) {
  __shared__ Smem sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = ntt * ntd;
  const int g = tile / per_g, rem = tile % per_g, tt = rem / ntd, td = rem % ntd;
  const int g0 = g * G, g1 = min(g0 + G, T);
  const int t_start = g0 + tt * BM;
  if (t_start >= g1) return;
  const int t_end = min(t_start + BM, g1);
  const int d0 = td * BN;
  const float* Wg = g == 0 ? W0 + b * w0_b : Wsnap + b * snap_b + long(g - 1) * snap_g;
  f32x16 acc[MT][NT];
  zero_acc(acc);
  {
    RowsBF16<BM> la{Z + b * z_b + long(t_start) * F, F, t_end - t_start, 0, F, {}};
    RowsF32<BN> lb{Wg + long(d0) * F, F, min(BN, D - d0), 0, F, {}, {}, {}, 0};
    mma_segment(acc, la, lb, 0, F, sm, tid);
  }
  const int cs_last = ((t_end - 1) / C) * C;
  if (S != nullptr && cs_last > g0) {
    const int sbase = g0 & ~7;
    const uint16_t* Sg = S + b * s_b + g * s_g;
    RowsBF16<BM> la{Sg + long(t_start - g0) * Gp, Gp, t_end - t_start, g0 - sbase,
                    cs_last - sbase, {}};
    RowsBF16<BN> lb{Vt + b * vt_b + long(d0) * ldt + sbase, ldt, min(BN, D - d0), g0 - sbase,
                    cs_last - sbase, {}};
    mma_segment(acc, la, lb, g0 - sbase, cs_last - sbase, sm, tid);
  }
  TOut* ob = O + b * o_b;
  for_each_acc(acc, tid, [&](int row, int col, float v) {
    const int t = t_start + row, d = d0 + col;
    if (t < t_end && d < D) st_elem(ob, size_t(t) * D + d, v);
  });
}

// ---------------------------------------------------------------------------------------------
struct Plan {
  int k, G, n_groups, Tp, Gp, ntt, nst, ntd, tiles_m, tiles_n;
  size_t off_zt, off_vt, off_snap, off_s, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Plan make_plan(int B, int T, int F, int D, int C) {
  Plan p{};
  int target = 1024;
  if (const char* s = getenv("TTT_SCAN_GROUP_TOKENS")) {
    const int v = atoi(s);
    if (v > 0) target = v;
  }
  p.k = (target + C / 2) / C;
  if (p.k < 1) p.k = 1;
  const int n_chunks = (T + C - 1) / C;
  if (p.k > n_chunks) p.k = n_chunks;
  p.G = p.k * C;
  p.n_groups = (T + p.G - 1) / p.G;
  p.Tp = (T + 63) / 64 * 64;
  const int pad = (p.G % 8) ? 7 : 0;
  p.nst = (p.G + pad + BN - 1) / BN;
  p.Gp = p.nst * BN;
  p.ntt = (p.G + BM - 1) / BM;
  p.ntd = (D + BN - 1) / BN;
  p.tiles_m = (D + BM - 1) / BM;
  p.tiles_n = (F + BN - 1) / BN;
  size_t off = 0;
  p.off_zt = off;
  off = align256(off + size_t(B) * F * p.Tp * 2);
  p.off_vt = off;
  off = align256(off + size_t(B) * D * p.Tp * 2);
  p.off_snap = off;
  off = align256(off + size_t(B) * (p.n_groups - 1) * D * F * 4);
  p.off_s = off;
  if (p.k > 1) off = align256(off + size_t(B) * p.n_groups * p.G * p.Gp * 2);
  p.total = off;
  return p;
}

template <typename TOut>
hipError_t run(const ScanArgs& a, PhaseClock* clk) {
  const Plan p = make_plan(a.B, a.T, a.F, a.D, a.C);
  char* ws = static_cast<char*>(a.ws);
  uint16_t* Zt = reinterpret_cast<uint16_t*>(ws + p.off_zt);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(ws + p.off_vt);
  float* snap = reinterpret_cast<float*>(ws + p.off_snap);
  uint16_t* S = p.k > 1 ? reinterpret_cast<uint16_t*>(ws + p.off_s) : nullptr;
  const uint16_t* Z = static_cast<const uint16_t*>(a.Z);
  const uint16_t* V = static_cast<const uint16_t*>(a.V);
  const long DF = long(a.D) * a.F;
  const long z_b = long(a.T) * a.F, v_b = long(a.T) * a.D;
  const long zt_b = long(a.F) * p.Tp, vt_b = long(a.D) * p.Tp;
  const long w0_b = a.w0_shared ? 0 : DF;
  const long snap_b = long(p.n_groups - 1) * DF;
  const long s_g = long(p.G) * p.Gp, s_b = long(p.n_groups) * s_g;

  // 0: token-major operand copies
  if (clk) clk->open(0);
  hipLaunchKernelGGL(k_stage, dim3(p.Tp / 64, (a.F + 63) / 64, a.B), dim3(256), 0, a.stream, Z,
                     Zt, a.T, p.Tp, a.F, z_b, zt_b);
  hipLaunchKernelGGL(k_stage, dim3(p.Tp / 64, (a.D + 63) / 64, a.B), dim3(256), 0, a.stream, V,
                     Vt, a.T, p.Tp, a.D, v_b, vt_b);
  if (clk) clk->close(2);

  // 1: intra-group correction blocks
  if (p.k > 1) {
    if (clk) clk->open(1);
    hipLaunchKernelGGL(k_corr, dim3(p.n_groups * p.ntt * p.nst, a.B), dim3(NTHR), 0, a.stream,
                       Z, z_b, S, s_b, s_g, p.Gp, a.T, a.F, a.C, p.G, p.ntt, p.nst, a.eta);
    if (clk) clk->close(1);
  }

  auto update = [&](int g, float* out, long out_b) {
    const float* win = g == 0 ? a.W0 : snap + long(g - 1) * DF;
    const long win_b = g == 0 ? w0_b : snap_b;
    const int t0 = g * p.G, t1 = t0 + p.G < a.T ? t0 + p.G : a.T;
    hipLaunchKernelGGL(k_update, dim3(p.tiles_m * p.tiles_n, a.B), dim3(NTHR), 0, a.stream, Vt,
                       Zt, long(p.Tp), vt_b, zt_b, win, win_b, out, out_b, a.D, a.F, t0, t1,
                       a.eta, p.tiles_m);
  };

  // 2: state chain up to the last group's starting state
  if (p.n_groups > 1) {
    if (clk) clk->open(2);
    for (int g = 0; g + 1 < p.n_groups; ++g) update(g, snap + long(g) * DF, snap_b);
    if (clk) clk->close(p.n_groups - 1);
  }

  // 3: apply for every group
  if (clk) clk->open(3);
  hipLaunchKernelGGL((k_apply<TOut>), dim3(p.n_groups * p.ntt * p.ntd, a.B), dim3(NTHR), 0,
                     a.stream, Z, z_b, a.W0, w0_b, snap, DF, snap_b, S, s_b, s_g, p.Gp, Vt,
                     long(p.Tp), vt_b, static_cast<TOut*>(a.O), v_b, a.T, a.F, a.D, a.C, p.G,
                     p.ntt, p.ntd);
  if (clk) clk->close(1);

  // 2 (last): final state
  if (a.W_final) {
    if (clk) clk->open(2);
    update(p.n_groups - 1, a.W_final, DF);
    if (clk) clk->close(1);
  }
  return hipGetLastError();
}

}  // namespace

size_t scan_mfma_workspace(int B, int T, int F, int D, int C) {
  return make_plan(B, T, F, D, C).total;
}

hipError_t scan_mfma(const ScanArgs& a, PhaseClock* clk) {
  return a.out_bf16 ? run<uint16_t>(a, clk) : run<float>(a, clk);
}

}  // namespace ttt
