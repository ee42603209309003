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
//   0 stage      token-major copies Zt, Vt so that every product below reads operands with the
//                contraction index contiguous -- K-blocked [Tp/64][rows][64] when the shapes
//                allow whole 64-token steps (each step of a tile is then one contiguous block,
//                which keeps address translation local), else row-major [rows][Tp] -- and
//                bf16(W_0);
//   1 corr       S_g = eta * mask(Z_g Z_g^T) blocks for all groups at once (bf16);
//   2 update     W_{g+1} = W_g + eta * Vt_g Zt_g^T for all groups in one launch: each workgroup
//                owns a tile of the fp32 state for the whole sequence and writes a bf16
//                snapshot of it at every group boundary (K-blocked by 32: [d_ff/32][d_model][32]);
//   3 apply      O_g = Z_g bf16(W_g)^T + S_g V_g for all groups in one launch.
//
// The unmasked state chain, correction blocks (whole 256-token chunks) and apply (whole 32-token
// chunks) run on the eight-wave engine of pingpong.hpp (512 threads, 256 x 256 tiles, 32-wide K
// steps through four direct-copy LDS stages). The masked forms use one workgroup shape: 256 threads as 2x2 waves, a 256 x BN output tile
// (BN = 256 or 128) built from v_mfma_f32_32x32x16_bf16 blocks, K steps of 64 staged through
// double-buffered LDS. Within a K step the fragments of sub-step s+1 are read while sub-step s
// multiplies, and the next K step's tile is written to the idle LDS buffer (with the global loads
// for the step after it issued right behind) while the current one multiplies: one barrier per
// K step. Products are oriented so that the accumulator's M axis is the contiguous axis of the
// output, and the epilogue goes through LDS so that stores are 1 KB runs per wave. Tiles are mapped so that each XCD works on a
// contiguous range of logical tiles that share operand panels in its L2.
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "dma.hpp"
#include "engine.hpp"
#include "launch.hpp"
#include "pingpong.hpp"

namespace ttt {
namespace {

// ---------------------------------------------------------------------------------------------
// Phase 0: token-major copy of in[b][t][c] (t < T; zero for T <= t < Tp; N % 16 == 0).
// BLOCKED: out[b][t / 32][c][t % 32], so that one 32-token K step of any row range is one
// contiguous block (a 256-row tile's step: 16 KB, read as whole cache lines); otherwise
// out[b][c][t] with row pitch Tp.
template <bool BLOCKED>
__global__ __launch_bounds__(256) void k_stage(const uint16_t* __restrict__ in,
                                               uint16_t* __restrict__ out, int T, int Tp, int N,
                                               long in_b, long out_b, unsigned* __restrict__ zero,
                                               int nzero) {
  __shared__ uint16_t tile[64][64 + 2];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z, tid = threadIdx.x;
  // (when bf16(W_0) is not converted separately, the state chain's flags are zeroed here)
  if (t0 == 0 && c0 == 0 && b == 0)
    for (int i = tid; i < nzero; i += 256) zero[i] = 0u;
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
      uint4* p = reinterpret_cast<uint4*>(
          BLOCKED ? out + long((t0 + tq) / 32) * N * 32 + long(c0 + c) * 32 + (tq & 31)
                  : out + long(c0 + c) * Tp + t0 + tq);
      p[0] = make_uint4(w[0], w[1], w[2], w[3]);
      p[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

// Phase 0: bf16 snapshot of the initial state in[b] ([D][F] row-major fp32; in_b = 0 when every
// sequence starts from the same state). BLOCKED: K-blocked by 32, out[f / 32][d][f % 32] (the
// layout of every snapshot of the unmasked path); else out[d][f].
template <bool BLOCKED>
__global__ __launch_bounds__(256) void k_to_bf16(const float* __restrict__ in, long in_b,
                                                 uint16_t* __restrict__ out, long out_b, int D,
                                                 int F, unsigned* __restrict__ zero, int nzero) {
  const int b = blockIdx.y;
  // the state chain's hand-over flags start every call at zero
  if (b == 0 && blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0u;
  const float4* src = reinterpret_cast<const float4*>(in + b * in_b);
  uint16_t* dst = out + b * out_b;
  const long n4 = long(D) * F / 4;
  for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += long(gridDim.x) * blockDim.x) {
    const long e = 4 * i;
    const int d = int(e / F), f = int(e % F);
    const long o = BLOCKED ? long(f / 32) * D * 32 + long(d) * 32 + f % 32 : e;
    *reinterpret_cast<uint2*>(dst + o) = pack4(src[i]);
  }
}

// ---------------------------------------------------------------------------------------------
// Phase 1: S_g[t - g0][s - sbase] = eta * (z_t . z_s) if g0 <= s and chunk(s) < chunk(t), else 0,
// for t in group g = [g0, g1) and s up to the chunk start of the tile's last row.
// Product orientation: M = s (contiguous in S), N = t.
constexpr int CORR_BN = 128;
constexpr int APP_BN = 256;  // token tile of the apply phase (declared here: k_corr covers its reads)
static_assert(APP_BN % CORR_BN == 0, "correction tiles must nest in apply tiles");
template <bool FAST>
__global__ __launch_bounds__(NTHR, 1) void k_corr(const uint16_t* __restrict__ Z, long z_b,
                                                  uint16_t* __restrict__ S, long s_b, long s_g,
                                                  int Gp, int T, int F, int C, int G, int ntt,
                                                  int nst, float eta) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = ntt * nst;
  const int g = tile / per_g, rem = tile % per_g, tt = rem / nst, st = rem % nst;
  const int g0 = g * G, g1 = min(g0 + G, T);
  const int t_start = g0 + tt * CORR_BN;
  if (t_start >= g1) return;
  const int t_end = min(t_start + CORR_BN, g1);
  // The apply tile holding these rows reads S columns up to the chunk start of ITS last row,
  // so every such column must be written here (zeros where the mask removes it).
  const int app_end = min(g0 + ((t_start - g0) / APP_BN + 1) * APP_BN, g1);
  const int cs_need = ((app_end - 1) / C) * C;
  const int sbase = g0 & ~7;
  const int s_start = sbase + st * BM;
  if (!(s_start < cs_need && s_start + BM > g0)) return;
  const uint16_t* Zb = Z + b * z_b;
  Acc<CORR_BN> acc;
  zero_acc<CORR_BN>(acc);
  __shared__ Smem<CORR_BN> sm;
  Rows<BM, FAST> la(Zb + long(s_start) * F, F, min(BM, T - s_start), 0, F, tid);
  Rows<CORR_BN, FAST> lb(Zb + long(t_start) * F, F, t_end - t_start, 0, F, tid);
  mma_segment<CORR_BN>(acc, la, lb, 0, F, sm, tid);
  float* stage = reinterpret_cast<float*>(&sm);
  uint16_t* Sg = S + b * s_b + g * s_g;
  store_tile_raw<CORR_BN>(acc, stage, tid, [&](int n, int m, float4 v) {
    const int s = s_start + m, t = t_start + n;
    if (t < t_end && s - sbase < Gp) {
      const int ct = t / C;
      float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool keep = s + u >= g0 && (s + u) / C < ct;
        e[u] = keep ? eta * e[u] : 0.f;
      }
      *reinterpret_cast<uint2*>(Sg + long(t - g0) * Gp + (s - sbase)) =
          pack4(make_float4(e[0], e[1], e[2], e[3]));
    }
  });
}

// Fast correction blocks, for chunks that are whole 256-token tiles and whole 64-wide K steps.
// A chunk pair (tc, sc), sc < tc, of a group is (C / 256)^2 tiles of 256 (t) x 256 (s), each
// either wholly kept or wholly masked, so only the kept tiles are formed: on the eight-wave engine
// of pingpong.hpp, with the d_ff contraction split in two halves on two workgroups (the kept
// tiles of a 32k-token sequence in 1024-token groups are 128, too few to fill the chip), each
// writing its fp32 partial tile. k_corr_finish adds the halves, scales by eta and writes the
// bf16 S blocks the apply reads. Tile id = (group, pair, t sub-tile, s sub-tile); pairs in the
// order (1,0), (2,0), (2,1), (3,0), ...
__device__ __forceinline__ void corr_tile(int tile, int tpg, int sub, int G, int C, int& g,
                                          int& t0, int& s0) {
  g = tile / tpg;
  const int r = tile % tpg, sub2 = sub * sub;
  const int pair = r / sub2, ab = r % sub2;
  int tc = 1, first = 0;
  while (first + tc <= pair) {
    first += tc;
    ++tc;
  }
  const int sc = pair - first;
  t0 = g * G + tc * C + (ab / sub) * PP_T;
  s0 = g * G + sc * C + (ab % sub) * PP_T;
}

__global__ __launch_bounds__(512, 1) void k_corr_pp(const uint16_t* __restrict__ Z, long z_b,
                                                   float* __restrict__ part, long part_half,
                                                   int T, int F, int C, int G, int tpg, int sub,
                                                   int n_tiles, int ksplit) {
  __shared__ PPSmem<4> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int id = xcd_remap(blockIdx.x, gridDim.x);  // the tiles of a group meet in one L2
  const int half = id & 1, tile = id >> 1;
  int g, t0, s0;
  corr_tile(tile, tpg, sub, G, C, g, t0, s0);
  if (t0 >= T) return;  // the ragged last group has fewer chunks
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nt = min(PP_T, T - t0);  // rows past T re-read row T - 1 (never stored)
  const int kbeg = half ? ksplit : 0, kend = half ? F / PP_BK : ksplit;  // 32-wide K steps
  const uint16_t* Zb = Z + b * z_b + long(kbeg) * PP_BK;
  const PPOp oa(Zb + long(s0) * F, 128, 0, wave, lane, [=](int r) { return r * F * 2; });
  const PPOp ob(Zb + long(t0) * F, 128, PP_OPB, wave, lane,
                [=](int r) { return min(r, nt - 1) * F * 2; });
  PPAcc acc;
  pp_zero(acc);
  pp_segment<4>(acc, oa, ob, kend - kbeg, sm, wave, lane);
  // partial tile [t - t0][s - s0] fp32; acc[i][j] holds s = pp_row(.., i, 0..3) of t = pp_col
  float* pt = part + half * part_half + (long(b) * n_tiles + tile) * (PP_T * PP_T);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(pt + pp_col(wave, lane, j) * PP_T + pp_row(wave, lane, i, 0)) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
}

// S_g[t - g0][s - g0] = bf16(eta * (P0 + P1)) over the kept tiles; one thread per 8 columns
__global__ __launch_bounds__(256) void k_corr_finish(const float* __restrict__ part,
                                                     long part_half, uint16_t* __restrict__ S,
                                                     long s_b, long s_g, int Gp, int T, int C,
                                                     int G, int tpg, int sub, int n_tiles,
                                                     float eta) {
  const int b = blockIdx.y;
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;  // tile, row, 8-column group
  const int tile = int(i / (PP_T * PP_T / 8)), w = int(i % (PP_T * PP_T / 8));
  if (tile >= n_tiles) return;
  const int tl = w / (PP_T / 8), sl = (w % (PP_T / 8)) * 8;
  int g, t0, s0;
  corr_tile(tile, tpg, sub, G, C, g, t0, s0);
  if (t0 + tl >= T) return;
  const float* p0 = part + (long(b) * n_tiles + tile) * (PP_T * PP_T) + tl * PP_T + sl;
  const float* p1 = p0 + part_half;
  const float4 a0 = *reinterpret_cast<const float4*>(p0), a1 = *reinterpret_cast<const float4*>(p0 + 4);
  const float4 c0 = *reinterpret_cast<const float4*>(p1), c1 = *reinterpret_cast<const float4*>(p1 + 4);
  const uint2 lo = pack4(make_float4(eta * (a0.x + c0.x), eta * (a0.y + c0.y),
                                     eta * (a0.z + c0.z), eta * (a0.w + c0.w)));
  const uint2 hi = pack4(make_float4(eta * (a1.x + c1.x), eta * (a1.y + c1.y),
                                     eta * (a1.z + c1.z), eta * (a1.w + c1.w)));
  const int g0 = g * G;
  *reinterpret_cast<uint4*>(S + b * s_b + g * s_g + long(t0 + tl - g0) * Gp + (s0 + sl - g0)) =
      make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// ---------------------------------------------------------------------------------------------
// Phase 2: the whole state chain in one launch. The recurrence W_{g+1} = W_g + eta * dW_g is
// local to every (f, d) element, so a workgroup owns one 256 (f) x 128 (d) tile of W for the
// whole sequence. The tile lives in the product accumulator itself, scaled by 1/eta
// (U = W / eta): the matrix cores then add Vt Zt^T straight into the state, with no second
// register copy and no per-group fold. The tokens stream through one uninterrupted K pipeline
// (A = Zt rows f, B = Vt rows d, K = tokens); at each group start the bf16 snapshot
// W_g = bf16(eta * U) is packed into registers and written a slice per K step while the group
// runs. W_0 is read once and W_final = eta * U written once. (eta = 0 never comes here.)
constexpr int UPD_BN = 128;
// Masked variant (any shape): one mma_segment per group on the register-staged engine; the unmasked
// shapes use k_update_pp below.
template <bool FAST>
__global__ __launch_bounds__(NTHR, 1) void k_update_chain(
    const uint16_t* __restrict__ Zt, const uint16_t* __restrict__ Vt, long ldt, long zt_b,
    long vt_b, const float* W0, long w0_b, float* W_final, uint16_t* __restrict__ Wbf,
    long wbf_b, int D, int F, int T, int G, int n_groups, float eta, int tiles_n) {
  __shared__ Smem<UPD_BN> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile / tiles_n, tn = tile % tiles_n;  // consecutive tiles share the Zt panel
  const int f0 = tm * BM, d0 = tn * UPD_BN;
  const int wave = tid >> 6, lane = tid & 63, wm = wave >> 1, wn = wave & 1;
  constexpr int NT = UPD_BN / 64;
  static_assert(NT == 2 && MT == 4, "snapshot slices assume a 256 x 128 state tile");
  const long DF = long(D) * F;

  // U in the accumulator layout: acc[i][j][e] = W[d][f] / eta at
  // f = f0 + wm*128 + i*32 + 8*(e/4) + 4*(lane/32) + e%4, d = d0 + wn*64 + j*32 + lane%32
  Acc<UPD_BN> acc;
  const float* w0 = W0 + b * w0_b;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = f0 + wm * 128 + i * 32 + 8 * q + 4 * (lane >> 5);
        const int d = d0 + wn * 64 + j * 32 + (lane & 31);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (d < D && f < F) v = *reinterpret_cast<const float4*>(w0 + long(d) * F + f);
        acc[i][j][4 * q] = v.x / eta;
        acc[i][j][4 * q + 1] = v.y / eta;
        acc[i][j][4 * q + 2] = v.z / eta;
        acc[i][j][4 * q + 3] = v.w / eta;
      }

  uint16_t* wbf = Wbf + b * wbf_b;
  // element offset of snapshot element (d, f): FAST snapshots are [F/32][D][32]
  auto snap_off = [&](int d, int f) -> long {
    return FAST ? long(f / 32) * D * 32 + long(d) * 32 + f % 32 : long(d) * F + f;
  };
  auto snap4 = [&](int i, int j, int q) {
    return pack4(make_float4(eta * acc[i][j][4 * q], eta * acc[i][j][4 * q + 1],
                             eta * acc[i][j][4 * q + 2], eta * acc[i][j][4 * q + 3]));
  };
  // The whole snapshot gi at once, through a per-wave LDS staging block (64 d x 64 f, rows
  // padded to 72) so that every pass is one contiguous 8 KB run.
  __shared__ __attribute__((aligned(16))) uint16_t stg[4][64 * 72];
  uint16_t* my = stg[wave];
  auto burst = [&](int gi) {
    uint16_t* snap = wbf + long(gi) * DF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // f rows [wm*128 + 64h, +64) of this wave's sub-tile
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = j * 32 + (lane & 31);
            const int ml = ii * 32 + 8 * q + 4 * (lane >> 5);
            *reinterpret_cast<uint2*>(my + nl * 72 + ml) = snap4(2 * h + ii, j, q);
          }
      // (LDS instructions of one wave execute in order: no wait between write and read-back)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int nl = r * 8 + (lane >> 3), ml = (lane & 7) * 8;
        const int d = d0 + wn * 64 + nl, f = f0 + wm * 128 + 64 * h + ml;
        const uint4 v = *reinterpret_cast<const uint4*>(my + nl * 72 + ml);
        if (d < D && f < F) *reinterpret_cast<uint4*>(snap + snap_off(d, f)) = v;
      }
    }
  };

  {
    for (int g = 0; g < n_groups; ++g) {
      const int t0 = g * G, t1 = min(t0 + G, T);
      if (g > 0) burst(g);
      Rows<BM, false> la(Zt + b * zt_b + long(f0) * ldt, ldt, min(BM, F - f0), t0, t1, tid);
      Rows<UPD_BN, false> lb(Vt + b * vt_b + long(d0) * ldt, ldt, min(UPD_BN, D - d0), t0, t1,
                             tid);
      mma_segment<UPD_BN>(acc, la, lb, t0, t1, sm, tid);
    }
  }

  if (W_final) {
    float* wf = W_final + b * DF;
    store_tile<UPD_BN>(acc, sm, tid, [&](int n, int m, float4 v) {
      const int d = d0 + n, f = f0 + m;
      if (d < D && f < F)
        *reinterpret_cast<float4*>(wf + long(d) * F + f) =
            make_float4(eta * v.x, eta * v.y, eta * v.z, eta * v.w);
    });
  }
}

// Unmasked variant on the eight-wave engine (pingpong.hpp): one pipeline over every token (group
// boundaries fall between 32-token steps), 256 (f) x 256 (d) state tiles, 512 threads. Wave w
// owns rows f0 + 128 ((w >> 1) & 1) + [0, 128) and columns d0 + 64 ((w & 1) + 2 (w >> 2)) + [0, 64)
// of the tile. A = Z read in its own token-major layout (no transposed copy), B = the staged Vt.
// At the start of group g each wave writes its part of the snapshot W_g = bf16(eta U) straight
// from the accumulator: packed, two lane permutes per pair of blocks, then 16 store instructions
// of one contiguous 1 KB each (K-blocked by 32, below; no LDS round trip). (Holding the packed snapshot in registers
// to spread its stores over the group, as a four-wave kernel can, does not fit here: two waves
// share each SIMD's registers.) Lanes whose element lies outside W write to `sink`, so a flush is
// always 16 store instructions (the copy waits count them).
constexpr int UPD_T = PP_T;  // state tile edge (f and d)
constexpr int UPD_NS = 4;    // LDS stages of 32 KB
constexpr int UPD_TILE_FLOATS = UPD_T * UPD_T;  // one state tile handed from the first half
// Bounded wait of a second-half workgroup for its first half: by default 2^19 polls with
// s_sleep 8 between them (about 0.1 s) plus 16 polls (about 4 us) per 32-token step of the first
// half, which takes about 1 us per step: a first half takes about a millisecond at 32k tokens
// and the bound grows with it. Workgroups are dispatched in index order and every first half
// precedes every second half, so the wait always ends. If it ever ran out, the second half does
// not use the hand-over at all: it starts from W_0 at token 0 and runs the first half's steps
// itself (the same products in the same order, so the same bits; the snapshots it writes on the
// way equal the first half's), and counts the event in the workspace. The result is then
// correct, only later. (A test sets the number of polls to 0 to run this path.)
constexpr int UPD_SPIN_LIMIT = 1 << 19;
constexpr int UPD_STAGGER_TICKS = 400;  // 4 us of the 100 MHz real-time counter

// Token split of the state chain. 256 x 256 tiles of a 2560 x 9728 state are 380 workgroups,
// about 1.5 rounds of the 256 compute units. Splitting every tile's token stream at a group
// boundary near its middle gives 2 x 380 half-length workgroups, about three even rounds: the
// first half (workgroups [0, n)) starts from W_0, runs to the split and hands its fp32 state
// to the second half (workgroups [n, 2n)), which continues from it to the end. The result is
// bit for bit that of one unsplit pass (same products in the same order).
//   mid    [B][n][8 waves][32][64 lanes][4] fp32 state in accumulator order (1 KB per store)
//   flags  [B][n] 0 before the call (zeroed by k_to_bf16), 1 once the first half's state is out
//   err    one word, incremented by a second half whose wait ran out (it then recomputed the
//          first half's steps itself)
template <bool RESETS>
__global__ __launch_bounds__(512, 1) void k_update_pp(
    const uint16_t* __restrict__ Z, const uint16_t* __restrict__ Vt, long z_b, long vt_b,
    const float* W0, long w0_b, float* W_final, uint16_t* __restrict__ Wbf, long wbf_b,
    uint16_t* sink, float* mid, unsigned* flags, unsigned* err, int D, int F, int T, int G,
    float eta, int tiles_n, int n_tiles, int split_steps, int spin_limit, int n_units,
    int steps_per_unit, int inside, ResetMask resets) {
  __shared__ PPSmem<UPD_NS> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const bool second = split_steps > 0 && int(blockIdx.x) >= n_tiles;
  const bool first = split_steps > 0 && !second;
  const int tile = xcd_remap(int(blockIdx.x) - (second ? n_tiles : 0), n_tiles);
  const int tm = tile / tiles_n, tn = tile % tiles_n;  // consecutive tiles share the Z panel
  const int f0 = tm * UPD_T, d0 = tn * UPD_T;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int fw = f0 + 128 * ((wave >> 1) & 1), dw = d0 + 64 * ((wave & 1) + 2 * (wave >> 2));
  const long DF = long(D) * F;
  const int nk_all = (T + PP_BK - 1) / PP_BK;
  float* my_mid = mid + (long(b) * n_tiles + tile) * UPD_TILE_FLOATS + wave * 8192 + lane * 4;
  unsigned* my_flag = flags + long(b) * n_tiles + tile;

  if (!second && (first ? split_steps : nk_all) >= 16 * (G / PP_BK)) {
    // Workgroups that start at token 0 reach every group boundary at about the same time, and
    // every one then writes its 128 KB snapshot at once. On streams of 16 groups or more they
    // start in four phases UPD_STAGGER_TICKS apart (by blockIdx.x mod 4; the offsets carry over
    // to the workgroups that later take their compute units), which spreads those bursts: 0.5-0.6%
    // off the step at 32k tokens in interleaved runs, same bits. The wait is bounded by the
    // 100 MHz real-time counter.
    const long delay = long(blockIdx.x & 3) * UPD_STAGGER_TICKS;
    if (delay > 0) {
      const long t0 = long(__builtin_amdgcn_s_memrealtime());
      while (long(__builtin_amdgcn_s_memrealtime()) - t0 < delay) __builtin_amdgcn_s_sleep(8);
    }
  }
  // U = W / eta in the accumulator layout: acc[i][j][e] holds
  // f = fw + 16 i + 4 (lane / 16) + e, d = dw + 16 j + lane % 16
  PPAcc acc;
  bool handed = false;  // a second half that received its first half's state
  if (second) {
    if (tid == 0) {
      bool seen = false;
      for (int spins = 0; spins < spin_limit; ++spins) {
        if (__hip_atomic_load(my_flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          seen = true;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      // (the word sits in the first stage, which no copy has reached yet)
      *reinterpret_cast<volatile int*>(&sm.st[0][0]) = seen ? 1 : 0;
      if (!seen) __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    handed = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(&sm.st[0][0])) != 0;
    __syncthreads();  // every wave has read the word before the first copies overwrite it
  }
  // steps [s0, s1): a first half runs [0, split), a second half [split, end) from the handed
  // state or, if its wait ran out, [0, end) from W_0 like an unsplit workgroup
  const int s0 = handed ? split_steps : 0, s1 = first ? split_steps : nk_all;
  // acc = W_0 itself (scale false) or W_0 / eta
  auto load_w0 = [&](bool scale) {
    const float* w0 = W0 + b * w0_b;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = fw + i * 16 + 4 * (lane >> 4);
        const int d = dw + j * 16 + (lane & 15);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (d < D && f < F) v = *reinterpret_cast<const float4*>(w0 + long(d) * F + f);
        acc[i][j][0] = scale ? v.x / eta : v.x;
        acc[i][j][1] = scale ? v.y / eta : v.y;
        acc[i][j][2] = scale ? v.z / eta : v.z;
        acc[i][j][3] = scale ? v.w / eta : v.w;
      }
  };
  // The starting state, loaded by one loop whichever its source (so that the accumulator is
  // defined once): the handed state, already U = W / eta in accumulator order, or W_0 itself
  // (divided by eta below, after its bf16 snapshot has been written from it)
  {
    const float* w0 = W0 + b * w0_b;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = fw + i * 16 + 4 * (lane >> 4);
        const int d = dw + j * 16 + (lane & 15);
        const float* src = handed ? my_mid + (i * 4 + j) * 256 : w0 + long(d) * F + f;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (handed || (d < D && f < F)) v = *reinterpret_cast<const float4*>(src);
        acc[i][j][0] = v.x;
        acc[i][j][1] = v.y;
        acc[i][j][2] = v.z;
        acc[i][j][3] = v.w;
      }
  }

  // Snapshot W_g = bf16(eta U) at the start of group g (g >= 1; group 0's is bf16(W_0), written
  // by the first workgroups from W_0 itself before the stream starts, or in the document
  // instance by the separate conversion kernel), written from the accumulator in step gstart's
  // memory phase, before any product of the group. The snapshot is K-blocked by 32,
  // [F/32][D][32]: row d of block q holds f = 32 q .. 32 q + 31 (64 bytes), and the rows of a
  // block follow one another. Lane l of 16-lane row g = l / 16 holds, for accumulator block
  // (i, j), f = fw + 16 i + 4 g + 0..3 of row d = dw + 16 j + l % 16 (8 bytes once packed). For a
  // pair of blocks X = (2 q, j), Y = (2 q + 1, j), a permlane32 swap and then a permlane16 swap
  // leave row g of (X, Y) holding rows (g, g + 1) of X for g = 0, (2, 3) of X for g = 1, (0, 1)
  // of Y for g = 2 and (2, 3) of Y for g = 3: every lane then holds f = fw + 32 q + 8 g + 0..7 of
  // its row d, and one store instruction writes 16 rows d x 64 bytes, a contiguous 1 KB.
  uint16_t* wbf = Wbf + b * wbf_b;
  uint16_t* const lane_sink = sink + lane * 8;
  const int lg = lane >> 4;
  const int lane_el = (lane & 15) * 32 + 8 * lg;  // this lane's 16 bytes inside a 1 KB run
  const bool whole = d0 + UPD_T <= D && f0 + UPD_T <= F;  // no lane of the tile is outside W
  // blocks q = 2 h .. 2 h + 1 (f pairs), columns j = 2 jj .. 2 jj + 1: four store instructions
  auto flush = [&](uint16_t* snap, int h, int jj, float scale) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int jl = 0; jl < 2; ++jl) {
        const int q = 2 * h + qq, j = 2 * jj + jl;
        const f32x4& x = acc[2 * q][j];
        const f32x4& y = acc[2 * q + 1][j];
        const uint2 px = pack4(make_float4(scale * x[0], scale * x[1], scale * x[2], scale * x[3]));
        const uint2 py = pack4(make_float4(scale * y[0], scale * y[1], scale * y[2], scale * y[3]));
        // rows 2, 3 of X <-> rows 0, 1 of Y; then odd rows of X <-> even rows of Y
        const auto ax = __builtin_amdgcn_permlane32_swap(px.x, py.x, false, false);
        const auto ay = __builtin_amdgcn_permlane32_swap(px.y, py.y, false, false);
        const auto bx = __builtin_amdgcn_permlane16_swap(ax[0], ax[1], false, false);
        const auto by = __builtin_amdgcn_permlane16_swap(ay[0], ay[1], false, false);
        uint16_t* p = snap + (long((fw >> 5) + q) * D + dw + 16 * j) * 32 + lane_el;
        if (!whole) {
          const int f = fw + 32 * q + 8 * lg, d = dw + 16 * j + (lane & 15);
          if (!(d < D && f < F)) p = lane_sink;
        }
        // streamed past the caches: the snapshots are read back only by a later phase, and the
        // L2 is better spent on the operand panels other workgroups of this XCD still need
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4_t{bx[0], by[0], bx[1], by[1]},
                                    reinterpret_cast<u32x4_t*>(p));
        __builtin_amdgcn_sched_barrier(0);  // one run at a time: few registers in flight
      }
  };
  if (!handed) {
    // group 0's snapshot bf16(W_0), from W_0 itself (its stores drain behind the first copies)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) flush(wbf, h, j, 1.f);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = acc[i][j][e] / eta;
  }
  // group boundaries fall on multiples of spg steps; the split is one of them
  const int spg = G / PP_BK;
  int next_group = s0 > 0 ? s0 : spg;  // first step (absolute) of the next group
  // The snapshot of each group boundary the stream reaches, from the accumulator, in the memory
  // phase of the boundary's step (before any product of the group). `base` is the absolute step
  // of the stream's first step.
  auto post_from = [&](int base) {
    return [&, base](int u, int& ops) {
      if (base + u == next_group) {
        uint16_t* snap = wbf + long(next_group / spg) * DF;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 2; ++j) flush(snap, h, j, eta);
        ops += 16;
        next_group += spg;
      }
    };
  };
  auto pre = [](int) {};
  // waits: copies of whole steps (4 operations each) plus the block stores issued since: 8 in
  // the steady state (two later steps' copies), 24 in the three steps after a snapshot (its 16
  // stores besides), checked by equality first; other counts (the tail) round down
  using WL = WaitFast<std::integer_sequence<int, 8, 24>, WaitList<20, 16, 12, 8, 4, 0>>;
  const int nd = min(UPD_T, D - d0);
  // steps [a, e) through the streaming loop (a run of whole 32-token steps from token 32 a)
  auto stream = [&](int a, int e) {
    const long k0 = long(a) * PP_BK;  // first token (a multiple of 32)
    const PPOpN oa(Z + b * z_b + k0 * F + f0, long(F) * 2, T - int(k0), min(UPD_T, F - f0), 0,
                   wave, lane);
    // V_hat^T is K-blocked by 32: each 32-token step of the tile is one contiguous 16 KB block
    const PPOpS ob(Vt + b * vt_b + (k0 / 32) * long(D) * 32 + long(d0) * 32, long(D) * 64, 64,
                   16, PP_OPB, wave, lane, nd);
    pp_stream<UPD_NS, WL>(acc, oa, ob, e - a, sm, wave, lane, pre, post_from(a));
  };
  if constexpr (RESETS) {
    // Documents: a start puts the state back to W_0. At a group boundary the snapshot is then
    // bf16(W_0) from W_0 itself and the accumulator W_0 / eta, as at the start of a scan (the
    // same bits as a separate scan of the document); a start inside a group (`inside`, on a
    // multiple of steps_per_unit steps) only puts the accumulator back to W_0 / eta. The stream
    // runs one document segment at a time through the same streaming loop as the plain scan,
    // and the resets fall between segments, outside it: with the reset test inside the loop,
    // the loop's register allocation cost a third of the chain's time. (The W_0 loads are
    // ordinary loads; each segment's loop starts with no copy in flight.)
    auto reset_at = [&](int step) {  // uniform: the mask word through readfirstlane
      const int bit = b * n_units + step / steps_per_unit;
      const uint32_t word = __builtin_amdgcn_readfirstlane(resets.bits[bit >> 5]);
      return ((word >> (bit & 31)) & 1u) != 0u;
    };
    auto is_reset = [&](int s) {
      return s % steps_per_unit == 0 && (s % spg == 0 || inside) && reset_at(s);
    };
    int a = s0;
    while (a < s1) {
      if (is_reset(a)) {
        load_w0(false);
        if (a % spg == 0) {
          uint16_t* snap = wbf + long(a / spg) * DF;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 2; ++j) flush(snap, h, j, 1.f);
          next_group = a + spg;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = acc[i][j][e] / eta;
      }
      int e = (a / steps_per_unit + 1) * steps_per_unit;  // the next unit start after a
      while (e < s1 && !is_reset(e)) e += steps_per_unit;
      e = min(e, s1);
      stream(a, e);
      a = e;
    }
  } else {
    stream(s0, s1);
  }

  if (first) {
    // hand the state over: every thread's stores are done and ordered before thread 0's release
    // (workgroup barrier, then an agent-scope release store that makes them visible to every XCD)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(my_mid + (i * 4 + j) * 256) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's state is in the L2
    __syncthreads();
    if (tid == 0) __hip_atomic_store(my_flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else if (W_final) {
    // straight from the accumulator: each store writes 64 bytes (16 consecutive f) of 16 rows
    // d; a wave's stores complete whole 512-byte runs of every row it touches
    float* wf = W_final + b * DF;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = fw + i * 16 + 4 * (lane >> 4);
        const int d = dw + j * 16 + (lane & 15);
        if (d < D && f < F)
          *reinterpret_cast<float4*>(wf + long(d) * F + f) =
              make_float4(eta * acc[i][j][0], eta * acc[i][j][1], eta * acc[i][j][2],
                          eta * acc[i][j][3]);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Phase 3: O[t][d] = sum_f bf16(W_g)[d][f] Z[t][f] + sum_s Vt[d][s] S_g[t][s] for every group g.
// Product orientation: M = d (contiguous in O), N = t.
template <typename TOut, bool FAST>
__global__ __launch_bounds__(NTHR, 1) void k_apply(
    const uint16_t* __restrict__ Z, long z_b, const uint16_t* __restrict__ Wbf, long wbf_g,
    long wbf_b, const uint16_t* S, long s_b, long s_g, int Gp, const uint16_t* __restrict__ Vt,
    long ldt, long vt_b, TOut* __restrict__ O, long o_b, int T, int F, int D, int C, int G,
    int ntt, int ntd) {
  __shared__ Smem<APP_BN> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = ntt * ntd;
  const int g = tile / per_g, rem = tile % per_g, tt = rem / ntd, td = rem % ntd;
  const int g0 = g * G, g1 = min(g0 + G, T);
  const int t_start = g0 + tt * APP_BN;
  if (t_start >= g1) return;
  const int t_end = min(t_start + APP_BN, g1);
  const int d0 = td * BM;
  const uint16_t* Wg = Wbf + b * wbf_b + long(g) * wbf_g;
  Acc<APP_BN> acc;
  zero_acc<APP_BN>(acc);
  {
    // FAST snapshots are K-blocked by 32: [F/32][D][32]
    Rows<BM, FAST> la(Wg + long(d0) * (FAST ? 32 : F), FAST ? 32 : F, min(BM, D - d0), 0, F, tid,
                      FAST ? long(D) * BK : BK, FAST ? long(D) * 32 : 0);
    Rows<APP_BN, FAST> lb(Z + b * z_b + long(t_start) * F, F, t_end - t_start, 0, F, tid);
    mma_segment<APP_BN>(acc, la, lb, 0, F, sm, tid);
  }
  const int cs_last = ((t_end - 1) / C) * C;
  if (S != nullptr && cs_last > g0) {
    const int sbase = g0 & ~7;
    const uint16_t* Sg = S + b * s_b + g * s_g;
    // FAST: Vt is K-blocked by 32 and g0 = sbase is a whole number of blocks
    Rows<BM, FAST> la(FAST ? Vt + b * vt_b + long(g0 / 32) * D * 32 + long(d0) * 32
                           : Vt + b * vt_b + long(d0) * ldt + sbase,
                      FAST ? 32 : ldt, min(BM, D - d0), g0 - sbase, cs_last - sbase, tid,
                      FAST ? long(D) * BK : BK, FAST ? long(D) * 32 : 0);
    Rows<APP_BN, FAST> lb(Sg + long(t_start - g0) * Gp, Gp, t_end - t_start, g0 - sbase,
                          cs_last - sbase, tid);
    mma_segment<APP_BN>(acc, la, lb, g0 - sbase, cs_last - sbase, sm, tid);
  }
  TOut* ob = O + b * o_b;
  store_tile<APP_BN>(acc, sm, tid, [&](int n, int m, float4 v) {
    const int d = d0 + m, t = t_start + n;
    if (t < t_end && d < D) {
      if constexpr (sizeof(TOut) == 2)
        *reinterpret_cast<uint2*>(ob + size_t(t) * D + d) = pack4(v);
      else
        *reinterpret_cast<float4*>(ob + size_t(t) * D + d) = v;
    }
  });
}

// ---------------------------------------------------------------------------------------------
// Unmasked apply on the eight-wave engine (pingpong.hpp), for chunks that are whole 32-token steps:
// the same 256 (d) x 256 (t) tiles and products as k_apply, each as a plain segment of 32-wide
// K steps (bit-identical results, about 0.1 ms faster at the 32k-token workload). A = the
// snapshot rows d (K-blocked), B = the Z rows t; then, for tiles past a group's first chunk,
// A = the V_hat^T rows d (K-blocked over tokens), B = the S rows t.
// RESETS: documents may also start at chunks inside a group, on token tile edges (the host
// checks). A tile at or after such a start (the last one in its group at or before the tile)
// applies bf16(W_0), group 0's snapshot, and takes the correction only from that start on.
static_assert(APP_BN == PP_T, "the eight-wave apply uses the apply phase's token tiles");
template <typename TOut, bool RESETS>
__global__ __launch_bounds__(512, 1) void k_apply_pp(
    const uint16_t* __restrict__ Z, long z_b, const uint16_t* __restrict__ Wbf, long wbf_g,
    long wbf_b, const uint16_t* S, long s_b, long s_g, int Gp, const uint16_t* __restrict__ Vt,
    long vt_b, TOut* __restrict__ O, long o_b, int T, int F, int D, int C, int G, int ntt,
    int ntd, int unit, int n_units, ResetMask resets) {
  __shared__ PPSmem<4> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = ntt * ntd;
  // consecutive tiles of a group share a W_g panel: the token tiles of one d tile follow one another
  const int g = tile / per_g, rem = tile % per_g, tt = rem % ntt, td = rem / ntt;
  const int g0 = g * G, g1 = min(g0 + G, T);
  const int t_start = g0 + tt * PP_T;
  if (t_start >= g1) return;
  const int t_end = min(t_start + PP_T, g1);
  const int d0 = td * PP_T;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nd = min(PP_T, D - d0), nt = t_end - t_start;
  const uint16_t* Wg = Wbf + b * wbf_b + long(g) * wbf_g;
  int k_from = g0;  // first token of the tile's document inside the group
  if constexpr (RESETS) {
    for (int u = t_start / unit; u * unit > g0; --u) {
      const int bit = b * n_units + u;
      const uint32_t word = __builtin_amdgcn_readfirstlane(resets.bits[bit >> 5]);
      if ((word >> (bit & 31)) & 1u) {
        k_from = u * unit;
        break;
      }
    }
    k_from = __builtin_amdgcn_readfirstlane(k_from);  // the same in every lane
    if (k_from > g0) Wg = Wbf + b * wbf_b;
  }
  PPAcc acc;
  pp_zero(acc);
  {
    // the snapshot is K-blocked by 32, [F/32][D][32]: each step of the tile is one 16 KB block
    const PPOpS oa(Wg + long(d0) * 32, long(D) * 64, 64, 16, 0, wave, lane, nd);
    const PPOp ob(Z + b * z_b + long(t_start) * F, 128, PP_OPB, wave, lane,
                  [=](int r) { return long(min(r, nt - 1)) * F * 2; });
    pp_segment<4>(acc, oa, ob, F / PP_BK, sm, wave, lane);
  }
  const int cs_last = ((t_end - 1) / C) * C;
  if (S != nullptr && cs_last > k_from) {
    const uint16_t* Sg = S + b * s_b + g * s_g;
    const PPOpS oa(Vt + b * vt_b + long(k_from / 32) * D * 32 + long(d0) * 32, long(D) * 64, 64,
                   16, 0, wave, lane, nd);
    const PPOp ob(Sg + long(t_start - g0) * Gp + (k_from - g0), 128, PP_OPB, wave, lane,
                  [=](int r) { return long(min(r, nt - 1)) * Gp * 2; });
    pp_segment<4>(acc, oa, ob, (cs_last - k_from) / PP_BK, sm, wave, lane);
  }
  TOut* ob_ = O + b * o_b;
  if constexpr (sizeof(TOut) == 2) {
    // bf16 O: staged in the free stage ring, stored as whole 512-byte token rows
    char* st = &sm.st[0][0];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pp_stage_put<PP_T>(st, pp_col(wave, lane, j), pp_row(wave, lane, i, 0),
                           pack4(make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2],
                                             acc[i][j][3])));
    __syncthreads();
    pp_stage_drain<PP_T>(st, tid, [&](int n, int c, const uint4& v) {
      if (n < nt && c * 8 < nd) pp_store_nt(ob_ + size_t(t_start + n) * D + d0 + c * 8, v);
    });
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t_start + pp_col(wave, lane, j);
      if (t >= t_end) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = d0 + pp_row(wave, lane, i, 0);
        if (d >= D) continue;
        *reinterpret_cast<float4*>(ob_ + size_t(t) * D + d) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

// Token unit of the reset bits: group starts (multiples of G) and starts inside a group on the
// apply's token-tile edges (g * G + a multiple of PP_T) are all multiples of gcd(G, PP_T), itself a
// multiple of 32 on the unmasked path (G is a whole number of 64-token K steps there).
int reset_unit(int G) {
  int a = G, b = PP_T;
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

struct Plan {
  int k, G, n_groups, Tp, Gp, ntt_corr, nst, ntt_app, ntd;
  int tiles_m, tiles_n;    // state tiles of the masked update (256 x 128)
  int utiles_m, utiles_n;  // state tiles of the unmasked update (256 x 256)
  int split_steps;         // unmasked update: 32-token step where the token split falls (0: none)
  int nflags;              // hand-over flags (+1: the timeout counter)
  int spin_limit;          // polls of a second half's bounded wait
  int corr_tiles, corr_tpg, corr_sub;  // fast correction: kept 256 x 256 tiles (0: k_corr instead)
  size_t off_zt, off_vt, off_wbf, off_s, off_sink, off_mid, off_flags, off_cp, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Process-wide overrides of three schedule choices, for tests only (set through
// ttt_scan_test_overrides; the defaults below otherwise): the group size in tokens (0: about
// 1024), the state chain's token split (-1: where it pays, 0: never) and the number of polls of a
// second half's bounded wait (-1: the default bound).
std::atomic<int> g_group_tokens{0}, g_split{-1}, g_spin_limit{-1};

Plan make_plan(int B, int T, int F, int D, int C) {
  Plan p{};
  int target = 1024;
  if (const int v = g_group_tokens.load(std::memory_order_relaxed); v > 0) target = v;
  p.k = (target + C / 2) / C;
  if (p.k < 1) p.k = 1;
  const int n_chunks = (T + C - 1) / C;
  if (p.k > n_chunks) p.k = n_chunks;
  p.G = p.k * C;
  p.n_groups = (T + p.G - 1) / p.G;
  p.Tp = (T + 63) / 64 * 64;
  const int pad = (p.G % 8) ? 7 : 0;
  p.nst = (p.G + pad + BM - 1) / BM;
  p.Gp = p.nst * BM;
  p.ntt_corr = (p.G + CORR_BN - 1) / CORR_BN;
  p.ntt_app = (p.G + APP_BN - 1) / APP_BN;
  p.ntd = (D + BM - 1) / BM;
  p.tiles_m = (F + BM - 1) / BM;
  p.tiles_n = (D + UPD_BN - 1) / UPD_BN;
  p.utiles_m = (F + UPD_T - 1) / UPD_T;
  p.utiles_n = (D + UPD_T - 1) / UPD_T;
  const size_t DF = size_t(D) * F;
  size_t off = 0;
  p.off_zt = off;  // token-major Z copy: only the masked path reads one (the other reads Z in place)
  if (!(p.G % BK == 0 && F % BK == 0)) off = align256(off + size_t(B) * F * p.Tp * 2);
  p.off_vt = off;
  off = align256(off + size_t(B) * D * p.Tp * 2);
  p.off_wbf = off;   // bf16 snapshots W_0 .. W_{n-1}
  off = align256(off + size_t(B) * p.n_groups * DF * 2);
  p.off_s = off;
  if (p.k > 1) off = align256(off + size_t(B) * p.n_groups * p.G * p.Gp * 2);
  p.off_sink = off;  // 1 KB written by out-of-range lanes of the update's snapshot stores
  off = align256(off + 1024);
  // token split of the unmasked update: at the group boundary nearest the middle
  p.split_steps = p.n_groups >= 2 ? ((p.n_groups + 1) / 2) * (p.G / 32) : 0;
  if (g_split.load(std::memory_order_relaxed) == 0) p.split_steps = 0;
  p.spin_limit = int(std::min<long>(long(UPD_SPIN_LIMIT) + 16L * p.split_steps, 1L << 30));
  if (const int v = g_spin_limit.load(std::memory_order_relaxed); v >= 0) p.spin_limit = v;
  const size_t n_ut = size_t(p.utiles_m) * p.utiles_n;
  p.nflags = int(size_t(B) * n_ut) + 1;
  p.off_mid = off;  // first-half states handed to the second halves
  if (p.split_steps > 0) off = align256(off + size_t(B) * n_ut * UPD_TILE_FLOATS * 4);
  p.off_flags = off;
  off = align256(off + size_t(p.nflags) * 4);
  // fast correction blocks: chunks of whole 256-token tiles, whole 64-wide K steps
  p.corr_sub = C / PP_T;
  p.corr_tpg = p.k * (p.k - 1) / 2 * p.corr_sub * p.corr_sub;
  p.corr_tiles = (p.k > 1 && C % PP_T == 0 && p.G % BK == 0 && F % BK == 0)
                     ? p.n_groups * p.corr_tpg : 0;
  p.off_cp = off;  // the two fp32 partial tiles of every kept tile
  off = align256(off + size_t(2) * B * p.corr_tiles * PP_T * PP_T * 4);
  p.total = off;
  return p;
}

template <typename TOut, bool FAST>
hipError_t run(const ScanArgs& a, const Plan& p, PhaseClock* clk) {
  char* ws = static_cast<char*>(a.ws);
  uint16_t* Zt = reinterpret_cast<uint16_t*>(ws + p.off_zt);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(ws + p.off_vt);
  uint16_t* Wbf = reinterpret_cast<uint16_t*>(ws + p.off_wbf);
  uint16_t* S = p.k > 1 ? reinterpret_cast<uint16_t*>(ws + p.off_s) : nullptr;
  unsigned* flags = reinterpret_cast<unsigned*>(ws + p.off_flags);
  const uint16_t* Z = static_cast<const uint16_t*>(a.Z);
  const uint16_t* V = static_cast<const uint16_t*>(a.V);
  const long DF = long(a.D) * a.F;
  const long ts = a.T_stride > 0 ? a.T_stride : a.T;  // tokens between sequences
  const long z_b = ts * a.F, v_b = ts * a.D;
  const long zt_b = long(a.F) * p.Tp, vt_b = long(a.D) * p.Tp;
  const long w0_b = a.w0_shared ? 0 : DF;
  const long wbf_b = long(p.n_groups) * DF;
  const long s_g = long(p.G) * p.Gp, s_b = long(p.n_groups) * s_g;

  // With eta = 0 the state never moves: every group applies bf16(W_0), there is no correction
  // and W_final is W_0 bit for bit. Otherwise the chain runs whenever its snapshots or its final
  // state are needed.
  const bool moving = a.eta != 0.f;
  const bool chain = moving && (p.n_groups > 1 || a.W_final != nullptr);
  const bool corr = moving && p.k > 1;
  if (!corr) S = nullptr;

  // 0: token-major operand copies and bf16(W_0)
  if (clk) clk->open(0);
  // the unmasked update writes bf16(W_0) itself (its first workgroups hold W_0 at the start)
  bool any_reset = false;
  if (a.resets)
    for (uint32_t w : a.resets->bits) any_reset = any_reset || w != 0u;
  const bool own_w0 = FAST && chain;
  // reset bits: their token unit, and whether any start falls inside a group
  const int U = reset_unit(p.G);
  bool inside = false;
  if (any_reset) {
    const int n_units = (a.T + U - 1) / U;
    for (int b = 0; b < a.B && !inside; ++b)
      for (int u = 0; u < n_units && !inside; ++u) {
        const int bit = b * n_units + u;
        inside = ((a.resets->bits[bit >> 5] >> (bit & 31)) & 1u) && (u * U) % p.G != 0;
      }
  }
  int n0 = 0;
  if (chain && !FAST) {  // the unmasked update reads Z in place
    hipLaunchKernelGGL(k_stage<FAST>, dim3(p.Tp / 64, (a.F + 63) / 64, a.B), dim3(256), 0,
                       a.stream, Z, Zt, a.T, p.Tp, a.F, z_b, zt_b, flags, 0);
    ++n0;
  }
  if (chain || corr) {
    hipLaunchKernelGGL(k_stage<FAST>, dim3(p.Tp / 64, (a.D + 63) / 64, a.B), dim3(256), 0,
                       a.stream, V, Vt, a.T, p.Tp, a.D, v_b, vt_b, flags, own_w0 ? p.nflags : 0);
    ++n0;
  }
  if (!own_w0) {
    hipLaunchKernelGGL(k_to_bf16<FAST>, dim3(1024, a.B), dim3(256), 0, a.stream, a.W0, w0_b, Wbf,
                       wbf_b, a.D, a.F, flags, p.nflags);
    ++n0;
  }
  if (clk) clk->close(n0);

  // 1: intra-group correction blocks
  if (corr) {
    if (clk) clk->open(1);
    if (FAST && p.corr_tiles > 0) {
      float* part = reinterpret_cast<float*>(ws + p.off_cp);
      const long part_half = long(a.B) * p.corr_tiles * PP_T * PP_T;
      hipLaunchKernelGGL(k_corr_pp, dim3(p.corr_tiles * 2, a.B), dim3(512), 0, a.stream, Z, z_b,
                         part, part_half, a.T, a.F, a.C, p.G, p.corr_tpg, p.corr_sub,
                         p.corr_tiles, (a.F / PP_BK) / 2);
      hipLaunchKernelGGL(k_corr_finish, dim3(p.corr_tiles * (PP_T * PP_T / 8 / 256), a.B),
                         dim3(256), 0, a.stream, part, part_half, S, s_b, s_g, p.Gp, a.T, a.C,
                         p.G, p.corr_tpg, p.corr_sub, p.corr_tiles, a.eta);
      if (clk) clk->close(2);
    } else {
      hipLaunchKernelGGL(k_corr<FAST>, dim3(p.n_groups * p.ntt_corr * p.nst, a.B), dim3(NTHR),
                         0, a.stream, Z, z_b, S, s_b, s_g, p.Gp, a.T, a.F, a.C, p.G, p.ntt_corr,
                         p.nst, a.eta);
      if (clk) clk->close(1);
    }
  }

  // 2: the state chain, one launch (eta = 0: W_final = W_0)
  if (chain) {
    if (clk) clk->open(2);
    if constexpr (FAST) {
      const int n_ut = p.utiles_m * p.utiles_n;
      hipLaunchKernelGGL(any_reset ? k_update_pp<true> : k_update_pp<false>,
                         dim3(n_ut * (p.split_steps > 0 ? 2 : 1), a.B), dim3(512), 0, a.stream, Z, Vt, z_b, vt_b, a.W0, w0_b, a.W_final, Wbf, wbf_b,
                         reinterpret_cast<uint16_t*>(ws + p.off_sink),
                         reinterpret_cast<float*>(ws + p.off_mid), flags, flags + p.nflags - 1,
                         a.D, a.F, a.T, p.G, a.eta, p.utiles_n, n_ut, p.split_steps,
                         p.spin_limit, (a.T + U - 1) / U, U / PP_BK, inside ? 1 : 0,
                         a.resets ? *a.resets : ResetMask{});
    } else {
      hipLaunchKernelGGL((k_update_chain<false>), dim3(p.tiles_m * p.tiles_n, a.B), dim3(NTHR),
                         0, a.stream, Zt, Vt, long(p.Tp), zt_b, vt_b, a.W0, w0_b, a.W_final, Wbf,
                         wbf_b, a.D, a.F, a.T, p.G, p.n_groups, a.eta, p.tiles_n);
    }
    if (clk) clk->close(1);
  } else if (!moving && a.W_final && a.W_final != a.W0) {
    if (clk) clk->open(2);
    for (int b = 0; b < a.B; ++b) {
      const hipError_t e =
          hipMemcpyAsync(a.W_final + b * DF, a.W0 + b * w0_b, size_t(DF) * sizeof(float),
                         hipMemcpyDeviceToDevice, a.stream);
      if (e != hipSuccess) return e;
    }
    if (clk) clk->close(a.B);
  }

  // 3: apply for every group (eta = 0: every group reads snapshot 0)
  if (clk) clk->open(3);
  if (FAST && a.F % PP_BK == 0 && a.C % PP_BK == 0) {
    hipLaunchKernelGGL((any_reset ? k_apply_pp<TOut, true> : k_apply_pp<TOut, false>),
                       dim3(p.n_groups * p.ntt_app * p.ntd, a.B), dim3(512), 0, a.stream, Z, z_b,
                       Wbf, moving ? DF : 0L, wbf_b, S, s_b, s_g, p.Gp, Vt, vt_b,
                       static_cast<TOut*>(a.O), v_b, a.T, a.F, a.D, a.C, p.G, p.ntt_app, p.ntd,
                       U, (a.T + U - 1) / U, a.resets ? *a.resets : ResetMask{});
  } else
  hipLaunchKernelGGL((k_apply<TOut, FAST>), dim3(p.n_groups * p.ntt_app * p.ntd, a.B),
                     dim3(NTHR), 0, a.stream, Z, z_b, Wbf, moving ? DF : 0L, wbf_b, S, s_b, s_g,
                     p.Gp, Vt, long(p.Tp), vt_b, static_cast<TOut*>(a.O), v_b, a.T, a.F, a.D,
                     a.C, p.G, p.ntt_app, p.ntd);
  if (clk) clk->close(1);
  return hipGetLastError();
}

// The unmasked kernels need every K step to lie inside valid or zero-padded data: groups and
// d_ff must be whole K steps (Zt/Vt are zero-padded to a whole step past T).
bool fast_shapes(const Plan& p, int F) { return p.G % BK == 0 && F % BK == 0; }

template <typename TOut>
hipError_t run_any(const ScanArgs& a, PhaseClock* clk) {
  const Plan p = make_plan(a.B, a.T, a.F, a.D, a.C);
  return fast_shapes(p, a.F) ? run<TOut, true>(a, p, clk) : run<TOut, false>(a, p, clk);
}

}  // namespace

size_t scan_mfma_workspace(int B, int T, int F, int D, int C) {
  return make_plan(B, T, F, D, C).total;
}

namespace {
__global__ void k_copy_word(const unsigned* __restrict__ src, unsigned* __restrict__ dst) {
  if (threadIdx.x == 0) dst[0] = src ? src[0] : 0u;
}
}  // namespace

hipError_t scan_mfma_copy_word(const void* src, unsigned* dst, hipStream_t stream) {
  hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(64), 0, stream,
                     static_cast<const unsigned*>(src), dst);
  return hipGetLastError();
}

void scan_mfma_test_overrides(int group_tokens, int split, int spin_limit) {
  g_group_tokens.store(group_tokens > 0 ? group_tokens : 0, std::memory_order_relaxed);
  g_split.store(split == 0 ? 0 : -1, std::memory_order_relaxed);
  g_spin_limit.store(spin_limit >= 0 ? spin_limit : -1, std::memory_order_relaxed);
}

size_t scan_mfma_timeout_word(int B, int T, int F, int D, int C) {
  const Plan p = make_plan(B, T, F, D, C);
  return p.off_flags + size_t(p.nflags - 1) * 4;
}

int scan_mfma_group(int B, int T, int F, int D, int C) { return make_plan(B, T, F, D, C).G; }

int scan_mfma_reset_group(int B, int T, int F, int D, int C, bool* inside, int* tile,
                          int* unit) {
  const Plan p = make_plan(B, T, F, D, C);
  const int U = reset_unit(p.G);
  const bool ok = fast_shapes(p, F) && long(B) * ((T + U - 1) / U) <= kResetBits;
  // starts inside a group need the eight-wave apply (and its whole-tile token ranges)
  *inside = ok && F % PP_BK == 0 && C % PP_BK == 0;
  *tile = PP_T;
  *unit = U;
  return ok ? p.G : 0;
}

hipError_t scan_mfma(const ScanArgs& a, PhaseClock* clk) {
  return a.out_bf16 ? run_any<uint16_t>(a, clk) : run_any<float>(a, clk);
}

}  // namespace ttt
