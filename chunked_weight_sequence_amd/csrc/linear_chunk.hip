// TTT-Linear, mini-batch gradient descent, run in chunks of several mini-batches (TTT layers page,
// ai-jitan-hub, on arXiv 2407.04620: the hidden state is a linear model and each mini-batch of b
// tokens takes one gradient step of the reconstruction loss). Per mini-batch m, at the
// start-of-mini-batch state W and with beta = eta / b:
//     R_m = K_m W - V_m;  O_m = Q_m W - beta tril(Q_m K_m^T) R_m;  W <- W - beta K_m^T R_m.
//
// The step is linear in W, so a chunk of L = 64 tokens (64 / b mini-batches) needs only the state
// at its first token. With W that state and U the chunk's residuals (row t of U = k_t W_j - v_t,
// W_j the start state of t's mini-batch j):
//     U_j = (K_j W - V_j) - beta sum_{l<j} (K_j K_l^T) U_l     forward substitution over blocks
//     O   = Q W - beta tril(Q K^T) U                          mask s <= t over the whole chunk
//     W  <- W - beta K^T U;   loss_t = ||u_t||^2
// which follows from W_j = W - beta sum_{l<j} K_l^T U_l. The substitution runs over 16-token
// blocks; the blocks of one mini-batch do not feed each other (b = 64: U = K W - V). Per chunk the
// state goes through one product with K, three short 16 x 16 substitution steps and one product
// with K^T, where the mini-batch loop takes two dependent products per mini-batch; the state's
// hi/lo split and update run once per chunk.
//
// One 512-thread workgroup per (sequence, head), two waves per SIMD that share a 16-column block
// of the state. Wave w < 4 runs the state's chain for columns [16w, 16w + 16): K W - V, the
// substitution and the update, the state held in its registers in the 16 x 16 matrix-core result
// layout. Wave w + 4 does the work off that chain: the chunk's 16 x 16 blocks K_j K_l^T (each
// output wave a share, for all four chain waves) before the chain needs them, and one chunk
// later the outputs and losses from the chunk-start state and U that the chain hands over as
// hi/lo bf16 operands (the blocks of tril(K Q^T) again shared out). Each SIMD interleaves the two
// instruction streams. Two barriers per chunk: the first closes the previous chunk, the second
// publishes the blocks the chain's substitution reads. The chunk tiles (q, k, v: 64 token rows
// of 128 bytes each) are copied straight into LDS rings three chunks ahead by the chain waves.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "linear_tile.hpp"

namespace ttt {
namespace {

constexpr int LC_L = 64;             // tokens per chunk: four 16-token blocks
constexpr int LC_TILE = LC_L * 128;  // bytes per tensor per chunk
constexpr int LC_AHEAD = 3;          // chunks copied ahead
constexpr int LC_NQK = LC_AHEAD + 1;  // q/k: chunk c's tiles are read in iteration c only
constexpr int LC_VAHEAD = LC_AHEAD - 1;  // v tiles: copied one chunk later than q and k
constexpr int LC_NV = LC_VAHEAD + 1;      // v: read by the chain only

struct alignas(16) LcSmem {
  char qk[LC_NQK][2][LC_TILE];
  char v[LC_NV][LC_TILE];
  float4 xe[4][4][64];  // (Q W)^T of the chunk: [column block][token block][lane]
  uint4 xu[4][4][64];  // U: [column block][uh01, uh23, ul01, ul23][lane]
  uint2 nb[7][2][64];  // K_j K_l^T blocks as A operands: [block][hi, lo][lane]; 6: sink
  uint2 kq[2][11][64];  // masked K_s Q_t^T blocks as B operands, bf16: [chunk & 1][pair][lane]; 10: sink
  float lossp[4][LC_L];
};
static_assert(sizeof(LcSmem) <= 160 * 1024, "LDS");

// The blocks l of a chunk that feed block j (l < j, another mini-batch): l < lc_nfeed(j).
template <int NB>
__device__ constexpr int lc_nfeed(int j) {
  return (j / NB) * NB;
}
// index of block pair (j, l) among the feeding pairs, j-major
template <int NB>
__device__ constexpr int lc_nbi(int j, int l) {
  int n = 0;
  for (int jj = 0; jj < j; ++jj) n += lc_nfeed<NB>(jj);
  return n + l;
}
template <int NB>
__device__ constexpr int lc_nblocks() {
  return lc_nbi<NB>(4, 0);
}
// index of the output pair (s block sb <= t block tb), tb-major
__device__ constexpr int lc_kqi(int sb, int tb) { return tb * (tb + 1) / 2 + sb; }

// Every accumulator chain here uses one product shape: a 16 x 16 x 16 product accumulating onto a
// 16 x 16 x 32 result (or the reverse) gave wrong, run-to-run varying values when the two were
// scheduled back to back (the default instruction scheduler placed them so; the same chains were
// right under another schedule). K = 16 terms accumulate in their own registers and are added
// with VALU operations.

// Rows 4g + i (i < 4) of two 16 x 16 result blocks X (rows 0..15) and Y (rows 16..31), packed
// bf16 in lane (g, n), regrouped so that lane (g, n) holds rows 8g .. 8g + 7 of the pair in order:
// the permlane32 swap trades rows 2, 3 of X with rows 0, 1 of Y, the permlane16 swap then odd rows
// of X with even rows of Y.
__device__ __forceinline__ uint4 rows8(const uint2& x, const uint2& y) {
  const auto ax = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
  const auto ay = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
  const auto bx = __builtin_amdgcn_permlane16_swap(ax[0], ax[1], false, false);
  const auto by = __builtin_amdgcn_permlane16_swap(ay[0], ay[1], false, false);
  return make_uint4(bx[0], by[0], bx[1], by[1]);
}

// x ? a : b on native vectors (a select of the vector structs went through scratch memory)
__device__ __forceinline__ uint4 sel4(bool x, const uint4& a, const uint4& b) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 va = __builtin_bit_cast(u32x4, a), vb = __builtin_bit_cast(u32x4, b);
  const unsigned m = x ? ~0u : 0u;
  return __builtin_bit_cast(uint4, (va & m) | (vb & ~m));
}

__device__ __forceinline__ void lc_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The same barrier without draining this wave's LDS operations first: for a wave whose LDS
// writes before it are read only after a later barrier (which drains them), and whose reads
// before it touch nothing that is written after it.
__device__ __forceinline__ void lc_barrier_nodrain() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// A operand block (j, l) of the substitution: lane (g, n) holds k_{16l + 4g + i} . k_{16j + n}
__device__ __forceinline__ f32x4 lc_gram(const char* tk, int j, int l, int g, int cl) {
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    x = mfma16x16x32(t_rd16(tk, 16 * l + cl, 32 * hh + 8 * g),
                     t_rd16(tk, 16 * j + cl, 32 * hh + 8 * g), x);
  return x;
}

template <int NB, typename TOut, bool LOSS>
__global__ __launch_bounds__(512, 1) void k_linear_chunk(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V,
                                                         const float* W0, TOut* __restrict__ O,
                                                         float* Wf, float* loss, int T, int H,
                                                         float eta) {
  __shared__ LcSmem sm;
  constexpr int NBLK = lc_nblocks<NB>();

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wave < 4;
  const int wq = wave & 3;  // the state's column block [16 wq, 16 wq + 16)
  const int g = lane >> 4, cl = lane & 15;
  const long rs = long(H) * DH;                  // elements between tokens
  const long base = (long(b) * T * H + h) * DH;  // token 0 of (b, h)
  const float beta = eta / float(16 * NB);
  const int nch = T / LC_L;
  const uint32_t qk0 = __builtin_amdgcn_readfirstlane(lds_u32(&sm.qk[0][0][0]));
  const uint32_t v0 = __builtin_amdgcn_readfirstlane(lds_u32(&sm.v[0][0]));

  // copies, by the chain waves (the output waves' stores then never delay a copy's wait): wave w
  // brings token rows 16w .. 16w + 15 of each tensor, 8 rows per instruction; lane l brings chunk
  // (l % 8) ^ (row % 8) of row 16w + 8p + l / 8 into slot l % 8
  uint32_t voff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    voff[p] = uint32_t(long(16 * wq + 8 * p + (lane >> 3)) * rs * 2 +
                       (((lane & 7) ^ (lane >> 3)) << 4));
  auto issue_qk = [&](int c) {  // 4 copy instructions
    const long tok = (base + long(c) * LC_L * rs) * 2;
    const uint32_t dq = qk0 + uint32_t((c % LC_NQK) * 2 * LC_TILE + wq * 2048);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      dma16(voff[p], reinterpret_cast<const char*>(Q) + tok, dq + uint32_t(p * 1024));
      dma16(voff[p], reinterpret_cast<const char*>(K) + tok, dq + uint32_t(LC_TILE + p * 1024));
    }
  };
  auto issue_v = [&](int c) {  // 2 copy instructions
    const long tok = (base + long(c) * LC_L * rs) * 2;
    const uint32_t dv = v0 + uint32_t((c % LC_NV) * LC_TILE + wq * 2048);
#pragma unroll
    for (int p = 0; p < 2; ++p)
      dma16(voff[p], reinterpret_cast<const char*>(V) + tok, dv + uint32_t(p * 1024));
  };
  // Copy order: q/k of chunks 0, 1, v of chunk 0, q/k of 2, v of 1, then during chunk c's work
  // q/k of c + 3 and v of c + 2. Chunk c's v tile is then its last copy, issued after its
  // q/k, and the copies issued after it are q/k of c + 2 and v of c + 1 (those that exist). The
  // waits count only this wave's copies.
  using WL = WaitList<6, 2, 0>;

  // bf16 identity and its negative as 16 x 16 x 16 operands: lane (g, n) holds rows 4g + i of
  // column n (B) or columns 4g + i of row n (A); both are [i == n - 4g]
  uint2 eye, neg_eye;
  {
    uint32_t e[4], n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = (4 * g + i == cl) ? 0x3F80u : 0u;  // bf16 1.0
      n[i] = (4 * g + i == cl) ? 0xBF80u : 0u;  // bf16 -1.0
    }
    eye = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
    neg_eye = make_uint2(n[0] | (n[1] << 16), n[2] | (n[3] << 16));
  }

  // output waves' shares: K_j K_l^T block slots (wq, wq + 4, ...); slots past the last block
  // are skipped (their entries here, block (1, 0) into the sink, are never used)
  constexpr int LC_NBS = (NBLK + 3) / 4;
  int nbj[LC_NBS > 0 ? LC_NBS : 1], nbl[LC_NBS > 0 ? LC_NBS : 1], nbs[LC_NBS > 0 ? LC_NBS : 1];
#pragma unroll
  for (int sl = 0; sl < LC_NBS; ++sl) {
    const int bi = wq + 4 * sl;
    nbj[sl] = 1;
    nbl[sl] = 0;
    nbs[sl] = bi < NBLK ? bi : 6;
#pragma unroll
    for (int j = 1; j < 4; ++j)
#pragma unroll
      for (int l = 0; l < lc_nfeed<NB>(j); ++l)
        if (lc_nbi<NB>(j, l) == bi) {
          nbj[sl] = j;
          nbl[sl] = l;
        }
  }
  // chain waves' shares of the masked blocks P[s][t] (s block sb <= t block tb), as (sb, tb):
  // slot 0 (wq, 3); slot 1 (wq, 2) for wq <= 2; slot 2 (wq, 1) for wq <= 1 and (0, 0) for wave
  // 2. Slots 0 and 1 take their Q operand from the fragments the wave already holds for Q W and
  // their K operand from one shared fragment; wave 3's slots 1 and 2 write the sink entry.
  const int kq_sb2 = wq == 2 ? 0 : wq, kq_tb2 = wq == 2 ? 0 : 1;
  const int kqp0 = lc_kqi(wq, 3), kqp1 = wq <= 2 ? lc_kqi(wq, 2) : 10,
            kqp2 = wq <= 2 ? lc_kqi(kq_sb2, kq_tb2) : 10;

  // chain waves: w[blk][i] = W[16*blk + 4*g + i][16 wq + cl]
  float w[4][4];
  {
    const float* w0 = (chain && W0) ? W0 + long(bh) * DH * DH : nullptr;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[blk][i] = w0 ? w0[(16 * blk + 4 * g + i) * DH + 16 * wq + cl] : 0.f;
  }

  if (chain) {
    if (nch > 0) issue_qk(0);
    if (nch > 1) issue_qk(1);
    if (nch > 0) issue_v(0);
    if (nch > 2) issue_qk(2);
    if (nch > 1) issue_v(1);
  }

  // iteration c: the chain takes chunk c; the output waves form chunk c's K_j K_l^T blocks and
  // chunk c - 1's outputs
  for (int c = 0; c <= nch; ++c) {
    if (chain) {
      if (c < nch) WL::wait((c + 2 < nch ? 4 : 0) + (c + 1 < nch ? 2 : 0));  // rows of chunk c
      lc_barrier();  // every wave's rows of chunk c are in; chunk c - 1 is closed
      if (c >= nch) {
        lc_barrier();
        continue;
      }
      const char* tk = &sm.qk[c % LC_NQK][1][0];
      const char* tv = &sm.v[c % LC_NV][0];

      // the chunk-start state as hi/lo operands, rows 32hh + 8g + 0..7: the lane's rows 4g + i of
      // blocks 2hh and 2hh + 1 regrouped by a permlane32 and a permlane16 swap per register (rows
      // 4g'.. of both blocks for g' = 2g mod 4 and 2g mod 4 + 1), so that the K and Q fragments
      // they meet are single 16-byte LDS reads (two 8-byte reads of rows r and r + 8 share banks)
      uint4 whi[2], wlo[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint2 h0, l0, h1, l1;
        split4(w[2 * hh], h0, l0);
        split4(w[2 * hh + 1], h1, l1);
        whi[hh] = rows8(h0, h1);
        wlo[hh] = rows8(l0, l1);
      }
      // Per 32-wide half hh of the head dimension, with the K and Q fragments of the half in
      // registers (lane: token row 16 blk + cl, elements 32 hh + 8g + 0..7; every product here
      // takes its contraction in this order):
      //   K_j W      (lane: row 16j + 4g + i, column 16 wq + cl), -V_j added after;
      //   the outputs' Q W part, E[c = 16 wq + 4g + i][t = 16tb + cl] from W^T Q^T, handed over
      //   in fp32 while the output waves form the K_j K_l^T blocks;
      //   this wave's share of the blocks P[s = 4g + i][t = cl] = k_s . q_t, masked to s <= t
      //   and kept in bf16 for the output waves one chunk later.
      const char* tq = &sm.qk[c % LC_NQK][0][0];
      f32x4 kw[4], e[4], pp[3];
#pragma unroll
      for (int k = 0; k < 4; ++k) kw[k] = e[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 3; ++sl) pp[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        auto frag = [&](const char* t, int blk) { return t_rd16(t, 16 * blk + cl, 32 * hh + 8 * g); };
        uint4 bq[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          bq[tb] = frag(tq, tb);
          e[tb] = mfma16x16x32(whi[hh], bq[tb], e[tb]);
          e[tb] = mfma16x16x32(wlo[hh], bq[tb], e[tb]);
        }
        uint4 a0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 a = frag(tk, j);
          if (j == 0) a0 = a;
          kw[j] = mfma16x16x32(a, whi[hh], kw[j]);
          kw[j] = mfma16x16x32(a, wlo[hh], kw[j]);
        }
        const uint4 ka = frag(tk, wq);
        const bool w2 = wq == 2;  // wave-uniform
        pp[0] = mfma16x16x32(ka, bq[3], pp[0]);
        pp[1] = mfma16x16x32(ka, bq[2], pp[1]);
        pp[2] = mfma16x16x32(sel4(w2, a0, ka), sel4(w2, bq[0], bq[1]), pp[2]);
      }
      // -V_j enters as (-I) V_j
      f32x4 u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 nv = mfma16x16x16(neg_eye, t_tr(tv, 16 * j + 4 * g, 16 * wq, cl),
                                      f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) u[j][i] = kw[j][i] + nv[i];
      }
      auto put_kq = [&](const f32x4& x, int sb, int tb, int slot) {
        float pm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[i] = (sb < tb || 4 * g + i <= cl) ? x[i] : 0.f;
        sm.kq[c & 1][slot][lane] = pack4bf(pm);
      };
      put_kq(pp[0], wq, 3, kqp0);
      put_kq(pp[1], wq, 2, kqp1);
      put_kq(pp[2], kq_sb2, kq_tb2, kqp2);
      // The output waves' K_j K_l^T blocks of chunk c are in, and their reads of chunk c - 1's
      // hand-off are done (they drain before this barrier). This wave's own masked-block
      // stores are read only in the next iteration, after the first barrier, and its reads so
      // far (chunk c's tiles) are of stages no copy below overwrites: no drain here.
      lc_barrier_nodrain();
      // q/k of chunk c + 3 and v of chunk c + 2 into the stages chunks c - 2 and c - 1 used (the
      // last reads of both were before the first barrier), issued here so that they go out while
      // the substitution waits for its blocks (issued at the start of the chunk's work, the copies
      // held up the products behind them; at its end, 1-3% slower than here)
      if (c + LC_AHEAD < nch) issue_qk(c + LC_AHEAD);
      if (c + LC_VAHEAD < nch) issue_v(c + LC_VAHEAD);
      // K^T operands of the update, read ahead of the substitution that hides their latency
      uint4 kta[4][2];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          kta[blk][p] = cat(t_tr(tk, 32 * p + 4 * g, 16 * blk, cl),
                            t_tr(tk, 32 * p + 16 + 4 * g, 16 * blk, cl));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        sm.xe[wq][tb][lane] = make_float4(e[tb][0], e[tb][1], e[tb][2], e[tb][3]);

      // forward substitution: U_j -= beta sum_l (K_j K_l^T) U_l over the blocks l that feed j,
      // two blocks per product where they come in pairs
      uint2 uh[4], ul[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nf = lc_nfeed<NB>(j);
        if (nf > 0) {
          f32x4 s = {0.f, 0.f, 0.f, 0.f}, s16 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int l = 0; l < nf; l += 2) {
            const int b0 = lc_nbi<NB>(j, l);
            if (l + 1 < nf) {
              const uint4 nh = cat(sm.nb[b0][0][lane], sm.nb[b0 + 1][0][lane]);
              const uint4 nl = cat(sm.nb[b0][1][lane], sm.nb[b0 + 1][1][lane]);
              const uint4 bh = cat(uh[l], uh[l + 1]), bl = cat(ul[l], ul[l + 1]);
              s = mfma16x16x32(nh, bh, s);
              s = mfma16x16x32(nh, bl, s);
              s = mfma16x16x32(nl, bh, s);
            } else {
              const uint2 nh = sm.nb[b0][0][lane], nl = sm.nb[b0][1][lane];
              s16 = mfma16x16x16(nh, uh[l], s16);
              s16 = mfma16x16x16(nh, ul[l], s16);
              s16 = mfma16x16x16(nl, uh[l], s16);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) u[j][i] -= beta * (s[i] + s16[i]);
        }
        const float uf[4] = {u[j][0], u[j][1], u[j][2], u[j][3]};
        split4(uf, uh[j], ul[j]);
      }
      sm.xu[wq][0][lane] = cat(uh[0], uh[1]);
      sm.xu[wq][1][lane] = cat(uh[2], uh[3]);
      sm.xu[wq][2][lane] = cat(ul[0], ul[1]);
      sm.xu[wq][3][lane] = cat(ul[2], ul[3]);

      // W -= beta K^T U   (result lane: dW[16blk + 4g + i][col]); the contraction runs over the
      // token pairs (32p + 4g + e, 32p + 16 + 4g + e), the lane's own U values
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint4 a = kta[blk][p];
          dw = mfma16x16x32(a, cat(uh[2 * p], uh[2 * p + 1]), dw);
          dw = mfma16x16x32(a, cat(ul[2 * p], ul[2 * p + 1]), dw);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) w[blk][i] -= beta * dw[i];
      }
    } else {
      lc_barrier();
      // The work before the second barrier reads only what the first one closed: the chain's
      // hand-off of chunk cc = c - 1 and the tiles of chunks cc and c. It is straight-line code
      // (the first iteration computes on stale data and discards it) so that its independent
      // products overlap.
      const int cc = c - 1;  // the chunk whose outputs this iteration forms
      float4 xe4[4];
      uint4 xu4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xe4[k] = sm.xe[wq][k][lane];
        xu4[k] = sm.xu[wq][k][lane];
      }
      if (LOSS && cc >= 1 && lane < 16) {
        // chunk cc - 1: output wave wq writes the losses of its tokens 16 wq .. 16 wq + 15
        const int t = 16 * wq + lane;
        loss[(long(b) * T + long(cc - 1) * LC_L + t) * H + h] =
            ((sm.lossp[0][t] + sm.lossp[1][t]) + sm.lossp[2][t]) + sm.lossp[3][t];
      }
      const uint2 uh[4] = {make_uint2(xu4[0].x, xu4[0].y), make_uint2(xu4[0].z, xu4[0].w),
                           make_uint2(xu4[1].x, xu4[1].y), make_uint2(xu4[1].z, xu4[1].w)};
      const uint2 ul[4] = {make_uint2(xu4[2].x, xu4[2].y), make_uint2(xu4[2].z, xu4[2].w),
                           make_uint2(xu4[3].x, xu4[3].y), make_uint2(xu4[3].z, xu4[3].w)};

      // this wave's share of chunk c's K_j K_l^T blocks, split into hi/lo A operands (slots past
      // the last block are skipped)
      {
        const char* tk = &sm.qk[c % LC_NQK][1][0];
#pragma unroll
        for (int sl = 0; sl < LC_NBS; ++sl) {
          if (wq + 4 * sl >= NBLK) continue;  // wave-uniform: no block in this slot
          const f32x4 x = lc_gram(tk, nbj[sl], nbl[sl], g, cl);
          const float xf[4] = {x[0], x[1], x[2], x[3]};
          uint2 nh, nl;
          split4(xf, nh, nl);
          sm.nb[nbs[sl]][0][lane] = nh;
          sm.nb[nbs[sl]][1][lane] = nl;
        }
      }
      // per-token partial losses over this block's 16 columns. U_j^T times the identity turns
      // the lane's four tokens of one column into one token's four columns (hi + lo summed in
      // fp32): lane (g, n) then holds u[16j + n][16 wq + 4g + i]. The four-column sums are
      // added over the four 16-lane rows by row swaps, which also leave row g with block g.
      float lsum = 0.f;
      if constexpr (LOSS) {
        float sj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 r = mfma16x16x32(cat(uh[j], ul[j]), cat(eye, eye),
                                       f32x4{0.f, 0.f, 0.f, 0.f});
          sj[j] = fmaf(r[3], r[3], fmaf(r[2], r[2], fmaf(r[1], r[1], r[0] * r[0])));
        }
        const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sj[0]),
                                                          __float_as_uint(sj[2]), false, false);
        const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sj[1]),
                                                          __float_as_uint(sj[3]), false, false);
        // rows 0, 1: block 0 (resp. 1) summed over the row pairs (0, 2) and (1, 3); rows 2, 3:
        // block 2 (resp. 3)
        const float t02 = __uint_as_float(a02[0]) + __uint_as_float(a02[1]);
        const float t13 = __uint_as_float(a13[0]) + __uint_as_float(a13[1]);
        const auto bb = __builtin_amdgcn_permlane16_swap(__float_as_uint(t02),
                                                         __float_as_uint(t13), false, false);
        lsum = __uint_as_float(bb[0]) + __uint_as_float(bb[1]);
      }
      lc_barrier();  // chunk c's K_j K_l^T blocks are in
      if (cc < 0) continue;
      if constexpr (LOSS) sm.lossp[wq][16 * g + cl] = lsum;

      // O_t = (Q W)_t - beta sum_{s <= t} (q_t . k_s) u_s   (result lane: O[t = 16tb + cl]
      // [c = 16 wq + 4g + i], from U^T P, two s blocks per product where paired)
      TOut* orow = O + base + long(cc) * LC_L * rs;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f}, d16 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb <= tb; sb += 2) {
          if (sb + 1 <= tb) {
            const uint4 pb = cat(sm.kq[cc & 1][lc_kqi(sb, tb)][lane],
                                 sm.kq[cc & 1][lc_kqi(sb + 1, tb)][lane]);
            d = mfma16x16x32(cat(uh[sb], uh[sb + 1]), pb, d);
            d = mfma16x16x32(cat(ul[sb], ul[sb + 1]), pb, d);
          } else {
            const uint2 pb = sm.kq[cc & 1][lc_kqi(sb, tb)][lane];
            d16 = mfma16x16x16(uh[sb], pb, d16);
            d16 = mfma16x16x16(ul[sb], pb, d16);
          }
        }
        float o[4];
        const float ef[4] = {xe4[tb].x, xe4[tb].y, xe4[tb].z, xe4[tb].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = ef[i] - beta * (d[i] + d16[i]);
        TOut* dst = orow + long(16 * tb + cl) * rs + 16 * wq + 4 * g;
        if constexpr (sizeof(TOut) == 2)
          *reinterpret_cast<uint2*>(dst) = pack4bf(o);
        else
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }

  if (LOSS && nch > 0) {
    lc_barrier();
    if (!chain && lane < 16) {
      const int t = 16 * wq + lane;
      loss[(long(b) * T + long(nch - 1) * LC_L + t) * H + h] =
          ((sm.lossp[0][t] + sm.lossp[1][t]) + sm.lossp[2][t]) + sm.lossp[3][t];
    }
  }
  if (chain && Wf) {
    float* wf = Wf + long(bh) * DH * DH;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[(16 * blk + 4 * g + i) * DH + 16 * wq + cl] = w[blk][i];
  }
}

template <int NB, typename TOut>
void launch_chunk(const LinearArgs& a) {
  const auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(512), 0, a.stream,
                       static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                       static_cast<const uint16_t*>(a.V), a.W0, static_cast<TOut*>(a.O),
                       a.W_final, a.loss, a.T, a.H, a.eta);
  };
  if (a.loss)
    args(k_linear_chunk<NB, TOut, true>);
  else
    args(k_linear_chunk<NB, TOut, false>);
}

template <typename TOut>
void launch_chunk_nb(const LinearArgs& a) {
  switch (a.b) {
    case 16: launch_chunk<1, TOut>(a); break;
    case 32: launch_chunk<2, TOut>(a); break;
    default: launch_chunk<4, TOut>(a); break;
  }
}

}  // namespace

bool linear_chunk_supported(const LinearArgs& a) {
  return a.in_bf16 && a.dh == DH && (a.b == 16 || a.b == 32 || a.b == 64) && a.T % LC_L == 0;
}

hipError_t linear_chunk(const LinearArgs& a) {
  if (a.out_bf16)
    launch_chunk_nb<uint16_t>(a);
  else
    launch_chunk_nb<float>(a);
  return hipGetLastError();
}

}  // namespace ttt
