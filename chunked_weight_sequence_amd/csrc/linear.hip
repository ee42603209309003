// TTT-Linear, mini-batch gradient descent (TTT layers page, ai-jitan-hub, on arXiv 2407.04620:
// the hidden state is a linear model whose update is one self-supervised gradient step; with
// mini-batch 1 and no LayerNorm/residual it is DeltaNet). Per mini-batch m of b tokens, with W
// the start-of-mini-batch state:
//     R = K_m W - V_m;  O_m = Q_m W - (eta/b) tril(Q_m K_m^T) R;  W -= (eta/b) K_m^T R.
//
// The kernels here run one mini-batch per step; they serve b = 48, b = 16 and 32 when T is not a
// multiple of 64, and the fp32 path. linear_chunk.hip runs the other bf16 cases in 64-token chunks.
//
// Matrix-core kernel (bf16 inputs, b = 16*NB): one 256-thread workgroup per (sequence, head);
// wave w owns columns [16w, 16w+16) of the 64x64 fp32 state, held in registers in the 16x16
// matrix-core result layout for the whole sequence. The columns of W evolve independently, so
// the four waves never exchange state; they share the staged Q/K/V tiles (double-buffered in
// LDS, next mini-batch prefetched during the current one) and sum their loss partials in LDS.
// Register-layout choices that avoid any shuffle of the state:
//   * products against W are formed as K W and W^T Q^T with the contraction index permuted so
//     that each lane's own state values are its operand (the K and Q operands are read from LDS
//     in the matching order);
//   * R, tril(K Q^T) and the output correction come out of one product in the layout the next
//     product consumes (R^T's operand layout equals R's result layout);
//   * the state enters each product as a two-term bf16 split (hi + lo), as does R in the
//     update, so the fp32 state keeps ~16-bit operand precision.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "linear_tile.hpp"

namespace ttt {
namespace {

// Staging of one mini-batch: BS rows of 64 bf16 for each of q, k, v, moved as 16-byte chunks
// (chunk c of a tensor = row c / 8, columns 8 * (c % 8) .. +8).
template <int BS>
struct Stage {
  static constexpr int PER = BS * 8;
  static constexpr int NR = (PER + 255) / 256;
  uint4 q[NR], k[NR], v[NR];
};

template <int BS>
__device__ __forceinline__ void stage_load(Stage<BS>& st, const uint16_t* Q, const uint16_t* K,
                                           const uint16_t* V, long base, long rs, int mb,
                                           int tid) {
#pragma unroll
  for (int r = 0; r < Stage<BS>::NR; ++r) {
    const int c = tid + 256 * r;
    if (c < Stage<BS>::PER) {
      const long off = base + long(mb * BS + (c >> 3)) * rs + (c & 7) * 8;
      st.q[r] = *reinterpret_cast<const uint4*>(Q + off);
      st.k[r] = *reinterpret_cast<const uint4*>(K + off);
      st.v[r] = *reinterpret_cast<const uint4*>(V + off);
    }
  }
}

// Row-major copies of q, k, v and a transposed copy of k (kt[d][s]) for the state update.
template <int BS, int RP, int TP>
__device__ __forceinline__ void stage_store(const Stage<BS>& st, uint16_t* qs, uint16_t* ks,
                                            uint16_t* vs, uint16_t* kts, int tid) {
#pragma unroll
  for (int r = 0; r < Stage<BS>::NR; ++r) {
    const int c = tid + 256 * r;
    if (c < Stage<BS>::PER) {
      const int row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(qs + row * RP + kc * 8) = st.q[r];
      *reinterpret_cast<uint4*>(ks + row * RP + kc * 8) = st.k[r];
      *reinterpret_cast<uint4*>(vs + row * RP + kc * 8) = st.v[r];
      const uint32_t wd[4] = {st.k[r].x, st.k[r].y, st.k[r].z, st.k[r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kts[(kc * 8 + 2 * q) * TP + row] = uint16_t(wd[q] & 0xFFFFu);
        kts[(kc * 8 + 2 * q + 1) * TP + row] = uint16_t(wd[q] >> 16);
      }
    }
  }
}

template <int NB, typename TOut>
__global__ __launch_bounds__(256, 1) void k_linear_mfma(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const float* W0,
                                                        TOut* __restrict__ O, float* Wf,
                                                        float* loss, int T, int H, float eta) {
  constexpr int BS = 16 * NB;
  constexpr int RP = DH + 8;                   // padded row pitch (bf16 elements)
  constexpr int TP = BS + 8;                   // pitch of the transposed k tile
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][BS * RP], ks[2][BS * RP], vs[2][BS * RP];
  __shared__ __attribute__((aligned(16))) uint16_t kts[2][DH * TP];
  __shared__ float lossp[2][4][BS];

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int tid = threadIdx.x, slab = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, cl = lane & 15;
  const long rs = long(H) * DH;                           // elements between tokens
  const long base = (long(b) * T * H + h) * DH;           // token 0 of (b, h)
  const int col = 16 * slab + cl;                         // state column owned by this lane
  const float lr = eta / float(BS);
  const int nmb = T / BS;

  // state: w[blk][i] = W[16*blk + 4*g + i][col]
  float w[4][4];
  {
    const float* w0 = W0 ? W0 + long(bh) * DH * DH : nullptr;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[blk][i] = w0 ? w0[(16 * blk + 4 * g + i) * DH + col] : 0.f;
  }

  Stage<BS> st;
  stage_load(st, Q, K, V, base, rs, 0, tid);
  stage_store<BS, RP, TP>(st, qs[0], ks[0], vs[0], kts[0], tid);
  __syncthreads();

  for (int mb = 0; mb < nmb; ++mb) {
    const int cur = mb & 1;
    if (mb + 1 < nmb) stage_load(st, Q, K, V, base, rs, mb + 1, tid);
    const uint16_t* q_ = qs[cur];
    const uint16_t* k_ = ks[cur];
    const uint16_t* v_ = vs[cur];
    const uint16_t* kt_ = kts[cur];

    // state operands: for half hh, slots 0..3 <-> rows 32hh+4g+i, slots 4..7 <-> 32hh+16+4g+i
    uint4 whi[2], wlo[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint2 h0, l0, h1, l1;
      split4(w[2 * hh], h0, l0);
      split4(w[2 * hh + 1], h1, l1);
      whi[hh] = cat(h0, h1);
      wlo[hh] = cat(l0, l1);
    }

    float racc[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // R_j = K_j W - V_j   (result lane: R[s = 4g+i][c = col])
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = k_ + (16 * j + cl) * RP;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint2 a0 = *reinterpret_cast<const uint2*>(krow + 32 * hh + 4 * g);
        const uint2 a1 = *reinterpret_cast<const uint2*>(krow + 32 * hh + 16 + 4 * g);
        const uint4 a = cat(a0, a1);
        r = mfma16x16x32(a, whi[hh], r);
        r = mfma16x16x32(a, wlo[hh], r);
      }
      float lp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        racc[j][i] = r[i] - bf2f(v_[(16 * j + 4 * g + i) * RP + col]);
        lp[i] = racc[j][i] * racc[j][i];
      }
      if (loss) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = lp[i];
          s += __shfl_xor(s, 1);
          s += __shfl_xor(s, 2);
          s += __shfl_xor(s, 4);
          s += __shfl_xor(s, 8);
          if (cl == 0) lossp[cur][slab][16 * j + 4 * g + i] = s;
        }
      }
    }

#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // E_j = W^T Q_j^T   (result lane: E[c = 4g+i][t = 16j+cl])
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* qrow = q_ + (16 * j + cl) * RP;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint2 b0 = *reinterpret_cast<const uint2*>(qrow + 32 * hh + 4 * g);
        const uint2 b1 = *reinterpret_cast<const uint2*>(qrow + 32 * hh + 16 + 4 * g);
        const uint4 bq = cat(b0, b1);
        e = mfma16x16x32(whi[hh], bq, e);
        e = mfma16x16x32(wlo[hh], bq, e);
      }
      // D_j = sum_{j' <= j} R_j'^T tril(K_j' Q_j^T)   (result lane: D[c = 4g+i][t = cl])
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp <= j; ++jp) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint4 a = *reinterpret_cast<const uint4*>(k_ + (16 * jp + cl) * RP + 32 * hh + 8 * g);
          const uint4 bq = *reinterpret_cast<const uint4*>(qrow + 32 * hh + 8 * g);
          p = mfma16x16x32(a, bq, p);   // P[s = 4g+i][t = cl] = k_s . q_t
        }
        float pm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[i] = (jp < j || 4 * g + i <= cl) ? p[i] : 0.f;
        uint2 rhi, rlo;
        split4(racc[jp], rhi, rlo);
        const uint2 pb = pack4bf(pm);
        d = mfma16x16x16(rhi, pb, d);
        d = mfma16x16x16(rlo, pb, d);
      }
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = e[i] - lr * d[i];
      TOut* dst = O + base + long(mb * BS + 16 * j + cl) * rs + 16 * slab + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) st_elem(dst, i, o[i]);
    }

    // W -= (eta/b) sum_j K_j^T R_j   (result lane: dW[16blk + 4g + i][col])
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint2 a = *reinterpret_cast<const uint2*>(kt_ + (16 * blk + cl) * TP + 16 * j + 4 * g);
        uint2 rhi, rlo;
        split4(racc[j], rhi, rlo);
        dw = mfma16x16x16(a, rhi, dw);
        dw = mfma16x16x16(a, rlo, dw);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) w[blk][i] -= lr * dw[i];
    }

    if (mb + 1 < nmb)
      stage_store<BS, RP, TP>(st, qs[cur ^ 1], ks[cur ^ 1], vs[cur ^ 1], kts[cur ^ 1], tid);
    __syncthreads();
    if (loss && tid < BS) {
      const float s = ((lossp[cur][0][tid] + lossp[cur][1][tid]) + lossp[cur][2][tid]) +
                      lossp[cur][3][tid];
      loss[(long(b) * T + mb * BS + tid) * H + h] = s;
    }
  }

  if (Wf) {
    float* wf = Wf + long(bh) * DH * DH;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[(16 * blk + 4 * g + i) * DH + col] = w[blk][i];
  }
}

// Private-tile variant for b = 16 and 32 (bf16 inputs): the same per-wave arithmetic, but every
// wave copies the mini-batch tiles it reads straight into its own LDS ring, NS mini-batches
// ahead (direct global -> LDS copies), so the waves never wait for each other inside the loop.
// K^T for the state update and the V column block for the residual come from transposing LDS
// reads (ds_read_b64_tr_b16) of the token-major tiles. Per-token losses (sums over all 64
// columns) pass through a small LDS ring and are reduced every LSYNC mini-batches behind one
// barrier. Tile layout: token row r (128 bytes) keeps 16-byte chunk c at chunk c ^ (r % 8).
template <int NB>
struct LinDma {
  static constexpr int BS = 16 * NB;
  static constexpr int NS = NB == 1 ? 4 : 3;  // mini-batches in flight per wave
  static constexpr int TILE = BS * 128;       // bytes: BS tokens x 64 bf16
  static constexpr int STG = 3 * TILE;        // q, k, v
  static constexpr int IPT = TILE / 1024;     // copy instructions per tensor
  static constexpr int LSYNC = 8, LR = 2 * LSYNC;
};

template <int NB, typename TOut>
__global__ __launch_bounds__(256, 1) void k_linear_dma(const uint16_t* __restrict__ Q,
                                                       const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       const float* W0, TOut* __restrict__ O,
                                                       float* Wf, float* loss, int T, int H,
                                                       float eta) {
  using P = LinDma<NB>;
  constexpr int BS = P::BS, NS = P::NS, TILE = P::TILE, STG = P::STG, IPT = P::IPT;
  __shared__ __attribute__((aligned(16))) char tiles[4][NS][STG];
  __shared__ float lossp[P::LR][4][BS];

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, cl = lane & 15;
  const long rs = long(H) * DH;                  // elements between tokens
  const long base = (long(b) * T * H + h) * DH;  // token 0 of (b, h)
  const int col = 16 * wave + cl;                // state column owned by this lane
  const float lr = eta / float(BS);
  const int nmb = T / BS;
  char* const my = &tiles[wave][0][0];
  const uint32_t my_lds = __builtin_amdgcn_readfirstlane(lds_u32(my));

  // copies: instruction p of a tensor fills token rows 8p .. 8p+7; lane l brings chunk
  // (l % 8) ^ (row % 8) of row 8p + l / 8 into slot l % 8
  uint32_t voff[IPT];
#pragma unroll
  for (int p = 0; p < IPT; ++p) {
    const int row = 8 * p + (lane >> 3);
    voff[p] = uint32_t(long(row) * rs * 2 + (((lane & 7) ^ (row & 7)) << 4));
  }
  auto issue = [&](int mb, int st) {
    const long tok = (base + long(mb) * BS * rs) * 2;
    const char* src[3] = {reinterpret_cast<const char*>(Q) + tok,
                          reinterpret_cast<const char*>(K) + tok,
                          reinterpret_cast<const char*>(V) + tok};
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int p = 0; p < IPT; ++p)
        dma16(voff[p], src[t], my_lds + uint32_t(st * STG + t * TILE + p * 1024));
  };
  // waits count only this wave's copies (any other memory operation only waits longer)
  using WL = WaitList<(NS - 1) * 3 * IPT, (NS - 2) * 3 * IPT, (NS > 3 ? NS - 3 : 0) * 3 * IPT, 0>;

  // state: w[blk][i] = W[16*blk + 4*g + i][col]
  float w[4][4];
  {
    const float* w0 = W0 ? W0 + long(bh) * DH * DH : nullptr;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[blk][i] = w0 ? w0[(16 * blk + 4 * g + i) * DH + col] : 0.f;
  }

#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nmb) issue(s, s);

  for (int mb = 0; mb < nmb; ++mb) {
    const int st = mb % NS;
    WL::wait(min(NS - 1, nmb - 1 - mb) * 3 * IPT);  // this mini-batch's tiles have landed
    const char* tq = my + st * STG;
    const char* tk = tq + TILE;
    const char* tv = tk + TILE;

    uint4 whi[2], wlo[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint2 h0, l0, h1, l1;
      split4(w[2 * hh], h0, l0);
      split4(w[2 * hh + 1], h1, l1);
      whi[hh] = cat(h0, h1);
      wlo[hh] = cat(l0, l1);
    }

    float racc[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // R_j = K_j W - V_j   (result lane: R[s = 4g+i][c = col])
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 a = cat(t_rd8(tk, 16 * j + cl, 32 * hh + 4 * g),
                            t_rd8(tk, 16 * j + cl, 32 * hh + 16 + 4 * g));
        r = mfma16x16x32(a, whi[hh], r);
        r = mfma16x16x32(a, wlo[hh], r);
      }
      const uint2 vv = t_tr(tv, 16 * j + 4 * g, 16 * wave, cl);  // V[16j + 4g + i][col]
      const float vf[4] = {bf2f(uint16_t(vv.x & 0xFFFFu)), bf2f(uint16_t(vv.x >> 16)),
                           bf2f(uint16_t(vv.y & 0xFFFFu)), bf2f(uint16_t(vv.y >> 16))};
#pragma unroll
      for (int i = 0; i < 4; ++i) racc[j][i] = r[i] - vf[i];
      if (loss) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sl = row16_sum(racc[j][i] * racc[j][i]);
          if (cl == 0) lossp[mb % P::LR][wave][16 * j + 4 * g + i] = sl;
        }
      }
    }

#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // E_j = W^T Q_j^T   (result lane: E[c = 4g+i][t = 16j+cl])
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 bq = cat(t_rd8(tq, 16 * j + cl, 32 * hh + 4 * g),
                             t_rd8(tq, 16 * j + cl, 32 * hh + 16 + 4 * g));
        e = mfma16x16x32(whi[hh], bq, e);
        e = mfma16x16x32(wlo[hh], bq, e);
      }
      // D_j = sum_{j' <= j} R_j'^T tril(K_j' Q_j^T)   (result lane: D[c = 4g+i][t = cl])
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp <= j; ++jp) {
        f32x4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)  // P[s = 4g+i][t = cl] = k_s . q_t
          pp = mfma16x16x32(t_rd16(tk, 16 * jp + cl, 32 * hh + 8 * g),
                            t_rd16(tq, 16 * j + cl, 32 * hh + 8 * g), pp);
        float pm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[i] = (jp < j || 4 * g + i <= cl) ? pp[i] : 0.f;
        uint2 rhi, rlo;
        split4(racc[jp], rhi, rlo);
        const uint2 pb = pack4bf(pm);
        d = mfma16x16x16(rhi, pb, d);
        d = mfma16x16x16(rlo, pb, d);
      }
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = e[i] - lr * d[i];
      TOut* dst = O + base + long(mb * BS + 16 * j + cl) * rs + 16 * wave + 4 * g;
      if constexpr (sizeof(TOut) == 2)
        *reinterpret_cast<uint2*>(dst) = pack4bf(o);
      else
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    }

    // W -= (eta/b) sum_j K_j^T R_j   (result lane: dW[16blk + 4g + i][col])
    uint2 rh[NB], rl[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) split4(racc[j], rh[j], rl[j]);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint2 a = t_tr(tk, 16 * j + 4 * g, 16 * blk, cl);  // K[16j + 4g + e][16blk + cl]
        dw = mfma16x16x16(a, rh[j], dw);
        dw = mfma16x16x16(a, rl[j], dw);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) w[blk][i] -= lr * dw[i];
    }

    // this stage's reads are done: refill it with mini-batch mb + NS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (mb + NS < nmb) issue(mb + NS, st);

    if (loss && (mb % P::LSYNC == P::LSYNC - 1 || mb == nmb - 1)) {
      __syncthreads();  // every wave's partials up to mb are in the ring
      const int first = mb - mb % P::LSYNC, cnt = (mb - first + 1) * BS;
      for (int k = tid; k < cnt; k += 256) {
        const int m2 = first + k / BS, t = k % BS, sl = m2 % P::LR;
        const float sum = ((lossp[sl][0][t] + lossp[sl][1][t]) + lossp[sl][2][t]) + lossp[sl][3][t];
        loss[(long(b) * T + m2 * BS + t) * H + h] = sum;
      }
    }
  }

  if (Wf) {
    float* wf = Wf + long(bh) * DH * DH;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[(16 * blk + 4 * g + i) * DH + col] = w[blk][i];
  }
}

// fp32 kernel, any mini-batch size: the same step accumulated token by token. Lane c owns
// column c of W and of the running within-mini-batch gradient P = sum_{s<=t} k_s^T r_s, so the
// output o_t = q_t (W - (eta/b) P) includes exactly the tokens s <= t of the mini-batch.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(64) void k_linear_simt(const TIn* __restrict__ Q,
                                                    const TIn* __restrict__ K,
                                                    const TIn* __restrict__ V,
                                                    const float* W0,
                                                    TOut* __restrict__ O, float* Wf, float* loss,
                                                    int T, int H, int bsz, float eta) {
  __shared__ float qs[16][DH], ks[16][DH];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, c = threadIdx.x;
  const long rs = long(H) * DH;
  const long base = (long(b) * T * H + h) * DH;
  float W[DH], P[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    W[d] = W0 ? W0[long(bh) * DH * DH + d * DH + c] : 0.f;
    P[d] = 0.f;
  }
  const float lr = eta / float(bsz);
  for (int t0 = 0; t0 < T; t0 += 16) {
    for (int e = 0; e < 16; ++e) {
      const int t = t0 + e;
      qs[e][c] = t < T ? ld_elem(Q, base + t * rs + c) : 0.f;
      ks[e][c] = t < T ? ld_elem(K, base + t * rs + c) : 0.f;
    }
    __syncthreads();
    for (int e = 0; e < 16 && t0 + e < T; ++e) {
      const int t = t0 + e;
      float r = -ld_elem(V, base + t * rs + c);
#pragma unroll
      for (int d = 0; d < DH; ++d) r = fmaf(ks[e][d], W[d], r);
      if (loss) {
        float s = r * r;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m);
        if (c == 0) loss[(long(b) * T + t) * H + h] = s;
      }
      float o = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        P[d] = fmaf(ks[e][d], r, P[d]);
        o = fmaf(qs[e][d], W[d] - lr * P[d], o);
      }
      st_elem(O, base + t * rs + c, o);
      if ((t + 1) % bsz == 0) {
#pragma unroll
        for (int d = 0; d < DH; ++d) {
          W[d] -= lr * P[d];
          P[d] = 0.f;
        }
      }
    }
    __syncthreads();
  }
  if (Wf) {
#pragma unroll
    for (int d = 0; d < DH; ++d) Wf[long(bh) * DH * DH + d * DH + c] = W[d];
  }
}

template <int NB, typename TOut>
void launch_mfma(const LinearArgs& a) {
  hipLaunchKernelGGL((k_linear_mfma<NB, TOut>), dim3(a.B * a.H), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), a.W0, static_cast<TOut*>(a.O), a.W_final,
                     a.loss, a.T, a.H, a.eta);
}

template <int NB, typename TOut>
void launch_dma(const LinearArgs& a) {
  hipLaunchKernelGGL((k_linear_dma<NB, TOut>), dim3(a.B * a.H), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), a.W0, static_cast<TOut*>(a.O), a.W_final,
                     a.loss, a.T, a.H, a.eta);
}

#ifndef TTT_LINEAR_B32_TU
template <typename TOut>
void launch_mfma_nb(const LinearArgs& a) {
  // b = 16 and 32 with T a multiple of 64, and every b = 64, run in chunks (linear_chunk.hip)
  switch (a.b / 16) {
    case 1: launch_dma<1, TOut>(a); break;
    case 2: linear_dma_b32(a); break;  // in its own translation unit (linear_b32.hip)
    default: launch_mfma<3, TOut>(a); break;
  }
}

template <typename TIn, typename TOut>
void launch_simt(const LinearArgs& a) {
  hipLaunchKernelGGL((k_linear_simt<TIn, TOut>), dim3(a.B * a.H), dim3(64), 0, a.stream,
                     static_cast<const TIn*>(a.Q), static_cast<const TIn*>(a.K),
                     static_cast<const TIn*>(a.V), a.W0, static_cast<TOut*>(a.O), a.W_final,
                     a.loss, a.T, a.H, a.b, a.eta);
}

#endif  // TTT_LINEAR_B32_TU

}  // namespace

#ifdef TTT_LINEAR_B32_TU
// b = 32 kernels, compiled with the default scheduler (the instruction-level-parallelism one
// that suits the other mini-batch sizes makes this one about 3% slower)
void linear_dma_b32(const LinearArgs& a) {
  if (a.out_bf16)
    launch_dma<2, uint16_t>(a);
  else
    launch_dma<2, float>(a);
}
#else
bool linear_mfma_supported(const LinearArgs& a) {
  return a.in_bf16 && a.dh == DH && a.b % 16 == 0 && a.b >= 16 && a.b <= 48;
}

hipError_t linear_mfma(const LinearArgs& a) {
  if (a.out_bf16)
    launch_mfma_nb<uint16_t>(a);
  else
    launch_mfma_nb<float>(a);
  return hipGetLastError();
}

hipError_t linear_simt(const LinearArgs& a) {
  if (a.in_bf16) {
    if (a.out_bf16) launch_simt<uint16_t, uint16_t>(a);
    else launch_simt<uint16_t, float>(a);
  } else {
    if (a.out_bf16) launch_simt<float, uint16_t>(a);
    else launch_simt<float, float>(a);
  }
  return hipGetLastError();
}
#endif  // TTT_LINEAR_B32_TU

}  // namespace ttt
