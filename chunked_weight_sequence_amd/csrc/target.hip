// LM-aligned target producer ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv
// 2604.06169: section 4, the target is a 1-D convolution of the token embeddings followed by a
// learnable projection, V_hat = Conv1D(X0) W_target, reaching the next and near-future tokens;
// section 6, padding at chunk boundaries keeps the convolution from reading another chunk, and
// the convolution is depthwise). Two launches on the caller's stream:
//   1. k_target_conv: A[b][t][c] = bf16( sum_{j=1..width} w[j-1][c] X0[b][t+j][c] ), where a
//      token at or past the end of t's chunk (or past T) contributes zero; fp32 arithmetic;
//   2. k_target_gemm: V_hat[b][t][o] = sum_c A[b][t][c] W_target[c][o] on the direct-to-LDS
//      engine, fp32 accumulation: the tile's M axis is o (W_target is read K-major through
//      transposing LDS reads), N is t, K is c.
#include "common.hpp"
#include "dma.hpp"
#include "engine.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

// One thread per 8 channels of one token: width 16-byte loads of X0, one 16-byte store of A.
__global__ __launch_bounds__(256) void k_target_conv(const uint16_t* __restrict__ X0,
                                                     const float* __restrict__ w, int width,
                                                     uint16_t* __restrict__ A, int T, int D,
                                                     int chunk) {
  const int b = blockIdx.y;
  const int c8 = D / 8;
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= long(T) * c8) return;
  const int t = int(i / c8), c = int(i % c8) * 8;
  const int end = min((t / chunk + 1) * chunk, T);  // first token of the next chunk
  const uint16_t* x = X0 + long(b) * T * D;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 1; j <= width && t + j < end; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + long(t + j) * D + c);
    const float4 w0 = *reinterpret_cast<const float4*>(w + long(j - 1) * D + c);
    const float4 w1 = *reinterpret_cast<const float4*>(w + long(j - 1) * D + c + 4);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(ww[2 * q], bf2f(uint16_t(u[q] & 0xFFFFu)), acc[2 * q]);
      acc[2 * q + 1] = fmaf(ww[2 * q + 1], bf2f(uint16_t(u[q] >> 16)), acc[2 * q + 1]);
    }
  }
  *reinterpret_cast<uint4*>(A + long(b) * T * D + long(t) * D + c) =
      make_uint4(pack2bf(acc[0], acc[1]), pack2bf(acc[2], acc[3]), pack2bf(acc[4], acc[5]),
                 pack2bf(acc[6], acc[7]));
}

constexpr int TG_BN = 128, TG_NS = 3;

template <typename TOut>
__global__ __launch_bounds__(NTHR, 1) void k_target_gemm(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ Wt,
                                                         TOut* __restrict__ Vh, int T, int Din,
                                                         int Dout, int tiles_n) {
  __shared__ SmemD<TG_BN, 64, TG_NS> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile / tiles_n, tn = tile % tiles_n;  // consecutive tiles share W columns
  const int o0 = tm * BM, t0 = tn * TG_BN;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const DOpN<64> oa(Wt + o0, Dout, Din, min(BM, Dout - o0), 0, wave, lane);
  const DOp<TG_BN, 64> ob(A + long(b) * T * Din + long(t0) * Din, Din, min(TG_BN, T - t0), 64,
                          BM * 128, wave, lane);
  const DFrag<TG_BN, 64, true> fr(wave >> 1, wave & 1, lane);
  Acc<TG_BN> acc;
  zero_acc<TG_BN>(acc);
  dma_segment<TG_BN, 64, TG_NS>(acc, oa, ob, Din / 64, sm, fr);
  TOut* vb = Vh + long(b) * T * Dout;
  store_tile_raw<TG_BN>(acc, reinterpret_cast<float*>(&sm), tid, [&](int n, int m, float4 v) {
    const int t = t0 + n, o = o0 + m;
    if (t < T && o < Dout) {
      if constexpr (sizeof(TOut) == 2)
        *reinterpret_cast<uint2*>(vb + long(t) * Dout + o) = pack4(v);
      else
        *reinterpret_cast<float4*>(vb + long(t) * Dout + o) = v;
    }
  });
}

}  // namespace

hipError_t lm_target(const TargetArgs& a) {
  uint16_t* A = static_cast<uint16_t*>(a.ws);
  const long n8 = long(a.T) * (a.Din / 8);
  hipLaunchKernelGGL(k_target_conv, dim3(unsigned((n8 + 255) / 256), a.B), dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.X0), a.conv_w, a.width, A, a.T,
                     a.Din, a.chunk);
  const int tiles_m = (a.Dout + BM - 1) / BM, tiles_n = (a.T + TG_BN - 1) / TG_BN;
  if (a.out_bf16)
    hipLaunchKernelGGL((k_target_gemm<uint16_t>), dim3(tiles_m * tiles_n, a.B), dim3(NTHR), 0,
                       a.stream, A, static_cast<const uint16_t*>(a.Wt),
                       static_cast<uint16_t*>(a.Vh), a.T, a.Din, a.Dout, tiles_n);
  else
    hipLaunchKernelGGL((k_target_gemm<float>), dim3(tiles_m * tiles_n, a.B), dim3(NTHR), 0,
                       a.stream, A, static_cast<const uint16_t*>(a.Wt),
                       static_cast<float*>(a.Vh), a.T, a.Din, a.Dout, tiles_n);
  return hipGetLastError();
}

}  // namespace ttt
