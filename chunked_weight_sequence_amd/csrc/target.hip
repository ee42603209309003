// LM-aligned target producer ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv
// 2604.06169: section 4, the target is a 1-D convolution of the token embeddings followed by a
// learnable projection, V_hat = Conv1D(X0) W_target, reaching the next and near-future tokens;
// section 6, padding at chunk boundaries keeps the convolution from reading another chunk, and
// the convolution is depthwise). Three launches on the caller's stream:
//   1. k_target_conv: A[b][t][c] = bf16( sum_{j=1..width} w[j-1][c] X0[b][t+j][c] ), where a
//      token at or past the end of t's chunk (or past T) contributes zero; fp32 arithmetic;
//   2. k_target_wt: W_target transposed into the workspace ([Dout][Din], 2 Din Dout bytes);
//   3. k_target_gemm: V_hat[b][t][o] = sum_c A[b][t][c] W_target[c][o] on the eight-wave
//      ping-pong engine, fp32 accumulation: the tile's M axis is o, N is t, K is c, both
//      operands read with c contiguous.
#include "common.hpp"
#include "dma.hpp"
#include "engine.hpp"
#include "launch.hpp"
#include "pingpong.hpp"

namespace ttt {
namespace {

// One workgroup per 64 tokens x 64 channels: the X0 rows the tile reads (its 64 tokens' next
// `width` neighbours, at most 79 rows of 128 bytes) and the tile's conv_w columns are staged
// once in LDS, so every X0 row is fetched from HBM about once instead of `width` times. Thread
// (g = tid % 8, r = tid / 8) owns channels 8g..8g+7 of tokens r and r + 32; the sum runs over
// j = 1..width in order, in fp32.
constexpr int CONV_TT = 64, CONV_TC = 64, CONV_WMAX = 16;
__global__ __launch_bounds__(256) void k_target_conv(const uint16_t* __restrict__ X0,
                                                     const float* __restrict__ w, int width,
                                                     uint16_t* __restrict__ A, int T, int D,
                                                     int chunk) {
  __shared__ uint4 xs[CONV_TT + CONV_WMAX - 1][CONV_TC / 8];
  __shared__ float4 ws[CONV_WMAX][CONV_TC / 4];
  const int t0 = blockIdx.x * CONV_TT, c0 = blockIdx.y * CONV_TC, b = blockIdx.z;
  const int tid = threadIdx.x, g = tid & 7, r = tid >> 3;
  const uint16_t* x = X0 + long(b) * T * D;
  // rows t0+1 .. t0+nrows of X0 (none at or past T)
  const int nrows = min(CONV_TT + width - 1, T - 1 - t0);
  for (int e = tid; e < nrows * 8; e += 256) {
    const int row = e >> 3, q = e & 7;
    xs[row][q] = *reinterpret_cast<const uint4*>(x + long(t0 + 1 + row) * D + c0 + 8 * q);
  }
  for (int e = tid; e < width * (CONV_TC / 4); e += 256) {
    const int j = e / (CONV_TC / 4), q = e % (CONV_TC / 4);
    ws[j][q] = *reinterpret_cast<const float4*>(w + long(j) * D + c0 + 4 * q);
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = t0 + r + 32 * h;
    if (t >= T) break;
    const int end = min((t / chunk + 1) * chunk, T);  // first token of the next chunk
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 1; j <= width && t + j < end; ++j) {
      const uint4 v = xs[t + j - t0 - 1][g];
      const float4 w0 = ws[j - 1][2 * g], w1 = ws[j - 1][2 * g + 1];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(ww[2 * q], bf2f(uint16_t(u[q] & 0xFFFFu)), acc[2 * q]);
        acc[2 * q + 1] = fmaf(ww[2 * q + 1], bf2f(uint16_t(u[q] >> 16)), acc[2 * q + 1]);
      }
    }
    *reinterpret_cast<uint4*>(A + long(b) * T * D + long(t) * D + c0 + 8 * g) =
        make_uint4(pack2bf(acc[0], acc[1]), pack2bf(acc[2], acc[3]), pack2bf(acc[4], acc[5]),
                   pack2bf(acc[6], acc[7]));
  }
}

// W_target [Din][Dout] -> its transpose [Dout][Din] (rows = output columns, the contraction
// index contiguous) through a 64 x 64 LDS tile; Din % 64 == 0 and Dout % 16 == 0.
__global__ __launch_bounds__(256) void k_target_wt(const uint16_t* __restrict__ W,
                                                   uint16_t* __restrict__ Wt, int Din, int Dout) {
  __shared__ uint16_t tile[64][64 + 2];
  const int k0 = blockIdx.x * 64, o0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    tile[r][c] = o0 + c < Dout ? W[long(k0 + r) * Dout + o0 + c] : uint16_t(0);
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) {
    const int o = e >> 6, k = e & 63;
    if (o0 + o < Dout) Wt[long(o0 + o) * Din + k0 + k] = tile[k][o];
  }
}

constexpr int TG_NS = 4;  // LDS stages of 32 K each

// V_hat tile: 256 output columns o (rows of the transposed W_target) x 256 tokens t, K = Din, on
// the eight-wave ping-pong engine. acc[i][j][e] holds o = o0 + pp_row(w, lane, i, e) and
// t = t0 + pp_col(w, lane, j).
template <typename TOut>
__global__ __launch_bounds__(512, 1) void k_target_gemm(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ Wt,
                                                        TOut* __restrict__ Vh, int T, int Din,
                                                        int Dout, int tiles_m) {
  __shared__ PPSmem<TG_NS> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  // Consecutive tiles share the token panel of A, and each XCD takes a contiguous run of them
  // (xcd_remap), so every panel of A is fetched into one L2 only; W_target (Din x Dout, 13 MB at
  // 2560) is what every XCD reads.
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int o0 = tm * PP_T, t0 = tn * PP_T;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int no = min(PP_T, Dout - o0), nt = min(PP_T, T - t0);
  const PPOp oa(Wt + long(o0) * Din, 128, 0, wave, lane,
                [&](int r) { return long(min(r, no - 1)) * Din * 2; });
  const PPOp ob(A + long(b) * T * Din + long(t0) * Din, 128, PP_OPB, wave, lane,
                [&](int r) { return long(min(r, nt - 1)) * Din * 2; });
  PPAcc acc;
  pp_zero(acc);
  pp_segment<TG_NS>(acc, oa, ob, Din / PP_BK, sm, wave, lane);
  TOut* vb = Vh + long(b) * T * Dout;
  if constexpr (sizeof(TOut) == 2) {
    // bf16 V_hat: staged in the free stage ring, stored as whole 512-byte token rows
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
      if (n < nt && c * 8 < no) pp_store_nt(vb + long(t0 + n) * Dout + o0 + c * 8, v);
    });
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + pp_col(wave, lane, j);
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = o0 + pp_row(wave, lane, i, 0);
      if (o >= Dout) continue;
      *reinterpret_cast<float4*>(vb + long(t) * Dout + o) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

}  // namespace

size_t lm_target_workspace(int B, int T, int Din, int Dout) {
  return ((size_t(B) * T * Din * 2 + 255) & ~size_t(255)) + size_t(Din) * Dout * 2;
}

hipError_t lm_target(const TargetArgs& a) {
  uint16_t* A = static_cast<uint16_t*>(a.ws);
  uint16_t* Wt = reinterpret_cast<uint16_t*>(static_cast<char*>(a.ws) +
                                             ((size_t(a.B) * a.T * a.Din * 2 + 255) & ~size_t(255)));
  hipLaunchKernelGGL(k_target_conv, dim3((a.T + CONV_TT - 1) / CONV_TT, a.Din / CONV_TC, a.B),
                     dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.X0), a.conv_w, a.width, A, a.T,
                     a.Din, a.chunk);
  hipLaunchKernelGGL(k_target_wt, dim3(a.Din / 64, (a.Dout + 63) / 64), dim3(256), 0, a.stream,
                     static_cast<const uint16_t*>(a.Wt), Wt, a.Din, a.Dout);
  const int tiles_m = (a.Dout + PP_T - 1) / PP_T, tiles_n = (a.T + PP_T - 1) / PP_T;
  if (a.out_bf16)
    hipLaunchKernelGGL((k_target_gemm<uint16_t>), dim3(tiles_m * tiles_n, a.B), dim3(512), 0,
                       a.stream, A, Wt, static_cast<uint16_t*>(a.Vh), a.T, a.Din, a.Dout, tiles_m);
  else
    hipLaunchKernelGGL((k_target_gemm<float>), dim3(tiles_m * tiles_n, a.B), dim3(512), 0,
                       a.stream, A, Wt, static_cast<float*>(a.Vh), a.T, a.Din, a.Dout, tiles_m);
  return hipGetLastError();
}

}  // namespace ttt
