// In-Place TTT chunk scan, fp32 path ("In-Place Test-Time Training", iplexlaw.co.kr blog,
// sections 2-3): for each chunk, O_i = Z_i W^T with the pre-update state, then
// W += eta * V_i^T Z_i. Plain fp32 FMA tiles; this path serves fp32 inputs, where the
// contract is fp32 accuracy rather than matrix-core throughput.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int TS = 64;   // output tile edge
constexpr int KS = 16;   // K step

// O[t][d] = sum_f Z[t][f] W[d][f], rows t in [t0, t1).
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_simt_apply(const TIn* __restrict__ Z,
                                                    const float* __restrict__ W,
                                                    TOut* __restrict__ O, int F, int D, int t0,
                                                    int t1, long z_b, long w_b, long o_b) {
  __shared__ float zs[KS][TS + 1];
  __shared__ float ws[KS][TS + 1];
  const int b = blockIdx.z;
  Z += b * z_b;
  W += b * w_b;
  O += b * o_b;
  const int d0 = blockIdx.x * TS, r0 = t0 + blockIdx.y * TS;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int f0 = 0; f0 < F; f0 += KS) {
    for (int e = threadIdx.x; e < TS * KS; e += 256) {
      const int r = e / KS, c = e % KS, f = f0 + c;
      const int t = r0 + r, d = d0 + r;
      zs[c][r] = (t < t1 && f < F) ? ld_elem(Z, size_t(t) * F + f) : 0.f;
      ws[c][r] = (d < D && f < F) ? W[size_t(d) * F + f] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = zs[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = ws[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = r0 + ty * 4 + i;
    if (t >= t1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = d0 + tx * 4 + j;
      if (d < D) st_elem(O, size_t(t) * D + d, acc[i][j]);
    }
  }
}

// W[d][f] += eta * sum_{t in [t0, t1)} V[t][d] Z[t][f].
template <typename TIn>
__global__ __launch_bounds__(256) void k_simt_update(const TIn* __restrict__ Z,
                                                     const TIn* __restrict__ V,
                                                     float* __restrict__ W, int F, int D, int t0,
                                                     int t1, float eta, long z_b, long v_b,
                                                     long w_b) {
  __shared__ float vs[KS][TS];
  __shared__ float zs[KS][TS];
  const int b = blockIdx.z;
  Z += b * z_b;
  V += b * v_b;
  W += b * w_b;
  const int f0 = blockIdx.x * TS, d0 = blockIdx.y * TS;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int tt = t0; tt < t1; tt += KS) {
    for (int e = threadIdx.x; e < TS * KS; e += 256) {
      const int k = e / TS, c = e % TS, t = tt + k;
      vs[k][c] = (t < t1 && d0 + c < D) ? ld_elem(V, size_t(t) * D + d0 + c) : 0.f;
      zs[k][c] = (t < t1 && f0 + c < F) ? ld_elem(Z, size_t(t) * F + f0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float a[4], z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = vs[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = zs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], z[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = d0 + ty * 4 + i;
    if (d >= D) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = f0 + tx * 4 + j;
      if (f < F) {
        const size_t idx = size_t(d) * F + f;
        W[idx] = W[idx] + eta * acc[i][j];
      }
    }
  }
}

template <typename TIn, typename TOut>
hipError_t run(const ScanArgs& a, PhaseClock* clk) {
  const size_t DF = size_t(a.D) * a.F;
  float* Wbuf = a.W_final ? a.W_final : static_cast<float*>(a.ws);
  const TIn* Z = static_cast<const TIn*>(a.Z);
  const TIn* V = static_cast<const TIn*>(a.V);
  TOut* O = static_cast<TOut*>(a.O);
  if (Wbuf != a.W0) {
    for (int b = 0; b < a.B; ++b) {
      const float* src = a.W0 + (a.w0_shared ? 0 : b * DF);
      hipError_t e = hipMemcpyAsync(Wbuf + b * DF, src, DF * sizeof(float),
                                    hipMemcpyDeviceToDevice, a.stream);
      if (e != hipSuccess) return e;
    }
  }
  const long ts = a.T_stride > 0 ? a.T_stride : a.T;  // tokens between sequences
  const long z_b = ts * a.F, v_b = ts * a.D, o_b = ts * a.D;
  const dim3 blk(256);
  for (int t0 = 0; t0 < a.T; t0 += a.C) {
    const int t1 = t0 + a.C < a.T ? t0 + a.C : a.T;
    const dim3 ga((a.D + TS - 1) / TS, (t1 - t0 + TS - 1) / TS, a.B);
    if (clk) clk->open(3);
    hipLaunchKernelGGL((k_simt_apply<TIn, TOut>), ga, blk, 0, a.stream, Z, Wbuf, O, a.F, a.D,
                       t0, t1, z_b, long(DF), o_b);
    if (clk) clk->close(1);
    if (t1 < a.T || a.W_final) {
      const dim3 gu((a.F + TS - 1) / TS, (a.D + TS - 1) / TS, a.B);
      if (clk) clk->open(2);
      hipLaunchKernelGGL((k_simt_update<TIn>), gu, blk, 0, a.stream, Z, V, Wbuf, a.F, a.D, t0,
                         t1, a.eta, z_b, v_b, long(DF));
      if (clk) clk->close(1);
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t scan_simt_workspace(int B, int T, int F, int D, int C) {
  (void)T;
  (void)C;
  return size_t(B) * D * F * sizeof(float);  // working state when W_final is not requested
}

hipError_t scan_simt(const ScanArgs& a, PhaseClock* clk) {
  if (a.in_bf16)
    return a.out_bf16 ? run<uint16_t, uint16_t>(a, clk) : run<uint16_t, float>(a, clk);
  return a.out_bf16 ? run<float, uint16_t>(a, clk) : run<float, float>(a, clk);
}

}  // namespace ttt
