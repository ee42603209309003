// Per-chunk clipping of the fast-weight update ("In-Place Test-Time Training", iplexlaw.co.kr
// blog on arXiv 2604.06169, section 6: for long contexts the Frobenius norm of every update
// delta is limited to a threshold, which keeps the accumulated state stable).
//
// Chunk i's delta is dW_i = eta V_i^T Z_i (d_model x d_ff); its clipped form is
// dW_i * min(1, tau / ||dW_i||_F). Two facts make this cheap on the device:
//   * ||V_i^T Z_i||_F^2 = <Z_i Z_i^T, V_i V_i^T>_F, an inner product of two C x C Gram matrices,
//     so the norm never needs the d_model x d_ff delta;
//   * the delta is linear in V_i, so the clipped scan is the plain scan run on the targets with
//     chunk i's rows scaled by its factor.
// Three launches on the caller's stream:
//   1. the norm slots: for bf16 inputs, per (chunk, 256-row block s, 256-row block t) with
//      t >= s, the two Gram tiles on the eight-wave engine (k_gram_pp; fp32 accumulation; blocks
//      above the diagonal count twice), or the register-staged engine on 256 x 128 blocks when
//      d_ff or d_model is not a multiple of 32 (k_gram_norm); for fp32 inputs, per (chunk, row s)
//      with fp32 dot products (k_gram_norm_f32). Each writes the fp64 sum of
//      (z_s . z_t)(v_s . v_t) over its in-chunk pairs to its own slot;
//   2. k_clip_finish: per chunk, the slots summed in a fixed order in fp64 (the result does not
//      depend on scheduling), ||dW_i|| = |eta| sqrt(sum), factor = min(1, tau / ||dW_i||);
//   3. k_scale_rows: V'[t] = factor(chunk of t) * V[t], rounded to the input type.
#include "common.hpp"
#include "engine.hpp"
#include "launch.hpp"
#include "pingpong.hpp"

namespace ttt {
namespace {

constexpr int GN_BN = 128;

__device__ __forceinline__ double block_sum(double v, double* red, int tid) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <bool FAST>
__global__ __launch_bounds__(NTHR, 1) void k_gram_norm(const uint16_t* __restrict__ Z,
                                                       const uint16_t* __restrict__ V, long z_b,
                                                       long v_b, double* __restrict__ part,
                                                       int T, int F, int D, int C, int ns,
                                                       int nt, int nch) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int per = ns * nt;
  const int ch = blockIdx.x / per, r = blockIdx.x % per, st = r / nt, tt = r % nt;
  const int c0 = ch * C, c1 = min(c0 + C, T);
  const int s0 = c0 + st * BM, t0 = c0 + tt * GN_BN;
  double* out = part + (long(b) * nch + ch) * per + r;
  // Both Gram matrices are symmetric, so the blocks wholly below the diagonal (every t < every s)
  // are skipped and the blocks wholly above it (every t > every s) count twice.
  if (s0 >= c1 || t0 >= c1 || t0 + GN_BN <= s0) {
    if (tid == 0) *out = 0.0;
    return;
  }
  const double weight = t0 >= s0 + BM ? 2.0 : 1.0;
  const int ms = min(BM, c1 - s0), mt = min(GN_BN, c1 - t0);
  __shared__ Smem<GN_BN> sm;
  __shared__ double red[4];
  Acc<GN_BN> az, av;
  zero_acc<GN_BN>(az);
  zero_acc<GN_BN>(av);
  {
    Rows<BM, FAST> la(Z + b * z_b + long(s0) * F, F, ms, 0, F, tid);
    Rows<GN_BN, FAST> lb(Z + b * z_b + long(t0) * F, F, mt, 0, F, tid);
    mma_segment<GN_BN>(az, la, lb, 0, F, sm, tid);
  }
  __syncthreads();  // the LDS buffers are reused by the second product
  {
    Rows<BM, FAST> la(V + b * v_b + long(s0) * D, D, ms, 0, D, tid);
    Rows<GN_BN, FAST> lb(V + b * v_b + long(t0) * D, D, mt, 0, D, tid);
    mma_segment<GN_BN>(av, la, lb, 0, D, sm, tid);
  }
  // az[i][j][e], av[i][j][e]: row s0 + m, column t0 + n of the two Gram matrices
  const int wave = tid >> 6, lane = tid & 63, wm = wave >> 1, wn = wave & 1;
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < GN_BN / 64; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = wm * (BM / 2) + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        const int n = wn * (GN_BN / 2) + j * 32 + (lane & 31);
        if (m < ms && n < mt) sum += double(az[i][j][e]) * double(av[i][j][e]);
      }
  const double tot = block_sum(sum, red, tid);
  if (tid == 0) *out = weight * tot;
}

// bf16 inputs with d_ff and d_model multiples of 32: the eight-wave engine on 256 x 256 tiles.
// Workgroup (chunk, s, t) with t >= s forms the V Gram tile first, parks it in its own 256 KB of
// the scratch `gv` (accumulator order: every store and load instruction moves 1 KB), forms the Z
// Gram tile in the same registers, and sums (z_s . z_t)(v_s . v_t) in fp64 over its in-chunk
// pairs; tiles above the diagonal count twice, those below write 0.
__global__ __launch_bounds__(512, 1) void k_gram_pp(const uint16_t* __restrict__ Z,
                                                    const uint16_t* __restrict__ V, long z_b,
                                                    long v_b, double* __restrict__ part,
                                                    float* __restrict__ gv, int T, int F, int D,
                                                    int C, int ns, int nch) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int per = ns * ns, ntri = ns * (ns + 1) / 2;
  const int ch = blockIdx.x / per, r = blockIdx.x % per, st = r / ns, tt = r % ns;
  const int c0 = ch * C, c1 = min(c0 + C, T);
  const int s0 = c0 + st * PP_T, t0 = c0 + tt * PP_T;
  double* out = part + (long(b) * nch + ch) * per + r;
  if (tt < st || s0 >= c1 || t0 >= c1) {
    if (tid == 0) *out = 0.0;
    return;
  }
  const double weight = tt > st ? 2.0 : 1.0;
  const int ms = min(PP_T, c1 - s0), mt = min(PP_T, c1 - t0);
  __shared__ PPSmem<4> sm;
  __shared__ double red[8];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int tri = st * ns - st * (st - 1) / 2 + (tt - st);
  float* my = gv + ((long(b) * nch + ch) * ntri + tri) * (PP_T * PP_T) + wave * 8192 + lane * 4;
  PPAcc acc;
  pp_zero(acc);
  {
    const PPOp oa(V + b * v_b + long(s0) * D, 128, 0, wave, lane,
                  [&](int q) { return long(min(q, ms - 1)) * D * 2; });
    const PPOp ob(V + b * v_b + long(t0) * D, 128, PP_OPB, wave, lane,
                  [&](int q) { return long(min(q, mt - 1)) * D * 2; });
    pp_segment<4>(acc, oa, ob, D / PP_BK, sm, wave, lane);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(my + (i * 4 + j) * 256) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  pp_zero(acc);
  __syncthreads();  // every wave is past the first product's last LDS read
  {
    const PPOp oa(Z + b * z_b + long(s0) * F, 128, 0, wave, lane,
                  [&](int q) { return long(min(q, ms - 1)) * F * 2; });
    const PPOp ob(Z + b * z_b + long(t0) * F, 128, PP_OPB, wave, lane,
                  [&](int q) { return long(min(q, mt - 1)) * F * 2; });
    pp_segment<4>(acc, oa, ob, F / PP_BK, sm, wave, lane);  // ends with its stores drained too
  }
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(my + (i * 4 + j) * 256);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      const int n = pp_col(wave, lane, j);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pp_row(wave, lane, i, e) < ms && n < mt) sum += double(acc[i][j][e]) * double(vv[e]);
    }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < 8; ++w) tot += red[w];
    *out = weight * tot;
  }
}

// fp32 inputs: one workgroup per (chunk, row s); thread t' takes rows t of the chunk in turn.
__global__ __launch_bounds__(256) void k_gram_norm_f32(const float* __restrict__ Z,
                                                       const float* __restrict__ V, long z_b,
                                                       long v_b, double* __restrict__ part,
                                                       int T, int F, int D, int C, int nch) {
  __shared__ double red[4];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int ch = blockIdx.x / C, sl = blockIdx.x % C;
  const int c0 = ch * C, c1 = min(c0 + C, T), s = c0 + sl;
  double* out = part + (long(b) * nch + ch) * C + sl;
  if (s >= c1) {
    if (tid == 0) *out = 0.0;
    return;
  }
  const float* zs = Z + b * z_b + long(s) * F;
  const float* vs = V + b * v_b + long(s) * D;
  double sum = 0.0;
  for (int t = c0 + tid; t < c1; t += 256) {
    const float* zt = Z + b * z_b + long(t) * F;
    const float* vt = V + b * v_b + long(t) * D;
    float dz = 0.f, dv = 0.f;
    for (int f = 0; f < F; ++f) dz = fmaf(zs[f], zt[f], dz);
    for (int d = 0; d < D; ++d) dv = fmaf(vs[d], vt[d], dv);
    sum += double(dz) * double(dv);
  }
  const double tot = block_sum(sum, red, tid);
  if (tid == 0) *out = tot;
}

__global__ void k_clip_finish(const double* __restrict__ part, int P, int n, float eta,
                              float tau, float* __restrict__ scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double s2 = 0.0;
  for (int p = 0; p < P; ++p) s2 += part[long(i) * P + p];
  const double norm = fabs(double(eta)) * sqrt(fmax(s2, 0.0));
  scale[i] = norm > double(tau) ? float(double(tau) / norm) : 1.f;
}

// V'[b][t][:] = scale[b][t / C] * V[b][t][:]; 8 elements per thread
template <typename TIn>
__global__ __launch_bounds__(256) void k_scale_rows(const TIn* __restrict__ V,
                                                    const float* __restrict__ scale,
                                                    TIn* __restrict__ Vs, long T, int D, int C,
                                                    int nch, long n8) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const long e = i * 8;
  const long row = e / D;  // b * T + t
  const long b = row / T, t = row % T;
  const float s = scale[b * nch + t / C];
  if constexpr (sizeof(TIn) == 2) {
    const uint4 v = *reinterpret_cast<const uint4*>(V + e);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack2bf(s * bf2f(uint16_t(w[q] & 0xFFFFu)), s * bf2f(uint16_t(w[q] >> 16)));
    *reinterpret_cast<uint4*>(Vs + e) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(V + e);
    const float4 c = *reinterpret_cast<const float4*>(V + e + 4);
    *reinterpret_cast<float4*>(Vs + e) = make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
    *reinterpret_cast<float4*>(Vs + e + 4) = make_float4(s * c.x, s * c.y, s * c.z, s * c.w);
  }
}

int gram_slots(int C, bool bf16) {
  return bf16 ? ((C + BM - 1) / BM) * ((C + GN_BN - 1) / GN_BN) : C;
}

}  // namespace

// V Gram tiles parked by k_gram_pp: 256 KB per tile on or above the diagonal
size_t gram_scratch(int B, int T, int C, bool in_bf16) {
  if (!in_bf16) return 0;
  const int nch = (T + C - 1) / C, ns = (C + PP_T - 1) / PP_T;
  return size_t(B) * nch * (ns * (ns + 1) / 2) * PP_T * PP_T * 4;
}

size_t clip_workspace(int B, int T, int D, int C, bool in_bf16) {
  const int nch = (T + C - 1) / C;
  const size_t v = (size_t(B) * T * D * (in_bf16 ? 2 : 4) + 255) & ~size_t(255);
  const size_t p = (size_t(B) * nch * gram_slots(C, in_bf16) * 8 + 255) & ~size_t(255);
  const size_t s = (size_t(B) * nch * 4 + 255) & ~size_t(255);
  return v + p + s + gram_scratch(B, T, C, in_bf16);
}

hipError_t clip_targets(const ClipArgs& a) {
  const int nch = (a.T + a.C - 1) / a.C;
  const int P = gram_slots(a.C, a.in_bf16);
  char* ws = static_cast<char*>(a.ws);
  const size_t vbytes = (size_t(a.B) * a.T * a.D * (a.in_bf16 ? 2 : 4) + 255) & ~size_t(255);
  double* part = reinterpret_cast<double*>(ws + vbytes);
  const size_t pbytes = (size_t(a.B) * nch * P * 8 + 255) & ~size_t(255);
  float* scale = reinterpret_cast<float*>(ws + vbytes + pbytes);
  const long z_b = long(a.T) * a.F, v_b = long(a.T) * a.D;
  int P_used = P;  // slots per chunk written by the norm kernel
  if (a.in_bf16) {
    const auto* Z = static_cast<const uint16_t*>(a.Z);
    const auto* V = static_cast<const uint16_t*>(a.V);
    if (a.F % PP_BK == 0 && a.D % PP_BK == 0) {
      const int ns = (a.C + PP_T - 1) / PP_T;
      const size_t sbytes = (size_t(a.B) * nch * 4 + 255) & ~size_t(255);
      float* gv = reinterpret_cast<float*>(ws + vbytes + pbytes + sbytes);
      P_used = ns * ns;
      hipLaunchKernelGGL(k_gram_pp, dim3(unsigned(nch * ns * ns), unsigned(a.B)), dim3(512), 0,
                         a.stream, Z, V, z_b, v_b, part, gv, a.T, a.F, a.D, a.C, ns, nch);
    } else {
      const int ns = (a.C + BM - 1) / BM, nt = (a.C + GN_BN - 1) / GN_BN;
      const dim3 grid(unsigned(nch * ns * nt), unsigned(a.B));
      hipLaunchKernelGGL(k_gram_norm<false>, grid, dim3(NTHR), 0, a.stream, Z, V, z_b, v_b,
                         part, a.T, a.F, a.D, a.C, ns, nt, nch);
    }
  } else {
    hipLaunchKernelGGL(k_gram_norm_f32, dim3(unsigned(nch * a.C), unsigned(a.B)), dim3(256), 0,
                       a.stream, static_cast<const float*>(a.Z), static_cast<const float*>(a.V),
                       z_b, v_b, part, a.T, a.F, a.D, a.C, nch);
  }
  const int n = a.B * nch;
  hipLaunchKernelGGL(k_clip_finish, dim3((n + 255) / 256), dim3(256), 0, a.stream, part, P_used, n,
                     a.eta, a.tau, scale);
  const long n8 = long(a.B) * a.T * a.D / 8;
  const dim3 g8(unsigned((n8 + 255) / 256));
  if (a.in_bf16)
    hipLaunchKernelGGL(k_scale_rows<uint16_t>, g8, dim3(256), 0, a.stream,
                       static_cast<const uint16_t*>(a.V), scale, reinterpret_cast<uint16_t*>(ws),
                       long(a.T), a.D, a.C, nch, n8);
  else
    hipLaunchKernelGGL(k_scale_rows<float>, g8, dim3(256), 0, a.stream,
                       static_cast<const float*>(a.V), scale, reinterpret_cast<float*>(ws),
                       long(a.T), a.D, a.C, nch, n8);
  return hipGetLastError();
}

}  // namespace ttt
