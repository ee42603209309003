// SR-TTT residual-cache readout with alpha fusion ("SR-TTT: Surprisal-Aware Residual Test-Time
// Training", gist.science summary of arXiv 2603.06642, section 2.1: the routed tokens' keys and
// values form a fixed-capacity cache beside the fast weights, and the layer output is the TTT
// output plus a clamp-parameterised gate alpha times the attention output over that cache;
// section 5: eviction behaves FIFO-like once the cache is full).
//
// A token of routing chunk c reads the cache as it stood when chunk c began: the newest
// `capacity` routed tokens with index < c * chunk. Per head h (dh = 64):
//     a = sum_j softmax_j(scale * q . k_j) v_j   (zero when the cache is empty)
//     out = ttt_out + clamp(alpha, 0, 1) * a      (per channel of the H * dh output)
//
// One workgroup per (64-token block, head, sequence), 4 waves of 16 tokens:
//   1. the visible token indices, newest first: 2048 mask bytes below the chunk start per pass,
//      8 per thread, ranked by a block-wide scan;
//   2. the cached key rows of head h go to LDS as rows (padded), the value rows transposed;
//   3. S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS, the wave's 16 queries from
//      global memory), fp32; masked softmax per token with fp32 exponentials;
//   4. O = P V on v_mfma_f32_16x16x16_bf16: the S^T result layout (lane l: token l % 16, cache
//      rows 4 (l / 16) + i) is the A-operand layout of that instruction, so the bf16 weights go
//      from registers straight into the product; the normaliser is the sum of the same rounded
//      weights, applied to the fp32 result.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int RO_TOK = 64, RO_CAP = 256, RO_DH = 64;
constexpr int RO_KP = RO_DH + 8;    // key row pitch (bf16): 144 bytes, conflict-free 16-byte reads
// transposed value row pitch (bf16): 130 four-byte words, so the 8-byte reads of 16 consecutive
// rows fall on 16 distinct bank pairs (132 words put rows r and r + 8 on the same pair)
constexpr int RO_VP = RO_CAP + 4;

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename TOut>
__global__ __launch_bounds__(256) void k_cache_readout(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint8_t* __restrict__ routed, const TOut* ttt, TOut* out, const float* __restrict__ alpha,
    int T, int H, int chunk, int cap, float scale) {
  __shared__ uint16_t ks[RO_CAP * RO_KP];
  __shared__ uint16_t vt[RO_DH * RO_VP];
  __shared__ int idx[RO_CAP];
  __shared__ int nvis_s, wsum[4];
  const int t0 = blockIdx.x * RO_TOK, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long HD = long(H) * RO_DH;
  const long seq = long(b) * T;

  // 1. visible cache entries: routed tokens before the chunk start, newest first. Each pass
  // covers the 2048 tokens below `wend`: thread i reads the 8 mask bytes of tokens
  // [wend - 8 (i + 1), wend - 8 i), a block-wide exclusive scan over i ranks them from the
  // newest, and the first `cap` ranks are kept.
  {
    const int end = (t0 / chunk) * chunk;
    const uint8_t* mrow = routed + seq;
    int found = 0;  // uniform
    for (int wend = end; wend > 0 && found < cap; wend -= 8 * 256) {
      const int lo = wend - 8 * (tid + 1);  // a multiple of 8: whole groups or none below 0
      uint2 m = make_uint2(0, 0);
      if (lo >= 0) m = *reinterpret_cast<const uint2*>(mrow + lo);
      uint32_t flags = 0;  // bit k: token lo + k is routed
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        flags |= ((m.x >> (8 * k)) & 0xFFu) ? (1u << k) : 0u;
        flags |= ((m.y >> (8 * k)) & 0xFFu) ? (1u << (k + 4)) : 0u;
      }
      const int n = __popc(flags);
      int incl = n;  // inclusive scan within the wave
#pragma unroll
      for (int d = 1; d < 64; d *= 2) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      int before = incl - n;
      for (int w = 0; w < wave; ++w) before += wsum[w];
      const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
      int pos = found + before;
#pragma unroll
      for (int k = 7; k >= 0; --k)  // newest first
        if (flags & (1u << k)) {
          if (pos < cap) idx[pos] = lo + k;
          ++pos;
        }
      found += total;
      __syncthreads();  // wsum is reused by the next pass
    }
    if (tid == 0) nvis_s = min(found, cap);
  }
  __syncthreads();
  const int nvis = nvis_s;
  const int tok = t0 + 16 * wave;  // this wave's first token
  if (nvis == 0) {  // empty cache: the output is the TTT output itself
    for (int e = lane; e < 16 * RO_DH; e += 64) {
      const long o = (seq + tok + e / RO_DH) * HD + h * RO_DH + e % RO_DH;
      out[o] = ttt[o];
    }
    return;
  }
  const int nj = (nvis + 15) / 16;  // 16-row blocks of the cache in use
  // the wave's queries and TTT outputs, loaded ahead of the cache gather
  const int col = lane & 15, grp = lane >> 4;
  uint4 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    qf[s] = *reinterpret_cast<const uint4*>(Q + (seq + tok + col) * HD + h * RO_DH + 32 * s +
                                            8 * grp);
  float base[RO_DH / 16][4];  // element (token 4 grp + i, channel 16 dt + col)
#pragma unroll
  for (int dt = 0; dt < RO_DH / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      base[dt][i] = ld_elem(ttt, size_t((seq + tok + 4 * grp + i) * HD + h * RO_DH + 16 * dt + col));

  // 2. key rows and transposed value rows of head h; rows >= nvis are zero
  for (int e = tid; e < nj * 16 * 8; e += 256) {
    const int j = e >> 3, c = e & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < nvis)
      v = *reinterpret_cast<const uint4*>(K + (seq + idx[j]) * HD + h * RO_DH + c * 8);
    *reinterpret_cast<uint4*>(ks + j * RO_KP + c * 8) = v;
  }
  for (int e = tid; e < nj * 8 * 8; e += 256) {
    const int j = (e >> 3) * 2, c = e & 7;  // rows j, j + 1, channels 8c .. 8c + 7
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (j < nvis)
      v0 = *reinterpret_cast<const uint4*>(V + (seq + idx[j]) * HD + h * RO_DH + c * 8);
    if (j + 1 < nvis)
      v1 = *reinterpret_cast<const uint4*>(V + (seq + idx[j + 1]) * HD + h * RO_DH + c * 8);
    const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, bb[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint32_t*>(vt + (c * 8 + 2 * q) * RO_VP + j) =
          (a[q] & 0xFFFFu) | (bb[q] << 16);
      *reinterpret_cast<uint32_t*>(vt + (c * 8 + 2 * q + 1) * RO_VP + j) =
          (a[q] >> 16) | (bb[q] & 0xFFFF0000u);
    }
  }
  __syncthreads();

  // 3. S^T[j][token] for the wave's 16 tokens
  f32x4 sc[RO_CAP / 16];
#pragma unroll
  for (int jt = 0; jt < RO_CAP / 16; ++jt) {
    sc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (jt < nj) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 ka =
            *reinterpret_cast<const uint4*>(ks + (16 * jt + col) * RO_KP + 32 * s + 8 * grp);
        sc[jt] = mfma16x16x32(ka, qf[s], sc[jt]);
      }
    }
  }
  // masked softmax over j for token `col`: lanes col, col+16, col+32, col+48 share a token
  float mx = -INFINITY;
#pragma unroll
  for (int jt = 0; jt < RO_CAP / 16; ++jt)
    if (jt < nj) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * jt + 4 * grp + i;
        const float x = j < nvis ? sc[jt][i] * scale : -INFINITY;
        sc[jt][i] = x;
        mx = fmaxf(mx, x);
      }
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sum = 0.f;
  uint2 pw[RO_CAP / 16];
#pragma unroll
  for (int jt = 0; jt < RO_CAP / 16; ++jt) {
    pw[jt] = make_uint2(0, 0);
    if (jt < nj) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __expf(sc[jt][i] - mx);  // exp(-inf) = 0
      pw[jt] = make_uint2(pack2bf(p[0], p[1]), pack2bf(p[2], p[3]));
      sum += lo_bf(pw[jt].x) + hi_bf(pw[jt].x) + lo_bf(pw[jt].y) + hi_bf(pw[jt].y);
    }
  }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);

  // 4. O[token][d] = sum_j P[token][j] V[j][d]; lane l ends with d = 16 dt + l % 16 and tokens
  // 4 (l / 16) + i
  f32x4 o[RO_DH / 16];
#pragma unroll
  for (int dt = 0; dt < RO_DH / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < RO_CAP / 16; ++jt)
    if (jt < nj) {
#pragma unroll
      for (int dt = 0; dt < RO_DH / 16; ++dt) {
        const uint2 vb =
            *reinterpret_cast<const uint2*>(vt + (16 * dt + col) * RO_VP + 16 * jt + 4 * grp);
        o[dt] = mfma16x16x16(pw[jt], vb, o[dt]);
      }
    }
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv[i] = 1.f / __shfl(sum, 4 * grp + i);
#pragma unroll
  for (int dt = 0; dt < RO_DH / 16; ++dt) {
    const int d = h * RO_DH + 16 * dt + col;
    const float g = fminf(fmaxf(alpha[d], 0.f), 1.f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long e = (seq + tok + 4 * grp + i) * HD + d;
      st_elem(out, size_t(e), base[dt][i] + g * (o[dt][i] * inv[i]));
    }
  }
}

}  // namespace

hipError_t cache_readout(const ReadoutArgs& a) {
  const dim3 grid(unsigned(a.T / RO_TOK), unsigned(a.H), unsigned(a.B));
  const auto* Q = static_cast<const uint16_t*>(a.Q);
  const auto* K = static_cast<const uint16_t*>(a.K);
  const auto* V = static_cast<const uint16_t*>(a.V);
  if (a.out_bf16)
    hipLaunchKernelGGL((k_cache_readout<uint16_t>), grid, dim3(256), 0, a.stream, Q, K, V,
                       a.routed, static_cast<const uint16_t*>(a.ttt),
                       static_cast<uint16_t*>(a.out), a.alpha, a.T, a.H, a.chunk, a.cap,
                       a.scale);
  else
    hipLaunchKernelGGL((k_cache_readout<float>), grid, dim3(256), 0, a.stream, Q, K, V,
                       a.routed, static_cast<const float*>(a.ttt), static_cast<float*>(a.out),
                       a.alpha, a.T, a.H, a.chunk, a.cap, a.scale);
  return hipGetLastError();
}

}  // namespace ttt
