// SR-TTT surprisal routing ("SR-TTT: Surprisal-Aware Residual Test-Time Training", gist.science,
// arXiv 2603.06642, section 2.1 Surprisal Filter and Residual Cache; FIFO-like eviction from
// section 5). One 1024-thread workgroup per sequence:
//   1. L_t = sum_h loss[t, h] in fp32, head order, into LDS;
//   2. per routing chunk (one wave each): nearest-rank percentile by rank counting, and the
//      chunk mean as an fp64 pairwise sum (adjacent pairs level by level, zero padding to a power
//      of two: in-lane levels first, then across lanes with the same pairing, tree64);
//   3. one thread runs the tau recurrence tau = fl32(fl32(ema*tau) + fl32(fl32(1-ema)*p)) with
//      explicit single roundings (no fused multiply-add) and the condition mean >= ratio*tau in
//      fp64;
//   4. flags L_t > tau_c, compaction in token order with wave ballots and a segment prefix;
//   5. the newest `capacity` routed tokens go to slot (rank % capacity), and their key/value rows
//      are copied with 16-byte moves; empty slots get index -1 and zero rows.
// The copy is the bulk of the traffic, so a sequence gets several workgroups (gridDim.y
// slices): each recomputes the sequence's decisions (they are deterministic, and cheap next to
// the copy), slice 0 writes the per-sequence outputs, and slice y copies cache slots
// [y * cap / slices, (y + 1) * cap / slices).
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int RT_THREADS = 1024;
constexpr int RT_MAX_T = 8192;
constexpr int RT_MAX_CAP = 4096;
constexpr int RT_MAX_NC = 1024;  // routing chunks per sequence

template <int Q>
__device__ __forceinline__ double lane_tree(const float* x, int n, int l) {
  double a[Q];
#pragma unroll
  for (int e = 0; e < Q; ++e) {
    const int i = l * Q + e;
    a[e] = i < n ? double(x[i]) : 0.0;
  }
#pragma unroll
  for (int w = Q; w > 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < w / 2; ++e) a[e] = a[2 * e] + a[2 * e + 1];
  return a[0];
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  const uint2 r = make_uint2(
      uint32_t(__builtin_amdgcn_update_dpp(0, int(u.x), CTRL, 0xF, 0xF, false)),
      uint32_t(__builtin_amdgcn_update_dpp(0, int(u.y), CTRL, 0xF, 0xF, false)));
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(double, make_uint2(uint32_t(__builtin_amdgcn_readlane(int(u.x), l)),
                                               uint32_t(__builtin_amdgcn_readlane(int(u.y), l))));
}
// Pairwise tree over the 64 lanes' values, adjacent pairs level by level (lane 0 with 1, lanes
// 0-1 with 2-3, ...). Levels 1-2 swap within quads, so every lane holds its quad's sum; the
// half-row mirror (lane i with 7 - i) then pairs quad 0 with quad 1 of each 8 lanes, and the row
// mirror (i with 15 - i) the two halves of each 16-lane row: at each level both operands are the
// two adjacent sub-sums (their order does not matter: addition commutes exactly). Levels 5-6
// combine the four rows. The result is wave-uniform.
__device__ __forceinline__ double tree64(double s) {
  s = s + dpp_d<0xB1>(s);   // quad_perm [1, 0, 3, 2]: lane i with i ^ 1
  s = s + dpp_d<0x4E>(s);   // quad_perm [2, 3, 0, 1]: lane i with i ^ 2
  s = s + dpp_d<0x141>(s);  // row_half_mirror
  s = s + dpp_d<0x140>(s);  // row_mirror
  return (readlane_d(s, 0) + readlane_d(s, 16)) + (readlane_d(s, 32) + readlane_d(s, 48));
}

__global__ __launch_bounds__(RT_THREADS) void k_route(
    const float* __restrict__ loss, const uint4* __restrict__ K, const uint4* __restrict__ V,
    int row16, int T, int H, int chunk, int kq, float pct, float ema, float ratio, int cap,
    float* tau_out, uint8_t* mask, int* idx, uint4* ck, uint4* cv, int* count, int* total) {
  // Every rounding on the decision path is a single IEEE operation: HIP contracts a*b+c into an
  // fma by default, which would change tau in its last bit. (The file is also built with
  // -ffp-contract=off.)
#pragma clang fp contract(off)
  __shared__ float Ls[RT_MAX_T];
  __shared__ float taus[RT_MAX_NC];
  __shared__ float pcs[RT_MAX_NC];
  __shared__ double means[RT_MAX_NC];
  __shared__ uint8_t oks[RT_MAX_NC];
  __shared__ int slot_tok[RT_MAX_CAP];
  __shared__ int segcnt[RT_MAX_T / 64 + 1];
  (void)pct;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slice = blockIdx.y, nslice = gridDim.y;
  const bool lead = slice == 0;  // writes the per-sequence outputs
  const int nwaves = RT_THREADS / 64;
  const int nc = T / chunk;

  // 1. per-token loss, fp32 sum in head order (rows read as 16-byte vectors when they allow)
  if (H % 4 == 0) {
    for (int t = tid; t < T; t += RT_THREADS) {
      const float4* p = reinterpret_cast<const float4*>(loss + (long(b) * T + t) * H);
      float s = 0.f;
      for (int h4 = 0; h4 < H / 4; ++h4) {
        const float4 v = p[h4];
        s = s + v.x;
        s = s + v.y;
        s = s + v.z;
        s = s + v.w;
      }
      Ls[t] = s;
    }
  } else {
    for (int t = tid; t < T; t += RT_THREADS) {
      const float* p = loss + (long(b) * T + t) * H;
      float s = 0.f;
      for (int h = 0; h < H; ++h) s = s + p[h];
      Ls[t] = s;
    }
  }
  for (int s = tid; s < cap; s += RT_THREADS) slot_tok[s] = -1;
  __syncthreads();

  // 2. percentile and mean per chunk
  int m = 64;
  while (m < chunk) m <<= 1;
  const int q = m / 64;  // values per lane in the pairwise tree
  for (int c = wave; c < nc; c += nwaves) {
    const float* x = Ls + c * chunk;
    if (chunk <= 64) {
      // lane i holds value i; the others come from the lanes' registers one by one
      const float v = lane < chunk ? x[lane] : 0.f;
      int less = 0, leq = 0;
      for (int j = 0; j < chunk; ++j) {
        const float xj =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
        less += xj < v;
        leq += xj <= v;
      }
      if (lane < chunk && less < kq && kq <= leq) pcs[c] = v;  // all writers store the same
    } else {
      for (int i = lane; i < chunk; i += 64) {
        const float v = x[i];
        int less = 0, leq = 0;
        for (int j = 0; j < chunk; ++j) {
          less += x[j] < v;
          leq += x[j] <= v;
        }
        if (less < kq && kq <= leq) pcs[c] = v;  // every writer stores the same value
      }
    }
    double s;
    switch (q) {
      case 1: s = lane_tree<1>(x, chunk, lane); break;
      case 2: s = lane_tree<2>(x, chunk, lane); break;
      case 4: s = lane_tree<4>(x, chunk, lane); break;
      case 8: s = lane_tree<8>(x, chunk, lane); break;
      default: s = lane_tree<16>(x, chunk, lane); break;
    }
    s = tree64(s);
    if (lane == 0) means[c] = s / double(chunk);
  }
  __syncthreads();

  // 3. threshold recurrence and the chunk condition. Up to 64 chunks: wave 0, lane c holding
  //    chunk c's percentile and mean; the recurrence steps through the lanes with readlane (the
  //    same two-rounding fp32 operations), and each lane finishes its own chunk.
  if (nc <= 64) {
    if (wave == 0) {
      const float pv = lane < nc ? pcs[lane] : 0.f;
      const float w = 1.0f - ema;
      float tau = 0.f, mine = 0.f;
      for (int c = 0; c < nc; ++c) {
        const float p = __builtin_bit_cast(float,
                                           __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), c));
        const float a = ema * tau;
        const float bb = w * p;
        tau = c == 0 ? p : a + bb;
        mine = lane == c ? tau : mine;
      }
      if (lane < nc) {
        taus[lane] = mine;
        const double thr = double(ratio) * double(mine);
        oks[lane] = means[lane] >= thr ? 1 : 0;
        if (tau_out && lead) tau_out[long(b) * nc + lane] = mine;
      }
    }
  } else if (tid == 0) {
    const float w = 1.0f - ema;
    float tau = 0.f;
    for (int c = 0; c < nc; ++c) {
      const float p = pcs[c];
      const float a = ema * tau;
      const float bb = w * p;
      tau = c == 0 ? p : a + bb;
      taus[c] = tau;
      const double thr = double(ratio) * double(tau);
      oks[c] = means[c] >= thr ? 1 : 0;
      if (tau_out && lead) tau_out[long(b) * nc + c] = tau;
    }
  }
  __syncthreads();

  // 4. flags and token-order ranks
  const int nseg = (T + 63) / 64;
  for (int sg = wave; sg < nseg; sg += nwaves) {
    const int t = sg * 64 + lane;
    bool f = false;
    if (t < T) {
      const int c = t / chunk;
      f = oks[c] && Ls[t] > taus[c];
      if (mask && lead) mask[long(b) * T + t] = f ? 1 : 0;
    }
    const unsigned long long bal = __ballot(f);
    if (lane == 0) segcnt[sg] = __popcll(bal);
  }
  __syncthreads();
  // exclusive prefix of the segment counts: wave 0 scans 64 segments at a time
  if (wave == 0) {
    int carry = 0;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
      const int sg = s0 + lane;
      const int c = sg < nseg ? segcnt[sg] : 0;
      int inc = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int up = __shfl_up(inc, o);
        if (lane >= o) inc += up;
      }
      if (sg < nseg) segcnt[sg] = carry + inc - c;
      carry += __shfl(inc, 63);
    }
    if (lane == 0) segcnt[nseg] = carry;
  }
  __syncthreads();
  const int R = segcnt[nseg];
  for (int sg = wave; sg < nseg; sg += nwaves) {
    const int t = sg * 64 + lane;
    bool f = false;
    if (t < T) {
      const int c = t / chunk;
      f = oks[c] && Ls[t] > taus[c];
    }
    const unsigned long long bal = __ballot(f);
    const int r = segcnt[sg] + __popcll(bal & ((1ull << lane) - 1ull));
    if (f && r >= R - cap) slot_tok[r % cap] = t;
  }
  __syncthreads();

  // 5. cache contents: this slice's slots
  if (lead) {
    for (int s = tid; s < cap; s += RT_THREADS) idx[long(b) * cap + s] = slot_tok[s];
    if (tid == 0) {
      count[b] = R < cap ? R : cap;
      total[b] = R;
    }
  }
  if (ck || cv) {
    const int s0 = int(long(slice) * cap / nslice), s1 = int(long(slice + 1) * cap / nslice);
    const long n = long(s1 - s0) * row16;
    for (long i = tid; i < n; i += RT_THREADS) {
      const int s = s0 + int(i / row16), c = int(i % row16);
      const int t = slot_tok[s];
      const long dst = (long(b) * cap + s) * row16 + c;
      const long src = (long(b) * T + t) * row16 + c;
      if (ck) ck[dst] = t >= 0 ? K[src] : make_uint4(0, 0, 0, 0);
      if (cv) cv[dst] = t >= 0 ? V[src] : make_uint4(0, 0, 0, 0);
    }
  }
}

}  // namespace

hipError_t route(const RouteArgs& a) {
  const int row16 = a.H * a.dh * a.elem_bytes / 16;
  double kd = ceil(double(a.pct) * double(a.chunk));
  int kq = int(kd);
  if (kq < 1) kq = 1;
  if (kq > a.chunk) kq = a.chunk;
  // about 8 cache slots per workgroup, at most 32 workgroups per sequence
  int slices = a.capacity / 8;
  if (slices < 1) slices = 1;
  if (slices > 32) slices = 32;
  hipLaunchKernelGGL(k_route, dim3(a.B, slices), dim3(RT_THREADS), 0, a.stream, a.loss,
                     static_cast<const uint4*>(a.K), static_cast<const uint4*>(a.V), row16, a.T,
                     a.H, a.chunk, kq, a.pct, a.ema, a.ratio, a.capacity, a.tau, a.mask, a.idx,
                     static_cast<uint4*>(a.ck), static_cast<uint4*>(a.cv), a.count, a.total);
  return hipGetLastError();
}

}  // namespace ttt
