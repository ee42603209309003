// SR-TTT surprisal routing ("SR-TTT: Surprisal-Aware Residual Test-Time Training", gist.science,
// arXiv 2603.06642, section 2.1 Surprisal Filter and Residual Cache; FIFO-like eviction from
// section 5). One 1024-thread workgroup per sequence:
//   1. L_t = sum_h loss[t, h] in fp32, head order, into LDS;
//   2. per routing chunk (one wave each): nearest-rank percentile (up to 64 values: repeated wave
//      maxima when it lies within RT_TOP values of the top, else rank counting; past 64 values a
//      radix select over 8-bit digits of the value's order-preserving key, where counting would
//      take chunk^2 compares), and the
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
constexpr int RT_TOP = 8;  // percentiles within this many values of the top: by repeated maxima

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

// Order-preserving map of an fp32 value to an unsigned key (negative values reversed below the
// positive ones), and its inverse.
__device__ __forceinline__ uint32_t rt_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float rt_unkey(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Maximum over the 64 lanes (every lane ends with it): the row steps of a DPP reduction, then the
// four rows by lane reads. fmaxf returns one of its operands, so the result is one lane's value.
template <int CTRL>
__device__ __forceinline__ float dpp_fl(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_fl<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_fl<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_fl<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_fl<0x140>(x));  // row_mirror
  const auto rl = [&](int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  };
  return fmaxf(fmaxf(rl(0), rl(16)), fmaxf(rl(32), rl(48)));
}

template <bool WINDOWED>
__global__ __launch_bounds__(RT_THREADS) void k_route(
    const float* __restrict__ loss, const uint4* __restrict__ K, const uint4* __restrict__ V,
    int row16, int T, int H, int chunk, int kq, float pct, float ema, float ratio, int cap,
    float* tau_out, uint8_t* mask, int* idx, uint4* ck, uint4* cv, int* count, int* total) {
  // Every rounding on the decision path is a single IEEE operation: HIP contracts a*b+c into an
  // fma by default, which would change tau in its last bit. (The file is also built with
  // -ffp-contract=off.)
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float Ls[RT_MAX_T];
  __shared__ float taus[RT_MAX_NC];
  __shared__ float pcs[RT_MAX_NC];
  __shared__ double means[RT_MAX_NC];
  __shared__ uint8_t oks[RT_MAX_NC];
  __shared__ int slot_tok[RT_MAX_CAP];
  __shared__ int segcnt[RT_MAX_T / 64 + 1];
  __shared__ __attribute__((aligned(16))) int hsel[RT_THREADS / 64][256];  // radix-select bins
  (void)pct;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slice = blockIdx.y, nslice = gridDim.y;
  const bool lead = slice == 0;  // writes the per-sequence outputs
  const int nwaves = RT_THREADS / 64;
  const int nc = T / chunk;
  // The sequence is taken in windows of whole chunks that fit the LDS arrays (at most RT_MAX_T
  // tokens and RT_MAX_NC chunks); the threshold and the routed count carry from one window to
  // the next, and the ring of slots is filled in token order across them.
  const int wch = min(RT_MAX_T / chunk, RT_MAX_NC);  // chunks per window
  __shared__ float tau_carry;   // the threshold of the last chunk so far
  __shared__ int routed_carry;  // tokens routed so far
  if (WINDOWED && tid == 0) {
    tau_carry = 0.f;
    routed_carry = 0;
  }
  for (int s = tid; s < cap; s += RT_THREADS) slot_tok[s] = -1;
  // window by window (one pass over the whole sequence in the instance without windows, which
  // carries nothing in or out)
  constexpr bool single = !WINDOWED;
  int R = 0;  // tokens routed in the sequence
  int c0 = 0;
  do {
    const int ncw = WINDOWED ? min(wch, nc - c0) : nc;  // chunks in this window
    const int w0 = c0 * chunk, Tw = ncw * chunk;          // its first token and its tokens
    const float* lrow = loss + (long(b) * T + w0) * H;

    // 1. per-token loss, fp32 sum in head order. Each thread takes two tokens at a time and issues
    //    all their loads before the first add (one memory latency per pair of tokens, where a loop
    //    that added each load before issuing the next paid one per load)
    if (H % 4 == 0 && H <= 32) {
      const int H4 = H / 4;
      for (int t0 = tid; t0 < Tw; t0 += 2 * RT_THREADS) {
        const int t1 = t0 + RT_THREADS;
        const float4* p0 = reinterpret_cast<const float4*>(lrow + long(t0) * H);
        const float4* p1 = reinterpret_cast<const float4*>(lrow + long(t1 < Tw ? t1 : t0) * H);
        float4 a0[8], a1[8];
#pragma unroll
        for (int h4 = 0; h4 < 8; ++h4)
          if (h4 < H4) {
            a0[h4] = p0[h4];
            a1[h4] = p1[h4];
          }
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int h4 = 0; h4 < 8; ++h4)
          if (h4 < H4) {
            s0 = s0 + a0[h4].x;
            s0 = s0 + a0[h4].y;
            s0 = s0 + a0[h4].z;
            s0 = s0 + a0[h4].w;
            s1 = s1 + a1[h4].x;
            s1 = s1 + a1[h4].y;
            s1 = s1 + a1[h4].z;
            s1 = s1 + a1[h4].w;
          }
        Ls[t0] = s0;
        if (t1 < Tw) Ls[t1] = s1;
      }
    } else {
      for (int t = tid; t < Tw; t += RT_THREADS) {
        const float* p = lrow + long(t) * H;
        float s = 0.f;
        for (int h = 0; h < H; ++h) s = s + p[h];
        Ls[t] = s;
      }
    }
    __syncthreads();

    // 2. percentile and mean per chunk
    int m = 64;
    while (m < chunk) m <<= 1;
    const int q = m / 64;  // values per lane in the pairwise tree
    for (int c = wave; c < ncw; c += nwaves) {
      const float* x = Ls + c * chunk;
      if (chunk <= 64 && chunk - kq < RT_TOP) {
        // the kq-th smallest is the r-th largest, r = chunk - kq + 1 (the 95th percentile of 64
        // values: the 4th largest): r - 1 times the wave maximum is found and one lane holding
        // it (the lowest) drops out, then the maximum of the rest is the value. Each round
        // removes one occurrence, so ties count with their multiplicity, as in the sorted order;
        // the result is one of the inputs, the same one the rank count below selects.
        float cur = lane < chunk ? x[lane] : -__builtin_inff();
        float best = wave_max(cur);
        for (int i = 1; i < chunk - kq + 1; ++i) {
          // nonzero for any input but NaN (best is one lane's value); bit 63 keeps the count defined
          // for a chunk of NaNs, where dropping lane 63 changes nothing
          const unsigned long long hit = __ballot(cur == best) | (1ull << 63);
          if (lane == __builtin_ctzll(hit)) cur = -__builtin_inff();
          best = wave_max(cur);
        }
        if (lane == 0) pcs[c] = best;
      } else if (chunk <= 64) {
        // lane i holds value i and counts the chunk's values below it. The kq-th smallest value is
        // the largest v with fewer than kq values below it (every larger value has at least kq
        // below it), so one count and a wave maximum suffice.
        const float v = lane < chunk ? x[lane] : 0.f;
        int less = 0;
        if ((chunk & 15) == 0) {
          // four 16-byte reads in flight per step
          for (int j = 0; j < chunk; j += 16) {
            const float4* q4 = reinterpret_cast<const float4*>(x + j);
            const float4 a0 = q4[0], a1 = q4[1], a2 = q4[2], a3 = q4[3];
            const float e[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                 a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
#pragma unroll
            for (int k = 0; k < 16; ++k) less += e[k] < v ? 1 : 0;
          }
        } else {
          for (int j = 0; j < chunk; ++j) less += x[j] < v ? 1 : 0;
        }
        const float cand = (lane < chunk && less < kq) ? v : -__builtin_inff();
        const float best = wave_max(cand);
        if (lane == 0) pcs[c] = best;
      } else {
        // radix select of the kq-th smallest value: four passes over 8-bit digits of the
        // order-preserving integer key, each a histogram of the values still in range
        int* hist = &hsel[wave][0];
        uint32_t prefix = 0, pmask = 0;
        int k = kq;
        for (int shift = 24; shift >= 0; shift -= 8) {
          for (int e = lane; e < 256; e += 64) hist[e] = 0;
          __builtin_amdgcn_wave_barrier();
          for (int i = lane; i < chunk; i += 64) {
            const uint32_t u = rt_key(x[i]);
            if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
          }
          __builtin_amdgcn_wave_barrier();
          // lane l holds bins 4l .. 4l + 3; an inclusive scan of the lane sums finds the bin that
          // holds the k-th value
          const int4 hc = *reinterpret_cast<const int4*>(hist + 4 * lane);
          const int cs = hc.x + hc.y + hc.z + hc.w;
          int inc = cs;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int up = __shfl_up(inc, o);
            if (lane >= o) inc += up;
          }
          const int exc = inc - cs;
          const unsigned long long hit = __ballot(exc < k && k <= inc);
          const int hl = hit ? __builtin_ctzll(hit) : 63;  // always hit: the bins hold k values
          const int below = __shfl(exc, hl);
          const int4 hb = *reinterpret_cast<const int4*>(hist + 4 * hl);
          int kk = k - below, bin = 4 * hl;
          if (kk > hb.x) { kk -= hb.x; ++bin;
            if (kk > hb.y) { kk -= hb.y; ++bin;
              if (kk > hb.z) { kk -= hb.z; ++bin; } } }
          k = kk;
          prefix |= uint32_t(bin) << shift;
          pmask |= 0xFFu << shift;
          __builtin_amdgcn_wave_barrier();
        }
        if (lane == 0) pcs[c] = rt_unkey(prefix);
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

    // 3. threshold recurrence and the chunk condition, continuing from the previous window's
    //    last threshold. Up to 64 chunks: wave 0, lane c holding chunk c's percentile and mean;
    //    the recurrence steps through the lanes with readlane (the same two-rounding fp32
    //    operations), and each lane finishes its own chunk.
    if (ncw <= 64) {
      if (wave == 0) {
        const float pv = lane < ncw ? pcs[lane] : 0.f;
        const float w = 1.0f - ema;
        float tau = single ? 0.f : tau_carry, mine = 0.f;
        for (int c = 0; c < ncw; ++c) {
          const float p = __builtin_bit_cast(float,
                                             __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), c));
          const float a = ema * tau;
          const float bb = w * p;
          tau = c0 + c == 0 ? p : a + bb;
          mine = lane == c ? tau : mine;
        }
        if (lane < ncw) {
          taus[lane] = mine;
          const double thr = double(ratio) * double(mine);
          oks[lane] = means[lane] >= thr ? 1 : 0;
          if (tau_out && lead) tau_out[long(b) * nc + c0 + lane] = mine;
        }
        if (!single && lane == 0) tau_carry = tau;  // after every lane's read of it (in order)
      }
    } else if (tid == 0) {
      const float w = 1.0f - ema;
      float tau = single ? 0.f : tau_carry;
      for (int c = 0; c < ncw; ++c) {
        const float p = pcs[c];
        const float a = ema * tau;
        const float bb = w * p;
        tau = c0 + c == 0 ? p : a + bb;
        taus[c] = tau;
        const double thr = double(ratio) * double(tau);
        oks[c] = means[c] >= thr ? 1 : 0;
        if (tau_out && lead) tau_out[long(b) * nc + c0 + c] = tau;
      }
      if (!single) tau_carry = tau;
    }
    __syncthreads();

    // 4. flags and token-order ranks
    const int nseg = (Tw + 63) / 64;
    for (int sg = wave; sg < nseg; sg += nwaves) {
      const int t = sg * 64 + lane;
      bool f = false;
      if (t < Tw) {
        const int c = t / chunk;
        f = oks[c] && Ls[t] > taus[c];
        if (mask && lead) mask[long(b) * T + w0 + t] = f ? 1 : 0;
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
    // ranks count from the sequence start; of two tokens of this window that share a slot only
    // the newer is written (their ranks differ by at least cap), and a later window's tokens
    // overwrite an earlier window's, so the ring ends with the newest `cap` routed tokens
    const int rb = single ? 0 : routed_carry, re = rb + segcnt[nseg];
    for (int sg = wave; sg < nseg; sg += nwaves) {
      const int t = sg * 64 + lane;
      bool f = false;
      if (t < Tw) {
        const int c = t / chunk;
        f = oks[c] && Ls[t] > taus[c];
      }
      const unsigned long long bal = __ballot(f);
      const int r = rb + segcnt[sg] + __popcll(bal & ((1ull << lane) - 1ull));
      if (f && r >= re - cap) slot_tok[r % cap] = w0 + t;
    }
    R = re;
    if constexpr (WINDOWED) {
      __syncthreads();  // every read of this window's Ls, segcnt and carry is done
      if (tid == 0) routed_carry = re;
    }
  } while (WINDOWED && (c0 += wch) < nc);
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
  // sequences that fit one window take the instance without the window loop
  const bool windowed = a.T / a.chunk > std::min(RT_MAX_T / a.chunk, RT_MAX_NC);
  hipLaunchKernelGGL(windowed ? k_route<true> : k_route<false>, dim3(a.B, slices),
                     dim3(RT_THREADS), 0, a.stream, a.loss,
                     static_cast<const uint4*>(a.K), static_cast<const uint4*>(a.V), row16, a.T,
                     a.H, a.chunk, kq, a.pct, a.ema, a.ratio, a.capacity, a.tau, a.mask, a.idx,
                     static_cast<uint4*>(a.ck), static_cast<uint4*>(a.cv), a.count, a.total);
  return hipGetLastError();
}

}  // namespace ttt
