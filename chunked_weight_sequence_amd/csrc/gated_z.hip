// Gated-MLP intermediate activation ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv
// 2604.06169, section 2: the MLP passes its input through a gate projection and an up projection,
// combines them through the gate, and the result Z is what the fast-weight projection W_down
// consumes). One launch on the caller's stream:
//     Z[b][t][f] = SiLU(g) * u,   g = X[b][t] . W_gu[f],   u = X[b][t] . W_gu[d_ff + f]
// with the fused weight W_gu stored as a linear layer stores its weight ([out][in] =
// [2 d_ff][d_model], each output's weights contiguous): rows 0 .. d_ff-1 the gate projection,
// rows d_ff .. 2 d_ff-1 the up projection. fp32 accumulation, SiLU and the product in fp32, Z
// rounded once to its output type.
//
// Tile: 256 accumulator rows (the gate and up rows of 128 columns f) times 256 tokens, K =
// d_model in steps of 32 through four LDS stages, on the eight-wave ping-pong engine with both
// operands K-contiguous. The rows are gathered so that every wave holds the gate and the up sums
// of the same (f, t) in the same lane: the epilogue forms Z in registers and writes it
// token-major (the layout the chunk scan reads in place) with no LDS exchange. Z never exists in
// fp32 in memory.
#include "common.hpp"
#include "dma.hpp"
#include "engine.hpp"
#include "launch.hpp"
#include "pingpong.hpp"

namespace ttt {
namespace {

constexpr int GZ_GROUP = 4;  // tile rows per group in the XCD-local tile order
constexpr int GZ_NS = 4;     // LDS stages of 32 K each (128 KB)
constexpr int GZ_HALF = 128; // columns f per tile (their gate and up rows make 256 A rows)

// Tile order: each XCD (bid % 8) owns a block of the tile grid (tiles_m / rm by tiles_n / (8 /
// rm) when that splits evenly, else a contiguous range of the row-major order); inside it, tiles
// go down groups of GZ_GROUP tile rows column by column, so the tiles resident at once on one
// XCD share their W_gu and X panels in that XCD's L2.
__device__ __forceinline__ void gz_tile(int bid, int n_tiles, int tiles_m, int tiles_n, int rm,
                                        int& tm, int& tn) {
  int bm, bn, om, on, q;
  if (rm > 0) {
    const int rn = 8 / rm, x = bid % 8;
    q = bid / 8;
    bm = tiles_m / rm;
    bn = tiles_n / rn;
    om = (x / rn) * bm;
    on = (x % rn) * bn;
  } else {
    const int t = xcd_remap(bid, n_tiles);
    tm = t / tiles_n;
    tn = t % tiles_n;
    return;
  }
  const int gsz = GZ_GROUP * bn, g = q / gsz, r = q % gsz;
  const int first = g * GZ_GROUP, gh = min(GZ_GROUP, bm - first);
  tm = om + first + r % gh;
  tn = on + r / gh;
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// One 256 (W_gu rows) x 256 (tokens) tile on the eight-wave ping-pong engine, K in 32-wide steps.
// The A rows are gathered so that rows 128 h .. 128 h + 63 are the gate rows of columns
// f0 + 64 h .. + 63 and rows 128 h + 64 .. + 127 their up rows; the waves that own rows
// 128 h .. + 127 then hold, in accumulator blocks i and i + 4, the gate and up sums of the same
// (f, t) in the same lane. Columns f >= d_ff re-read the half's last valid row (never stored).
template <typename TOut>
__global__ __launch_bounds__(512, 1) void k_gated_z(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ Wgu,
                                                       TOut* __restrict__ Z, int T, int D, int F,
                                                       int tiles_m, int tiles_n, int rm) {
  __shared__ PPSmem<GZ_NS> sm;
  const int b = blockIdx.y, tid = threadIdx.x;
  int tm, tn;
  gz_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, rm, tm, tn);
  const int f0 = tm * GZ_HALF, t0 = tn * PP_T;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ncols = min(GZ_HALF, F - f0), nrows = min(PP_T, T - t0);
  const PPOp oa(Wgu + long(f0) * D, 128, 0, wave, lane, [&](int r) {
    const int fl = min(64 * (r / 128) + r % 64, ncols - 1);
    return long((r % 128 >= 64 ? F : 0) + fl) * D * 2;
  });
  const PPOp ob(X + long(b) * T * D + long(t0) * D, 128, PP_OPB, wave, lane,
                [&](int r) { return long(min(r, nrows - 1)) * D * 2; });
  PPAcc acc;
  pp_zero(acc);
  pp_segment<GZ_NS>(acc, oa, ob, D / PP_BK, sm, wave, lane);
  // acc[i][j][e]: A row pp_row(.., i, e), token pp_col(.., j); blocks i < 4 of a wave are gate
  // rows 64 wm + 16 i + 4 (lane / 16) + e of the tile's columns, blocks i + 4 their up rows
  const int wm = (wave >> 1) & 1;
  TOut* zb = Z + long(b) * T * F;
  if constexpr (sizeof(TOut) == 2) {
    // bf16 Z: staged in the free stage ring, stored as whole 256-byte token rows
    char* st = &sm.st[0][0];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = silu(acc[i][j][e]) * acc[i + 4][j][e];
        pp_stage_put<GZ_HALF>(st, pp_col(wave, lane, j), wm * 64 + i * 16 + 4 * (lane >> 4),
                              pack4(make_float4(z[0], z[1], z[2], z[3])));
      }
    __syncthreads();
    pp_stage_drain<GZ_HALF>(st, tid, [&](int n, int c, const uint4& v) {
      if (n < nrows && c * 8 < ncols) pp_store_nt(zb + long(t0 + n) * F + f0 + c * 8, v);
    });
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + pp_col(wave, lane, j);
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = f0 + wm * 64 + i * 16 + 4 * (lane >> 4);
      if (f >= F) continue;
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = silu(acc[i][j][e]) * acc[i + 4][j][e];
      const float4 v = make_float4(z[0], z[1], z[2], z[3]);
      if constexpr (sizeof(TOut) == 2)
        *reinterpret_cast<uint2*>(zb + long(t) * F + f) = pack4(v);
      else
        *reinterpret_cast<float4*>(zb + long(t) * F + f) = v;
    }
  }
}

// The XCD split of a tiles_m x tiles_n grid: the even split (tile rows per XCD block = tiles_m /
// rm) whose blocks are closest to square, or 0 (contiguous ranges) when none divides.
int gz_split(int tiles_m, int tiles_n) {
  int best = 0;
  double best_r = 0;
  for (int rm = 1; rm <= 8; rm *= 2) {
    const int rn = 8 / rm;
    if (tiles_m % rm || tiles_n % rn) continue;
    const double a = double(tiles_m / rm), c = double(tiles_n / rn);
    const double r = a < c ? a / c : c / a;
    if (best == 0 || r > best_r) {
      best = rm;
      best_r = r;
    }
  }
  return best;
}

}  // namespace

hipError_t gated_z(const GatedZArgs& a) {
  const int tiles_m = (a.F + GZ_HALF - 1) / GZ_HALF, tiles_n = (a.T + PP_T - 1) / PP_T;
  const int rm = gz_split(tiles_m, tiles_n);
  const dim3 grid(unsigned(tiles_m * tiles_n), unsigned(a.B));
  const auto* X = static_cast<const uint16_t*>(a.X);
  const auto* W = static_cast<const uint16_t*>(a.Wgu);
  if (a.out_bf16)
    hipLaunchKernelGGL((k_gated_z<uint16_t>), grid, dim3(512), 0, a.stream, X, W,
                       static_cast<uint16_t*>(a.Z), a.T, a.D, a.F, tiles_m, tiles_n, rm);
  else
    hipLaunchKernelGGL((k_gated_z<float>), grid, dim3(512), 0, a.stream, X, W,
                       static_cast<float*>(a.Z), a.T, a.D, a.F, tiles_m, tiles_n, rm);
  return hipGetLastError();
}

}  // namespace ttt
