// Host-side launch interface between the C ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace ttt {

// Optional per-phase timing used by ttt_chunk_scan_profile: every open()/close() pair records
// two events on the stream around a run of launches belonging to one phase.
struct PhaseClock {
  static constexpr int kPhases = 4;
  struct Seg {
    int phase;
    hipEvent_t a, b;
  };
  hipStream_t stream = nullptr;
  std::vector<Seg> segs;
  int launches[kPhases] = {0, 0, 0, 0};
  hipError_t err = hipSuccess;

  void open(int phase) {
    Seg s{phase, nullptr, nullptr};
    if (err == hipSuccess) err = hipEventCreate(&s.a);
    if (err == hipSuccess) err = hipEventCreate(&s.b);
    if (err == hipSuccess) err = hipEventRecord(s.a, stream);
    segs.push_back(s);
  }
  void close(int n_launches) {
    Seg& s = segs.back();
    if (err == hipSuccess) err = hipEventRecord(s.b, stream);
    launches[s.phase] += n_launches;
  }
  // Waits for the stream, sums the segments per phase and releases the events.
  hipError_t finish(float* ms, int* counts) {
    hipError_t e = err == hipSuccess ? hipStreamSynchronize(stream) : err;
    float acc[kPhases] = {0, 0, 0, 0};
    for (Seg& s : segs) {
      float t = 0.f;
      if (e == hipSuccess && s.a && s.b) e = hipEventElapsedTime(&t, s.a, s.b);
      acc[s.phase] += t;
      if (s.a) (void)hipEventDestroy(s.a);
      if (s.b) (void)hipEventDestroy(s.b);
    }
    segs.clear();
    for (int p = 0; p < kPhases; ++p) {
      if (ms) ms[p] = acc[p];
      if (counts) counts[p] = launches[p];
    }
    return e;
  }
};

// Document starts for the unmasked bf16 scan: bit b * n_units + u set when sequence b starts a
// new document at token u * U (the state goes back to W_0 there), where U is the reset unit of
// scan_mfma_reset_group and n_units = ceil(T / U). 1 KB, passed to the kernels by value.
constexpr int kResetBits = 8192;
struct ResetMask {
  uint32_t bits[kResetBits / 32];
};

struct ScanArgs {
  const void* Z;
  const void* V;
  bool in_bf16;
  const float* W0;
  bool w0_shared;
  void* O;
  bool out_bf16;
  float* W_final;
  int B, T, F, D, C;  // batch, tokens, d_ff, d_model, chunk
  float eta;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  const ResetMask* resets = nullptr;  // bf16 path only, and only where scan_mfma_reset_group allows
  int T_stride = 0;  // tokens between consecutive sequences of Z, V and O (0: T)
};

// fp32 path: per-chunk apply then update with fp32 FMA kernels.
size_t scan_simt_workspace(int B, int T, int F, int D, int C);
hipError_t scan_simt(const ScanArgs& a, PhaseClock* clk);

// bf16 path: matrix-core kernels over groups of chunks.
size_t scan_mfma_workspace(int B, int T, int F, int D, int C);
// Group size G of the bf16 scan when it can take document starts in one batched call
// (ScanArgs::resets), else 0. It takes starts at multiples of G and, when *inside is set, also
// starts whose offset inside their group is a multiple of *tile tokens (the apply's token tiles).
// *unit = U, the token unit of ResetMask's bits (every start it takes is a multiple of U), and
// B * ceil(T / U) <= kResetBits.
int scan_mfma_reset_group(int B, int T, int F, int D, int C, bool* inside, int* tile, int* unit);
// Group size G (tokens) of the bf16 scan's schedule for these sizes.
int scan_mfma_group(int B, int T, int F, int D, int C);
hipError_t scan_mfma(const ScanArgs& a, PhaseClock* clk);
// Test-only schedule overrides (process-wide): group tokens (<= 0: default), token split (0: off,
// else default), polls of the hand-over wait (< 0: default).
void scan_mfma_test_overrides(int group_tokens, int split, int spin_limit);
// Byte offset in the bf16 scan's workspace of the word that counts hand-over waits that ran out.
size_t scan_mfma_timeout_word(int B, int T, int F, int D, int C);
// Device address of this device's copy of the scan's static scratch array (TTT_SCAN_SCRATCH_BYTES),
// resolved once per device; `device` must be the current device.
hipError_t scan_scratch(int device, void** ptr);
// dst[0] = src ? *src : 0 (4 bytes), enqueued on the stream.
hipError_t scan_mfma_copy_word(const void* src, unsigned* dst, hipStream_t stream);

struct LinearArgs {
  const void* Q;
  const void* K;
  const void* V;
  bool in_bf16;
  const float* W0;
  void* O;
  bool out_bf16;
  float* W_final;
  float* loss;
  int B, T, H, dh, b;
  float eta;
  hipStream_t stream;
};
bool linear_mfma_supported(const LinearArgs& a);
bool linear_chunk_supported(const LinearArgs& a);  // linear_chunk.hip
hipError_t linear_chunk(const LinearArgs& a);
hipError_t linear_mfma(const LinearArgs& a);
hipError_t linear_simt(const LinearArgs& a);
void linear_dma_b32(const LinearArgs& a);  // the b = 32 launch (linear_b32.hip)

struct RouteArgs {
  const float* loss;
  const void* K;
  const void* V;
  int elem_bytes;
  int B, T, H, dh, chunk;
  float pct, ema, ratio;
  int capacity;
  float* tau;
  uint8_t* mask;
  int* idx;
  void* ck;
  void* cv;
  int* count;
  int* total;
  hipStream_t stream;
};
hipError_t route(const RouteArgs& a);


// LM-aligned target producer: A = conv(X0) into the workspace, then V_hat = A W_target.
struct TargetArgs {
  const void* X0;      // [B, T, Din] bf16
  const float* conv_w; // [width, Din]
  int width;
  const void* Wt;      // [Din, Dout] bf16
  void* Vh;            // [B, T, Dout]
  bool out_bf16;
  int B, T, Din, Dout, chunk;
  void* ws;            // [B, T, Din] bf16, then W_target transposed [Dout, Din] bf16
  hipStream_t stream;
};
hipError_t lm_target(const TargetArgs& a);
size_t lm_target_workspace(int B, int T, int Din, int Dout);

// Gated-MLP activation Z = SiLU(X W_gate) * (X W_up), W_gu = [W_gate | W_up].
struct GatedZArgs {
  const void* X;    // [B, T, D] bf16
  const void* Wgu;  // [D, 2F] bf16
  void* Z;          // [B, T, F]
  bool out_bf16;
  int B, T, D, F;
  hipStream_t stream;
};
hipError_t gated_z(const GatedZArgs& a);

// Residual-cache readout: out = ttt + clamp(alpha, 0, 1) * attention over the visible cache.
struct ReadoutArgs {
  const void *Q, *K, *V;        // [B, T, H * 64] bf16
  const uint8_t* routed;        // [B, T]
  const void* ttt;              // [B, T, H * 64]
  void* out;                    // [B, T, H * 64], may be ttt itself
  const float* alpha;           // [H * 64]
  bool out_bf16;
  int B, T, H, chunk, cap;
  float scale;
  hipStream_t stream;
};
hipError_t cache_readout(const ReadoutArgs& a);

// Per-chunk update clipping: writes V' = factor(chunk) * V at the start of `ws` (then the norm
// slots and the factors), factor = min(1, tau / ||eta V_i^T Z_i||_F).
struct ClipArgs {
  const void *Z, *V;  // [B, T, F], [B, T, D]
  bool in_bf16;
  int B, T, F, D, C;
  float eta, tau;
  void* ws;           // clip_workspace(...) bytes
  hipStream_t stream;
};
size_t clip_workspace(int B, int T, int D, int C, bool in_bf16);
hipError_t clip_targets(const ClipArgs& a);

}  // namespace ttt
