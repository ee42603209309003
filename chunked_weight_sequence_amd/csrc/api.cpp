// C ABI of libttt_mi355x: host-side validation, kernel selection and launch on the caller's
// stream. Every check runs before anything is enqueued, so a rejected call touches neither the
// device nor any output. The library never allocates device memory and never synchronises
// (except ttt_chunk_scan_profile, which is documented to).
#include <cmath>
#include <math.h>
#include <stdint.h>

#include "../../include/ttt_mi355x.h"
#include "launch.hpp"

#define TTT_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool valid_dtype(int d) { return d == TTT_F32 || d == TTT_BF16; }
size_t dsize(int d) { return d == TTT_BF16 ? 2 : 4; }

// `segments`: a bf16 workspace smaller than the full need is accepted here (the caller then
// runs the scan in segments, see scan_run); the range checked for overlaps is the one given.
ttt_status scan_check(const void* Z, const void* Vhat, ttt_dtype in_dtype, const float* W0,
                      int w0_shared, void* O, ttt_dtype out_dtype, float* W_final, int B, int T,
                      int d_ff, int d_model, int chunk, float eta, void* ws, size_t ws_bytes,
                      size_t* need, bool segments = false) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TTT_E_DTYPE;
  if (!Z || !Vhat || !W0 || !O) return TTT_E_NULL;
  if (B < 1 || T < 1 || chunk < 1 || d_ff < 16 || d_model < 16) return TTT_E_SHAPE;
  if (d_ff % 16 || d_model % 16) return TTT_E_SHAPE;
  if (T > (1 << 26) || d_ff > (1 << 20) || d_model > (1 << 20) || B > 65535) return TTT_E_SHAPE;
  if (!isfinite(eta)) return TTT_E_SHAPE;
  // The bf16 path carries the state as W / eta in the matrix-core accumulator, so a nonzero eta
  // must keep that quotient in fp32 range.
  if (in_dtype == TTT_BF16 && eta != 0.f && !(fabsf(eta) >= 1e-18f && fabsf(eta) <= 1e18f))
    return TTT_E_UNSUPPORTED;
  if (!aligned16(Z) || !aligned16(Vhat) || !aligned16(W0) || !aligned16(O) ||
      !aligned16(W_final) || !aligned16(ws))
    return TTT_E_ALIGN;
  const size_t isz = dsize(in_dtype), osz = dsize(out_dtype);
  const size_t DF = size_t(d_model) * d_ff;
  const Range rz{Z, size_t(B) * T * d_ff * isz}, rv{Vhat, size_t(B) * T * d_model * isz};
  const Range rw0{W0, (w0_shared ? 1 : size_t(B)) * DF * 4};
  const Range ro{O, size_t(B) * T * d_model * osz};
  const Range rwf{W_final, W_final ? size_t(B) * DF * 4 : 0};
  *need = in_dtype == TTT_BF16 ? ttt::scan_mfma_workspace(B, T, d_ff, d_model, chunk)
                               : ttt::scan_simt_workspace(B, T, d_ff, d_model, chunk);
  const bool seg = segments && in_dtype == TTT_BF16 && ws_bytes < *need;
  const Range rws{ws, seg ? ws_bytes : *need};
  if (overlap(ro, rz) || overlap(ro, rv) || overlap(ro, rw0) || overlap(ro, rwf))
    return TTT_E_ALIAS;
  if (overlap(rwf, rz) || overlap(rwf, rv)) return TTT_E_ALIAS;
  if (W_final && overlap(rwf, rw0)) {
    const bool inplace = static_cast<const void*>(W_final) == static_cast<const void*>(W0) &&
                         (!w0_shared || B == 1);
    if (!inplace) return TTT_E_ALIAS;
  }
  if (*need > 0) {
    if (!ws || (!seg && ws_bytes < *need)) return TTT_E_WORKSPACE;
    if (overlap(rws, rz) || overlap(rws, rv) || overlap(rws, rw0) || overlap(rws, ro) ||
        overlap(rws, rwf))
      return TTT_E_ALIAS;
  }
  return TTT_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Segments of the bf16 scan for a workspace smaller than the whole sequence needs: the longest
// run of whole groups (Ts tokens) whose own workspace, plus an fp32 state buffer of
// B x d_model x d_ff when the caller gives no W_final to carry the state in, fits.
struct SegPlan {
  int Ts = 0;
  size_t seg_bytes = 0, state_off = 0;
};
bool seg_plan(int B, int T, int F, int D, int C, bool need_state, size_t ws_bytes, SegPlan* sp) {
  const int G = ttt::scan_mfma_group(B, T, F, D, C);
  const int n_g = (T + G - 1) / G;
  const size_t state = need_state ? align256(size_t(B) * D * F * 4) : 0;
  for (int m = n_g - 1; m >= 1; --m) {
    const size_t wsb = align256(ttt::scan_mfma_workspace(B, m * G, F, D, C));
    if (wsb + state <= ws_bytes) {
      sp->Ts = m * G;
      sp->seg_bytes = wsb;
      sp->state_off = wsb;
      return true;
    }
  }
  return false;
}

size_t scan_min_workspace(int B, int T, int F, int D, int C) {
  const int G = ttt::scan_mfma_group(B, T, F, D, C);
  const size_t full = ttt::scan_mfma_workspace(B, T, F, D, C);
  if (G >= T) return full;
  const size_t one = align256(ttt::scan_mfma_workspace(B, G, F, D, C)) +
                     align256(size_t(B) * D * F * 4);
  return one < full ? one : full;
}

ttt_status scan_run(const void* Z, const void* Vhat, ttt_dtype in_dtype, const float* W0,
                    int w0_shared, void* O, ttt_dtype out_dtype, float* W_final, int B, int T,
                    int d_ff, int d_model, int chunk, float eta, void* ws, size_t ws_bytes,
                    hipStream_t stream, ttt::PhaseClock* clk) {
  size_t need = 0;
  const ttt_status st = scan_check(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T,
                                   d_ff, d_model, chunk, eta, ws, ws_bytes, &need, true);
  if (st != TTT_OK) return st;
  if (in_dtype == TTT_BF16 && ws_bytes < need) {
    // Workspace below the whole sequence's need: the scan runs over segments of whole groups,
    // each resuming from the state the previous one ended with (W0 of segment s + 1 = W_final
    // of segment s; with C dividing every segment start this is the same scan, up to the
    // rounding of the state handed across).
    SegPlan sp;
    if (!seg_plan(B, T, d_ff, d_model, chunk, W_final == nullptr, ws_bytes, &sp))
      return TTT_E_WORKSPACE;
    float* state = W_final ? W_final : reinterpret_cast<float*>(static_cast<char*>(ws) + sp.state_off);
    const size_t isz = dsize(in_dtype), osz = dsize(out_dtype);
    (void)hipGetLastError();
    for (int t0 = 0; t0 < T; t0 += sp.Ts) {
      const int Tn = T - t0 < sp.Ts ? T - t0 : sp.Ts;
      const bool first = t0 == 0, last = t0 + Tn >= T;
      ttt::ScanArgs a{static_cast<const char*>(Z) + size_t(t0) * d_ff * isz,
                      static_cast<const char*>(Vhat) + size_t(t0) * d_model * isz, true,
                      first ? W0 : state, first ? (w0_shared != 0 || B == 1) : B == 1,
                      static_cast<char*>(O) + size_t(t0) * d_model * osz, out_dtype == TTT_BF16,
                      last ? W_final : state, B, Tn, d_ff, d_model, chunk, eta, ws, sp.seg_bytes,
                      stream};
      a.T_stride = T;
      if (ttt::scan_mfma(a, clk) != hipSuccess) return TTT_E_LAUNCH;
    }
    return TTT_OK;
  }
  ttt::ScanArgs a{Z, Vhat, in_dtype == TTT_BF16, W0, w0_shared != 0 || B == 1, O,
                  out_dtype == TTT_BF16, W_final, B, T, d_ff, d_model, chunk, eta, ws,
                  ws_bytes, stream};
  (void)hipGetLastError();  // clear any stale error so it is not attributed to this call
  const hipError_t e = a.in_bf16 ? ttt::scan_mfma(a, clk) : ttt::scan_simt(a, clk);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

}  // namespace

TTT_EXPORT ttt_status ttt_chunk_scan(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                     const float* W0, int w0_shared, void* O,
                                     ttt_dtype out_dtype, float* W_final, int B, int T, int d_ff,
                                     int d_model, int chunk, float eta, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return scan_run(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T, d_ff, d_model,
                  chunk, eta, workspace, workspace_bytes, stream, nullptr);
}

TTT_EXPORT ttt_status ttt_chunk_scan_noalloc(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                             const float* W0, int w0_shared, void* O,
                                             ttt_dtype out_dtype, float* W_final, int B, int T,
                                             int d_ff, int d_model, int chunk, float eta,
                                             hipStream_t stream) {
  // host-only checks first (a size beyond the static scratch is refused before any HIP call)
  size_t need = 0;
  const ttt_status st = scan_check(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T,
                                   d_ff, d_model, chunk, eta, nullptr, 0, &need);
  if (st != TTT_OK && st != TTT_E_WORKSPACE) return st;
  if (need > TTT_SCAN_SCRATCH_BYTES) {
    // too large for one pass in the scratch: segments of whole groups, if one fits
    SegPlan sp;
    if (in_dtype != TTT_BF16 || !seg_plan(B, T, d_ff, d_model, chunk, W_final == nullptr,
                                          TTT_SCAN_SCRATCH_BYTES, &sp))
      return TTT_E_WORKSPACE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TTT_E_LAUNCH;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return TTT_E_LAUNCH;
    if (sdev != dev) return TTT_E_UNSUPPORTED;
  }
  void* ws = nullptr;
  if (need > 0 && ttt::scan_scratch(dev, &ws) != hipSuccess) return TTT_E_LAUNCH;
  return scan_run(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T, d_ff, d_model,
                  chunk, eta, ws, need > 0 ? size_t(TTT_SCAN_SCRATCH_BYTES) : 0, stream, nullptr);
}

TTT_EXPORT size_t ttt_chunk_scan_workspace(int B, int T, int d_ff, int d_model, int chunk,
                                           ttt_dtype in_dtype) {
  if (!valid_dtype(in_dtype) || B < 1 || T < 1 || chunk < 1 || d_ff < 16 || d_model < 16 ||
      d_ff % 16 || d_model % 16 || T > (1 << 26) || d_ff > (1 << 20) || d_model > (1 << 20) ||
      B > 65535)
    return 0;
  return in_dtype == TTT_BF16 ? ttt::scan_mfma_workspace(B, T, d_ff, d_model, chunk)
                              : ttt::scan_simt_workspace(B, T, d_ff, d_model, chunk);
}

TTT_EXPORT ttt_status ttt_chunk_scan_profile(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                             const float* W0, int w0_shared, void* O,
                                             ttt_dtype out_dtype, float* W_final, int B, int T,
                                             int d_ff, int d_model, int chunk, float eta,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream, float* phase_ms,
                                             int* phase_launches) {
  ttt::PhaseClock clk;
  clk.stream = stream;
  const ttt_status st = scan_run(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T,
                                 d_ff, d_model, chunk, eta, workspace, workspace_bytes, stream,
                                 &clk);
  const hipError_t e = clk.finish(phase_ms, phase_launches);
  if (st != TTT_OK) return st;
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

TTT_EXPORT size_t ttt_chunk_scan_workspace_min(int B, int T, int d_ff, int d_model, int chunk,
                                               ttt_dtype in_dtype) {
  const size_t full = ttt_chunk_scan_workspace(B, T, d_ff, d_model, chunk, in_dtype);
  if (full == 0 || in_dtype != TTT_BF16) return full;
  return scan_min_workspace(B, T, d_ff, d_model, chunk);
}

TTT_EXPORT ttt_status ttt_chunk_scan_handover_timeouts(int B, int T, int d_ff, int d_model,
                                                       int chunk, ttt_dtype in_dtype,
                                                       const void* workspace,
                                                       size_t workspace_bytes, unsigned* count,
                                                       hipStream_t stream) {
  if (!valid_dtype(in_dtype)) return TTT_E_DTYPE;
  if (!count) return TTT_E_NULL;
  const size_t need = ttt_chunk_scan_workspace(B, T, d_ff, d_model, chunk, in_dtype);
  if (need == 0 && in_dtype == TTT_BF16) return TTT_E_SHAPE;
  if (!aligned16(count) || !aligned16(workspace)) return TTT_E_ALIGN;
  const void* src = nullptr;
  if (in_dtype == TTT_BF16) {
    if (!workspace || workspace_bytes < need) return TTT_E_WORKSPACE;
    src = static_cast<const char*>(workspace) +
          ttt::scan_mfma_timeout_word(B, T, d_ff, d_model, chunk);
  }
  if (overlap(Range{count, 4}, Range{workspace, need})) return TTT_E_ALIAS;
  (void)hipGetLastError();
  return ttt::scan_mfma_copy_word(src, count, stream) == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

TTT_EXPORT ttt_status ttt_scan_test_overrides(int group_tokens, int token_split,
                                              int spin_limit) {
  ttt::scan_mfma_test_overrides(group_tokens, token_split, spin_limit);
  return TTT_OK;
}

namespace {
bool clip_on(float tau) { return tau > 0.f && std::isfinite(tau); }

// Workspace of ttt_chunk_scan_docs: the scan's own, then (clipping) the scaled targets, the norm
// slots and the factors.
size_t docs_workspace(int B, int T, int d_ff, int d_model, int chunk, ttt_dtype in_dtype,
                      float tau, size_t* scan_part) {
  const size_t sc = in_dtype == TTT_BF16 ? ttt::scan_mfma_workspace(B, T, d_ff, d_model, chunk)
                                         : ttt::scan_simt_workspace(B, T, d_ff, d_model, chunk);
  *scan_part = (sc + 255) & ~size_t(255);
  return *scan_part +
         (clip_on(tau) ? ttt::clip_workspace(B, T, d_model, chunk, in_dtype == TTT_BF16) : 0);
}
}  // namespace

TTT_EXPORT size_t ttt_chunk_scan_docs_workspace(int B, int T, int d_ff, int d_model, int chunk,
                                                ttt_dtype in_dtype, float clip_tau) {
  if (!valid_dtype(in_dtype) || B < 1 || T < 1 || chunk < 1 || d_ff < 16 || d_model < 16 ||
      d_ff % 16 || d_model % 16 || T > (1 << 26) || d_ff > (1 << 20) || d_model > (1 << 20) ||
      B > 65535 || std::isnan(clip_tau))
    return 0;
  size_t part = 0;
  return docs_workspace(B, T, d_ff, d_model, chunk, in_dtype, clip_tau, &part);
}

TTT_EXPORT ttt_status ttt_chunk_scan_docs(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                          const float* W0, int w0_shared, void* O,
                                          ttt_dtype out_dtype, float* W_final, int B, int T,
                                          int d_ff, int d_model, int chunk, float eta,
                                          const int* doc_starts, const int* doc_counts,
                                          float clip_tau, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  size_t scan_need = 0;
  const ttt_status st = scan_check(Z, Vhat, in_dtype, W0, w0_shared, O, out_dtype, W_final, B, T,
                                   d_ff, d_model, chunk, eta, workspace, workspace_bytes,
                                   &scan_need);
  if (st != TTT_OK) return st;
  if (std::isnan(clip_tau)) return TTT_E_SHAPE;
  // document starts: per sequence, strictly increasing multiples of chunk inside (0, T)
  if (doc_counts) {
    if (!doc_starts) {
      for (int b = 0; b < B; ++b)
        if (doc_counts[b] != 0) return TTT_E_NULL;
    }
    long k = 0;
    for (int b = 0; b < B; ++b) {
      if (doc_counts[b] < 0 || doc_counts[b] > T) return TTT_E_SHAPE;
      int prev = 0;
      for (int i = 0; i < doc_counts[b]; ++i, ++k) {
        const int s = doc_starts[k];
        if (s <= prev || s >= T || s % chunk) return TTT_E_SHAPE;
        prev = s;
      }
    }
  }
  size_t scan_part = 0;
  const size_t need =
      docs_workspace(B, T, d_ff, d_model, chunk, in_dtype, clip_tau, &scan_part);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TTT_E_WORKSPACE;
    const size_t isz = dsize(in_dtype), DF = size_t(d_model) * d_ff;
    const Range rws{workspace, need}, rz{Z, size_t(B) * T * d_ff * isz},
        rv{Vhat, size_t(B) * T * d_model * isz}, rw0{W0, (w0_shared ? 1 : size_t(B)) * DF * 4},
        ro{O, size_t(B) * T * d_model * dsize(out_dtype)},
        rwf{W_final, W_final ? size_t(B) * DF * 4 : 0};
    for (Range r : {rz, rv, rw0, ro, rwf})
      if (overlap(rws, r)) return TTT_E_ALIAS;
  }
  const bool bf = in_dtype == TTT_BF16;
  (void)hipGetLastError();
  const void* Vsrc = Vhat;
  if (clip_on(clip_tau) && eta != 0.f) {
    ttt::ClipArgs c{Z, Vhat, bf, B, T, d_ff, d_model, chunk, eta, clip_tau,
                    static_cast<char*>(workspace) + scan_part, stream};
    if (ttt::clip_targets(c) != hipSuccess) return TTT_E_LAUNCH;
    Vsrc = static_cast<char*>(workspace) + scan_part;  // the scaled targets
  }
  auto launch = [&](const ttt::ScanArgs& a) {
    return bf ? ttt::scan_mfma(a, nullptr) : ttt::scan_simt(a, nullptr);
  };
  bool any_doc = false;
  if (doc_counts)
    for (int b = 0; b < B; ++b) any_doc = any_doc || doc_counts[b] > 0;
  if (!any_doc) {
    ttt::ScanArgs a{Z, Vsrc, bf, W0, w0_shared != 0 || B == 1, O, out_dtype == TTT_BF16,
                    W_final, B, T, d_ff, d_model, chunk, eta, workspace, scan_part, stream};
    return launch(a) == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
  }
  // Documents that start on the bf16 scan's group boundaries, or inside a group on an edge of
  // the apply's token tiles: one batched scan whose state chain goes back to W0 at each start.
  // Starts on group boundaries give the bits of separate scans of the documents; a start inside
  // a group gives the document other group edges than a separate scan would (results within
  // rounding of it).
  if (bf) {
    bool inside = false;
    int tile = 0, unit = 1;
    const int G = ttt::scan_mfma_reset_group(B, T, d_ff, d_model, chunk, &inside, &tile, &unit);
    bool aligned = G > 0;
    long k = 0;
    for (int b = 0; b < B && aligned; ++b) {
      for (int i = 0; i < doc_counts[b]; ++i) {
        const int off = doc_starts[k + i] % G;
        aligned = aligned && (off == 0 || (inside && off % tile == 0));
      }
      k += doc_counts[b];
    }
    if (aligned) {
      const int n_units = (T + unit - 1) / unit;
      ttt::ResetMask mask{};
      k = 0;
      for (int b = 0; b < B; ++b) {
        for (int i = 0; i < doc_counts[b]; ++i) {
          const int bit = b * n_units + doc_starts[k + i] / unit;
          mask.bits[bit >> 5] |= 1u << (bit & 31);
        }
        k += doc_counts[b];
      }
      ttt::ScanArgs a{Z, Vsrc, bf, W0, w0_shared != 0 || B == 1, O, out_dtype == TTT_BF16,
                      W_final, B, T, d_ff, d_model, chunk, eta, workspace, scan_part, stream,
                      &mask};
      return launch(a) == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
    }
  }
  // otherwise every document is an independent scan from W0; only a sequence's last one sets
  // W_final
  const size_t isz = dsize(in_dtype), osz = dsize(out_dtype);
  const size_t DF = size_t(d_model) * d_ff;
  long k = 0;
  for (int b = 0; b < B; ++b) {
    const int n = doc_counts[b];
    for (int i = 0; i <= n; ++i) {
      const int s = i == 0 ? 0 : doc_starts[k + i - 1];
      const int e = i == n ? T : doc_starts[k + i];
      const size_t row = size_t(b) * T + s;
      ttt::ScanArgs a{static_cast<const char*>(Z) + row * d_ff * isz,
                      static_cast<const char*>(Vsrc) + row * d_model * isz, bf,
                      W0 + (w0_shared ? 0 : size_t(b) * DF), true,
                      static_cast<char*>(O) + row * d_model * osz, out_dtype == TTT_BF16,
                      i == n && W_final ? W_final + size_t(b) * DF : nullptr, 1, e - s, d_ff,
                      d_model, chunk, eta, workspace, scan_part, stream};
      if (launch(a) != hipSuccess) return TTT_E_LAUNCH;
    }
    k += n;
  }
  return TTT_OK;
}

TTT_EXPORT ttt_status ttt_linear_minibatch(const void* Q, const void* K, const void* V,
                                           ttt_dtype in_dtype, const float* W0, void* O,
                                           ttt_dtype out_dtype, float* W_final, float* loss,
                                           int B, int T, int H, int dh, int minibatch, float eta,
                                           hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TTT_E_DTYPE;
  if (!Q || !K || !V || !O) return TTT_E_NULL;
  if (B < 1 || T < 1 || H < 1 || dh < 1 || minibatch < 1 || T % minibatch) return TTT_E_SHAPE;
  if (T > (1 << 26) || B > 65535 || H > 4096 || size_t(B) * H > 65535u * 1024u)
    return TTT_E_SHAPE;
  if (!isfinite(eta)) return TTT_E_SHAPE;
  if (dh != 64) return TTT_E_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(W0) ||
      !aligned16(W_final) || !aligned16(loss))
    return TTT_E_ALIGN;
  const size_t n = size_t(B) * T * H * dh, isz = dsize(in_dtype);
  const Range rq{Q, n * isz}, rk{K, n * isz}, rv{V, n * isz}, ro{O, n * dsize(out_dtype)};
  const size_t wbytes = size_t(B) * H * dh * dh * 4;
  const Range rw0{W0, W0 ? wbytes : 0}, rwf{W_final, W_final ? wbytes : 0};
  const Range rl{loss, loss ? size_t(B) * T * H * 4 : 0};
  for (Range r : {rq, rk, rv, rw0})
    if (overlap(ro, r) || overlap(rwf, r.p == W0 ? Range{nullptr, 0} : r) || overlap(rl, r))
      return TTT_E_ALIAS;
  if (W_final && W0 && overlap(rwf, rw0) && W_final != W0) return TTT_E_ALIAS;
  if (overlap(ro, rwf) || overlap(ro, rl) || overlap(rwf, rl)) return TTT_E_ALIAS;
  ttt::LinearArgs a{Q, K, V, in_dtype == TTT_BF16, W0, O, out_dtype == TTT_BF16, W_final, loss,
                    B, T, H, dh, minibatch, eta, stream};
  (void)hipGetLastError();
  const hipError_t e = ttt::linear_chunk_supported(a)  ? ttt::linear_chunk(a)
                       : ttt::linear_mfma_supported(a) ? ttt::linear_mfma(a)
                                                       : ttt::linear_simt(a);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

TTT_EXPORT ttt_status ttt_surprisal_route(const float* loss, const void* K, const void* V,
                                          ttt_dtype kv_dtype, int B, int T, int H, int dh,
                                          int chunk, float pct, float ema, float chunk_ratio,
                                          int capacity, float* tau, unsigned char* routed_mask,
                                          int* cache_idx, void* cache_k, void* cache_v,
                                          int* cache_count, int* routed_total,
                                          hipStream_t stream) {
  if (!valid_dtype(kv_dtype)) return TTT_E_DTYPE;
  if (!loss || !cache_idx || !cache_count || !routed_total) return TTT_E_NULL;
  if ((cache_k && !K) || (cache_v && !V)) return TTT_E_NULL;
  if (B < 1 || T < 1 || H < 1 || dh < 1 || chunk < 1 || capacity < 1) return TTT_E_SHAPE;
  if (T % chunk || chunk > 1024 || T > (1 << 22) || capacity > 4096 ||
      B > 65535)
    return TTT_E_SHAPE;
  if (!(pct > 0.f && pct <= 1.f) || !(ema >= 0.f && ema <= 1.f) || !isfinite(chunk_ratio))
    return TTT_E_SHAPE;
  const size_t esz = dsize(kv_dtype);
  if ((size_t(H) * dh * esz) % 16) return TTT_E_SHAPE;
  if (!aligned16(loss) || !aligned16(K) || !aligned16(V) || !aligned16(tau) ||
      !aligned16(routed_mask) || !aligned16(cache_idx) || !aligned16(cache_k) ||
      !aligned16(cache_v) || !aligned16(cache_count) || !aligned16(routed_total))
    return TTT_E_ALIGN;
  const size_t row = size_t(H) * dh * esz;
  const Range ins[] = {{loss, size_t(B) * T * H * 4}, {K, cache_k ? size_t(B) * T * row : 0},
                       {V, cache_v ? size_t(B) * T * row : 0}};
  const Range outs[] = {{tau, tau ? size_t(B) * (T / chunk) * 4 : 0},
                        {routed_mask, routed_mask ? size_t(B) * T : 0},
                        {cache_idx, size_t(B) * capacity * 4},
                        {cache_k, cache_k ? size_t(B) * capacity * row : 0},
                        {cache_v, cache_v ? size_t(B) * capacity * row : 0},
                        {cache_count, size_t(B) * 4},
                        {routed_total, size_t(B) * 4}};
  for (const Range& o : outs) {
    for (const Range& i : ins)
      if (overlap(o, i)) return TTT_E_ALIAS;
    for (const Range& o2 : outs)
      if (&o2 != &o && overlap(o, o2)) return TTT_E_ALIAS;
  }
  ttt::RouteArgs a{loss, K, V, int(esz), B, T, H, dh, chunk, pct, ema, chunk_ratio, capacity,
                   tau, routed_mask, cache_idx, cache_k, cache_v, cache_count, routed_total,
                   stream};
  (void)hipGetLastError();
  const hipError_t e = ttt::route(a);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

namespace {
bool target_shape_ok(int B, int T, int d_in, int d_out, int chunk, int width) {
  return B >= 1 && T >= 1 && chunk >= 1 && width >= 1 && width <= 16 && d_in >= 64 &&
         d_out >= 16 && d_in % 64 == 0 && d_out % 16 == 0 && T <= (1 << 26) &&
         d_in <= (1 << 16) && d_out <= (1 << 16) && B <= 65535 &&
         size_t(T) * (d_in / 8) / 256 < (1u << 31);
}
}  // namespace

TTT_EXPORT size_t ttt_lm_target_workspace(int B, int T, int d_in, int d_out) {
  if (!target_shape_ok(B, T, d_in, d_out, 1, 1)) return 0;
  return ttt::lm_target_workspace(B, T, d_in, d_out);
}

TTT_EXPORT ttt_status ttt_lm_target(const void* X0, ttt_dtype in_dtype, const float* conv_w,
                                    int width, const void* W_target, void* V_hat,
                                    ttt_dtype out_dtype, int B, int T, int d_in, int d_out,
                                    int chunk, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TTT_E_DTYPE;
  if (!X0 || !conv_w || !W_target || !V_hat) return TTT_E_NULL;
  if (!target_shape_ok(B, T, d_in, d_out, chunk, width)) return TTT_E_SHAPE;
  if (in_dtype != TTT_BF16) return TTT_E_UNSUPPORTED;
  if (!aligned16(X0) || !aligned16(conv_w) || !aligned16(W_target) || !aligned16(V_hat) ||
      !aligned16(workspace))
    return TTT_E_ALIGN;
  const size_t need = ttt_lm_target_workspace(B, T, d_in, d_out);
  if (!workspace || workspace_bytes < need) return TTT_E_WORKSPACE;
  const Range rx{X0, size_t(B) * T * d_in * 2}, rc{conv_w, size_t(width) * d_in * 4},
      rw{W_target, size_t(d_in) * d_out * 2}, rv{V_hat, size_t(B) * T * d_out * dsize(out_dtype)},
      rs{workspace, need};
  for (Range r : {rx, rc, rw})
    if (overlap(rv, r) || overlap(rs, r)) return TTT_E_ALIAS;
  if (overlap(rv, rs)) return TTT_E_ALIAS;
  ttt::TargetArgs a{X0, conv_w, width, W_target, V_hat, out_dtype == TTT_BF16, B, T, d_in,
                    d_out, chunk, workspace, stream};
  (void)hipGetLastError();
  const hipError_t e = ttt::lm_target(a);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

namespace {
bool gated_z_shape_ok(int B, int T, int d_model, int d_ff) {
  return B >= 1 && B <= 65535 && T >= 1 && T <= (1 << 26) && d_model >= 64 &&
         d_model % 64 == 0 && d_model <= (1 << 16) && d_ff >= 8 && d_ff % 8 == 0 &&
         d_ff <= (1 << 20) && size_t((d_ff + 127) / 128) * ((T + 127) / 128) < (1u << 31) &&
         (size_t(d_ff) + 128) * d_model * 2 < (size_t(1) << 32);
}
}  // namespace

TTT_EXPORT ttt_status ttt_gated_z(const void* X, ttt_dtype in_dtype, const void* W_gu, void* Z,
                                  ttt_dtype out_dtype, int B, int T, int d_model, int d_ff,
                                  hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TTT_E_DTYPE;
  if (!X || !W_gu || !Z) return TTT_E_NULL;
  if (!gated_z_shape_ok(B, T, d_model, d_ff)) return TTT_E_SHAPE;
  if (in_dtype != TTT_BF16) return TTT_E_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(W_gu) || !aligned16(Z)) return TTT_E_ALIGN;
  const Range rx{X, size_t(B) * T * d_model * 2}, rw{W_gu, size_t(d_model) * d_ff * 4},
      rz{Z, size_t(B) * T * d_ff * dsize(out_dtype)};
  if (overlap(rz, rx) || overlap(rz, rw)) return TTT_E_ALIAS;
  ttt::GatedZArgs a{X, W_gu, Z, out_dtype == TTT_BF16, B, T, d_model, d_ff, stream};
  (void)hipGetLastError();
  const hipError_t e = ttt::gated_z(a);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

TTT_EXPORT ttt_status ttt_cache_readout(const void* Q, const void* K, const void* V,
                                        ttt_dtype qkv_dtype, const unsigned char* routed_mask,
                                        const void* ttt_out, void* out, ttt_dtype out_dtype,
                                        const float* alpha, int B, int T, int H, int dh,
                                        int chunk, int capacity, float scale,
                                        hipStream_t stream) {
  if (!valid_dtype(qkv_dtype) || !valid_dtype(out_dtype)) return TTT_E_DTYPE;
  if (!Q || !K || !V || !routed_mask || !ttt_out || !out || !alpha) return TTT_E_NULL;
  if (B < 1 || B > 65535 || T < 1 || T > (1 << 24) || H < 1 || H > 65535 || dh < 1 ||
      chunk < 1 || T % chunk || capacity < 1 || !std::isfinite(scale))
    return TTT_E_SHAPE;
  if (qkv_dtype != TTT_BF16 || dh != 64 || chunk % 64 || capacity > 256) return TTT_E_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(ttt_out) ||
      !aligned16(out) || !aligned16(alpha) || !aligned16(routed_mask))
    return TTT_E_ALIGN;
  const size_t n = size_t(B) * T * H * dh;
  const Range rq{Q, n * 2}, rk{K, n * 2}, rv{V, n * 2}, rm{routed_mask, size_t(B) * T},
      ra{alpha, size_t(H) * dh * 4}, rt{ttt_out, n * dsize(out_dtype)},
      ro{out, n * dsize(out_dtype)};
  for (Range r : {rq, rk, rv, rm, ra})
    if (overlap(ro, r)) return TTT_E_ALIAS;
  if (out != ttt_out && overlap(ro, rt)) return TTT_E_ALIAS;  // in place is allowed
  ttt::ReadoutArgs a{Q, K, V, routed_mask, ttt_out, out, alpha, out_dtype == TTT_BF16,
                     B, T, H, chunk, capacity, scale, stream};
  (void)hipGetLastError();
  const hipError_t e = ttt::cache_readout(a);
  return e == hipSuccess ? TTT_OK : TTT_E_LAUNCH;
}

TTT_EXPORT const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "TTT_OK: success";
    case TTT_E_NULL: return "TTT_E_NULL: a required pointer is NULL";
    case TTT_E_SHAPE: return "TTT_E_SHAPE: a size or parameter is out of range";
    case TTT_E_DTYPE: return "TTT_E_DTYPE: unknown dtype code";
    case TTT_E_ALIGN: return "TTT_E_ALIGN: a pointer is not 16-byte aligned";
    case TTT_E_WORKSPACE: return "TTT_E_WORKSPACE: workspace missing or too small";
    case TTT_E_UNSUPPORTED: return "TTT_E_UNSUPPORTED: valid request this library does not implement";
    case TTT_E_LAUNCH: return "TTT_E_LAUNCH: the HIP runtime rejected a launch";
    case TTT_E_ALIAS: return "TTT_E_ALIAS: an output overlaps an input";
  }
  return "unknown ttt_status";
}

TTT_EXPORT int ttt_abi_version(void) { return TTT_ABI_VERSION; }
