/*
 * ttt_mi355x.h -- C ABI of the chunked test-time-training fast-weight scan for MI355X (gfx950).
 *
 * The hot-path operations, each named after the source pages' statement of the problem:
 *
 *   ttt_chunk_scan        In-Place TTT: per chunk, apply the pre-update fast weight W_down, then
 *                         add eta * V_hat_i^T Z_i ("In-Place Test-Time Training", iplexlaw.co.kr
 *                         blog on arXiv 2604.06169: section 2 for the update formula, section 3
 *                         for apply-then-update, section 6 for the additive exclusive prefix).
 *   ttt_linear_minibatch  TTT-Linear: one gradient step of 1/2 ||k W - v||^2 per mini-batch, with
 *                         the output in dual form (TTT layers page, ai-jitan-hub, on
 *                         arXiv 2407.04620; DeltaNet equivalence at mini-batch 1).
 *   ttt_surprisal_route   SR-TTT surprisal filter and residual cache ("SR-TTT: Surprisal-Aware
 *                         Residual Test-Time Training", gist.science, arXiv 2603.06642, section
 *                         2.1; FIFO-like eviction from section 5).
 *
 * and the steps next to them on the path, declared further down: ttt_chunk_scan_docs (document
 * resets and update clipping), ttt_lm_target (the LM-aligned target), ttt_gated_z (the scan's
 * input Z) and ttt_cache_readout (the residual-cache readout).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or keeps them. Tensors are dense, row-major, with the stated shapes.
 *   - Every pointer must be 16-byte aligned (TTT_E_ALIGN otherwise).
 *   - Arguments are validated on the host before anything is enqueued. On any status other than
 *     TTT_OK nothing has been launched and no output has been written.
 *   - On TTT_OK the kernels are enqueued on `stream` (0 = the default stream) and the call returns
 *     without synchronising. Faults during execution surface at the caller's synchronisation.
 *   - Calls keep no state between them and may be made from several host threads; calls that
 *     share output or workspace buffers must be ordered by the caller.
 *   - A call may be captured into a HIP graph (stream capture) and replayed: it enqueues kernel
 *     launches only (device-to-device copies for eta = 0 and the fp32 scan's state), and what
 *     must start at zero in a workspace is cleared by the library's own kernels on every run, not
 *     by memset nodes. ttt_chunk_scan_profile synchronises and is not capturable.
 */
#ifndef TTT_MI355X_H
#define TTT_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 7

typedef enum {
  TTT_OK = 0,
  TTT_E_NULL = 1,         /* a required pointer is NULL                                      */
  TTT_E_SHAPE = 2,        /* a size is out of range or violates a divisibility rule          */
  TTT_E_DTYPE = 3,        /* unknown dtype code                                              */
  TTT_E_ALIGN = 4,        /* a pointer is not 16-byte aligned                                */
  TTT_E_WORKSPACE = 5,    /* workspace smaller than the size query returned                  */
  TTT_E_UNSUPPORTED = 6,  /* valid request outside what this library implements              */
  TTT_E_LAUNCH = 7,       /* the HIP runtime rejected a launch or an enqueue                 */
  TTT_E_ALIAS = 8         /* an output overlaps an input in a way the operation forbids      */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* ------------------------------------------------------------------------------------------ */
/* In-Place TTT chunk scan.
 *
 * For each sequence b and each chunk i = rows [iC, min((i+1)C, T)):
 *     O_i     = Z_i W_i^T                 (apply the state from before chunk i's update)
 *     W_{i+1} = W_i + eta * V_i^T Z_i     (then update; chunk i never sees its own delta)
 * W is the down projection in nn.Linear [out, in] storage, [d_model, d_ff], exactly as the page
 * writes the update dW_down = eta * V_hat^T * Z. A last chunk shorter than C is allowed.
 *
 *   Z        [B, T, d_ff]      in_dtype (TTT_F32 or TTT_BF16)   intermediate activation
 *   Vhat     [B, T, d_model]   in_dtype                          LM-aligned target
 *   W0       [d_model, d_ff] fp32 if w0_shared != 0, else [B, d_model, d_ff] fp32
 *   O        [B, T, d_model]   out_dtype                         chunk outputs
 *   W_final  [B, d_model, d_ff] fp32, or NULL to skip. It may be the same buffer as W0 when
 *            w0_shared == 0 or B == 1 (in-place continuation); any other overlap with an input
 *            or with O gives TTT_E_ALIAS.
 *   d_ff, d_model: multiples of 16; chunk >= 1; T >= 1; B >= 1.
 *   eta: finite (else TTT_E_SHAPE). With bf16 inputs a nonzero eta must satisfy
 *            1e-18 <= |eta| <= 1e18 (else TTT_E_UNSUPPORTED): that path keeps the state as
 *            W / eta. eta = 0 is exact on both paths: W_final is W0 bit for bit.
 *   workspace: device scratch (may be NULL when ttt_chunk_scan_workspace(...) is 0); its contents
 *            on entry do not matter; it is clobbered. With ttt_chunk_scan_workspace(...) bytes the
 *            sequence runs in one pass. With bf16 inputs any size from
 *            ttt_chunk_scan_workspace_min(...) up is also accepted: the scan then runs over
 *            segments of whole groups of chunks, each resuming from the fp32 state the previous
 *            one ended with (held in W_final, or in the workspace when W_final is NULL). The
 *            result is the same scan (chunk starts and the state are those of one pass) up to
 *            the rounding of the state handed across segments; the workspace stays bounded
 *            however long the sequence (TTT_E_WORKSPACE below the minimum).
 *
 * Arithmetic: bf16 inputs use bf16 matrix-core products with fp32 accumulation and an fp32 state
 * (the state is rounded to bf16 only as a product operand); fp32 inputs use fp32 throughout.
 * O in bf16 is rounded to nearest even from the fp32 result.
 *
 * Hand-over inside the bf16 state chain: each state tile's token stream is split in two
 * workgroups, the second continuing from the state the first hands over through the workspace.
 * The second one waits for it with a bounded wait (about 0.1 s plus about 4 us per 32 tokens of
 * the first half). Workgroups are dispatched in order, so the wait ends; if it ever ran out, the
 * second workgroup does not use the hand-over and recomputes the first half's tokens from W0
 * itself. The outputs are then the same bits, produced later. Such events are counted in the
 * workspace (see ttt_chunk_scan_handover_timeouts); nothing else reports them.
 */
ttt_status ttt_chunk_scan(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                          const float* W0, int w0_shared,
                          void* O, ttt_dtype out_dtype,
                          float* W_final,
                          int B, int T, int d_ff, int d_model, int chunk, float eta,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ttt_chunk_scan for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments and results without
 * a workspace argument. The workspace comes from a static device array of
 * TTT_SCAN_SCRATCH_BYTES held by every GPU the library runs on until the process ends (its
 * device address is resolved once per device, on the first call there). The call allocates and
 * frees nothing.
 *   - Shapes whose ttt_chunk_scan_workspace(...) exceeds TTT_SCAN_SCRATCH_BYTES run in segments
 *     inside the scratch when ttt_chunk_scan_workspace_min(...) fits (bf16 inputs, see
 *     ttt_chunk_scan's workspace), and are otherwise refused with TTT_E_WORKSPACE before
 *     anything is enqueued (use ttt_chunk_scan with a workspace).
 *   - Every call on one GPU uses the same scratch, which keeps the last call's contents (the
 *     kernels clear what must start at zero): calls that overlap in time on one GPU (other
 *     streams, other threads) race and give wrong results; order them on one stream.
 *   - `stream` must belong to the current device (TTT_E_UNSUPPORTED otherwise).
 */
#define TTT_SCAN_SCRATCH_BYTES (64u << 20)
ttt_status ttt_chunk_scan_noalloc(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                  const float* W0, int w0_shared, void* O, ttt_dtype out_dtype,
                                  float* W_final, int B, int T, int d_ff, int d_model, int chunk,
                                  float eta, hipStream_t stream);

/* Bytes of workspace ttt_chunk_scan needs for these sizes to run in one pass (0 if none).
 * Returns 0 for arguments ttt_chunk_scan would reject. */
size_t ttt_chunk_scan_workspace(int B, int T, int d_ff, int d_model, int chunk,
                                ttt_dtype in_dtype);

/* The least workspace ttt_chunk_scan accepts for these sizes: with bf16 inputs, that of
 * segments of one group of chunks (about 1024 tokens) plus an fp32 state of
 * B x d_model x d_ff; otherwise ttt_chunk_scan_workspace(...). 0 for rejected arguments. */
size_t ttt_chunk_scan_workspace_min(int B, int T, int d_ff, int d_model, int chunk,
                                    ttt_dtype in_dtype);

/* Enqueues on `stream` a 4-byte copy into the device word `count` of how many state-chain
 * hand-over waits ran out (and were recomputed, see above) in the last ttt_chunk_scan or
 * ttt_chunk_scan_docs call that used `workspace` with these sizes (for the docs call when it ran
 * its documents as separate scans: in the last of them). 0 for fp32 inputs, which have no
 * hand-over. workspace must hold ttt_chunk_scan_workspace(...) bytes (TTT_E_WORKSPACE);
 * count: device pointer, 16-byte aligned, outside the workspace. Does not synchronise. */
ttt_status ttt_chunk_scan_handover_timeouts(int B, int T, int d_ff, int d_model, int chunk,
                                            ttt_dtype in_dtype, const void* workspace,
                                            size_t workspace_bytes, unsigned* count,
                                            hipStream_t stream);

/* FOR TESTS ONLY: process-wide overrides of three schedule choices of the bf16 scan, read by
 * every later ttt_chunk_scan*, workspace query and call (the workspace size depends on the
 * first): group_tokens > 0 sets the group of chunks to about that many tokens (default about
 * 1024); token_split == 0 turns the state chain's token split off (any other value: default);
 * spin_limit >= 0 sets the number of polls of the hand-over wait (0 makes every wait run out at
 * once; < 0: default). ttt_scan_test_overrides(0, -1, -1) restores the defaults. Results never
 * depend on these settings beyond rounding order (the group size) and never on the last two.
 * Not to be changed while another thread is inside a scan call. Always returns TTT_OK. */
ttt_status ttt_scan_test_overrides(int group_tokens, int token_split, int spin_limit);

/* In-Place TTT chunk scan with document-boundary reset and per-chunk update clipping
 * ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv 2604.06169, section 6: the fast
 * weight goes back to its pre-trained state when a document ends, and the Frobenius norm of
 * each update delta is limited to a threshold for long contexts). Same arguments and results as
 * ttt_chunk_scan, and:
 *   doc_counts  host int[B] or NULL: how many documents start inside sequence b (besides the
 *               one at token 0)
 *   doc_starts  host int[sum of doc_counts]: sequence 0's starts, then sequence 1's, ...; each
 *               sequence's strictly increasing, multiples of chunk, inside (0, T)
 *               (else TTT_E_SHAPE). Both arrays are read during the call only.
 *   clip_tau    absolute threshold: chunk i's delta dW_i = eta Vhat_i^T Z_i is replaced by
 *               dW_i * min(1, clip_tau / ||dW_i||_F); clip_tau <= 0 or infinite: no clipping;
 *               NaN: TTT_E_SHAPE.
 * A chunk that starts a document is applied with W0 and only earlier chunks of its own document
 * contribute to later ones; W_final is the state after the sequence's last chunk (its last
 * document's). The norms come from the identity ||Vhat_i^T Z_i||_F^2 = <Z_i Z_i^T,
 * Vhat_i Vhat_i^T>_F (fp32 Gram products, fp64 sums in a fixed order); the clipped deltas are
 * formed by scanning targets whose chunk rows are scaled by their factors (rounded to in_dtype).
 *   workspace: at least ttt_chunk_scan_docs_workspace(...) bytes (larger than ttt_chunk_scan's
 *   when clipping). With bf16 inputs on the unmasked shapes (d_ff a multiple of 64, the scan's
 *   group of chunks, about 1024 tokens, a multiple of 64 tokens), the documents run as one
 *   batched scan whose state goes back to W0 at each start when every start is a multiple of
 *   the group or, with chunk and d_ff multiples of 32, lies 256 x n tokens after the start of
 *   its group (and B * T / gcd(group, 256) <= 8192); otherwise as separate scans on `stream`,
 *   one after the other. Starts on group boundaries give the bits of separate scans; a start
 *   inside a group leaves the document's later groups where the sequence's fall, so its
 *   results equal separate scans' up to rounding order.
 */
ttt_status ttt_chunk_scan_docs(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                               const float* W0, int w0_shared, void* O, ttt_dtype out_dtype,
                               float* W_final, int B, int T, int d_ff, int d_model, int chunk,
                               float eta, const int* doc_starts, const int* doc_counts,
                               float clip_tau, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of workspace ttt_chunk_scan_docs needs (0 for sizes ttt_chunk_scan would reject). */
size_t ttt_chunk_scan_docs_workspace(int B, int T, int d_ff, int d_model, int chunk,
                                     ttt_dtype in_dtype, float clip_tau);

/* Instrumented ttt_chunk_scan for profiling: same arguments and results, but it records HIP
 * events on `stream` around each internal phase, WAITS for the stream to finish, and fills
 *   phase_ms[p]       milliseconds spent in phase p (from the first to the last launch of it),
 *   phase_launches[p] number of kernel launches in phase p,
 * for p < TTT_SCAN_NPHASE:
 *   0 operand staging (token-major copies of Z and V_hat),
 *   1 intra-group correction products (eta * Z_a Z_b^T blocks),
 *   2 state-update chain (W_{g+1} = W_g + eta * V_g^T Z_g),
 *   3 apply (O = Z W_g^T plus the intra-group correction).
 * The fp32 path reports its per-chunk apply/update launches as phases 3 and 2.
 * Either array may be NULL. Not for production use: it synchronises. */
#define TTT_SCAN_NPHASE 4
ttt_status ttt_chunk_scan_profile(const void* Z, const void* Vhat, ttt_dtype in_dtype,
                                  const float* W0, int w0_shared,
                                  void* O, ttt_dtype out_dtype,
                                  float* W_final,
                                  int B, int T, int d_ff, int d_model, int chunk, float eta,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  float* phase_ms, int* phase_launches);

/* ------------------------------------------------------------------------------------------ */
/* TTT-Linear, mini-batch gradient descent in dual form (no LayerNorm, no residual).
 *
 * For each sequence b, head h and mini-batch m = rows [m b_, (m+1) b_), with W the
 * start-of-mini-batch state (a [dh, dh] map of row vectors, o = q W):
 *     R    = K_m W - V_m
 *     O_m  = Q_m W - (eta / b_) tril(Q_m K_m^T) R      (inclusive: token t sees s <= t)
 *     W   <- W - (eta / b_) K_m^T R
 *     loss[t] = ||r_t||^2                             (squared residual at the start-of-mini-batch W)
 *
 *   Q, K, V  [B, T, H, dh]   in_dtype
 *   W0       [B, H, dh, dh] fp32, or NULL for a zero initial state
 *   O        [B, T, H, dh]   out_dtype
 *   W_final  [B, H, dh, dh] fp32 or NULL; may equal W0
 *   loss     [B, T, H] fp32 or NULL
 *   dh must be 64 (TTT_E_UNSUPPORTED otherwise); T % minibatch == 0.
 * bf16 inputs with minibatch in {16, 32, 48, 64} use matrix-core kernels (the fp32 state enters
 * the products as a two-term bf16 split); other mini-batch sizes and fp32 inputs use an fp32
 * kernel that accumulates the same step token by token.
 */
ttt_status ttt_linear_minibatch(const void* Q, const void* K, const void* V, ttt_dtype in_dtype,
                                const float* W0,
                                void* O, ttt_dtype out_dtype,
                                float* W_final, float* loss,
                                int B, int T, int H, int dh, int minibatch, float eta,
                                hipStream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* SR-TTT surprisal routing into a FIFO residual cache.
 *
 * Per sequence: L_t = sum_h loss[t, h] (fp32, head order). For each routing chunk c (in order):
 *     p_c   = nearest-rank pct-quantile of the chunk's L (k = ceil(pct * chunk) in fp64)
 *     tau_c = p_0 if c == 0 else fl32(fl32(ema * tau_{c-1}) + fl32(fl32(1 - ema) * p_c))
 *     ok_c  = mean_c >= chunk_ratio * tau_c   (fp64; mean_c = fp64 pairwise sum / chunk)
 *     route token t iff ok_c and L_t > tau_c
 * Routed tokens enter a ring of `capacity` slots in token order: the r-th routed token goes to
 * slot r % capacity, so the ring ends with the newest `capacity` routed tokens.
 *
 *   loss         [B, T, H] fp32 (as written by ttt_linear_minibatch)
 *   K, V         [B, T, H * dh] kv_dtype; rows of routed tokens are copied bit for bit
 *   tau          [B, T / chunk] fp32 or NULL: the threshold each chunk was routed with
 *   routed_mask  [B, T] uint8 or NULL: 1 for every routed token (including ones later evicted)
 *   cache_idx    [B, capacity] int32: token index per slot, -1 for an empty slot
 *   cache_k/v    [B, capacity, H * dh] kv_dtype or NULL; empty slots are zero-filled
 *   cache_count  [B] int32: min(routed, capacity); routed_total [B] int32: routed
 *   Requirements: T % chunk == 0, 1 <= chunk <= 1024, T <= 2^22, 1 <= capacity <= 4096,
 *   0 < pct <= 1, 0 <= ema <= 1, (H * dh * element size) % 16 == 0.
 */
ttt_status ttt_surprisal_route(const float* loss, const void* K, const void* V, ttt_dtype kv_dtype,
                               int B, int T, int H, int dh, int chunk,
                               float pct, float ema, float chunk_ratio, int capacity,
                               float* tau, unsigned char* routed_mask,
                               int* cache_idx, void* cache_k, void* cache_v,
                               int* cache_count, int* routed_total,
                               hipStream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* LM-aligned target producer ("In-Place Test-Time Training", iplexlaw.co.kr blog on arXiv
 * 2604.06169, section 4: V_hat = Conv1D(X0) W_target, the convolution reaching the next and
 * near-future tokens; section 6: padding at chunk boundaries keeps it from reading another
 * chunk, and it is depthwise). For each sequence b and token t:
 *     A[t]     = sum_{j=1..width} conv_w[j-1] * X0[t+j]   (per channel; a token at or past
 *                                                          the end of t's chunk, or past T,
 *                                                          contributes 0)
 *     V_hat[t] = A[t] W_target
 * A is computed in fp32 and rounded to bf16 (the matrix-core operand); the product accumulates
 * in fp32 and V_hat is rounded to out_dtype.
 *
 *   X0        [B, T, d_in]   bf16 (in_dtype must be TTT_BF16, else TTT_E_UNSUPPORTED)
 *   conv_w    [width, d_in]  fp32, shared by the batch; 1 <= width <= 16
 *   W_target  [d_in, d_out]  bf16, shared by the batch (row vectors times the matrix)
 *   V_hat     [B, T, d_out]  out_dtype; must not overlap any input or the workspace
 *   d_in % 64 == 0, d_out % 16 == 0, chunk >= 1, T >= 1, B >= 1.
 *   workspace: at least ttt_lm_target_workspace(B, T, d_in, d_out) bytes (the bf16 A, then
 *   W_target transposed, bf16).
 */
ttt_status ttt_lm_target(const void* X0, ttt_dtype in_dtype, const float* conv_w, int width,
                         const void* W_target, void* V_hat, ttt_dtype out_dtype,
                         int B, int T, int d_in, int d_out, int chunk,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ttt_lm_target needs (0 for arguments it would reject). */
size_t ttt_lm_target_workspace(int B, int T, int d_in, int d_out);

/* ------------------------------------------------------------------------------------------ */
/* Gated-MLP intermediate activation ("In-Place Test-Time Training", iplexlaw.co.kr blog on
 * arXiv 2604.06169, section 2: the MLP combines a gate projection and an up projection of its
 * input through the gate into Z, the input of the fast-weight projection W_down, so Z is what
 * ttt_chunk_scan consumes). For each sequence b and token t, f < d_ff:
 *     Z[b][t][f] = SiLU(X[b][t] . W_gu[f]) * (X[b][t] . W_gu[d_ff + f]),
 *     SiLU(g) = g / (1 + exp(-g))
 * i.e. Z = SiLU(X W_gate) * (X W_up) with W_gate = W_gu[0 .. d_ff-1]^T, W_up = W_gu[d_ff ..]^T.
 * Both sums accumulate in fp32 from bf16 operands; SiLU and the product are fp32; Z is rounded
 * once to out_dtype. Z is written token-major, the layout ttt_chunk_scan reads.
 *
 *   X     [B, T, d_model]      bf16 (in_dtype must be TTT_BF16, else TTT_E_UNSUPPORTED)
 *   W_gu  [2 d_ff, d_model]    bf16, shared by the batch, stored as a linear layer stores its
 *                              weight (one row of d_model weights per output): rows 0 .. d_ff-1
 *                              the gate projection, rows d_ff .. 2 d_ff-1 the up projection
 *   Z     [B, T, d_ff]         out_dtype (TTT_BF16 or TTT_F32); must not overlap X or W_gu
 *   d_model % 64 == 0, d_ff % 8 == 0, (d_ff + 128) * d_model < 2^31, T >= 1, B >= 1; no
 *   workspace; all pointers 16-byte aligned. The call only enqueues work on `stream`.
 */
ttt_status ttt_gated_z(const void* X, ttt_dtype in_dtype, const void* W_gu, void* Z,
                       ttt_dtype out_dtype, int B, int T, int d_model, int d_ff,
                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------ */
/* SR-TTT residual-cache readout with alpha fusion ("SR-TTT: Surprisal-Aware Residual Test-Time
 * Training", gist.science summary of arXiv 2603.06642, section 2.1: routed tokens' keys and
 * values form a fixed-capacity cache beside the fast weights; the layer output is the TTT
 * output plus a clamp-parameterised gate alpha times the attention output over the cache;
 * section 5: eviction is FIFO-like once the cache is full). For sequence b, token t in routing
 * chunk c = t / chunk, head h:
 *     visible = the newest min(capacity, R) routed tokens among tokens < c * chunk
 *               (R = how many there are): the cache as it stood when chunk c began
 *     a[h]    = sum_{j in visible} softmax_j(scale * Q[t,h] . K[j,h]) V[j,h]   (0 if empty)
 *     out[t]  = ttt_out[t] + clamp(alpha, 0, 1) * a          (per channel of H * dh)
 * Logits and exponentials in fp32; the weights enter the value product as bf16 and are
 * normalised by the sum of the same rounded weights; out is rounded once to out_dtype. With no
 * visible entry out[t] is a bit-exact copy of ttt_out[t].
 *
 *   Q, K, V      [B, T, H * dh] qkv_dtype (must be TTT_BF16, else TTT_E_UNSUPPORTED); K and V
 *                are the tensors given to ttt_surprisal_route (rows of routed tokens are read)
 *   routed_mask  [B, T] uint8, nonzero = routed (as written by ttt_surprisal_route); 16-byte
 *                aligned like every other pointer
 *   ttt_out      [B, T, H * dh] out_dtype: the TTT output (e.g. of ttt_linear_minibatch)
 *   out          [B, T, H * dh] out_dtype; may be ttt_out itself (in place), must not overlap
 *                any other input
 *   alpha        [H * dh] fp32 gate, clamped to [0, 1]
 *   T % chunk == 0; this library implements dh == 64, chunk % 64 == 0, capacity <= 256
 *   (TTT_E_UNSUPPORTED otherwise); scale finite (1 / sqrt(dh) is the usual choice).
 */
ttt_status ttt_cache_readout(const void* Q, const void* K, const void* V, ttt_dtype qkv_dtype,
                             const unsigned char* routed_mask, const void* ttt_out, void* out,
                             ttt_dtype out_dtype, const float* alpha, int B, int T, int H,
                             int dh, int chunk, int capacity, float scale, hipStream_t stream);

/* ------------------------------------------------------------------------------------------ */
const char* ttt_status_string(ttt_status s);  /* static string, never NULL */
int ttt_abi_version(void);                     /* TTT_ABI_VERSION of the built library */

#ifdef __cplusplus
}
#endif
#endif /* TTT_MI355X_H */
