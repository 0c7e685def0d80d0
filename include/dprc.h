/*
 * dprc.h - C ABI of the DP-SGD-with-randomized-clipping hot path on MI355X.
 *
 * The library (libdprc.so, hand-written HIP kernels for gfx950) runs steps 3-5
 * of the algorithm in the randomized-clipping summary, "技術的サマリー：ランダム化
 * クリッピングを備えた LLM 向け効率的な DP-SGD", section アルゴリズム的フロー:
 *   3. per-sample squared-norm estimation of each linear layer's gradient
 *      (dp_norm_est: Hutch, Hutch++, and the exact ghost / FGC baselines),
 *   4. per-sample clip factors c_i = min(1, C / sqrt(n_i)),
 *   5. the clipped sum of per-sample gradients (dp_clip_aggregate), then
 *      Gaussian noise and the SGD update (dp_noise_update),
 * with the clip / noise / update formulas of the glossary page
 * "DP-SGD（差分プライバシー確率的勾配降下法）とは？", section DP-SGDのアルゴリズム,
 * steps 3-5.
 *
 * Notation (the pages'): B samples of T tokens; a linear layer of shape (p, d)
 * has per-sample activations A_i (T x d) and output gradients G_i (T x p); its
 * per-sample weight gradient is G_i^T A_i (p x d) and
 * ||A_i^T G_i||_F^2 = tr(G_i^T A_i A_i^T G_i) (section 中核メカニズム).
 *
 * Conventions for every entry point:
 *  - Tensors are caller-owned DEVICE memory, dense row-major, and 16-byte
 *    aligned (A, G, S, theta, workspace) or 4-byte aligned (n_sq, c_out).
 *    The library never allocates, frees or prints, and never synchronises
 *    except in dp_read_device_status.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously.  A DP_OK return means "validated and enqueued".
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is enqueued and no output is touched.  DP_ERR_HIP means a
 *    launch failed (hipGetLastError); outputs are then undefined.
 *  - Calls are thread-safe (the only mutable global state is the lock-guarded
 *    per-device address table of dp_norm_est_noalloc).  Concurrent calls that
 *    share a workspace or an output buffer race, as any stream work would.
 *  - Results are deterministic: no floating-point atomics; the same inputs and
 *    seeds give the same bits on the same device.
 */
#ifndef DPRC_H
#define DPRC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DPRC_ABI_VERSION 4

typedef void *dp_stream_t; /* a hipStream_t */

typedef enum {
  DP_OK = 0,
  DP_ERR_INVALID_ARG = 1, /* bad size, pointer, alignment or parameter */
  DP_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. dtype/method combination) */
  DP_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the matching *_workspace() query */
  DP_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} dp_status_t;

typedef enum { DP_F32 = 0, DP_BF16 = 1 } dp_dtype_t; /* A and G share one dtype */

typedef enum {
  DP_NORM_HUTCH = 0,   /* Hutchinson, k Gaussian probes (section 中核メカニズム, item 1) */
  DP_NORM_HUTCHPP = 1, /* Hutch++: QR head + Hutchinson tail (item 2) */
  DP_NORM_GHOST = 2,   /* exact, T x T Gram products (ghost clipping, baseline) */
  DP_NORM_FGC = 3      /* exact, materialised d x p per-sample gradient (baseline) */
} dp_norm_method_t;

/* dp_norm_est flags */
#define DP_ACCUMULATE 1u   /* n_sq[i] += estimate (sum over layers) instead of n_sq[i] = estimate */
#define DP_PROBE_SHARED 2u /* one probe matrix for the whole batch (the sample-0 stream) */
/* Rademacher probes: entries +1 / -1 (the summary's section 意義と主張 names
 * {+-1}-valued sketching matrices as a way to cut the overhead further) instead
 * of N(0, 1); the same counters and lanes as the Gaussian probe, +1 when the
 * 32-bit word's top bit is 0.  The estimate keeps the 1/k (E[P P^T] = k I). */
#define DP_PROBE_RADEMACHER 4u

/*
 * Device status flags.  Every call that forms clip factors (dp_clip_aggregate,
 * dp_clip_aggregate_update, dp_clip_aggregate_update_layers,
 * dp_rmsnorm_clip_aggregate_update, dp_embedding_clip_aggregate_update) ORs them into a sticky status word kept
 * in the first 8 bytes of its workspace; the word stays set over any number of
 * calls that reuse the workspace until dp_read_device_status reads and clears
 * it.  A newly allocated workspace must start with that word at zero: allocate
 * it zeroed, or call dp_read_device_status on it once and discard the result.
 */
#define DP_STATUS_NONFINITE_NORM 1u /* some n_sq[i] was NaN/Inf: its c_i was set to 0 */

int dp_abi_version(void);
const char *dp_status_string(dp_status_t s);

/*
 * Bytes of workspace dp_norm_est needs for these arguments (0 if none), or
 * (size_t)-1 if the arguments are invalid.
 */
size_t dp_norm_est_workspace(int method, int dtype, int B, int T, int d, int p, int k);

/*
 * Per-sample squared gradient norm of one linear layer, n_i ~ ||A_i^T G_i||_F^2.
 *
 *  method  dp_norm_method_t.  HUTCH: n_i = ||A_i^T (G_i P_i)||_F^2 / k with
 *          P_i (p x k) i.i.d. N(0,1) (section 中核メカニズム, item 1; the 1/k
 *          makes it unbiased).  HUTCHPP: s = k/3 sketch columns, Q = orth(O S),
 *          n_i = ||A^T G Q||^2 + ||A^T G (I - Q Q^T) W||^2 / r with r = k - 2s
 *          (item 2).  GHOST: <A_i A_i^T, G_i G_i^T>_F.  FGC: ||A_i^T G_i||_F^2
 *          with A_i^T G_i materialised in the workspace.
 *  dtype   DP_F32 or DP_BF16 for A and G (fp32 accumulation either way).
 *  B, T    batch size (>= 0) and tokens per sample (>= 0); B = 0 is a no-op,
 *          T = 0 gives n_i = 0.
 *  d, p    layer input / output widths (>= 1).
 *  k       probes: HUTCH 1 <= k <= p; HUTCHPP 3 <= k <= p with s = k/3 <= 32 and
 *          r = k - 2s <= 32 (so k <= 96, k != 95); ignored for exact methods.
 *  A       [B][T][d] device, dtype.      G  [B][T][p] device, dtype.
 *  seed    64-bit Philox4x32-10 key of the probe stream.
 *  layer   layer index (counter word), so layers draw independent probes.
 *          Probe entry (row r, column j) of sample i is lane r mod 4 of the
 *          counter (r / 4, j, i, layer).
 *  flags   DP_ACCUMULATE | DP_PROBE_SHARED | DP_PROBE_RADEMACHER.
 *  n_sq    [B] fp32 device output (or accumulator with DP_ACCUMULATE).
 *  ws      device workspace of ws_bytes >= dp_norm_est_workspace(...).
 */
dp_status_t dp_norm_est(int method, int dtype, int B, int T, int d, int p, int k,
                        const void *A, const void *G, uint64_t seed, uint32_t layer,
                        uint32_t flags, float *n_sq, void *ws, size_t ws_bytes,
                        dp_stream_t stream);

/*
 * dp_norm_est without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The arguments, results and errors are those of
 * dp_norm_est (the same kernels); the workspace is instead a library-owned
 * scratch array of DP_NOALLOC_SCRATCH_BYTES in device memory, one per GPU,
 * held from the first call on that GPU until the process ends.  No call
 * allocates or frees anything.
 *  - Returns DP_ERR_WORKSPACE, with nothing enqueued, when
 *    dp_norm_est_workspace(...) of the arguments exceeds
 *    DP_NOALLOC_SCRATCH_BYTES (it covers Hutch and Hutch++ with k <= 32 on
 *    every layer of a Llama-3.2-1B-sized model at B = 8, T = 4096, and the
 *    ghost baseline; FGC's per-sample d x p matrices mostly do not fit).
 *  - Every call on one GPU shares that GPU's array: calls that may overlap
 *    (different streams, or different host threads, on the same GPU) race and
 *    must be ordered by the caller.  Calls on one stream are ordered.
 *  - The array keeps the last call's contents; the kernels need no part of it
 *    to start at zero.
 *  - The first call on a GPU looks up the array's device address (a host-side
 *    runtime query, guarded by a lock); DP_ERR_HIP if that fails.
 */
#define DP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dp_status_t dp_norm_est_noalloc(int method, int dtype, int B, int T, int d, int p, int k,
                                const void *A, const void *G, uint64_t seed, uint32_t layer,
                                uint32_t flags, float *n_sq, dp_stream_t stream);

/* Bytes of workspace dp_clip_aggregate needs, or (size_t)-1 if invalid. */
size_t dp_clip_aggregate_workspace(int dtype, int B, int T, int d, int p);

/*
 * Which kernels serve a call: 1 if the MFMA kernels do (bf16 inputs on their
 * tiles), 0 if the generic kernels do (one thread per output element with
 * plain loads: correct, and covered by the same tests, but one to three orders
 * of magnitude slower), -1 if the arguments are invalid.  Host-only; nothing
 * is enqueued.  The MFMA conditions: the Hutchinson sketch and projection need
 * T % 128 == 0, p % 256 == 0, d % 128 == 0 and k <= 32 (Hutch++: s + r <= 32
 * and the same conditions on both widths); ghost needs T % 128 == 0 and d, p
 * multiples of 64; FGC and the clipped sum need T % 128 == 0 and d, p
 * multiples of 256.  Arguments as for the calls they describe (for these
 * queries B, T, d, p follow the call's validation; k is ignored for ghost and
 * FGC).  The pages fix no kernel; these only report this library's choice.
 */
int dp_norm_est_uses_mfma(int method, int dtype, int B, int T, int d, int p, int k);
int dp_clip_aggregate_uses_mfma(int dtype, int B, int T, int d, int p);

/*
 * Clip factors and the clipped sum of per-sample gradients of one layer.
 *
 *  c_i = 1 if n_sq[i] <= C^2 (0 and negative values included), C / sqrt(n_sq[i])
 *  otherwise, 0 if n_sq[i] is not finite (the sample is dropped and
 *  DP_STATUS_NONFINITE_NORM is ORed into the workspace's status word); then
 *      S[o][q] = sum_i c_i sum_t G_i[t][o] A_i[t][q]          (S = sum_i c_i G_i^T A_i)
 *  which is the second backward pass on the loss rescaled by c_i (glossary
 *  step 3-4 without the noise; summary step 4-5).
 *
 *  A [B][T][d], G [B][T][p] device (dtype); n_sq [B] fp32 device (squared norms
 *  summed over all layers); C > 0 finite.
 *  c_out   [B] fp32 device output, or NULL.
 *  S       [p][d] fp32 device output (the (p, d) weight layout), overwritten.
 *  ws      device workspace of ws_bytes >= dp_clip_aggregate_workspace(...);
 *          its first 8 bytes hold the sticky status word (see above).
 */
dp_status_t dp_clip_aggregate(int dtype, int B, int T, int d, int p, const void *A,
                              const void *G, const float *n_sq, float C, float *c_out, float *S,
                              void *ws, size_t ws_bytes, dp_stream_t stream);

/*
 * Noise and SGD update of one (p, d) fp32 parameter block, in place:
 *      theta[e] <- theta[e] - (eta / B) * (S[e] + sigma * C * xi[e]),  xi ~ N(0, 1)
 * (glossary, section DP-SGDのアルゴリズム, steps 4-5 with |B| = B).
 *  xi[e] for the flat index e = o * d + q is lane e mod 4 of the Philox4x32-10
 *  counter (low word of e/4, high word of e/4, 0xFFFFFFFF, layer) under key
 *  `seed`, turned into normals by Box-Muller on 24-bit uniforms.
 *  d, p >= 1; B >= 1; sigma >= 0 and C > 0 finite; eta finite.
 *  theta, S: [p][d] fp32 device (theta in/out, S read-only; they must not overlap).
 */
dp_status_t dp_noise_update(int d, int p, float *theta, const float *S, float sigma,
                            float C, float eta, int B, uint64_t seed, uint32_t layer,
                            dp_stream_t stream);

/* Bytes of workspace dp_clip_aggregate_update needs, or (size_t)-1 if invalid. */
size_t dp_clip_aggregate_update_workspace(int dtype, int B, int T, int d, int p);

/*
 * Steps 4-5 for one layer in one call: the clip factors and clipped sum of
 * dp_clip_aggregate, then the noise and update of dp_noise_update (same seed,
 * layer and B), i.e. theta <- theta - (eta / B) (sum_i c_i G_i^T A_i + sigma C xi)
 * (summary, section アルゴリズム的フロー, step 5; glossary steps 3-5).  The
 * result is bit-identical to dp_clip_aggregate followed by dp_noise_update;
 * the clipped sum is formed inside the update pass instead of being written
 * and read back (one launch and 8 bytes per parameter fewer when the sum is
 * split over token ranges).
 *  B >= 1 (it is also the |B| of the update); the other arguments as in the
 *  two calls.  S may be NULL (then the clipped sum is not stored); theta and S
 *  must not overlap.
 *  ws      device workspace of ws_bytes >= dp_clip_aggregate_update_workspace(...).
 */
dp_status_t dp_clip_aggregate_update(int dtype, int B, int T, int d, int p, const void *A,
                                     const void *G, const float *n_sq, float C, float sigma,
                                     float eta, uint64_t seed, uint32_t layer, float *theta,
                                     float *S, float *c_out, void *ws, size_t ws_bytes,
                                     dp_stream_t stream);

/*
 * The sticky device status flags of a workspace (DP_STATUS_* bits ORed by the
 * clip-factor calls above and below since the previous read), e.g.
 * DP_STATUS_NONFINITE_NORM when some sample's summed squared norm was NaN or
 * Inf and the sample was dropped (its c_i = 0; the randomized-clipping
 * summary, section アルゴリズム的フロー, step 4, leaves such values open).
 *  ws         the workspace passed to those calls (16-byte aligned device).
 *  flags_out  host pointer receiving the flags.
 * Enqueues an atomic read-and-clear of the word on `stream`, copies the value
 * to the host and synchronises `stream`: the only call of the library that
 * blocks the host.  Not for use under stream capture.  DP_ERR_INVALID_ARG for
 * a NULL or misaligned pointer; DP_ERR_HIP if a HIP call fails (then
 * *flags_out is unchanged).
 */
dp_status_t dp_read_device_status(void *ws, uint32_t *flags_out, dp_stream_t stream);

/* ---- batched calls over the linear layers of one step ----
 * One training step applies the method to every linear layer of the model:
 * the per-sample norm is summed over all layers before anything is clipped
 * (glossary page, section DP-SGDのアルゴリズム, steps 2-3: one clip factor per
 * sample from the whole gradient's norm), and each layer then gets its clipped
 * sum, noise and update (steps 4-5; summary, section アルゴリズム的フロー,
 * steps 3-6).  These two calls take all layers at once and compute exactly
 * what the per-layer calls compute, with fewer launches: the norm call draws
 * the probes of all layers in one launch (per 64 layers) and adds the layers'
 * estimates into n_sq in one pass; the update call forms the clip factors once.
 */
typedef struct dp_linear_layer {
  int d;              /* input width (columns of A) */
  int p;              /* output width (columns of G) */
  uint32_t layer;     /* layer id: keys the probe and noise streams, as `layer` above */
  const void *A;      /* [B][T][d] layer inputs, row-major, dtype of the call */
  const void *G;      /* [B][T][p] output gradients, row-major */
  float *theta;       /* [p][d] fp32 parameters (updated in place; unused by the norm call) */
} dp_linear_layer_t;

/* Bytes of workspace dp_norm_est_layers needs, or (size_t)-1 if invalid. */
size_t dp_norm_est_layers_workspace(int method, int dtype, int B, int T, int k, int nlayers,
                                    const dp_linear_layer_t *layers);

/*
 * n_sq[i] (= or, with DP_ACCUMULATE, +=) sum over the layers of the estimate
 * dp_norm_est gives for each (same method, k, seed, layer ids and flags).
 *  layers   host array of nlayers >= 1 descriptors (read during the call only;
 *           theta is not used); every layer's A and G as in dp_norm_est.
 * Hutch on bf16 inputs whose layers all take the MFMA path with at least 256
 * column blocks of the projection (e.g. B 8, T 4096, d >= 2048) runs batched:
 * one probe launch, sketch and projection per layer, one per-sample sum in
 * fp64 (the sum over layers is rounded to fp32 once, not once per layer).
 * Anything else runs the per-layer calls in order on the same workspace.
 * Errors: as dp_norm_est, for any layer.
 */
dp_status_t dp_norm_est_layers(int method, int dtype, int B, int T, int k, int nlayers,
                               const dp_linear_layer_t *layers, uint64_t seed, uint32_t flags,
                               float *n_sq, void *ws, size_t ws_bytes, dp_stream_t stream);

/* Bytes of workspace dp_clip_aggregate_update_layers needs, or (size_t)-1 if invalid. */
size_t dp_clip_aggregate_update_layers_workspace(int dtype, int B, int T, int nlayers,
                                                 const dp_linear_layer_t *layers);

/*
 * dp_clip_aggregate_update for every layer (same n_sq, C, sigma, eta and seed;
 * each layer's own id and theta), with the clip factors formed once.  S is not
 * stored.  c_out (may be NULL) and the status word as in dp_clip_aggregate.
 *  layers   host array of nlayers >= 1 descriptors (read during the call only);
 *           the thetas must not overlap each other or the workspace.
 * Launches.  A bf16 layer on the MFMA contraction whose count of 256 x 256
 * output tiles, (p / 256) (d / 256), is below 256 and divides 256 shares one
 * contraction launch with the next layers of the same tile count in the
 * array, 256 / tiles of them (at most 16) per launch: a full group fills the
 * chip without splitting the tokens, so each sum is written once instead of
 * as token-split partials that the update adds.  Such a layer's sum then adds
 * the tokens in fewer, longer runs than the per-layer call's, and its theta
 * agrees with the per-layer call's to fp32 rounding (still the same result
 * from run to run).  Every other layer, including one that finds no partner,
 * runs exactly the per-layer call's kernels: its theta is bit-identical.
 * Errors: as dp_clip_aggregate_update, for any layer.
 */
dp_status_t dp_clip_aggregate_update_layers(int dtype, int B, int T, int nlayers,
                                            const dp_linear_layer_t *layers, const float *n_sq,
                                            float C, float sigma, float eta, uint64_t seed,
                                            float *c_out, void *ws, size_t ws_bytes,
                                            dp_stream_t stream);

/* ---- timed variants: the same calls, plus live kernel timing ----
 * Identical to the call without "_timed", and additionally record the two
 * hipEvent_t handles ev_begin / ev_end (either may be NULL) on `stream`
 * immediately before the first and after the last launch of the call's main
 * kernels: dp_norm_est - the streaming passes over A and G (Hutch: sketch and
 * projection; Hutch++: all three passes with the QR between them; ghost: the
 * Gram kernel; FGC: the materialising contraction); dp_clip_aggregate - the
 * clipped-sum contraction (not the clip factors nor the split reduction);
 * dp_noise_update - the noise + update kernel.  The caller owns the events.
 */
dp_status_t dp_norm_est_timed(int method, int dtype, int B, int T, int d, int p, int k,
                              const void *A, const void *G, uint64_t seed, uint32_t layer,
                              uint32_t flags, float *n_sq, void *ws, size_t ws_bytes,
                              dp_stream_t stream, void *ev_begin, void *ev_end);
dp_status_t dp_clip_aggregate_timed(int dtype, int B, int T, int d, int p, const void *A,
                                    const void *G, const float *n_sq, float C, float *c_out,
                                    float *S, void *ws, size_t ws_bytes, dp_stream_t stream,
                                    void *ev_begin, void *ev_end);
dp_status_t dp_noise_update_timed(int d, int p, float *theta, const float *S, float sigma,
                                  float C, float eta, int B, uint64_t seed, uint32_t layer,
                                  dp_stream_t stream, void *ev_begin, void *ev_end);
/* dp_clip_aggregate_update with two event pairs: around the clipped-sum
 * contraction and around the (split-summing) noise + update kernel. */
dp_status_t dp_clip_aggregate_update_timed(int dtype, int B, int T, int d, int p, const void *A,
                                           const void *G, const float *n_sq, float C,
                                           float sigma, float eta, uint64_t seed, uint32_t layer,
                                           float *theta, float *S, float *c_out, void *ws,
                                           size_t ws_bytes, dp_stream_t stream,
                                           void *ev_agg_begin, void *ev_agg_end,
                                           void *ev_upd_begin, void *ev_upd_end);
/* Number of clipped-sum contraction launches dp_clip_aggregate_update_layers
 * makes for these layers (layers sharing a launch count once), or -1 if the
 * arguments are invalid; for timing and per-launch accounting. */
int dp_clip_aggregate_update_layers_launches(int dtype, int B, int T, int nlayers,
                                             const dp_linear_layer_t *layers);
/* dp_norm_est_layers, with ev_begin / ev_end around all layers' streaming
 * passes (after the probe launch, before the per-sample sum). */
dp_status_t dp_norm_est_layers_timed(int method, int dtype, int B, int T, int k, int nlayers,
                                     const dp_linear_layer_t *layers, uint64_t seed,
                                     uint32_t flags, float *n_sq, void *ws, size_t ws_bytes,
                                     dp_stream_t stream, void *ev_begin, void *ev_end);
/* dp_clip_aggregate_update_layers, with agg_begin[l] / agg_end[l] around layer
 * l's clipped-sum contraction and upd_begin[l] / upd_end[l] around its noise +
 * update kernel (arrays of nlayers hipEvent_t, any of them NULL).  A
 * contraction launch shared by several layers is bracketed by the pair of the
 * first of them; the others' pairs are both recorded right after it (zero
 * duration), so the pairs still add up to the contraction time of the call. */
dp_status_t dp_clip_aggregate_update_layers_timed(int dtype, int B, int T, int nlayers,
                                                  const dp_linear_layer_t *layers,
                                                  const float *n_sq, float C, float sigma,
                                                  float eta, uint64_t seed, float *c_out,
                                                  void *ws, size_t ws_bytes, dp_stream_t stream,
                                                  void *const *agg_begin, void *const *agg_end,
                                                  void *const *upd_begin, void *const *upd_end);

/* ---- RMSNorm gains (a parameter that is not a linear layer) ----
 *
 * The glossary page (section DP-SGDのアルゴリズム, steps 2-3) clips each
 * sample's whole gradient; for a gain gamma of RMSNorm (y_t = gamma * xhat_t)
 * sample i's gradient is v_i[c] = sum_t xhat_{i,t}[c] * delta_{i,t}[c], with
 * delta = dl_i/dy.  dp_rmsnorm_norm writes v (if not NULL) and n_sq[i] (=, or
 * += with DP_ACCUMULATE, to sum with the other layers) = ||v_i||^2.
 *  xhat, delta  [B][T][d], fp32 or bf16 (dtype), 16-byte aligned.
 *  v            [B][d] fp32 device, or NULL.
 *  ws           device workspace, ws_bytes >= dp_rmsnorm_norm_workspace(...).
 * dp_rmsnorm_clip_aggregate_update then takes the clip factors
 * c_i = min(1, C / sqrt(n_i)) of the summed norms (the same rule as
 * dp_clip_aggregate: non-finite n_i gives c_i = 0 and the status bit in the
 * workspace's status word) and
 * updates gamma [d] fp32: gamma <- gamma - (eta / B) (sum_i c_i v_i + sigma C xi),
 * xi from the noise stream of `layer` (give each parameter its own layer id).
 * S [d] (optional) receives the clipped sum; c_out [B] optional.
 */
size_t dp_rmsnorm_norm_workspace(int dtype, int B, int T, int d);
dp_status_t dp_rmsnorm_norm(int dtype, int B, int T, int d, const void *xhat, const void *delta,
                            uint32_t flags, float *n_sq, float *v, void *ws, size_t ws_bytes,
                            dp_stream_t stream);
size_t dp_rmsnorm_update_workspace(int B, int d);
dp_status_t dp_rmsnorm_clip_aggregate_update(int B, int d, const float *v, const float *n_sq,
                                             float C, float sigma, float eta, uint64_t seed,
                                             uint32_t layer, float *gamma, float *S,
                                             float *c_out, void *ws, size_t ws_bytes,
                                             dp_stream_t stream);

/* ---- embedding tables (a parameter that is not a linear layer) ----
 *
 * For an embedding table E [V][d] (h_t = E[id_t]) sample i's gradient has
 * row v equal to the sum of delta_{i,t} (= dl_i/dh_t) over the tokens with
 * id_t = v; dp_embedding_norm writes n_sq[i] (=, or += with DP_ACCUMULATE)
 * = the sum over the distinct ids of the squared row norms.
 *  ids    [B][T] int32 device; delta [B][T][d] fp32 or bf16 (16-byte aligned).
 *  T      0 <= T <= 16384 (the per-sample sort runs in LDS).
 * dp_embedding_clip_aggregate_update updates every row of E [V][d] fp32:
 * E <- E - (eta / B) (sum_i c_i grad_i + sigma C xi), with c_i = min(1,
 * C / sqrt(n_i)) as in dp_clip_aggregate and xi from the noise stream of
 * `layer` at flat index v d + column (the noise covers rows no token uses).
 * Ids outside [0, V) contribute nothing to the update.
 */
size_t dp_embedding_norm_workspace(int dtype, int B, int T, int d);
dp_status_t dp_embedding_norm(int dtype, int B, int T, int d, const int32_t *ids,
                              const void *delta, uint32_t flags, float *n_sq, void *ws,
                              size_t ws_bytes, dp_stream_t stream);
size_t dp_embedding_update_workspace(int dtype, int B, int T, int d, int V);
dp_status_t dp_embedding_clip_aggregate_update(int dtype, int B, int T, int d, int V,
                                               const int32_t *ids, const void *delta,
                                               const float *n_sq, float C, float sigma,
                                               float eta, uint64_t seed, uint32_t layer, float *E,
                                               float *c_out, void *ws, size_t ws_bytes,
                                               dp_stream_t stream);

/* ---- Poisson subsampling of the minibatch ----
 *
 * Glossary page, section DP-SGDのアルゴリズム, step 1: each step draws its
 * minibatch by Poisson subsampling, every one of the N training examples
 * independently with probability q (so |B| is random); step 5 divides the
 * noisy clipped sum by |B|.
 *
 * Example n is in step `step`'s minibatch when word n mod 4 of Philox4x32-10
 * at the counter (lo(n / 4), hi(n / 4), step, 0xFFFFFFFE) under key `seed` is
 * below floor(q 2^32) (integer comparison: q = 1 takes every example, q = 0
 * none).  Layer ids must stay below 0xFFFFFFFE so that this stream, the probe
 * stream and the noise stream never share a counter.
 *
 *  N       examples, 0 <= N <= 2^40; q in [0, 1].
 *  idx     int64 device array of idx_cap entries (NULL when idx_cap == 0):
 *          the first min(|B|, idx_cap) selected indices, ascending.
 *  count   int64 device scalar: |B| (also when it exceeds idx_cap).
 *  ws      device workspace, ws_bytes >= dp_poisson_sample_workspace(N).
 * Deterministic: the same arguments give the same indices on every call.
 * The caller gathers the selected examples into the first |B| slots of the
 * batch and passes B = |B| to the calls above, whose update divides by B
 * (the realized batch size).  For another denominator (the expected size
 * q N, say), pass eta' = eta B / denominator.  An empty minibatch has no
 * clipped sum; its noise-only update is dp_noise_update with S = 0, B = 1
 * and eta' = eta / denominator.
 */
size_t dp_poisson_sample_workspace(int64_t N); /* bytes, or (size_t)-1 if N is out of range */
dp_status_t dp_poisson_sample(uint64_t seed, uint32_t step, int64_t N, double q, int64_t *idx,
                              int64_t idx_cap, int64_t *count, void *ws, size_t ws_bytes,
                              dp_stream_t stream);

/* ---- Forward pass and backward pass 1 of a Llama MLP block ----
 *
 * The randomized-clipping summary (section アルゴリズム的フロー, steps 1-2)
 * runs a forward pass for the activations, then backward pass 1 for every
 * layer's per-sample output gradient; steps 3-5 are the calls above.  The
 * block is the MLP half of a Llama decoder layer (M = B T token rows, width d,
 * hidden width f; bf16 activations, fp32 accumulation):
 *   rstd = 1 / sqrt(mean(x^2) + eps), xhat = x rstd, y = gamma xhat     (RMSNorm)
 *   g = y Wg^T, u = y Wu^T, h = silu(g) u, out = x + h Wd^T   (SwiGLU, residual)
 * and, given the output gradient R = dL/d(out) from the layers above,
 *   G_down = R, dh = R Wd, G_gate = dh u silu'(g), G_up = dh silu(g),
 *   dy = G_gate Wg + G_up Wu, dx = rstd (gamma dy - xhat mean(gamma dy xhat)) + R.
 * The DP step then takes (A, G) = (y, G_gate), (y, G_up), (h, R) for the
 * three linears and (xhat, dy) for the gain (dp_rmsnorm_norm).
 *
 * Layouts: activations row-major [M][width] bf16, 16-byte aligned; weights
 * Wg, Wu [f][d] and Wd [d][f] bf16 (dp_weights_bf16 of the fp32 parameters);
 * the backward takes their transposes WgT, WuT [d][f] and WdT [f][d].  d and f
 * multiples of 256; any M >= 0.  Every buffer is caller-owned device memory;
 * outputs must not overlap inputs (out may equal x).  No workspace.
 */

/* W [p][d] = bf16(theta) and Wt [d][p] = its transpose (round to nearest
 * even); theta fp32 [p][d]; p, d multiples of 64; theta, W 16-byte aligned,
 * Wt 8-byte aligned. */
dp_status_t dp_weights_bf16(int p, int d, const float *theta, void *W, void *Wt,
                            dp_stream_t stream);

/* C [M][N] = bf16(A W^T (+ residual)): the forward of one linear layer.
 * A [M][K], W [N][K], residual [M][N] or NULL, C [M][N], all bf16; K a
 * multiple of 32, N of 256; A, W 16-byte aligned, residual and C 8-byte.
 * C must not overlap A or W. */
dp_status_t dp_linear_forward(int64_t M, int N, int K, const void *A, const void *W,
                              const void *residual, void *C, dp_stream_t stream);

/* Forward: x [M][d] -> xhat, y [M][d], rstd [M] fp32, g, u, h [M][f], out [M][d].
 * gamma [d] fp32 16-byte aligned; eps >= 0. */
dp_status_t dp_mlp_forward(int B, int T, int d, int f, float eps, const void *x,
                           const float *gamma, const void *Wg, const void *Wu, const void *Wd,
                           void *xhat, void *y, float *rstd, void *g, void *u, void *h, void *out,
                           dp_stream_t stream);

/* Backward pass 1: from x, rstd, g, u of the forward and dout = R [M][d],
 * writes G_gate, G_up [M][f], dy [M][d] and dx [M][d]. */
dp_status_t dp_mlp_backward(int B, int T, int d, int f, const void *x, const float *rstd,
                            const float *gamma, const void *g, const void *u, const void *WgT,
                            const void *WuT, const void *WdT, const void *dout, void *G_gate,
                            void *G_up, void *dy, void *dx, dp_stream_t stream);

/* ---- Forward pass and backward pass 1 of a Llama attention block ----
 *
 * The attention half of a Llama decoder layer (the randomized-clipping
 * summary, section アルゴリズム的フロー, steps 1-2), head width 64, H query
 * heads sharing KV key/value heads (head h uses key/value head h / (H / KV)):
 *   xhat, y = RMSNorm(x), gamma xhat
 *   q = y Wq^T [M][64 H], k = y Wk^T, v = y Wv^T [M][64 KV]
 *   q, k <- RoPE: in each head the pair (i, i + 32) is rotated by
 *           t base^(-i / 32) at position t (t = row % T)
 *   o_h = softmax(q_h k^T / 8 + causal mask) v,  out = x + o Wo^T
 * Layouts as for the MLP block; Wq [64 H][d], Wk, Wv [64 KV][d], Wo [d][64 H]
 * bf16; lse [B][H][T] fp32 is the natural log of each softmax row's
 * normaliser (the backward pass reads it).  T a multiple of 128, d, 64 H and
 * 64 KV multiples of 256.  No workspace.
 */

/* In place RoPE of x [M][64 n_heads] bf16 (16-byte aligned); inverse = 1 rotates
 * by the opposite angle (the transpose, used on gradients). */
dp_status_t dp_rope(int64_t M, int T, int n_heads, double base, int inverse, void *x,
                    dp_stream_t stream);

/* Causal grouped-query attention of B sequences of T tokens: q [B T][64 H],
 * k, v [B T][64 KV] -> o [B T][64 H], lse [B][H][T]. */
dp_status_t dp_attention_forward(int B, int T, int H, int KV, const void *q, const void *k,
                                 const void *v, void *o, float *lse, dp_stream_t stream);

/* The whole block forward: x [B T][d] -> xhat, y [B T][d], rstd [B T], q, k, v
 * (after RoPE), o, lse and out = x + o Wo^T. */
dp_status_t dp_attn_forward(int B, int T, int d, int H, int KV, float eps, double rope_base,
                            const void *x, const float *gamma, const void *Wq, const void *Wk,
                            const void *Wv, const void *Wo, void *xhat, void *y, float *rstd,
                            void *q, void *k, void *v, void *o, float *lse, void *out,
                            dp_stream_t stream);

/* Backward of the attention: from q, k, v, o, lse of the forward and dO [B T][64 H],
 * dq [B T][64 H], dk, dv [B T][64 KV] (dk, dv summed over each group's query
 * heads).  ws: device workspace, ws_bytes >= dp_attention_backward_workspace. */
size_t dp_attention_backward_workspace(int B, int T, int H);
dp_status_t dp_attention_backward(int B, int T, int H, int KV, const void *q, const void *k,
                                  const void *v, const void *o, const float *lse, const void *dO,
                                  void *dq, void *dk, void *dv, void *ws, size_t ws_bytes,
                                  dp_stream_t stream);

/* The whole block's backward pass 1: from the forward's x, rstd, q, k, v, o, lse,
 * the transposed bf16 weights WqT [d][64 H], WkT, WvT [d][64 KV], WoT [64 H][d]
 * and dout = R [B T][d], writes G_q [B T][64 H], G_k, G_v [B T][64 KV] (the output
 * gradients of the q, k, v projections, through RoPE's transpose), dy and dx
 * [B T][d].  The o projection's output gradient is R itself.
 * ws_bytes >= dp_attn_backward_workspace(B, T, H). */
size_t dp_attn_backward_workspace(int B, int T, int H);
dp_status_t dp_attn_backward(int B, int T, int d, int H, int KV, double rope_base, const void *x,
                             const float *rstd, const float *gamma, const void *q, const void *k,
                             const void *v, const void *o, const float *lse, const void *WqT,
                             const void *WkT, const void *WvT, const void *WoT, const void *dout,
                             void *G_q, void *G_k, void *G_v, void *dy, void *dx, void *ws,
                             size_t ws_bytes, dp_stream_t stream);

/* ---- test hooks: expose the random streams for bit-level parity checks ---- */

/*
 * Measurement hook (not part of the method): a plain streaming read of `bytes`
 * (a multiple of 16) at `buf` (16-byte aligned device memory) with nblocks
 * workgroups (1 .. 65536) of 256 threads, 16-byte loads, eight in flight per
 * thread; out[x] (device, nblocks uint32) receives the XOR of every 32-bit word
 * workgroup x read.  It gives the practical HBM read ceiling that the
 * bandwidth-bound kernels are compared with.  DP_ERR_INVALID_ARG for bad
 * pointers or sizes.
 */
dp_status_t dp_stream_read(const void *buf, size_t bytes, uint32_t *out, int nblocks,
                           dp_stream_t stream);

/* out[4 n] = Philox4x32-10 words of the n counters ctr[4 n] (device arrays). */
dp_status_t dp_philox_u32(uint64_t seed, const uint32_t *ctr, uint32_t *out, size_t n,
                          dp_stream_t stream);

/* Pt[j][r] (fp32 device, [k][p]) = entry (r, j) of the probe P of `sample` in `layer`. */
dp_status_t dp_probe_fill(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k,
                          float *Pt, dp_stream_t stream);

/* The same with probe flags: DP_PROBE_RADEMACHER gives the sign probe (fp32
 * +1 / -1); other bits are rejected. */
dp_status_t dp_probe_fill_ex(uint64_t seed, uint32_t layer, uint32_t sample, int p, int k,
                             uint32_t flags, float *Pt, dp_stream_t stream);

/* xi[e - offset] for e in [offset, offset + n): the noise normals (fp32 device). */
dp_status_t dp_noise_fill(uint64_t seed, uint32_t layer, uint64_t offset, size_t n,
                          float *xi, dp_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DPRC_H */
