/*
 * orpo_head.h — C ABI of the MI355X (gfx950) flash-CCE ORPO head.
 *
 * The head turns response hidden states h[M,d] into per-token log-probs through an LM head W[V,d]
 * without ever materialising the [M,V] logits, reduces them to per-branch means, takes the ORPO
 * loss, and back-propagates it to dh[M,d] and dW[V,d] by recomputing the logits tile by tile.
 * Sources (the pages): "Training — design (ORPO, flash-CCE head, prefix sharing, segmented
 * backward)" §1 "The objective" and §5.1 "The head"; its older revision "ORPO training — design",
 * "Memory & speed optimization", ranked lever 1 and its "Implementation spec — fused linear-CE
 * log-prob head"; "Steel flash-CCE — handoff", "The architecture" and Glossary D "The epilogue".
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) must point to device memory of the GPU that is current on the calling
 *    thread; pointers marked (host) to host memory. All device buffers are owned by the caller: the
 *    library allocates nothing in these calls and keeps no pointer after a call returns.
 *  - Work is enqueued asynchronously on `stream`. Outputs are valid once the stream has reached
 *    the call's end; inputs and the workspace must stay alive until then.
 *  - Host-detectable argument errors (null pointers, sizes, formats, a workspace that is too small)
 *    return an error status before anything is enqueued; the library never aborts. Data errors
 *    that only the device can see (a label outside [0,V) that is not the ignore index, a branch
 *    without a valid token, non-monotone segment offsets) set bits in a status word held in the
 *    workspace, readable with orpo_read_status().
 *  - Calls that share one workspace must not overlap (same stream, or ordered by the caller).
 *  - Results are deterministic: no atomics take part in any floating-point reduction.
 */
#ifndef ORPO_HEAD_H
#define ORPO_HEAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORPO_OK = 0,
  ORPO_EINVAL = -1,        /* null pointer, negative or inconsistent size, bad option          */
  ORPO_EUNSUPPORTED = -2,  /* a valid request this library does not implement (see each call)   */
  ORPO_ENOWS = -3,         /* workspace pointer null or smaller than the *_workspace_bytes size */
  ORPO_EHIP = -4,          /* a HIP runtime call failed (see orpo_last_hip_error)               */
  ORPO_EDATA = -5          /* orpo_check only: the device set a data-error bit in the status word */
} orpo_status;

/* Storage formats. ORPO_Q4G64: 4-bit affine codes, w = scale * q + bias per group of 64 along d,
 * packed 8 codes per uint32 word, LSB first (code j of a row is bits [4(j%8), 4(j%8)+4) of word
 * j/8), with bf16 scale[V, d/64] and bias[V, d/64] ("ORPO training — design", the flash-CCE Metal
 * kernel note on in-kernel affine dequantisation; "Steel flash-CCE — handoff", Gotchas item 4). */
typedef enum { ORPO_F32 = 0, ORPO_BF16 = 1, ORPO_Q4G64 = 2 } orpo_fmt;

/* Bits of the device status word. */
enum {
  ORPO_DATA_BAD_LABEL = 1u << 0,    /* a label outside [0,V) that is not ignore_index (treated as ignored) */
  ORPO_DATA_EMPTY_BRANCH = 1u << 1, /* a branch with no valid token (its mean, the loss and g are NaN)      */
  ORPO_DATA_BAD_OFFSETS = 1u << 2   /* segment offsets not monotone within [0,M] (loss and g are NaN)       */
};

/* Option bits of orpo_head_desc.flags. */
enum {
  ORPO_DW_ACCUMULATE = 1u << 0,     /* orpo_head_bwd adds into dW instead of overwriting it */
  ORPO_DH_BF16 = 1u << 1            /* orpo_head_bwd writes dh as bf16 (bf16 and 4-bit heads)  */
};

typedef struct {
  int64_t M;            /* tokens (rows of h), >= 0                                             */
  int64_t d;            /* hidden size, > 0, multiple of 64                                     */
  int64_t V;            /* vocabulary size, > 0                                                 */
  int32_t h_fmt;        /* ORPO_F32 or ORPO_BF16; row-major [M,d]                               */
  int32_t w_fmt;        /* ORPO_F32 (needs h_fmt F32), ORPO_BF16 or ORPO_Q4G64 (need h_fmt BF16) */
  float softcap;        /* > 0: z = softcap * tanh(raw / softcap); <= 0: z = raw. At most 1024 */
                        /* (ORPO_EUNSUPPORTED above: z is evaluated in fp32 as               */
                        /* softcap * (1 - 2 / (1 + e^(2 raw / softcap))), whose absolute error */
                        /* grows like softcap * 2^-22)                                         */
  int32_t ignore_index; /* label value of ignored / padding tokens (conventionally -100)        */
  uint32_t flags;       /* ORPO_DW_ACCUMULATE | ORPO_DH_BF16                                    */
  float skip_eps;       /* backward coefficient filter: 0 = exact backward; > 0 (bf16 and 4-bit
                         * heads only) drops from dh every 256-token x 64-entry coefficient block,
                         * and from dW every 256-entry x 64-token block, whose max |coeff| < skip_eps
                         * (their GEMM K steps are skipped). An approximation, opt-in; the pages'
                         * default is 1e-5 ("Steel flash-CCE — handoff", Glossary E "Backward
                         * approximations"). With skip_eps > 0 orpo_head_fwd also records per-tile
                         * logit maxima in its workspace, for orpo_head_bwd's cold-tile skip.    */
} orpo_head_desc;

/* The head weights: `w` is W[V,d] row-major in w_fmt (for ORPO_Q4G64 the packed uint32 words
 * [V, d/8]); `scales` and `biases` are bf16 [V, d/64] for ORPO_Q4G64 and must be NULL otherwise. */
typedef struct {
  const void* w;
  const void* scales;
  const void* biases;
} orpo_weight;

/* Workspace sizes in bytes (0 on invalid arguments). The forward workspace grows as 256 + 8 * NBLK
 * * M (per-token partials over NBLK vocabulary splits, like lse it is O(M)); the backward
 * workspace holds two coefficient tiles of fixed size (double-buffered), independent of M beyond
 * one token chunk, and for a small M (few dh tiles, each with a long vocabulary K, split over
 * several workgroups) up to 64 MiB of fp32 dh partial sums, which are added in a fixed order. The
 * loss workspace (O(n_pairs)) serves both orpo_loss and orpo_loss_full. */
size_t orpo_head_fwd_workspace_bytes(const orpo_head_desc* desc);
size_t orpo_head_bwd_workspace_bytes(const orpo_head_desc* desc);
size_t orpo_loss_workspace_bytes(int64_t M, int32_t n_pairs);

/*
 * orpo_head_fwd — per-token log-prob and log-sum-exp without the [M,V] logits.
 *   z_tv = softcap(h_t . W_v); lse_t = log sum_v exp(z_tv); logp_t = z_t[y_t] - lse_t.
 * ("Training — design" §5.1 "The head"; older revision, the spec's forward: online softmax over
 * vocabulary tiles with target capture, storing O(M) state only; "Steel flash-CCE — handoff",
 * "The architecture", forward: per-split partials merged across splits.)
 *   h      (device) [M,d] in desc->h_fmt
 *   W      (device) see orpo_weight
 *   labels (device) int32 [M]; ignore_index marks tokens that get no log-prob
 *   logp   (device) float [M] out: logp_t, 0 for ignored tokens
 *   lse    (device) float [M] out: lse_t for every row (kept for orpo_head_bwd)
 *   ws     (device) >= orpo_head_fwd_workspace_bytes(desc) bytes, 256-byte aligned
 * Returns ORPO_EUNSUPPORTED for d not a multiple of 64 or format combinations not listed above.
 */
orpo_status orpo_head_fwd(const orpo_head_desc* desc, const void* h, orpo_weight W,
                          const int32_t* labels, float* logp, float* lse, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/*
 * orpo_head_fwd_noalloc — orpo_head_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * kernels and results, bit for bit, with the workspace taken from a file-scope device array of
 * ORPO_NOALLOC_SCRATCH_BYTES bytes (4 MiB) that the library holds on each GPU it runs on
 * until the process ends. No hipMalloc, hipFree or other allocation happens in the call.
 *   desc, h, W, labels, logp, lse, stream as for orpo_head_fwd (no ws arguments).
 *   Returns ORPO_ENOWS when the forward's workspace for desc (orpo_head_fwd_workspace_bytes)
 *   exceeds that size: about 256 + 8 * max(65536, M) bytes (+ 32 per 256 x 256 tile with
 *   skip_eps > 0), i.e. up to ~500k tokens; nothing is enqueued then.
 *   Every call on a GPU shares that GPU's array, so calls that overlap on one GPU (different
 *   streams, or threads) race and must be ordered by the caller. The array's device status word
 *   is overwritten by the next call: data-error bits are not reported by this entry point (a bad
 *   label is still treated as ignored, as in orpo_head_fwd).
 */
#define ORPO_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
orpo_status orpo_head_fwd_noalloc(const orpo_head_desc* desc, const void* h, orpo_weight W,
                                  const int32_t* labels, float* logp, float* lse,
                                  hipStream_t stream);

/*
 * orpo_loss — segmented per-branch mean, scalar ORPO epilogue (float64) and per-token cotangent.
 *   ell_b = mean of logp over the valid tokens of branch b = [off[b], off[b+1]); branch 2p is the
 *   chosen, 2p+1 the rejected response of pair p. With log1mexp(x) = log(max(1 - e^x, 1e-12)):
 *   log_odds_p = (lw - lr) - (log1mexp(lw) - log1mexp(lr)); or = mean_p softplus(-log_odds_p);
 *   nll = mean_p(-lw); loss = nll + lambda * or. g_t = dloss/dlogp_t = (dloss/dell_b) / n_b.
 * ("Training — design" §1 "The objective"; older revision, "File-by-file changes", orpoLoss and
 * orpoMetrics; §4's note on the 1/(1-P) factor of the odds-ratio gradient.)
 *   M, n_pairs     tokens (>= 0) and pairs (>= 1)
 *   seg_offsets    (device) int32 [2*n_pairs + 1], monotone within [0, M]
 *   logp, labels   (device) [M] as produced for / consumed by orpo_head_fwd
 *   V, ignore_index the vocabulary size and ignore label: only labels in [0,V) that differ from
 *                  ignore_index count (a bad label is ignored here too, as in orpo_head_fwd)
 *   out            (device) double [5 + 2*n_pairs] out: loss, nll, or, accuracy (mean 1[lw > lr]),
 *                  margin (mean log_odds), then lw[n_pairs], then lr[n_pairs]
 *   g              (device) float [M] out: the cotangent fed to orpo_head_bwd (0 off-branch / ignored)
 *   ws             (device) >= orpo_loss_workspace_bytes(M, n_pairs) bytes
 */
orpo_status orpo_loss(int64_t M, int32_t n_pairs, const int32_t* seg_offsets, const float* logp,
                      const int32_t* labels, int64_t V, int32_t ignore_index, double lambda,
                      double* out, float* g, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * orpo_loss_full — orpo_loss with the full-scope NLL: the chosen sequence's NLL covers its
 * supervised prompt positions as well as the response.
 *   Spans per pair p: prompt [off[3p], off[3p+1]), chosen [off[3p+1], off[3p+2]), rejected
 *   [off[3p+2], off[3p+3]). With n_q, n_w the valid-token counts and pm, lw the means of the prompt
 *   and chosen spans: NLL_p = -(n_q pm + n_w lw) / (n_q + n_w), the pages' combination
 *   -((P-1) pm + M lw) / ((P-1) + M) with P-1 supervised prompt positions and M response tokens;
 *   nll = mean_p NLL_p. The odds ratio, accuracy and margin use the response means lw, lr exactly
 *   as in orpo_loss, and lambda weights only the odds ratio. g_t = (dloss/dmean_s) / n_s for a
 *   valid token of span s, prompt tokens included. ("Training — design" §1 "The objective", the
 *   sft_scope `full` option.)
 *   seg_offsets    (device) int32 [3*n_pairs + 1], monotone within [0, M]
 *   out            (device) double [5 + 3*n_pairs] out: loss, nll, or, accuracy, margin, then
 *                  lw[n_pairs], lr[n_pairs], then pm[n_pairs] (0 for a prompt span without a valid
 *                  token)
 *   Other arguments, the workspace size and the error behaviour as for orpo_loss. A prompt span
 *   without a valid token is allowed (it then weighs nothing and every result equals orpo_loss's on
 *   the two response spans); a response span without one sets ORPO_DATA_EMPTY_BRANCH.
 */
orpo_status orpo_loss_full(int64_t M, int32_t n_pairs, const int32_t* seg_offsets,
                           const float* logp, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double lambda, double* out, float* g, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * Sibling objectives on the same per-token log-probs (orpo_head_fwd's logp) and the same backward
 * (orpo_head_bwd takes their g). Workspace for both entry points below:
 * orpo_objective_workspace_bytes(M, n_spans) with n_spans = 2 * n_pairs or n_seqs.
 */
size_t orpo_objective_workspace_bytes(int64_t M, int32_t n_spans);

typedef enum {
  ORPO_PREF_SIMPO = 1,
  ORPO_PREF_DPO = 2,
  ORPO_PREF_IPO = 3,
  ORPO_PREF_HINGE = 4
} orpo_pref_kind;

/*
 * orpo_pref_loss — pairwise preference losses (chosen span 2p, rejected span 2p+1 of seg_offsets,
 * [2*n_pairs + 1] monotone within [0, M]; only valid labels count, as in orpo_loss).
 *   ORPO_PREF_SIMPO: lw, lr = mean logp of each span; per pair
 *     L = softplus(-beta ((lw - lr) - gamma)); accuracy = mean 1[lw > lr]; margin = mean (lw - lr).
 *     ("Training — design" §8.3 "Objective variants and data".)
 *   ORPO_PREF_DPO: sw, sr = summed logp of each span (the sequence log-prob); with the cached
 *     reference sums ref_sums (device double [2*n_pairs], same span order),
 *     Delta = beta [(sw - ref_w) - (sr - ref_r)], L = -log sigmoid(Delta); accuracy = mean
 *     1[Delta > 0]; margin = mean Delta. gamma is unused. (The post-training design page, "Stage
 *     P1 — DPO": seq_logprob as a per-sequence sum, the DPO loss, only policy terms carry
 *     gradient.)
 *   ORPO_PREF_IPO and ORPO_PREF_HINGE: "Training — design" §8.3 names IPO and hinge/SLiC as
 *     siblings without formulas; both are read as the published losses on the log-ratio margin
 *     h = (v_w - ref_w) - (v_r - ref_r), where ref_sums holds reference values of the same kind
 *     (means for IPO, sums for hinge) and is optional (NULL: reference-free, ref = 0).
 *     IPO: v = mean logp (as SimPO), L = (h - 1/(2 beta))^2, beta > 0 required.
 *     HINGE: v = summed logp (as DPO), L = max(0, 1 - beta h), zero gradient at the kink.
 *     accuracy = mean 1[h > 0]; margin = mean h. gamma is unused.
 *   loss = mean over pairs. g_t = dloss/dlogp_t: dL/dv / n for the means (SimPO, IPO), dL/dv for
 *   the sums (DPO, hinge); 0 for ignored / off-span tokens.
 *   out   (device) double [3 + 2*n_pairs]: loss, accuracy, margin, then the chosen values [n_pairs]
 *         (lw or sw), then the rejected ones [n_pairs]
 *   Errors and status bits as for orpo_loss (ORPO_EINVAL also for an unknown kind, a DPO call
 *   without ref_sums, or IPO with beta <= 0).
 */
orpo_status orpo_pref_loss(int32_t kind, int64_t M, int32_t n_pairs, const int32_t* seg_offsets,
                           const float* logp, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double beta, double gamma, const double* ref_sums,
                           double* out, float* g, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * orpo_grpo_loss — GRPO's clipped policy-gradient loss with the k3 KL term, per completion token
 * (the post-training design page, "Stage P3 — GRPO", (c) and (d)).
 *   Completion s covers tokens [seg_offsets[s], seg_offsets[s+1]) (int32 [n_seqs + 1], monotone
 *   within [0, M]); only its valid labels count. With rho_t = exp(logp_t - old_logp_t) and the
 *   completion's advantage A_s (advantages: device float [n_seqs], e.g. group-normalised rewards):
 *     pg_t = -min(rho_t A_s, clip(rho_t, 1 - clip_eps, 1 + clip_eps) A_s),
 *     k3_t = exp(ref_t - logp_t) - (ref_t - logp_t) - 1,
 *     loss = mean_s [ mean_{t in s} (pg_t + beta k3_t) ]   (per-completion token mean, then mean).
 *   g_t = (dpg_t + beta dk3_t) / (n_s n_seqs): dpg_t = -A_s rho_t where the unclipped term is the
 *   minimum (ties included), 0 where the clipped one is; dk3_t = 1 - exp(ref_t - logp_t).
 *   old_logp, ref_logp (device) float [M]: the sampling policy's and the reference's log-probs of
 *   the same tokens (inputs; no gradient flows into them).
 *   out   (device) double [4]: loss, pg (mean policy-gradient term), kl (mean k3), clip fraction
 *         (share of valid tokens whose clipped term is the strict minimum)
 *   Errors and status bits as for orpo_loss (an empty completion sets ORPO_DATA_EMPTY_BRANCH).
 */
orpo_status orpo_grpo_loss(int64_t M, int32_t n_seqs, const int32_t* seg_offsets,
                           const float* logp, const float* old_logp, const float* ref_logp,
                           const float* advantages, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double clip_eps, double beta, double* out,
                           float* g, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * orpo_head_bwd — dh = coeff . W and dW = coeff^T . h, recomputing the logits tile by tile.
 *   coeff_tv = g_t * (1[v = y_t] - exp(z_tv - lse_t)) * sech^2(raw_tv / softcap)   (sech^2 = 1
 *   without a softcap). ("ORPO training — design", the spec's backward: recompute each vocabulary
 *   tile from the saved lse and form g (onehot - softmax) sech^2; "Steel flash-CCE — handoff",
 *   Glossary D "softmax-onehot coeff". dW is the same chain rule for the weight operand.)
 *   h, W, labels   as for orpo_head_fwd
 *   lse            (device) float [M] from orpo_head_fwd on the same h, W, labels
 *   g              (device) float [M] dloss/dlogp (e.g. from orpo_loss); ignored tokens must hold 0
 *   dh             (device) float [M,d] out (overwritten); with ORPO_DH_BF16 bf16 [M,d]: the
 *                  same fp32 sums, rounded to nearest even once (the workspace then also holds an
 *                  fp32 [C,d] accumulator when V spans several backward blocks; ORPO_EUNSUPPORTED
 *                  for fp32 heads). The sum over vocabulary blocks stays fp32 either way: the
 *                  pages found bf16 summation across blocks to be the dominant gradient error
 *                  ("ORPO training — design", "Memory & speed optimization", the vocab-blocked
 *                  note).
 *   dW             (device) float [V,d] out (overwritten, or accumulated with ORPO_DW_ACCUMULATE);
 *                  NULL computes dh only. Must be NULL for ORPO_Q4G64 (a quantised head is frozen).
 *                  With M = 0 it is set to zero (left as is with ORPO_DW_ACCUMULATE).
 *   ws             (device) >= orpo_head_bwd_workspace_bytes(desc) bytes
 *   fwd_ws         (device, optional) the workspace of the orpo_head_fwd call that produced lse,
 *                  with the same desc; read only with desc->skip_eps > 0, where its per-tile logit
 *                  maxima let the backward skip whole cold coefficient tiles (exactly the blocks
 *                  the filter would drop). NULL: the filter alone. Ignored when skip_eps is 0.
 *   With desc->skip_eps > 0 (the coefficient filter) the workspace also holds the filter's block
 *   flags, and ORPO_EUNSUPPORTED is returned (and 0 by orpo_head_bwd_workspace_bytes) for fp32
 *   heads and for a vocabulary block or token chunk of more than 8192 64-wide slices, i.e. above
 *   524288 entries or tokens (reachable only through orpo_set_bwd_tiling: the default 256 MiB
 *   budget keeps bf16 blocks within it). The launches are then traced with the exact method's work
 *   (skipped blocks included).
 */
orpo_status orpo_head_bwd(const orpo_head_desc* desc, const void* h, orpo_weight W,
                          const int32_t* labels, const float* lse, const float* g, void* dh,
                          float* dW, void* ws, size_t ws_bytes, const void* fwd_ws,
                          hipStream_t stream);

/* ---- The FP8 head: low-precision logit operands (opt-in approximation) ----------------------
 * The pages plan a lower-precision head ("Training — design", §8.1 "Deferred performance levers",
 * the W4A16 head GEMM item): half-width operands for the head's logit GEMM with fp32 accumulation, the
 * forward first, the backward's gradient GEMMs left at the higher precision until a range probe
 * clears them (their surviving coefficients are tiny tails), the exact mode kept as the parity
 * mode. On gfx950 the next format below bf16 is the 8-bit float of its 32x32x64 MFMA, so here:
 *   - h and W are quantised per row to FP8 E4M3 with one power-of-two scale per row
 *     (orpo_quantize_fp8; the MFMA applies the scales itself, so the products are exact);
 *   - orpo_head_fwd_fp8 takes logp and lse over raw = dequant(hq) . dequant(Wq)^T;
 *   - orpo_head_bwd_fp8 recomputes those logits for the coefficients and forms dh = coeff . W and
 *     dW = coeff^T . h with the unquantised bf16 h and W, as orpo_head_bwd does.
 * Results differ from the exact head by the quantisation (per element at most 2^-4 relative); they
 * match a float64 evaluation of the same definition on the same codes up to fp32 accumulation. */
typedef struct {
  const uint8_t* hq;     /* (device) [M, d] E4M3 codes of h, row-major                               */
  const uint8_t* h_exp;  /* (device) [M] E8M0 row exponents: row t of h is hq[t] * 2^(h_exp[t] - 127) */
  const uint8_t* wq;     /* (device) [V, d] E4M3 codes of W                                            */
  const uint8_t* w_exp;  /* (device) [V] E8M0 row exponents of W                                       */
} orpo_fp8_operands;

/*
 * orpo_quantize_fp8 — bf16 rows to E4M3 codes and power-of-two row scales.
 *   x    (device) bf16 [rows, cols] row-major, finite, 16-byte aligned; cols a multiple of 8
 *   q    (device) uint8 [rows, cols] out, 8-byte aligned: the E4M3 code nearest to x * 2^-e, ties to
 *        the even code, a negative value that rounds to zero keeping its sign (code 0x80). E4M3:
 *        1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, largest value 448; the NaN code
 *        S.1111.111 is never produced
 *   exps (device) uint8 [rows] out: e + 127, with 2^e the smallest power of two (e >= -127) for
 *        which max|x| <= 448 * 2^e (e = 0 for an all-zero row)
 * Returns ORPO_EINVAL for negative rows, cols not a positive multiple of 8, null or misaligned
 * pointers (rows > 0). One launch on `stream`, no workspace.
 */
orpo_status orpo_quantize_fp8(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* exps,
                              hipStream_t stream);

/*
 * orpo_q4_stage — a 4-bit head (ORPO_Q4G64) dequantised once into bf16 rows, so that a step can run
 * the bf16 kernels on it instead of dequantising the same weight tile again in every token tile.
 * The map is the format's affine one ("ORPO training — design", the flash-CCE Metal kernel note
 * on in-kernel affine dequantisation; "Training — design" §5.1 "The head", where the 4-bit head's
 * operands are dequantised for the logit products): w_bf16[v, k] = bf16(scale * q + bias), the
 * product and sum in fp32 and one rounding to nearest even, the same arithmetic the 4-bit tiled
 * loops apply to each tile they stage. orpo_head_fwd / orpo_head_bwd with w_fmt = ORPO_BF16 on the
 * staged rows therefore see the operand values that w_fmt = ORPO_Q4G64 gives them.
 *   W       device: words [V, d/8] (uint32, 4-byte aligned), bf16 scales and biases [V, d/64]
 *   V, d    V > 0 and at most INT32_MAX; d > 0, a multiple of 64 and at most 2^20
 *   w_bf16  device output, bf16 [V, d] row-major, 16-byte aligned, caller-owned (2 V d bytes);
 *           it must not overlap W
 * Errors: ORPO_EINVAL for bad sizes, a null or misaligned pointer (nothing is launched). Reads
 * and writes only the arrays named; asynchronous on `stream`.
 */
orpo_status orpo_q4_stage(orpo_weight W, int64_t V, int64_t d, void* w_bf16, hipStream_t stream);

/*
 * orpo_head_fwd_fp8 — orpo_head_fwd with the logits taken from FP8 operands.
 *   desc   the bf16 head being approximated: h_fmt = w_fmt = ORPO_BF16 and d a multiple of 128
 *          (else ORPO_EUNSUPPORTED); M, V, softcap, ignore_index, skip_eps as for orpo_head_fwd,
 *          except that skip_eps > 0 with a softcap above 40 is ORPO_EUNSUPPORTED here
 *   q      the quantised h and W (orpo_quantize_fp8); NULL or a NULL member (M > 0): ORPO_EINVAL
 *   labels, logp, lse, ws, ws_bytes, stream as for orpo_head_fwd (ws: orpo_head_fwd_workspace_bytes)
 */
orpo_status orpo_head_fwd_fp8(const orpo_head_desc* desc, const orpo_fp8_operands* q,
                              const int32_t* labels, float* logp, float* lse, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * orpo_head_bwd_fp8 — orpo_head_bwd for the FP8 head: lse from orpo_head_fwd_fp8 on the same
 * operands, the coefficients g (onehot - softmax) sech^2 from the recomputed FP8 logits, and
 * dh = coeff . W, dW = coeff^T . h with the bf16 h and W given here. Arguments as for
 * orpo_head_bwd (ws: orpo_head_bwd_workspace_bytes, ORPO_DH_BF16 and ORPO_DW_ACCUMULATE honoured),
 * plus q as for orpo_head_fwd_fp8 (and desc under the same restrictions); fwd_ws (optional) is
 * that forward's workspace.
 */
orpo_status orpo_head_bwd_fp8(const orpo_head_desc* desc, const orpo_fp8_operands* q,
                              const void* h, orpo_weight W, const int32_t* labels,
                              const float* lse, const float* g, void* dh, float* dW, void* ws,
                              size_t ws_bytes, const void* fwd_ws, hipStream_t stream);

/* Backward tiling: the token chunk C (a multiple of 256, default 8192) and the byte budget of one
 * coefficient tile [C, BVb] (two are used). With a budget, BVb is the largest multiple of 256 that
 * fits (at least 256). By default (0) the budget is 256 MiB and BVb is further limited to
 * max(16384, V/8 rounded up to 256) (and never above V), so that a small vocabulary still
 * pipelines over several blocks. 0 restores a default. Process-wide; call it only while no call of this library is in
 * flight, and size workspaces after it. Returns ORPO_EINVAL for a chunk that is not a multiple of
 * 256, a negative value, a chunk above 2^31 tokens or a budget above 2^40 bytes (these bounds keep
 * every workspace size far from wrapping a size_t). */
orpo_status orpo_set_bwd_tiling(int64_t chunk_tokens, size_t coeff_bytes);

/* Kernel tracing (a profiling aid). While enabled, every kernel this library launches is bracketed
 * by a pair of HIP events recorded on the launch's stream (up to max_launches launches), tagged with
 * its kind and its algorithmic floating-point work (2*d flops per (token, vocabulary) product for
 * the forward and for coefficient tiles, 4*d for dh + dW tiles (2*d for dh alone); 0 for merge and
 * loss).
 * orpo_trace_collect waits for the recorded events of one kind and returns their totals;
 * orpo_trace_reset starts a new record.
 * Process-wide and not thread-safe; enabling allocates events (host API only, no device memory). */
typedef enum {
  ORPO_K_FWD = 0,    /* forward logits + online softmax                                  */
  ORPO_K_MERGE = 1,  /* cross-split merge -> lse, logp                                   */
  ORPO_K_LOSS = 2,   /* segmented means + ORPO epilogue + g                              */
  ORPO_K_COEFF = 3,  /* backward launch with coefficient tiles only (first of a pass)    */
  ORPO_K_DHDW = 4,   /* backward launch with dh / dW tiles only (last of a pass)         */
  ORPO_K_BWD = 5,    /* backward launch with both (all the others)                       */
  ORPO_K_QUANT = 6,  /* FP8 row quantisation (orpo_quantize_fp8)                          */
  ORPO_K_STAGE = 7,  /* 4-bit head staged as bf16 rows (orpo_q4_stage)                    */
  ORPO_K_DHSUM = 8,  /* sum of split dh tiles' partials (small M; orpo_head_bwd)          */
  ORPO_K_COUNT = 9
} orpo_kernel_kind;
orpo_status orpo_trace_enable(int32_t max_launches);   /* 0 disables and releases the events */
orpo_status orpo_trace_collect(int32_t kind, int64_t* launches, double* total_ms, double* flops);
orpo_status orpo_trace_reset(void);                    /* forget the records, keep the events  */

/* Waits for `stream` and copies the status word of `ws` (a workspace used by any call above) to
 * *status_out (host). Returns ORPO_EHIP if the wait or copy fails. */
orpo_status orpo_read_status(const void* ws, uint32_t* status_out, hipStream_t stream);

/*
 * orpo_check — the data-error check of the boundary: waits for `stream`, then reads the status
 * word of `ws` (device; a workspace used by orpo_head_fwd, orpo_loss or a sibling loss) and
 * returns ORPO_OK when no bit is set, ORPO_EDATA when one is (orpo_read_status gives the bits:
 * ORPO_DATA_*). The device never aborts on bad data; the affected tokens or branches are treated
 * as documented under each call. ORPO_EINVAL for a null ws, ORPO_EHIP if the wait or copy fails.
 */
orpo_status orpo_check(const void* ws, hipStream_t stream);

/* Text for a status code (static storage). Takes any int32 value (an orpo_status is passed as
 * one); codes outside orpo_status give "unknown status". */
const char* orpo_status_string(int32_t status);

/* The last HIP error code seen by this library on the calling thread (hipSuccess if none). */
int32_t orpo_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ORPO_HEAD_H */
