/*
 * libkdloss: fused, chunked KL distillation loss over a language model's
 * output head, for AMD Instinct MI355X (gfx950).
 *
 * The loss is the forward KL divergence KL(p_teacher || q_student) of
 * "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
 * Chunked KL Loss" (§1; §3 "Online distillation").  Two variants:
 *
 *  - top-K (§3 "Offline distillation"): the teacher is a cached top-K per
 *    token.  Its K logits are renormalised at temperature tau; the student's
 *    log-probabilities are gathered at the K cached indices, and log Z over the
 *    whole vocabulary is the only full-vocabulary reduction.
 *  - full vocabulary (KDFlow abstract, thelatestinai.com/papers/2606.20005):
 *    teacher logits are recomputed from the teacher's final hidden states
 *    through a frozen copy of the teacher's output head.
 *
 * Both are fused with the output projection Z = H.W (§3 "Fused chunked KL"):
 * logit tiles live on chip only, the full [T, V] logit tensor is never
 * written, and the backward pass recomputes the projection chunk by chunk of
 * token rows (one extra projection per chunk, as in output-head gradient
 * checkpointing).  Each variant also has a single forward + backward call
 * that keeps one chunk's logits instead of recomputing them, and _ex calls
 * with optional parts of the loss (per-token temperature, a partial-mass
 * teacher, an LM cross-entropy term, KL mixing); see their sections.
 *
 * Definitions, per valid row t (s = z / tau with z = H_t . W, L_t = logsumexp(s)):
 *   top-K:  p = softmax(A_t / tau) over the K entries;
 *           KL_t = sum_k p_k (log p_k - s[I_tk] + L_t)
 *           dZ_t = (g_t / tau) (softmax(s) - scatter_add(I_t, p))
 *   full:   u = (Ht_t . Wt) / tau, p = softmax(u), Lt = logsumexp(u);
 *           KL_t = sum_v p_v (u_v - s_v) - Lt + L_t
 *           dZ_t = (g_t / tau) (softmax(s) - p)
 *   dH = dZ . W^T, dW = H^T . dZ.  There is no tau^2 factor; the caller may
 *   scale g.  Duplicate top-K indices add (scatter-add).
 *
 * Conventions shared by every call:
 *  - All tensors are dense and row-major.  H [T,d], W [d,V], Ht [T,dt],
 *    Wt [dt,V], topk_idx [T,K] int32, topk_logits [T,K] float32, mask [T]
 *    uint8 (1 = valid row, 0 = masked; NULL = all rows valid), grad_kl [T]
 *    float32, kl/lse [T] float32, z_topk [T,K] float32, dH [T,d] in the input
 *    dtype, dW [d,V] float32.  A weight stored as nn.Linear's [V,d] must be
 *    transposed by the caller.
 *  - dtype KD_BF16: H, W, Ht, Wt and dH are bfloat16; products accumulate in
 *    float32.  KD_F32: they are float32 and the contraction runs on fp32
 *    matrix cores.  kl, lse, grad_kl, dW are float32 in both cases.
 *  - d, dt and V must be multiples of 8 (bf16) or 4 (fp32); 1 <= K <= V,
 *    K <= KD_MAX_K and T * (K + 1) < 2^31.  Otherwise the call returns
 *    KD_ERR_UNSUPPORTED.
 *  - Pointers to H, W, Ht, Wt, dH, dW must be 16-byte aligned, all other
 *    arrays 4-byte aligned, the workspace 256-byte aligned
 *    (KD_ERR_ALIGNMENT).
 *  - Masked rows get kl = 0, lse = 0, z_topk = 0 and dH = 0, add nothing to
 *    dW and are never read beyond mask[t] (NaN or out-of-range indices there
 *    do not leak).  Their flops are skipped: valid rows are compacted on the
 *    device.
 *  - Ownership: the caller allocates every buffer, including the workspace.
 *    The library never allocates device memory, so the extra device memory of
 *    a call is exactly its workspace.  The library keeps no state between
 *    calls except the optional profiling record (kd_profile_*), is safe to
 *    call from several host threads, and is asynchronous: each call enqueues
 *    its kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *    returns without synchronising.
 *  - Errors: arguments are checked on the host before any kernel is
 *    enqueued; a failed check returns its status and enqueues nothing.  A
 *    failed launch returns KD_ERR_HIP.  kd_last_error() gives a message for
 *    the last failure on the calling thread.  Index range is checked on the
 *    device only on request (kd_topk_opts.check_indices); otherwise an index
 *    outside [0, V) in a valid row is ignored by the gather (its teacher
 *    probability still counts in the teacher terms).
 *  - T = 0: the forward calls enqueue nothing; the backward calls set dW to
 *    zero (the gradient of an empty sum) and touch nothing else.
 *  - Deterministic: split reductions run in a fixed order, so the same call
 *    on the same inputs gives the same bits.
 */
#ifndef KDLOSS_H
#define KDLOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KD_MAX_K 8192
#define KD_DEFAULT_CHUNK_ROWS 4096

typedef enum kd_status {
  KD_OK = 0,
  KD_ERR_INVALID_ARG = 1,          /* null pointer, negative size, bad tau, K < 1 ... */
  KD_ERR_UNSUPPORTED = 2,          /* valid but not handled: K > KD_MAX_K, d or V not a multiple of 8/4 */
  KD_ERR_ALIGNMENT = 3,            /* a pointer is not aligned as required */
  KD_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes below the size query's answer */
  KD_ERR_INDEX_OUT_OF_RANGE = 5,   /* a cached index or label of a valid row outside [0, V), found by the
                                      index check that kd_topk_opts.check_indices asks for */
  KD_ERR_HIP = 6                   /* a HIP launch or runtime call failed */
} kd_status;

/* KD_DTYPE_MAX_ENUM makes every non-negative int a value of the type, so
 * that a wrong code from a C caller is a value the checks reject
 * (KD_ERR_INVALID_ARG) rather than an out-of-range enumeration. */
typedef enum kd_dtype { KD_F32 = 0, KD_BF16 = 1, KD_DTYPE_MAX_ENUM = 0x7fffffff } kd_dtype;

/* ---------------------------------------------------------------- top-K */

/* Workspace bytes that both kd_topk_kl_fwd and kd_topk_kl_bwd need for this
 * shape (one size serves both calls).  chunk_rows: token rows per backward
 * chunk (0 = KD_DEFAULT_CHUNK_ROWS; rounded up to a multiple of 256; clamped
 * to the rows present; for bf16 also clamped so that the chunk's dZ buffer,
 * chunk * roundup(V, 256) * 2 bytes, stays under 4 GiB, the reach of the
 * direct-to-LDS loads that read it, that cap being rounded down to a
 * multiple of KD_DEFAULT_CHUNK_ROWS when it is at least that: 16384 rows at
 * V = 128256).  Every call
 * taking chunk_rows applies the same rule.  Larger chunks trade workspace
 * for speed at long context (fewer read-modify-writes of dW).  The size is
 * affine in T for a fixed chunk size: the per-row part is about 10*K + 44
 * bytes, the rest does not depend on T.
 * Returns KD_OK and writes *bytes, or an argument error. */
kd_status kd_topk_kl_workspace_size(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                                    int64_t chunk_rows, size_t* bytes);

/* Forward: per-token KL and the saved log-normaliser.
 *   H [T,d], W [d,V] (dtype dt); topk_idx [T,K]; topk_logits [T,K];
 *   mask [T] or NULL; tau > 0 and finite.
 *   kl [T] (out), lse [T] (out: L_t = logsumexp_v(z_tv / tau), kept for the
 *   backward call), z_topk [T,K] (out, optional: the raw logits z at the
 *   cached indices, NULL to skip).
 * Logits are produced tile by tile on chip; a running max and sum give
 * lse and the index-match epilogue gathers the K cached entries
 * (§3 "Offline distillation" and "Fused chunked KL"). */
kd_status kd_topk_kl_fwd(const void* H, const void* W, const int32_t* topk_idx,
                         const float* topk_logits, const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                         float* kl, float* lse, float* z_topk,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Backward: dH [T,d] (dtype dt, overwritten) and dW [d,V] (float32,
 * overwritten) for the upstream per-token gradient grad_kl [T] (the caller
 * owns the reduction: a mean over N valid tokens passes 1/N).  lse must be
 * the forward call's output for the same inputs.  Rows are processed in
 * chunks of chunk_rows valid rows: each chunk recomputes its logit tiles,
 * writes dZ for that chunk only, then runs dH = dZ.W^T and dW += H^T.dZ
 * (§3 "Fused chunked KL": one extra output projection per chunk). */
kd_status kd_topk_kl_bwd(const void* H, const void* W, const int32_t* topk_idx,
                         const float* topk_logits, const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                         const float* lse, const float* grad_kl,
                         void* dH, float* dW, int64_t chunk_rows,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Forward and backward in one call, for callers that know grad_kl before
 * the loss is evaluated (a mean over a known token count, the loss-only
 * benchmark).  Same arguments and outputs as kd_topk_kl_fwd followed by
 * kd_topk_kl_bwd with the same chunk_rows, and the same bits: each chunk's
 * forward keeps its logits (fp32, in the workspace), so dZ is computed from
 * them instead of from a second projection.  That trades the pages'
 * recompute (§3 "Fused chunked KL": one extra output projection per chunk,
 * like output-head gradient checkpointing) for C * roundup(V, 256) * 4 more
 * workspace bytes, where C is the chunk size, plus T * (K + 1) * 4 for the
 * z_topk gather.  kd_topk_kl_fwd_bwd_workspace_size
 * gives the size; T = 0 sets dW to zero and touches nothing else. */
kd_status kd_topk_kl_fwd_bwd_workspace_size(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                                            int64_t chunk_rows, size_t* bytes);
kd_status kd_topk_kl_fwd_bwd(const void* H, const void* W, const int32_t* topk_idx,
                             const float* topk_logits, const uint8_t* mask, float tau,
                             int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                             const float* grad_kl, float* kl, float* lse, float* z_topk,
                             void* dH, float* dW, int64_t chunk_rows,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- top-K options
 * Optional parts of the top-K loss.  The _ex calls take the same arguments
 * as the calls above plus `opts`; opts = NULL, or every field zero, is the
 * plain call.  The backward call must get the same options as the forward
 * call that produced lse.  With every option, per valid row t:
 *   tau_t = tau_rows[t] (else tau);  s = z / tau_t;  L_t = logsumexp(s)
 *   p_k   = exp(A_tk / tau_t - teacher_lse[t])  (else softmax(A_t / tau_t));
 *   m_t   = sum_k p_k (1 when renormalised)
 *   KD_t  = sum_k p_k log p_k - sum_k p_k s[I_tk] + m_t L_t
 *   CE_t  = L_t - s[labels[t]]
 *   kl_t  = (1 - ce_weight) KD_t + ce_weight CE_t
 *   dZ_t  = (g_t / tau_t) ((1 - ce_weight)(m_t softmax(s) - scatter_add(I_t, p))
 *                          + ce_weight (softmax(s) - onehot(labels[t])))
 * Sources: per-token temperature, the adaptive-distillation abstract on the
 * WASD page (thelatestinai.com/papers/2610.07706); cached probabilities with
 * their unnormalised partial mass and the support identity above, §3
 * "Offline distillation"; the language-modelling loss mixed with the
 * distillation loss, the teacher-strength abstract
 * (thelatestinai.com/papers/2605.11513), with CE the one-entry case of the
 * same loss at the same temperature (tau = 1 gives the plain LM loss).
 * KL mixing (rev_weight = r > 0) adds the reverse direction on the cached
 * entries, where both sides are known: with q~ = softmax_k(s[I_tk]) and
 * p^ = softmax_k(A_tk / tau_t), both over the K entries (each entry its own
 * outcome, p^ renormalised also under a partial mass),
 *   RKL_t = sum_k q~_k (log q~_k - log p^_k)
 *   KD_t is replaced by (1 - r) KD_t + r RKL_t in kl_t, and dZ_t gains
 *   (g_t / tau_t)(1 - ce_weight) r q~_k (log q~_k - log p^_k - RKL_t)
 *   at column I_tk (scatter-add).
 * q~ is computed from the raw logits at the cached entries that the forward
 * writes to z_topk: with r > 0 the forward and single calls need their
 * z_topk output, and the backward call gets the forward's z_topk in
 * opts.z_topk (KD_ERR_INVALID_ARG if NULL).  Source: forward and
 * reverse token-level KL and their mixture, the KL-direction abstract
 * (thelatestinai.com/papers/2606.20005); the restriction to the cached
 * entries is this library's reading, since the teacher is known only there.
 * The vocabulary shard calls reject r > 0 (KD_ERR_UNSUPPORTED): q~ needs the
 * student's logits at all K entries.
 * Only the per-row constants and the weights of the support entries change,
 * so every option keeps the tiles, workspace size and speed of the plain
 * call (KL mixing adds one small per-row pass).  Argument errors: ce_weight
 * or rev_weight outside [0, 1] or not finite, ce_weight > 0 without labels,
 * or rev_weight > 0 without z_topk: KD_ERR_INVALID_ARG; ce_weight > 0 with
 * K = KD_MAX_K: KD_ERR_UNSUPPORTED (the label is entry K + 1); misaligned
 * arrays: KD_ERR_ALIGNMENT.  Values are not checked: tau_rows must be
 * finite and > 0 and labels in [0, V) on valid rows (masked rows are never
 * read).
 * Index check on request (check_indices != 0): the teacher preparation
 * counts, on the device, the cached indices (and labels) of valid rows that
 * lie outside [0, V); the call then waits for that count (one
 * synchronisation of `stream`) and, if it is not zero, returns
 * KD_ERR_INDEX_OUT_OF_RANGE without enqueuing anything more: kl, lse,
 * z_topk, dH and dW are left as they were.  Masked rows are not checked.
 * Without it an out-of-range index of a valid row matches no vocabulary
 * column (its probability still counts in the teacher terms).  The shard
 * calls do not know the whole head's width and reject the flag
 * (KD_ERR_UNSUPPORTED). */
typedef struct kd_topk_opts {
  const float* tau_rows;     /* [T] per-token temperature, or NULL */
  const float* teacher_lse;  /* [T] teacher log-normaliser at tau_t (partial mass), or NULL */
  const int32_t* labels;     /* [T] next-token labels of the CE term, or NULL */
  float ce_weight;           /* weight of the CE term in [0, 1]; 0 = distillation only */
  int32_t check_indices;     /* nonzero: check the index range on the device (see above) */
  float rev_weight;          /* weight r of the reverse KL on the cached entries in [0, 1]; 0 = none */
  const float* z_topk;       /* [T,K] the forward's z_topk, read by the backward call when r > 0 */
} kd_topk_opts;

kd_status kd_topk_kl_fwd_ex(const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logits, const uint8_t* mask, float tau,
                            const kd_topk_opts* opts,
                            int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                            float* kl, float* lse, float* z_topk,
                            void* workspace, size_t workspace_bytes, void* stream);
kd_status kd_topk_kl_bwd_ex(const void* H, const void* W, const int32_t* topk_idx,
                            const float* topk_logits, const uint8_t* mask, float tau,
                            const kd_topk_opts* opts,
                            int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                            const float* lse, const float* grad_kl,
                            void* dH, float* dW, int64_t chunk_rows,
                            void* workspace, size_t workspace_bytes, void* stream);
kd_status kd_topk_kl_fwd_bwd_ex(const void* H, const void* W, const int32_t* topk_idx,
                                const float* topk_logits, const uint8_t* mask, float tau,
                                const kd_topk_opts* opts,
                                int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                                const float* grad_kl, float* kl, float* lse, float* z_topk,
                                void* dH, float* dW, int64_t chunk_rows,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- top-K, one vocabulary shard
 * The top-K loss with the output head split by vocabulary columns over R
 * ranks, the tensor-parallel layout of an output head (the loss-only
 * benchmark reports time and memory at the largest tensor-parallel rank,
 * App. B).  Rank r holds W_r = columns [v0, v0 + V) of the head, [d,V]
 * row-major (V here is the shard's width), and every rank holds all of H,
 * topk_idx (indices into the whole head), topk_logits, mask and the options.
 * One step:
 *   1. each rank: kd_topk_kl_fwd_shard -> rec_r [T,4], trow [T,2]
 *   2. all-gather rec over the ranks into rec [R,T,4] (rank order)
 *   3. each rank: kd_topk_kl_shard_combine -> kl [T] and lse [T], the
 *      log-normaliser over the whole head (the same on every rank)
 *   4. each rank: kd_topk_kl_bwd_shard with that lse -> dH_r [T,d] float32,
 *      a partial of dH, and dW_r [d,V] float32, the shard's columns of dW
 *   5. sum dH_r over the ranks (all-reduce); dW stays sharded.
 * The library does none of the exchanges; the caller's collectives move
 * 16 bytes per row in step 2 and d float32 per row in step 5.  The results
 * are those of the unsharded calls up to rounding (the shard records merge
 * like the kernels' own split partials).  The single call has no shard form:
 * its backward needs the whole head's lse before the exchange.
 *
 * Records, per valid row t (s = z / tau_t over the shard's columns, hits =
 * the cached entries whose index lies in [v0, v0 + V)):
 *   rec[t]  = (m, l, c, 0) with m + log2(l) = log2(sum over the shard of
 *             exp(s)) (m a base-2 maximum, l a scaled sum) and
 *             c = sum over hits of w_k s[I_tk] (w: the entries' weights,
 *             p_k, or with a CE term (1 - ce_weight) p_k and ce_weight at the
 *             label); masked rows: all zero
 *   trow[t] = (sum_k w_k log p_k, mass), the teacher terms over all K entries
 *             (the same on every rank; masked rows: zero)
 *   the combine: L_t = ln 2 * log2(sum_r l_r 2^(m_r - M)) + ln 2 * M with
 *   M = max_r m_r; kl_t = trow.x - sum_r c_r + trow.y * L_t.
 * Argument rules are those of the _ex calls, except that K may exceed the
 * shard's width V, v0 must be >= 0 (KD_ERR_INVALID_ARG) and v0 + V below
 * 2^30 (KD_ERR_UNSUPPORTED).  rec must be 16-byte and trow 8-byte aligned;
 * dH here is always float32 (the partial is summed before any rounding). */
/* Workspace bytes for a shard's forward and backward (one size serves
 * both; the rules of kd_topk_kl_workspace_size at the shard's width V). */
kd_status kd_topk_kl_shard_workspace_size(int64_t T, int64_t d, int64_t V, int64_t v0, int64_t K,
                                          kd_dtype dt, int64_t chunk_rows, size_t* bytes);
/* z_topk, when given, holds the logits of the shard's hits and 0 elsewhere,
 * so the ranks' arrays add up to the unsharded one. */
kd_status kd_topk_kl_fwd_shard(const void* H, const void* W, const int32_t* topk_idx,
                               const float* topk_logits, const uint8_t* mask, float tau,
                               const kd_topk_opts* opts,
                               int64_t T, int64_t d, int64_t V, int64_t v0, int64_t K, kd_dtype dt,
                               float* rec, float* trow, float* z_topk,
                               void* workspace, size_t workspace_bytes, void* stream);
/* rec [R,T,4] (R records in rank order), trow [T,2] -> kl [T], lse [T];
 * masked rows get 0.  R >= 1 and R * T < 2^31.  No workspace. */
kd_status kd_topk_kl_shard_combine(const float* rec, int64_t R, const float* trow, const uint8_t* mask,
                                   int64_t T, float* kl, float* lse, void* stream);
kd_status kd_topk_kl_bwd_shard(const void* H, const void* W, const int32_t* topk_idx,
                               const float* topk_logits, const uint8_t* mask, float tau,
                               const kd_topk_opts* opts,
                               int64_t T, int64_t d, int64_t V, int64_t v0, int64_t K, kd_dtype dt,
                               const float* lse, const float* grad_kl,
                               float* dH, float* dW, int64_t chunk_rows,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- full vocabulary */

/* Workspace bytes for kd_full_kl_fwd and kd_full_kl_bwd (one size serves
 * both).  dt_hidden is the teacher's hidden width. */
kd_status kd_full_kl_workspace_size(int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                                    int64_t chunk_rows, size_t* bytes);

/* Forward: kl [T], lse_s [T] (student), lse_t [T] (teacher), all float32 out.
 * Student logits H.Ws and teacher logits Ht.Wt (the teacher's final hidden
 * states through its frozen output head: KDFlow abstract) are produced tile
 * by tile side by side; a dual running max/sum and the running sum of
 * p_v (u_v - s_v) give the KL without either [T,V] tensor (the online
 * coupled two-distribution form of the StreamKL abstract). */
kd_status kd_full_kl_fwd(const void* H, const void* Ws, const void* Ht, const void* Wt,
                         const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                         float* kl, float* lse_s, float* lse_t,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Backward to the student only: dH [T,d] (dtype dt) and dWs [d,V] float32,
 * both overwritten.  No gradient flows to Ht or the frozen Wt. */
kd_status kd_full_kl_bwd(const void* H, const void* Ws, const void* Ht, const void* Wt,
                         const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                         const float* lse_s, const float* lse_t, const float* grad_kl,
                         void* dH, float* dWs, int64_t chunk_rows,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Forward and backward in one call, when grad_kl is known up front.  Same
 * arguments and outputs as kd_full_kl_fwd followed by kd_full_kl_bwd with
 * the same chunk_rows, equal up to rounding: each chunk's two projections
 * run one head at a time through the 256-column top-K tiles, which keep the
 * logits (fp32, in the workspace); one elementwise pass over them then gives
 * both KL terms with the final log-normalisers and dZ, instead of
 * recomputing both projections (the trade of §3 "Fused chunked KL", made the
 * other way).  That costs 2 * C * roundup(V, 256) * 4 more workspace bytes
 * for a chunk of C rows; kd_full_kl_fwd_bwd_workspace_size gives the size.
 * T = 0 sets dWs to zero and touches nothing else. */
kd_status kd_full_kl_fwd_bwd_workspace_size(int64_t T, int64_t d, int64_t dt_hidden, int64_t V,
                                            kd_dtype dt, int64_t chunk_rows, size_t* bytes);
kd_status kd_full_kl_fwd_bwd(const void* H, const void* Ws, const void* Ht, const void* Wt,
                             const uint8_t* mask, float tau,
                             int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                             const float* grad_kl, float* kl, float* lse_s, float* lse_t,
                             void* dH, float* dWs, int64_t chunk_rows,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- full-vocabulary options
 * The _ex calls take the arguments of the calls above plus `opts` (NULL or
 * every field zero = the plain call) and kl_rev [T] float32, the reverse
 * KL(q || p) of each row: written by the forward calls when not NULL (zero
 * on masked rows), and read by kd_full_kl_bwd_ex, which needs the forward
 * call's values when rev_weight > 0 (KD_ERR_INVALID_ARG if NULL then).  The
 * backward call must get the same options as the forward call.  Per valid
 * row t, with tau_t = tau_rows[t] (else tau), s = z / tau_t, u = Ht_t.Wt / tau_t,
 * q = softmax(s), p = softmax(u) and r = rev_weight:
 *   kl_t = (1 - r) KL(p || q) + r KL(q || p)
 *   dZ_t = (g_t / tau_t) [(1 - r)(q - p) + r q (log q - log p - KL(q || p))]
 * (KL mixing of the forward and reverse token-level KL: the KL-direction
 * abstract, thelatestinai.com/papers/2606.20005; per-token temperature: the
 * adaptive-distillation abstract on the WASD page).  The forward tiles keep
 * both running sums, so no option changes the tiles' work.  Argument
 * errors: rev_weight outside [0, 1] or not finite: KD_ERR_INVALID_ARG;
 * misaligned tau_rows or kl_rev: KD_ERR_ALIGNMENT.  tau_rows values must be
 * finite and > 0 on valid rows (not checked). */
typedef struct kd_full_opts {
  const float* tau_rows;  /* [T] per-token temperature, or NULL */
  float rev_weight;       /* weight r of the reverse KL in [0, 1]; 0 = forward KL */
} kd_full_opts;

kd_status kd_full_kl_fwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt,
                            const uint8_t* mask, float tau, const kd_full_opts* opts,
                            int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                            float* kl, float* lse_s, float* lse_t, float* kl_rev,
                            void* workspace, size_t workspace_bytes, void* stream);
kd_status kd_full_kl_bwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt,
                            const uint8_t* mask, float tau, const kd_full_opts* opts,
                            int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                            const float* lse_s, const float* lse_t, const float* kl_rev,
                            const float* grad_kl, void* dH, float* dWs, int64_t chunk_rows,
                            void* workspace, size_t workspace_bytes, void* stream);
kd_status kd_full_kl_fwd_bwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt,
                                const uint8_t* mask, float tau, const kd_full_opts* opts,
                                int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                                const float* grad_kl, float* kl, float* lse_s, float* lse_t,
                                float* kl_rev, void* dH, float* dWs, int64_t chunk_rows,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- full vocabulary, one vocabulary shard
 * The full-vocabulary loss with both heads split by the same vocabulary
 * columns over R ranks (the tensor-parallel layout of the top-K shard
 * section above).  Rank r holds Ws_r and Wt_r, columns [v0, v0 + V) of the
 * student's and the teacher's heads ([d,V] and [dt,V] row-major, V the
 * shard's width), and all of H, Ht, mask and the options.  One step:
 *   1. each rank: kd_full_kl_fwd_shard -> rec_r [T,8]
 *   2. all-gather rec over the ranks into rec [R,T,8] (rank order)
 *   3. each rank: kd_full_kl_shard_combine -> kl, lse_s, lse_t (and kl_rev),
 *      those of the whole heads
 *   4. each rank: kd_full_kl_bwd_shard with them -> dH_r [T,d] float32, a
 *      partial of dH, and dWs_r [d,V] float32, the shard's columns of dWs
 *   5. sum dH_r over the ranks; dWs stays sharded.
 * Record, per valid row t, over the shard's columns (y = x log2(e) / tau_t
 * for the student's logits ys and the teacher's yt):
 *   rec[t] = (ms, ls, mt, lt, R, R2, 0, 0) with ms + log2(ls) and
 *   mt + log2(lt) the base-2 log-normalisers of ys and yt over the shard,
 *   R = sum 2^(yt - mt) (yt - ys), R2 = sum 2^(ys - ms) (ys - yt);
 *   masked rows: all zero.  Records merge like the forward's own split
 *   partials.  The workspace is kd_full_kl_workspace_size at the shard's
 *   width; rec must be 16-byte aligned.  The combine takes the rev_weight
 *   of the options (the record does not depend on it); the backward needs
 *   the same options as the forward and, when rev_weight > 0, kl_rev. */
kd_status kd_full_kl_fwd_shard(const void* H, const void* Ws, const void* Ht, const void* Wt,
                               const uint8_t* mask, float tau, const kd_full_opts* opts,
                               int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                               float* rec, void* workspace, size_t workspace_bytes, void* stream);
/* rec [R,T,8] -> kl, lse_s, lse_t [T] and kl_rev [T] (nullable); masked rows
 * get 0.  R >= 1, R * T < 2^30, rev_weight in [0, 1].  No workspace. */
kd_status kd_full_kl_shard_combine(const float* rec, int64_t R, const uint8_t* mask, int64_t T,
                                   float rev_weight, float* kl, float* lse_s, float* lse_t,
                                   float* kl_rev, void* stream);
kd_status kd_full_kl_bwd_shard(const void* H, const void* Ws, const void* Ht, const void* Wt,
                               const uint8_t* mask, float tau, const kd_full_opts* opts,
                               int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                               const float* lse_s, const float* lse_t, const float* kl_rev,
                               const float* grad_kl, float* dH, float* dWs, int64_t chunk_rows,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- top-K forward without a workspace
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and bits as kd_topk_kl_fwd, without the workspace: the
 * forward's scratch (the sorted teacher entries, the compaction list, the
 * split partials and the panel copy of a chunk's rows of H) lives in a fixed
 * device array of KD_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or event; the kd_profile_* record skips it) and reads
 * the array's device address once per device, on its first call there, with
 * that device current; `stream` must belong to the current device.
 * A shape whose forward needs more scratch than that returns
 * KD_ERR_UNSUPPORTED before anything is enqueued (at d = 3072,
 * V = 128256, K = 64 in bf16, 37,823 rows fit, or 27,293 with z_topk,
 * whose gather needs 4 (K + 1) bytes more per row); the other argument
 * errors are kd_topk_kl_fwd's.  Every call on one GPU shares its array:
 * calls that overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.  Nothing in the array needs to start
 * at zero; each call writes what it reads. */
#define KD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kd_status kd_topk_kl_fwd_noalloc(const void* H, const void* W, const int32_t* topk_idx,
                                 const float* topk_logits, const uint8_t* mask, float tau,
                                 int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                                 float* kl, float* lse, float* z_topk, void* stream);

/* ---------------------------------------------------------------- errors, version */

const char* kd_status_string(kd_status s);
/* Message for the last failed call on the calling thread ("" if none). */
const char* kd_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int kd_version(void);

/* ---------------------------------------------------------------- profiling
 * While enabled, every kernel the library enqueues is bracketed by a pair of
 * HIP events on the same stream.  kd_profile_count() waits for the recorded
 * events and folds them into per-kernel totals; kd_profile_get() reads entry
 * i: the kernel's name, its launch count and its summed duration in ms.
 * kd_profile_reset() drops the record.  Not thread-safe against concurrent
 * calls that profile. */
kd_status kd_profile_enable(int on);
int kd_profile_count(void);
kd_status kd_profile_get(int i, const char** name, int64_t* launches, double* total_ms);
kd_status kd_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* KDLOSS_H */
