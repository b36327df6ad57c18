/*
 * am.h - C ABI of the MI355X (gfx950) attention-matching KV compaction library.
 *
 * Per KV head and a set of n reference queries, the library computes the full-cache
 * statistics (row log-normalizer, attention output, per-key attention score), selects
 * t of the T keys, fits per-key biases beta so that the compacted attention mass matches
 * the full cache, and fits compacted values C_v so that the compacted attention output
 * matches it. The problem statement followed is the one in the "Compaction" blog post,
 * §Fast KV Compaction via Attention Matching: K, V in R^{T x d} become C_k, C_v in
 * R^{t x d} with C_k a subset of K, plus beta in R^t; the three steps are highest-attention
 * key selection, NNLS on the mass equations for w = exp(beta), and least squares on the
 * output equations for C_v. Attention follows "Latent Compaction with Test-Time Training",
 * §3 Preliminaries (Eq. 1) and §3.1 (Eq. 2-4, biased compacted attention).
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer owned by the caller, 16-byte aligned.
 *     The library keeps no pointer after a call returns and allocates no device memory:
 *     scratch comes from the caller's workspace (size from am_workspace_bytes).
 *   - Tensors are dense row-major, batched over h independent head problems:
 *     Q [h, n, d], K and V [h, T, d] in the problem dtype; lse [h, n] f32; O [h, n, d] f32;
 *     key_score [h, T] f32; idx [h, t] int32; C_k [h, t, d] problem dtype; beta [h, t] f32;
 *     C_v [h, t, d] f32.
 *   - Causal problems put query i at position i / group and let it see keys
 *     0 .. i / group; compacted keys keep their original positions (Latent Compaction,
 *     §3.1 "Handling Subsequent Tokens": no renumbering), so the same rule masks them.
 *   - Calls only ENQUEUE work on `stream` (NULL = the default stream) and never
 *     synchronize. Inputs, outputs and workspace must stay alive until the stream has
 *     passed the work. Calls on different streams with disjoint buffers are independent.
 *   - Arguments are validated on the host before any launch. A failed validation returns
 *     an error and launches nothing. Conditions found on the device (NNLS not converged,
 *     a singular ridge system, non-finite values) are reported per head through the
 *     optional head_status array (AM_HEAD_* bits), never by a return code.
 *   - Results are deterministic: fixed reduction orders and no floating-point atomics.
 */
#ifndef AM_H
#define AM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* am_stream_t;

typedef enum {
  AM_OK = 0,
  AM_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, t outside [1, T], ... */
  AM_ERR_UNSUPPORTED = -2, /* valid request the library does not implement: d not 64/128,
                              n or T above 2^30, or t above 8192 in the fit calls */
  AM_ERR_WORKSPACE = -3,   /* ws_bytes smaller than am_workspace_bytes() */
  AM_ERR_DEVICE = -4       /* a HIP launch or device query failed */
} am_status;

typedef enum { AM_F32 = 0, AM_BF16 = 1 } am_dtype;

/* Per-key selection statistic of p_ij = exp(s_ij - lse_i) over the n queries.
 * RMS sqrt(sum_i p^2 / n) is the one the Attention Matching baseline uses (Latent
 * Compaction, App. A.3); MEAN is sum_i p / n; MAX is max_i p (Latent Compaction Eq. 6). */
typedef enum { AM_SCORE_RMS = 0, AM_SCORE_MEAN = 1, AM_SCORE_MAX = 2 } am_score_mode;

/* Weighting of the mass equations (blog, §Choosing beta). RELATIVE divides equation i by
 * its full-cache mass Z_i (design M_ij = exp(s_i,c_j - lse_i), target 1). ABSOLUTE keeps
 * the literal equations, shifted by the largest lse so that they fit fp32. */
typedef enum { AM_MASS_RELATIVE = 0, AM_MASS_ABSOLUTE = 1 } am_mass_mode;

/* Per-head device status bits (head_status arrays). */
enum {
  AM_HEAD_OK = 0,
  AM_HEAD_NNLS_NOT_CONVERGED = 1, /* KKT tolerance not reached within nnls_max_iter */
  AM_HEAD_CHOL_PIVOT = 2,         /* a ridge Cholesky pivot not above 2^-40 times its
                                     diagonal entry: A^T A + lambda I is singular at the
                                     precision of the solve (lambda = 0 with dependent
                                     columns of A); C_v is then not meaningful */
  AM_HEAD_NONFINITE = 4,          /* a non-finite value reached a fit */
  AM_HEAD_TIMEOUT = 8             /* workgroups of a multi-workgroup step did not meet in
                                     time (the head's outputs are then incomplete) */
};

typedef struct {
  int64_t heads;   /* 1 <= h <= 65535 independent head problems */
  int64_t n;       /* reference queries per head, >= 1 */
  int64_t T;       /* full-cache keys per head, >= 1 */
  int64_t d;       /* head dimension: 64 or 128 */
  int32_t causal;  /* 0 or 1 */
  int32_t group;   /* queries per position (>= 1); causal problems need n == group * T */
  float scale;     /* score scale, normally 1 / sqrt(d) */
  am_dtype dtype;  /* dtype of Q, K, V and C_k */
} am_problem;

/* How am_compact_head sets beta: NNLS on the mass equations (blog §Choosing beta, the
 * Attention Matching fit), or uniform redistribution of the missing mass (same section,
 * the fast variant; see am_beta_redistribute). */
typedef enum { AM_BETA_NNLS = 0, AM_BETA_REDISTRIBUTE = 1 } am_beta_mode;

/* How am_compact_head sets C_v: ridge least squares on the output equations (blog
 * §Choosing C_v), or the selected keys' own values C_v = V[idx] ("direct", same section). */
typedef enum { AM_VALUES_FIT = 0, AM_VALUES_DIRECT = 1 } am_value_mode;

typedef struct {
  am_score_mode score;   /* key selection statistic (default RMS) */
  am_mass_mode mass;     /* mass-equation weighting (default RELATIVE) */
  float w_lo, w_hi;      /* box for w = exp(beta); defaults 0 and +inf */
  int32_t nnls_max_iter; /* projected-gradient iterations cap (default 500) */
  float nnls_tol;        /* relative KKT tolerance (default 1e-6) */
  float ridge_lambda;    /* absolute ridge on A^T A (default 1e-3) */
  am_beta_mode beta;     /* default AM_BETA_NNLS */
  am_value_mode values;  /* default AM_VALUES_FIT */
} am_options;

/* Fills *opt with the defaults listed above. */
void am_default_options(am_options* opt);

/*
 * am_targets - full-cache statistics (Latent Compaction §3 Preliminaries, Eq. 1; the
 * first step of the blog's §Fast KV Compaction, "keys with the highest attention").
 *   lse[h, n]       = log sum_{j visible} exp(scale * q_i . k_j)      (natural log)
 *   O[h, n, d]      = sum_j exp(scale * q_i . k_j - lse_i) v_j        (optional, NULL skips)
 *   key_score[h, T] = per-key statistic of the mode above over all n queries
 *                     (optional, NULL skips the second pass)
 * A fused flash pass produces lse and O; a second pass recomputes the scores with lse
 * known and reduces them per key.
 */
am_status am_targets(const am_problem* p, const void* Q, const void* K, const void* V,
                     float* lse, float* O, float* key_score, am_score_mode mode,
                     void* ws, size_t ws_bytes, am_stream_t stream);

/*
 * am_select_keys - the t keys of largest key_score per head (blog §Fast KV Compaction,
 * step 1; C_k is a subset of K). Ties go to the lower key index; idx[h, t] is returned in
 * ascending order. C_k[h, t, d] = K[idx] and, if V_sel is not NULL, V_sel = V[idx]
 * (bit-exact copies in the problem dtype). Requires 1 <= t <= T.
 */
am_status am_select_keys(const am_problem* p, const float* key_score, int64_t t,
                         const void* K, const void* V, int32_t* idx, void* Ck, void* V_sel,
                         void* ws, size_t ws_bytes, am_stream_t stream);

/*
 * am_fit_beta_nnls - beta from the mass equations by non-negative least squares on
 * w = exp(beta) (blog, §Choosing beta). With M the mass design of the selected keys
 * (see am_mass_mode), w = argmin_{w_lo <= w <= w_hi} ||M w - b||^2, solved on the device
 * from the Gram form G = M^T M, h = M^T b by accelerated projected gradient. beta = log w
 * (w = 0 gives -inf). lse[h, n] is the natural-log normalizer from am_targets. idx must
 * be ascending (as am_select_keys returns it); it gives the compacted keys' positions.
 * Optional outputs (NULL skips each):
 *   w[h, t];
 *   mass_resid[h] = ||M w - b||^2 / n;
 *   kkt_resid[h]  = max_j viol_j / max_j |h_j|, the optimality-condition residual of the
 *                   returned w on the Gram system the library formed (fp32): with
 *                   g = G w - h, viol_j = |g_j| where w_lo < w_j < w_hi, max(-g_j, 0) where
 *                   w_j = w_lo and max(g_j, 0) where w_j = w_hi;
 *   iters[h]      = projected-gradient steps taken (the solve stops when its scaled
 *                   gradient-mapping norm is below nnls_tol, or after nnls_max_iter steps);
 *   head_status[h].
 * For t > 256 the solve runs on several workgroups per head that wait on each other; it
 * needs them all resident at once and returns AM_ERR_DEVICE if the device cannot hold them
 * (am_fit_beta_plan reports the schedule). A head whose workgroups still fail to meet
 * within about a second gets AM_HEAD_TIMEOUT.
 */
am_status am_fit_beta_nnls(const am_problem* p, const void* Q, const void* Ck,
                           const int32_t* idx, const float* lse, int64_t t,
                           const am_options* opt, float* beta, float* w, float* mass_resid,
                           float* kkt_resid, int32_t* iters, int32_t* head_status, void* ws,
                           size_t ws_bytes, am_stream_t stream);

/* How am_fit_beta_nnls (and am_compact_head) schedule the NNLS of a problem on the current
 * device. */
typedef struct {
  int32_t workgroups_per_head;    /* 1: one workgroup holds a head's whole system (t <= 256) */
  int32_t launches;               /* heads are solved in this many batches */
  int32_t heads_per_launch;       /* heads in each batch but possibly the last */
  int32_t rows_per_workgroup;     /* rows of G each workgroup of a full batch owns */
  int32_t lds_rows_per_workgroup; /* of those, the rows held in LDS for the whole solve; the
                                     others are read from memory at every step */
} am_nnls_plan;

/* Fills *out for problem p and budget t (host only; AM_ERR_DEVICE if the device cannot be
 * queried). */
am_status am_fit_beta_plan(const am_problem* p, int64_t t, am_nnls_plan* out);

/*
 * am_fit_values_ols - C_v from the output equations (blog, §Choosing C_v) by ridge least
 * squares: A_i = softmax over the visible selected keys of (scale * q_i . C_k + beta)
 * (Latent Compaction Eq. 2-3), Y = O (targets from am_targets), and
 * C_v = (A^T A + lambda I)^{-1} A^T Y by Cholesky and two triangular solves.
 * lambda = 0 is ordinary least squares and needs A of rank t.
 * Optional outputs: out_resid[h] = ||A C_v - Y||_F^2 / ||Y||_F^2; head_status[h] (OR-ed).
 */
am_status am_fit_values_ols(const am_problem* p, const void* Q, const void* Ck,
                            const int32_t* idx, const float* beta, const float* O, int64_t t,
                            float ridge_lambda, float* Cv, float* out_resid,
                            int32_t* head_status, void* ws, size_t ws_bytes,
                            am_stream_t stream);

/*
 * am_beta_redistribute - beta without a fit: uniform redistribution of the missing mass
 * ("Compaction" blog, §Choosing beta). With m_j = (1/n) sum_i exp(s_i,c_j) over the
 * queries that see compacted key j and Delta = (1/n) sum_i Z_i - sum_j m_j, where
 * Z_i = exp(lse_i) is query i's mass over the reference key set (lse from am_targets, or
 * over a shortlist), beta_j = log((m_j + Delta / t) / m_j): every selected key receives the
 * same share of the mass the compacted keys miss. A key with m_j = 0 in fp32 on the common
 * scale exp(s - max_i lse_i) gets +inf (0 when Delta <= 0). Optional outputs: w = exp(beta),
 * mass_resid[h] as for am_fit_beta_nnls. idx ascending as am_select_keys returns it.
 */
am_status am_beta_redistribute(const am_problem* p, const void* Q, const void* Ck,
                               const int32_t* idx, const float* lse, int64_t t, float* beta,
                               float* w, float* mass_resid, void* ws, size_t ws_bytes,
                               am_stream_t stream);

/*
 * am_select_two_pass - key selection without the full n x T score pass ("Compaction"
 * blog, §Choosing C_k, Attempt #3 "Two-Pass"). Pass 1 scores all T keys against the query
 * subset sub[h, s] (ascending query indices in [0, n), e.g. a seeded random sample; the
 * statistic's divisor is s) and keeps the kt = min(k_mult * t, T) best keys as a
 * shortlist. Pass 2 scores the shortlist against all n queries, each query's softmax
 * normalized over the shortlist keys it sees, and keeps the t best (ties to the lower
 * index at both stages). Outputs idx[h, t] (ascending original key indices), Ck[h, t, d],
 * V_sel (optional) and lse_short[h, n] = log sum over the visible shortlist keys (-inf for
 * a query that sees none), the Z_i that am_beta_redistribute takes for this method.
 * Workspace: am_two_pass_workspace_bytes.
 */
am_status am_select_two_pass(const am_problem* p, const void* Q, const void* K, const void* V,
                             const int32_t* sub, int64_t s, int64_t t, int32_t k_mult,
                             am_score_mode mode, int32_t* idx, void* Ck, void* V_sel,
                             float* lse_short, void* ws, size_t ws_bytes, am_stream_t stream);

/*
 * am_compact_two_pass - the blog's fast method end to end ("Compaction", §Results,
 * "two_pass"): am_select_two_pass, beta by uniform redistribution over the shortlist's
 * mass (am_beta_redistribute with lse_short), and direct values C_v = V[idx] (f32).
 * Outputs idx, Ck, beta, Cv; optional resid_out[2, h]: the mass residual against the
 * shortlist's mass and the output residual is not computed (row 1 is set to -1).
 */
am_status am_compact_two_pass(const am_problem* p, const void* Q, const void* K, const void* V,
                              const int32_t* sub, int64_t s, int64_t t, int32_t k_mult,
                              am_score_mode mode, int32_t* idx, void* Ck, float* beta, float* Cv,
                              float* resid_out, void* ws, size_t ws_bytes, am_stream_t stream);

/* Workspace bytes of am_select_two_pass (compact = 0) or am_compact_two_pass (compact = 1). */
size_t am_two_pass_workspace_bytes(const am_problem* p, int64_t t, int64_t s, int32_t k_mult,
                                   int32_t compact);

/*
 * am_init_anchor_diverse - anchor + diversifier initialization of an M-slot budget
 * (Latent Compaction §3.2, "Budget Allocation"): n_anchor anchors are the first entry and
 * the n_anchor - 1 other entries of highest maximum attention a_i = max_q softmax(s K q)_i
 * over the n reference queries (Eq. 6, causal masks as for am_targets); the other
 * M - n_anchor entries are added by farthest-first traversal (Eq. 7): each step adds the
 * key, not yet chosen, whose smallest squared Euclidean distance to the chosen keys is
 * largest (ties to the lower index; distances in fp32 from the input dtype).
 * idx[h, M] receives the chosen entries in ascending order; order[h, M] (optional) the
 * selection order (anchors ascending, then the traversal). Requires 1 <= n_anchor <= M
 * <= min(T, 8192) and at most 16384 keys per workgroup of the traversal
 * (AM_ERR_UNSUPPORTED otherwise). head_status (optional) gets AM_HEAD_TIMEOUT if the
 * traversal's workgroups could not meet. Workspace: am_workspace_bytes(p, M,
 * AM_CALL_INIT) (sized for n_anchor = M).
 */
am_status am_init_anchor_diverse(const am_problem* p, const void* Q, const void* K, int64_t M,
                                 int64_t n_anchor, int32_t* idx, int32_t* order,
                                 int32_t* head_status, void* ws, size_t ws_bytes,
                                 am_stream_t stream);

/*
 * am_eval_residuals - quality of a compacted cache on a set of queries (for instance a
 * held-out set; "Compaction" blog, §Choosing beta and §Choosing C_v report errors on
 * held-out queries): the full-cache targets of Q against K, V, then
 *   resid_out[0, h] = mean_i (Z_cmp,i / Z_i - 1)^2                 (mass)
 *   resid_out[1, h] = sum_i ||A_cmp(q_i) - O_i||^2 / sum_i ||O_i||^2 (output)
 * with Z_cmp and A_cmp the biased compacted attention (Latent Compaction Eq. 2-4) of
 * (idx, Ck, beta, Cv). p describes the queries and the full cache (p->n queries, p->T
 * keys; causal problems need n == group * T).
 */
am_status am_eval_residuals(const am_problem* p, const void* Q, const void* K, const void* V,
                            const int32_t* idx, const void* Ck, const float* beta,
                            const float* Cv, int64_t t, float* resid_out, void* ws,
                            size_t ws_bytes, am_stream_t stream);

/*
 * am_compact_head - the whole path per head (the per-layer map over H heads of "The
 * Optimization Landscape of Learning Compacted Context Models", §2 Eq. 1): targets ->
 * selection -> beta -> C_v. Outputs idx, C_k, beta, C_v; optional lse_out, O_out,
 * score_out (full-cache statistics), resid_out[2, h] (row 0: mass residuals, row 1: output
 * residuals, as defined for the two fit calls) and head_status[h]. opt->beta and
 * opt->values choose the fits or the blog's fast variants (redistributed beta, direct
 * values); the fast variants skip the Gram builds and solves they replace.
 */
am_status am_compact_head(const am_problem* p, const void* Q, const void* K, const void* V,
                          int64_t t, const am_options* opt, int32_t* idx, void* Ck,
                          float* beta, float* Cv, float* lse_out, float* O_out,
                          float* score_out, float* resid_out, int32_t* head_status,
                          void* ws, size_t ws_bytes, am_stream_t stream);

/*
 * am_compact_head_noalloc - am_compact_head for callers that cannot allocate device memory
 * (work captured into graphs, tight serving loops, harnesses that forbid allocation): the
 * same computation and outputs, with the scratch taken from a fixed array of
 * AM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on (from the first
 * call on that GPU until the process ends) instead of a workspace argument. Problems whose
 * am_workspace_bytes(p, t, AM_CALL_COMPACT) exceeds that size return AM_ERR_WORKSPACE and
 * launch nothing; invalid arguments return what am_compact_head returns. Every call on one
 * GPU uses the same array: calls that overlap on one GPU (other streams or host threads)
 * race and must be serialized by the caller. No allocation is made by the call.
 */
#define AM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
am_status am_compact_head_noalloc(const am_problem* p, const void* Q, const void* K,
                                  const void* V, int64_t t, const am_options* opt, int32_t* idx,
                                  void* Ck, float* beta, float* Cv, float* lse_out, float* O_out,
                                  float* score_out, float* resid_out, int32_t* head_status,
                                  am_stream_t stream);

/*
 * am_cache_attention - attention of queries through a compacted cache whose slots carry
 * learned biases, optionally followed by ordinary entries appended after it (Latent
 * Compaction §3.1 Eq. 2-5; App. A.2, normalizer-aware cache attention: a biased,
 * slot-masked document branch and an unbiased causal branch, combined through their
 * log-normalizers). Here p->T is the number of cache slots t, p->n the queries per head,
 * p->dtype the dtype of Q, Ck, Kn and Vn; p->causal masks the document branch by original
 * position (no n == group * T requirement for this call).
 *   document branch: l_ij = scale * q_i . Ck_j + bias_j over slots j < nvalid[h] (every
 *     slot when nvalid is NULL; values are clamped to [0, t]); with p->causal, slot j is
 *     also hidden from query i unless keypos[h, j] <= i / group (keypos required then,
 *     ascending per head as am_select_keys returns it).
 *     A_cmp = softmax(l) Cv and log Z_cmp = logsumexp(l).
 *   new branch (m > 0): s_ij = scale * q_i . Kn_j, no bias; entry j is visible to query i
 *     when j <= i / group (new_causal = 1) or always (new_causal = 0).
 *   out[h, n, d] = (Z_cmp A_cmp + Z_new A_new) / (Z_cmp + Z_new), weights in log space;
 *   lse[h, n] = log(Z_cmp + Z_new); lse_cmp[h, n] = log Z_cmp (optional, NULL skips).
 *   A query with no visible entry in either branch gets lse = -inf and a zero row.
 * Shapes: Ck [h, t, d] problem dtype; Cv [h, t, d] f32 (rounded to the problem dtype for
 * the products); bias [h, t] f32; keypos [h, t] int32; nvalid [h] int32; Kn, Vn [h, m, d].
 * Workspace: am_workspace_bytes(p, m, AM_CALL_CACHE_ATTENTION) (the budget argument is m).
 */
am_status am_cache_attention(const am_problem* p, const void* Q, const void* Ck, const float* Cv,
                             const float* bias, const int32_t* keypos, const int32_t* nvalid,
                             int64_t m, const void* Kn, const void* Vn, int32_t new_causal,
                             float* out, float* lse, float* lse_cmp, void* ws, size_t ws_bytes,
                             am_stream_t stream);

/*
 * am_attention_merge - combine two attention results over disjoint entry sets (Latent
 * Compaction Eq. 5, in log space): for each of `rows` rows of d floats,
 *   lse_out = logaddexp(lse1, lse2),
 *   out = exp(lse1 - lse_out) O1 + exp(lse2 - lse_out) O2;
 * rows where both normalizers are -inf get -inf and zeros. d must be a positive multiple
 * of 4. out may be O1 or O2 and lse_out may be lse1 or lse2 (in-place merge); no
 * workspace.
 */
am_status am_attention_merge(int64_t rows, int64_t d, const float* O1, const float* lse1,
                             const float* O2, const float* lse2, float* out, float* lse_out,
                             am_stream_t stream);

/*
 * Stage-1 attention fitting (Latent Compaction §3.3, Eq. 8; App. A.2): the compacted keys,
 * values and biases of a cache become trainable f32 parameters, fitted so that the
 * compacted attention (Eq. 2-4) reproduces the full cache's outputs and log-normalizers on
 * sampled query positions. Here p->T is the slot count t, p->n the reference queries per
 * head (a multiple of group; row i sits at position i / group), p->dtype the dtype of Q;
 * p->causal masks slot j from row i unless keypos[h, j] <= i / group.
 * Inputs: Q [h, n, d]; O_full [h, n, d] f32 and lse_full [h, n] f32, the full cache's
 * attention output and log-normalizer of every row (am_targets computes both);
 * samples [S] (one evaluation) or [steps, S] (fit) int32 positions in [0, n / group)
 * (values outside are clamped); each update uses every query head of its S positions
 * (N = S * group rows).
 * The loss of one update, per head: with g the row's query head and sa_g, sz_g the
 * population standard deviations of O_full over that query head's rows and channels and of
 * lse_full over its rows (both floored at 1e-4, computed once per call),
 *   L = mean over rows and channels of ((A - O_full) / sa_g)^2
 *     + mean over rows of ((log Z - lse_full) / sz_g)^2,
 * where A = softmax(l) Cv, log Z = logsumexp(l), l = scale Ck q + bias over visible slots.
 * Rows that see no slot are left out of both means (L = 0 if none is left).
 * Parameters: Ck, Cv [h, t, d] f32 and bias [h, t] f32.
 */

/* One evaluation at samples [S]: loss_out [h] (optional) and the gradients
 * gCk, gCv [h, t, d] and gbias [h, t] of L with respect to Ck, Cv and bias. */
am_status am_stage1_loss_grad(const am_problem* p, const void* Q, const float* O_full,
                              const float* lse_full, const int32_t* keypos,
                              const int32_t* samples, int64_t S, const float* Ck,
                              const float* Cv, const float* bias, float* loss_out, float* gCk,
                              float* gCv, float* gbias, void* ws, size_t ws_bytes,
                              am_stream_t stream);

/* `steps` AdamW updates (beta1 0.9, beta2 0.999, eps 1e-8, bias-corrected moments, decoupled
 * weight decay theta <- theta (1 - lr wd) before the Adam step, constant lr; moments start
 * at zero) of Ck, Cv and bias IN PLACE, update k on the positions samples[k, :].
 * trainable [h, t] uint8 (optional, NULL trains every slot): slots with 0 keep their key,
 * value and bias. loss_out [steps, h] (optional) receives each update's loss, evaluated
 * before that update. */
am_status am_fit_stage1(const am_problem* p, const void* Q, const float* O_full,
                        const float* lse_full, const int32_t* keypos, const int32_t* samples,
                        int64_t S, int64_t steps, const uint8_t* trainable, float lr, float wd,
                        float* Ck, float* Cv, float* bias, float* loss_out, void* ws,
                        size_t ws_bytes, am_stream_t stream);

/* Workspace bytes of am_stage1_loss_grad and am_fit_stage1 for S positions per update. */
size_t am_stage1_workspace_bytes(const am_problem* p, int64_t S);

/* Which call a workspace size is for. */
typedef enum {
  AM_CALL_TARGETS = 0,
  AM_CALL_SELECT = 1,
  AM_CALL_FIT_BETA = 2,
  AM_CALL_FIT_VALUES = 3,
  AM_CALL_COMPACT = 4,
  AM_CALL_CACHE_ATTENTION = 5, /* the budget argument of am_workspace_bytes is m */
  AM_CALL_BETA_REDIST = 6,
  AM_CALL_EVAL = 7,
  AM_CALL_INIT = 8             /* the budget argument is M */
} am_call;

/* Workspace bytes a call needs for problem p and budget t (0 if the problem is invalid). */
size_t am_workspace_bytes(const am_problem* p, int64_t t, am_call which);

/* Static string for a status code. */
const char* am_status_str(am_status s);

/* ABI version (incremented on any incompatible change). */
int am_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AM_H */
