// Host-side interface between the C ABI and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace amc {

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// per-head device status bits (same values as the AM_HEAD_* constants of am.h)
constexpr int AM_HEAD_NNLS_BIT = 1;
constexpr int AM_HEAD_CHOL_BIT = 2;
constexpr int AM_HEAD_NONFINITE_BIT = 4;
constexpr int AM_HEAD_TIMEOUT_BIT = 8;
// largest compacted size the fits support (the NNLS keeps a t-vector in LDS)
constexpr int kMaxFitT = 8192;
inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct TargetsArgs {
  const void* Q; const void* K; const void* V;
  void* Vt;          // workspace: transposed values [h, d, Tpad]
  void* rowstat;     // workspace: per-query (max, log2 sum) [h, n] float2
  float* lse; float* O; float* score;
  int mode;
  int heads, n, T, d, group;
  bool causal, bf16;
  float scale;
  hipStream_t stream;
  const int32_t* qpos = nullptr;   // query subset: positions [h, n], ascending per head
  float* colpart = nullptr;        // workspace for the causal column pass's query-chunk
                                   // partials [kColSplit, h, T] (null: one chunk)
};
hipError_t launch_targets(const TargetsArgs& a);
constexpr int kColSplit = 8;       // query chunks of the causal column-score pass
size_t targets_colpart_bytes(int64_t heads, int64_t T);
size_t targets_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize);
size_t targets_vt_bytes(int64_t heads, int64_t T, int64_t d, int esize);

// Biased compacted attention (the flash pass over C_k with per-key bias and original
// positions). Cv null: statistics only. Y set: per-query residuals instead of O.
struct CmpAttnArgs {
  const void* Q; const void* Ck; const float* Cv; const float* bias; const int32_t* keypos;
  const float* Y;
  void* Vt;             // workspace [h, d, round_up(t, 64)] when Cv is set
  int2* tstat;          // causal: workspace [h, ceil(t / 32)] for per-tile (min, max)
                        // positions, or null (every tile then takes the masked path)
  float* lse; float2* rowstat; float* O; float2* rowres;
  int heads, n, t, d, group;
  bool causal, bf16;
  float scale;
  hipStream_t stream;
};
hipError_t launch_cmp_attention(const CmpAttnArgs& a);
size_t cmp_vt_bytes(int64_t heads, int64_t t, int64_t d, int esize);
size_t cmp_tstat_bytes(int64_t heads, int64_t t);

// Per-key masses m_j = (1/n) sum over queries i that see key j of exp(scale q_i . Ck_j -
// shift_h), shift2[h] = shift_h log2(e), in log form: log2 m_j = kmax_j + log2 kmean_j
// (keys carry original positions keypos[h, t])
constexpr int kKeyMassMaxSplit = 64;   // query chunks per key block (partials [split, h, t])
struct KeyMassArgs {
  const void* Q; const void* Ck; const int32_t* keypos; const float* shift2;
  float* kmax; float* kmean;
  float* part;   // workspace of key_mass_part_bytes
  int heads, n, t, d, group;
  bool causal, bf16;
  float scale;
  hipStream_t stream;
};
hipError_t launch_key_mass(const KeyMassArgs& a);
size_t key_mass_part_bytes(int64_t heads, int64_t n, int64_t t);

// score[h, j] = selection statistic (mode as am_score_mode) over all n queries of the keys
// Ck [h, t] at original positions keypos, with p = 2^(scale q.k log2 e - (m + log2 l)) from
// the row statistics (m, log2 l) [h, n] over the same keys
struct KeyScoreArgs {
  const void* Q; const void* Ck; const int32_t* keypos; const float2* rowstat;
  float* score;
  float* part;   // workspace of key_mass_part_bytes
  int mode;
  int heads, n, t, d, group;
  bool causal, bf16;
  float scale;
  hipStream_t stream;
};
hipError_t launch_key_score(const KeyScoreArgs& a);

// Two-pass key selection (query subset against all keys, then all queries against a
// shortlist of k * t keys); workspace two_pass_ws_bytes
struct TwoPassArgs {
  const void* Q; const void* K; const void* V; const int32_t* sub;
  int32_t* idx; void* Ck; void* Vsel; float* lse_short;
  int heads, n, T, d, group, s, t, kt, mode;
  bool causal, bf16;
  float scale;
  void* ws;
  hipStream_t stream;
};
hipError_t launch_two_pass(const TwoPassArgs& a);
hipError_t launch_fill_f32(float* p, long long count, float v, hipStream_t st);

// Anchor + diversifier initialization of an M-slot budget (na anchors, the first entry
// among them); idx [h, M] ascending, order [h, M] the selection order (may be null);
// workspace init_ws_bytes
struct InitArgs {
  const void* Q; const void* K;
  int32_t* idx; int32_t* order; int32_t* head_status;
  int heads, n, T, d, group, M, na;
  bool causal, bf16;
  float scale;
  void* ws;
  hipStream_t stream;
};
hipError_t launch_init_anchor_diverse(const InitArgs& a);
size_t init_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize, int64_t M,
                     int64_t na);
int init_max_chunk(int heads, int T);   // keys per workgroup of the traversal (LDS floats)

// Stage-1 attention fitting: steps AdamW updates of Ck, Cv, b (f32, updated in place) on
// the sampled positions samples [steps, S]; with steps == 0 one evaluation of the loss and
// its gradients (gCk, gCv, gb) at samples [S]
struct Stage1Args {
  const void* Q; const float* O_full; const float* lse_full; const int32_t* keypos;
  const uint8_t* trainable; const int32_t* samples;
  float* Ck; float* Cv; float* b; float* loss;
  float* gCk; float* gCv; float* gb;
  int heads, n, d, group, t, S, steps;
  bool causal, bf16;
  float scale, lr, wd;
  void* ws;
  hipStream_t stream;
};
hipError_t launch_stage1(const Stage1Args& a);
size_t stage1_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d, int64_t S,
                       int64_t group);
constexpr int kInitMaxChunk = 16384;
constexpr int kInitMaxM = 8192;
size_t two_pass_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize, int64_t s,
                         int64_t kt);

// Log-space merge of two attention results (rows of d floats, d % 4 == 0); O2 may be null.
struct MergeArgs {
  const float* O1; const float* lse1; const float* O2; const float* lse2;
  float* out; float* lse;
  long long rows; int d;
  hipStream_t stream;
};
hipError_t launch_attention_merge(const MergeArgs& a);
// bias with the slots j >= nvalid[h] set to -inf
hipError_t launch_mask_bias(const float* bias, const int32_t* nvalid, float* out, int heads,
                            int t, hipStream_t st);

struct SelectArgs {
  const float* score; const void* K; const void* V;
  int32_t* idx; void* Ck; void* Vsel;
  int heads, T, t, d;
  bool bf16;
  hipStream_t stream;
};
hipError_t launch_select(const SelectArgs& a);

struct FitArgs {
  const void* Q; const void* Ck; const int32_t* idx; const float* lse;
  const float* beta_in;  // value fit: beta of the selected keys
  const float* O;        // value fit: targets Y [h, n, d]
  float* beta; float* w; float* mass_resid; float* Cv; float* out_resid;
  float* kkt;            // beta fit: relative KKT residual per head (optional)
  int32_t* iters;        // beta fit: projected-gradient steps per head (optional)
  int32_t* head_status;
  int heads, n, t, d, group;
  bool causal, bf16, absolute;
  float scale, w_lo, w_hi, tol, lambda;
  int max_iter;
  bool keep_status;     // value fit after the beta fit: OR into head_status instead of clearing
  bool keep_cmp_stats;  // beta fit: leave the compacted row statistics at the workspace start
  bool have_cmp_stats;  // value fit: those statistics (same beta) are already there
  void* ws; size_t ws_bytes;
  hipStream_t stream;
};
// Gram builds for t > kSyrkMinT: the bf16 design X (key rows, then Y^T rows for the value
// fit) is stored once and its Gram formed by a tiled MFMA product with split-K partials.
constexpr int kSyrkMinT = 256;
struct SyrkBuffers {
  void* X;        // [h, xrows, npad] bf16
  float* part;    // [h, chunks, tiles, 256, 256] Gram partials
  float* hpart;   // mass: [h, tpad, npad / 128] partials of M^T b
};
bool syrk_path(int t);
// value fit: number of per-head partials of ||Y||^2 the Y^T rows kernel writes
int syrk_yy_blocks(int64_t heads, int64_t n, int64_t t, int64_t d);
// carve the buffers at base + off (base null: sizing only); off advances past them
SyrkBuffers syrk_carve(char* base, size_t& off, int64_t heads, int64_t n, int64_t t, int64_t d,
                       bool value);
struct SyrkGramArgs {
  const void* Q; const void* Ck; const int32_t* keypos;
  const float* bias;     // value: beta of the selected keys
  const float* shift2;   // per query, log2 domain
  const float* target;   // mass: right-hand side (null = 1)
  const float* Y;        // value: targets [h, n, d]
  SyrkBuffers buf;
  double* yyp = nullptr;  // value: partials of ||Y||^2 [h, syrk_yy_blocks] (null: not formed)
  float* Gf; float* hv;   // mass outputs: G [h, t, t], M^T b [h, t]
  double* Gd; double* R;  // value outputs: A^T A + lambda I [h, ld, ld], A^T Y [h, ld, d]
  int heads, n, t, d, group, ld;
  bool causal, bf16, value;
  float c2, lambda;
  hipStream_t stream;
};
hipError_t launch_syrk_gram(const SyrkGramArgs& a);

// Fast variants and evaluation (workspace: fast_ws_bytes; T_eval = keys of the full cache
// for the evaluation, else 0).
// beta by uniform redistribution from a.lse (writes a.beta, a.w, a.mass_resid if set)
hipError_t launch_beta_redistribute(const FitArgs& a);
// C_v = V[idx] in f32 (a.Cv); a.out_resid against a.O with a.beta_in if set
hipError_t launch_values_direct(const FitArgs& a, const void* V, int T);
// resid[0, h]: mass residual, resid[1, h]: output residual of (a.idx, a.Ck, a.beta_in, a.Cv)
// on the queries a.Q against the full cache K, V (T keys)
hipError_t launch_eval_residuals(const FitArgs& a, const void* K, const void* V, int T,
                                 float* resid);
size_t fast_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d, int esize, int64_t T_eval);

hipError_t launch_zero_status(int32_t* status, int heads, hipStream_t st);

hipError_t launch_fit_beta(const FitArgs& a);
// How the NNLS of a beta fit is scheduled: one workgroup per head (t <= 256; P = 1), or P
// workgroups per head that meet at per-head barriers, heads_per_launch heads per launch.
struct NnlsParts { int P, rb, nlds; size_t shmem; };   // rb rows per workgroup, nlds in LDS
struct NnlsSchedule { int heads_per_launch, launches; NnlsParts first; };
NnlsParts nnls_parts(int hb, int t, int ncu);
NnlsSchedule nnls_schedule(int heads, int t, int ncu);
int device_cu_count();   // of the current device (0 if the query fails)
// An ordinary launch of a kernel whose workgroups wait on each other: refused with
// hipErrorCooperativeLaunchTooLarge unless the whole grid can be resident at once.
hipError_t launch_all_resident(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem,
                               hipStream_t st);
hipError_t launch_fit_values(const FitArgs& a);
size_t fit_beta_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d);
size_t fit_values_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d);

}  // namespace amc
