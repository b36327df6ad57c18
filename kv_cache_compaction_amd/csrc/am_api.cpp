// C ABI of the compaction library: argument validation, workspace carving and launch
// sequencing on the caller's stream. Every check runs on the host before any launch; no
// call synchronizes, allocates device memory or keeps a pointer after it returns.
#include <math.h>
#include <string.h>

#include "../../include/am.h"
#include "am_internal.hpp"

using namespace amc;

namespace {

constexpr int kAbiVersion = 4;

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// An enum argument or field as the int the caller passed, read through its bytes: in C++ a
// load of an enum-typed value outside the enumeration's range is undefined, and the C
// callers of this ABI may pass any int (validation must reject it, not depend on it).
template <typename E> int ival(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

int esize(const am_problem* p) { return p->dtype == AM_BF16 ? 2 : 4; }

am_status check_problem(const am_problem* p) {
  if (!p) return AM_ERR_INVALID_ARG;
  if (p->heads < 1 || p->n < 1 || p->T < 1 || p->d < 1) return AM_ERR_INVALID_ARG;
  if (p->group < 1 || (p->causal != 0 && p->causal != 1)) return AM_ERR_INVALID_ARG;
  if (ival(p->dtype) != AM_F32 && ival(p->dtype) != AM_BF16) return AM_ERR_INVALID_ARG;
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return AM_ERR_INVALID_ARG;
  if (p->causal && p->n != (int64_t)p->group * p->T) return AM_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return AM_ERR_UNSUPPORTED;
  // row indices are 32-bit inside the kernels; heads index a grid dimension of <= 65535
  if (p->n > (int64_t)1 << 30 || p->T > (int64_t)1 << 30 || p->heads > 65535)
    return AM_ERR_UNSUPPORTED;
  if ((p->heads * p->n) > ((int64_t)1 << 40) || (p->heads * p->T) > ((int64_t)1 << 40))
    return AM_ERR_UNSUPPORTED;
  return AM_OK;
}

am_status check_t(const am_problem* p, int64_t t) {
  if (t < 1 || t > p->T) return AM_ERR_INVALID_ARG;
  return AM_OK;
}

am_status check_fit_t(int64_t t) { return t > kMaxFitT ? AM_ERR_UNSUPPORTED : AM_OK; }

am_status check_opts(const am_options* o) {
  if (!o) return AM_ERR_INVALID_ARG;
  if (ival(o->score) < AM_SCORE_RMS || ival(o->score) > AM_SCORE_MAX) return AM_ERR_INVALID_ARG;
  if (ival(o->mass) != AM_MASS_RELATIVE && ival(o->mass) != AM_MASS_ABSOLUTE) return AM_ERR_INVALID_ARG;
  if (!(o->w_lo >= 0.f) || isnan(o->w_hi) || !(o->w_hi > o->w_lo) || isinf(o->w_lo))
    return AM_ERR_INVALID_ARG;
  if (o->nnls_max_iter < 1 || !(o->nnls_tol >= 0.f) || !(o->ridge_lambda >= 0.f) ||
      !isfinite(o->ridge_lambda))
    return AM_ERR_INVALID_ARG;
  if (ival(o->beta) != AM_BETA_NNLS && ival(o->beta) != AM_BETA_REDISTRIBUTE) return AM_ERR_INVALID_ARG;
  if (ival(o->values) != AM_VALUES_FIT && ival(o->values) != AM_VALUES_DIRECT) return AM_ERR_INVALID_ARG;
  return AM_OK;
}

am_status from_hip(hipError_t e) { return e == hipSuccess ? AM_OK : AM_ERR_DEVICE; }

size_t ws_targets(const am_problem* p) {
  return targets_ws_bytes(p->heads, p->n, p->T, p->d, esize(p));
}
size_t ws_fit_beta(const am_problem* p, int64_t t) {
  return fit_beta_ws_bytes(p->heads, p->n, t, p->d);
}
size_t ws_fit_values(const am_problem* p, int64_t t) {
  return fit_values_ws_bytes(p->heads, p->n, t, p->d);
}
// The cache-attention problem: p->T is the slot count; causal masks by original position.
am_status check_cache_problem(const am_problem* p) {
  if (!p) return AM_ERR_INVALID_ARG;
  if (p->heads < 1 || p->n < 1 || p->T < 1 || p->d < 1) return AM_ERR_INVALID_ARG;
  if (p->group < 1 || (p->causal != 0 && p->causal != 1)) return AM_ERR_INVALID_ARG;
  if (ival(p->dtype) != AM_F32 && ival(p->dtype) != AM_BF16) return AM_ERR_INVALID_ARG;
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return AM_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return AM_ERR_UNSUPPORTED;
  if (p->n > (int64_t)1 << 30 || p->T > (int64_t)1 << 30 || p->heads > 65535)
    return AM_ERR_UNSUPPORTED;
  if ((p->heads * p->n) > ((int64_t)1 << 40) || (p->heads * p->T) > ((int64_t)1 << 40))
    return AM_ERR_UNSUPPORTED;
  return AM_OK;
}

struct CacheWs {
  size_t vt, tstat, bias, lse1, vt_new, o2, lse2, total;
};
CacheWs cache_ws(const am_problem* p, int64_t m) {
  CacheWs w;
  const int es = esize(p);
  w.vt = cmp_vt_bytes(p->heads, p->T, p->d, es);
  w.tstat = p->causal ? cmp_tstat_bytes(p->heads, p->T) : 0;
  w.bias = align_up((size_t)p->heads * p->T * 4);
  w.lse1 = align_up((size_t)p->heads * p->n * 4);
  w.vt_new = m > 0 ? targets_vt_bytes(p->heads, m, p->d, es) : 0;
  w.o2 = m > 0 ? align_up((size_t)p->heads * p->n * p->d * 4) : 0;
  w.lse2 = m > 0 ? align_up((size_t)p->heads * p->n * 4) : 0;
  w.total = w.vt + w.tstat + w.bias + w.lse1 + w.vt_new + w.o2 + w.lse2;
  return w;
}

size_t ws_fast(const am_problem* p, int64_t t, int64_t T_eval) {
  return fast_ws_bytes(p->heads, p->n, t, p->d, esize(p), T_eval);
}
size_t ws_compact(const am_problem* p, int64_t t) {
  // lse, O and score live in the workspace when the caller does not want them
  const size_t own = align_up((size_t)p->heads * p->n * 4) +
                     align_up((size_t)p->heads * p->n * p->d * 4) +
                     align_up((size_t)p->heads * p->T * 4);
  size_t fit = ws_fit_beta(p, t);
  const size_t fv = ws_fit_values(p, t);
  if (fv > fit) fit = fv;
  const size_t ff = ws_fast(p, t, 0);
  if (ff > fit) fit = ff;
  size_t stage = ws_targets(p);
  if (fit > stage) stage = fit;
  return own + stage;
}

TargetsArgs targets_args(const am_problem* p, const void* Q, const void* K, const void* V,
                         float* lse, float* O, float* score, int mode, void* ws,
                         hipStream_t s) {
  TargetsArgs a;
  a.Q = Q; a.K = K; a.V = V;
  a.Vt = ws;
  a.rowstat = (char*)ws + targets_vt_bytes(p->heads, p->T, p->d, esize(p));
  a.colpart = (float*)((char*)a.rowstat + align_up((size_t)p->heads * p->n * 8));
  a.lse = lse; a.O = O; a.score = score; a.mode = mode;
  a.heads = (int)p->heads; a.n = (int)p->n; a.T = (int)p->T; a.d = (int)p->d;
  a.group = p->group; a.causal = p->causal != 0; a.bf16 = p->dtype == AM_BF16;
  a.scale = p->scale; a.stream = s;
  return a;
}

FitArgs fit_args(const am_problem* p, const void* Q, const void* Ck, const int32_t* idx,
                 int64_t t, void* ws, size_t ws_bytes, hipStream_t s) {
  FitArgs a;
  memset(&a, 0, sizeof a);
  a.Q = Q; a.Ck = Ck; a.idx = idx;
  a.heads = (int)p->heads; a.n = (int)p->n; a.t = (int)t; a.d = (int)p->d;
  a.group = p->group; a.causal = p->causal != 0; a.bf16 = p->dtype == AM_BF16;
  a.scale = p->scale; a.ws = ws; a.ws_bytes = ws_bytes; a.stream = s;
  return a;
}

}  // namespace

extern "C" {

int am_abi_version(void) { return kAbiVersion; }

const char* am_status_str(am_status s) {
  switch (ival(s)) {
    case AM_OK: return "ok";
    case AM_ERR_INVALID_ARG: return "invalid argument";
    case AM_ERR_UNSUPPORTED: return "unsupported problem";
    case AM_ERR_WORKSPACE: return "workspace too small";
    case AM_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

void am_default_options(am_options* o) {
  if (!o) return;
  o->score = AM_SCORE_RMS;
  o->mass = AM_MASS_RELATIVE;
  o->w_lo = 0.f;
  o->w_hi = INFINITY;
  o->nnls_max_iter = 500;
  o->nnls_tol = 1e-6f;
  o->ridge_lambda = 1e-3f;
  o->beta = AM_BETA_NNLS;
  o->values = AM_VALUES_FIT;
}

size_t am_workspace_bytes(const am_problem* p, int64_t t, am_call which_arg) {
  const int which = ival(which_arg);
  if (which == AM_CALL_CACHE_ATTENTION) {
    if (check_cache_problem(p) != AM_OK || t < 0 || t > ((int64_t)1 << 30)) return 0;
    return cache_ws(p, t).total;
  }
  if (check_problem(p) != AM_OK) return 0;
  if (which != AM_CALL_TARGETS && check_t(p, t) != AM_OK) return 0;
  switch (which) {
    case AM_CALL_TARGETS: return ws_targets(p);
    case AM_CALL_SELECT: return 0;
    case AM_CALL_FIT_BETA: return t > kMaxFitT ? 0 : ws_fit_beta(p, t);
    case AM_CALL_FIT_VALUES: return t > kMaxFitT ? 0 : ws_fit_values(p, t);
    case AM_CALL_COMPACT: return t > kMaxFitT ? 0 : ws_compact(p, t);
    case AM_CALL_BETA_REDIST: return ws_fast(p, t, 0);
    case AM_CALL_EVAL: return ws_fast(p, t, p->T);
    case AM_CALL_CACHE_ATTENTION: return 0;
    case AM_CALL_INIT:
      return t > kInitMaxM ? 0 : init_ws_bytes(p->heads, p->n, p->T, p->d, esize(p), t, t);
  }
  return 0;
}

am_status am_targets(const am_problem* p, const void* Q, const void* K, const void* V,
                     float* lse, float* O, float* key_score, am_score_mode mode, void* ws,
                     size_t ws_bytes, am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if (!Q || !K || !lse || (O && !V)) return AM_ERR_INVALID_ARG;
  if (ival(mode) < AM_SCORE_RMS || ival(mode) > AM_SCORE_MAX) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || (V && !al16(V)) || !al16(lse) || (O && !al16(O)) ||
      (key_score && !al16(key_score)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_targets(p)) return AM_ERR_WORKSPACE;
  return from_hip(launch_targets(
      targets_args(p, Q, K, V, lse, O, key_score, (int)mode, ws, (hipStream_t)stream)));
}

am_status am_select_keys(const am_problem* p, const float* key_score, int64_t t, const void* K,
                         const void* V, int32_t* idx, void* Ck, void* V_sel, void* ws,
                         size_t ws_bytes, am_stream_t stream) {
  (void)ws; (void)ws_bytes;
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if (!key_score || !K || !idx || !Ck || (V_sel && !V)) return AM_ERR_INVALID_ARG;
  if (!al16(key_score) || !al16(K) || !al16(idx) || !al16(Ck) || (V && !al16(V)) ||
      (V_sel && !al16(V_sel)))
    return AM_ERR_INVALID_ARG;
  SelectArgs a;
  a.score = key_score; a.K = K; a.V = V; a.idx = idx; a.Ck = Ck; a.Vsel = V_sel;
  a.heads = (int)p->heads; a.T = (int)p->T; a.t = (int)t; a.d = (int)p->d;
  a.bf16 = p->dtype == AM_BF16; a.stream = (hipStream_t)stream;
  return from_hip(launch_select(a));
}

am_status am_fit_beta_nnls(const am_problem* p, const void* Q, const void* Ck,
                           const int32_t* idx, const float* lse, int64_t t,
                           const am_options* opt, float* beta, float* w, float* mass_resid,
                           float* kkt_resid, int32_t* iters, int32_t* head_status, void* ws,
                           size_t ws_bytes, am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if ((st = check_opts(opt)) != AM_OK) return st;
  if ((st = check_fit_t(t)) != AM_OK) return st;
  if (!Q || !Ck || !idx || !lse || !beta) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(Ck) || !al16(idx) || !al16(lse) || !al16(beta) || (w && !al16(w)) ||
      (mass_resid && !al16(mass_resid)) || (kkt_resid && !al16(kkt_resid)) ||
      (iters && !al16(iters)) || (head_status && !al16(head_status)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_fit_beta(p, t)) return AM_ERR_WORKSPACE;
  FitArgs a = fit_args(p, Q, Ck, idx, t, ws, ws_bytes, (hipStream_t)stream);
  a.lse = lse; a.beta = beta; a.w = w; a.mass_resid = mass_resid; a.head_status = head_status;
  a.kkt = kkt_resid; a.iters = iters;
  a.absolute = opt->mass == AM_MASS_ABSOLUTE;
  a.w_lo = opt->w_lo; a.w_hi = opt->w_hi; a.tol = opt->nnls_tol; a.max_iter = opt->nnls_max_iter;
  return from_hip(launch_fit_beta(a));
}

am_status am_fit_beta_plan(const am_problem* p, int64_t t, am_nnls_plan* out) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if ((st = check_fit_t(t)) != AM_OK) return st;
  if (!out) return AM_ERR_INVALID_ARG;
  const int ncu = device_cu_count();
  if (ncu < 1) return AM_ERR_DEVICE;
  const NnlsSchedule sc = nnls_schedule((int)p->heads, (int)t, ncu);
  out->workgroups_per_head = sc.first.P;
  out->launches = sc.launches;
  out->heads_per_launch = sc.heads_per_launch;
  out->rows_per_workgroup = sc.first.rb;
  out->lds_rows_per_workgroup = sc.first.nlds;
  return AM_OK;
}

am_status am_fit_values_ols(const am_problem* p, const void* Q, const void* Ck,
                            const int32_t* idx, const float* beta, const float* O, int64_t t,
                            float ridge_lambda, float* Cv, float* out_resid,
                            int32_t* head_status, void* ws, size_t ws_bytes,
                            am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if ((st = check_fit_t(t)) != AM_OK) return st;
  if (!Q || !Ck || !idx || !beta || !O || !Cv) return AM_ERR_INVALID_ARG;
  if (!(ridge_lambda >= 0.f) || !isfinite(ridge_lambda)) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(Ck) || !al16(idx) || !al16(beta) || !al16(O) || !al16(Cv) ||
      (out_resid && !al16(out_resid)) || (head_status && !al16(head_status)) ||
      (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_fit_values(p, t)) return AM_ERR_WORKSPACE;
  FitArgs a = fit_args(p, Q, Ck, idx, t, ws, ws_bytes, (hipStream_t)stream);
  a.beta_in = beta; a.O = O; a.Cv = Cv; a.out_resid = out_resid; a.head_status = head_status;
  a.lambda = ridge_lambda;
  return from_hip(launch_fit_values(a));
}

am_status am_compact_head(const am_problem* p, const void* Q, const void* K, const void* V,
                          int64_t t, const am_options* opt, int32_t* idx, void* Ck,
                          float* beta, float* Cv, float* lse_out, float* O_out,
                          float* score_out, float* resid_out, int32_t* head_status, void* ws,
                          size_t ws_bytes, am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if ((st = check_opts(opt)) != AM_OK) return st;
  if ((st = check_fit_t(t)) != AM_OK) return st;
  if (!Q || !K || !V || !idx || !Ck || !beta || !Cv) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || !al16(V) || !al16(idx) || !al16(Ck) || !al16(beta) ||
      !al16(Cv) || (lse_out && !al16(lse_out)) || (O_out && !al16(O_out)) ||
      (score_out && !al16(score_out)) || (resid_out && !al16(resid_out)) ||
      (head_status && !al16(head_status)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_compact(p, t)) return AM_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* lse = (float*)w;  w += align_up((size_t)p->heads * p->n * 4);
  float* O = (float*)w;    w += align_up((size_t)p->heads * p->n * p->d * 4);
  float* sc = (float*)w;   w += align_up((size_t)p->heads * p->T * 4);
  const size_t stage_bytes = ws_bytes - (size_t)(w - (char*)ws);
  if (lse_out) lse = lse_out;
  if (O_out) O = O_out;
  if (score_out) sc = score_out;
  hipError_t e = launch_targets(targets_args(p, Q, K, V, lse, O, sc, (int)opt->score, w, s));
  if (e != hipSuccess) return AM_ERR_DEVICE;
  SelectArgs sa;
  sa.score = sc; sa.K = K; sa.V = V; sa.idx = idx; sa.Ck = Ck; sa.Vsel = nullptr;
  sa.heads = (int)p->heads; sa.T = (int)p->T; sa.t = (int)t; sa.d = (int)p->d;
  sa.bf16 = p->dtype == AM_BF16; sa.stream = s;
  if ((e = launch_select(sa)) != hipSuccess) return AM_ERR_DEVICE;
  FitArgs fa = fit_args(p, Q, Ck, idx, t, w, stage_bytes, s);
  fa.lse = lse; fa.beta = beta; fa.w = nullptr; fa.head_status = head_status;
  fa.mass_resid = resid_out ? resid_out : nullptr;
  fa.absolute = opt->mass == AM_MASS_ABSOLUTE;
  fa.w_lo = opt->w_lo; fa.w_hi = opt->w_hi; fa.tol = opt->nnls_tol;
  fa.max_iter = opt->nnls_max_iter;
  fa.lambda = opt->ridge_lambda;
  const bool redist = opt->beta == AM_BETA_REDISTRIBUTE;
  if (redist) {
    if (head_status && (e = launch_zero_status(head_status, (int)p->heads, s)) != hipSuccess)
      return AM_ERR_DEVICE;
    if ((e = launch_beta_redistribute(fa)) != hipSuccess) return AM_ERR_DEVICE;
  } else {
    fa.keep_cmp_stats = true;
    if ((e = launch_fit_beta(fa)) != hipSuccess) return AM_ERR_DEVICE;
  }
  fa.keep_cmp_stats = false;
  fa.have_cmp_stats = !redist;   // the NNLS path left the compacted row statistics
  fa.beta_in = beta; fa.O = O; fa.Cv = Cv;
  fa.mass_resid = nullptr;
  fa.keep_status = true;
  fa.out_resid = resid_out ? resid_out + p->heads : nullptr;
  if (opt->values == AM_VALUES_DIRECT)
    e = launch_values_direct(fa, V, (int)p->T);
  else
    e = launch_fit_values(fa);
  return e == hipSuccess ? AM_OK : AM_ERR_DEVICE;
}

am_status am_beta_redistribute(const am_problem* p, const void* Q, const void* Ck,
                               const int32_t* idx, const float* lse, int64_t t, float* beta,
                               float* w, float* mass_resid, void* ws, size_t ws_bytes,
                               am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if (!Q || !Ck || !idx || !lse || !beta) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(Ck) || !al16(idx) || !al16(lse) || !al16(beta) || (w && !al16(w)) ||
      (mass_resid && !al16(mass_resid)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_fast(p, t, 0)) return AM_ERR_WORKSPACE;
  FitArgs a = fit_args(p, Q, Ck, idx, t, ws, ws_bytes, (hipStream_t)stream);
  a.lse = lse; a.beta = beta; a.w = w; a.mass_resid = mass_resid;
  return from_hip(launch_beta_redistribute(a));
}

namespace {
am_status check_two_pass(const am_problem* p, int64_t s, int64_t t, int32_t k_mult) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if (s < 1 || s > p->n || k_mult < 1) return AM_ERR_INVALID_ARG;
  return AM_OK;
}
int64_t two_pass_kt(const am_problem* p, int64_t t, int32_t k_mult) {
  const int64_t kt = t * (int64_t)k_mult;
  return kt < p->T ? kt : p->T;
}
size_t ws_two_pass(const am_problem* p, int64_t t, int64_t s, int32_t k_mult) {
  return two_pass_ws_bytes(p->heads, p->n, p->T, p->d, esize(p), s, two_pass_kt(p, t, k_mult));
}
size_t ws_compact_two_pass(const am_problem* p, int64_t t, int64_t s, int32_t k_mult) {
  size_t stage = ws_two_pass(p, t, s, k_mult);
  const size_t f = ws_fast(p, t, 0);
  if (f > stage) stage = f;
  return align_up((size_t)p->heads * p->n * 4) + stage;   // lse_short, then the stages
}
TwoPassArgs two_pass_args(const am_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* sub, int64_t s, int64_t t, int32_t k_mult, int mode,
                          int32_t* idx, void* Ck, void* Vsel, float* lse_short, void* ws,
                          hipStream_t st) {
  TwoPassArgs a;
  a.Q = Q; a.K = K; a.V = V; a.sub = sub; a.idx = idx; a.Ck = Ck; a.Vsel = Vsel;
  a.lse_short = lse_short;
  a.heads = (int)p->heads; a.n = (int)p->n; a.T = (int)p->T; a.d = (int)p->d; a.group = p->group;
  a.s = (int)s; a.t = (int)t; a.kt = (int)two_pass_kt(p, t, k_mult); a.mode = mode;
  a.causal = p->causal != 0; a.bf16 = p->dtype == AM_BF16; a.scale = p->scale;
  a.ws = ws; a.stream = st;
  return a;
}
}  // namespace

size_t am_two_pass_workspace_bytes(const am_problem* p, int64_t t, int64_t s, int32_t k_mult,
                                   int32_t compact) {
  if (check_two_pass(p, s, t, k_mult) != AM_OK) return 0;
  return compact ? ws_compact_two_pass(p, t, s, k_mult) : ws_two_pass(p, t, s, k_mult);
}

am_status am_select_two_pass(const am_problem* p, const void* Q, const void* K, const void* V,
                             const int32_t* sub, int64_t s, int64_t t, int32_t k_mult,
                             am_score_mode mode, int32_t* idx, void* Ck, void* V_sel,
                             float* lse_short, void* ws, size_t ws_bytes, am_stream_t stream) {
  am_status st = check_two_pass(p, s, t, k_mult);
  if (st != AM_OK) return st;
  if (ival(mode) < AM_SCORE_RMS || ival(mode) > AM_SCORE_MAX) return AM_ERR_INVALID_ARG;
  if (!Q || !K || !sub || !idx || !Ck || !lse_short || (V_sel && !V)) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || (V && !al16(V)) || !al16(sub) || !al16(idx) || !al16(Ck) ||
      (V_sel && !al16(V_sel)) || !al16(lse_short) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_two_pass(p, t, s, k_mult)) return AM_ERR_WORKSPACE;
  return from_hip(launch_two_pass(two_pass_args(p, Q, K, V_sel ? V : nullptr, sub, s, t, k_mult,
                                                (int)mode, idx, Ck, V_sel, lse_short, ws,
                                                (hipStream_t)stream)));
}

am_status am_compact_two_pass(const am_problem* p, const void* Q, const void* K, const void* V,
                              const int32_t* sub, int64_t s, int64_t t, int32_t k_mult,
                              am_score_mode mode, int32_t* idx, void* Ck, float* beta, float* Cv,
                              float* resid_out, void* ws, size_t ws_bytes, am_stream_t stream) {
  am_status st = check_two_pass(p, s, t, k_mult);
  if (st != AM_OK) return st;
  if (ival(mode) < AM_SCORE_RMS || ival(mode) > AM_SCORE_MAX) return AM_ERR_INVALID_ARG;
  if (!Q || !K || !V || !sub || !idx || !Ck || !beta || !Cv) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || !al16(V) || !al16(sub) || !al16(idx) || !al16(Ck) ||
      !al16(beta) || !al16(Cv) || (resid_out && !al16(resid_out)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_compact_two_pass(p, t, s, k_mult)) return AM_ERR_WORKSPACE;
  const hipStream_t sm = (hipStream_t)stream;
  float* lse_short = (float*)ws;
  char* stage = (char*)ws + align_up((size_t)p->heads * p->n * 4);
  hipError_t e = launch_two_pass(two_pass_args(p, Q, K, nullptr, sub, s, t, k_mult, (int)mode,
                                               idx, Ck, nullptr, lse_short, stage, sm));
  if (e != hipSuccess) return AM_ERR_DEVICE;
  FitArgs a = fit_args(p, Q, Ck, idx, t, stage, ws_bytes - (size_t)(stage - (char*)ws), sm);
  a.lse = lse_short; a.beta = beta; a.w = nullptr; a.mass_resid = resid_out;
  if ((e = launch_beta_redistribute(a)) != hipSuccess) return AM_ERR_DEVICE;
  a.beta_in = beta; a.Cv = Cv; a.O = nullptr; a.out_resid = nullptr;
  if ((e = launch_values_direct(a, V, (int)p->T)) != hipSuccess) return AM_ERR_DEVICE;
  if (resid_out && (e = launch_fill_f32(resid_out + p->heads, (long long)p->heads, -1.f, sm)) !=
                       hipSuccess)
    return AM_ERR_DEVICE;
  return AM_OK;
}

am_status am_init_anchor_diverse(const am_problem* p, const void* Q, const void* K, int64_t M,
                                 int64_t n_anchor, int32_t* idx, int32_t* order,
                                 int32_t* head_status, void* ws, size_t ws_bytes,
                                 am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, M)) != AM_OK) return st;
  if (n_anchor < 1 || n_anchor > M) return AM_ERR_INVALID_ARG;
  if (M > kInitMaxM || init_max_chunk((int)p->heads, (int)p->T) > kInitMaxChunk)
    return AM_ERR_UNSUPPORTED;
  if (!Q || !K || !idx) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || !al16(idx) || (order && !al16(order)) ||
      (head_status && !al16(head_status)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < init_ws_bytes(p->heads, p->n, p->T, p->d, esize(p), M, M))
    return AM_ERR_WORKSPACE;
  InitArgs a;
  a.Q = Q; a.K = K; a.idx = idx; a.order = order; a.head_status = head_status;
  a.heads = (int)p->heads; a.n = (int)p->n; a.T = (int)p->T; a.d = (int)p->d;
  a.group = p->group; a.M = (int)M; a.na = (int)n_anchor;
  a.causal = p->causal != 0; a.bf16 = p->dtype == AM_BF16; a.scale = p->scale;
  a.ws = ws; a.stream = (hipStream_t)stream;
  return from_hip(launch_init_anchor_diverse(a));
}

am_status am_eval_residuals(const am_problem* p, const void* Q, const void* K, const void* V,
                            const int32_t* idx, const void* Ck, const float* beta,
                            const float* Cv, int64_t t, float* resid_out, void* ws,
                            size_t ws_bytes, am_stream_t stream) {
  am_status st = check_problem(p);
  if (st != AM_OK) return st;
  if ((st = check_t(p, t)) != AM_OK) return st;
  if (!Q || !K || !V || !idx || !Ck || !beta || !Cv || !resid_out) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(K) || !al16(V) || !al16(idx) || !al16(Ck) || !al16(beta) || !al16(Cv) ||
      !al16(resid_out) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_fast(p, t, p->T)) return AM_ERR_WORKSPACE;
  FitArgs a = fit_args(p, Q, Ck, idx, t, ws, ws_bytes, (hipStream_t)stream);
  a.beta_in = beta; a.Cv = (float*)Cv;
  return from_hip(launch_eval_residuals(a, K, V, (int)p->T, resid_out));
}

am_status am_cache_attention(const am_problem* p, const void* Q, const void* Ck, const float* Cv,
                             const float* bias, const int32_t* keypos, const int32_t* nvalid,
                             int64_t m, const void* Kn, const void* Vn, int32_t new_causal,
                             float* out, float* lse, float* lse_cmp, void* ws, size_t ws_bytes,
                             am_stream_t stream) {
  am_status st = check_cache_problem(p);
  if (st != AM_OK) return st;
  if (m < 0 || (new_causal != 0 && new_causal != 1)) return AM_ERR_INVALID_ARG;
  if (m > ((int64_t)1 << 30) || p->heads * m > ((int64_t)1 << 40)) return AM_ERR_UNSUPPORTED;
  if (!Q || !Ck || !Cv || !bias || !out || !lse || (p->causal && !keypos) ||
      (m > 0 && (!Kn || !Vn)))
    return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(Ck) || !al16(Cv) || !al16(bias) || !al16(out) || !al16(lse) ||
      (keypos && !al16(keypos)) || (nvalid && !al16(nvalid)) || (lse_cmp && !al16(lse_cmp)) ||
      (m > 0 && (!al16(Kn) || !al16(Vn))) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  const CacheWs w = cache_ws(p, m);
  if (!ws || ws_bytes < w.total) return AM_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  char* c = (char*)ws;
  void* vt = c;                 c += w.vt;
  int2* tstat = (int2*)c;       c += w.tstat;
  float* bias_eff = (float*)c;  c += w.bias;
  float* lse1 = (float*)c;      c += w.lse1;
  void* vt_new = c;             c += w.vt_new;
  float* O2 = (float*)c;        c += w.o2;
  float* lse2 = (float*)c;
  if (lse_cmp) lse1 = lse_cmp;
  hipError_t e = hipSuccess;
  if (nvalid) {
    e = launch_mask_bias(bias, nvalid, bias_eff, (int)p->heads, (int)p->T, s);
    if (e != hipSuccess) return AM_ERR_DEVICE;
  }
  CmpAttnArgs ca;
  ca.Q = Q; ca.Ck = Ck; ca.Cv = Cv; ca.bias = nvalid ? bias_eff : bias;
  ca.keypos = p->causal ? keypos : nullptr; ca.Y = nullptr;
  ca.Vt = vt; ca.tstat = p->causal ? tstat : nullptr;
  ca.lse = lse1; ca.rowstat = nullptr; ca.O = out; ca.rowres = nullptr;
  ca.heads = (int)p->heads; ca.n = (int)p->n; ca.t = (int)p->T; ca.d = (int)p->d;
  ca.group = p->group; ca.causal = p->causal != 0; ca.bf16 = p->dtype == AM_BF16;
  ca.scale = p->scale; ca.stream = s;
  if ((e = launch_cmp_attention(ca)) != hipSuccess) return AM_ERR_DEVICE;
  if (m > 0) {
    TargetsArgs ta;
    ta.Q = Q; ta.K = Kn; ta.V = Vn; ta.Vt = vt_new; ta.rowstat = nullptr;
    ta.lse = lse2; ta.O = O2; ta.score = nullptr; ta.mode = 0;
    ta.heads = (int)p->heads; ta.n = (int)p->n; ta.T = (int)m; ta.d = (int)p->d;
    ta.group = p->group; ta.causal = new_causal != 0; ta.bf16 = p->dtype == AM_BF16;
    ta.scale = p->scale; ta.stream = s;
    if ((e = launch_targets(ta)) != hipSuccess) return AM_ERR_DEVICE;
  }
  MergeArgs ma;
  ma.O1 = out; ma.lse1 = lse1; ma.O2 = m > 0 ? O2 : nullptr; ma.lse2 = m > 0 ? lse2 : nullptr;
  ma.out = out; ma.lse = lse; ma.rows = (long long)p->heads * p->n; ma.d = (int)p->d;
  ma.stream = s;
  return from_hip(launch_attention_merge(ma));
}

am_status am_attention_merge(int64_t rows, int64_t d, const float* O1, const float* lse1,
                             const float* O2, const float* lse2, float* out, float* lse_out,
                             am_stream_t stream) {
  if (rows < 0 || d < 4 || d % 4 != 0) return AM_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) || d > (1 << 20)) return AM_ERR_UNSUPPORTED;
  if (!O1 || !lse1 || !O2 || !lse2 || !out || !lse_out) return AM_ERR_INVALID_ARG;
  if (!al16(O1) || !al16(O2) || !al16(out) || (((uintptr_t)lse1 | (uintptr_t)lse2 |
      (uintptr_t)lse_out) & 3u))
    return AM_ERR_INVALID_ARG;
  MergeArgs ma;
  ma.O1 = O1; ma.lse1 = lse1; ma.O2 = O2; ma.lse2 = lse2; ma.out = out; ma.lse = lse_out;
  ma.rows = (long long)rows; ma.d = (int)d; ma.stream = (hipStream_t)stream;
  return from_hip(launch_attention_merge(ma));
}

namespace {
// Stage-1 fitting: p->T is the slot count t; query row i sits at position i / group
am_status check_stage1(const am_problem* p, const void* Q, const float* O_full,
                       const float* lse_full, const int32_t* keypos, const int32_t* samples,
                       int64_t S, const void* ws) {
  am_status st = check_cache_problem(p);
  if (st != AM_OK) return st;
  if (p->n % p->group != 0 || S < 1 || S * p->group > ((int64_t)1 << 24)) return AM_ERR_INVALID_ARG;
  if (p->group > 65535) return AM_ERR_UNSUPPORTED;   // a grid dimension of the statistics pass
  if (!Q || !O_full || !lse_full || !samples || (p->causal && !keypos)) return AM_ERR_INVALID_ARG;
  if (!al16(Q) || !al16(O_full) || !al16(lse_full) || !al16(samples) ||
      (keypos && !al16(keypos)) || (ws && !al16(ws)))
    return AM_ERR_INVALID_ARG;
  return AM_OK;
}

Stage1Args stage1_args(const am_problem* p, const void* Q, const float* O_full,
                       const float* lse_full, const int32_t* keypos, const int32_t* samples,
                       int64_t S, void* ws, am_stream_t stream) {
  Stage1Args a;
  memset(&a, 0, sizeof a);
  a.Q = Q; a.O_full = O_full; a.lse_full = lse_full; a.keypos = p->causal ? keypos : nullptr;
  a.samples = samples;
  a.heads = (int)p->heads; a.n = (int)p->n; a.d = (int)p->d; a.group = p->group;
  a.t = (int)p->T; a.S = (int)S;
  a.causal = p->causal != 0; a.bf16 = p->dtype == AM_BF16; a.scale = p->scale;
  a.ws = ws; a.stream = (hipStream_t)stream;
  return a;
}
}  // namespace

size_t am_stage1_workspace_bytes(const am_problem* p, int64_t S) {
  if (check_cache_problem(p) != AM_OK || S < 1 || p->n % p->group != 0 ||
      S * p->group > ((int64_t)1 << 24) || p->group > 65535)
    return 0;
  return stage1_ws_bytes(p->heads, p->n, p->T, p->d, S, p->group);
}

am_status am_stage1_loss_grad(const am_problem* p, const void* Q, const float* O_full,
                              const float* lse_full, const int32_t* keypos,
                              const int32_t* samples, int64_t S, const float* Ck,
                              const float* Cv, const float* bias, float* loss_out, float* gCk,
                              float* gCv, float* gbias, void* ws, size_t ws_bytes,
                              am_stream_t stream) {
  am_status st = check_stage1(p, Q, O_full, lse_full, keypos, samples, S, ws);
  if (st != AM_OK) return st;
  if (!Ck || !Cv || !bias || !gCk || !gCv || !gbias) return AM_ERR_INVALID_ARG;
  if (!al16(Ck) || !al16(Cv) || !al16(bias) || !al16(gCk) || !al16(gCv) || !al16(gbias) ||
      (loss_out && !al16(loss_out)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < stage1_ws_bytes(p->heads, p->n, p->T, p->d, S, p->group))
    return AM_ERR_WORKSPACE;
  Stage1Args a = stage1_args(p, Q, O_full, lse_full, keypos, samples, S, ws, stream);
  a.Ck = (float*)Ck; a.Cv = (float*)Cv; a.b = (float*)bias; a.loss = loss_out;
  a.gCk = gCk; a.gCv = gCv; a.gb = gbias; a.steps = 0;
  return from_hip(launch_stage1(a));
}

am_status am_fit_stage1(const am_problem* p, const void* Q, const float* O_full,
                        const float* lse_full, const int32_t* keypos, const int32_t* samples,
                        int64_t S, int64_t steps, const uint8_t* trainable, float lr, float wd,
                        float* Ck, float* Cv, float* bias, float* loss_out, void* ws,
                        size_t ws_bytes, am_stream_t stream) {
  am_status st = check_stage1(p, Q, O_full, lse_full, keypos, samples, S, ws);
  if (st != AM_OK) return st;
  if (steps < 1 || steps > (1 << 20) || !(lr >= 0.f) || !isfinite(lr) || !(wd >= 0.f) ||
      !isfinite(wd))
    return AM_ERR_INVALID_ARG;
  if (!Ck || !Cv || !bias) return AM_ERR_INVALID_ARG;
  if (!al16(Ck) || !al16(Cv) || !al16(bias) || (trainable && !al16(trainable)) ||
      (loss_out && !al16(loss_out)))
    return AM_ERR_INVALID_ARG;
  if (!ws || ws_bytes < stage1_ws_bytes(p->heads, p->n, p->T, p->d, S, p->group))
    return AM_ERR_WORKSPACE;
  Stage1Args a = stage1_args(p, Q, O_full, lse_full, keypos, samples, S, ws, stream);
  a.Ck = Ck; a.Cv = Cv; a.b = bias; a.loss = loss_out; a.trainable = trainable;
  a.steps = (int)steps; a.lr = lr; a.wd = wd;
  return from_hip(launch_stage1(a));
}

}  // extern "C"
