// Two-pass key selection ("Compaction" blog, §Choosing C_k, Attempt #3 "Two-Pass"):
//   pass 1: a query subset (ascending query indices, e.g. a seeded random sample) against
//           all T keys gives a per-key statistic; the k * t best keys form a shortlist;
//   pass 2: all n queries against the shortlist, each query's softmax normalized over the
//           shortlist keys it sees; the t best shortlist keys are the selection.
// Both passes reuse the flash pass (row statistics) and the column pass (per-key
// statistic); queries of the subset and keys of the shortlist carry their positions for
// the causal mask.
#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

// Qs[h, i] = Q[h, sub[h, i]] and its position qpos[h, i] = sub[h, i] / group (indices
// clamped into [0, n)). One thread per 16 bytes of a row.
template <typename T>
__global__ __launch_bounds__(256) void gather_queries_kernel(const T* __restrict__ Q,
                                                             const int32_t* __restrict__ sub,
                                                             T* __restrict__ Qs,
                                                             int32_t* __restrict__ qpos, int n,
                                                             int s, int d, int group) {
  const int head = blockIdx.y;
  const int cpr = d * (int)sizeof(T) / 16;   // 16-byte chunks per row
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)s * cpr) return;
  const int i = (int)(e / cpr), c = (int)(e - (long long)i * cpr);
  const int src = min(max(sub[(size_t)head * s + i], 0), n - 1);
  const uint4* from = (const uint4*)(Q + ((size_t)head * n + src) * d);
  uint4* to = (uint4*)(Qs + ((size_t)head * s + i) * d);
  to[c] = from[c];
  if (c == 0) qpos[(size_t)head * s + i] = src / group;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, long long count,
                                                       float v) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < count) p[e] = v;
}

// idx[h, r] = shortlist[h, loc[h, r]] (both ascending, so idx is ascending)
__global__ __launch_bounds__(256) void map_idx_kernel(const int32_t* __restrict__ shortlist,
                                                      const int32_t* __restrict__ loc,
                                                      int32_t* __restrict__ idx, int kt, int t) {
  const int head = blockIdx.y, r = blockIdx.x * 256 + threadIdx.x;
  if (r >= t) return;
  const int j = min(max(loc[(size_t)head * t + r], 0), kt - 1);
  idx[(size_t)head * t + r] = shortlist[(size_t)head * kt + j];
}

namespace {
struct TwoPassPlan {
  void* Qs; int32_t* qpos; float* lse1; float2* rs1; float* score1;
  int32_t* sidx; void* Ks; void* Vs; float* zbias; int2* tstat; float2* rs2; float* score2;
  float* part; int32_t* loc;
  size_t bytes;
};
struct Carve2 {
  char* base; size_t off;
  template <typename X> X* take(size_t count) {
    X* p = base ? (X*)(base + off) : nullptr;   // sizing only: no address
    off = align_up(off + count * sizeof(X));
    return p;
  }
};
TwoPassPlan plan(char* base, int64_t h, int64_t n, int64_t T, int64_t d, int es, int64_t s,
                 int64_t kt) {
  Carve2 c{base, 0};
  TwoPassPlan p;
  p.Qs = c.take<char>((size_t)h * s * d * es);
  p.qpos = c.take<int32_t>(h * s);
  p.lse1 = c.take<float>(h * s);
  p.rs1 = c.take<float2>(h * s);
  p.score1 = c.take<float>(h * T);
  p.sidx = c.take<int32_t>(h * kt);
  p.Ks = c.take<char>((size_t)h * kt * d * es);
  p.Vs = c.take<char>((size_t)h * kt * d * es);
  p.zbias = c.take<float>(h * kt);
  p.tstat = (int2*)c.take<char>(cmp_tstat_bytes(h, kt));
  p.rs2 = c.take<float2>(h * n);
  p.score2 = c.take<float>(h * kt);
  p.part = (float*)c.take<char>(key_mass_part_bytes(h, n, kt));
  p.loc = c.take<int32_t>(h * kt);
  p.bytes = c.off;
  return p;
}
unsigned cdiv2(long long a, long long b) { return (unsigned)((a + b - 1) / b); }
}  // namespace

hipError_t launch_fill_f32(float* p, long long count, float v, hipStream_t st) {
  if (count > 0)
    hipLaunchKernelGGL(fill_f32_kernel, dim3(cdiv2(count, 256)), dim3(256), 0, st, p, count, v);
  return hipGetLastError();
}

size_t two_pass_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize, int64_t s,
                         int64_t kt) {
  return plan(nullptr, heads, n, T, d, esize, s, kt).bytes;
}

hipError_t launch_two_pass(const TwoPassArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, es = a.bf16 ? 2 : 4;
  TwoPassPlan pl = plan((char*)a.ws, H, a.n, a.T, a.d, es, a.s, a.kt);
  // pass 1: the query subset against every key
  const int cpr = a.d * es / 16;
  const dim3 gq(cdiv2((long long)a.s * cpr, 256), H);
  if (a.bf16)
    hipLaunchKernelGGL(gather_queries_kernel<bf16>, gq, dim3(256), 0, st, (const bf16*)a.Q, a.sub,
                       (bf16*)pl.Qs, pl.qpos, a.n, a.s, a.d, a.group);
  else
    hipLaunchKernelGGL(gather_queries_kernel<float>, gq, dim3(256), 0, st, (const float*)a.Q,
                       a.sub, (float*)pl.Qs, pl.qpos, a.n, a.s, a.d, a.group);
  TargetsArgs ta;
  ta.Q = pl.Qs; ta.K = a.K; ta.V = nullptr; ta.Vt = nullptr; ta.rowstat = pl.rs1;
  ta.lse = pl.lse1; ta.O = nullptr; ta.score = pl.score1; ta.mode = a.mode;
  ta.heads = H; ta.n = a.s; ta.T = a.T; ta.d = a.d; ta.group = a.group; ta.causal = a.causal;
  ta.bf16 = a.bf16; ta.scale = a.scale; ta.stream = st;
  ta.qpos = a.causal ? pl.qpos : nullptr;
  hipError_t e = launch_targets(ta);
  if (e != hipSuccess) return e;
  // shortlist: the k * t best keys, with their rows
  SelectArgs sa;
  sa.score = pl.score1; sa.K = a.K; sa.V = a.V; sa.idx = pl.sidx; sa.Ck = pl.Ks;
  sa.Vsel = a.V ? pl.Vs : nullptr;
  sa.heads = H; sa.T = a.T; sa.t = a.kt; sa.d = a.d; sa.bf16 = a.bf16; sa.stream = st;
  if ((e = launch_select(sa)) != hipSuccess) return e;
  // pass 2: every query against the shortlist (row statistics, then the key statistic)
  const long long zb = (long long)H * a.kt;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(cdiv2(zb, 256)), dim3(256), 0, st, pl.zbias, zb, 0.f);
  CmpAttnArgs ca;
  ca.Q = a.Q; ca.Ck = pl.Ks; ca.Cv = nullptr; ca.bias = pl.zbias;
  ca.keypos = a.causal ? pl.sidx : nullptr; ca.Y = nullptr;
  ca.Vt = nullptr; ca.tstat = a.causal ? pl.tstat : nullptr;
  ca.lse = a.lse_short; ca.rowstat = pl.rs2; ca.O = nullptr; ca.rowres = nullptr;
  ca.heads = H; ca.n = a.n; ca.t = a.kt; ca.d = a.d; ca.group = a.group; ca.causal = a.causal;
  ca.bf16 = a.bf16; ca.scale = a.scale; ca.stream = st;
  if ((e = launch_cmp_attention(ca)) != hipSuccess) return e;
  KeyScoreArgs ks;
  ks.Q = a.Q; ks.Ck = pl.Ks; ks.keypos = pl.sidx; ks.rowstat = pl.rs2; ks.score = pl.score2;
  ks.part = pl.part; ks.mode = a.mode;
  ks.heads = H; ks.n = a.n; ks.t = a.kt; ks.d = a.d; ks.group = a.group; ks.causal = a.causal;
  ks.bf16 = a.bf16; ks.scale = a.scale; ks.stream = st;
  if ((e = launch_key_score(ks)) != hipSuccess) return e;
  // the t best of the shortlist, gathered from the shortlist rows, then original indices
  SelectArgs s2;
  s2.score = pl.score2; s2.K = pl.Ks; s2.V = a.Vsel ? pl.Vs : nullptr; s2.idx = pl.loc;
  s2.Ck = a.Ck; s2.Vsel = a.Vsel;
  s2.heads = H; s2.T = a.kt; s2.t = a.t; s2.d = a.d; s2.bf16 = a.bf16; s2.stream = st;
  if ((e = launch_select(s2)) != hipSuccess) return e;
  hipLaunchKernelGGL(map_idx_kernel, dim3(cdiv2(a.t, 256), H), dim3(256), 0, st,
                     (const int32_t*)pl.sidx, (const int32_t*)pl.loc, a.idx, a.kt, a.t);
  return hipGetLastError();
}

}  // namespace amc
