// Stage-1 attention fitting ("Latent Compaction with Test-Time Training", §3.3 Eq. 8; App.
// A.2: sampled query positions per update, AdamW with constant learning rate): the compacted
// keys C_k, values C_v and biases b (fp32) move to match the full cache's attention outputs
// and log-normalizers on sampled query positions, each error standardized by fixed teacher
// scales per query head.
//
// One update on N = S * group query rows (every query head of S sampled positions):
//   forward   l = scale C_k q + b over the visible slots, P = softmax(l), A = P C_v,
//             log Z = logsumexp(l)                           (s1_forward_kernel)
//   loss      L = mean((A - A_full)^2 / sa_g^2) + mean((log Z - log Z_full)^2 / sz_g^2),
//             rows that see no slot left out                  (s1_count_kernel, s1_out_grad_kernel)
//   backward  dA, dlogZ; dS = P (dA . C_v,j - dA . A + dlogZ); dC_v = P^T dA; dC_k = scale
//             dS^T Q; db = colsum dS                           (s1_dscore_kernel, s1_grad_kernel)
//   AdamW     decoupled decay, bias-corrected moments, trainable slots only (s1_adamw_kernel)
// The sizes are small (N a few hundred to a few thousand rows, t slots), so the kernels are
// plain fp32 loops over LDS-staged rows; every sum runs in a fixed order.
#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

constexpr int kS1Rows = 16;   // query rows per workgroup in the row kernels

// rows r of the update: query i = pos * group + r % group for pos = samples[r / group]
__device__ __forceinline__ int s1_row_query(const int32_t* samples, int r, int group, int n) {
  const int pos = samples[r / group];
  return min(max(pos * group + r % group, 0), n - 1);
}

template <typename T>
__global__ __launch_bounds__(256) void s1_gather_kernel(const T* __restrict__ Q,
                                                        const float* __restrict__ O_full,
                                                        const float* __restrict__ lse_full,
                                                        const int32_t* __restrict__ samples,
                                                        float* __restrict__ Qs, float* __restrict__ Y,
                                                        float* __restrict__ lzt, int* __restrict__ qpos,
                                                        int n, int d, int N, int group) {
  const int head = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)N * d) return;
  const int r = (int)(e / d), c = (int)(e - (long long)r * d);
  const int i = s1_row_query(samples, r, group, n);
  const size_t src = ((size_t)head * n + i) * d + c, dst = ((size_t)head * N + r) * d + c;
  Qs[dst] = (float)Q[src];
  Y[dst] = O_full[src];
  if (c == 0) {
    lzt[(size_t)head * N + r] = lse_full[(size_t)head * n + i];
    qpos[(size_t)head * N + r] = i / group;
  }
}

// P [h, N, t], A [h, N, d], lz [h, N] for a block of kS1Rows rows; thread (row, lane of 16)
template <int D>
__global__ __launch_bounds__(256) void s1_forward_kernel(const float* __restrict__ Qs,
                                                         const int* __restrict__ qpos,
                                                         const float* __restrict__ Ck,
                                                         const float* __restrict__ Cv,
                                                         const float* __restrict__ b,
                                                         const int32_t* __restrict__ keypos,
                                                         float* __restrict__ P, float* __restrict__ A,
                                                         float* __restrict__ lz, int N, int t,
                                                         float scale, int causal) {
  __shared__ float qs[kS1Rows][D + 1];
  const int head = blockIdx.y, r0 = blockIdx.x * kS1Rows, tid = threadIdx.x;
  const int rr = tid >> 4, c = tid & 15, r = r0 + rr;
  for (int e = tid; e < kS1Rows * D; e += 256) {
    const int a = e / D, k = e % D;
    qs[a][k] = r0 + a < N ? Qs[((size_t)head * N + r0 + a) * D + k] : 0.f;
  }
  __syncthreads();
  const float* Ckh = Ck + (size_t)head * t * D;
  const float* Cvh = Cv + (size_t)head * t * D;
  float* Pr = P + ((size_t)head * N + min(r, N - 1)) * t;
  const int qp = r < N ? qpos[(size_t)head * N + r] : 0;
  // scores and the row max
  float mx = -INFINITY;
  for (int j = c; j < t; j += 16) {
    float s = -INFINITY;
    if (!causal || keypos[(size_t)head * t + j] <= qp) {
      float acc = 0.f;
      const float* kr = Ckh + (size_t)j * D;
      for (int k = 0; k < D; ++k) acc = __builtin_fmaf(qs[rr][k], kr[k], acc);
      s = scale * acc + b[(size_t)head * t + j];
    }
    if (r < N) Pr[j] = s;
    mx = fmaxf(mx, s);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  // exponentials and the normalizer
  float sum = 0.f;
  for (int j = c; j < t; j += 16) {
    const float e = (mx == -INFINITY || r >= N) ? 0.f : expf(Pr[j] - mx);
    if (r < N) Pr[j] = e;
    sum += e;
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int j = c; j < t; j += 16)
    if (r < N) Pr[j] *= inv;
  __syncthreads();   // the row's probabilities are complete before the product reads them
  if (r >= N) return;
  if (c == 0) lz[(size_t)head * N + r] = sum > 0.f ? mx + logf(sum) : -INFINITY;
  for (int ch = c; ch < D; ch += 16) {
    float acc = 0.f;
    for (int j = 0; j < t; ++j) acc = __builtin_fmaf(Pr[j], Cvh[(size_t)j * D + ch], acc);
    A[((size_t)head * N + r) * D + ch] = acc;
  }
}

// rows that see at least one slot, per head
__global__ __launch_bounds__(256) void s1_count_kernel(const float* __restrict__ lz,
                                                       int* __restrict__ kept, int N) {
  __shared__ int red[256];
  const int head = blockIdx.x;
  int c = 0;
  for (int r = threadIdx.x; r < N; r += 256) c += lz[(size_t)head * N + r] > -INFINITY ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) red[threadIdx.x] += red[threadIdx.x + s2];
    __syncthreads();
  }
  if (threadIdx.x == 0) kept[head] = red[0];
}

// dA [h, N, d], dlz and D = dA . A [h, N], the row's loss term [h, N]; one row per 64 threads
template <int D>
__global__ __launch_bounds__(256) void s1_out_grad_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ Y,
                                                          const float* __restrict__ lz,
                                                          const float* __restrict__ lzt,
                                                          const float* __restrict__ sa,
                                                          const float* __restrict__ sz,
                                                          const int* __restrict__ kept,
                                                          float* __restrict__ dA,
                                                          float* __restrict__ dlz,
                                                          float* __restrict__ Dr,
                                                          float* __restrict__ lrow, int N,
                                                          int group) {
  const int head = blockIdx.y, r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= N) return;
  const size_t o = (size_t)head * N + r;
  const int g = r % group, nk = kept[head];
  const float z = lz[o];
  const bool keep = z > -INFINITY && nk > 0;
  const float wa = 1.f / (sa[head * group + g] * sa[head * group + g]);
  const float wz = 1.f / (sz[head * group + g] * sz[head * group + g]);
  float da_dot = 0.f, sq = 0.f;
  for (int ch = lane; ch < D; ch += 64) {
    const size_t q = o * D + ch;
    const float e = A[q] - Y[q];
    const float g2 = keep ? 2.f * wa * e / ((float)nk * D) : 0.f;
    dA[q] = g2;
    da_dot += g2 * A[q];
    sq += keep ? wa * e * e : 0.f;
  }
#pragma unroll
  for (int s2 = 32; s2 > 0; s2 >>= 1) {
    da_dot += __shfl_xor(da_dot, s2, 64);
    sq += __shfl_xor(sq, s2, 64);
  }
  if (lane == 0) {
    const float ez = keep ? z - lzt[o] : 0.f;
    dlz[o] = keep ? 2.f * wz * ez / (float)nk : 0.f;
    Dr[o] = da_dot;
    lrow[o] = keep ? sq / ((float)nk * D) + wz * ez * ez / (float)nk : 0.f;
  }
}

// dS [h, N, t] = P (dA . C_v,j - D + dlz); thread (row, lane of 16) over the slots
template <int D>
__global__ __launch_bounds__(256) void s1_dscore_kernel(const float* __restrict__ P,
                                                        const float* __restrict__ dA,
                                                        const float* __restrict__ Dr,
                                                        const float* __restrict__ dlz,
                                                        const float* __restrict__ Cv,
                                                        float* __restrict__ dS, int N, int t) {
  __shared__ float ds[kS1Rows][D + 1];
  const int head = blockIdx.y, r0 = blockIdx.x * kS1Rows, tid = threadIdx.x;
  const int rr = tid >> 4, c = tid & 15, r = r0 + rr;
  for (int e = tid; e < kS1Rows * D; e += 256) {
    const int a = e / D, k = e % D;
    ds[a][k] = r0 + a < N ? dA[((size_t)head * N + r0 + a) * D + k] : 0.f;
  }
  __syncthreads();
  if (r >= N) return;
  const size_t o = (size_t)head * N + r;
  const float base = dlz[o] - Dr[o];
  const float* Cvh = Cv + (size_t)head * t * D;
  for (int j = c; j < t; j += 16) {
    const float pj = P[o * t + j];
    float acc = 0.f;
    if (pj != 0.f) {
      const float* vr = Cvh + (size_t)j * D;
      for (int k = 0; k < D; ++k) acc = __builtin_fmaf(ds[rr][k], vr[k], acc);
    }
    dS[o * t + j] = pj * (acc + base);
  }
}

// dCk, dCv [h, t, d] and db [h, t]: thread (slot of 16, lane of 16) over the rows in order
template <int D>
__global__ __launch_bounds__(256) void s1_grad_kernel(const float* __restrict__ P,
                                                      const float* __restrict__ dS,
                                                      const float* __restrict__ dA,
                                                      const float* __restrict__ Qs,
                                                      float* __restrict__ gCk, float* __restrict__ gCv,
                                                      float* __restrict__ gb, int N, int t,
                                                      float scale) {
  const int head = blockIdx.y, j = blockIdx.x * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  if (j >= t) return;
  float ak[D / 16], av[D / 16], sb = 0.f;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) ak[u] = av[u] = 0.f;
  for (int r = 0; r < N; ++r) {
    const size_t o = (size_t)head * N + r;
    const float pj = P[o * t + j], sj = dS[o * t + j];
    sb += sj;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const int ch = c + 16 * u;
      av[u] = __builtin_fmaf(pj, dA[o * D + ch], av[u]);
      ak[u] = __builtin_fmaf(sj, Qs[o * D + ch], ak[u]);
    }
  }
  const size_t q = ((size_t)head * t + j) * D;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    gCv[q + c + 16 * u] = av[u];
    gCk[q + c + 16 * u] = scale * ak[u];
  }
  if (c == 0) gb[(size_t)head * t + j] = sb;
}

// AdamW on `count` parameters of `per_slot` values each (slot = e / per_slot)
__global__ __launch_bounds__(256) void s1_adamw_kernel(float* __restrict__ th,
                                                       const float* __restrict__ g,
                                                       float* __restrict__ m, float* __restrict__ v,
                                                       const uint8_t* __restrict__ trainable,
                                                       long long count, int per_slot, float lr,
                                                       float wd, float bc1, float bc2) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= count) return;
  if (trainable && !trainable[e / per_slot]) return;
  const float gg = g[e];
  const float mm = 0.9f * m[e] + 0.1f * gg;
  const float vv = 0.999f * v[e] + 0.001f * gg * gg;
  m[e] = mm;
  v[e] = vv;
  th[e] = th[e] * (1.f - lr * wd) - lr * (mm / bc1) / (sqrtf(vv / bc2) + 1e-8f);
}

// loss[h] = sum of the row terms in order
__global__ __launch_bounds__(256) void s1_loss_kernel(const float* __restrict__ lrow,
                                                      float* __restrict__ loss, int N) {
  __shared__ double red[256];
  const int head = blockIdx.x;
  double acc = 0.0;
  for (int r = threadIdx.x; r < N; r += 256) acc += (double)lrow[(size_t)head * N + r];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) red[threadIdx.x] += red[threadIdx.x + s2];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[head] = (float)red[0];
}

// teacher scales per (head, query head): population std of the outputs over positions and
// channels and of the log-normalizers over positions, floored at 1e-4
__global__ __launch_bounds__(256) void s1_scales_kernel(const float* __restrict__ O_full,
                                                        const float* __restrict__ lse_full,
                                                        float* __restrict__ sa,
                                                        float* __restrict__ sz, int n, int d,
                                                        int group) {
  __shared__ double red[4][256];
  const int head = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  double s1 = 0.0, s2 = 0.0, z1 = 0.0, z2 = 0.0;
  for (int i = g; i < n; i += group) {
    const float* row = O_full + ((size_t)head * n + i) * d;
    for (int c = tid; c < d; c += 256) {
      const double x = row[c];
      s1 += x;
      s2 += x * x;
    }
    if (tid == 0) {
      const double z = lse_full[(size_t)head * n + i];
      z1 += z;
      z2 += z * z;
    }
  }
  red[0][tid] = s1; red[1][tid] = s2; red[2][tid] = z1; red[3][tid] = z2;
  __syncthreads();
  for (int h2 = 128; h2 > 0; h2 >>= 1) {
    if (tid < h2)
      for (int k = 0; k < 4; ++k) red[k][tid] += red[k][tid + h2];
    __syncthreads();
  }
  if (tid == 0) {
    const double rows = (double)((n - g + group - 1) / group);
    const double cnt = rows * d;
    const double va = fmax(red[1][0] / cnt - (red[0][0] / cnt) * (red[0][0] / cnt), 0.0);
    const double vz = fmax(red[3][0] / rows - (red[2][0] / rows) * (red[2][0] / rows), 0.0);
    sa[head * group + g] = (float)fmax(sqrt(va), 1e-4);
    sz[head * group + g] = (float)fmax(sqrt(vz), 1e-4);
  }
}

namespace {
struct Carve4 {
  char* base; size_t off;
  template <typename X> X* take(size_t count) {
    X* q = (X*)(base + off);
    off = align_up(off + count * sizeof(X));
    return q;
  }
};
struct S1Plan {
  float *Qs, *Y, *lzt, *P, *dS, *A, *lz, *dA, *dlz, *Dr, *lrow, *sa, *sz;
  int *qpos, *kept;
  float *gCk, *gCv, *gb, *mCk, *vCk, *mCv, *vCv, *mb, *vb;
  size_t bytes;
};
S1Plan plan_s1(char* base, int64_t h, int64_t t, int64_t d, int64_t N, int64_t group) {
  Carve4 c{base, 0};
  S1Plan q;
  q.Qs = c.take<float>((size_t)h * N * d);
  q.Y = c.take<float>((size_t)h * N * d);
  q.lzt = c.take<float>(h * N);
  q.qpos = c.take<int>(h * N);
  q.P = c.take<float>((size_t)h * N * t);
  q.dS = c.take<float>((size_t)h * N * t);
  q.A = c.take<float>((size_t)h * N * d);
  q.lz = c.take<float>(h * N);
  q.dA = c.take<float>((size_t)h * N * d);
  q.dlz = c.take<float>(h * N);
  q.Dr = c.take<float>(h * N);
  q.lrow = c.take<float>(h * N);
  q.kept = c.take<int>(h);
  q.sa = c.take<float>(h * group);
  q.sz = c.take<float>(h * group);
  q.gCk = c.take<float>((size_t)h * t * d);
  q.gCv = c.take<float>((size_t)h * t * d);
  q.gb = c.take<float>(h * t);
  q.mCk = c.take<float>((size_t)h * t * d);
  q.vCk = c.take<float>((size_t)h * t * d);
  q.mCv = c.take<float>((size_t)h * t * d);
  q.vCv = c.take<float>((size_t)h * t * d);
  q.mb = c.take<float>(h * t);
  q.vb = c.take<float>(h * t);
  q.bytes = c.off;
  return q;
}
unsigned cdiv4(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

// forward + loss + gradients of one update (rows from `samples`), into the plan's buffers
template <int D>
hipError_t s1_eval(const Stage1Args& a, const S1Plan& pl, const int32_t* samples, float* loss,
                   float* gCk, float* gCv, float* gb) {
  const hipStream_t st = a.stream;
  const int H = a.heads, N = a.S * a.group, t = a.t;
  const dim3 gg(cdiv4((long long)N * D, 256), H);
  if (a.bf16)
    hipLaunchKernelGGL(s1_gather_kernel<bf16>, gg, dim3(256), 0, st, (const bf16*)a.Q, a.O_full,
                       a.lse_full, samples, pl.Qs, pl.Y, pl.lzt, pl.qpos, a.n, D, N, a.group);
  else
    hipLaunchKernelGGL(s1_gather_kernel<float>, gg, dim3(256), 0, st, (const float*)a.Q, a.O_full,
                       a.lse_full, samples, pl.Qs, pl.Y, pl.lzt, pl.qpos, a.n, D, N, a.group);
  const dim3 gr(cdiv4(N, kS1Rows), H);
  hipLaunchKernelGGL(s1_forward_kernel<D>, gr, dim3(256), 0, st, (const float*)pl.Qs,
                     (const int*)pl.qpos, (const float*)a.Ck, (const float*)a.Cv,
                     (const float*)a.b, a.keypos, pl.P, pl.A, pl.lz, N, t, a.scale,
                     a.causal ? 1 : 0);
  hipLaunchKernelGGL(s1_count_kernel, dim3(H), dim3(256), 0, st, (const float*)pl.lz, pl.kept, N);
  hipLaunchKernelGGL(s1_out_grad_kernel<D>, dim3(cdiv4(N, 4), H), dim3(256), 0, st,
                     (const float*)pl.A, (const float*)pl.Y, (const float*)pl.lz,
                     (const float*)pl.lzt, (const float*)pl.sa, (const float*)pl.sz,
                     (const int*)pl.kept, pl.dA, pl.dlz, pl.Dr, pl.lrow, N, a.group);
  if (loss)
    hipLaunchKernelGGL(s1_loss_kernel, dim3(H), dim3(256), 0, st, (const float*)pl.lrow, loss, N);
  hipLaunchKernelGGL(s1_dscore_kernel<D>, gr, dim3(256), 0, st, (const float*)pl.P,
                     (const float*)pl.dA, (const float*)pl.Dr, (const float*)pl.dlz,
                     (const float*)a.Cv, pl.dS, N, t);
  hipLaunchKernelGGL(s1_grad_kernel<D>, dim3(cdiv4(t, 16), H), dim3(256), 0, st,
                     (const float*)pl.P, (const float*)pl.dS, (const float*)pl.dA,
                     (const float*)pl.Qs, gCk, gCv, gb, N, t, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t s1_run(const Stage1Args& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, t = a.t;
  S1Plan pl = plan_s1((char*)a.ws, H, t, D, (int64_t)a.S * a.group, a.group);
  hipLaunchKernelGGL(s1_scales_kernel, dim3(a.group, H), dim3(256), 0, st, a.O_full, a.lse_full,
                     pl.sa, pl.sz, a.n, D, a.group);
  if (a.steps == 0)   // one evaluation: gradients to the caller
    return s1_eval<D>(a, pl, a.samples, a.loss, a.gCk, a.gCv, a.gb);
  const long long nkv = (long long)H * t * D, nb = (long long)H * t;
  float* zeros[] = {pl.mCk, pl.vCk, pl.mCv, pl.vCv};
  for (float* z : zeros) {
    hipError_t e = launch_fill_f32(z, nkv, 0.f, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_fill_f32(pl.mb, nb, 0.f, st);
  if (e != hipSuccess) return e;
  if ((e = launch_fill_f32(pl.vb, nb, 0.f, st)) != hipSuccess) return e;
  for (int k = 1; k <= a.steps; ++k) {
    e = s1_eval<D>(a, pl, a.samples + (size_t)(k - 1) * a.S,
                   a.loss ? a.loss + (size_t)(k - 1) * H : nullptr, pl.gCk, pl.gCv, pl.gb);
    if (e != hipSuccess) return e;
    const float bc1 = (float)(1.0 - pow(0.9, k)), bc2 = (float)(1.0 - pow(0.999, k));
    hipLaunchKernelGGL(s1_adamw_kernel, dim3(cdiv4(nkv, 256)), dim3(256), 0, st, a.Ck,
                       (const float*)pl.gCk, pl.mCk, pl.vCk, a.trainable, nkv, D, a.lr, a.wd, bc1, bc2);
    hipLaunchKernelGGL(s1_adamw_kernel, dim3(cdiv4(nkv, 256)), dim3(256), 0, st, a.Cv,
                       (const float*)pl.gCv, pl.mCv, pl.vCv, a.trainable, nkv, D, a.lr, a.wd, bc1, bc2);
    hipLaunchKernelGGL(s1_adamw_kernel, dim3(cdiv4(nb, 256)), dim3(256), 0, st, a.b,
                       (const float*)pl.gb, pl.mb, pl.vb, a.trainable, nb, 1, a.lr, a.wd, bc1, bc2);
  }
  return hipGetLastError();
}
}  // namespace

size_t stage1_ws_bytes(int64_t heads, int64_t t, int64_t d, int64_t S, int64_t group) {
  return plan_s1(nullptr, heads, t, d, S * group, group).bytes;
}

hipError_t launch_stage1(const Stage1Args& a) {
  return a.d == 128 ? s1_run<128>(a) : s1_run<64>(a);
}

}  // namespace amc
