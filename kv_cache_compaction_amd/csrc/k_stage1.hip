// Stage-1 attention fitting ("Latent Compaction with Test-Time Training", §3.3 Eq. 8; App.
// A.2: sampled query positions per update, AdamW with constant learning rate): the compacted
// keys C_k, values C_v and biases b (fp32) move to match the full cache's attention outputs
// and log-normalizers on sampled query positions, each error standardized by fixed teacher
// scales per query head.
//
// One update on N = S * group query rows (every query head of S sampled positions), per
// head, with the products on fp32 MFMA (s1_gemm_kernel, 64x64 tiles):
//   scores    l = scale Q C_k^T + b, masked by position         (GEMM, score epilogue)
//   softmax   P = softmax(l), log Z                                (s1_softmax_kernel)
//   output    A = P C_v                                           (GEMM)
//   loss      L = mean((A - A_full)^2 / sa_g^2) + mean((log Z - log Z_full)^2 / sz_g^2)
//             over the rows that see a slot; dA, dlogZ            (s1_out_grad_kernel; the
//             sum in s1_colsum_kernel)
//   backward  dS = P (dA C_v^T - rowsum(dA A) + dlogZ)             (GEMM, dS epilogue, with
//             the column sums of each tile for db); dC_v = P^T dA; dC_k = scale dS^T Q (GEMMs)
//   AdamW     decoupled decay, bias-corrected moments, trainable slots only (s1_adamw_kernel)
// Every sum runs in a fixed order (no floating-point atomics).
#include <string.h>

#include <algorithm>

#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

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

// C[z] = alpha A[z] B[z] on fp32 MFMA (32x32x2): 64x64 output tiles, 4 waves of 32x32, k
// staged through LDS 32 deep. A(m, k) is A[m lda + k] (AK) or A[k lda + m]; B(k, n) is
// B[n ldb + k] (BK) or B[k ldb + n]; C[m ldc + n]. Out-of-range rows, columns and k are
// zero-filled on load and not stored.
struct S1Gemm {
  const float* A; long long sAz; int lda;
  const float* B; long long sBz; int ldb;
  float* C; long long sCz; int ldc;
  int M, N, K;
  float alpha;
  // score epilogue: + bias[z, n]; -inf where keypos[z, n] > qpos[z, m] (causal)
  const float* bias; const int32_t* keypos; long long sbz;
  const int* qpos; long long sqz; int causal;
  // dS epilogue: P[z, m, n] (C's layout) (acc - Dr[z, m] + dlz[z, m]); the column sums of
  // each 64-row tile to colpart[z, tile, n]
  const float* P; const float* Dr; const float* dlz; float* colpart;
  // blockIdx.z >= zsplit: a second product of the same shape and strides (A2, B2, C2, alpha2)
  int zsplit;
  // split k: blockIdx.z = z * ksplit + part; part s covers its share of k (whole 32-deep
  // tiles) and writes C + s * sCk
  int ksplit; long long sCk;
  const float* A2; const float* B2; float* C2; float alpha2;
};
enum { kEpiStore = 0, kEpiScore = 1, kEpiDS = 2 };
constexpr int kGT = 64, kGK = 32;

template <bool AK, bool BK, int EPI>
__global__ __launch_bounds__(256) void s1_gemm_kernel(const S1Gemm g) {
  __shared__ float As[kGK][kGT + 1];
  __shared__ float Bs[kGK][kGT + 1];
  __shared__ float csum[2][kGT];
  const bool second = (int)blockIdx.z >= g.zsplit;
  const int zz = second ? blockIdx.z - g.zsplit : blockIdx.z;
  const int z = zz / g.ksplit, kpart = zz - z * g.ksplit;
  const int kchunk = ((g.K + g.ksplit - 1) / g.ksplit + kGK - 1) / kGK * kGK;
  const int kbeg = kpart * kchunk, kend = min(g.K, kbeg + kchunk);
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const float* A = (second ? g.A2 : g.A) + z * g.sAz;
  const float* B = (second ? g.B2 : g.B) + z * g.sBz;
  float ra[8], rb[8];
  // element f of a 64x32 tile: k fastest when that dimension is contiguous in memory
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = tid + 256 * i;
      const int am = AK ? f >> 5 : f & 63, ak = AK ? f & 31 : f >> 6;
      const int gm = m0 + am, gk = k0 + ak;
      ra[i] = (gm < g.M && gk < kend)
                  ? (AK ? A[(size_t)gm * g.lda + gk] : A[(size_t)gk * g.lda + gm]) : 0.f;
      const int bn = BK ? f >> 5 : f & 63, bk = BK ? f & 31 : f >> 6;
      const int gn = n0 + bn, gkb = k0 + bk;
      rb[i] = (gn < g.N && gkb < kend)
                  ? (BK ? B[(size_t)gn * g.ldb + gkb] : B[(size_t)gkb * g.ldb + gn]) : 0.f;
    }
  };
  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  const int nk = kend > kbeg ? (kend - kbeg + kGK - 1) / kGK : 0;
  if (nk > 0) load(kbeg);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();   // the previous tile's products are done with the LDS tiles
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = tid + 256 * i;
      if (AK) As[f & 31][f >> 5] = ra[i]; else As[f >> 6][f & 63] = ra[i];
      if (BK) Bs[f & 31][f >> 5] = rb[i]; else Bs[f >> 6][f & 63] = rb[i];
    }
    __syncthreads();
    if (kt + 1 < nk) load(kbeg + (kt + 1) * kGK);
#pragma unroll
    for (int kk = 0; kk < kGK; kk += 2) {
      const float a = As[kk + (lane >> 5)][wm + (lane & 31)];
      const float b = Bs[kk + (lane >> 5)][wn + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
  }
  // the lane holds C[row wm + crow(j, lane / 32)][col wn + lane % 32] in acc[j]
  const int n = n0 + wn + (lane & 31);
  float* C = (second ? g.C2 : g.C) + z * g.sCz + kpart * g.sCk;
  const float alpha = second ? g.alpha2 : g.alpha;
  float cs = 0.f, bn = 0.f;
  int kp = 0;
  if (EPI == kEpiScore && n < g.N) {
    bn = g.bias[z * g.sbz + n];
    kp = g.causal ? g.keypos[z * g.sbz + n] : 0;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int m = m0 + wm + crow(j, lane >> 5);
    if (m >= g.M || n >= g.N) continue;
    const size_t o = (size_t)m * g.ldc + n;
    float v = alpha * acc[j];
    if (EPI == kEpiScore) {
      v += bn;
      if (g.causal && kp > g.qpos[z * g.sqz + m]) v = -INFINITY;
    } else if (EPI == kEpiDS) {
      v = g.P[z * g.sCz + o] * (v - g.Dr[z * g.sqz + m] + g.dlz[z * g.sqz + m]);
      cs += v;
    }
    C[o] = v;
  }
  if (EPI == kEpiDS) {
    // the tile's column sums: the two lane halves, then the two row halves of waves
    cs += __shfl_xor(cs, 32, 64);
    if (lane < 32) csum[wave >> 1][wn + lane] = cs;
    __syncthreads();
    if (tid < kGT && n0 + tid < g.N)
      g.colpart[((size_t)z * gridDim.y + blockIdx.y) * g.N + n0 + tid] = csum[0][tid] + csum[1][tid];
  }
}

// P = softmax of the score rows in place and lz = log-normalizer (-inf for a row that sees
// no slot); one wave per row.
// Rows of up to 64 * kS1SoftVals slots stay in registers (one read, one write).
constexpr int kS1SoftVals = 32;
template <bool REG>
__global__ __launch_bounds__(256) void s1_softmax_kernel(float* __restrict__ P,
                                                         float* __restrict__ lz, int N, int t) {
  const int head = blockIdx.y, r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= N) return;
  float* row = P + ((size_t)head * N + r) * t;
  float v[REG ? kS1SoftVals : 1];
  float mx = -INFINITY;
  if (REG) {
#pragma unroll
    for (int u = 0; u < kS1SoftVals; ++u) {
      const int j = u * 64 + lane;
      v[u] = j < t ? row[j] : -INFINITY;
      mx = fmaxf(mx, v[u]);
    }
  } else {
    for (int j = lane; j < t; j += 64) mx = fmaxf(mx, row[j]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float sum = 0.f;
  if (REG) {
#pragma unroll
    for (int u = 0; u < kS1SoftVals; ++u) {
      v[u] = mx == -INFINITY ? 0.f : expf(v[u] - mx);
      sum += v[u];
    }
  } else {
    for (int j = lane; j < t; j += 64) {
      const float e = mx == -INFINITY ? 0.f : expf(row[j] - mx);
      row[j] = e;
      sum += e;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (REG) {
#pragma unroll
    for (int u = 0; u < kS1SoftVals; ++u) {
      const int j = u * 64 + lane;
      if (j < t) row[j] = sum > 0.f ? v[u] / sum : 0.f;
    }
  } else {
    for (int j = lane; j < t; j += 64) row[j] = sum > 0.f ? row[j] / sum : 0.f;
  }
  if (lane == 0) lz[(size_t)head * N + r] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

// dA [h, N, d], dlz and D = dA . A [h, N], the row's loss term [h, N]; one row per 64 threads.
// A arrives as ksplit partial products (stride sk), summed here in order. The number of rows
// that see a slot, nk, is the group times the number of sampled positions at or after the
// head's earliest slot (every row when not causal), counted by each workgroup.
template <int D>
__global__ __launch_bounds__(256) void s1_out_grad_kernel(const float* __restrict__ Apart,
                                                          int ksplit, long long sk,
                                                          const float* __restrict__ Y,
                                                          const float* __restrict__ lz,
                                                          const float* __restrict__ lzt,
                                                          const float* __restrict__ sa,
                                                          const float* __restrict__ sz,
                                                          const int32_t* __restrict__ samples,
                                                          int S, int npos,
                                                          const int32_t* __restrict__ keypos,
                                                          int t, int causal,
                                                          float* __restrict__ dA,
                                                          float* __restrict__ dlz,
                                                          float* __restrict__ Dr,
                                                          float* __restrict__ lrow, int N,
                                                          int group) {
  __shared__ int red[256];
  const int head = blockIdx.y, tid = threadIdx.x;
  int first = 0;
  if (causal) {
    int mn = 0x7fffffff;
    for (int j = tid; j < t; j += 256) mn = min(mn, keypos[(size_t)head * t + j]);
    red[tid] = mn;
    __syncthreads();
    for (int h2 = 128; h2 > 0; h2 >>= 1) {
      if (tid < h2) red[tid] = min(red[tid], red[tid + h2]);
      __syncthreads();
    }
    first = red[0];
    __syncthreads();
  }
  int cnt = 0;
  for (int s2 = tid; s2 < S; s2 += 256) cnt += min(max(samples[s2], 0), npos - 1) >= first ? 1 : 0;
  red[tid] = cnt;
  __syncthreads();
  for (int h2 = 128; h2 > 0; h2 >>= 1) {
    if (tid < h2) red[tid] += red[tid + h2];
    __syncthreads();
  }
  const int nk = red[0] * group;
  const int r = blockIdx.x * 4 + (tid >> 6), lane = tid & 63;
  if (r >= N) return;
  const size_t o = (size_t)head * N + r;
  const int g = r % group;
  const float z = lz[o];
  const bool keep = z > -INFINITY && nk > 0;
  const float wa = 1.f / (sa[head * group + g] * sa[head * group + g]);
  const float wz = 1.f / (sz[head * group + g] * sz[head * group + g]);
  float da_dot = 0.f, sq = 0.f;
  for (int ch = lane; ch < D; ch += 64) {
    const size_t q = o * D + ch;
    float a = Apart[q];
    for (int s2 = 1; s2 < ksplit; ++s2) a += Apart[s2 * sk + q];
    const float e = a - Y[q];
    const float g2 = keep ? 2.f * wa * e / ((float)nk * D) : 0.f;
    dA[q] = g2;
    da_dot += g2 * a;
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

// db[h, j] = the tile column sums of dS, in tile order; the first workgroup of each head also
// sums the rows' loss terms in order into loss[h] (when loss is given)
__global__ __launch_bounds__(256) void s1_colsum_kernel(const float* __restrict__ part,
                                                        float* __restrict__ gb, int ntile, int t,
                                                        const float* __restrict__ lrow,
                                                        float* __restrict__ loss, int N) {
  __shared__ double red[256];
  const int head = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j < t) {
    float acc = 0.f;
    for (int k = 0; k < ntile; ++k) acc += part[((size_t)head * ntile + k) * t + j];
    gb[(size_t)head * t + j] = acc;
  }
  if (blockIdx.x != 0 || !loss) return;
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

// AdamW over the three parameter tensors in one launch: Ck and Cv [h, t, d], then b [h, t];
// slot j of head h trains where trainable[h, j] != 0 (or trainable is null)
struct S1Adam {
  float* th[3]; const float* g[3]; float* m[3]; float* v[3];
  long long nkv, nb;
  int d;
  const uint8_t* trainable;
  float lr, wd, bc1, bc2;
};
__global__ __launch_bounds__(256) void s1_adamw_kernel(const S1Adam a) {
  long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  int which;
  long long slot;
  if (e < a.nkv) {
    which = 0; slot = e / a.d;
  } else if (e < 2 * a.nkv) {
    which = 1; e -= a.nkv; slot = e / a.d;
  } else if (e < 2 * a.nkv + a.nb) {
    which = 2; e -= 2 * a.nkv; slot = e;
  } else {
    return;
  }
  if (a.trainable && !a.trainable[slot]) return;
  const float gg = a.g[which][e];
  const float mm = 0.9f * a.m[which][e] + 0.1f * gg;
  const float vv = 0.999f * a.v[which][e] + 0.001f * gg * gg;
  a.m[which][e] = mm;
  a.v[which][e] = vv;
  a.th[which][e] = a.th[which][e] * (1.f - a.lr * a.wd) -
                   a.lr * (mm / a.bc1) / (sqrtf(vv / a.bc2) + 1e-8f);
}

// teacher scales per (head, query head): population std of the outputs over positions and
// channels and of the log-normalizers over positions, floored at 1e-4. First pass: per
// (chunk of kS1ScaleRows rows of one query head, query head, head) the sums of x, x^2, z, z^2
// in double; second pass: the chunks in order.
constexpr int kS1ScaleRows = 256;

template <int D>
__global__ __launch_bounds__(256) void s1_scales_part_kernel(const float* __restrict__ O_full,
                                                             const float* __restrict__ lse_full,
                                                             double* __restrict__ part, int n,
                                                             int group, int nchunk) {
  __shared__ double red[4][256];
  const int chunk = blockIdx.x, g = blockIdx.y, head = blockIdx.z, tid = threadIdx.x;
  constexpr int V4 = D / 4, RPP = 256 / V4;   // float4 per row, rows per pass
  const int rows = (n - g + group - 1) / group;
  const int k0 = chunk * kS1ScaleRows, k1 = min(k0 + kS1ScaleRows, rows);
  double s1 = 0.0, s2 = 0.0, z1 = 0.0, z2 = 0.0;
  for (int k = k0 + tid / V4; k < k1; k += RPP) {
    const int i = g + k * group;
    const float4 x = reinterpret_cast<const float4*>(O_full + ((size_t)head * n + i) * D)[tid % V4];
    s1 += (double)x.x + (double)x.y + (double)x.z + (double)x.w;
    s2 += (double)x.x * x.x + (double)x.y * x.y + (double)x.z * x.z + (double)x.w * x.w;
  }
  for (int k = k0 + tid; k < k1; k += 256) {
    const double z = lse_full[(size_t)head * n + g + k * group];
    z1 += z;
    z2 += z * z;
  }
  red[0][tid] = s1; red[1][tid] = s2; red[2][tid] = z1; red[3][tid] = z2;
  __syncthreads();
  for (int h2 = 128; h2 > 0; h2 >>= 1) {
    if (tid < h2)
      for (int q = 0; q < 4; ++q) red[q][tid] += red[q][tid + h2];
    __syncthreads();
  }
  if (tid < 4) part[(((size_t)head * group + g) * nchunk + chunk) * 4 + tid] = red[tid][0];
}

__global__ __launch_bounds__(64) void s1_scales_kernel(const double* __restrict__ part,
                                                       float* __restrict__ sa,
                                                       float* __restrict__ sz, int n, int d,
                                                       int group, int nchunk) {
  const int g = blockIdx.x, head = blockIdx.y;
  if (threadIdx.x != 0) return;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const double* pp = part + ((size_t)head * group + g) * nchunk * 4;
  for (int c = 0; c < nchunk; ++c)
    for (int q = 0; q < 4; ++q) acc[q] += pp[c * 4 + q];
  const double rows = (double)((n - g + group - 1) / group);
  const double cnt = rows * d;
  const double va = fmax(acc[1] / cnt - (acc[0] / cnt) * (acc[0] / cnt), 0.0);
  const double vz = fmax(acc[3] / rows - (acc[2] / rows) * (acc[2] / rows), 0.0);
  sa[head * group + g] = (float)fmax(sqrt(va), 1e-4);
  sz[head * group + g] = (float)fmax(sqrt(vz), 1e-4);
}

namespace {
struct Carve4 {
  char* base; size_t off;
  template <typename X> X* take(size_t count) {
    X* q = base ? (X*)(base + off) : nullptr;   // sizing only: no address
    off = align_up(off + count * sizeof(X));
    return q;
  }
};
struct S1Plan {
  float *Qs, *Y, *lzt, *P, *dS, *A, *lz, *dA, *dlz, *Dr, *lrow, *sa, *sz, *colpart;
  double* spart;
  int* qpos;
  float *gCk, *gCv, *gb, *mCk, *vCk, *mCv, *vCv, *mb, *vb;
  size_t bytes;
};
int s1_nchunk(int64_t n, int64_t group) {
  const int64_t rows = (n + group - 1) / group;
  return (int)((rows + kS1ScaleRows - 1) / kS1ScaleRows);
}
int64_t s1_ntile(int64_t N) { return (N + kGT - 1) / kGT; }
// k split of A = P Cv (k = t slots): enough workgroups for the chip, at least two 32-deep
// tiles per part
constexpr int kS1MaxKSplit = 8;
int s1_ksplit(int64_t h, int64_t N, int64_t t, int64_t d) {
  const int64_t base = s1_ntile(N) * ((d + kGT - 1) / kGT) * h;
  int64_t ks = (512 + base - 1) / base;
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, (t + 2 * kGK - 1) / (2 * kGK)));
  return (int)std::max<int64_t>(1, std::min<int64_t>(ks, kS1MaxKSplit));
}
S1Plan plan_s1(char* base, int64_t h, int64_t n, int64_t t, int64_t d, int64_t N,
               int64_t group) {
  Carve4 c{base, 0};
  S1Plan q;
  q.spart = c.take<double>((size_t)h * group * s1_nchunk(n, group) * 4);
  q.Qs = c.take<float>((size_t)h * N * d);
  q.Y = c.take<float>((size_t)h * N * d);
  q.lzt = c.take<float>(h * N);
  q.qpos = c.take<int>(h * N);
  q.P = c.take<float>((size_t)h * N * t);
  q.dS = c.take<float>((size_t)h * N * t);
  q.colpart = c.take<float>((size_t)h * s1_ntile(N) * t);
  q.A = c.take<float>((size_t)s1_ksplit(h, N, t, d) * h * N * d);
  q.lz = c.take<float>(h * N);
  q.dA = c.take<float>((size_t)h * N * d);
  q.dlz = c.take<float>(h * N);
  q.Dr = c.take<float>(h * N);
  q.lrow = c.take<float>(h * N);
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

S1Gemm gemm_args(const float* A, long long sAz, int lda, const float* B, long long sBz,
                 int ldb, float* C, long long sCz, int ldc, int M, int N, int K, float alpha) {
  S1Gemm g;
  memset(&g, 0, sizeof g);
  g.A = A; g.sAz = sAz; g.lda = lda;
  g.B = B; g.sBz = sBz; g.ldb = ldb;
  g.C = C; g.sCz = sCz; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.alpha = alpha;
  g.zsplit = 1 << 30;
  g.ksplit = 1;
  return g;
}
dim3 gemm_grid(const S1Gemm& g, int heads) {
  return dim3(cdiv4(g.N, kGT), cdiv4(g.M, kGT), heads);
}

// forward + loss + gradients of one update (rows from `samples`)
template <int D>
hipError_t s1_eval(const Stage1Args& a, const S1Plan& pl, const int32_t* samples, float* loss,
                   float* gCk, float* gCv, float* gb) {
  const hipStream_t st = a.stream;
  const int H = a.heads, N = a.S * a.group, t = a.t;
  const long long Nd = (long long)N * D, Nt = (long long)N * t, td = (long long)t * D;
  const dim3 gg(cdiv4(Nd, 256), H);
  if (a.bf16)
    hipLaunchKernelGGL(s1_gather_kernel<bf16>, gg, dim3(256), 0, st, (const bf16*)a.Q, a.O_full,
                       a.lse_full, samples, pl.Qs, pl.Y, pl.lzt, pl.qpos, a.n, D, N, a.group);
  else
    hipLaunchKernelGGL(s1_gather_kernel<float>, gg, dim3(256), 0, st, (const float*)a.Q,
                       a.O_full, a.lse_full, samples, pl.Qs, pl.Y, pl.lzt, pl.qpos, a.n, D, N,
                       a.group);
  // scores l = scale Qs Ck^T + b (masked) into P
  S1Gemm g = gemm_args(pl.Qs, Nd, D, a.Ck, td, D, pl.P, Nt, t, N, t, D, a.scale);
  g.bias = a.b; g.keypos = a.keypos; g.sbz = t; g.qpos = pl.qpos; g.sqz = N;
  g.causal = a.causal ? 1 : 0;
  hipLaunchKernelGGL((s1_gemm_kernel<true, true, kEpiScore>), gemm_grid(g, H), dim3(256), 0, st, g);
  if (t <= 64 * kS1SoftVals)
    hipLaunchKernelGGL(s1_softmax_kernel<true>, dim3(cdiv4(N, 4), H), dim3(256), 0, st, pl.P,
                       pl.lz, N, t);
  else
    hipLaunchKernelGGL(s1_softmax_kernel<false>, dim3(cdiv4(N, 4), H), dim3(256), 0, st, pl.P,
                       pl.lz, N, t);
  // A = P Cv, split over k into ks partial products
  const int ks = s1_ksplit(H, N, t, D);
  g = gemm_args(pl.P, Nt, t, a.Cv, td, D, pl.A, Nd, D, N, D, t, 1.f);
  g.ksplit = ks; g.sCk = (long long)H * Nd;
  hipLaunchKernelGGL((s1_gemm_kernel<true, false, kEpiStore>), gemm_grid(g, H * ks), dim3(256), 0,
                     st, g);
  hipLaunchKernelGGL(s1_out_grad_kernel<D>, dim3(cdiv4(N, 4), H), dim3(256), 0, st,
                     (const float*)pl.A, ks, (long long)H * Nd, (const float*)pl.Y, (const float*)pl.lz,
                     (const float*)pl.lzt, (const float*)pl.sa, (const float*)pl.sz, samples, a.S,
                     a.n / a.group, a.keypos, t, a.causal ? 1 : 0, pl.dA, pl.dlz, pl.Dr, pl.lrow,
                     N, a.group);
  // dS = P (dA Cv^T - D + dlz), with the tile column sums for db
  g = gemm_args(pl.dA, Nd, D, a.Cv, td, D, pl.dS, Nt, t, N, t, D, 1.f);
  g.P = pl.P; g.Dr = pl.Dr; g.dlz = pl.dlz; g.sqz = N; g.colpart = pl.colpart;
  hipLaunchKernelGGL((s1_gemm_kernel<true, true, kEpiDS>), gemm_grid(g, H), dim3(256), 0, st, g);
  // dCv = P^T dA (z < H) and dCk = scale dS^T Qs (z >= H) in one launch
  g = gemm_args(pl.P, Nt, t, pl.dA, Nd, D, gCv, td, D, t, D, N, 1.f);
  g.zsplit = H; g.A2 = pl.dS; g.B2 = pl.Qs; g.C2 = gCk; g.alpha2 = a.scale;
  hipLaunchKernelGGL((s1_gemm_kernel<false, false, kEpiStore>), gemm_grid(g, 2 * H), dim3(256), 0,
                     st, g);
  hipLaunchKernelGGL(s1_colsum_kernel, dim3(cdiv4(t, 256), H), dim3(256), 0, st,
                     (const float*)pl.colpart, gb, (int)s1_ntile(N), t, (const float*)pl.lrow,
                     loss, N);
  return hipGetLastError();
}

template <int D>
hipError_t s1_run(const Stage1Args& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, t = a.t;
  S1Plan pl = plan_s1((char*)a.ws, H, a.n, t, D, (int64_t)a.S * a.group, a.group);
  const int nchunk = s1_nchunk(a.n, a.group);
  hipLaunchKernelGGL(s1_scales_part_kernel<D>, dim3(nchunk, a.group, H), dim3(256), 0, st,
                     a.O_full, a.lse_full, pl.spart, a.n, a.group, nchunk);
  hipLaunchKernelGGL(s1_scales_kernel, dim3(a.group, H), dim3(64), 0, st, (const double*)pl.spart,
                     pl.sa, pl.sz, a.n, D, a.group, nchunk);
  if (a.steps == 0)   // one evaluation: gradients to the caller
    return s1_eval<D>(a, pl, a.samples, a.loss, a.gCk, a.gCv, a.gb);
  const long long nkv = (long long)H * t * D, nb = (long long)H * t;
  // Adam moments start at zero; mCk, vCk, mCv, vCv, mb, vb are contiguous in the plan
  hipError_t e = launch_fill_f32(pl.mCk, (long long)((char*)(pl.vb + nb) - (char*)pl.mCk) / 4, 0.f, st);
  if (e != hipSuccess) return e;
  S1Adam ad;
  ad.th[0] = a.Ck; ad.th[1] = a.Cv; ad.th[2] = a.b;
  ad.g[0] = pl.gCk; ad.g[1] = pl.gCv; ad.g[2] = pl.gb;
  ad.m[0] = pl.mCk; ad.m[1] = pl.mCv; ad.m[2] = pl.mb;
  ad.v[0] = pl.vCk; ad.v[1] = pl.vCv; ad.v[2] = pl.vb;
  ad.nkv = nkv; ad.nb = nb; ad.d = D; ad.trainable = a.trainable; ad.lr = a.lr; ad.wd = a.wd;
  for (int k = 1; k <= a.steps; ++k) {
    e = s1_eval<D>(a, pl, a.samples + (size_t)(k - 1) * a.S,
                   a.loss ? a.loss + (size_t)(k - 1) * H : nullptr, pl.gCk, pl.gCv, pl.gb);
    if (e != hipSuccess) return e;
    ad.bc1 = (float)(1.0 - pow(0.9, k));
    ad.bc2 = (float)(1.0 - pow(0.999, k));
    hipLaunchKernelGGL(s1_adamw_kernel, dim3(cdiv4(2 * nkv + nb, 256)), dim3(256), 0, st, ad);
  }
  return hipGetLastError();
}
}  // namespace

size_t stage1_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d, int64_t S,
                       int64_t group) {
  return plan_s1(nullptr, heads, n, t, d, S * group, group).bytes;
}

hipError_t launch_stage1(const Stage1Args& a) {
  return a.d == 128 ? s1_run<128>(a) : s1_run<64>(a);
}

}  // namespace amc
