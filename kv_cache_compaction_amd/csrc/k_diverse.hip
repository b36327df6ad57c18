// Anchor + diversifier initialization ("Latent Compaction with Test-Time Training", §3.2
// Initialization, Budget Allocation, Eq. 6-7): anchors are the first entry and the entries
// of highest maximum attention; diversifiers are added by farthest-first traversal, each
// step taking the key farthest (squared Euclidean distance) from every key chosen so far.
//
// The traversal runs on P workgroups per head, all resident at once (an ordinary launch
// that is refused unless the whole grid fits on the device at the same time): each owns
// a contiguous range of keys and keeps their distances to the chosen set in LDS. A step
// streams the range once (a group of lanes per key row, 16 bytes per lane, so a wave reads
// contiguous rows), lowers the distances by the new key's, and finds the range's best
// candidate; the P candidates meet through a per-head barrier and every workgroup reduces
// them in the same way, so all agree on the next key without another round trip. For bf16
// keys whose ranges fit, fft_reg_kernel keeps each range in registers instead, so a step
// reads only the chosen key.
#include <climits>

#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

constexpr int kFftSpin = 1 << 22;   // polls before a barrier wait gives up (seconds)

// Device-scope loads and stores (the device's coherence point, not a CU's or an XCD's
// cache copy): the only data the workgroups of a head exchange, their candidate slots,
// goes through these.
__device__ __forceinline__ int ld_dev_i(const int* q) {
  return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_i(int* q, int v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier among the workgroups of one head (the m-th completes when the counter reaches
// m * P): every wave waits until its stores have completed (vmcnt 0), the workgroup's
// barrier orders its threads' writes before thread 0's counter add, which has release
// semantics at device scope; thread 0 polls the counter and ends its wait with an acquire
// fence at device scope, and the closing barrier orders the other threads' reads after it
// (the language memory model's release/acquire pattern). The candidate slots are still
// written and read with device-scope accesses. A wait longer than kFftSpin polls marks the
// workgroup as timed out; it then stops.
__device__ __forceinline__ void fft_barrier(int* ctr, int target, int* timed_out) {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0) only
  __syncthreads();
  if (threadIdx.x == 0 && !*timed_out) {
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kFftSpin) {
        *timed_out = 1;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// (value, index) order of the traversal: larger distance first, lower index on ties
__device__ __forceinline__ bool fft_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// score with the first entry forced to the top: the first entry is always an anchor
__global__ __launch_bounds__(256) void force_first_kernel(const float* __restrict__ score,
                                                          float* __restrict__ out, int T) {
  const int head = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= T) return;
  const size_t o = (size_t)head * T + j;
  out[o] = j == 0 ? INFINITY : score[o];
}

struct FftParams {
  const void* K; const int32_t* anchors; int32_t* order; int2* part; int* bar;
  int32_t* status;
  int heads, T, M, na, P, chunk;
};

template <typename Tt, int D>
__global__ __launch_bounds__(256) void fft_kernel(const FftParams p) {
  extern __shared__ float dsh[];          // distances of this workgroup's keys
  __shared__ float kn[D];                 // the key chosen last
  __shared__ float rv[4];
  __shared__ int ri[4], jsh, tout;
  constexpr int EPL = 16 / (int)sizeof(Tt);   // elements per lane
  constexpr int LPK = D / EPL;                // lanes per key row
  constexpr int KPI = 64 / LPK;               // keys per wave per pass
  const int head = blockIdx.x % p.heads, part = blockIdx.x / p.heads;
  const int b0 = part * p.chunk, b1 = min(p.T, b0 + p.chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPK, sl = lane % LPK;
  const Tt* Kh = (const Tt*)p.K + (size_t)head * p.T * D;
  for (int i = tid; i < b1 - b0; i += 256) dsh[i] = INFINITY;
  if (tid == 0) tout = 0;
  __syncthreads();
  int j = 0, nbar = 0;
  for (int step = 0; step < p.M; ++step) {
    if (step < p.na) j = p.anchors[(size_t)head * p.na + step];
    if (part == 0 && tid == 0) p.order[(size_t)head * p.M + step] = j;
    if (tid < D) kn[tid] = (float)Kh[(size_t)j * D + tid];
    __syncthreads();
    float kv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) kv[e] = kn[sl * EPL + e];
    for (int base = b0 + wave * KPI; base < b1; base += 4 * KPI) {
      const int i = base + sub;
      float acc = 0.f;
      if (i < b1) {
        const uint4 raw = *(const uint4*)(Kh + (size_t)i * D + sl * EPL);
        const Tt* x = (const Tt*)&raw;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float df = (float)x[e] - kv[e];
          acc = __builtin_fmaf(df, df, acc);
        }
      }
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (sl == 0 && i < b1) {
        const float cur = dsh[i - b0];
        dsh[i - b0] = i == j ? -1.f : fminf(cur, acc);   // chosen keys stay at -1
      }
    }
    __syncthreads();
    if (step + 1 >= p.M) break;
    if (step + 1 < p.na) continue;   // the next key is an anchor: nothing to search
    // this range's best candidate
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int i = tid; i < b1 - b0; i += 256) {
      const float v = dsh[i];
      if (fft_better(v, b0 + i, bv, bi)) {
        bv = v;
        bi = b0 + i;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (fft_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (lane == 0) {
      rv[wave] = bv;
      ri[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < 4; ++w)
        if (fft_better(rv[w], ri[w], bv, bi)) {
          bv = rv[w];
          bi = ri[w];
        }
      jsh = bi;
    }
    __syncthreads();
    if (p.P == 1) {
      j = jsh;
      continue;
    }
    // the head's P candidates: publish, meet, and reduce them identically everywhere
    int2* slot = p.part + ((size_t)head * 2 + (step & 1)) * p.P;
    if (tid == 0) {   // thread 0 holds the best
      st_dev_i(&slot[part].x, __float_as_int(bv));
      st_dev_i(&slot[part].y, jsh);
    }
    fft_barrier(&p.bar[head], ++nbar * p.P, &tout);
    if (tout) break;
    bv = -INFINITY;
    bi = INT_MAX;
    for (int q = tid; q < p.P; q += 256) {
      const float v = __int_as_float(ld_dev_i(&slot[q].x));
      const int ix = ld_dev_i(&slot[q].y);
      if (fft_better(v, ix, bv, bi)) {
        bv = v;
        bi = ix;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (fft_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    __syncthreads();
    if (lane == 0) {
      rv[wave] = bv;
      ri[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < 4; ++w)
        if (fft_better(rv[w], ri[w], bv, bi)) {
          bv = rv[w];
          bi = ri[w];
        }
      jsh = min(max(bi, 0), p.T - 1);
    }
    __syncthreads();
    j = jsh;
  }
  if (tout && tid == 0 && p.status) atomicOr(&p.status[head], AM_HEAD_TIMEOUT_BIT);
}

// The same traversal with the keys of each workgroup held in registers (bf16 inputs, a
// workgroup of 512 threads keeping kFftRegKeys(D) rows per thread): a step reads only the
// chosen key, so its cost is the distance arithmetic and the per-head barrier.
template <int D> constexpr int fft_reg_keys() { return D == 128 ? 2 : 4; }
typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;
constexpr int kFftRegThreads = 512;

template <int D>
__global__ __launch_bounds__(kFftRegThreads) void fft_reg_kernel(const FftParams p) {
  constexpr int RK = fft_reg_keys<D>();   // key rows per thread
  constexpr int W = D / 2;                // bf16 pairs per row
  constexpr int NW = kFftRegThreads / 64;
  __shared__ float rv[NW];
  __shared__ int ri[NW], jsh, tout;
  const int head = blockIdx.x % p.heads, part = blockIdx.x / p.heads;
  const int b0 = part * p.chunk, b1 = min(p.T, b0 + p.chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16* Kh = (const bf16*)p.K + (size_t)head * p.T * D;
  uint32_t kx[RK][W];
  float dist[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int i = b0 + tid + kFftRegThreads * k;
    const uint4* src = (const uint4*)(Kh + (size_t)min(i, p.T - 1) * D);
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const uint4 v = src[q];
      kx[k][4 * q + 0] = v.x;
      kx[k][4 * q + 1] = v.y;
      kx[k][4 * q + 2] = v.z;
      kx[k][4 * q + 3] = v.w;
    }
    dist[k] = i < b1 ? INFINITY : -INFINITY;   // rows past the range never win
  }
  if (tid == 0) tout = 0;
  __syncthreads();
  int j = 0, nbar = 0;
  for (int step = 0; step < p.M; ++step) {
    if (step < p.na) j = p.anchors[(size_t)head * p.na + step];
    if (part == 0 && tid == 0) p.order[(size_t)head * p.M + step] = j;
    j = __builtin_amdgcn_readfirstlane(j);
    // the new key's row through the scalar cache (a uniform read-only address), so its
    // values reach the vector instructions as scalar operands
    const cu32_ptr crow = (cu32_ptr)(uintptr_t)(Kh + (size_t)j * D);
    // the rows' bf16 words are re-expanded every step: an empty asm marks them as rewritten,
    // so the compiler keeps them packed instead of hoisting RK * D floats out of the loop
#pragma unroll
    for (int k = 0; k < RK; ++k)
#pragma unroll
      for (int q = 0; q < W; ++q) asm volatile("" : "+v"(kx[k][q]));
    // squared distances to the new key, four partial sums per row
    float acc[RK][4];
#pragma unroll
    for (int k = 0; k < RK; ++k)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[k][u] = 0.f;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) {
      const uint32_t c0 = crow[2 * q], c1 = crow[2 * q + 1];
      const float cx = __uint_as_float(c0 << 16), cy = __uint_as_float(c0 & 0xffff0000u);
      const float cz = __uint_as_float(c1 << 16), cw = __uint_as_float(c1 & 0xffff0000u);
#pragma unroll
      for (int k = 0; k < RK; ++k) {
        const uint32_t w0 = kx[k][2 * q], w1 = kx[k][2 * q + 1];
        const float d0 = __uint_as_float(w0 << 16) - cx;
        const float d1 = __uint_as_float(w0 & 0xffff0000u) - cy;
        const float d2 = __uint_as_float(w1 << 16) - cz;
        const float d3 = __uint_as_float(w1 & 0xffff0000u) - cw;
        acc[k][0] = __builtin_fmaf(d0, d0, acc[k][0]);
        acc[k][1] = __builtin_fmaf(d1, d1, acc[k][1]);
        acc[k][2] = __builtin_fmaf(d2, d2, acc[k][2]);
        acc[k][3] = __builtin_fmaf(d3, d3, acc[k][3]);
      }
    }
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const int i = b0 + tid + kFftRegThreads * k;
      const float dd = (acc[k][0] + acc[k][1]) + (acc[k][2] + acc[k][3]);
      if (i < b1) dist[k] = i == j ? -1.f : fminf(dist[k], dd);   // chosen keys stay at -1
    }
    if (step + 1 >= p.M) break;
    if (step + 1 < p.na) continue;   // the next key is an anchor: nothing to search
    // this workgroup's best candidate
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const int i = b0 + tid + kFftRegThreads * k;
      if (fft_better(dist[k], i, bv, bi)) {
        bv = dist[k];
        bi = i;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (fft_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (lane == 0) {
      rv[wave] = bv;
      ri[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w)
        if (fft_better(rv[w], ri[w], bv, bi)) {
          bv = rv[w];
          bi = ri[w];
        }
      jsh = min(max(bi, 0), p.T - 1);
    }
    __syncthreads();
    if (p.P == 1) {
      j = jsh;
      continue;
    }
    // the head's P candidates: publish, meet, and reduce them identically everywhere
    int2* slot = p.part + ((size_t)head * 2 + (step & 1)) * p.P;
    if (tid == 0) {   // thread 0 holds the best
      st_dev_i(&slot[part].x, __float_as_int(bv));
      st_dev_i(&slot[part].y, jsh);
    }
    fft_barrier(&p.bar[head], ++nbar * p.P, &tout);
    if (tout) break;
    bv = -INFINITY;
    bi = INT_MAX;
    for (int q = tid; q < p.P; q += kFftRegThreads) {
      const float v = __int_as_float(ld_dev_i(&slot[q].x));
      const int ix = ld_dev_i(&slot[q].y);
      if (fft_better(v, ix, bv, bi)) {
        bv = v;
        bi = ix;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (fft_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    __syncthreads();
    if (lane == 0) {
      rv[wave] = bv;
      ri[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w)
        if (fft_better(rv[w], ri[w], bv, bi)) {
          bv = rv[w];
          bi = ri[w];
        }
      jsh = min(max(bi, 0), p.T - 1);
    }
    __syncthreads();
    j = jsh;
  }
  if (tout && tid == 0 && p.status) atomicOr(&p.status[head], AM_HEAD_TIMEOUT_BIT);
}

// idx = the M chosen keys in ascending order (bitonic sort in LDS, M <= 8192)
__global__ __launch_bounds__(1024) void sort_order_kernel(const int32_t* __restrict__ order,
                                                          int32_t* __restrict__ idx, int M) {
  __shared__ int a[8192];
  const int head = blockIdx.x, tid = threadIdx.x;
  int n2 = 1;
  while (n2 < M) n2 <<= 1;
  for (int i = tid; i < n2; i += 1024) a[i] = i < M ? order[(size_t)head * M + i] : INT_MAX;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        const int l = i ^ jj;
        if (l > i) {
          const bool up = (i & k) == 0;
          const int x = a[i], y = a[l];
          if ((x > y) == up) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < M; i += 1024) idx[(size_t)head * M + i] = a[i];
}

namespace {
struct Carve3 {
  char* base; size_t off;
  template <typename X> X* take(size_t count) {
    X* q = base ? (X*)(base + off) : nullptr;   // sizing only: no address
    off = align_up(off + count * sizeof(X));
    return q;
  }
};
struct InitPlan {
  float* lse; float* score; float* forced; void* tws; int32_t* anchors; void* Ca; int32_t* order;
  int2* part; int* bar; int32_t* status;
  size_t bytes;
};
InitPlan plan_init(char* base, int64_t h, int64_t n, int64_t T, int64_t d, int es, int64_t M,
                   int64_t na, int P) {
  Carve3 c{base, 0};
  InitPlan q;
  q.lse = c.take<float>(h * n);
  q.score = c.take<float>(h * T);
  q.forced = c.take<float>(h * T);
  q.tws = c.take<char>(targets_ws_bytes(h, n, T, d, es));
  q.anchors = c.take<int32_t>(h * na);
  q.Ca = c.take<char>((size_t)h * na * d * es);
  q.order = c.take<int32_t>(h * M);
  q.part = c.take<int2>(h * 2 * (size_t)P);
  q.bar = c.take<int>(h);
  q.status = c.take<int32_t>(h);
  q.bytes = c.off;
  return q;
}
int fft_parts(int heads, int T) {
  int P = device_cu_count() / heads;
  P = min(P, (T + 255) / 256);   // at least 256 keys per workgroup
  return max(1, min(P, 256));
}
unsigned cdiv3(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

template <typename Tt, int D>
hipError_t launch_fft(FftParams fp, size_t shmem, hipStream_t st) {
  const dim3 g(fp.heads * fp.P), b(256);
  if (fp.P == 1) {
    hipLaunchKernelGGL((fft_kernel<Tt, D>), g, b, shmem, st, fp);
    return hipGetLastError();
  }
  (void)hipFuncSetAttribute((const void*)fft_kernel<Tt, D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  void* args[] = {&fp};
  return launch_all_resident((const void*)fft_kernel<Tt, D>, g, b, args, shmem, st);
}
template <int D>
hipError_t launch_fft_reg(FftParams fp, hipStream_t st) {
  const dim3 g(fp.heads * fp.P), b(kFftRegThreads);
  if (fp.P == 1) {
    hipLaunchKernelGGL((fft_reg_kernel<D>), g, b, 0, st, fp);
    return hipGetLastError();
  }
  void* args[] = {&fp};
  return launch_all_resident((const void*)fft_reg_kernel<D>, g, b, args, 0, st);
}
}  // namespace

size_t init_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize, int64_t M,
                     int64_t na) {
  return plan_init(nullptr, heads, n, T, d, esize, M, na, 256).bytes;
}

int init_max_chunk(int heads, int T) {
  const int P = fft_parts(heads, T);
  return (T + P - 1) / P;
}

hipError_t launch_init_anchor_diverse(const InitArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, es = a.bf16 ? 2 : 4;
  const int P = fft_parts(H, a.T);
  InitPlan pl = plan_init((char*)a.ws, H, a.n, a.T, a.d, es, a.M, a.na, 256);
  int32_t* status = a.head_status ? a.head_status : pl.status;
  hipError_t e = launch_zero_status(status, H, st);
  if (e != hipSuccess) return e;
  // Eq. 6: maximum attention of every entry over the reference queries
  TargetsArgs ta;
  ta.Q = a.Q; ta.K = a.K; ta.V = nullptr; ta.Vt = pl.tws;
  ta.rowstat = (char*)pl.tws + targets_vt_bytes(H, a.T, a.d, es);
  ta.colpart = (float*)((char*)ta.rowstat + align_up((size_t)H * a.n * 8));
  ta.lse = pl.lse; ta.O = nullptr; ta.score = pl.score; ta.mode = 2;
  ta.heads = H; ta.n = a.n; ta.T = a.T; ta.d = a.d; ta.group = a.group; ta.causal = a.causal;
  ta.bf16 = a.bf16; ta.scale = a.scale; ta.stream = st;
  if ((e = launch_targets(ta)) != hipSuccess) return e;
  // anchors: the first entry and the best of the rest, ascending
  hipLaunchKernelGGL(force_first_kernel, dim3(cdiv3(a.T, 256), H), dim3(256), 0, st,
                     (const float*)pl.score, pl.forced, a.T);
  SelectArgs sa;
  sa.score = pl.forced; sa.K = a.K; sa.V = nullptr; sa.idx = pl.anchors; sa.Ck = pl.Ca;
  sa.Vsel = nullptr; sa.heads = H; sa.T = a.T; sa.t = a.na; sa.d = a.d; sa.bf16 = a.bf16;
  sa.stream = st;
  if ((e = launch_select(sa)) != hipSuccess) return e;
  // Eq. 7: farthest-first traversal from the anchors
  if ((e = launch_zero_status(pl.bar, H, st)) != hipSuccess) return e;
  FftParams fp;
  fp.K = a.K; fp.anchors = pl.anchors; fp.order = a.order ? a.order : pl.order; fp.part = pl.part;
  fp.bar = pl.bar; fp.status = status;
  fp.heads = H; fp.T = a.T; fp.M = a.M; fp.na = a.na; fp.P = P; fp.chunk = (a.T + P - 1) / P;
  const size_t shmem = (size_t)fp.chunk * sizeof(float);
  if (a.bf16 && fp.chunk <= kFftRegThreads * (a.d == 128 ? fft_reg_keys<128>() : fft_reg_keys<64>()))
    e = a.d == 128 ? launch_fft_reg<128>(fp, st) : launch_fft_reg<64>(fp, st);
  else if (a.bf16)
    e = a.d == 128 ? launch_fft<bf16, 128>(fp, shmem, st) : launch_fft<bf16, 64>(fp, shmem, st);
  else
    e = a.d == 128 ? launch_fft<float, 128>(fp, shmem, st) : launch_fft<float, 64>(fp, shmem, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sort_order_kernel, dim3(H), dim3(1024), 0, st, (const int32_t*)fp.order,
                     a.idx, a.M);
  return hipGetLastError();
}

}  // namespace amc
