// Top-t key selection and row gather on gfx950.
//
// Selection follows the "Compaction" blog, §Fast KV Compaction via Attention Matching,
// step 1 (the keys with the highest attention; C_k is a subset of K). Compacted entries
// keep their original positions (Latent Compaction with Test-Time Training, §3.1
// "Handling Subsequent Tokens"), so indices are emitted in ascending order and ties at
// the threshold go to the lower index.
//
// One workgroup per head. Scores map to order-preserving uint32 keys; a 4-pass, 8-bit
// radix select (LDS histograms with integer atomics) finds the t-th largest key theta
// and how many keys equal to theta are still needed. A stable compaction in index order
// then writes every key above theta and the lowest-index keys equal to theta, already
// sorted: each thread owns a contiguous segment of keys, counts its keys above and equal
// to theta, and two block-wide scans give it the rank of its first equal key and of its
// first output. No sort of the t survivors is needed. The gather copies the selected K
// (and V) rows bit for bit.
#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
// Scores a thread has in flight at once: 8 where every thread has at least 16 keys (latency,
// not bandwidth, bounds the passes), else 1 (with a few keys per thread the guarded batch
// costs more than it hides: 26 against 16 us for 512 heads of 2048 keys)
constexpr int kSelBatchMinKeys = 16 * kSelThreads;

__device__ __forceinline__ unsigned order_key(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive sum of one count per thread (thread order) and the block total.
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* total, unsigned* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  unsigned x = v;   // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const unsigned s = wsum[i];
    before += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

template <int kSelB>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const float* __restrict__ score,
                                                                  int32_t* __restrict__ idx,
                                                                  int Tk, int t) {
  __shared__ unsigned hist[256];
  __shared__ unsigned wsum[kSelWaves];
  __shared__ unsigned sh_prefix, sh_remaining;
  const int tid = threadIdx.x;
  const float* sc = score + (size_t)blockIdx.x * Tk;
  int32_t* out = idx + (size_t)blockIdx.x * t;

  unsigned prefix = 0, mask = 0, remaining = (unsigned)t;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j0 = tid; j0 < Tk; j0 += kSelThreads * kSelB) {
      float f[kSelB];
#pragma unroll
      for (int b = 0; b < kSelB; ++b) {
        const int j = j0 + b * kSelThreads;
        f[b] = j < Tk ? sc[j] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < kSelB; ++b) {
        const unsigned u = order_key(f[b]);
        if (j0 + b * kSelThreads < Tk && (u & mask) == prefix)
          atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    // the digit: the largest dg whose count from the top, sum_{k >= dg} hist[k], reaches
    // `remaining` (thread i takes digit 255 - i, so a scan in thread order sums from the top)
    {
      const int dg = 255 - tid;
      const unsigned hc = tid < 256 ? hist[dg] : 0u;
      unsigned total;
      const unsigned above = block_excl_scan(hc, &total, wsum);   // sum over digits > dg
      if (tid < 256 && above < remaining && above + hc >= remaining) {
        sh_prefix = prefix | ((unsigned)dg << shift);
        sh_remaining = remaining - above;
      }
      if (tid == 0 && total < remaining) {   // cannot happen for t <= Tk; keep a defined state
        sh_prefix = prefix;
        sh_remaining = remaining - total;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix = theta, the t-th largest key; the `remaining` lowest-index keys equal to theta
  // are taken. Thread segments in thread order are index order.
  const int seg = (Tk + kSelThreads - 1) / kSelThreads;
  const int j0 = min(Tk, tid * seg), j1 = min(Tk, j0 + seg);
  unsigned n_eq = 0, n_gt = 0;
  for (int jb = j0; jb < j1; jb += kSelB) {
    float f[kSelB];
#pragma unroll
    for (int b = 0; b < kSelB; ++b) f[b] = jb + b < j1 ? sc[jb + b] : 0.f;
#pragma unroll
    for (int b = 0; b < kSelB; ++b) {
      const unsigned u = order_key(f[b]);
      n_eq += jb + b < j1 && u == prefix;
      n_gt += jb + b < j1 && u > prefix;
    }
  }
  unsigned eq_total, take_total;
  const unsigned eq_before = block_excl_scan(n_eq, &eq_total, wsum);
  const unsigned eq_take = eq_before >= remaining ? 0u : min(n_eq, remaining - eq_before);
  unsigned pos = block_excl_scan(n_gt + eq_take, &take_total, wsum);
  unsigned eq_seen = 0;
  for (int jb = j0; jb < j1; jb += kSelB) {
    float f[kSelB];
#pragma unroll
    for (int b = 0; b < kSelB; ++b) f[b] = jb + b < j1 ? sc[jb + b] : 0.f;
#pragma unroll
    for (int b = 0; b < kSelB; ++b) {
      if (jb + b >= j1) break;
      const unsigned u = order_key(f[b]);
      bool take = u > prefix;
      if (u == prefix) take = eq_seen++ < eq_take;
      if (take) {
        if (pos < (unsigned)t) out[pos] = jb + b;
        ++pos;
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ K,
                                                          const T* __restrict__ V,
                                                          const int32_t* __restrict__ idx,
                                                          T* __restrict__ Ck, T* __restrict__ Vs,
                                                          int Tk, int t) {
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int CPR = D / E;
  const int head = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= t * CPR) return;
  const int i = c / CPR, col = (c % CPR) * E;
  const int src = min(max(idx[(size_t)head * t + i], 0), Tk - 1);
  const size_t so = ((size_t)head * Tk + src) * D + col;
  const size_t dst = ((size_t)head * t + i) * D + col;
  *(uint4*)(Ck + dst) = *(const uint4*)(K + so);
  if (Vs) *(uint4*)(Vs + dst) = *(const uint4*)(V + so);
}

template <typename T, int D>
static void launch_gather(const SelectArgs& a) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const dim3 g((a.t * CPR + 255) / 256, a.heads);
  hipLaunchKernelGGL((gather_rows_kernel<T, D>), g, dim3(256), 0, a.stream, (const T*)a.K,
                     (const T*)a.V, a.idx, (T*)a.Ck, (T*)a.Vsel, a.T, a.t);
}

hipError_t launch_select(const SelectArgs& a) {
  if (a.T >= kSelBatchMinKeys)
    hipLaunchKernelGGL(topk_select_kernel<8>, dim3(a.heads), dim3(kSelThreads), 0, a.stream, a.score,
                       a.idx, a.T, a.t);
  else
    hipLaunchKernelGGL(topk_select_kernel<1>, dim3(a.heads), dim3(kSelThreads), 0, a.stream, a.score,
                       a.idx, a.T, a.t);
  if (a.bf16) {
    if (a.d == 128) launch_gather<bf16, 128>(a); else launch_gather<bf16, 64>(a);
  } else {
    if (a.d == 128) launch_gather<float, 128>(a); else launch_gather<float, 64>(a);
  }
  return hipGetLastError();
}

}  // namespace amc
