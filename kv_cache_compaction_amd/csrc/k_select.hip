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
// (wave ballots plus a 16-entry LDS scan per 1024 keys) then writes every key above
// theta and the lowest-index keys equal to theta, already sorted. No sort of the t
// survivors is needed. The gather copies the selected K (and V) rows bit for bit.
#include "am_common.hpp"
#include "am_internal.hpp"

namespace amc {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ unsigned order_key(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive count of set flags before this thread (thread order) and the block total.
__device__ __forceinline__ unsigned block_excl_count(bool f, unsigned* total, unsigned* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned long long bal = __ballot(f);
  const unsigned in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(bal);
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const unsigned v = wsum[i];
    before += (i < w) ? v : 0u;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

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
    for (int j = tid; j < Tk; j += kSelThreads) {
      const unsigned u = order_key(sc[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned c = 0;
      int dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        const unsigned hc = hist[dg];
        if (c + hc >= remaining) {
          dsel = dg;
          break;
        }
        c += hc;
      }
      sh_prefix = prefix | ((unsigned)dsel << shift);
      sh_remaining = remaining - c;
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix = theta, the t-th largest key; `remaining` keys equal to theta are taken.
  unsigned base_eq = 0, base_out = 0;
  for (int c0 = 0; c0 < Tk; c0 += kSelThreads) {
    const int j = c0 + tid;
    const bool valid = j < Tk;
    const unsigned u = valid ? order_key(sc[j]) : 0u;
    const bool eq = valid && u == prefix;
    const bool gt = valid && u > prefix;
    unsigned eq_total, take_total;
    const unsigned eq_before = block_excl_count(eq, &eq_total, wsum);
    const bool take = gt || (eq && base_eq + eq_before < remaining);
    const unsigned pos = block_excl_count(take, &take_total, wsum);
    if (take && base_out + pos < (unsigned)t) out[base_out + pos] = j;
    base_eq += eq_total;
    base_out += take_total;
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
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.heads), dim3(kSelThreads), 0, a.stream, a.score,
                     a.idx, a.T, a.t);
  if (a.bf16) {
    if (a.d == 128) launch_gather<bf16, 128>(a); else launch_gather<bf16, 64>(a);
  } else {
    if (a.d == 128) launch_gather<float, 128>(a); else launch_gather<float, 64>(a);
  }
  return hipGetLastError();
}

}  // namespace amc
