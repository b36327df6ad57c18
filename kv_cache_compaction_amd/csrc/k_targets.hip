// Full-cache statistics on gfx950: the fused flash pass (lse and outputs) and the
// per-key column-score pass.
//
// What is computed follows "Latent Compaction with Test-Time Training", §3 Preliminaries,
// Eq. 1 (A(q) and Z(q) over the causally visible entries, scale 1/sqrt(d)), and the
// "Compaction" blog, §Fast KV Compaction via Attention Matching, step 1 (per-key attention
// of the reference queries, from which the highest-attention keys are chosen).
//
// Layout: Q [h, n, D], K [h, T, D] in the input dtype; V is first transposed once into the
// workspace as Vt [h, D, Tpad] (Tpad = T rounded up to the key tile, zero padded) so the
// P.V product can read key-contiguous 16-byte fragments from LDS.
//
// Flash pass (one workgroup = WAVES waves x 32 queries): each lane owns one query. The
// score tile is computed transposed, S^T = K Q^T, with Q held in registers as the MFMA B
// operand and 64-key K tiles staged in LDS (double buffered through registers). K rows are
// loaded in the kperm order, so the lane's 32 probabilities of a tile are already the B
// operand of O^T += V^T P^T: no shuffle or LDS round trip between the two products. The
// row max needs one swap between the lane halves; the running sum stays per lane until
// the end. Scores are kept in the log2 domain (x = s * scale * log2 e).
//
// Column-score pass (one workgroup = WAVES waves x 32 keys): K fragments stay in
// registers, query tiles stream through LDS with one shift per query, u = m + log2 l from
// the flash pass's row statistics, and p = 2^(x - u) with the same MFMA operands and order
// as the flash pass. Each lane accumulates 16 queries of its key in fp32 and folds the
// partial into fp64 once per 32-query block; the two lane halves are combined at the end.
// No atomics: every key is owned by one lane.
#include "am_common.hpp"
#include "am_internal.hpp"

#include <type_traits>

namespace amc {

constexpr int kBN = 64;  // keys per flash-pass tile
constexpr int kBQ = 64;  // queries per column-score tile

template <typename T> constexpr int epc() { return 16 / (int)sizeof(T); }  // elements per 16 B

// ------------------------------------------------------------------------------------
// V [h, T, D] -> Vt [h, D, Tpad], zero padded beyond T (Ti -> T converts, e.g. fitted
// fp32 values to the problem dtype for the compacted-attention pass).
// ------------------------------------------------------------------------------------
template <typename Ti, typename T, int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const Ti* __restrict__ V,
                                                          T* __restrict__ Vt, int Tk, int Tpad) {
  constexpr int E = epc<T>();
  constexpr int Ei = epc<Ti>();
  __shared__ T tile[kBN][D + 1];
  const int head = blockIdx.y;
  const int k0 = blockIdx.x * kBN;
  const Ti* Vh = V + (size_t)head * Tk * D;
  for (int c = threadIdx.x; c < kBN * D / Ei; c += 256) {
    const int row = c / (D / Ei), col = (c % (D / Ei)) * Ei;
    const int key = k0 + row;
    if (key < Tk) {
      const uint4 v = *(const uint4*)(Vh + (size_t)key * D + col);
      const Ti* e = (const Ti*)&v;
#pragma unroll
      for (int i = 0; i < Ei; ++i) tile[row][col + i] = (T)(float)e[i];
    } else {
#pragma unroll
      for (int i = 0; i < Ei; ++i) tile[row][col + i] = (T)0.0f;
    }
  }
  __syncthreads();
  T* Vth = Vt + (size_t)head * D * Tpad;
  for (int c = threadIdx.x; c < D * kBN / E; c += 256) {
    const int d = c / (kBN / E), kk = (c % (kBN / E)) * E;
    uint4 v;
    T* e = (T*)&v;
#pragma unroll
    for (int i = 0; i < E; ++i) e[i] = tile[kk + i][d];
    *(uint4*)(Vth + (size_t)d * Tpad + k0 + kk) = v;
  }
}

// ------------------------------------------------------------------------------------
// Flash pass.
// ------------------------------------------------------------------------------------
template <typename T, int D, int BN>
struct FlashLds {
  static constexpr int KP = D + epc<T>();    // K tile row pitch (+16 B against bank conflicts)
  static constexpr int VP = BN + epc<T>();   // Vt tile row pitch
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int BUF = K_ELEMS + D * VP;
};

// One kernel serves the full cache and the biased compacted cache. With BIASED, key j
// carries a bias b_j (natural log, may be -inf) added to its score and an original
// position keypos[j] that the causal mask compares against (Latent Compaction §3.1,
// Eq. 2-4: l(q) = s K_cmp q + b and Z_cmp = 1^T exp(l)). With Y set, the epilogue writes
// (||O_i - Y_i||^2, ||Y_i||^2) per query instead of O.
struct FlashParams {
  const void* Q; const void* K; const void* Vt;
  const float* bias; const int32_t* keypos; const float* Y;
  const int2* tstat;   // biased causal: per key tile (min, max) original position, or null
  const int32_t* qpos; // query positions [h, n], ascending per head, or null (position i / group)
  float* lse; float2* rowstat; float* O; float2* rowres;
  int n, Tk, Tpad, group, heads, n_qtiles;
  float c2;
};

// Launch shape (measured on MI355X at the long causal workload): 8 waves of 32 queries
// each, two waves per SIMD (waves w and w + 4) running their tile phases half a tile apart,
// so one wave's softmax meets the other's MFMAs; 64-key tiles (32 for fp32 operands at
// d = 128, for LDS) in a ring of four LDS buffers with one barrier per tile; the running
// max is rescaled lazily.
constexpr int kFlashWaves = 8;

// Workgroup b -> (head, item) for a grid of heads x nper workgroups. Linear id b runs on
// XCD b % 8; when the heads split evenly over the eight XCDs, each XCD takes whole heads
// (head = 8 j + b % 8) and walks one head's items before the next, so the workgroups that
// run together on an XCD share that head's K, V^T or Q tiles in its L2. Otherwise heads
// are interleaved (head = b % heads). Items run in ascending order per head either way.
__device__ __forceinline__ void head_major(int b, int heads, int nper, int& head, int& item) {
  if ((heads & 7) == 0) {
    const int slot = b >> 3;
    head = (slot / nper) * 8 + (b & 7);
    item = slot % nper;
  } else {
    head = b % heads;
    item = b / heads;
  }
}
template <typename T, int D> constexpr int flash_bn() { return (sizeof(T) == 4 && D == 128) ? 32 : 64; }
constexpr float kLazyTau = 8.f;  // rescale only when the row max grows by more than 2^8

template <typename T, int D, int WAVES, bool CAUSAL, bool WITH_O, bool BIASED>
__global__ __launch_bounds__(WAVES * 64, 2) void flash_fwd_kernel(const FlashParams p) {
  constexpr int BN = flash_bn<T, D>();
  using L = FlashLds<T, D, BN>;
  typedef typename V8<T>::type v8;
  constexpr int NKB = BN / 32;                // 32-key blocks per tile
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * 32;
  constexpr int NBUF = 4;
  constexpr int E = epc<T>();
  constexpr int KCPR = D / E;                 // 16-byte chunks per K row
  constexpr int VCPR = BN / E;                // 16-byte chunks per Vt row
  constexpr int KCH = BN * KCPR, VCH = D * VCPR;   // 16-byte chunks per K / Vt tile
  constexpr int KPT = (KCH + NT - 1) / NT;         // K chunks per thread
  constexpr int VPT = WITH_O ? (VCH + NT - 1) / NT : 0;
  constexpr int KC = D / 16;                  // 16-deep k-steps over the head dim
  constexpr int DB = D / 32;

  __shared__ __align__(16) T lds[NBUF * L::BUF];
  __shared__ float kbias[BIASED ? NBUF : 1][BIASED ? BN : 1];
  __shared__ int kposs[BIASED ? NBUF : 1][BIASED ? BN : 1];

  const int n = p.n, Tk = p.Tk, group = p.group;
  const int b = blockIdx.x;
  int head, item;
  head_major(b, p.heads, p.n_qtiles, head, item);
  const int tile = p.n_qtiles - 1 - item;  // late (longest under the causal mask) first
  const int q0 = tile * BM;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)

  const T* Qh = (const T*)p.Q + (size_t)head * n * D;
  const T* Kh = (const T*)p.K + (size_t)head * Tk * D;
  const T* Vh = (const T*)p.Vt + (size_t)head * D * p.Tpad;

  const int wq0 = q0 + wave * 32;            // first query of this wave
  const int qi = wq0 + r;                    // this lane's query (column of S^T)
  // a query subset carries its positions (ascending); else query i sits at i / group
  auto qposf = [&](int q) { return p.qpos ? p.qpos[(size_t)head * n + q] : q / group; };
  const int qpos = p.qpos ? qposf(min(qi, n - 1)) : qi / group;
  v8 bq[KC];
  {
    const int qrow = min(qi, n - 1);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) bq[kc] = *(const v8*)(Qh + (size_t)qrow * D + kc * 16 + hh * 8);
  }

  int kend = Tk;
  if (CAUSAL && !BIASED) kend = min(Tk, qposf(min(q0 + BM, n) - 1) + 1);
  // leading tiles this wave can take without any mask
  int nfull = Tk / BN;
  if (CAUSAL && !BIASED)
    nfull = min(nfull, ((p.qpos ? qposf(min(wq0, n - 1)) : wq0 / group) + 1) / BN);
  if (CAUSAL && BIASED) {
    // compacted keys carry their original positions: tiles past the last one holding a
    // key visible to the workgroup's last query are dropped, and leading tiles whose every
    // key is visible to this wave's first query need no mask
    int nf = 0, last = -1;
    if (p.tstat) {
      const int2* ts = p.tstat + (size_t)head * ((Tk + BN - 1) / BN);
      const int qmax = qposf(min(q0 + BM, n) - 1);
      const int qmin = p.qpos ? qposf(min(wq0, n - 1)) : wq0 / group;
      bool lead = true;
      for (int i = 0; i < (Tk + BN - 1) / BN; ++i) {
        const int2 v = ts[i];
        if (v.x <= qmax) last = i;
        lead = lead && v.y <= qmin;
        if (lead) nf = i + 1;
      }
      kend = min(Tk, (last + 1) * BN);
    }
    nfull = min(nfull, nf);
  }
  const int ntiles = (kend + BN - 1) / BN;
  nfull = min(nfull, ntiles);

  u32x4 kreg[KPT];
  u32x4 vreg[VPT > 0 ? VPT : 1];
  float breg = 0.f;
  int preg = 0;
  auto gload = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / KCPR, col = (c % KCPR) * E;
        const int kr = min(k0 + row, Tk - 1);
        kreg[i] = *(const u32x4*)(Kh + (size_t)kr * D + col);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (VCH % NT == 0 || c < VCH) {
        const int row = c / VCPR, col = (c % VCPR) * E;
        vreg[i] = *(const u32x4*)(Vh + (size_t)row * p.Tpad + k0 + col);
      }
    }
    if (BIASED && tid < BN) {
      const int kr = min(k0 + tid, Tk - 1);
      breg = p.bias[(size_t)head * Tk + kr] * kLog2e;
      if (CAUSAL) preg = p.keypos[(size_t)head * Tk + kr];   // positions only mask causal rows
    }
  };
  auto sstore = [&](int buf) {
    T* Ks = lds + buf * L::BUF;
    T* Vs = Ks + L::K_ELEMS;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (KCH % NT == 0 || c < KCH) *(u32x4*)(Ks + (c / KCPR) * L::KP + (c % KCPR) * E) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (VCH % NT == 0 || c < VCH) *(u32x4*)(Vs + (c / VCPR) * L::VP + (c % VCPR) * E) = vreg[i];
    }
    if (BIASED && tid < BN) {
      kbias[buf][tid] = breg;
      kposs[buf][tid] = preg;
    }
  };

  f32x16 oacc[WITH_O ? DB : 1];
#pragma unroll
  for (int db = 0; db < (WITH_O ? DB : 1); ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m = -INFINITY, l = 0.f;

  // One tile in three phases: X, S^T = K Q^T (MFMA); Y, the lazy online softmax (vector
  // ALU); Z, O^T += V^T P^T (MFMA). MASK is a compile-time choice so unmasked tiles carry
  // no per-element visibility code. The two waves that share a SIMD (wave w and w + 4) run
  // the phases half a tile apart: the first group does X(k) Y(k) Z(k) between barriers k
  // and k + 1, the second Y(k-1) Z(k-1) X(k), so one wave's softmax meets the other's
  // products. A four-buffer LDS ring keeps tile k - 1 readable while tile k + 2 is stored.
  const bool lag = wave >= WAVES / 2;   // (wave-uniform)
  f32x16 s[NKB];
  float x[NKB * 16];
  auto phase_x = [&](int kt) {
    const T* Ks = lds + (kt % NBUF) * L::BUF + kperm(r) * L::KP + hh * 8;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        mma16(s[kb], *(const v8*)(Ks + kb * 32 * L::KP + kc * 16), bq[kc]);
  };
  auto phase_y = [&](int kt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = kt % NBUF;
    const int k0 = kt * BN;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kl = kb * 32 + (j < 8 ? 8 * hh + j : 16 + 8 * hh + (j - 8));
        float v = BIASED ? s[kb][j] * p.c2 + kbias[buf][kl] : s[kb][j];
        if (MASK) {
          const int key = k0 + kl;
          const int pos = BIASED ? kposs[buf][kl] : key;
          v = (key < Tk && (!CAUSAL || pos <= qpos)) ? v : -INFINITY;
        }
        x[kb * 16 + j] = v;
      }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < NKB * 16; i += 2) tmax = vmax3(tmax, x[i], i + 1 < NKB * 16 ? x[i + 1] : x[i]);
    tmax = vmax(tmax, shfl_xor32(tmax));
    if (!BIASED) tmax *= p.c2;
    const bool need = tmax > m + kLazyTau;
    if (__ballot(need)) {
      const float mnew = need ? tmax : m;
      // 0 when m was -inf, 1 when unchanged (also for a row that has seen no entry yet)
      const float alpha = m == mnew ? 1.f : ex2(m - mnew);
      l *= alpha;
      if constexpr (WITH_O) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      }
      m = mnew;
    }
    const float msafe = m == -INFINITY ? 0.f : m;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NKB * 16; ++i) {
      x[i] = BIASED ? ex2(x[i] - msafe) : ex2(__builtin_fmaf(x[i], p.c2, -msafe));
      psum += x[i];
    }
    l += psum;
  };
  auto phase_z = [&](int kt) {
    if constexpr (WITH_O) {
      const T* Vs = lds + (kt % NBUF) * L::BUF + L::K_ELEMS + r * L::VP + hh * 8;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const v8 pb = AM_PACK8(T, x, kb * 16 + kk * 8);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            mma16(oacc[db], *(const v8*)(Vs + db * 32 * L::VP + kb * 32 + kk * 16), pb);
        }
    }
  };
  if (ntiles > 0) {
    gload(0);
    sstore(0);
    if (ntiles > 1) {
      gload(1);
      sstore(1);
    }
  }
  __syncthreads();
  // every wave runs ntiles intervals with one barrier each; only the phase order differs
  auto interval_end = [&](int kt) {
    if (kt + 2 < ntiles) sstore((kt + 2) % NBUF);
    __syncthreads();
  };
  if (!lag) {
    for (int kt = 0; kt < nfull; ++kt) {
      if (kt + 2 < ntiles) gload(kt + 2);
      phase_x(kt);
      phase_y(kt, std::false_type{});
      phase_z(kt);
      interval_end(kt);
    }
    for (int kt = nfull; kt < ntiles; ++kt) {
      if (kt + 2 < ntiles) gload(kt + 2);
      phase_x(kt);
      phase_y(kt, std::true_type{});
      phase_z(kt);
      interval_end(kt);
    }
  } else if (ntiles > 0) {
    if (2 < ntiles) gload(2);
    phase_x(0);
    interval_end(0);
    const int kmid = min(nfull, ntiles - 1);
    for (int kt = 1; kt <= kmid; ++kt) {   // tile kt - 1 < nfull: no mask
      if (kt + 2 < ntiles) gload(kt + 2);
      phase_y(kt - 1, std::false_type{});
      phase_z(kt - 1);
      phase_x(kt);
      interval_end(kt);
    }
    for (int kt = max(kmid + 1, 1); kt < ntiles; ++kt) {
      if (kt + 2 < ntiles) gload(kt + 2);
      phase_y(kt - 1, std::true_type{});
      phase_z(kt - 1);
      phase_x(kt);
      interval_end(kt);
    }
    // the last tile's buffer is no longer refilled
    if (ntiles - 1 < nfull) phase_y(ntiles - 1, std::false_type{});
    else phase_y(ntiles - 1, std::true_type{});
    phase_z(ntiles - 1);
  }

  const float ltot = l + shfl_xor32(l);
  if constexpr (WITH_O) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (p.Y) {
      float e = 0.f, yy = 0.f;
      const float* Yrow = p.Y + ((size_t)head * n + min(qi, n - 1)) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const float4 y = *(const float4*)(Yrow + db * 32 + jq * 8 + hh * 4);
          const float d0 = oacc[db][jq * 4 + 0] * inv - y.x;
          const float d1 = oacc[db][jq * 4 + 1] * inv - y.y;
          const float d2 = oacc[db][jq * 4 + 2] * inv - y.z;
          const float d3 = oacc[db][jq * 4 + 3] * inv - y.w;
          e += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
          yy += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
        }
      e += shfl_xor32(e);
      yy += shfl_xor32(yy);
      if (qi < n && hh == 0) p.rowres[(size_t)head * n + qi] = make_float2(e, yy);
    } else if (qi < n) {
      float* Orow = p.O + ((size_t)head * n + qi) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          float4 v;
          v.x = oacc[db][jq * 4 + 0] * inv;
          v.y = oacc[db][jq * 4 + 1] * inv;
          v.z = oacc[db][jq * 4 + 2] * inv;
          v.w = oacc[db][jq * 4 + 3] * inv;
          *(float4*)(Orow + db * 32 + jq * 8 + hh * 4) = v;
        }
    }
  }
  if (qi < n && hh == 0) {
    const float lgl = lg2(ltot);
    if (p.lse) p.lse[(size_t)head * n + qi] = (m + lgl) * kLn2;
    if (p.rowstat) p.rowstat[(size_t)head * n + qi] = make_float2(m, lgl);
  }
}

// ------------------------------------------------------------------------------------
// Column-score pass.
// ------------------------------------------------------------------------------------
// MODE: 0 = RMS (sum of p^2), 1 = MEAN (sum of p), 2 = MAX (max of p), 3 = the log2 of
// MAX (no final exponentiation, for masses far below the shift). Only the requested
// statistic is computed: with the row shift u = m + log2 l, RMS exponentiates 2 (x - u)
// directly (p^2; the doubling is exact) and MAX keeps the max of the exponent and
// exponentiates once at the end.
template <typename T, int D> constexpr int colscore_kb() { return (sizeof(T) == 4 && D == 128) ? 1 : 2; }

// KPOS: the keys carry original positions keypos[h, Tk] (ascending; compacted keys) for the
// causal mask instead of their index. head_shift (non-null): one shift per head, in log2
// units, replaces the per-query row statistics (unnormalized masses on a common scale);
// key_shift (KPOS only, non-null): a further per-key shift [h, Tk] in log2 units.
// Query split: gridDim.y workgroups share a key block, each taking qchunk queries (a
// multiple of kBQ); with more than one they write partials [split, h, Tk] (the log2 max,
// or the plain sum) for colscore_reduce_kernel.
// QPOS: the queries are a subset with positions qpos[h, n] (every tile takes the mask).
template <typename T, int D, int WAVES, bool CAUSAL, int MODE, bool KPOS, bool QPOS = false>
__global__ __launch_bounds__(WAVES * 64, 2) void colscore_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float2* __restrict__ rowstat,
    float* __restrict__ score, int n, int Tk, int group, float c2, int heads,
    const int32_t* __restrict__ keypos, const float* __restrict__ head_shift,
    const float* __restrict__ key_shift, int qchunk, const int32_t* __restrict__ qpos) {
  constexpr bool MAXM = MODE == 2 || MODE == 3;
  typedef typename V8<T>::type v8;
  constexpr int KB = colscore_kb<T, D>();  // 32-key blocks per wave
  constexpr int NT = WAVES * 64;
  constexpr int BK = WAVES * 32 * KB;
  constexpr int E = epc<T>();
  constexpr int QP = D + E;
  constexpr int QCPR = D / E;
  constexpr int QPT = kBQ * QCPR / NT;
  constexpr int KC = D / 16;
  static_assert(kBQ * QCPR % NT == 0, "tile/thread mismatch");
  static_assert(kBQ <= NT, "row statistics load");
  const float f = MODE == 0 ? 2.f : 1.f;   // exponent factor

  __shared__ __align__(16) T qs[2][kBQ * QP];
  __shared__ __align__(16) float rs[2][kBQ];   // f (m + log2 l) per query
  __shared__ int qps[QPOS ? 2 : 1][QPOS ? kBQ : 1];   // query positions of a subset

  const int b = blockIdx.x;
  int head, kblk;
  head_major(b, heads, gridDim.x / heads, head, kblk);
  const int k0 = kblk * BK;  // key block 0 (most queries under the causal mask) first
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const T* Qh = Q + (size_t)head * n * D;
  const T* Kh = K + (size_t)head * Tk * D;
  const float2* RSh = rowstat + (size_t)head * n;
  const int32_t* KPh = KPOS ? keypos + (size_t)head * Tk : nullptr;
  auto kpos = [&](int k) { return KPOS ? KPh[min(k, Tk - 1)] : k; };

  const int wk0 = k0 + wave * 32 * KB;
  v8 bk[KB][KC];
  int key[KB], kp[KB];
  float ksh[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    key[kb] = wk0 + kb * 32 + r;
    kp[kb] = kpos(key[kb]);
    ksh[kb] = (KPOS && key_shift) ? key_shift[(size_t)head * Tk + min(key[kb], Tk - 1)] : 0.f;
    const int krow = min(key[kb], Tk - 1);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      bk[kb][kc] = *(const v8*)(Kh + (size_t)krow * D + kc * 16 + hh * 8);
  }

  // query chunks are dealt last first: under the causal mask the last chunk is the one
  // every key block sees, so the heavy workgroups start first
  const int nsplit = gridDim.y, split = nsplit - 1 - (int)blockIdx.y;
  const int qlo = split * qchunk, qend = min(n, qlo + qchunk);
  int qbeg = qlo;
  if (CAUSAL && !QPOS) qbeg = max(qlo, (min(n, kpos(k0) * group) / kBQ) * kBQ);
  const int ntiles = qend > qbeg ? (qend - qbeg + kBQ - 1) / kBQ : 0;

  u32x4 qreg[QPT];
  float rreg = 0.f;
  int qpreg = 0;
  auto gload = [&](int it) {
    const int qt0 = qbeg + it * kBQ;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / QCPR, col = (c % QCPR) * E;
      qreg[i] = *(const u32x4*)(Qh + (size_t)min(qt0 + row, n - 1) * D + col);
    }
    if (QPOS && tid < kBQ) qpreg = qpos[(size_t)head * n + min(qt0 + tid, n - 1)];
    if (tid < kBQ) {
      if (head_shift) {
        rreg = f * head_shift[head];
      } else {
        const float2 st = RSh[min(qt0 + tid, n - 1)];
        rreg = f * (st.x + st.y);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + i * NT;
      *(u32x4*)(&qs[buf][(c / QCPR) * QP + (c % QCPR) * E]) = qreg[i];
    }
    if (tid < kBQ) rs[buf][tid] = rreg;
    if (QPOS && tid < kBQ) qps[buf][tid] = qpreg;
  };

  double acc[KB];
  float amx[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    acc[kb] = 0.0;
    amx[kb] = -INFINITY;
  }
  const float fc2 = f * c2;

  // One query tile; MASK is a compile-time choice (diagonal tiles and a ragged end only).
  auto tile_step = [&](int it, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it & 1;
    if (it + 1 < ntiles) gload(it + 1);
    const int qt0 = qbeg + it * kBQ;
#pragma unroll
    for (int qb = 0; qb < kBQ / 32; ++qb) {
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
      const T* arow = &qs[buf][(qb * 32 + r) * QP + hh * 8];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const v8 a = *(const v8*)(arow + kc * 16);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma16(s[kb], a, bk[kb][kc]);
      }
      // rows crow(4a .. 4a + 3, hh) are consecutive: one 16-byte read per four elements
      float sh[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 v = *(const float4*)&rs[buf][qb * 32 + a4 * 8 + hh * 4];
        sh[4 * a4 + 0] = v.x;
        sh[4 * a4 + 1] = v.y;
        sh[4 * a4 + 2] = v.z;
        sh[4 * a4 + 3] = v.w;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float part = MAXM ? -INFINITY : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float e = __builtin_fmaf(s[kb][j], fc2, -sh[j]);
          if (KPOS) e -= ksh[kb];
          if (MASK) {
            const int q = qt0 + qb * 32 + crow(j, hh);
            const int qp = QPOS ? qps[buf][qb * 32 + crow(j, hh)] : q / group;
            e = (q < qend && (!CAUSAL || kp[kb] <= qp)) ? e : -INFINITY;
          }
          if (MAXM) part = vmax(part, e);
          else part += ex2(e);
        }
        if (MAXM) amx[kb] = vmax(amx[kb], part);
        else acc[kb] += (double)part;
      }
    }
    if (it + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  // leading tiles on the causal diagonal and a ragged last tile need the mask
  int nhead = 0;
  if (CAUSAL) nhead = min(ntiles, max(0, (group * kpos(wk0 + 32 * KB - 1) - qbeg + kBQ - 1) / kBQ));
  if (CAUSAL && QPOS) nhead = ntiles;
  int nbody = ntiles - ((qbeg + ntiles * kBQ > qend) ? 1 : 0);
  nbody = max(nbody, nhead);
  for (int it = 0; it < nhead; ++it) tile_step(it, std::true_type{});
  for (int it = nhead; it < nbody; ++it) tile_step(it, std::false_type{});
  for (int it = nbody; it < ntiles; ++it) tile_step(it, std::true_type{});
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float out;
    if (MAXM) {
      const float mx = vmax(amx[kb], shfl_xor32(amx[kb]));
      out = (MODE == 3 || nsplit > 1) ? mx : ex2(mx);
    } else {
      const double tot = acc[kb] + __shfl_xor(acc[kb], 32, 64);
      out = nsplit > 1 ? (float)tot
                       : (MODE == 0 ? (float)sqrt(tot / (double)n) : (float)(tot / (double)n));
    }
    if (hh == 0 && key[kb] < Tk) score[((size_t)split * heads + head) * Tk + key[kb]] = out;
  }
}

// Combines the query-split partials [nsplit, h, Tk] of the column pass (fixed order).
__global__ __launch_bounds__(256) void colscore_reduce_kernel(const float* __restrict__ part,
                                                              float* __restrict__ out, int heads,
                                                              int Tk, int nsplit, int n, int mode) {
  const int head = blockIdx.y, key = blockIdx.x * 256 + threadIdx.x;
  if (key >= Tk) return;
  const size_t stride = (size_t)heads * Tk, o = (size_t)head * Tk + key;
  float r;
  if (mode >= 2) {
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) mx = vmax(mx, part[sp * stride + o]);
    r = mode == 3 ? mx : ex2(mx);
  } else {
    double tot = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) tot += (double)part[sp * stride + o];
    r = mode == 0 ? (float)sqrt(tot / (double)n) : (float)(tot / (double)n);
  }
  out[o] = r;
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
constexpr int kScoreWaves = 4;

template <typename T, int D, bool BIASED>
static void launch_flash(FlashParams fp, bool causal, bool with_o, hipStream_t st) {
  constexpr int BM = kFlashWaves * 32;
  fp.n_qtiles = (fp.n + BM - 1) / BM;
  const dim3 g(fp.n_qtiles * fp.heads), blk(kFlashWaves * 64);
#define AM_FLASH(C, W) \
  hipLaunchKernelGGL((flash_fwd_kernel<T, D, kFlashWaves, C, W, BIASED>), g, blk, 0, st, fp)
  if (causal) {
    if (with_o) AM_FLASH(true, true); else AM_FLASH(true, false);
  } else {
    if (with_o) AM_FLASH(false, true); else AM_FLASH(false, false);
  }
#undef AM_FLASH
}

template <typename T, int D>
static hipError_t launch_targets_t(const TargetsArgs& a) {
  const int Tpad = round_up(a.T, kBN);
  const float c2 = a.scale * kLog2e;
  if (a.O) {
    dim3 g(Tpad / kBN, a.heads);
    hipLaunchKernelGGL((transpose_v_kernel<T, T, D>), g, dim3(256), 0, a.stream, (const T*)a.V,
                       (T*)a.Vt, a.T, Tpad);
  }
  FlashParams fp;
  fp.Q = a.Q; fp.K = a.K; fp.Vt = a.Vt;
  fp.bias = nullptr; fp.keypos = nullptr; fp.Y = nullptr; fp.tstat = nullptr; fp.qpos = a.qpos;
  fp.lse = a.lse; fp.rowstat = (float2*)a.rowstat; fp.O = a.O; fp.rowres = nullptr;
  fp.n = a.n; fp.Tk = a.T; fp.Tpad = Tpad; fp.group = a.group; fp.heads = a.heads;
  fp.c2 = c2;
  launch_flash<T, D, false>(fp, a.causal, a.O != nullptr, a.stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.score) return e;
  const int BK = kScoreWaves * 32 * colscore_kb<T, D>();
  // causal: the query range is cut into up to kColSplit chunks (partial sums in a fixed
  // order), so the long key blocks near the start do not leave their CUs busy long after
  // the others have finished
  int nsplit = 1, qchunk = a.n;
  if (a.causal && !a.qpos && a.colpart) {
    qchunk = round_up((a.n + kColSplit - 1) / kColSplit, kBQ);
    nsplit = (a.n + qchunk - 1) / qchunk;
  }
  float* sdst = nsplit > 1 ? a.colpart : a.score;
  const dim3 gs(((a.T + BK - 1) / BK) * a.heads, nsplit), bs(kScoreWaves * 64);
#define AM_SCORE(C, M)                                                                          \
  hipLaunchKernelGGL((colscore_kernel<T, D, kScoreWaves, C, M, false>), gs, bs, 0, a.stream,   \
                     (const T*)a.Q, (const T*)a.K, (const float2*)a.rowstat, sdst, a.n, a.T,   \
                     a.group, c2, a.heads, (const int32_t*)nullptr, (const float*)nullptr,     \
                     (const float*)nullptr, qchunk, (const int32_t*)nullptr)
  if (a.causal && a.qpos) {   // a query subset with its positions: every tile masked
#define AM_SCORE_Q(M)                                                                           \
  hipLaunchKernelGGL((colscore_kernel<T, D, kScoreWaves, true, M, false, true>), gs, bs, 0,     \
                     a.stream, (const T*)a.Q, (const T*)a.K, (const float2*)a.rowstat, a.score, \
                     a.n, a.T, a.group, c2, a.heads, (const int32_t*)nullptr,                   \
                     (const float*)nullptr, (const float*)nullptr, a.n, a.qpos)
    if (a.mode == 0) AM_SCORE_Q(0); else if (a.mode == 1) AM_SCORE_Q(1); else AM_SCORE_Q(2);
#undef AM_SCORE_Q
  } else if (a.causal) {
    if (a.mode == 0) AM_SCORE(true, 0); else if (a.mode == 1) AM_SCORE(true, 1); else AM_SCORE(true, 2);
    if (nsplit > 1)
      hipLaunchKernelGGL(colscore_reduce_kernel, dim3((a.T + 255) / 256, a.heads), dim3(256), 0,
                         a.stream, (const float*)a.colpart, a.score, a.heads, a.T, nsplit, a.n,
                         a.mode);
  } else {
    if (a.mode == 0) AM_SCORE(false, 0); else if (a.mode == 1) AM_SCORE(false, 1); else AM_SCORE(false, 2);
  }
#undef AM_SCORE
  return hipGetLastError();
}

// Per-key masses of the compacted keys (original positions for the causal mask) in log
// form: kmax = max_i (scale q_i.k_j log2 e - shift2_h) over the queries that see key j,
// then kmean = (1/n) sum_i 2^(that exponent - kmax), so log2 m_j = kmax + log2 kmean holds
// masses far below the common shift without underflow. Two column passes (MAX, MEAN),
// each split over query chunks so that a few hundred compacted keys still fill the chip.
static void key_mass_split(int t, int heads, int n, int bk, int& nsplit, int& qchunk) {
  const int nkb = (t + bk - 1) / bk;
  int want = (1024 + nkb * heads - 1) / (nkb * heads);
  const int maxs = (n + kBQ - 1) / kBQ;
  want = max(1, min(want, min(maxs, kKeyMassMaxSplit)));
  qchunk = ((n + want - 1) / want + kBQ - 1) / kBQ * kBQ;
  nsplit = (n + qchunk - 1) / qchunk;
}
template <typename T, int D, bool C>
static void launch_key_mass_c(const KeyMassArgs& a) {
  const int BK = kScoreWaves * 32 * colscore_kb<T, D>();
  int nsplit, qchunk;
  key_mass_split(a.t, a.heads, a.n, BK, nsplit, qchunk);
  const dim3 gs(((a.t + BK - 1) / BK) * a.heads, nsplit), bs(kScoreWaves * 64);
  const dim3 gr((a.t + 255) / 256, a.heads);
  const float c2 = a.scale * kLog2e;
  float* o1 = nsplit > 1 ? a.part : a.kmax;
  hipLaunchKernelGGL((colscore_kernel<T, D, kScoreWaves, C, 3, true>), gs, bs, 0, a.stream,
                     (const T*)a.Q, (const T*)a.Ck, (const float2*)nullptr, o1, a.n, a.t,
                     a.group, c2, a.heads, a.keypos, a.shift2, (const float*)nullptr, qchunk,
                     (const int32_t*)nullptr);
  if (nsplit > 1)
    hipLaunchKernelGGL(colscore_reduce_kernel, gr, dim3(256), 0, a.stream, (const float*)a.part,
                       a.kmax, a.heads, a.t, nsplit, a.n, 3);
  float* o2 = nsplit > 1 ? a.part : a.kmean;
  hipLaunchKernelGGL((colscore_kernel<T, D, kScoreWaves, C, 1, true>), gs, bs, 0, a.stream,
                     (const T*)a.Q, (const T*)a.Ck, (const float2*)nullptr, o2, a.n, a.t,
                     a.group, c2, a.heads, a.keypos, a.shift2, (const float*)a.kmax, qchunk,
                     (const int32_t*)nullptr);
  if (nsplit > 1)
    hipLaunchKernelGGL(colscore_reduce_kernel, gr, dim3(256), 0, a.stream, (const float*)a.part,
                       a.kmean, a.heads, a.t, nsplit, a.n, 1);
}

// Selection statistic of keys with original positions (a shortlist) against all queries,
// with the queries' row statistics over the same keys: the column pass with KPOS, split
// over query chunks, then the fixed-order combination.
template <typename T, int D, bool C, int M>
static void launch_key_score_m(const KeyScoreArgs& a) {
  const int BK = kScoreWaves * 32 * colscore_kb<T, D>();
  int nsplit, qchunk;
  key_mass_split(a.t, a.heads, a.n, BK, nsplit, qchunk);
  const dim3 gs(((a.t + BK - 1) / BK) * a.heads, nsplit), bs(kScoreWaves * 64);
  const float c2 = a.scale * kLog2e;
  float* o = nsplit > 1 ? a.part : a.score;
  hipLaunchKernelGGL((colscore_kernel<T, D, kScoreWaves, C, M, true>), gs, bs, 0, a.stream,
                     (const T*)a.Q, (const T*)a.Ck, a.rowstat, o, a.n, a.t, a.group, c2, a.heads,
                     a.keypos, (const float*)nullptr, (const float*)nullptr, qchunk,
                     (const int32_t*)nullptr);
  if (nsplit > 1)
    hipLaunchKernelGGL(colscore_reduce_kernel, dim3((a.t + 255) / 256, a.heads), dim3(256), 0,
                       a.stream, (const float*)a.part, a.score, a.heads, a.t, nsplit, a.n, M);
}
template <typename T, int D>
static hipError_t launch_key_score_t(const KeyScoreArgs& a) {
#define AM_KS(C)                                                                   \
  do {                                                                             \
    if (a.mode == 0) launch_key_score_m<T, D, C, 0>(a);                            \
    else if (a.mode == 1) launch_key_score_m<T, D, C, 1>(a);                       \
    else launch_key_score_m<T, D, C, 2>(a);                                        \
  } while (0)
  if (a.causal) AM_KS(true); else AM_KS(false);
#undef AM_KS
  return hipGetLastError();
}
hipError_t launch_key_score(const KeyScoreArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_key_score_t<bf16, 128>(a) : launch_key_score_t<bf16, 64>(a);
  return a.d == 128 ? launch_key_score_t<float, 128>(a) : launch_key_score_t<float, 64>(a);
}

size_t key_mass_part_bytes(int64_t heads, int64_t n, int64_t t) {
  (void)n;
  return align_up((size_t)kKeyMassMaxSplit * heads * t * sizeof(float));
}
template <typename T, int D>
static hipError_t launch_key_mass_t(const KeyMassArgs& a) {
  if (a.causal) launch_key_mass_c<T, D, true>(a);
  else launch_key_mass_c<T, D, false>(a);
  return hipGetLastError();
}

hipError_t launch_key_mass(const KeyMassArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_key_mass_t<bf16, 128>(a) : launch_key_mass_t<bf16, 64>(a);
  return a.d == 128 ? launch_key_mass_t<float, 128>(a) : launch_key_mass_t<float, 64>(a);
}

hipError_t launch_targets(const TargetsArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_targets_t<bf16, 128>(a) : launch_targets_t<bf16, 64>(a);
  return a.d == 128 ? launch_targets_t<float, 128>(a) : launch_targets_t<float, 64>(a);
}

// (min, max) original position of the keys of each BN-key tile of the compacted cache.
__global__ __launch_bounds__(256) void tile_stat_kernel(const int32_t* __restrict__ keypos,
                                                        int2* __restrict__ tstat, int t, int bn,
                                                        int ntile) {
  const int head = blockIdx.y, tile = blockIdx.x * 256 + threadIdx.x;
  if (tile >= ntile) return;
  const int32_t* kp = keypos + (size_t)head * t;
  int lo = 0x7fffffff, hi = -1;
  for (int j = tile * bn; j < min(t, tile * bn + bn); ++j) {
    lo = min(lo, kp[j]);
    hi = max(hi, kp[j]);
  }
  tstat[(size_t)head * ntile + tile] = make_int2(lo, hi);
}

template <typename T, int D>
static hipError_t launch_cmp_t(const CmpAttnArgs& a) {
  const int Tpad = round_up(a.t, kBN);
  if (a.causal && a.tstat) {
    constexpr int BN = flash_bn<T, D>();
    const int ntile = (a.t + BN - 1) / BN;
    hipLaunchKernelGGL(tile_stat_kernel, dim3((ntile + 255) / 256, a.heads), dim3(256), 0,
                       a.stream, a.keypos, a.tstat, a.t, BN, ntile);
  }
  if (a.Cv) {
    dim3 g(Tpad / kBN, a.heads);
    hipLaunchKernelGGL((transpose_v_kernel<float, T, D>), g, dim3(256), 0, a.stream, a.Cv,
                       (T*)a.Vt, a.t, Tpad);
  }
  FlashParams fp;
  fp.Q = a.Q; fp.K = a.Ck; fp.Vt = a.Vt;
  fp.bias = a.bias; fp.keypos = a.keypos; fp.Y = a.Y; fp.tstat = a.causal ? a.tstat : nullptr;
  fp.qpos = nullptr;
  fp.lse = a.lse; fp.rowstat = a.rowstat; fp.O = a.O; fp.rowres = a.rowres;
  fp.n = a.n; fp.Tk = a.t; fp.Tpad = Tpad; fp.group = a.group; fp.heads = a.heads;
  fp.c2 = a.scale * kLog2e;
  launch_flash<T, D, true>(fp, a.causal, a.Cv != nullptr, a.stream);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Log-space merge of two attention results over disjoint entry sets, and slot masking
// ------------------------------------------------------------------------------------
// out = e^{l1 - L} O1 + e^{l2 - L} O2 with L = logaddexp(l1, l2) ("Latent Compaction with
// Test-Time Training", §3.1 Eq. 5, normalizers and weights in log space). One thread per
// four floats of a row; rows where both normalizers are -inf become -inf and zeros. O2
// null: out = O1 and L = l1. out and O1 (or O2) may be the same buffer: each thread reads
// its four floats of both inputs before writing them.
__global__ __launch_bounds__(256) void merge_kernel(const float* O1, const float* __restrict__ l1,
                                                    const float* O2, const float* __restrict__ l2,
                                                    float* out, float* lse_out, long long rows,
                                                    int d4) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * d4) return;
  const long long row = e / d4;
  const int c = (int)(e - row * d4);
  const float a = l1[row];
  const float b = O2 ? l2[row] : -INFINITY;
  const float mx = fmaxf(a, b);
  float L = -INFINITY, w1 = 0.f, w2 = 0.f;
  if (mx > -INFINITY) {
    const float ea = expf(a - mx), eb = expf(b - mx);
    L = mx + logf(ea + eb);
    w1 = ea / (ea + eb);
    w2 = eb / (ea + eb);
  }
  const float4 x = reinterpret_cast<const float4*>(O1 + row * d4 * 4)[c];
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  if (O2) y = reinterpret_cast<const float4*>(O2 + row * d4 * 4)[c];
  float4 r;
  r.x = w1 * x.x + w2 * y.x;
  r.y = w1 * x.y + w2 * y.y;
  r.z = w1 * x.z + w2 * y.z;
  r.w = w1 * x.w + w2 * y.w;
  if (O2 || mx == -INFINITY) reinterpret_cast<float4*>(out + row * d4 * 4)[c] = r;
  else if (out != O1) reinterpret_cast<float4*>(out + row * d4 * 4)[c] = x;
  if (c == 0) lse_out[row] = O2 ? L : a;
}

hipError_t launch_attention_merge(const MergeArgs& a) {
  const long long d4 = a.d / 4, nthr = a.rows * d4;
  if (nthr == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, a.stream,
                     a.O1, a.lse1, a.O2, a.lse2, a.out, a.lse, a.rows, (int)d4);
  return hipGetLastError();
}

// bias_eff[h, j] = bias[h, j] for j < nvalid[h] (clamped to [0, t]), else -inf: padded slots
// take no weight (the pseudocode's slot mask of the compacted branch).
__global__ __launch_bounds__(256) void mask_bias_kernel(const float* __restrict__ bias,
                                                        const int32_t* __restrict__ nvalid,
                                                        float* __restrict__ out, int t) {
  const int head = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= t) return;
  const int nv = min(max(nvalid[head], 0), t);
  out[(size_t)head * t + j] = j < nv ? bias[(size_t)head * t + j] : -INFINITY;
}

hipError_t launch_mask_bias(const float* bias, const int32_t* nvalid, float* out, int heads,
                            int t, hipStream_t st) {
  hipLaunchKernelGGL(mask_bias_kernel, dim3((t + 255) / 256, heads), dim3(256), 0, st, bias,
                     nvalid, out, t);
  return hipGetLastError();
}

hipError_t launch_cmp_attention(const CmpAttnArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_cmp_t<bf16, 128>(a) : launch_cmp_t<bf16, 64>(a);
  return a.d == 128 ? launch_cmp_t<float, 128>(a) : launch_cmp_t<float, 64>(a);
}

size_t targets_ws_bytes(int64_t heads, int64_t n, int64_t T, int64_t d, int esize) {
  const size_t vt = align_up((size_t)heads * d * round_up((int)T, kBN) * esize);
  const size_t rs = align_up((size_t)heads * n * sizeof(float2));
  return vt + rs + targets_colpart_bytes(heads, T);
}

size_t targets_colpart_bytes(int64_t heads, int64_t T) {
  return align_up((size_t)kColSplit * heads * T * sizeof(float));
}

size_t targets_vt_bytes(int64_t heads, int64_t T, int64_t d, int esize) {
  return align_up((size_t)heads * d * round_up((int)T, kBN) * esize);
}

}  // namespace amc

namespace amc {
size_t cmp_vt_bytes(int64_t heads, int64_t t, int64_t d, int esize) {
  return align_up((size_t)heads * d * round_up((int)t, kBN) * esize);
}
size_t cmp_tstat_bytes(int64_t heads, int64_t t) {
  return align_up((size_t)heads * ((t + 31) / 32) * sizeof(int2));   // 32-key tiles or larger
}
}  // namespace amc
