// The two fits on gfx950: beta from the mass equations by NNLS on w = exp(beta)
// ("Compaction" blog, §Choosing beta) and C_v from the output equations by ridge least
// squares (§Choosing C_v), with A_i the biased compacted softmax of "Latent Compaction with
// Test-Time Training", §3.1 Eq. 2-3.
//
// Gram builds for t <= 256 (larger t store the design once and multiply it in tiles, see
// k_syrk.hip). Neither the n x t design M nor A is stored here. A workgroup owns one
// 128 x 128 tile (ta >= tb) of the t x t Gram and one chunk of queries. For every 32
// queries, its four waves recompute the needed 32 x 32 score blocks Q C_k^T on bf16 MFMA
// (query rows loaded in the kperm order), turn them into design entries
// 2^(s * scale * log2 e + bias_j - shift_i) under the causal mask of the original key
// positions, and park them in LDS as bf16 MFMA fragments. Because of the kperm order, a
// lane's fragment of a score block is at once the A operand (as M^T) and the B operand
// (as M) of the Gram product over those queries, so M^T M accumulates with no transpose.
// Diagonal tiles also accumulate M^T b (mass) or A^T Y (values, Y staged as bf16 Y^T).
// Partial tiles per query chunk are summed in a fixed order by a reduce kernel: no
// floating-point atomics, bit-reproducible.
//
// NNLS. Accelerated projected gradient with Jacobi scaling (v = sqrt(diag G) * w),
// step 1/L with L an upper bound on the largest eigenvalue of the scaled G (below),
// momentum restarted when the step turns back
// (gradient-mapping test), stopped on the scaled gradient-mapping norm. t <= 256: one
// workgroup per head. Larger t: P workgroups per head, all resident at once (the launch
// is refused otherwise), each owning a slice of rows (of G too when they fit in LDS),
// meeting at a per-head barrier once per step; all reduce the same partials in the same
// fixed order. Heads are batched so that each gets at least four workgroups. Each solve
// also reports its step count and the KKT residual of the w it returns.
//
// Ridge solve. (G_A + lambda I) C = A^T Y in fp64: right-looking blocked Cholesky with
// 64 x 64 blocks (diagonal factor and its explicit inverse in one workgroup, panel as a
// product with that inverse, trailing update per block pair). The forward substitution
// runs as extra workgroups of the same launches, and each step's update launch also
// factors the next diagonal block; then blocked backward substitution with the stored
// diagonal inverses.
#include "am_common.hpp"
#include "am_internal.hpp"

#include <algorithm>
#include <type_traits>

namespace amc {

constexpr int kGT = 128;  // Gram tile (keys per side)
constexpr int kGQ = 32;   // queries per Gram step
constexpr int kRB = 16;   // NNLS rows per workgroup
constexpr int kNB = 64;   // Cholesky block
// NNLS step size. G = M^T M has no negative entry (M >= 0), nor has A = D^-1 G D^-1, so for
// any positive vector u the largest ratio (A u)_i / u_i bounds A's largest eigenvalue from
// above (Collatz-Wielandt). u starts at all ones and takes kCw - 1 steps u <- A u + kCwShift u
// (the small shift keeps u positive where A has an empty row) toward the dominant
// eigenvector; the bound from the last product, times 1 + 2^-10 for rounding, is L. Three
// products bring it within about 1.1x of the eigenvalue on the mass designs (1.47x with
// one), so every step 1/L is safe with no estimate to pad.
constexpr int kCw = 3;
constexpr float kCwShift = 0x1p-10f;
constexpr float kCwPad = 1.f + 0x1p-10f;

template <typename T> constexpr int epcf() { return 16 / (int)sizeof(T); }

__device__ __forceinline__ void tri_index(int k, int& ta, int& tb) {
  int a = (int)((sqrtf(8.f * (float)k + 1.f) - 1.f) * 0.5f);
  while ((a + 1) * (a + 2) / 2 <= k) ++a;
  while (a * (a + 1) / 2 > k) --a;
  ta = a;
  tb = k - a * (a + 1) / 2;
}

// ------------------------------------------------------------------------------------
// Gram builds
// ------------------------------------------------------------------------------------
struct GramParams {
  const void* Q; const void* Ck; const int32_t* keypos; const float* bias;
  const float* shift2;  // per query, log2 domain
  const float* target;  // mass: per-query right-hand side (null = 1)
  const float* Y;       // values: targets [h, n, D]
  float* Gpart;         // [h, nch, ntri, 128, 128]
  float* Vpart;         // mass: [h, nch, tpad]; values: [h, nch, tpad, D]
  // values without the causal mask: tile 0, which stages every target row of its chunk,
  // also writes the chunk's fp64 sum of squares of Y here [h, nch] (null: not formed)
  double* yyp = nullptr;
  int n, t, tpad, group, ntri, nch, chunk;
  int causal;
  float c2;
};

// Workgroup shape: 8 waves (two per SIMD, so one wave's exponentials overlap another's
// Gram MFMAs). Off-diagonal tiles: wave w owns key block w (a0..a3, b0..b3) and computes
// its 32 x 32 score blocks for every 32-query half of a step with one register copy of
// the C_k fragment; diagonal tiles split the four key blocks over the two query halves.
// A step's design fragments go to one of two LDS buffers; the Gram product of step i-1
// runs from the other buffer while step i's scores are computed, with one barrier per
// step. Q (and Y) tiles are prefetched through registers one step ahead.
template <typename T> constexpr int gram_gq() { return sizeof(T) == 4 ? 32 : 64; }

template <typename T, int D, bool VALUE>
__global__ __launch_bounds__(512, 2) void gram_kernel(const GramParams p) {
  typedef typename V8<T>::type v8;
  constexpr int GQ = gram_gq<T>();          // queries per step
  constexpr int QH = GQ / 32;               // 32-query halves per step
  constexpr int NT = 512;
  constexpr int E = epcf<T>(), QP = D + E, KC = D / 16, YP = GQ + 8;
  constexpr int QCPR = D / E;               // 16-byte chunks per Q row
  constexpr int QCH = GQ * QCPR;            // chunks per Q tile
  constexpr int QPT = (QCH + NT - 1) / NT;
  constexpr int YCH = VALUE ? GQ * D / 4 : 0;  // float4 chunks per Y tile
  constexpr int YPT = VALUE ? (YCH + NT - 1) / NT : 0;
  __shared__ __align__(16) T qs[2][GQ * QP];
  __shared__ float shs[2][GQ], tgs[2][GQ];
  __shared__ __align__(16) bf16x8 mb[2][8][QH][2][64];
  __shared__ __align__(16) bf16 yts[VALUE ? 2 : 1][VALUE ? D * YP : 8];
  __shared__ float hl[8][32];
  __shared__ double yyw[8];

  const int tri = blockIdx.x, chunk = blockIdx.y, head = blockIdx.z;
  // (uniform over the workgroup; tile 0 is diagonal and, without the mask, starts its chunk
  // at the chunk's first query)
  const bool want_yy = VALUE && p.yyp != nullptr && tri == 0 && !p.causal;
  double yy = 0.0;
  int ta, tb;
  tri_index(tri, ta, tb);
  const bool diag = ta == tb;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = p.n, t = p.t;
  const T* Qh = (const T*)p.Q + (size_t)head * n * D;
  const T* Ch = (const T*)p.Ck + (size_t)head * t * D;
  const float* Sh = p.shift2 + (size_t)head * n;
  const float* Yh = VALUE ? p.Y + (size_t)head * n * D : nullptr;

  // this wave's score work: key block `kbid` (0-3 a, 4-7 b) for query halves [qh0, qh1)
  const int kbid = diag ? (wave & 3) : wave;
  const int qh0 = diag ? (QH == 2 ? (wave >> 2) : 0) : 0;
  const int qh1 = diag ? (QH == 2 ? qh0 + 1 : (wave < 4 ? 1 : 0)) : QH;
  const int key = (kbid < 4) ? ta * kGT + 32 * kbid + r : tb * kGT + 32 * (kbid - 4) + r;
  const bool kval = key < t;
  const int kr = min(key, t - 1);
  v8 bck[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) bck[kc] = *(const v8*)(Ch + (size_t)kr * D + kc * 16 + hh * 8);
  // first query that sees this key under the causal mask. Keys past t (padding of the last
  // tile) repeat key t - 1: their Gram rows and columns are finite and never read.
  const int kq0 = p.causal ? p.keypos[(size_t)head * t + kr] * p.group : 0;
  const float kb2 = VALUE ? p.bias[(size_t)head * t + kr] * kLog2e : 0.f;
  int kq0max = kval ? kq0 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kq0max = max(kq0max, __shfl_xor(kq0max, o, 64));
  kq0max = __builtin_amdgcn_readfirstlane(kq0max);

  // this wave's Gram blocks: a-block gx, b-blocks gy0, gy0 + 1 (and R blocks on diagonal)
  const int gx = wave >> 1, gy0 = 2 * (wave & 1);

  const int qa = chunk * p.chunk;
  const int qb = min(n, qa + p.chunk);
  int qstart = qa;
  if (p.causal) {
    // queries before the later of the two blocks' first positions see nothing in one block
    const int f = max(p.keypos[(size_t)head * t + min(ta * kGT, t - 1)],
                      p.keypos[(size_t)head * t + min(tb * kGT, t - 1)]);
    qstart = max(qa, (int)min((long long)f * p.group, (long long)qb) / 32 * 32);
  }
  const int nsteps = (qb - qstart + GQ - 1) / GQ;

  u32x4 qreg[QPT];
  float4 yreg[YPT > 0 ? YPT : 1];
  float sreg = 0.f, treg = 1.f;
  auto qload = [&](int st) {
    const int q0 = qstart + st * GQ;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + i * NT;
      if (QCH % NT == 0 || c < QCH) {
        const int row = c / QCPR, col = (c % QCPR) * E;
        qreg[i] = *(const u32x4*)(Qh + (size_t)min(q0 + row, n - 1) * D + col);
      }
    }
    if (tid < GQ) {
      const int q = min(q0 + tid, n - 1);
      sreg = Sh[q];
      treg = p.target ? p.target[(size_t)head * n + q] : 1.f;
    }
  };
  auto qstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = tid + i * NT;
      if (QCH % NT == 0 || c < QCH)
        *(u32x4*)&qs[buf][(c / QCPR) * QP + (c % QCPR) * E] = qreg[i];
    }
    if (tid < GQ) {
      shs[buf][tid] = sreg;
      tgs[buf][tid] = treg;
    }
  };
  auto yload = [&](int st) {
    if constexpr (VALUE) {
      const int q0 = qstart + st * GQ;
#pragma unroll
      for (int i = 0; i < YPT; ++i) {
        const int c = tid + i * NT;
        if (YCH % NT == 0 || c < YCH) {
          const int row = c / (D / 4), col = (c % (D / 4)) * 4;
          yreg[i] = *(const float4*)(Yh + (size_t)min(q0 + row, n - 1) * D + col);
          if (want_yy && q0 + row < qb) {
            const float4 v = yreg[i];
            yy += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
          }
        }
      }
    }
  };
  auto ystore = [&](int buf) {
    if constexpr (VALUE) {
#pragma unroll
      for (int i = 0; i < YPT; ++i) {
        const int c = tid + i * NT;
        if (YCH % NT == 0 || c < YCH) {
          const int row = c / (D / 4), col = (c % (D / 4)) * 4;
          yts[buf][(col + 0) * YP + row] = (bf16)yreg[i].x;
          yts[buf][(col + 1) * YP + row] = (bf16)yreg[i].y;
          yts[buf][(col + 2) * YP + row] = (bf16)yreg[i].z;
          yts[buf][(col + 3) * YP + row] = (bf16)yreg[i].w;
        }
      }
    }
  };

  f32x16 gacc[2];
  f32x16 racc[VALUE ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) gacc[i][j] = 0.f;
#pragma unroll
  for (int i = 0; i < (VALUE ? 2 : 1); ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) racc[i][j] = 0.f;
  float hacc = 0.f;

  // Gram (and R) MFMAs over the design fragments of one finished step
  auto gram_part = [&](int buf) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 av = mb[buf][gx][qh][ks][lane];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int y = gy0 + i;
          mma16(gacc[i], av, mb[buf][diag ? y : 4 + y][qh][ks][lane]);
        }
        if (VALUE && diag) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
            if ((gy0 + i) * 32 < D)   // d = 64 has two 32-column blocks
              mma16(racc[i], av,
                    *(const bf16x8*)&yts[buf][((gy0 + i) * 32 + r) * YP + qh * 32 + ks * 16 + hh * 8]);
        }
      }
  };

  if (nsteps > 0) {
    qload(0);
    qstore(0);
    if (nsteps > 1) qload(1);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (diag) yload(st);   // this step's targets (diagonal tiles only); staged as Y^T below
    if (st > 0) gram_part(buf ^ 1);
    // scores, design entries, fragments for this step; NH independent 32-query halves are
    // interleaved so their MFMA chains overlap. MASK (wave-uniform) is needed only where
    // some query of the step cannot see a key of this wave's block, or past the chunk end.
    const int q0 = qstart + st * GQ;
    // MASK: 0 none, 1 causal (first visible query kq0 of this lane's key), 2 causal and the
    // chunk end. Element j of a lane holds query qbase + o_j with o_j = j (j < 8) or j + 8.
    auto scores = [&](auto nh_tag, int qhb, auto mask_tag) {
      constexpr int NH = decltype(nh_tag)::value;
      constexpr int MASK = decltype(mask_tag)::value;
      f32x16 sacc[NH];
#pragma unroll
      for (int u = 0; u < NH; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[u][j] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int u = 0; u < NH; ++u)
          mma16(sacc[u], *(const v8*)&qs[buf][((qhb + u) * 32 + kperm(r)) * QP + hh * 8 + kc * 16],
                bck[kc]);
#pragma unroll
      for (int u = 0; u < NH; ++u) {
        const int qh = qhb + u;
        // row shifts of this lane's 16 queries: rows 8h..8h+7 and 16+8h..16+8h+7 of the half
        const float4* s4 = (const float4*)&shs[buf][qh * 32 + 8 * hh];
        const float4 sa = s4[0], sb = s4[1], sc = s4[4], sd = s4[5];
        const float shv[16] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w,
                               sc.x, sc.y, sc.z, sc.w, sd.x, sd.y, sd.z, sd.w};
        float mv[16];
        const int qbase = q0 + qh * 32 + 8 * hh;
        const int lo = kq0 - qbase, hi = qb - qbase;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          // masked entries get exponent -inf (so pairs of fp32 values stay packable)
          float x = VALUE ? __builtin_fmaf(sacc[u][j], p.c2, kb2) - shv[j]
                          : __builtin_fmaf(sacc[u][j], p.c2, -shv[j]);
          const int o = j < 8 ? j : j + 8;
          if (MASK == 1) x = o >= lo ? x : -INFINITY;
          if (MASK == 2) x = (o >= lo && o < hi) ? x : -INFINITY;
          mv[j] = ex2(x);
        }
        if (!VALUE && diag) {
          const float4* t4 = (const float4*)&tgs[buf][qh * 32 + 8 * hh];
          const float4 ta4 = t4[0], tb4 = t4[1], tc4 = t4[4], td4 = t4[5];
          const float tg[16] = {ta4.x, ta4.y, ta4.z, ta4.w, tb4.x, tb4.y, tb4.z, tb4.w,
                                tc4.x, tc4.y, tc4.z, tc4.w, td4.x, td4.y, td4.z, td4.w};
#pragma unroll
          for (int j = 0; j < 16; ++j) hacc += mv[j] * tg[j];
        }
        mb[buf][kbid][qh][0][lane] = AM_PACK8(bf16, mv, 0);
        mb[buf][kbid][qh][1][lane] = AM_PACK8(bf16, mv, 8);
      }
    };
    const int mask = (q0 + GQ > qb) ? 2 : (q0 < kq0max ? 1 : 0);
    using M0 = std::integral_constant<int, 0>;
    using M1 = std::integral_constant<int, 1>;
    using M2 = std::integral_constant<int, 2>;
    auto scores_m = [&](auto nh_tag, int qhb) {
      if (mask == 0) scores(nh_tag, qhb, M0{});
      else if (mask == 1) scores(nh_tag, qhb, M1{});
      else scores(nh_tag, qhb, M2{});
    };
    if (!diag) {
      if constexpr (VALUE) {   // one query half at a time keeps the value variant in registers
#pragma unroll
        for (int qh = 0; qh < QH; ++qh) scores_m(std::integral_constant<int, 1>{}, qh);
      } else {
        scores_m(std::integral_constant<int, QH>{}, 0);
      }
    } else if (qh0 < qh1) {
      scores_m(std::integral_constant<int, 1>{}, qh0);
    }
    if (diag) ystore(buf);   // read by the Gram part of the next step
    // next step's query tile
    if (st + 1 < nsteps) qstore(buf ^ 1);
    if (st + 2 < nsteps) qload(st + 2);
    __syncthreads();
  }
  if (nsteps > 0) gram_part((nsteps - 1) & 1);

  float* Gp = p.Gpart + (((size_t)head * p.nch + chunk) * p.ntri + tri) * kGT * kGT;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      Gp[(gx * 32 + crow(j, hh)) * kGT + (gy0 + i) * 32 + r] = gacc[i][j];
  if (diag) {
    if (!VALUE) {
      hacc += shfl_xor32(hacc);   // (off-diagonal tiles never write h)
      if (hh == 0) hl[wave][r] = hacc;
      __syncthreads();
      if (wave < 4 && hh == 0) {
        const float hv = hl[wave][r] + (QH == 2 ? hl[wave + 4][r] : 0.f);
        p.Vpart[((size_t)head * p.nch + chunk) * p.tpad + ta * kGT + 32 * wave + r] = hv;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if ((gy0 + i) * 32 < D)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int row = ta * kGT + 32 * gx + crow(j, hh);
            p.Vpart[(((size_t)head * p.nch + chunk) * p.tpad + row) * D + (gy0 + i) * 32 + r] =
                racc[i][j];
          }
    }
  }
  if (want_yy) {   // fixed order: lanes by xor tree, then the eight waves in turn
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) yy += __shfl_xor(yy, o, 64);
    if (lane == 0) yyw[wave] = yy;
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < 8; ++w) tot += yyw[w];
      p.yyp[(size_t)head * p.nch + chunk] = tot;
    }
  }
}

// Full symmetric Gram from the chunk partials, into an ld x ld matrix per head:
// fp32 (NNLS, ld = t) or fp64 + lambda I with identity padding (Cholesky, ld >= t).
template <typename OT>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ Gpart,
                                                          OT* __restrict__ G, int t, int ld,
                                                          int ntri, int nch, float lambda) {
  const int head = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)ld * ld) return;
  const int i = (int)(e / ld), j = (int)(e % ld);
  double v;
  if (i < t && j < t) {
    int ta = i / kGT, tb = j / kGT, ii = i % kGT, jj = j % kGT;
    if (ta < tb) {
      const int x = ta; ta = tb; tb = x;
      const int y = ii; ii = jj; jj = y;
    }
    const int tri = ta * (ta + 1) / 2 + tb;
    float acc = 0.f;
    for (int c = 0; c < nch; ++c)
      acc += Gpart[(((size_t)head * nch + c) * ntri + tri) * kGT * kGT + ii * kGT + jj];
    v = (double)acc + (i == j ? (double)lambda : 0.0);
  } else {
    v = (i == j) ? 1.0 : 0.0;
  }
  G[(size_t)head * ld * ld + (size_t)i * ld + j] = (OT)v;
}

// Vector part: rows < t summed over chunks, rows in [t, ld) zero. width = 1 (M^T b) or D.
template <typename OT>
__global__ __launch_bounds__(256) void vec_reduce_kernel(const float* __restrict__ Vpart,
                                                         OT* __restrict__ out, int t, int tpad,
                                                         int ld, int width, int nch) {
  const int head = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)ld * width) return;
  const int i = (int)(e / width), c0 = (int)(e % width);
  float acc = 0.f;
  if (i < t)
    for (int c = 0; c < nch; ++c)
      acc += Vpart[(((size_t)head * nch + c) * tpad + i) * width + c0];
  out[(size_t)head * ld * width + e] = (OT)acc;
}

// A query that sees no selected key with w > 0 has compacted log-normalizer -inf and a zero
// row of A. Its shift is made a huge finite number instead, so that every design entry
// 2^(x + bias - shift) of the row underflows to 0 with no per-entry test (x + bias is at
// most a few hundred, or -inf for w = 0).
__device__ __forceinline__ float value_shift(float u) { return u == -INFINITY ? 1e30f : u; }

// Per-query shift (log2 domain) and mass right-hand side.
//   mode 0: shift = lse * log2 e (relative mass design)
//   mode 1: shift = max_i lse_i * log2 e, target = 2^(lse_i log2 e - shift) (absolute)
//   mode 2: shift = m + log2 l of the biased compacted pass (value design)
__global__ __launch_bounds__(256) void shift_rows_kernel(const float* __restrict__ lse,
                                                         const float2* __restrict__ rowstat,
                                                         float* __restrict__ shift2, int n,
                                                         int mode) {
  const int head = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const size_t o = (size_t)head * n + i;
  if (mode == 0) {
    shift2[o] = lse[o] * kLog2e;
  } else {
    const float2 st = rowstat[o];
    shift2[o] = value_shift(st.x + st.y);
  }
}

__global__ __launch_bounds__(256) void shift_kernel(const float* __restrict__ lse,
                                                    const float2* __restrict__ rowstat,
                                                    float* __restrict__ shift2,
                                                    float* __restrict__ target, int n, int mode) {
  const int head = blockIdx.x;
  __shared__ float red[256];
  float c = -INFINITY;
  if (mode == 1) {
    for (int i = threadIdx.x; i < n; i += 256) c = fmaxf(c, lse[(size_t)head * n + i]);
    red[threadIdx.x] = c;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
      __syncthreads();
    }
    c = red[0] * kLog2e;
  }
  for (int i = threadIdx.x; i < n; i += 256) {
    const size_t o = (size_t)head * n + i;
    if (mode == 0) {
      shift2[o] = lse[o] * kLog2e;
    } else if (mode == 1) {
      shift2[o] = c;
      target[o] = ex2(lse[o] * kLog2e - c);
    } else {
      const float2 st = rowstat[o];
      shift2[o] = value_shift(st.x + st.y);
    }
  }
}

// ------------------------------------------------------------------------------------
// NNLS by accelerated projected gradient
// ------------------------------------------------------------------------------------
struct NnlsState {
  const float* G;   // [h, t, t]
  const float* hv;  // [h, t]
  float* dinv;      // [h, t]   1 / sqrt(G_jj) (0 for empty columns)
  float* hs;        // [h, t]   scaled right-hand side
  float* V;         // [h, 3, t] iterates (ring of three)
  float* X;         // [h, 2, t] step-size iteration vectors
  float* PN;        // [h, 2, nblk] step-size partials (largest ratio of a workgroup's rows)
  float2* P;        // [h, 2, nblk] (restart dot, gradient-mapping max) partials
  float2* init;     // [h, nblk] (max |hs|, non-finite flag) partials
  float2* kktp;     // [h, nblk] (largest KKT violation, largest |h|) partials, zero-filled
  int* bar;         // [h] barrier counters (zero before the first launch)
  int t, nblk;
  float lo, hi, tol;
};

// Outputs of a solve: w (optional), beta, status (optional), the relative KKT residual
// (optional) and the number of projected-gradient steps taken (optional), all per head.
struct NnlsOut {
  float* w; float* beta; int32_t* status; float* kkt; int32_t* iters;
};

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) s = fmaxf(s, red[i]);
  return s;
}

// Violation of the optimality conditions of min 1/2 w^T G w - h^T w over lo <= w <= hi at
// one coordinate, with g = (G w - h)_j: a free coordinate needs g = 0, one at the lower
// bound g >= 0, one at the upper bound g <= 0.
__device__ __forceinline__ float kkt_violation(float g, float w, float lo, float hi) {
  if (w <= lo) return fmaxf(-g, 0.f);
  if (w >= hi) return fmaxf(g, 0.f);
  return fabsf(g);
}

// One workgroup per head for t <= kNnlsSingle (thread i owns row i): Jacobi scaling
// v = sqrt(diag G) w, step 1/L with L the Collatz-Wielandt bound, momentum restarted when the
// step turns back, stop on the scaled gradient-mapping norm; all vectors in LDS. By
// symmetry thread i forms (G z)_i as sum_j G[j][i] z_j, so every step of j reads one row of
// G coalesced; G itself is staged in LDS when it fits (t <= 128), otherwise read from L2.
constexpr int kNnlsSingle = 256;
constexpr int kNnlsLdsG = 128;

__global__ __launch_bounds__(kNnlsSingle) void nnls_single_kernel(NnlsState s, int max_iter,
                                                                  NnlsOut o) {
  __shared__ float zs[kNnlsSingle];
  __shared__ float Gl[kNnlsLdsG * kNnlsLdsG];
  __shared__ float red[kNnlsSingle / 64], red2[kNnlsSingle / 64];
  const int head = blockIdx.x, t = s.t, i = threadIdx.x;
  const bool own = i < t;
  const float* Gg = s.G + (size_t)head * t * t;
  const bool in_lds = t <= kNnlsLdsG;
  if (in_lds)
    for (int e = i; e < t * t; e += kNnlsSingle) Gl[e] = Gg[e];
  __syncthreads();
  const float* Gs = in_lds ? Gl : Gg;

  auto bsum = [&](float v) {
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) v += __shfl_xor(v, o2, 64);
    __syncthreads();
    if ((i & 63) == 0) red[i >> 6] = v;
    __syncthreads();
    float r = 0.f;
    for (int w = 0; w < kNnlsSingle / 64; ++w) r += red[w];
    return r;
  };
  auto bmax2 = [&](float v) {
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) v = fmaxf(v, __shfl_xor(v, o2, 64));
    __syncthreads();
    if ((i & 63) == 0) red2[i >> 6] = v;
    __syncthreads();
    float r = red2[0];
    for (int w = 1; w < kNnlsSingle / 64; ++w) r = fmaxf(r, red2[w]);
    return r;
  };
  // sum_j G[j][i] zs[j] times f (zs = D^-1 x: the scaled product (D^-1 G D^-1 x)_i with
  // f = d_i; zs = w: (G w)_i with f = 1)
  auto row = [&](float f) {
    float acc = 0.f;
    if (own)
      for (int j = 0; j < t; ++j) acc += Gs[(size_t)j * t + i] * zs[j];
    return acc * f;
  };

  float di = 0.f, hsi = 0.f, gii = 0.f, h_i = 0.f;
  if (own) {
    gii = Gs[(size_t)i * t + i];
    h_i = s.hv[(size_t)head * t + i];
    di = gii > 0.f ? rsqrtf(gii) : 0.f;
    hsi = h_i * di;
  }
  const float bad = bmax2((own && (!isfinite(gii) || !isfinite(h_i))) ? 1.f : 0.f);
  const float hsmax = bmax2(fabsf(hsi));
  const float lo_i = di > 0.f ? s.lo / di : 0.f;
  const float hi_i = di > 0.f ? (isinf(s.hi) ? INFINITY : s.hi / di) : 0.f;

  // L: the Collatz-Wielandt bound on lambda_max(D^-1 G D^-1) (kCw)
  float u = own ? 1.f : 0.f, ratio = 0.f;
  for (int k = 0; k < kCw; ++k) {
    __syncthreads();
    zs[i] = u * di;
    __syncthreads();
    const float y = row(di);
    if (k + 1 < kCw) u = y + kCwShift * u;
    else ratio = u > 0.f ? y / u : 0.f;
  }
  const float L = kCwPad * bmax2(ratio) + 1e-30f;

  float v = lo_i, vp = lo_i, tk = 1.f, dot = 0.f, gm = INFINITY;
  const float thr = s.tol * fmaxf(hsmax, 1e-30f);
  int it = 0;
  for (; it < max_iter; ++it) {
    if (it > 0 && gm <= thr) break;
    const bool restart = dot > 0.f;
    const float tn = restart ? 1.f : 0.5f * (1.f + sqrtf(1.f + 4.f * tk * tk));
    const float mom = restart ? 0.f : (tk - 1.f) / tn;
    const float y = v + mom * (v - vp);
    __syncthreads();
    zs[i] = y * di;
    __syncthreads();
    const float g = row(di) - hsi;
    const float vn = di > 0.f ? fminf(fmaxf(y - g / L, lo_i), hi_i) : 0.f;
    dot = bsum(own ? (vn - v) * (y - vn) : 0.f);
    gm = bmax2(own ? fabsf(y - vn) * L : 0.f);
    vp = v;
    v = vn;
    tk = tn;
  }
  bool badw = false;
  float wi = 0.f;
  if (own) {
    float w = di > 0.f ? v * di : s.lo;
    wi = fminf(fmaxf(w, s.lo), s.hi);
    badw = !isfinite(wi);
    if (o.w) o.w[(size_t)head * t + i] = wi;
    o.beta[(size_t)head * t + i] = wi > 0.f ? logf(wi) : -INFINITY;
  }
  const float nbw = bmax2(badw ? 1.f : 0.f);
  if (o.kkt) {   // the KKT residual of the returned w on the system solved
    __syncthreads();
    zs[i] = wi;
    __syncthreads();
    const float viol = own ? kkt_violation(row(1.f) - h_i, wi, s.lo, s.hi) : 0.f;
    const float vmx = bmax2(viol);
    const float hmx = bmax2(fabsf(h_i));
    if (i == 0) o.kkt[head] = vmx / fmaxf(hmx, 1e-30f);
  }
  if (i == 0) {
    if (o.iters) o.iters[head] = it;
    if (o.status)
      o.status[head] = (gm > thr ? AM_HEAD_NNLS_BIT : 0) |
                       ((bad > 0.f || nbw > 0.f) ? AM_HEAD_NONFINITE_BIT : 0);
  }
}

// Multi-workgroup solver for t > kNnlsSingle: the same iteration, with the rows of each
// head split over P workgroups and a barrier among those P between steps. The launch
// checks that every workgroup of the grid can be resident at once (one per CU here), since
// the barrier waits on the others. A workgroup keeps its rows of G in LDS when they fit,
// else reads them from L2; the iterate vectors go through global memory. All workgroups
// of a head reduce the head's per-workgroup partials in the same fixed order, so they take
// the same decisions (momentum, convergence, exit) and pass the same number of barriers;
// heads are independent and stop on their own. Heads are solved in batches of at most
// ncu / 4 per launch (so every head gets at least four workgroups); a launch takes heads
// h0 .. h0 + Hb - 1.
constexpr size_t kNnlsCoopLds = 144 * 1024;   // dynamic LDS for G rows + the vector
constexpr int kNnlsSpin = 1 << 22;            // polls before a barrier wait gives up

// Device-scope loads and stores: they read and write the device's coherence point, not a
// copy in a CU's or an XCD's cache, so values that change while the workgroups of a head
// run go through these.
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier among the workgroups of one head: the m-th completes when the head's counter
// reaches m * P. Every wave first waits until its own stores have completed (vmcnt 0), and
// the workgroup's barrier orders all of its threads' writes before thread 0's counter add,
// which has release semantics at device (agent) scope; thread 0 polls the counter and ends
// its wait with an acquire fence at device scope, and the closing barrier orders the other
// threads' later reads after it. This is the language memory model's release/acquire
// pattern, so the data exchanged through memory is visible whatever caches it passed
// (on this chip the release writes back the XCD's L2 and the acquire invalidates it; about
// 10 us per barrier). The exchanged vectors are still written and read with device-scope
// accesses (st_dev, ld_dev). A wait longer than kNnlsSpin polls (about a second) marks the
// workgroup as timed out, after which it waits no more and stops.
__device__ __forceinline__ void head_barrier(int* ctr, int target, int* timed_out) {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0) only
  __syncthreads();
  if (threadIdx.x == 0 && !*timed_out) {
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kNnlsSpin) {
        *timed_out = 1;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void nnls_coop_kernel(NnlsState s, int h0, int Hb, int P,
                                                        int max_iter, int nlds, NnlsOut o) {
  extern __shared__ __align__(16) float smem[];
  __shared__ float red[4];
  __shared__ float2 pst[256];   // staged partials of the head's workgroups (P <= 256)
  __shared__ int timed_out;
  const int head = h0 + (int)blockIdx.x % Hb, part = (int)blockIdx.x / Hb, t = s.t;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rb = (t + P - 1) / P, r0 = min(t, part * rb), r1 = min(t, r0 + rb);
  if (tid == 0) timed_out = 0;
  float* xs = smem;
  float* Gs = smem + t;
  // this workgroup's rows of the extrapolated iterate and of the current one, formed with xs
  float* yr = Gs + (size_t)nlds * t;
  float* vr = yr + rb;
  const float* G = s.G + (size_t)head * t * t;
  // the first nlds of this workgroup's rows of G are held in LDS, the others read each step
  for (int e = tid; e < min(nlds, r1 - r0) * t; e += 256) Gs[e] = G[(size_t)r0 * t + e];
  // G_i . xs for this workgroup's row i, one wave (the sum over lanes by xor tree). With t a
  // multiple of 4, 16-byte reads: rows in LDS directly, rows in memory four reads in flight
  // per lane (latency-bound otherwise: a row is 64 dependent steps of one read each).
  auto row_dot = [&](int i) -> float {
    float acc = 0.f;
    if ((t & 3) == 0) {
      const int t4 = t >> 2;
      const float4* x4 = (const float4*)xs;
      auto dot4 = [](const float4 a, const float4 c) {
        return a.x * c.x + a.y * c.y + a.z * c.z + a.w * c.w;
      };
      if (i - r0 < nlds) {
        const float4* g4 = (const float4*)(Gs + (size_t)(i - r0) * t);
        for (int j = lane; j < t4; j += 64) acc += dot4(g4[j], x4[j]);
      } else {
        const float4* g4 = (const float4*)(G + (size_t)i * t);
        int j = lane;
        for (; j + 192 < t4; j += 256) {
          const float4 a0 = g4[j], a1 = g4[j + 64], a2 = g4[j + 128], a3 = g4[j + 192];
          acc += dot4(a0, x4[j]) + dot4(a1, x4[j + 64]) + dot4(a2, x4[j + 128]) +
                 dot4(a3, x4[j + 192]);
        }
        for (; j < t4; j += 64) acc += dot4(g4[j], x4[j]);
      }
    } else {
      const float* gr = i - r0 < nlds ? Gs + (size_t)(i - r0) * t : G + (size_t)i * t;
      for (int j = lane; j < t; j += 64) acc += gr[j] * xs[j];
    }
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) acc += __shfl_xor(acc, o2, 64);
    return acc;
  };
  float* dinv = s.dinv + (size_t)head * t;
  float* hs = s.hs + (size_t)head * t;
  const size_t ps = (size_t)s.nblk;   // partial slots per head and parity
  int* bar = s.bar + head;
  int nbar = 0;
  // G's diagonal scaling dinv and hs are written once before the first barrier and read
  // with ordinary loads after it; the vectors and partials that change per step go through
  // st_dev / ld_dev
  auto barrier = [&]() { head_barrier(bar, ++nbar * P, &timed_out); };
  // the head's P partials (float2) staged once, one load per thread
  auto stage = [&](const float2* src) {
    for (int b = tid; b < P; b += 256) {
      const float* q = (const float*)(src + b);
      pst[b] = make_float2(ld_dev(q), ld_dev(q + 1));
    }
    __syncthreads();
  };

  // prep: own rows
  float hm = 0.f, nb = 0.f;
  for (int j = r0 + tid; j < r1; j += 256) {
    const float g = G[(size_t)j * t + j];
    const float h = s.hv[(size_t)head * t + j];
    if (!isfinite(g) || !isfinite(h)) nb = 1.f;
    const float di = g > 0.f ? rsqrtf(g) : 0.f;
    dinv[j] = di;
    const float hsj = h * di;
    hs[j] = hsj;
    hm = fmaxf(hm, fabsf(hsj));
    const float v0 = di > 0.f ? s.lo / di : 0.f;
    s.V[((size_t)head * 3 + 0) * t + j] = v0;
    s.V[((size_t)head * 3 + 2) * t + j] = v0;
    s.X[((size_t)head * 2 + 0) * t + j] = 1.f;
  }
  hm = block_max(hm, red);
  nb = block_max(nb, red);
  if (tid == 0) {
    if (part == 0 && o.status) o.status[head] = 0;   // parts OR their flags in at the end
    s.init[(size_t)head * ps + part] = make_float2(hm, nb);
    s.P[((size_t)head * 2 + 0) * ps + part] = make_float2(0.f, INFINITY);
  }
  head_barrier(bar, ++nbar * P, &timed_out);
  stage(s.init + (size_t)head * ps);
  float hsmax = 0.f;
  bool bad = false;
  for (int b = 0; b < P; ++b) {
    hsmax = fmaxf(hsmax, pst[b].x);
    bad |= pst[b].y > 0.f;
  }
  __syncthreads();
  const float thr = s.tol * fmaxf(hsmax, 1e-30f);

  // L: the Collatz-Wielandt bound on lambda_max(D^-1 G D^-1) (kCw); the iterate u lives in
  // X (parity k & 1), the own rows' entries also in vr
  float pmax = 0.f;
  for (int k = 0; k < kCw && !timed_out; ++k) {
    const float* xin = s.X + ((size_t)head * 2 + (k & 1)) * t;
    float* xout = s.X + ((size_t)head * 2 + ((k + 1) & 1)) * t;
    for (int j = tid; j < t; j += 256) {
      const float u = ld_dev(xin + j);
      xs[j] = u * dinv[j];
      if (j >= r0 && j < r1) vr[j - r0] = u;
    }
    __syncthreads();
    for (int i = r0 + wave; i < r1; i += 4) {
      const float y = row_dot(i) * dinv[i];
      const float u = vr[i - r0];
      if (lane == 0) {
        if (k + 1 < kCw) st_dev(xout + i, y + kCwShift * u);
        else pmax = fmaxf(pmax, u > 0.f ? y / u : 0.f);
      }
    }
    if (k + 1 == kCw) {
      pmax = block_max(pmax, red);
      if (tid == 0) st_dev(s.PN + ((size_t)head * 2 + (kCw & 1)) * ps + part, pmax);
    }
    barrier();
  }
  float Lmax = 0.f;
  {
    float* pnl = (float*)pst;
    const float* pn = s.PN + ((size_t)head * 2 + (kCw & 1)) * ps;
    for (int b = tid; b < P; b += 256) pnl[b] = ld_dev(pn + b);
    __syncthreads();
    for (int b = 0; b < P; ++b) Lmax = fmaxf(Lmax, pnl[b]);
    __syncthreads();
  }
  const float L = kCwPad * Lmax + 1e-30f;

  // accelerated projected gradient; iterate v_k in ring slot k % 3
  float tk = 1.f, gm = INFINITY;
  int k = 0;
  for (; k < max_iter && !timed_out; ++k) {
    // this head's previous-step partials, reduced in a fixed order
    stage(s.P + ((size_t)head * 2 + (k & 1)) * ps);
    float dot = 0.f;
    gm = 0.f;
    for (int b = 0; b < P; ++b) {
      dot += pst[b].x;
      gm = fmaxf(gm, pst[b].y);
    }
    __syncthreads();
    if (k > 0 && gm <= thr) break;   // the same decision in every workgroup of the head
    const bool restart = dot > 0.f;
    const float tn = restart ? 1.f : 0.5f * (1.f + sqrtf(1.f + 4.f * tk * tk));
    const float mom = restart ? 0.f : (tk - 1.f) / tn;
    const float* vprev = s.V + ((size_t)head * 3 + (k + 2) % 3) * t;
    const float* vcur = s.V + ((size_t)head * 3 + k % 3) * t;
    float* vnext = s.V + ((size_t)head * 3 + (k + 1) % 3) * t;
    for (int j = tid; j < t; j += 256) {
      const float vc = ld_dev(vcur + j), vp = ld_dev(vprev + j);
      const float y = vc + mom * (vc - vp);
      xs[j] = y * dinv[j];
      if (j >= r0 && j < r1) {
        yr[j - r0] = y;
        vr[j - r0] = vc;
      }
    }
    __syncthreads();
    float pdot = 0.f, pgm = 0.f;
    for (int i = r0 + wave; i < r1; i += 4) {
      const float acc = row_dot(i);
      const float di = dinv[i];
      const float vc = vr[i - r0], y = yr[i - r0];
      const float g = acc * di - hs[i];
      float vn = 0.f;
      if (di > 0.f) {
        const float lo = s.lo / di;
        const float hi = isinf(s.hi) ? INFINITY : s.hi / di;
        vn = fminf(fmaxf(y - g / L, lo), hi);
      }
      if (lane == 0) {
        st_dev(vnext + i, vn);
        pdot += (vn - vc) * (y - vn);
        pgm = fmaxf(pgm, fabsf(y - vn) * L);
      }
    }
    pdot = block_sum(pdot, red);
    pgm = block_max(pgm, red);
    if (tid == 0) {
      float* q = (float*)(s.P + ((size_t)head * 2 + ((k + 1) & 1)) * ps + part);
      st_dev(q, pdot);
      st_dev(q + 1, pgm);
    }
    tk = tn;
    barrier();
  }
  if (k == max_iter && !timed_out) {   // the last step's norm was not examined yet
    stage(s.P + ((size_t)head * 2 + (k & 1)) * ps);
    gm = 0.f;
    for (int b = 0; b < P; ++b) gm = fmaxf(gm, pst[b].y);
  }
  // the answer is v_k, whose rows were all written before the last barrier: every
  // workgroup forms the whole returned w (for the KKT product) and writes its own rows
  const float* v = s.V + ((size_t)head * 3 + k % 3) * t;
  for (int j = tid; j < t; j += 256) {
    const float di = dinv[j];
    const float w = di > 0.f ? ld_dev(v + j) * di : s.lo;
    xs[j] = fminf(fmaxf(w, s.lo), s.hi);
  }
  __syncthreads();
  float nbw = 0.f;
  for (int j = r0 + tid; j < r1; j += 256) {
    const float w = xs[j];
    if (!isfinite(w)) nbw = 1.f;
    if (o.w) o.w[(size_t)head * t + j] = w;
    o.beta[(size_t)head * t + j] = w > 0.f ? logf(w) : -INFINITY;
  }
  nbw = block_max(nbw, red);
  if (o.kkt) {   // KKT residual of the returned w on the system solved, own rows
    float pv = 0.f, ph = 0.f;
    for (int i = r0 + wave; i < r1; i += 4) {
      const float acc = row_dot(i);
      const float hi = s.hv[(size_t)head * t + i];
      if (lane == 0) {
        pv = fmaxf(pv, kkt_violation(acc - hi, xs[i], s.lo, s.hi));
        ph = fmaxf(ph, fabsf(hi));
      }
    }
    pv = block_max(pv, red);
    ph = block_max(ph, red);
    if (tid == 0) s.kktp[(size_t)head * ps + part] = make_float2(pv, ph);
  }
  if (tid == 0 && part == 0 && o.iters) o.iters[head] = k;
  if (tid == 0 && o.status) {
    const int bits = ((timed_out || k == 0 || !(gm <= thr)) ? AM_HEAD_NNLS_BIT : 0) |
                     ((bad || nbw > 0.f) ? AM_HEAD_NONFINITE_BIT : 0) |
                     (timed_out ? AM_HEAD_TIMEOUT_BIT : 0);
    if (bits) atomicOr(&o.status[head], bits);
  }
}

// kkt[h] = the largest violation over the head's workgroups / the largest |h_j|
__global__ __launch_bounds__(64) void nnls_kkt_final_kernel(const float2* __restrict__ kktp,
                                                            int nblk, float* __restrict__ kkt) {
  const int head = blockIdx.x;
  float v = 0.f, hm = 0.f;
  for (int b = threadIdx.x; b < nblk; b += 64) {
    const float2 p = kktp[(size_t)head * nblk + b];
    v = fmaxf(v, p.x);
    hm = fmaxf(hm, p.y);
  }
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) {
    v = fmaxf(v, __shfl_xor(v, o2, 64));
    hm = fmaxf(hm, __shfl_xor(hm, o2, 64));
  }
  if (threadIdx.x == 0) kkt[head] = v / fmaxf(hm, 1e-30f);
}

// ------------------------------------------------------------------------------------
// Blocked fp64 Cholesky and triangular solves on A [h, ld, ld], R [h, ld, D]
// ------------------------------------------------------------------------------------
// 64-row fp64 blocks staged through LDS for the block kernels. A loader issues all of
// its global loads (16-byte, one per register pair) before it writes any of them to LDS, so
// a block costs one memory latency rather than one per element.
// A pivot below kPivRel times its column's diagonal entry before the factorization (or not
// positive) marks the system as singular at the precision of the solve: AM_HEAD_CHOL_PIVOT.
// With the ridge lambda > 0 every pivot is at least lambda, far above this for any
// diagonal the designs produce (at most n <= 2^30 plus lambda).
constexpr double kPivRel = 0x1p-40;
constexpr int kLdp = kNB + 1;   // LDS row pitch (odd: column reads by 16 rows hit 16 banks)
// The workgroup bodies below take their LDS from the kernel that runs them, so kernels that
// combine two kinds of workgroup need only the larger of their footprints: two 64 x 65 tiles
// (and the 64 pivot slots of the diagonal factorization).
typedef double LdsTile[kNB][kLdp];

template <int W>
struct BlockRegs {
  static constexpr int N = kNB * W / 2 / 256;   // double2 per thread (256 threads)
  double2 r[N];
  // src[u][v], 0 <= u < 64, 0 <= v < W, row stride `stride` doubles
  __device__ __forceinline__ void load(const double* src, size_t stride, int tid) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int e = (tid + 256 * q) * 2, u = e / W, v = e % W;
      r[q] = *(const double2*)&src[(size_t)u * stride + v];
    }
  }
  // dst[u][v] = src[u][v]  (TR = false)  or  dst[v][u] = src[u][v]  (TR = true)
  template <bool TR, int P>
  __device__ __forceinline__ void store(double (*dst)[P], int tid) const {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int e = (tid + 256 * q) * 2, u = e / W, v = e % W;
      if (TR) {
        dst[v][u] = r[q].x;
        dst[v + 1][u] = r[q].y;
      } else {
        dst[u][v] = r[q].x;
        dst[u][v + 1] = r[q].y;
      }
    }
  }
};

// Factor the diagonal block kb in place (lower) and store its inverse in Linv[h, nb, 64, 64].
// The 64 x 64 block is split 2 x 2 into 32 x 32 blocks:
//   L11 = chol(A11), L21 = A21 L11^-T, L22 = chol(A22 - L21 L21^T),
//   L^-1 = [[L11^-1, 0], [-L22^-1 (L21 L11^-1), L22^-1]].
// Each 32 x 32 factorization (with its inverse) runs on one wave, as symmetric Gaussian
// elimination without pivoting. Lanes 0..31 (A half) hold the rows of A; lanes 32..63
// (X half) hold the columns of I, which become those of L^-1 by forward substitution.
// Step k: the trailing block stays symmetric, so its column k, which lanes r >= k post as
// their own a_rk, is also pivot row k: one 8-byte store per lane, read back as broadcasts.
// With u that column and p = u_k (the k-th pivot, L_kk^2), both halves apply
//   own_j -= (own_k / p) u_j  for j > k,
// for the A half on rows r > k only: the elimination of row r, and for the X half the
// substitution x_j -= L_jk (x_k / L_kk) with L_jk = u_j / sqrt(p), whose division by L_kk
// is deferred. Afterwards a_rr in row r of the A half is the r-th
// pivot, and the entries j < r it posted, unchanged since, are L(r, j) sqrt(u_jj); the X
// half ends with L^-1(j, c) = x_c(j) / sqrt(u_jj).
// Steps are unrolled (compile-time k) so each touches only the entries j > k that change.
template <int K>
__device__ __forceinline__ void chol32_step(double (&a)[32], double* col, int r, int half,
                                            bool& bad) {
  // lanes that post nothing write a slot of col[32..63] nobody reads: a store without a
  // branch around it (a branch per step more than doubles the registers the steps take)
  col[(!half && r >= K) ? r : 32 + r] = a[K];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // every read of the step is issued before any arithmetic waits on one
  constexpr int J0 = K & ~1;   // the pair holding entry K
  double u[32];
#pragma unroll
  for (int j = J0; j < 32; j += 2) {
    const double2 v = *(const double2*)&col[j];
    u[j] = v.x;
    u[j + 1] = v.y;
  }
  __builtin_amdgcn_sched_barrier(0);
  double p = u[K];
  if (!(p > 0.0)) {
    bad = true;
    p = 1e-300;
  }
  // 1 / p from the hardware estimate and two Newton steps (p > 0 here)
  double ip = __builtin_amdgcn_rcp(p);
  ip = __builtin_fma(ip, __builtin_fma(-p, ip, 1.0), ip);
  ip = __builtin_fma(ip, __builtin_fma(-p, ip, 1.0), ip);
  const double m = (half || r > K) ? a[K] * ip : 0.0;
#pragma unroll
  for (int j = K + 1; j < 32; ++j) a[j] -= m * u[j];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int K>
__device__ __forceinline__ void chol32_steps(double (&a)[32], double* col, int r, int half,
                                             bool& bad) {
  if constexpr (K < 32) {
    chol32_step<K>(a, col, r, half, bad);
    chol32_steps<K + 1>(a, col, r, half, bad);
  }
}

// col: 64 doubles of LDS (the posted column and, above it, the slots of lanes not posting);
// thr: the smallest pivot lane r accepts for its row (see kPivRel)
__device__ __forceinline__ void chol32_wave(double (*L)[kNB + 1], double (*Li)[kNB + 1], int o,
                                            double* col, bool& bad, double thr) {
  const int lane = threadIdx.x & 63, r = lane & 31, half = lane >> 5;
  double a[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const double v = L[o + (j <= r ? r : j)][o + (j <= r ? j : r)];   // lower triangle
    a[j] = half ? (j == r ? 1.0 : 0.0) : v;
  }
  chol32_steps<0>(a, col, r, half, bad);
  // Lane r of the A half posted a_rj at step j < r and left it unchanged since, and a_rr is
  // the r-th pivot: L(r, j) = a_rj / sqrt(u_jj) for j <= r. It posts 1 / sqrt(u_rr) (its own
  // pivot has a run-time register index: select).
  {
    double dr = a[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) dr = j == r ? a[j] : dr;
    if (!(dr > thr) && !half) bad = true;
    if (!(dr > 0.0)) dr = 1e-300;
    col[r + 32 * half] = 1.0 / sqrt(dr);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const double2 v = *(const double2*)&col[j];
    a[j] *= v.x;
    a[j + 1] *= v.y;
  }
  if (half == 0) {
#pragma unroll
    for (int j = 0; j < 32; ++j) L[o + r][o + j] = j <= r ? a[j] : 0.0;
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) Li[o + j][o + r] = j >= r ? a[j] : 0.0;
  }
}

// out[i][j] (i, j < 32; thread (tid / 8, tid % 8 + 8 m)) = sum_k P[i][k] Q[k][j] or
// P[i][k] Q[j][k] (TQ)
template <bool TQ>
__device__ __forceinline__ void mm32(double (&out)[4], const double (*P)[kNB + 1], int pr, int pc,
                                     const double (*Q)[kNB + 1], int qr, int qc, int tid) {
  const int i = tid >> 3, j0 = tid & 7;
#pragma unroll
  for (int m = 0; m < 4; ++m) out[m] = 0.0;
#pragma unroll 8
  for (int k = 0; k < 32; ++k) {
    const double pv = P[pr + i][pc + k];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      out[m] += pv * (TQ ? Q[qr + j0 + 8 * m][qc + k] : Q[qr + k][qc + j0 + 8 * m]);
  }
}

// The diagonal block kb of one head. LDS: L (the block, then its factor), Li (the inverse of
// the factor; while L22 is factored its upper right quadrant, zero in the result, holds
// T = L21 L11^-1), piv (the wave-level eliminations' pivot columns), badf.
__device__ __forceinline__ void chol_diag_body(double* A, double* Linv, const double* Dg, int ld,
                                               int kb, int nb, int32_t* status, int head,
                                               LdsTile& L, LdsTile& Li, double* piv, int& badf) {
  const int tid = threadIdx.x, wave = tid >> 6;
  // pivot thresholds of the rows lane r of wave 0 eliminates (rows r and 32 + r of the block)
  const double* dgb = Dg + (size_t)head * ld + kb * kNB + (tid & 31);
  const double thr0 = wave == 0 ? kPivRel * dgb[0] : 0.0;
  const double thr1 = wave == 0 ? kPivRel * dgb[32] : 0.0;
  double* Ah = A + (size_t)head * ld * ld + (size_t)kb * kNB * ld + kb * kNB;
  {
    BlockRegs<kNB> ra;
    ra.load(Ah, ld, tid);
    ra.store<false>(L, tid);
  }
  for (int e = tid; e < kNB * kNB; e += 256) Li[e >> 6][e & 63] = 0.0;
  if (tid == 0) badf = 0;
  __syncthreads();
  bool bad = false;
  if (wave == 0) chol32_wave(L, Li, 0, piv, bad, thr0);
  __syncthreads();
  const int i = tid >> 3, j0 = tid & 7;
  double acc[4];
  // L21 = A21 L11^-T: L21[i][j] = sum_k A21[i][k] Li11[j][k]
  mm32<true>(acc, L, 32, 0, Li, 0, 0, tid);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 4; ++m) L[32 + i][j0 + 8 * m] = acc[m];
  __syncthreads();
  // Schur complement A22 - L21 L21^T
  mm32<true>(acc, L, 32, 0, L, 32, 0, tid);
#pragma unroll
  for (int m = 0; m < 4; ++m) L[32 + i][32 + j0 + 8 * m] -= acc[m];
  __syncthreads();
  // wave 0: L22 and its inverse; the other waves meanwhile T = L21 L11^-1
  if (wave == 0) {
    chol32_wave(L, Li, 32, piv, bad, thr1);
  } else {
    for (int e = tid - 64; e < 32 * 32; e += 192) {
      const int ii = e >> 5, jj = e & 31;
      double v = 0.0;
      for (int k = jj; k < 32; ++k) v += L[32 + ii][k] * Li[k][jj];
      Li[ii][32 + jj] = v;   // T
    }
  }
  __syncthreads();
  // Li21 = -L22^-1 T
  mm32<false>(acc, Li, 32, 32, Li, 0, 32, tid);
#pragma unroll
  for (int m = 0; m < 4; ++m) Li[32 + i][j0 + 8 * m] = -acc[m];
  if (bad) badf = 1;
  __syncthreads();
  double* Lo = Linv + ((size_t)head * nb + kb) * kNB * kNB;
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int r = e >> 6, c = e & 63;
    Ah[(size_t)r * ld + c] = c <= r ? L[r][c] : 0.0;
    Lo[e] = c <= r ? Li[r][c] : 0.0;
  }
  if (tid == 0 && badf && status) atomicOr(&status[head], AM_HEAD_CHOL_BIT);
}

__global__ __launch_bounds__(256) void chol_diag_kernel(double* A, double* Linv, const double* Dg,
                                                        int ld, int kb, int nb, int32_t* status) {
  __shared__ LdsTile s0, s1;
  __shared__ __align__(16) double piv[64];
  __shared__ int badf;
  chol_diag_body(A, Linv, Dg, ld, kb, nb, status, blockIdx.x, s0, s1, piv, badf);
}

// Dg[h, i] = A[h, i, i] before the factorization (the reference of the pivot test)
__global__ __launch_bounds__(256) void diag_copy_kernel(const double* __restrict__ A,
                                                        double* __restrict__ Dg, int ld) {
  const int head = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i < ld) Dg[(size_t)head * ld + i] = A[(size_t)head * ld * ld + (size_t)i * ld + i];
}


// acc[a][b] = sum_k P[ti + 16 a][k] Q[tj + 16 b][k] over k < 64, for ti = tid / 16,
// tj = tid % 16 (a 64 x 64 product of two row-major LDS blocks, 4 x 4 per thread).
__device__ __forceinline__ void mm_rows64(double (&acc)[4][4], const double (*P)[kLdp],
                                          const double (*Q)[kLdp], int tid) {
  const int ti = tid >> 4, tj = tid & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 4
  for (int k = 0; k < kNB; ++k) {
    double p[4], q[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) p[a] = P[ti + 16 * a][k];
#pragma unroll
    for (int b = 0; b < 4; ++b) q[b] = Q[tj + 16 * b][k];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] += p[a] * q[b];
  }
}

// out[r][c] = sum_k M[r][k] X[k][c] for a 64 x 32 slice: rows tr, tr + 32 (tr = tid / 8),
// columns tc + 8 b (tc = tid % 8).
__device__ __forceinline__ void mm_slice(double (&acc)[2][4], const double (*M)[kLdp],
                                         const double (*X)[33], int tid) {
  const int tr = tid >> 3, tc = tid & 7;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 4
  for (int k = 0; k < kNB; ++k) {
    const double m0 = M[tr][k], m1 = M[tr + 32][k];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const double xv = X[k][tc + 8 * b];
      acc[0][b] += m0 * xv;
      acc[1][b] += m1 * xv;
    }
  }
}

__device__ __forceinline__ double (*as_slice(LdsTile& t))[33] { return (double (*)[33])&t[0][0]; }

// L_ik = A_ik Linv_kk^T for block row ib > kb: (A_ik Linv^T)[u][v] = sum_k A_ik[u][k] Linv[v][k].
__device__ __forceinline__ void chol_panel_body(double* A, const double* Linv, int ld, int kb,
                                                int nb, int ib, int head, LdsTile& x,
                                                LdsTile& li) {
  const int tid = threadIdx.x;
  double* Ai = A + (size_t)head * ld * ld + (size_t)ib * kNB * ld + kb * kNB;
  BlockRegs<kNB> ra, rl;
  ra.load(Ai, ld, tid);
  rl.load(Linv + ((size_t)head * nb + kb) * kNB * kNB, kNB, tid);
  ra.store<false>(x, tid);
  rl.store<false>(li, tid);
  __syncthreads();
  double acc[4][4];
  mm_rows64(acc, x, li, tid);
  const int ti = tid >> 4, tj = tid & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Ai[(size_t)(ti + 16 * a) * ld + tj + 16 * b] = acc[a][b];
}

// A_ij -= L_ik L_jk^T for the lower block pair (ib, jb), kb < jb <= ib.
__device__ __forceinline__ void chol_update_body(double* A, int ld, int kb, int ib, int jb,
                                                 int head, LdsTile& li, LdsTile& lj) {
  const int tid = threadIdx.x;
  double* Ah = A + (size_t)head * ld * ld;
  double* Aij = Ah + (size_t)ib * kNB * ld + jb * kNB;
  BlockRegs<kNB> ri, rj;
  ri.load(Ah + (size_t)ib * kNB * ld + kb * kNB, ld, tid);
  rj.load(Ah + (size_t)jb * kNB * ld + kb * kNB, ld, tid);
  const int ti = tid >> 4, tj = tid & 15;
  double cur[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) cur[a][b] = Aij[(size_t)(ti + 16 * a) * ld + tj + 16 * b];
  ri.store<false>(li, tid);
  rj.store<false>(lj, tid);
  __syncthreads();
  double acc[4][4];
  mm_rows64(acc, li, lj, tid);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Aij[(size_t)(ti + 16 * a) * ld + tj + 16 * b] = cur[a][b] - acc[a][b];
}

// R_kb <- Linv_kk R_kb (forward) or Linv_kk^T R_kb (backward) for the 32 columns from c0.
__device__ __forceinline__ void trsm_diag_body(double* R, const double* Linv, int ld, int D,
                                               int kb, int nb, int trans, int head, int c0,
                                               LdsTile& m, LdsTile& xt) {
  const int tid = threadIdx.x;
  double (*x)[33] = as_slice(xt);
  double* Rh = R + ((size_t)head * ld + (size_t)kb * kNB) * D + c0;
  BlockRegs<kNB> rm;
  BlockRegs<32> rx;
  rm.load(Linv + ((size_t)head * nb + kb) * kNB * kNB, kNB, tid);
  rx.load(Rh, D, tid);
  if (trans) rm.store<true>(m, tid);
  else rm.store<false>(m, tid);
  rx.store<false>(x, tid);
  __syncthreads();
  double acc[2][4];
  mm_slice(acc, m, x, tid);
  const int tr = tid >> 3, tc = tid & 7;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Rh[(size_t)(tr + 32 * a) * D + tc + 8 * b] = acc[a][b];
}

// forward: R_ib -= L_{ib,kb} R_kb (ib > kb);  backward: R_ib -= L_{kb,ib}^T R_kb (ib < kb);
// for the 32 columns from c0.
__device__ __forceinline__ void trsm_update_body(double* R, const double* A, int ld, int D,
                                                 int kb, int ib, int trans, int head, int c0,
                                                 LdsTile& m, LdsTile& xt) {
  const int tid = threadIdx.x;
  double (*x)[33] = as_slice(xt);
  const double* Ah = A + (size_t)head * ld * ld;
  double* Rh = R + (size_t)head * ld * D + c0;
  BlockRegs<kNB> rm;
  BlockRegs<32> rx;
  if (trans) rm.load(Ah + (size_t)kb * kNB * ld + ib * kNB, ld, tid);
  else rm.load(Ah + (size_t)ib * kNB * ld + kb * kNB, ld, tid);
  rx.load(Rh + (size_t)kb * kNB * D, D, tid);
  const int tr = tid >> 3, tc = tid & 7;
  double* Ri = Rh + (size_t)ib * kNB * D;
  double cur[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) cur[a][b] = Ri[(size_t)(tr + 32 * a) * D + tc + 8 * b];
  if (trans) rm.store<true>(m, tid);
  else rm.store<false>(m, tid);
  rx.store<false>(x, tid);
  __syncthreads();
  double acc[2][4];
  mm_slice(acc, m, x, tid);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Ri[(size_t)(tr + 32 * a) * D + tc + 8 * b] = cur[a][b] - acc[a][b];
}

// Step kb of the factorization, after the diagonal block: workgroups x < m (m = nb - kb - 1)
// form the panel L_ik, the next D / 32 the forward solve's Z_kb = Linv_kk R_kb, whose inputs
// (R_kb after the updates of steps < kb, and Linv_kk) are complete at this point.
__global__ __launch_bounds__(256) void chol_panel_kernel(double* A, const double* Linv,
                                                         double* R, int ld, int D, int kb,
                                                         int nb) {
  __shared__ LdsTile s0, s1;
  const int head = blockIdx.y, m = nb - kb - 1;
  if ((int)blockIdx.x < m) chol_panel_body(A, Linv, ld, kb, nb, kb + 1 + blockIdx.x, head, s0, s1);
  else trsm_diag_body(R, Linv, ld, D, kb, nb, 0, head, (blockIdx.x - m) * 32, s0, s1);
}

// Step kb's trailing update: workgroups x < m (m + 1) / 2 update the lower block pairs
// A_ij -= L_ik L_jk^T (kb < j <= i), the next m D / 32 the forward solve's R_i -= L_ik Z_kb.
// Workgroup 0 takes the pair (kb + 1, kb + 1) and then factors that block, the next step's
// diagonal block, while the others finish the update (lookahead: no launch of its own).
__global__ __launch_bounds__(256) void chol_update_kernel(double* A, double* R, double* Linv,
                                                          const double* Dg, int32_t* status,
                                                          int ld, int D, int kb, int nb) {
  __shared__ LdsTile s0, s1;
  __shared__ __align__(16) double piv[64];
  __shared__ int badf;
  const int head = blockIdx.y, m = nb - kb - 1, ntri = m * (m + 1) / 2;
  if ((int)blockIdx.x < ntri) {
    int a0, b0;
    tri_index(blockIdx.x, a0, b0);
    chol_update_body(A, ld, kb, kb + 1 + a0, kb + 1 + b0, head, s0, s1);
    if (blockIdx.x == 0) {   // a0 = b0 = 0: the block just written (same workgroup)
      __syncthreads();
      chol_diag_body(A, Linv, Dg, ld, kb + 1, nb, status, head, s0, s1, piv, badf);
    }
  } else {
    const int e = blockIdx.x - ntri, ns = D / 32;
    trsm_update_body(R, A, ld, D, kb, kb + 1 + e / ns, 0, head, (e % ns) * 32, s0, s1);
  }
}

// The backward solve, L^T C = Z, one block row at a time: R_kb <- Linv_kk^T R_kb ...
__global__ __launch_bounds__(256) void trsm_back_diag_kernel(double* R, const double* Linv,
                                                             int ld, int D, int kb, int nb) {
  __shared__ LdsTile s0, s1;
  trsm_diag_body(R, Linv, ld, D, kb, nb, 1, blockIdx.y, blockIdx.x * 32, s0, s1);
}

// ... then R_i -= L_{kb,i}^T R_kb for every block row i < kb. The workgroup of row kb - 1,
// the only one that touches it, then forms the next step's R_{kb-1} <- Linv^T R_{kb-1} itself
// (lookahead: the next diagonal product needs no launch of its own).
__global__ __launch_bounds__(256) void trsm_back_update_kernel(double* R, const double* A,
                                                               const double* Linv, int ld, int D,
                                                               int kb, int nb) {
  __shared__ LdsTile s0, s1;
  const int head = blockIdx.z, c0 = blockIdx.y * 32;
  trsm_update_body(R, A, ld, D, kb, blockIdx.x, 1, head, c0, s0, s1);
  if ((int)blockIdx.x == kb - 1) {
    __syncthreads();   // the rows just written are read back by this workgroup
    trsm_diag_body(R, Linv, ld, D, kb - 1, nb, 1, head, c0, s0, s1);
  }
}

// The whole backward solve in one launch, for factors of at most kBsMaxLd rows and few heads
// (the launcher's choice, below): each
// workgroup owns kBsW columns of one head's right-hand side, holds them in LDS from the
// first block step to the last and runs every step itself, so no two workgroups share
// data. Step kb: Z_kb <- Linv_kk^T Z_kb (one entry per thread, Linv_kk staged in LDS and
// fetched one step ahead), then Z_j -= sum_b L(kb*64 + b, j) Z_kb(b) for every row j < 64 kb
// (one row per thread; the row's column of the block row of L streamed from memory,
// coalesced along j, in four batches of 16 loads, each batch issued before the previous
// one's products). The broadcast reads of Z_kb from LDS bound the row loop, hence few
// columns per workgroup and many workgroups. The sums run over b in the same order, and
// each row's updates land in the same order, as in the per-step launches.
constexpr int kBsW = 4;
constexpr int kBsMaxLd = 1024;
__global__ __launch_bounds__(512) void trsm_back_cols_kernel(double* R, const double* A,
                                                             const double* Linv, int ld, int D,
                                                             int nb, int H) {
  __shared__ __align__(16) double zs[kBsMaxLd * kBsW];
  __shared__ __align__(16) double li[kNB * kNB];
  __shared__ __align__(16) double xs[kNB * kBsW];
  const int head = blockIdx.x % H, c0 = (blockIdx.x / H) * kBsW;
  const int tid = threadIdx.x;
  double* Rh = R + (size_t)head * ld * D + c0;
  const double* Ah = A + (size_t)head * ld * ld;
  for (int e = tid; e < ld * (kBsW / 2); e += 512) {
    const int row = e / (kBsW / 2), q = e % (kBsW / 2);
    *(double2*)&zs[row * kBsW + 2 * q] = *(const double2*)&Rh[(size_t)row * D + 2 * q];
  }
  const double2* Lh = (const double2*)(Linv + (size_t)head * nb * kNB * kNB);
  constexpr int kLi2 = kNB * kNB / 2;   // 16-byte pieces per Linv block
  double2 lin0 = Lh[(size_t)(nb - 1) * kLi2 + tid], lin1 = Lh[(size_t)(nb - 1) * kLi2 + tid + 512];
  double2 lin2 = Lh[(size_t)(nb - 1) * kLi2 + tid + 1024];
  double2 lin3 = Lh[(size_t)(nb - 1) * kLi2 + tid + 1536];
  for (int kb = nb - 1; kb >= 0; --kb) {
    ((double2*)li)[tid] = lin0;
    ((double2*)li)[tid + 512] = lin1;
    ((double2*)li)[tid + 1024] = lin2;
    ((double2*)li)[tid + 1536] = lin3;
    __syncthreads();   // (and the previous step's row updates are complete)
    if (tid < kNB * kBsW) {
      const int a = tid / kBsW, c = tid % kBsW;
      double acc = 0.0;
#pragma unroll 16
      for (int b = 0; b < kNB; ++b) acc += li[b * kNB + a] * zs[(kb * kNB + b) * kBsW + c];
      xs[a * kBsW + c] = acc;
    }
    __syncthreads();   // every read of Z_kb is done; X is complete
    if (tid < kNB * kBsW) zs[(kb * kNB + tid / kBsW) * kBsW + tid % kBsW] = xs[tid];
    if (kb > 0) {   // (after the barrier, whose fence would wait for the loads)
      const double2* Lk = Lh + (size_t)(kb - 1) * kLi2;
      lin0 = Lk[tid];
      lin1 = Lk[tid + 512];
      lin2 = Lk[tid + 1024];
      lin3 = Lk[tid + 1536];
    }
    const double* P = Ah + (size_t)kb * kNB * ld;
    // (at most two rows per thread: ld <= 1024; unrolled, so no per-row address streams)
#pragma unroll
    for (int rr = 0; rr < kBsMaxLd / 512; ++rr) {
      const int j = tid + 512 * rr;
      if (j >= kb * kNB) break;
      double acc[kBsW];
#pragma unroll
      for (int c = 0; c < kBsW; ++c) acc[c] = 0.0;
      double la[16], lb[16];
#define AM_BS_LOAD(buf, b0)                                                  \
  _Pragma("unroll") for (int i = 0; i < 16; ++i) buf[i] = (P + (size_t)((b0) + i) * ld)[(unsigned)j]; \
  __builtin_amdgcn_sched_barrier(0);
#define AM_BS_FMA(buf, b0)                                                   \
  _Pragma("unroll") for (int i = 0; i < 16; ++i) {                           \
    _Pragma("unroll") for (int q = 0; q < kBsW / 2; ++q) {                   \
      const double2 v = *(const double2*)&xs[((b0) + i) * kBsW + 2 * q];     \
      acc[2 * q] += buf[i] * v.x;                                            \
      acc[2 * q + 1] += buf[i] * v.y;                                        \
    }                                                                        \
  }                                                                          \
  __builtin_amdgcn_sched_barrier(0);
      AM_BS_LOAD(la, 0)
      AM_BS_LOAD(lb, 16)
      AM_BS_FMA(la, 0)
      AM_BS_LOAD(la, 32)
      AM_BS_FMA(lb, 16)
      AM_BS_LOAD(lb, 48)
      AM_BS_FMA(la, 32)
      AM_BS_FMA(lb, 48)
#undef AM_BS_LOAD
#undef AM_BS_FMA
#pragma unroll
      for (int c = 0; c < kBsW; ++c) zs[j * kBsW + c] -= acc[c];
    }
    // keeps the next step's store of the prefetched Linv below the row updates (hoisted
    // above them, it would wait for the prefetch at once)
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  for (int e = tid; e < ld * (kBsW / 2); e += 512) {
    const int row = e / (kBsW / 2), q = e % (kBsW / 2);
    *(double2*)&Rh[(size_t)row * D + 2 * q] = *(const double2*)&zs[row * kBsW + 2 * q];
  }
}

// C_v = float(C); with cpart set, the workgroup also writes the fp64 partial sums of
// C . R0 and C . C over its 256 entries to cpart[head, block] (for the output residual)
__global__ __launch_bounds__(256) void store_cv_kernel(const double* R, const double* R0,
                                                       float* Cv, int t, int ld, int D,
                                                       int32_t* status, double2* cpart) {
  __shared__ double r1[256], r2[256];
  const int head = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  double cr = 0.0, cc = 0.0;
  if (e < (long long)t * D) {
    const double v = R[(size_t)head * ld * D + e];
    Cv[(size_t)head * t * D + e] = (float)v;
    if (!isfinite(v) && status) atomicOr(&status[head], AM_HEAD_NONFINITE_BIT);
    if (cpart) {
      cr = v * R0[(size_t)head * ld * D + e];
      cc = v * v;
    }
  }
  if (!cpart) return;   // (uniform over the workgroup)
  r1[threadIdx.x] = cr;
  r2[threadIdx.x] = cc;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) {
      r1[threadIdx.x] += r1[threadIdx.x + s2];
      r2[threadIdx.x] += r2[threadIdx.x + s2];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) cpart[(size_t)head * gridDim.x + blockIdx.x] = make_double2(r1[0], r2[0]);
}

// ------------------------------------------------------------------------------------
// residual reductions (one workgroup per head, fixed order)
// ------------------------------------------------------------------------------------
// Two-level, fixed-order reductions: kResBlk workgroups per head write partial sums
// (fp64) that one workgroup per head then adds in order.
constexpr int kResBlk = 64;

// mass: per-query (Z_cmp / Z - b)^2 with Z_cmp / Z = 2^(lc - shift) from the biased pass
__global__ __launch_bounds__(256) void mass_resid_part_kernel(const float2* __restrict__ rowstat_cmp,
                                                              const float* __restrict__ shift2,
                                                              const float* __restrict__ target,
                                                              double2* __restrict__ part, int n) {
  __shared__ double red[256];
  const int head = blockIdx.y;
  double acc = 0.0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += kResBlk * 256) {
    const size_t o = (size_t)head * n + i;
    const float2 st = rowstat_cmp[o];
    const float b = target ? target[o] : 1.f;
    const float z = (st.y == -INFINITY) ? 0.f : ex2((st.x - shift2[o]) + st.y);
    acc += (double)(z - b) * (double)(z - b);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) red[threadIdx.x] += red[threadIdx.x + s2];
    __syncthreads();
  }
  if (threadIdx.x == 0)
    part[(size_t)head * kResBlk + blockIdx.x] = make_double2(red[0], blockIdx.x == 0 ? (double)n : 0.0);
}

__global__ __launch_bounds__(256) void out_resid_part_kernel(const float2* __restrict__ rowres,
                                                             double2* __restrict__ part, int n) {
  __shared__ double re[256], ry[256];
  const int head = blockIdx.y;
  double e = 0.0, y = 0.0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += kResBlk * 256) {
    const float2 v = rowres[(size_t)head * n + i];
    e += v.x;
    y += v.y;
  }
  re[threadIdx.x] = e;
  ry[threadIdx.x] = y;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) {
      re[threadIdx.x] += re[threadIdx.x + s2];
      ry[threadIdx.x] += ry[threadIdx.x + s2];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(size_t)head * kResBlk + blockIdx.x] = make_double2(re[0], ry[0]);
}

// out[h] = sum(x) / sum(y) over the partials (mass: y holds n, so this is the mean)
__global__ void resid_final_kernel(const double2* __restrict__ part, float* __restrict__ out,
                                   int heads) {
  const int head = blockIdx.x * 64 + threadIdx.x;
  if (head >= heads) return;
  double x = 0.0, y = 0.0;
  for (int b = 0; b < kResBlk; ++b) {
    const double2 v = part[(size_t)head * kResBlk + b];
    x += v.x;
    y += v.y;
  }
  out[head] = (float)(y > 0.0 ? x / y : 0.0);
}

// Sums of squares of Y [h, count] (count a multiple of 4) over kResBlk contiguous slices per
// head, each summed in a fixed order in fp64
__global__ __launch_bounds__(256) void sumsq_part_kernel(const float* __restrict__ Y,
                                                         double* __restrict__ part,
                                                         long long count) {
  __shared__ double red[256];
  const int head = blockIdx.y;
  const long long per = ((count + kResBlk - 1) / kResBlk + 3) / 4 * 4;
  const long long a0 = min(count, (long long)blockIdx.x * per), a1 = min(count, a0 + per);
  const float* y = Y + (size_t)head * count;
  double acc = 0.0;
  for (long long e = a0 + 4 * (long long)threadIdx.x; e < a1; e += 1024) {
    const float4 v = *(const float4*)(y + e);
    acc += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (threadIdx.x < s2) red[threadIdx.x] += red[threadIdx.x + s2];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(size_t)head * kResBlk + blockIdx.x] = red[0];
}

// The ridge fit's output residual ||A C - Y||^2 / ||Y||^2 without another pass over the
// queries: with C solving (A^T A + lambda I) C = A^T Y, A^T A C = A^T Y - lambda C, so
// ||A C - Y||^2 = ||Y||^2 - <C, A^T Y> - lambda ||C||^2. yyp holds nyy partials of ||Y||^2 per
// head, cpart ncp partials of (<C, A^T Y>, ||C||^2); each is summed in a fixed order. A
// rounding-level negative value is reported as 0.
__global__ __launch_bounds__(256) void resid_values_final_kernel(const double* __restrict__ yyp,
                                                                 int nyy,
                                                                 const double2* __restrict__ cpart,
                                                                 int ncp, float lambda,
                                                                 float* __restrict__ out) {
  __shared__ double r0[256], r1[256], r2[256];
  const int head = blockIdx.x, tid = threadIdx.x;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0;
  for (int i = tid; i < nyy; i += 256) a0 += yyp[(size_t)head * nyy + i];
  for (int i = tid; i < ncp; i += 256) {
    const double2 v = cpart[(size_t)head * ncp + i];
    a1 += v.x;
    a2 += v.y;
  }
  r0[tid] = a0;
  r1[tid] = a1;
  r2[tid] = a2;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (tid < s2) {
      r0[tid] += r0[tid + s2];
      r1[tid] += r1[tid + s2];
      r2[tid] += r2[tid + s2];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double yy = r0[0];
    const double res = yy > 0.0 ? (yy - r1[0] - (double)lambda * r2[0]) / yy : 0.0;
    out[head] = (float)fmax(res, 0.0);
  }
}

__global__ __launch_bounds__(256) void copy_f64_kernel(const double* __restrict__ src,
                                                       double* __restrict__ dst, long long count) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < count) dst[i] = src[i];
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ------------------------------------------------------------------------------------
// host side: workspace plans and launch sequences
// ------------------------------------------------------------------------------------
static int gram_ntile(int t) { return (t + kGT - 1) / kGT; }
static int gram_ntri(int t) { const int a = gram_ntile(t); return a * (a + 1) / 2; }
static int gram_nch(int heads, int n, int t) {
  const int ntri = gram_ntri(t);
  int want = (2048 + heads * ntri - 1) / (heads * ntri);
  int maxc = n / 2048;
  if (maxc < 1) maxc = 1;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  return want;
}
static int gram_chunk(int n, int nch) { return round_up((n + nch - 1) / nch, kGQ); }

struct Carve {
  char* base; size_t off;
  template <typename X> X* take(size_t count) {
    X* p = base ? (X*)(base + off) : nullptr;   // sizing only: no address
    off = align_up(off + count * sizeof(X));
    return p;
  }
};

struct BetaPlan {
  float* shift2; float* target; float* Gpart; float* hpart; float* G; float* hv;
  float* dinv; float* hs; float* V; float* X; float* PN; float2* P; float2* init; float2* kktp;
  int* bar; int2* tstat; float2* rowstat_cmp; double2* part; int32_t* status;
  SyrkBuffers sy;
  size_t bytes;
};

static BetaPlan plan_beta(char* base, int64_t heads, int64_t n, int64_t t, int64_t d) {
  (void)d;
  Carve c{base, 0};
  const int tpad = gram_ntile((int)t) * kGT;
  const int nch = gram_nch((int)heads, (int)n, (int)t);
  const int ntri = gram_ntri((int)t);
  const int nblk = ((int)t + kRB - 1) / kRB;
  BetaPlan p;
  p.rowstat_cmp = c.take<float2>(heads * n);   // first in both plans: shared with the value fit
  p.part = c.take<double2>(heads * kResBlk);
  p.shift2 = c.take<float>(heads * n);
  p.target = c.take<float>(heads * n);
  if (syrk_path((int)t)) {
    p.Gpart = p.hpart = nullptr;
    p.sy = syrk_carve(base, c.off, heads, n, t, d, false);
  } else {
    p.sy = SyrkBuffers{nullptr, nullptr, nullptr};
    p.Gpart = c.take<float>((size_t)heads * nch * ntri * kGT * kGT);
    p.hpart = c.take<float>((size_t)heads * nch * tpad);
  }
  p.G = c.take<float>((size_t)heads * t * t);
  p.hv = c.take<float>(heads * t);
  p.dinv = c.take<float>(heads * t);
  p.hs = c.take<float>(heads * t);
  p.V = c.take<float>(heads * 3 * t);
  p.X = c.take<float>(heads * 2 * t);
  p.PN = c.take<float>(heads * 2 * nblk);
  p.P = c.take<float2>(heads * 2 * nblk);
  p.init = c.take<float2>(heads * nblk);
  p.kktp = c.take<float2>(heads * nblk);
  p.bar = c.take<int>(heads);
  p.tstat = (int2*)c.take<char>(cmp_tstat_bytes(heads, t));
  p.status = c.take<int32_t>(heads);
  p.bytes = c.off;
  return p;
}

struct ValuePlan {
  float2* rowstat_cmp; double2* part; float* shift2; float* Gpart; float* Rpart; double* A;
  double* R; double* R0; double* Linv; double* Dg; double* yyp; double2* cpart; int2* tstat;
  int32_t* status; int nyy, ncp;
  SyrkBuffers sy;
  size_t bytes;
};

static int chol_ld(int t) { return round_up(t, kNB); }

static ValuePlan plan_values(char* base, int64_t heads, int64_t n, int64_t t, int64_t d) {
  Carve c{base, 0};
  const int tpad = gram_ntile((int)t) * kGT;
  const int nch = gram_nch((int)heads, (int)n, (int)t);
  const int ntri = gram_ntri((int)t);
  const int ld = chol_ld((int)t);
  ValuePlan p;
  p.rowstat_cmp = c.take<float2>(heads * n);
  p.part = c.take<double2>(heads * kResBlk);
  p.shift2 = c.take<float>(heads * n);
  if (syrk_path((int)t)) {
    p.Gpart = p.Rpart = nullptr;
    p.sy = syrk_carve(base, c.off, heads, n, t, d, true);
  } else {
    p.sy = SyrkBuffers{nullptr, nullptr, nullptr};
    p.Gpart = c.take<float>((size_t)heads * nch * ntri * kGT * kGT);
    p.Rpart = c.take<float>((size_t)heads * nch * tpad * d);
  }
  p.A = c.take<double>((size_t)heads * ld * ld);
  p.R = c.take<double>((size_t)heads * ld * d);
  p.Linv = c.take<double>((size_t)heads * (ld / kNB) * kNB * kNB);
  p.Dg = c.take<double>((size_t)heads * ld);
  p.R0 = c.take<double>((size_t)heads * ld * d);
  // partials of ||Y||^2: one per 64 queries from the Y^T rows kernel, else kResBlk slices
  p.nyy = syrk_path((int)t) ? syrk_yy_blocks(heads, n, t, d)
                            : std::max(kResBlk, gram_nch((int)heads, (int)n, (int)t));
  p.yyp = c.take<double>((size_t)heads * p.nyy);
  p.ncp = (int)((t * d + 255) / 256);
  p.cpart = c.take<double2>((size_t)heads * p.ncp);
  p.tstat = (int2*)c.take<char>(cmp_tstat_bytes(heads, t));
  p.status = c.take<int32_t>(heads);
  p.bytes = c.off;
  return p;
}

size_t fit_beta_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d) {
  return plan_beta(nullptr, heads, n, t, d).bytes;
}
size_t fit_values_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d) {
  return plan_values(nullptr, heads, n, t, d).bytes;
}

template <typename T, int D, bool VALUE>
static void launch_gram(const GramParams& gp, int heads, hipStream_t st) {
  hipLaunchKernelGGL((gram_kernel<T, D, VALUE>), dim3(gp.ntri, gp.nch, heads), dim3(512), 0, st, gp);
}

static void launch_gram_any(const GramParams& gp, int heads, int d, bool bf, bool value,
                            hipStream_t st) {
  if (bf) {
    if (d == 128) { if (value) launch_gram<bf16, 128, true>(gp, heads, st); else launch_gram<bf16, 128, false>(gp, heads, st); }
    else { if (value) launch_gram<bf16, 64, true>(gp, heads, st); else launch_gram<bf16, 64, false>(gp, heads, st); }
  } else {
    if (d == 128) { if (value) launch_gram<float, 128, true>(gp, heads, st); else launch_gram<float, 128, false>(gp, heads, st); }
    else { if (value) launch_gram<float, 64, true>(gp, heads, st); else launch_gram<float, 64, false>(gp, heads, st); }
  }
}

static unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

int device_cu_count() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return ncu;
}

hipError_t launch_all_resident(const void* fn, dim3 grid, dim3 block, void** args, size_t shmem,
                               hipStream_t st) {
  const int ncu = device_cu_count();
  int per_cu = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, fn, (int)(block.x * block.y * block.z), shmem);
  if (e != hipSuccess) return e;
  if ((long long)per_cu * ncu < (long long)grid.x * grid.y * grid.z)
    return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, grid, block, args, shmem, st);
}

// A batch of hb heads on the multi-workgroup solver: P workgroups per head (at most one per
// CU for the batch, at most one per 16 rows, at most 256), rb rows each, of which the
// first nlds are held in LDS (the vector, two row slices and as many rows of G as fit).
NnlsParts nnls_parts(int hb, int t, int ncu) {
  NnlsParts p;
  p.P = std::max(1, std::min(std::min(ncu / std::max(hb, 1), (t + kRB - 1) / kRB), 256));
  p.rb = (t + p.P - 1) / p.P;
  const size_t lds_f = kNnlsCoopLds / sizeof(float), fixed = (size_t)t + 2 * (size_t)p.rb;
  p.nlds = lds_f > fixed ? (int)std::min<size_t>((size_t)p.rb, (lds_f - fixed) / t) : 0;
  p.shmem = (fixed + (size_t)p.nlds * t) * sizeof(float);
  return p;
}

NnlsSchedule nnls_schedule(int heads, int t, int ncu) {
  NnlsSchedule sc;
  if (t <= kNnlsSingle) {
    sc.heads_per_launch = heads;
    sc.launches = 1;
    sc.first = NnlsParts{1, t, t <= kNnlsLdsG ? t : 0, 0};
    return sc;
  }
  // every head of a batch gets at least four workgroups (CUs)
  sc.heads_per_launch = std::max(1, std::min(heads, ncu / 4));
  sc.launches = (heads + sc.heads_per_launch - 1) / sc.heads_per_launch;
  sc.first = nnls_parts(sc.heads_per_launch, t, ncu);
  return sc;
}

hipError_t launch_fit_beta(const FitArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n, t = a.t, d = a.d;
  BetaPlan pl = plan_beta((char*)a.ws, H, n, t, d);
  int32_t* status = a.head_status ? a.head_status : pl.status;
  const int tpad = gram_ntile(t) * kGT, nch = gram_nch(H, n, t), ntri = gram_ntri(t);
  // row shifts and right-hand side
  if (a.absolute)
    hipLaunchKernelGGL(shift_kernel, dim3(H), dim3(256), 0, st, a.lse, (const float2*)nullptr,
                       pl.shift2, pl.target, n, 1);
  else
    hipLaunchKernelGGL(shift_rows_kernel, dim3(cdiv(n, 256), H), dim3(256), 0, st, a.lse,
                       (const float2*)nullptr, pl.shift2, n, 0);
  if (syrk_path(t)) {
    SyrkGramArgs sa;
    sa.Q = a.Q; sa.Ck = a.Ck; sa.keypos = a.idx; sa.bias = nullptr; sa.shift2 = pl.shift2;
    sa.target = a.absolute ? pl.target : nullptr; sa.Y = nullptr; sa.buf = pl.sy;
    sa.Gf = pl.G; sa.hv = pl.hv; sa.Gd = nullptr; sa.R = nullptr;
    sa.heads = H; sa.n = n; sa.t = t; sa.d = d; sa.group = a.group; sa.ld = t;
    sa.causal = a.causal; sa.bf16 = a.bf16; sa.value = false;
    sa.c2 = a.scale * kLog2e; sa.lambda = 0.f; sa.stream = st;
    const hipError_t e = launch_syrk_gram(sa);
    if (e != hipSuccess) return e;
  } else {
    GramParams gp;
    gp.Q = a.Q; gp.Ck = a.Ck; gp.keypos = a.idx; gp.bias = nullptr;
    gp.shift2 = pl.shift2; gp.target = a.absolute ? pl.target : nullptr; gp.Y = nullptr;
    gp.Gpart = pl.Gpart; gp.Vpart = pl.hpart;
    gp.n = n; gp.t = t; gp.tpad = tpad; gp.group = a.group; gp.ntri = ntri; gp.nch = nch;
    gp.chunk = gram_chunk(n, nch); gp.causal = a.causal; gp.c2 = a.scale * kLog2e;
    launch_gram_any(gp, H, d, a.bf16, false, st);
    hipLaunchKernelGGL((gram_reduce_kernel<float>), dim3(cdiv((long long)t * t, 256), H),
                       dim3(256), 0, st, pl.Gpart, pl.G, t, t, ntri, nch, 0.f);
    hipLaunchKernelGGL((vec_reduce_kernel<float>), dim3(cdiv(t, 256), H), dim3(256), 0, st,
                       pl.hpart, pl.hv, t, tpad, t, 1, nch);
  }
  // NNLS
  NnlsState s;
  s.G = pl.G; s.hv = pl.hv; s.dinv = pl.dinv; s.hs = pl.hs; s.V = pl.V; s.X = pl.X;
  s.PN = pl.PN; s.P = pl.P; s.init = pl.init; s.kktp = pl.kktp; s.bar = pl.bar;
  s.t = t; s.nblk = (t + kRB - 1) / kRB;
  s.lo = a.w_lo; s.hi = a.w_hi; s.tol = a.tol;
  NnlsOut o{a.w, a.beta, status, a.kkt, a.iters};
  if (t <= kNnlsSingle) {
    hipLaunchKernelGGL(nnls_single_kernel, dim3(H), dim3(kNnlsSingle), 0, st, s, a.max_iter, o);
  } else {
    const int ncu = device_cu_count();
    if (ncu < 1) return hipErrorInvalidDevice;
    hipLaunchKernelGGL(zero_i32_kernel, dim3(cdiv(H, 256)), dim3(256), 0, st, pl.bar, H);
    if (a.kkt)
      hipLaunchKernelGGL(zero_i32_kernel, dim3(cdiv((long long)H * s.nblk * 2, 256)), dim3(256), 0,
                         st, (int32_t*)pl.kktp, H * s.nblk * 2);
    const NnlsSchedule sc = nnls_schedule(H, t, ncu);
    int max_iter = a.max_iter;
    for (int h0 = 0; h0 < H; h0 += sc.heads_per_launch) {
      int hb = std::min(sc.heads_per_launch, H - h0);
      const NnlsParts pp = nnls_parts(hb, t, ncu);
      int P = pp.P, nlds = pp.nlds;
      void* args[] = {&s, &h0, &hb, &P, &max_iter, &nlds, &o};
      (void)hipFuncSetAttribute((const void*)nnls_coop_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)pp.shmem);
      const hipError_t e = launch_all_resident((const void*)nnls_coop_kernel, dim3(hb * P),
                                               dim3(256), args, pp.shmem, st);
      if (e != hipSuccess) return e;
    }
    if (a.kkt)
      hipLaunchKernelGGL(nnls_kkt_final_kernel, dim3(H), dim3(64), 0, st,
                         (const float2*)pl.kktp, s.nblk, a.kkt);
  }
  // mass residual from the biased compacted pass: Z_cmp / Z = 2^(lc - lse2); the pass's row
  // statistics are also what the value fit needs, so they are kept when asked for
  if (a.mass_resid || a.keep_cmp_stats) {
    CmpAttnArgs ca;
    ca.Q = a.Q; ca.Ck = a.Ck; ca.Cv = nullptr; ca.bias = a.beta; ca.keypos = a.idx; ca.Y = nullptr;
    ca.Vt = nullptr; ca.tstat = pl.tstat;
    ca.lse = nullptr; ca.rowstat = pl.rowstat_cmp; ca.O = nullptr; ca.rowres = nullptr;
    ca.heads = H; ca.n = n; ca.t = t; ca.d = d; ca.group = a.group; ca.causal = a.causal;
    ca.bf16 = a.bf16; ca.scale = a.scale; ca.stream = st;
    hipError_t e = launch_cmp_attention(ca);
    if (e != hipSuccess) return e;
    if (a.mass_resid) {
      hipLaunchKernelGGL(mass_resid_part_kernel, dim3(kResBlk, H), dim3(256), 0, st,
                         pl.rowstat_cmp, pl.shift2, a.absolute ? pl.target : nullptr, pl.part, n);
      hipLaunchKernelGGL(resid_final_kernel, dim3(cdiv(H, 64)), dim3(64), 0, st,
                         (const double2*)pl.part, a.mass_resid, H);
    }
  }
  return hipGetLastError();
}

hipError_t launch_fit_values(const FitArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n, t = a.t, d = a.d;
  ValuePlan pl = plan_values((char*)a.ws, H, n, t, d);
  int32_t* status = a.head_status ? a.head_status : pl.status;
  if (!a.head_status || !a.keep_status)
    hipLaunchKernelGGL(zero_i32_kernel, dim3(cdiv(H, 256)), dim3(256), 0, st, status, H);
  const int tpad = gram_ntile(t) * kGT, nch = gram_nch(H, n, t), ntri = gram_ntri(t);
  const int ld = chol_ld(t), nb = ld / kNB;
  // compacted log-normalizer per query (biased pass, statistics only)
  CmpAttnArgs ca;
  ca.Q = a.Q; ca.Ck = a.Ck; ca.Cv = nullptr; ca.bias = a.beta_in; ca.keypos = a.idx; ca.Y = nullptr;
  ca.Vt = nullptr; ca.tstat = pl.tstat;
  ca.lse = nullptr; ca.rowstat = pl.rowstat_cmp; ca.O = nullptr; ca.rowres = nullptr;
  ca.heads = H; ca.n = n; ca.t = t; ca.d = d; ca.group = a.group; ca.causal = a.causal;
  ca.bf16 = a.bf16; ca.scale = a.scale; ca.stream = st;
  hipError_t e = hipSuccess;
  if (!a.have_cmp_stats) {   // else the beta fit left them at the start of the workspace
    e = launch_cmp_attention(ca);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(shift_rows_kernel, dim3(cdiv(n, 256), H), dim3(256), 0, st,
                     (const float*)nullptr, (const float2*)pl.rowstat_cmp, pl.shift2, n, 2);
  if (syrk_path(t)) {
    SyrkGramArgs sa;
    sa.Q = a.Q; sa.Ck = a.Ck; sa.keypos = a.idx; sa.bias = a.beta_in; sa.shift2 = pl.shift2;
    sa.target = nullptr; sa.Y = a.O; sa.buf = pl.sy; sa.yyp = a.out_resid ? pl.yyp : nullptr;
    sa.Gf = nullptr; sa.hv = nullptr; sa.Gd = pl.A; sa.R = pl.R;
    sa.heads = H; sa.n = n; sa.t = t; sa.d = d; sa.group = a.group; sa.ld = ld;
    sa.causal = a.causal; sa.bf16 = a.bf16; sa.value = true;
    sa.c2 = a.scale * kLog2e; sa.lambda = a.lambda; sa.stream = st;
    e = launch_syrk_gram(sa);
    if (e != hipSuccess) return e;
  } else {
    GramParams gp;
    gp.Q = a.Q; gp.Ck = a.Ck; gp.keypos = a.idx; gp.bias = a.beta_in;
    gp.shift2 = pl.shift2; gp.target = nullptr; gp.Y = a.O;
    gp.Gpart = pl.Gpart; gp.Vpart = pl.Rpart;
    gp.n = n; gp.t = t; gp.tpad = tpad; gp.group = a.group; gp.ntri = ntri; gp.nch = nch;
    gp.chunk = gram_chunk(n, nch); gp.causal = a.causal; gp.c2 = a.scale * kLog2e;
    gp.yyp = (a.out_resid && !a.causal) ? pl.yyp : nullptr;
    launch_gram_any(gp, H, d, a.bf16, true, st);
    hipLaunchKernelGGL((gram_reduce_kernel<double>), dim3(cdiv((long long)ld * ld, 256), H),
                       dim3(256), 0, st, pl.Gpart, pl.A, t, ld, ntri, nch, a.lambda);
    hipLaunchKernelGGL((vec_reduce_kernel<double>), dim3(cdiv((long long)ld * d, 256), H),
                       dim3(256), 0, st, pl.Rpart, pl.R, t, tpad, ld, d, nch);
  }
  // the right-hand side A^T Y is kept for the residual (the solve overwrites R with C)
  if (a.out_resid)
    hipLaunchKernelGGL(copy_f64_kernel, dim3(cdiv((long long)H * ld * d, 256)), dim3(256), 0, st,
                       (const double*)pl.R, pl.R0, (long long)H * ld * d);
  // Cholesky, with the forward solve L Z = R folded into each step's panel and update
  // launches; then the backward solve L^T C = Z
  // (the diagonal blocks after the first are factored inside the previous step's update)
  hipLaunchKernelGGL(diag_copy_kernel, dim3(cdiv(ld, 256), H), dim3(256), 0, st,
                     (const double*)pl.A, pl.Dg, ld);
  hipLaunchKernelGGL(chol_diag_kernel, dim3(H), dim3(256), 0, st, pl.A, pl.Linv,
                     (const double*)pl.Dg, ld, 0, nb, status);
  for (int kb = 0; kb < nb; ++kb) {
    const int m = nb - kb - 1;
    hipLaunchKernelGGL(chol_panel_kernel, dim3(m + d / 32, H), dim3(256), 0, st, pl.A,
                       (const double*)pl.Linv, pl.R, ld, d, kb, nb);
    if (m > 0)
      hipLaunchKernelGGL(chol_update_kernel, dim3(m * (m + 1) / 2 + m * (d / 32), H), dim3(256),
                         0, st, pl.A, pl.R, pl.Linv, (const double*)pl.Dg, status, ld, d, kb,
                         nb);
  }
  // One launch pays while its workgroups fill the device about once: with few heads the
  // per-step launches are a chain of short dependent launches, but with many heads every one
  // of its workgroups re-reads its head's factor (8x the traffic of the per-step form, whose
  // workgroups each take 32 columns), and the per-step launches are the faster form
  const int ncu = device_cu_count();
  const long long nbw = (long long)H * (d / kBsW);
  if (ld <= kBsMaxLd && d % kBsW == 0 && nb >= 2 && ncu > 0 && nbw <= 2LL * ncu) {
    // one launch: each workgroup runs every step for its columns
    hipLaunchKernelGGL(trsm_back_cols_kernel, dim3(H * (d / kBsW)), dim3(512), 0, st, pl.R,
                       (const double*)pl.A, (const double*)pl.Linv, ld, d, nb, H);
  } else {
    // one launch per step (each update launch also forms the next block row's diagonal
    // product)
    hipLaunchKernelGGL(trsm_back_diag_kernel, dim3(d / 32, H), dim3(256), 0, st, pl.R,
                       (const double*)pl.Linv, ld, d, nb - 1, nb);
    for (int kb = nb - 1; kb > 0; --kb)
      hipLaunchKernelGGL(trsm_back_update_kernel, dim3(kb, d / 32, H), dim3(256), 0, st, pl.R,
                         (const double*)pl.A, (const double*)pl.Linv, ld, d, kb, nb);
  }
  hipLaunchKernelGGL(store_cv_kernel, dim3(pl.ncp, H), dim3(256), 0, st, (const double*)pl.R,
                     (const double*)pl.R0, a.Cv, t, ld, d, status,
                     a.out_resid ? pl.cpart : nullptr);
  if (a.out_resid) {
    // ||Y||^2: on the stored-design path the Y^T rows kernel has summed it (one partial per
    // 64 queries), without the causal mask the Gram kernel's tile 0 (one per chunk); else a
    // pass over Y (kResBlk slices)
    int nyy = pl.nyy;
    if (!syrk_path(t)) {
      if (a.causal) {
        hipLaunchKernelGGL(sumsq_part_kernel, dim3(kResBlk, H), dim3(256), 0, st, a.O, pl.yyp,
                           (long long)n * d);
        nyy = kResBlk;
      } else {
        nyy = nch;
      }
    }
    hipLaunchKernelGGL(resid_values_final_kernel, dim3(H), dim3(256), 0, st,
                       (const double*)pl.yyp, nyy, (const double2*)pl.cpart, pl.ncp, a.lambda,
                       a.out_resid);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Fast variants of the "Compaction" blog (no fits) and evaluation on other queries
// ------------------------------------------------------------------------------------
// Uniform redistribution (§Choosing beta): with m_j = (1/n) sum_i exp(s_i,c_j) over the
// queries that see c_j and Delta = (1/n) sum_i Z_i - sum_j m_j, beta_j = log(1 +
// Delta / (t m_j)). Every mass is taken on the common scale e^-C, C = max_i lse_i, which
// cancels in beta; m_j comes from the column passes in log form (log2 m_j = kmax_j +
// log2 kmean_j), and beta_j = logaddexp(log(Delta / t), log m_j) - log m_j, so keys of
// mass far below the scale still get a finite bias. Delta, a mass by definition, is
// clamped at 0 (a negative value is rounding).

// per head: shift2 = C log2(e) and zsum = sum_i exp(lse_i - C); one workgroup of 1024
// threads per head, each thread streaming every 1024th row with four independent loads in
// flight (the reduction order is fixed)
__global__ __launch_bounds__(1024) void redist_prep_kernel(const float* __restrict__ lse, int n,
                                                           float* __restrict__ shift2,
                                                           double* __restrict__ zsum) {
  __shared__ float red[16];
  __shared__ double dred[1024];
  const int head = blockIdx.x, tid = threadIdx.x;
  const float* l = lse + (size_t)head * n;
  float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int i = tid; i < n; i += 4096) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 1024 * u < n) m4[u] = fmaxf(m4[u], l[i + 1024 * u]);
  }
  const float mx = block_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])), red);
  const float c2 = mx == -INFINITY ? 0.f : mx * kLog2e;
  double a4[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = tid; i < n; i += 4096) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 1024 * u < n) a4[u] += (double)ex2(__builtin_fmaf(l[i + 1024 * u], kLog2e, -c2));
  }
  dred[tid] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
  __syncthreads();
  for (int s2 = 512; s2 > 0; s2 >>= 1) {
    if (tid < s2) dred[tid] += dred[tid + s2];
    __syncthreads();
  }
  if (tid == 0) {
    shift2[head] = c2;
    zsum[head] = dred[0];
  }
}

// beta (and w = e^beta) from the per-key masses in log form; a key that no query sees
// (log mass -inf) gets +inf when there is mass to hand out, else 0
__global__ __launch_bounds__(256) void redist_beta_kernel(const float* __restrict__ kmax,
                                                          const float* __restrict__ kmean,
                                                          const double* __restrict__ zsum, int n,
                                                          int t, float* __restrict__ beta,
                                                          float* __restrict__ w) {
  __shared__ double dred[256];
  const int head = blockIdx.x, tid = threadIdx.x;
  const size_t o = (size_t)head * t;
  auto lg2m = [&](int j) {   // log2 m_j on the common scale
    const double mx = (double)kmax[o + j], me = (double)kmean[o + j];
    return (mx == -INFINITY || !(me > 0.0)) ? -(double)INFINITY : mx + log2(me);
  };
  double acc = 0.0;
  for (int j = tid; j < t; j += 256) acc += exp2(lg2m(j));
  dred[tid] = acc;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) {
    if (tid < s2) dred[tid] += dred[tid + s2];
    __syncthreads();
  }
  const double delta = fmax(zsum[head] / (double)n - dred[0], 0.0);
  const double la = delta > 0.0 ? log2(delta / (double)t) : -(double)INFINITY;
  for (int j = tid; j < t; j += 256) {
    const double lm = lg2m(j);
    double b2;   // beta in log2 units
    if (la == -INFINITY) b2 = 0.0;
    else if (lm == -INFINITY) b2 = INFINITY;
    else {
      const double hi = fmax(la, lm), lo = fmin(la, lm);
      b2 = hi + log2(1.0 + exp2(lo - hi)) - lm;
    }
    const double b = b2 * 0.69314718055994530942;
    beta[o + j] = (float)b;
    if (w) w[o + j] = (float)exp2(b2);
  }
}

// Direct values (§Choosing C_v): C_v[h, j] = V[h, idx[h, j]] in f32. One thread per 4 values.
template <typename T>
__global__ __launch_bounds__(256) void gather_f32_kernel(const T* __restrict__ V,
                                                         const int32_t* __restrict__ idx,
                                                         float* __restrict__ Cv, int Tk, int t,
                                                         int d) {
  const int head = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int d4 = d / 4;
  if (e >= (long long)t * d4) return;
  const int j = (int)(e / d4), c = (int)(e - (long long)j * d4) * 4;
  const int src = min(max(idx[(size_t)head * t + j], 0), Tk - 1);
  const T* v = V + ((size_t)head * Tk + src) * d + c;
  float4 o;
  o.x = (float)v[0];
  o.y = (float)v[1];
  o.z = (float)v[2];
  o.w = (float)v[3];
  *(float4*)(Cv + ((size_t)head * t + j) * d + c) = o;
}

struct FastPlan {
  float* shift2h; double* zsum; float* kmax; float* kmean; float* kpart;   // redistribution
  float2* rowstat_cmp; float* shift2; double2* part;     // mass residual
  int2* tstat; void* Vt; float2* rowres;                 // output residual
  float* lse; float* O; void* tws;                       // evaluation: targets on the queries
  size_t bytes;
};

static FastPlan plan_fast(char* base, int64_t heads, int64_t n, int64_t t, int64_t d,
                          int esize, int64_t T_eval) {
  Carve c{base, 0};
  FastPlan p;
  p.shift2h = c.take<float>(heads);
  p.zsum = c.take<double>(heads);
  p.kmax = c.take<float>(heads * t);
  p.kmean = c.take<float>(heads * t);
  p.kpart = (float*)c.take<char>(key_mass_part_bytes(heads, n, t));
  p.rowstat_cmp = c.take<float2>(heads * n);
  p.shift2 = c.take<float>(heads * n);
  p.part = c.take<double2>(heads * kResBlk);
  p.tstat = (int2*)c.take<char>(cmp_tstat_bytes(heads, t));
  p.Vt = c.take<char>(cmp_vt_bytes(heads, t, d, esize));
  p.rowres = c.take<float2>(heads * n);
  p.lse = p.O = nullptr;
  p.tws = nullptr;
  if (T_eval > 0) {
    p.lse = c.take<float>(heads * n);
    p.O = c.take<float>((size_t)heads * n * d);
    p.tws = c.take<char>(targets_ws_bytes(heads, n, T_eval, d, esize));
  }
  p.bytes = c.off;
  return p;
}

size_t fast_ws_bytes(int64_t heads, int64_t n, int64_t t, int64_t d, int esize, int64_t T_eval) {
  return plan_fast(nullptr, heads, n, t, d, esize, T_eval).bytes;
}

// mass residual mean_i (Z_cmp,i / Z_i - 1)^2 of (idx, beta) on queries with log-normalizers lse
static hipError_t mass_residual(const FitArgs& a, const float* lse, const float* beta,
                                const FastPlan& pl, float* out) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n;
  hipLaunchKernelGGL(shift_rows_kernel, dim3(cdiv(n, 256), H), dim3(256), 0, st, lse,
                     (const float2*)nullptr, pl.shift2, n, 0);
  CmpAttnArgs ca;
  ca.Q = a.Q; ca.Ck = a.Ck; ca.Cv = nullptr; ca.bias = beta; ca.keypos = a.idx; ca.Y = nullptr;
  ca.Vt = nullptr; ca.tstat = pl.tstat;
  ca.lse = nullptr; ca.rowstat = pl.rowstat_cmp; ca.O = nullptr; ca.rowres = nullptr;
  ca.heads = H; ca.n = n; ca.t = a.t; ca.d = a.d; ca.group = a.group; ca.causal = a.causal;
  ca.bf16 = a.bf16; ca.scale = a.scale; ca.stream = st;
  const hipError_t e = launch_cmp_attention(ca);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mass_resid_part_kernel, dim3(kResBlk, H), dim3(256), 0, st, pl.rowstat_cmp,
                     pl.shift2, (const float*)nullptr, pl.part, n);
  hipLaunchKernelGGL(resid_final_kernel, dim3(cdiv(H, 64)), dim3(64), 0, st,
                     (const double2*)pl.part, out, H);
  return hipGetLastError();
}

// output residual sum ||A C_v - Y||^2 / sum ||Y||^2 of (idx, beta, C_v) against targets Y
static hipError_t output_residual(const FitArgs& a, const float* beta, const float* Cv,
                                  const float* Y, const FastPlan& pl, float* out) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n;
  CmpAttnArgs cr;
  cr.Q = a.Q; cr.Ck = a.Ck; cr.Cv = Cv; cr.bias = beta; cr.keypos = a.idx; cr.Y = Y;
  cr.Vt = pl.Vt; cr.tstat = pl.tstat;
  cr.lse = nullptr; cr.rowstat = nullptr; cr.O = nullptr; cr.rowres = pl.rowres;
  cr.heads = H; cr.n = n; cr.t = a.t; cr.d = a.d; cr.group = a.group; cr.causal = a.causal;
  cr.bf16 = a.bf16; cr.scale = a.scale; cr.stream = st;
  const hipError_t e = launch_cmp_attention(cr);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(out_resid_part_kernel, dim3(kResBlk, H), dim3(256), 0, st, pl.rowres,
                     pl.part, n);
  hipLaunchKernelGGL(resid_final_kernel, dim3(cdiv(H, 64)), dim3(64), 0, st,
                     (const double2*)pl.part, out, H);
  return hipGetLastError();
}

hipError_t launch_zero_status(int32_t* status, int heads, hipStream_t st) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(cdiv(heads, 256)), dim3(256), 0, st, status, heads);
  return hipGetLastError();
}

hipError_t launch_beta_redistribute(const FitArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads;
  FastPlan pl = plan_fast((char*)a.ws, H, a.n, a.t, a.d, a.bf16 ? 2 : 4, 0);
  hipLaunchKernelGGL(redist_prep_kernel, dim3(H), dim3(1024), 0, st, a.lse, a.n, pl.shift2h,
                     pl.zsum);
  KeyMassArgs km;
  km.Q = a.Q; km.Ck = a.Ck; km.keypos = a.idx; km.shift2 = pl.shift2h;
  km.kmax = pl.kmax; km.kmean = pl.kmean; km.part = pl.kpart;
  km.heads = H; km.n = a.n; km.t = a.t; km.d = a.d; km.group = a.group; km.causal = a.causal;
  km.bf16 = a.bf16; km.scale = a.scale; km.stream = st;
  hipError_t e = launch_key_mass(km);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(redist_beta_kernel, dim3(H), dim3(256), 0, st, pl.kmax, pl.kmean, pl.zsum,
                     a.n, a.t, a.beta, a.w);
  if (a.mass_resid && (e = mass_residual(a, a.lse, a.beta, pl, a.mass_resid)) != hipSuccess)
    return e;
  return hipGetLastError();
}

hipError_t launch_values_direct(const FitArgs& a, const void* V, int T) {
  const hipStream_t st = a.stream;
  const int H = a.heads;
  const dim3 g(cdiv((long long)a.t * (a.d / 4), 256), H);
  if (a.bf16)
    hipLaunchKernelGGL(gather_f32_kernel<bf16>, g, dim3(256), 0, st, (const bf16*)V, a.idx, a.Cv,
                       T, a.t, a.d);
  else
    hipLaunchKernelGGL(gather_f32_kernel<float>, g, dim3(256), 0, st, (const float*)V, a.idx,
                       a.Cv, T, a.t, a.d);
  if (a.out_resid) {
    FastPlan pl = plan_fast((char*)a.ws, H, a.n, a.t, a.d, a.bf16 ? 2 : 4, 0);
    const hipError_t e = output_residual(a, a.beta_in, a.Cv, a.O, pl, a.out_resid);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_eval_residuals(const FitArgs& a, const void* K, const void* V, int T,
                                 float* resid) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n, d = a.d, es = a.bf16 ? 2 : 4;
  FastPlan pl = plan_fast((char*)a.ws, H, n, a.t, d, es, T);
  TargetsArgs ta;
  ta.Q = a.Q; ta.K = K; ta.V = V; ta.Vt = pl.tws;
  ta.rowstat = (char*)pl.tws + targets_vt_bytes(H, T, d, es);
  ta.lse = pl.lse; ta.O = pl.O; ta.score = nullptr; ta.mode = 0;
  ta.heads = H; ta.n = n; ta.T = T; ta.d = d; ta.group = a.group; ta.causal = a.causal;
  ta.bf16 = a.bf16; ta.scale = a.scale; ta.stream = st;
  hipError_t e = launch_targets(ta);
  if (e != hipSuccess) return e;
  if ((e = mass_residual(a, pl.lse, a.beta_in, pl, resid)) != hipSuccess) return e;
  return output_residual(a, a.beta_in, a.Cv, pl.O, pl, resid + H);
}

}  // namespace amc
