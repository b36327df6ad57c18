// Gram builds for large compacted sizes (t > 256) on gfx950, in two kernels instead of one
// fused recompute: the design entries are formed once and stored, then their Gram is a
// plain bf16 MFMA product.
//
// What is built follows the "Compaction" blog, §Choosing beta (the mass equations, one row
// per reference query, one column per selected key) and §Choosing C_v (the output
// equations with A_i the biased compacted softmax of "Latent Compaction with Test-Time
// Training", §3.1 Eq. 2-3): the normal-equation matrices M^T M, M^T b, A^T A and A^T Y.
//
// Design kernel. X [h, xrows / 256, npad / 32, 256, 32] bf16: one row per selected key, in
// blocks of 256 rows, each block stored as 32-query stages of 256 rows x 32 queries (16 KB,
// contiguous), so a stage of a block, the unit the Gram product loads, is one run of memory:
// X[j][i] = 2^(s_ij scale log2 e + bias_j - shift_i) under the causal mask of the key's
// original position, 0 for padded queries. A workgroup forms 128 queries
// x 256 keys: its query tile sits in LDS (rows in the kperm order) and every wave keeps the
// C_k fragments of its 64 keys in registers, so a lane's share of a 32 x 32 score block is
// 8 + 8 consecutive queries of one key: two 16-byte stores per block. The mass variant also
// sums b_i X[j][i] per key over its 128 queries (partials of M^T b, reduced later).
// For the value fit the rows after the keys hold Y^T (bf16), so the product below also
// yields A^T Y.
//
// Gram kernel. part[h, chunk, tile] = X_a X_b^T over one chunk of queries, for the 256 x 256
// row-block pairs a >= b (lower triangle; for the value fit the pair of the Y^T block with
// itself is skipped, and in its pairs with the key blocks only the half of the Y^T block
// that holds rows is staged and multiplied). Eight waves, two per SIMD, each own a 128 x 64 block (8 MFMA
// accumulators), so one wave's LDS reads and barrier wait overlap the other's products;
// 32-query stages are staged by direct global-to-LDS loads (one barrier per stage). Under the causal mask a key block has no entry before the first
// query that sees its first key, so each tile starts its chunk there.
//
// Reductions sum the chunk partials in a fixed order: no floating-point atomics.
#include "am_common.hpp"
#include "am_internal.hpp"

#include <type_traits>

namespace amc {

constexpr int kSyT = 256;   // Gram tile side (rows of X per block)
constexpr int kSyK = 32;    // queries per Gram step (one LDS stage)
constexpr int kDsQ = 128;   // queries per design workgroup
constexpr int kDsK = 256;   // keys per design workgroup (4 waves x 64)
// Rows of the Y^T block that are written and multiplied (d <= 128 of them hold Y^T, the rest
// of these zeros); its other 128 rows are neither written nor read.
constexpr int kSyYRows = 128;

// Element (row R of a 256-row block, query q) within that block of the stored design: the
// stage q / 32 is 256 rows x 32 queries, row-major.
__device__ __forceinline__ size_t xoff(int R, int q) {
  return (size_t)(q >> 5) * (kSyT * kSyK) + (size_t)R * kSyK + (q & 31);
}

__device__ __forceinline__ void sy_tri(int k, int& a, int& b) {
  int x = (int)((sqrtf(8.f * (float)k + 1.f) - 1.f) * 0.5f);
  while ((x + 1) * (x + 2) / 2 <= k) ++x;
  while (x * (x + 1) / 2 > k) --x;
  a = x;
  b = k - x * (x + 1) / 2;
}

struct DesignParams {
  const void* Q; const void* Ck; const int32_t* keypos; const float* bias;
  const float* shift2;   // per query, log2 domain
  const float* target;   // mass: per-query right-hand side (null = 1)
  bf16* X; float* hpart;
  int n, npad, t, tpad, xrows, group, causal;
  float c2;
};

template <typename T, int D, bool VALUE>
__global__ __launch_bounds__(256) void design_kernel(const DesignParams p) {
  typedef typename V8<T>::type v8;
  constexpr int E = 16 / (int)sizeof(T), QP = D + E, KC = D / 16, QCPR = D / E;
  constexpr int QPT = kDsQ * QCPR / 256;
  static_assert(kDsQ * QCPR % 256 == 0, "query tile / thread mismatch");
  __shared__ __align__(16) T qs[kDsQ * QP];
  __shared__ __align__(16) float shs[kDsQ];
  __shared__ __align__(16) float tgs[kDsQ];

  const int qb = blockIdx.x, kblk = blockIdx.y, head = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = p.n, t = p.t, q0 = qb * kDsQ;
  const T* Qh = (const T*)p.Q + (size_t)head * n * D;
  const T* Ch = (const T*)p.Ck + (size_t)head * t * D;
  // Under the causal mask the Gram product reads this key block only from the first query
  // that sees its first key (rounded down to its 32-query steps); earlier query tiles hold
  // zeros nobody reads, so they are neither computed nor written (M^T b partials: 0).
  if (p.causal) {
    const int first = p.keypos[(size_t)head * t + min(kblk * kDsK, t - 1)] * p.group;
    if (q0 + kDsQ <= (first / kSyK) * kSyK) {
      if (!VALUE)
        for (int k = tid; k < kDsK; k += 256)
          p.hpart[((size_t)head * p.tpad + kblk * kDsK + k) * gridDim.x + qb] = 0.f;
      return;
    }
  }

#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = tid + i * 256;
    const int row = c / QCPR, col = (c % QCPR) * E;
    *(u32x4*)&qs[row * QP + col] = *(const u32x4*)(Qh + (size_t)min(q0 + row, n - 1) * D + col);
  }
  if (tid < kDsQ) {
    const int q = min(q0 + tid, n - 1);
    shs[tid] = p.shift2[(size_t)head * n + q];
    tgs[tid] = (!VALUE && p.target) ? p.target[(size_t)head * n + q] : 1.f;
  }

  // this lane's two keys (one per 32-key block of the wave); rows past t repeat key t - 1
  int key[2], kq0[2];
  float kb2[2];
  v8 bck[2][KC];
  int kq0max = 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    key[kb] = kblk * kDsK + wave * 64 + kb * 32 + r;
    const int kr = min(key[kb], t - 1);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) bck[kb][kc] = *(const v8*)(Ch + (size_t)kr * D + kc * 16 + hh * 8);
    kq0[kb] = p.causal ? p.keypos[(size_t)head * t + kr] * p.group : 0;
    kb2[kb] = VALUE ? p.bias[(size_t)head * t + kr] * kLog2e : 0.f;
    kq0max = max(kq0max, kq0[kb]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kq0max = max(kq0max, __shfl_xor(kq0max, o, 64));
  kq0max = __builtin_amdgcn_readfirstlane(kq0max);
  __syncthreads();

  float hsum[2] = {0.f, 0.f};
  bf16* Xh = p.X + (size_t)head * p.xrows * p.npad;
#pragma unroll 1
  for (int sb = 0; sb < kDsQ / 32; ++sb) {
    const int qs0 = q0 + sb * 32;
    // MASK (wave-uniform): some query of the sub-block precedes a key's first visible query,
    // or lies past n
    const bool mask = qs0 < kq0max || qs0 + 32 > n;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
    const T* arow = &qs[(sb * 32 + kperm(r)) * QP + hh * 8];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const v8 a = *(const v8*)(arow + kc * 16);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma16(s[kb], a, bck[kb][kc]);
    }
    // element j of a lane is query qs0 + 8 hh + o_j, o_j = j (j < 8) or j + 8
    const float4* s4 = (const float4*)&shs[sb * 32 + 8 * hh];
    const float4 sa = s4[0], sbv = s4[1], sc = s4[4], sd = s4[5];
    const float shv[16] = {sa.x, sa.y, sa.z, sa.w, sbv.x, sbv.y, sbv.z, sbv.w,
                           sc.x, sc.y, sc.z, sc.w, sd.x, sd.y, sd.z, sd.w};
    float tg[16];
    if (!VALUE) {
      const float4* t4 = (const float4*)&tgs[sb * 32 + 8 * hh];
      const float4 ta = t4[0], tb = t4[1], tc = t4[4], td = t4[5];
      const float tv[16] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w,
                            tc.x, tc.y, tc.z, tc.w, td.x, td.y, td.z, td.w};
#pragma unroll
      for (int j = 0; j < 16; ++j) tg[j] = tv[j];
    }
    const int qbase = qs0 + 8 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float v[16];
      const int lo = kq0[kb] - qbase, hi = n - qbase;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = VALUE ? __builtin_fmaf(s[kb][j], p.c2, kb2[kb]) - shv[j]
                        : __builtin_fmaf(s[kb][j], p.c2, -shv[j]);
        if (mask) {
          const int o = j < 8 ? j : j + 8;
          x = (o >= lo && o < hi) ? x : -INFINITY;
        }
        v[j] = ex2(x);
      }
      if (!VALUE) {
#pragma unroll
        for (int j = 0; j < 16; ++j) hsum[kb] += v[j] * tg[j];
      }
      // key j: block j / 256 (its base is j / 256 * 256 rows of npad), row j % 256
      bf16* row = Xh + (size_t)(key[kb] / kSyT) * kSyT * p.npad + xoff(key[kb] % kSyT, qbase);
      *(bf16x8*)row = AM_PACK8(bf16, v, 0);
      *(bf16x8*)(row + 16) = AM_PACK8(bf16, v, 8);
    }
  }
  if (!VALUE) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float tot = hsum[kb] + shfl_xor32(hsum[kb]);
      if (hh == 0) p.hpart[((size_t)head * p.tpad + key[kb]) * gridDim.x + qb] = tot;
    }
  }
}

// Y^T rows of the value design: X[tpad + c][i] = bf16(Y[i][c]) for c < D and i < n; rows
// c in [D, 256) and queries past n are zero. One workgroup per 64 queries. With yyp set, the
// workgroup also writes the fp64 sum of squares of its fp32 Y entries to yyp[head, block]
// (partials of ||Y||^2 for the output residual; fixed order).
template <int D>
__global__ __launch_bounds__(256) void design_yt_kernel(const float* __restrict__ Y, bf16* X,
                                                        int n, int npad, int tpad, int xrows,
                                                        double* __restrict__ yyp) {
  __shared__ float ys[64][D + 1];
  __shared__ double red[256];
  const int q0 = blockIdx.x * 64, head = blockIdx.y, tid = threadIdx.x;
  const float* Yh = Y + (size_t)head * n * D;
  double sq = 0.0;
  for (int e = tid; e < 64 * D / 4; e += 256) {
    const int row = e / (D / 4), col = (e % (D / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q0 + row < n) v = *(const float4*)(Yh + (size_t)(q0 + row) * D + col);
    sq += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    ys[row][col] = v.x;
    ys[row][col + 1] = v.y;
    ys[row][col + 2] = v.z;
    ys[row][col + 3] = v.w;
  }
  if (yyp) {   // (uniform over the workgroup)
    red[tid] = sq;
    __syncthreads();
    for (int s2 = 128; s2 > 0; s2 >>= 1) {
      if (tid < s2) red[tid] += red[tid + s2];
      __syncthreads();
    }
    if (tid == 0) yyp[(size_t)head * gridDim.x + blockIdx.x] = red[0];
  }
  __syncthreads();
  static_assert(D <= kSyYRows, "Y^T rows exceed the part of the block the products read");
  bf16* Xh = X + ((size_t)head * xrows + tpad) * npad;   // the Y^T block
  // kSyYRows rows x 64 queries, 8 queries (16 bytes) per store
  for (int e = tid; e < kSyYRows * 8; e += 256) {
    const int c = e / 8, qq = (e % 8) * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c < D ? ys[qq + i][c] : 0.f;
    *(bf16x8*)(Xh + xoff(c, q0 + qq)) = AM_PACK8(bf16, v, 0);
  }
}

struct SyrkParams {
  const bf16* X; float* part; const int32_t* keypos;
  int xrows, npad, nkb;   // nkb: row blocks holding key rows (later blocks hold Y^T)
  int ntiles, nch, chunk, t, group, causal, nhead;
};

// Workgroup order: consecutive workgroups go to the eight XCDs in turn, so linear id L runs
// on XCD L % 8. The tiles of one (head, chunk) read the same rows of X over the same
// queries; they are given consecutive slots L / 8 of one XCD, so they run together and
// share that XCD's L2. Ids past the last group exit at once.
//
// Staging: kSyS stages of kSyK queries in LDS, filled by direct global-to-LDS loads
// (global_load_lds_dwordx4: lane l of a load writes the 16 bytes at base + 16 l), issued
// kSyS - 1 stages ahead. A stage holds 256 rows x 64 bytes per operand with no padding;
// the four 16-byte chunks of row R are stored in the order c ^ ((R >> 2) & 3), so the 16
// lanes of an MFMA fragment read (16 consecutive rows, one chunk) hit 16 distinct bank
// groups. A stage is consumed after a wait on this wave's own loads (vmcnt) and a plain
// s_barrier; every wave also drains its LDS reads (lgkmcnt 0) before that barrier, since
// the buffer read in the previous step is refilled right after it.
constexpr int kSyS = 4;                  // LDS stages
constexpr int kSyRow = kSyK;             // bf16 per staged row (64 bytes)
constexpr int kSyWaves = 8;              // two waves per SIMD, each a 128 x 64 block
constexpr int kSyLoads = kSyT / 16 / kSyWaves;  // loads per wave per operand per stage (2)

__device__ __forceinline__ void sy_wait_stages(int pending, bool diag) {
  // vmcnt <= pending stages' loads of this wave, lgkmcnt 0, expcnt untouched (7)
  // (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14])
  const int per = diag ? kSyLoads : 2 * kSyLoads;
  switch (pending * per) {
    case 0: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8)); break;
    case 2: __builtin_amdgcn_s_waitcnt(2 | (7 << 4) | (0 << 8)); break;
    case 4: __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (0 << 8)); break;
    case 6: __builtin_amdgcn_s_waitcnt(6 | (7 << 4) | (0 << 8)); break;
    case 8: __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (0 << 8)); break;
    default: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8)); break;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(kSyWaves * 64) void syrk_kernel(const SyrkParams p) {
  static_assert(kSyK == 32 && kSyS == 4, "staging layout assumes 32-query stages");
  __shared__ __align__(16) bf16 xs[kSyS][2][kSyT * kSyRow];
  // Groups (head, chunk) in decreasing expected work (later chunks hold more causally
  // visible pairs; heads alike) are dealt to the XCDs in snake order: XCD x takes groups
  // 8k + x for even k and 8k + 7 - x for odd k, so the XCDs get equal shares and each
  // starts with its largest groups.
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int k = slot / p.ntiles, tile = slot % p.ntiles;
  const int sgrp = 8 * k + ((k & 1) ? 7 - xcd : xcd);
  if (sgrp >= p.nch * p.nhead) return;
  const int ch = p.nch - 1 - sgrp / p.nhead, head = sgrp % p.nhead;
  int ra, rb;
  sy_tri(tile, ra, rb);
  const bool diag = ra == rb;   // (wave-uniform)
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wy = wave >> 2, wx = wave & 3;
  // In a tile of the Y^T block (always operand a) the waves of rows 128..255 hold no output:
  // they neither stage those rows nor multiply (the products read only the first kSyYRows).
  static_assert(kSyYRows == 128 && kSyLoads * 16 * (kSyWaves / 2) == 128,
                "waves 4..7 stage exactly rows 128..255 of operand a");
  const bool idle_a = ra == p.nkb && wy == 1;   // (wave-uniform)
  // first query with an entry in a block: that of its first key (keys ascend by position)
  auto kfirst = [&](int blk) -> int {
    if (!p.causal || blk >= p.nkb) return 0;
    return p.keypos[(size_t)head * p.t + min(blk * kSyT, p.t - 1)] * p.group;
  };
  const int kbeg = max(ch * p.chunk, (max(kfirst(ra), kfirst(rb)) / kSyK) * kSyK);
  const int kend = min(p.npad, (ch + 1) * p.chunk);
  const int nsteps = kend > kbeg ? (kend - kbeg) / kSyK : 0;
  const bf16* Xa = p.X + ((size_t)head * p.xrows + (size_t)ra * kSyT) * p.npad;
  const bf16* Xb = p.X + ((size_t)head * p.xrows + (size_t)rb * kSyT) * p.npad;

  // this lane's source of load i: row R = 16 (kSyLoads wave + i) + l / 4, logical chunk
  // (l % 4) ^ ((R >> 2) & 3)
  size_t soff[kSyLoads];
#pragma unroll
  for (int i = 0; i < kSyLoads; ++i) {
    const int R = 16 * (kSyLoads * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((R >> 2) & 3);
    soff[i] = xoff(R, kbeg) + c * 8;   // (kbeg is a stage boundary)
  }
  // fragment reads: row base + 32 i + r, logical chunk 2 kk + hh
  const int swz = (r >> 2) & 3;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // DIAG (a compile-time choice): the two row blocks coincide, one operand is staged
  auto run = [&](auto diag_tag) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    auto issue = [&](int st) {
      const int buf = st % kSyS;
      const size_t k = (size_t)st * (kSyT * kSyK);   // next stage: the next 16 KB run
#pragma unroll
      for (int i = 0; i < kSyLoads; ++i) {
        const int R0 = 16 * (kSyLoads * wave + i);
        if (!idle_a)
          __builtin_amdgcn_global_load_lds((const void*)(Xa + soff[i] + k),
                                           (lds_ptr_t)&xs[buf][0][R0 * kSyRow], 16, 0, 0);
        if (!DIAG)
          __builtin_amdgcn_global_load_lds((const void*)(Xb + soff[i] + k),
                                           (lds_ptr_t)&xs[buf][1][R0 * kSyRow], 16, 0, 0);
      }
    };
#pragma unroll
    for (int s0 = 0; s0 < kSyS - 1; ++s0)
      if (s0 < nsteps) issue(s0);
    for (int st = 0; st < nsteps; ++st) {
      sy_wait_stages(min(kSyS - 2, nsteps - 1 - st), DIAG || idle_a);
      __builtin_amdgcn_s_barrier();
      if (st + kSyS - 1 < nsteps) issue(st + kSyS - 1);
      if (idle_a) continue;
      const int buf = st % kSyS;
      const bf16* A = &xs[buf][0][(wy * 128 + r) * kSyRow];
      const bf16* B = &xs[buf][DIAG ? 0 : 1][(wx * 64 + r) * kSyRow];
      bf16x8 af[2][4], bfr[2][2];
      auto frag = [&](int kk, int slot) {
        const int off = ((2 * kk + hh) ^ swz) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[slot][i] = *(const bf16x8*)(A + i * 32 * kSyRow + off);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[slot][j] = *(const bf16x8*)(B + j * 32 * kSyRow + off);
      };
      // sub-step 0's six reads, its first two MFMAs, then sub-step 1's reads
      frag(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) mma16(acc[0][j], af[0][0], bfr[0][j]);
      __builtin_amdgcn_sched_barrier(0);
      frag(1, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 1; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma16(acc[i][j], af[0][i], bfr[0][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma16(acc[i][j], af[1][i], bfr[1][j]);
    }
  };
  if (diag) run(std::true_type{});
  else run(std::false_type{});

  if (idle_a) return;
  float* P = p.part + (((size_t)head * p.nch + ch) * p.ntiles + tile) * kSyT * kSyT;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        P[(size_t)(wy * 128 + i * 32 + crow(e, hh)) * kSyT + wx * 64 + j * 32 + r] = acc[i][j][e];
}

// Symmetric Gram of the key rows, chunk partials summed in order, into an ld x ld matrix
// per head: fp32 (NNLS, ld = t) or fp64 + lambda I with identity padding (Cholesky).
// One workgroup per 64 x 64 output block (bi, bj): it sums the stored lower block
// (max, min) with coalesced reads and, above the diagonal, writes it transposed via LDS.
template <typename OT>
__global__ __launch_bounds__(256) void syrk_reduce_g_kernel(const float* __restrict__ part,
                                                            OT* __restrict__ G, int t, int ld,
                                                            int ntiles, int nch, float lambda) {
  __shared__ float blk[64][65];
  // one workgroup per lower 64 x 64 block (si >= sj): it writes the block and its mirror
  const int head = blockIdx.z, tid = threadIdx.x;
  int si, sj;
  sy_tri(blockIdx.x, si, sj);
  const int a = si * 64 / kSyT, b = sj * 64 / kSyT;
  const int tile = a * (a + 1) / 2 + b;
  const float* src = part + ((size_t)head * nch * ntiles + tile) * kSyT * kSyT +
                     (size_t)(si * 64 % kSyT) * kSyT + sj * 64 % kSyT;
  const size_t cstride = (size_t)ntiles * kSyT * kSyT;
  // 16 entries per thread, summed over the chunks in order
  constexpr int PER = 64 * 64 / 256;
  float acc[PER];
  bool live[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + 256 * u, r = e >> 6, c = e & 63;
    acc[u] = 0.f;
    live[u] = si * 64 + r < t && sj * 64 + c < t;
  }
  // every address lies in a chunk's 256 x 256 partial tile, so the loads are unconditional
  // (a branch per load would wait for each one) and the padding is masked by a select; four
  // chunks' loads are issued before their sums, which still run in chunk order
  auto load_chunk = [&](int ch, float (&v)[PER]) {
    const float* sc = src + ch * cstride;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u, r = e >> 6, c = e & 63;
      v[u] = sc[(size_t)r * kSyT + c];
    }
  };
  int ch = 0;
  for (; ch + 4 <= nch; ch += 4) {
    float v[4][PER];
#pragma unroll
    for (int q = 0; q < 4; ++q) load_chunk(ch + q, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += live[u] ? v[q][u] : 0.f;
  }
  for (; ch < nch; ++ch) {
    float v[PER];
    load_chunk(ch, v);
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] += live[u] ? v[u] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + 256 * u;
    blk[e >> 6][e & 63] = acc[u];
  }
  __syncthreads();
  OT* dst = G + (size_t)head * ld * ld;
  for (int mirror = 0; mirror < (si != sj ? 2 : 1); ++mirror) {
    const int bi = mirror ? sj : si, bj = mirror ? si : sj;
    for (int e = tid; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63, i = bi * 64 + r, j = bj * 64 + c;
      if (i >= ld || j >= ld) continue;
      double v;
      if (i < t && j < t) v = (double)(mirror ? blk[c][r] : blk[r][c]) + (i == j ? (double)lambda : 0.0);
      else v = (i == j) ? 1.0 : 0.0;
      dst[(size_t)i * ld + j] = (OT)v;
    }
  }
}

// A^T Y from the tiles pairing the Y^T block (index nkb) with the key blocks:
// R[j][c] = sum over chunks of part[tile (nkb, j / 256)][c][j % 256]; rows in [t, ld) zero.
__global__ __launch_bounds__(256) void syrk_reduce_r_kernel(const float* __restrict__ part,
                                                            double* __restrict__ R, int t, int ld,
                                                            int D, int nkb, int ntiles, int nch) {
  const int head = blockIdx.y;
  // thread (c, j), j fastest, so a wave reads consecutive floats of one partial row
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)ld * D) return;
  const int c = (int)(e / ld), j = (int)(e % ld);
  float acc = 0.f;
  if (j < t) {
    const int tile = nkb * (nkb + 1) / 2 + j / kSyT;
#pragma unroll 8   // several chunks' loads in flight; the sum still runs in chunk order
    for (int ch = 0; ch < nch; ++ch)
      acc += part[(((size_t)head * nch + ch) * ntiles + tile) * kSyT * kSyT +
                  (size_t)c * kSyT + j % kSyT];
  }
  R[((size_t)head * ld + j) * D + c] = (double)acc;
}

// M^T b: hv[j] = sum over query blocks of the design kernel's partials (key-major
// [h, tpad, nqb]); one wave per key, lanes take every 64th partial, then a fixed-order
// shuffle tree.
__global__ __launch_bounds__(256) void syrk_reduce_h_kernel(const float* __restrict__ hpart,
                                                            float* __restrict__ hv, int t,
                                                            int tpad, int nqb) {
  const int head = blockIdx.y, j = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (j >= t) return;
  const float* src = hpart + ((size_t)head * tpad + j) * nqb;
  float acc = 0.f;
  for (int b = lane; b < nqb; b += 64) acc += src[b];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) hv[(size_t)head * t + j] = acc;
}

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
namespace {
struct SyrkShape {
  int npad, tpad, nkb, nrb, xrows, ntiles, nch, chunk, nqb;
};
SyrkShape syrk_shape(int heads, int n, int t, int d, bool value) {
  SyrkShape s;
  s.npad = round_up(n, kDsQ);
  s.tpad = round_up(t, kSyT);
  s.nkb = s.tpad / kSyT;
  s.nrb = s.nkb + (value ? 1 : 0);
  s.xrows = s.nrb * kSyT;
  s.ntiles = s.nrb * (s.nrb + 1) / 2 - (value ? 1 : 0);   // the Y^T block with itself is unused
  // chunks: at least ~1024 workgroups, then the count that wastes the least of the last
  // round of 256 (time ~ rounds / chunks), with chunks of at least 1024 queries
  const int g = heads * s.ntiles;
  int maxc = s.npad / 1024;
  if (maxc < 1) maxc = 1;
  int want = (1024 + g - 1) / g;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  s.nch = want;
  double best = 1e30;
  for (int c = want; c <= 2 * want && c <= maxc; ++c) {
    const double cost = (double)((g * c + 255) / 256) / c;
    if (cost < best - 1e-12) {
      best = cost;
      s.nch = c;
    }
  }
  s.chunk = round_up((s.npad + s.nch - 1) / s.nch, kSyK);
  s.nqb = s.npad / kDsQ;
  (void)d;
  return s;
}
}  // namespace

bool syrk_path(int t) { return t > kSyrkMinT; }

int syrk_yy_blocks(int64_t heads, int64_t n, int64_t t, int64_t d) {
  return syrk_shape((int)heads, (int)n, (int)t, (int)d, true).npad / 64;
}

SyrkBuffers syrk_carve(char* base, size_t& off, int64_t heads, int64_t n, int64_t t, int64_t d,
                       bool value) {
  const SyrkShape s = syrk_shape((int)heads, (int)n, (int)t, (int)d, value);
  SyrkBuffers b;
  auto take = [&](size_t bytes) {
    char* q = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return q;
  };
  b.X = (void*)take((size_t)heads * s.xrows * s.npad * sizeof(bf16));
  b.part = (float*)take((size_t)heads * s.nch * s.ntiles * kSyT * kSyT * sizeof(float));
  b.hpart = value ? nullptr : (float*)take((size_t)heads * s.nqb * s.tpad * sizeof(float));
  return b;
}

template <typename T, int D>
static void launch_design_t(const DesignParams& dp, const SyrkShape& s, int heads, bool value,
                            hipStream_t st) {
  const dim3 g(s.nqb, s.tpad / kDsK, heads);
  if (value) hipLaunchKernelGGL((design_kernel<T, D, true>), g, dim3(256), 0, st, dp);
  else hipLaunchKernelGGL((design_kernel<T, D, false>), g, dim3(256), 0, st, dp);
}

hipError_t launch_syrk_gram(const SyrkGramArgs& a) {
  const hipStream_t st = a.stream;
  const int H = a.heads, n = a.n, t = a.t, d = a.d;
  const SyrkShape s = syrk_shape(H, n, t, d, a.value);
  DesignParams dp;
  dp.Q = a.Q; dp.Ck = a.Ck; dp.keypos = a.keypos; dp.bias = a.bias; dp.shift2 = a.shift2;
  dp.target = a.target; dp.X = (bf16*)a.buf.X; dp.hpart = a.buf.hpart;
  dp.n = n; dp.npad = s.npad; dp.t = t; dp.tpad = s.tpad; dp.xrows = s.xrows; dp.group = a.group;
  dp.causal = a.causal; dp.c2 = a.c2;
  if (a.bf16) {
    if (d == 128) launch_design_t<bf16, 128>(dp, s, H, a.value, st);
    else launch_design_t<bf16, 64>(dp, s, H, a.value, st);
  } else {
    if (d == 128) launch_design_t<float, 128>(dp, s, H, a.value, st);
    else launch_design_t<float, 64>(dp, s, H, a.value, st);
  }
  if (a.value) {
    const dim3 g(s.npad / 64, H);
    if (d == 128)
      hipLaunchKernelGGL((design_yt_kernel<128>), g, dim3(256), 0, st, a.Y, (bf16*)a.buf.X, n, s.npad,
                         s.tpad, s.xrows, a.yyp);
    else
      hipLaunchKernelGGL((design_yt_kernel<64>), g, dim3(256), 0, st, a.Y, (bf16*)a.buf.X, n, s.npad,
                         s.tpad, s.xrows, a.yyp);
  }
  SyrkParams sp;
  sp.X = (const bf16*)a.buf.X; sp.part = a.buf.part; sp.keypos = a.keypos;
  sp.xrows = s.xrows; sp.npad = s.npad; sp.nkb = s.nkb;
  sp.ntiles = s.ntiles; sp.nch = s.nch; sp.chunk = s.chunk; sp.t = t; sp.group = a.group;
  sp.causal = a.causal; sp.nhead = H;
  const int ngrp = s.nch * H;
  hipLaunchKernelGGL(syrk_kernel, dim3(8 * s.ntiles * ((ngrp + 7) / 8)), dim3(kSyWaves * 64), 0,
                     st, sp);
  const int nb64 = (a.ld + 63) / 64;
  const dim3 gb(nb64 * (nb64 + 1) / 2, 1, H);   // lower 64 x 64 blocks
  if (a.value) {
    hipLaunchKernelGGL((syrk_reduce_g_kernel<double>), gb, dim3(256), 0, st,
                       (const float*)a.buf.part, a.Gd, t, a.ld, s.ntiles, s.nch, a.lambda);
    const unsigned gr = (unsigned)(((long long)a.ld * d + 255) / 256);
    hipLaunchKernelGGL(syrk_reduce_r_kernel, dim3(gr, H), dim3(256), 0, st,
                       (const float*)a.buf.part, a.R, t, a.ld, d, s.nkb, s.ntiles, s.nch);
  } else {
    hipLaunchKernelGGL((syrk_reduce_g_kernel<float>), gb, dim3(256), 0, st,
                       (const float*)a.buf.part, a.Gf, t, a.ld, s.ntiles, s.nch, 0.f);
    hipLaunchKernelGGL(syrk_reduce_h_kernel, dim3((t + 3) / 4, H), dim3(256), 0, st,
                       (const float*)a.buf.hpart, a.hv, t, s.tpad, s.nqb);
  }
  return hipGetLastError();
}

}  // namespace amc
