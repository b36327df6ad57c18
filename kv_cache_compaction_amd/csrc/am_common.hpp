// Device-side helpers shared by the gfx950 kernels: vector types, the 32x32 MFMA step,
// exp2/log2 on the hardware transcendental unit, and the launch-side error check.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace amc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte staging chunk (a native vector type, so arrays of it stay in registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements along the contraction dimension: the per-lane share of one
// 16-deep k-step of a 32x32 MFMA tile (lane l holds k = 8 * (l / 32) .. + 7).
template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 type; };
template <> struct V8<float> { typedef f32x8 type; };

// C[32x32] += A[32x16] * B[16x32].
// Lane l supplies A[row l%32][k 8*(l/32)..+7] and B[k 8*(l/32)..+7][col l%32]; it holds
// C[row (j/4)*8 + (l/32)*4 + j%4][col l%32] in c[j], j = 0..15.
__device__ __forceinline__ void mma16(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp32 operands: eight 32x32x2 steps. Step i contracts k = 8*(l/32) + i in both operands,
// so the eight steps together cover the same 16 k values with full fp32 products.
__device__ __forceinline__ void mma16(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
}

// Eight floats to the operand type, by value (no address taken, so the temporaries stay
// in registers).
template <typename T>
__device__ __forceinline__ typename V8<T>::type pack8(float a0, float a1, float a2, float a3,
                                                      float a4, float a5, float a6, float a7) {
  typename V8<T>::type r;
  r[0] = (T)a0; r[1] = (T)a1; r[2] = (T)a2; r[3] = (T)a3;
  r[4] = (T)a4; r[5] = (T)a5; r[6] = (T)a6; r[7] = (T)a7;
  return r;
}
#define AM_PACK8(T, x, o) \
  pack8<T>((x)[(o) + 0], (x)[(o) + 1], (x)[(o) + 2], (x)[(o) + 3], (x)[(o) + 4], (x)[(o) + 5], \
           (x)[(o) + 6], (x)[(o) + 7])

template <typename T> __device__ __forceinline__ typename V8<T>::type cvt8(const float* x);
template <> __device__ __forceinline__ bf16x8 cvt8<bf16>(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
  return r;
}
template <> __device__ __forceinline__ f32x8 cvt8<float>(const float* x) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = x[i];
  return r;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Row of the 32x32 C tile held in element j by a lane in half h (= lane / 32).
__device__ __forceinline__ constexpr int crow(int j, int h) { return (j >> 2) * 8 + h * 4 + (j & 3); }

// Row permutation for an operand whose product feeds a second MFMA from registers:
// loading A row r from source row kperm(r) makes a lane of half h hold source rows
// 8h .. 8h+7 in c[0..7] and 16+8h .. 16+8h+7 in c[8..15], which is exactly the B-operand
// share (k = 8h .. 8h+7) of the two 16-deep k-steps that follow.
__device__ __forceinline__ constexpr int kperm(int r) {
  const int h = (r & 7) >> 2;
  const int j = (r >> 3) * 4 + (r & 3);
  return j < 8 ? 8 * h + j : 16 + 8 * h + (j - 8);
}

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Maximum of finite or infinite floats as v_maximum(3)_f32: unlike fmaxf, it needs no
// quieting of its operands, which would cost one extra instruction per operand.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

}  // namespace amc
