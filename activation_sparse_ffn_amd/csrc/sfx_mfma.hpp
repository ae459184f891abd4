// Matrix-core building blocks shared by the predictor kernels: the 16x16x32 fp16 /
// bf16 MFMA with fp32 accumulation, and the exact split of an fp32 value into 16-bit
// pieces for it.
//
// Lane layout of v_mfma_f32_16x16x32 (checked against a CPU product): lane l holds
// A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16], and D[4 (l / 16) + i][l % 16]
// for i = 0..3.
//
// Split: fp16 weights take v = hi + 2^-11 lo with hi = fp16(v), lo = fp16((v - hi) 2^11)
// (22 significant bits, lo scaled so it does not fall into fp16 subnormals); bf16
// weights take v = hi + mid + lo, three bf16 terms (24 bits, exact for normal values).
// Products of two 16-bit values are exact in fp32, so the pieces multiply exactly.
#pragma once
#include "sfx_common.hpp"

namespace sfx {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class T>
struct Mma;
template <>
struct Mma<TF16> {
  __device__ __forceinline__ static f32x4 run(const Raw<16>& a, const Raw<16>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                  0, 0);
  }
};
template <>
struct Mma<TBF16> {
  __device__ __forceinline__ static f32x4 run(const Raw<16>& a, const Raw<16>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

template <class T>
struct Split;
template <>
struct Split<TF16> {
  static constexpr int pieces = 2;
  static constexpr int accumulators = 2;     // hi and lo are summed apart (lo is scaled)
  static constexpr float max_finite = 65504.0f;   // largest value whose hi piece is finite
  __device__ __forceinline__ static void run(float v, uint16_t* out) {
    const _Float16 hi = (_Float16)v;
    const _Float16 lo = (_Float16)((v - (float)hi) * 2048.0f);
    out[0] = __builtin_bit_cast(uint16_t, hi);
    out[1] = __builtin_bit_cast(uint16_t, lo);
  }
  // value of the pieces' products, accumulated apart
  __device__ __forceinline__ static float combine(float a0, float a1) { return a0 + a1 * (1.0f / 2048.0f); }
};
template <>
struct Split<TBF16> {
  static constexpr int pieces = 3;
  static constexpr int accumulators = 1;     // the three pieces share one accumulator
  static constexpr float max_finite = 0.0f;  // no limit: bf16 pieces cover the fp32 range
  __device__ __forceinline__ static void run(float v, uint16_t* out) {
    const __bf16 hi = (__bf16)v;
    const float r1 = v - (float)hi;
    const __bf16 mid = (__bf16)r1;
    const float r2 = r1 - (float)mid;
    const __bf16 lo = (__bf16)r2;
    out[0] = __builtin_bit_cast(uint16_t, hi);
    out[1] = __builtin_bit_cast(uint16_t, mid);
    out[2] = __builtin_bit_cast(uint16_t, lo);
  }
  __device__ __forceinline__ static float combine(float a0, float) { return a0; }
};

__device__ __forceinline__ Raw<16> zero16() {
  Raw<16> z;
  z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0u;
  return z;
}

}  // namespace sfx
