// Device-side helpers shared by the libminf kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/minf.h"

namespace minf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Matrix-core products.  16x16 output tiles; lane l holds column l%16 and
// rows 4*(l/16)+[0..3] of the result.
__device__ __forceinline__ floatx4 mma_bf16(const u32x4& a, const u32x4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_f32(float a, float b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 (round to nearest even), two values packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  floatx2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

template <typename T>
__device__ __forceinline__ T ldg(const T* p) { return *p; }

__device__ __forceinline__ int div_up(int a, int b) { return (a + b - 1) / b; }

// Small per-head table passed by value as a kernel argument.
struct HeadTable {
  int32_t kind[MINF_MAX_HEADS];
  int32_t a[MINF_MAX_HEADS];   // ASHAPE: sink   VSLASH: last_q     BSPARSE: topk
  int32_t b[MINF_MAX_HEADS];   // ASHAPE: window VSLASH: n_vertical BSPARSE: force flags
  int32_t c[MINF_MAX_HEADS];   //                VSLASH: n_slash
};

}  // namespace minf
