// qi_common.h -- types and small device helpers shared by the gfx950 kernels.
//
// Everything here is written for CDNA4 (gfx950) wave64 execution.  The MFMA
// operand layouts below were checked on the device:
//   v_mfma_f32_32x32x16_bf16: A lane l holds A[l%32][8*(l/32) + t], t=0..7;
//     B lane l holds B[8*(l/32) + t][l%32]; accumulator register r of lane l
//     holds C[8*(r/4) + 4*(l/32) + r%4][l%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qi {

constexpr int kHeadDim = 128;
constexpr int kMaxBatchPerLaunch = 64;  // txt_len travels in the kernel arguments

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed BF16 pair (lo = a, hi = b), round to nearest
// even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// Exact widening of the low / high BF16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Strided [B, S, H, 128] view, strides in elements.
template <typename T>
struct View {
  T* p;
  int64_t sb, ss, sh;
  __device__ __forceinline__ T* row(int b, int s, int h) const {
    return p + (int64_t)b * sb + (int64_t)s * ss + (int64_t)h * sh;
  }
};

}  // namespace qi
