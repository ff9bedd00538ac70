// qi_attn_contract.h -- the frozen per-row arithmetic of the attention
// forward, shared by the fused kernel and the three unfused operators
// (scores, softmax, A.V) so that both use the same constants, the same key
// tiling and the same operand roundings.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// joint_attn_qk_gemm, joint_attn_softmax, joint_attn_av_gemm and
// joint_attention_fused (the fusion must reproduce the composition of the
// three byte for byte); [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Numerical
// requirements".
#pragma once

#include "qi_common.h"
#include "qi_kernels.h"

namespace qi {
namespace attn {

// log2(e) / sqrt(128), rounded once to FP32: p = exp2(s*c - m*c)
constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);
constexpr float kLn2 = 0.69314718055994530942f;
// V enters P*V as FP16 of v * 2^-8; the epilogue divides by l * 2^-8.
constexpr float kVScale = 0x1p-8f;
// Threshold on raw scores for moving the reference max: 8 in the exp2 domain.
constexpr float kTauRaw = (float)(8.0 / (1.4426950408889634074 / 11.313708498984760390));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed FP16 pair (lo = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Logical key tile t of a row with valid text length L: ceil(L/64) text
// tiles from key 0, then image tiles from key T_txt.
__device__ __forceinline__ void tile_bounds(int t, int ntxt, int L, int T_txt, int T_img, int& key0,
                                            int& nvalid) {
  if (t < ntxt) {
    key0 = t * kFwdBN;
    nvalid = min(kFwdBN, L - key0);
  } else {
    const int ti = t - ntxt;
    key0 = T_txt + ti * kFwdBN;
    nvalid = min(kFwdBN, T_img - ti * kFwdBN);
  }
}

// Key (within its 64-key tile) of accumulator register r of a 32x32 score
// block kb, for the half-wave hh: 32*kb + 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ constexpr int score_key(int kb, int r, int hh) {
  return 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
}

}  // namespace attn
}  // namespace qi
