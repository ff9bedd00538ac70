// qi_attn_merge.hip -- fixed-order merge of key-block row states on gfx950.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", row
// joint_attention_fused (marked for Ulysses / Ring sequence parallelism);
// [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap, ablation
// matrix and integration plan", "Numerical requirements" (fixed reduction
// order, one output cast).  The row states come from attn_fwd_partial_kernel
// (the forward kernel's tile loop over one key block); this pass is
// HBM-bound: it reads n states of 520 bytes per row (each byte once, so with
// the non-temporal hint) and writes O and LSE.
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_attn_contract.h"

namespace qi {

using namespace attn;

// Merge of key-block row states in the fixed block order k = 0, 1, ...:
// m = max_k m_k; alpha_k = exp2((m_k - m) c); acc = alpha_0 acc_0 + alpha_1
// acc_1 + ...; l likewise; then the forward's epilogue, O = acc / (l 2^-8)
// and LSE = (m c + log2 l) ln 2.  With one block alpha_0 = exp2(0) = 1 and
// the result is the whole-row forward's, bit for bit.  A block without keys
// for a row (m = -inf, acc = l = 0) gets alpha = 0.  32 lanes per row, 4
// channels per lane; the states are read eight blocks at a time (all their
// loads in flight together), then folded one by one in block order.
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int kU = 8;  // blocks per batch of loads
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= a.rows) return;
  const int c0 = 4 * (threadIdx.x & 31);
  float m = -INFINITY;
  for (int k0 = 0; k0 < a.n; k0 += kU) {
    float mk[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) mk[j] = k0 + j < a.n ? a.m[(k0 + j) * a.rows + row] : -INFINITY;
#pragma unroll
    for (int j = 0; j < kU; ++j) m = fmaxf(m, mk[j]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int k0 = 0; k0 < a.n; k0 += kU) {
    float mk[kU], lk[kU];
    f32x4 xk[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int k = k0 + j;
      if (k < a.n) {
        mk[j] = a.m[k * a.rows + row];
        lk[j] = a.l[k * a.rows + row];
        xk[j] = __builtin_nontemporal_load((const f32x4*)(a.acc + (k * a.rows + row) * kHeadDim + c0));
      }
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int k = k0 + j;
      if (k < a.n) {
        const float al = __builtin_amdgcn_exp2f((mk[j] - m) * kC);
        if (k == 0) {
          for (int e = 0; e < 4; ++e) acc[e] = al * xk[j][e];
          l = al * lk[j];
        } else {
          for (int e = 0; e < 4; ++e) acc[e] = acc[e] + al * xk[j][e];
          l = l + al * lk[j];
        }
      }
    }
  }
  const float l_div = l * kVScale;
  const int64_t bh = row / a.S;
  const int qrow = (int)(row - bh * a.S);
  const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
  const float o0 = acc[0] / l_div, o1 = acc[1] / l_div, o2 = acc[2] / l_div, o3 = acc[3] / l_div;
  const u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
  *(u32x2*)(a.o.row(b, qrow, h) + c0) = ov;
  if (a.of) *(f32x4*)(a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim + c0) = f32x4{o0, o1, o2, o3};
  if (c0 == 0) a.lse[row] = (m * kC + log2f(l)) * kLn2;
}

}  // namespace qi
