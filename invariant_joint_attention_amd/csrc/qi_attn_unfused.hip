// qi_attn_unfused.hip -- the unfused attention forward on gfx950: the score
// GEMM, the masked softmax with fixed tiling, and the A.V GEMM as three
// separate operators with their intermediates in HBM.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// joint_attn_qk_gemm (Q K^T / sqrt(d) over the joint sequence),
// joint_attn_softmax (online softmax over the key sequence with a fixed
// tiling and reduction order), joint_attn_av_gemm (A.V), and
// joint_attention_fused, whose output must equal the composition of these
// three byte for byte; [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Numerical
// requirements" (fused kernels reproduce the unfused result byte for byte).
//
// Each operator performs, per query row, exactly the arithmetic that the
// fused kernel performs for that row, in the same order, with the same
// instructions and operand layouts:
//  * attn_qk_kernel: raw scores q'.k' of each 64-key logical tile, two
//    32-key blocks of v_mfma_f32_32x32x16_bf16 (S^T = K Q^T), the 8 head-dim
//    chunks of a block accumulated in order from zero.  The 1/sqrt(128)
//    scale is not applied here: it enters the softmax's exponent as the FP32
//    constant c = log2(e)/sqrt(128) (p = exp2(s*c - m*c), one fma), which is
//    how the fused kernel applies it.  Masked slots hold -inf.
//  * attn_softmax_kernel: per tile, the exact tile max (both half-rows), the
//    lazy reference max m (moved only when the tile max exceeds it by more
//    than 8/c), alpha = exp2((m_old - m_new) c) (1 where m did not move),
//    p = exp2(s c - m c), and the row sum kept as two half sums (keys
//    8g + 4hh + {0..3} of half hh, in register order) updated as
//    l_hh = l_hh * alpha + sum, then l = l_0 + l_1.  P is stored as FP16
//    (RNE), alpha per (row, tile), and LSE = (m c + log2 l) ln 2.
//  * attn_av_kernel: acc = alpha_t * acc + P_t V_t per tile with
//    v_mfma_f32_32x32x16_f16 on FP16 P and FP16 v * 2^-8 (the transposed key
//    tiles that v_tiles_kernel writes), 16-key chunks in key order; then
//    O = acc / (l 2^-8), one BF16 rounding.
// A factor of exactly 1 leaves a value unchanged, so multiplying every tile
// by alpha gives the bits of the fused kernel, which skips the rescale
// where no row of a wave moved its reference max.
//
// Launch shape (free): 4 waves x 32 query rows per workgroup, one (b, h)
// per grid row; operands are read straight from global memory (L2).
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_attn_contract.h"

namespace qi {

using namespace attn;

namespace {

struct RowTiles {
  int L, ntxt, nt;
};
__device__ __forceinline__ RowTiles row_tiles(const int* txt_len, int b, int T_img) {
  RowTiles r;
  r.L = txt_len[b];
  r.ntxt = (r.L + kFwdBN - 1) / kFwdBN;
  r.nt = r.ntxt + (T_img + kFwdBN - 1) / kFwdBN;
  return r;
}

}  // namespace

__global__ __launch_bounds__(256) void attn_qk_kernel(QkArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qrow = blockIdx.x * kUnfRows + wave * 32 + lr;
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;

  bf16x8 q[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qrow < a.S) z = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
    q[kk] = __builtin_bit_cast(bf16x8, z);
  }
  float* const srow = a.s + (((int64_t)b * a.H + h) * a.S + qrow) * Kp;

  for (int t = 0; t < a.nt_max; ++t) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    int nv = 0;
    if (t < rt.nt) {  // uniform over the workgroup
      int key0;
      tile_bounds(t, rt.ntxt, rt.L, a.T_txt, a.T_img, key0, nv);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // rows past the valid count repeat the last valid row; their scores are masked
        const uint16_t* krow = a.k.row(b, key0 + min(32 * kb + lr, nv - 1), h);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + 16 * kk + 8 * hh));
          if (kk == 0)
            s[kb] = mfma32(kf, q[0], f32x16{});
          else
            s[kb] = mfma32(kf, q[kk], s[kb]);
        }
      }
    }
    if (qrow < a.S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = score_key(kb, 4 * g + e, hh) < nv ? s[kb][4 * g + e] : -INFINITY;
          *(f32x4*)(srow + kFwdBN * t + 32 * kb + 8 * g + 4 * hh) = v;
        }
    }
  }
}

__global__ __launch_bounds__(256) void attn_softmax_kernel(SoftmaxArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qrow = blockIdx.x * kUnfRows + wave * 32 + (lane & 31);
  const int qr = min(qrow, a.S - 1);  // rows past S compute on a valid row and store nothing
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;
  const int64_t row = ((int64_t)b * a.H + h) * a.S + qr;
  const float* const srow = a.s + row * Kp;
  uint16_t* const prow = a.p + row * Kp;
  float* const arow = a.alpha + row * a.nt_max;
  const bool store = qrow < a.S;

  float m_used = -INFINITY, l = 0.f;
  for (int t = 0; t < rt.nt; ++t) {
    f32x16 sx[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = *(const f32x4*)(srow + kFwdBN * t + 32 * kb + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) sx[kb][4 * g + e] = v[e];
      }
    // exact tile max over the row's 64 slots: this half-row, then the other
    float mt = sx[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sx[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sx[1][r]);
    {
      const uint32_t u = __float_as_uint(mt);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool move = mt > m_used + kTauRaw;
    const float m_new = move ? mt : m_used;
    const float alpha = (m_new == m_used) ? 1.0f : __builtin_amdgcn_exp2f((m_used - m_new) * kC);
    l = l * alpha;
    m_used = m_new;
    const float mc = m_used * kC;
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sx[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[kb][r], kC, -mc));
        ts = ts + sx[kb][r];
      }
    l = l + ts;
    if (store) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 pv = {pack_f16x2(sx[kb][4 * g], sx[kb][4 * g + 1]),
                            pack_f16x2(sx[kb][4 * g + 2], sx[kb][4 * g + 3])};
          *(u32x2*)(prow + kFwdBN * t + 32 * kb + 8 * g + 4 * hh) = pv;
        }
      if (hh == 0) arow[t] = alpha;
    }
  }
  if (store) {
    for (int t = rt.nt; t < a.nt_max; ++t) {
      const u32x2 z = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) *(u32x2*)(prow + kFwdBN * t + 8 * j + 4 * hh) = z;
      if (hh == 0) arow[t] = 1.0f;
    }
  }
  const uint32_t lu = __float_as_uint(l);
  const auto sw = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (store && hh == 0) {
    a.l[row] = l_tot;
    a.lse[row] = (m_used * kC + log2f(l_tot)) * kLn2;
  }
}

__global__ __launch_bounds__(256) void attn_av_kernel(AvArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qrow = blockIdx.x * kUnfRows + wave * 32 + lr;
  const int qr = min(qrow, a.S - 1);
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t row = bh * a.S + qr;
  const uint16_t* const prow = a.p + row * Kp;
  const float* const arow = a.alpha + row * a.nt_max;
  const uint16_t* const vt_bh = a.vt + bh * a.nt_max * kVtileElems;

  f32x16 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  for (int t = 0; t < rt.nt; ++t) {
    const float al = arow[t];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = acc[d][r] * al;
    const uint16_t* const vtile = vt_bh + (int64_t)t * kVtileElems;
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      // B operand: P^T rows 8*hh .. 8*hh+7 of chunk c2 = keys 16*c2 + 4*hh + {0..3}, 16*c2 + 8 + 4*hh + {0..3}
      const u32x2 lo = *(const u32x2*)(prow + kFwdBN * t + 16 * c2 + 4 * hh);
      const u32x2 hi = *(const u32x2*)(prow + kFwdBN * t + 16 * c2 + 8 + 4 * hh);
      const u32x4 pw = {lo[0], lo[1], hi[0], hi[1]};
      const f16x8 pf = __builtin_bit_cast(f16x8, pw);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // A operand: V^T channel 32*d + lr, positions 8*hh .. 8*hh+7 of chunk c2 (the tile's key order)
        const u32x4 vw = *(const u32x4*)(vtile + (32 * d + lr) * kFwdBN + 16 * c2 + 8 * hh);
        acc[d] = mfma32h(__builtin_bit_cast(f16x8, vw), pf, acc[d]);
      }
    }
  }
  // O = acc / (l * 2^-8), one RNE cast
  const float l_div = a.l[row] * kVScale;
  if (qrow < a.S) {
    uint16_t* orow = a.o.row(b, qrow, h);
    float* frow = a.of ? a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim : nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        const float o0 = acc[d][4 * g4] / l_div, o1 = acc[d][4 * g4 + 1] / l_div;
        const float o2 = acc[d][4 * g4 + 2] / l_div, o3 = acc[d][4 * g4 + 3] / l_div;
        const u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)(orow + d0) = ov;
        if (frow) *(f32x4*)(frow + d0) = f32x4{o0, o1, o2, o3};
      }
  }
}

}  // namespace qi
