// qi_vtiles.h -- the V -> FP16 V^T key-tile conversion of one (tile, head,
// sample), shared by the forward's own conversion kernel and by the fused
// Q/K/V prologue launch.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", row
// joint_attn_av_gemm (A.V over a fixed key tiling); the operand format is
// this library's own (FP16 P times FP16 v * 2^-8).
#pragma once
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_attn_contract.h"

namespace qi {

// One logical key tile t of (b, h): the tile's valid key rows are staged in
// LDS as BF16, then written out as 128 channel rows of 64 FP16 values
// v * 2^-8 (the multiply is exact, the conversion rounds to nearest even),
// the keys of each 16-key chunk in the A.V reduction order (position p holds
// key p with bits 2 and 3 swapped).  Keys past the tile's valid count are
// written as zero, so the attention kernel loads whole tiles and a masked
// key's V slot is exactly zero.  For a key-block forward only the block's
// tiles are converted.  256 threads; every thread of the workgroup calls it
// with the same (t, h, b).
__device__ __forceinline__ void v_tile_body(const VtileArgs& a, int t, int h, int b) {
  __shared__ uint32_t tl[kFwdBN][kHeadDim / 2 + 1];  // [key][channel pair]; one pad word per row
  const int L = a.txt_len[b];
  const int ntxt = (L + kFwdBN - 1) / kFwdBN;
  const int nt = ntxt + (a.T_img + kFwdBN - 1) / kFwdBN;
  if (t >= nt) return;
  if (t < ntxt ? !a.with_text : (t - ntxt < a.img_t0 || t - ntxt >= a.img_t1)) return;  // outside the key block
  int key0, nvalid;
  attn::tile_bounds(t, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
  for (int i = threadIdx.x; i < kFwdBN * 16; i += 256) {
    const int key = i >> 4, c = i & 15;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < nvalid) w = *(const u32x4*)(a.v.row(b, key0 + key, h) + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) tl[key][4 * c + e] = w[e];
  }
  __syncthreads();
  uint16_t* const out = a.out + (((int64_t)b * a.H + h) * a.nt_max + t) * kVtileElems;
  for (int i = threadIdx.x; i < kHeadDim * 8; i += 256) {
    const int d = i >> 3, j = i & 7;  // channel row, 8-key chunk of the row
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = 8 * (j & 1) + e;  // position within 16-key chunk j/2
      const int key = 16 * (j >> 1) + ((p & 3) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3));
      const uint32_t w = tl[key][d >> 1];
      f[e] = ((d & 1) ? bf16_hi(w) : bf16_lo(w)) * attn::kVScale;
    }
    const u32x4 o = {attn::pack_f16x2(f[0], f[1]), attn::pack_f16x2(f[2], f[3]), attn::pack_f16x2(f[4], f[5]),
                     attn::pack_f16x2(f[6], f[7])};
    *(u32x4*)(out + d * kFwdBN + 8 * j) = o;
  }
}

}  // namespace qi
