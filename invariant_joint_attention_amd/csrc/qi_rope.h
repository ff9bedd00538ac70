// qi_rope.h -- positions and rotation angles of the three-axis rotary
// embedding, shared by the prologue kernels and the cos/sin table that the
// fused QKV projection reads (so both use the same FP32 values).
//
// Pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
// ablation matrix and integration plan", "Model contract" row RoPE (axes of
// 16/56/56 channels, theta, centred image indices, text offset max(h/2, w/2));
// [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", row
// multi_axis_rope (text on the grid diagonal).
#pragma once

#include "qi_common.h"

namespace qi {

// Position triple of token s ([Roadmap] row RoPE; [Kernel list] row
// multi_axis_rope): image tokens are centred, text sits on the diagonal.
__device__ __forceinline__ void token_position(int s, int T_txt, int gh, int gw, int& p0,
                                               int& p1, int& p2) {
  if (s < T_txt) {
    const int o = max(gh / 2, gw / 2);
    p0 = p1 = p2 = o + s;
  } else {
    const int t = s - T_txt;
    const int row = t / gw, col = t - row * gw;
    p0 = 0;
    p1 = row - (gh + 1) / 2;
    p2 = col - (gw + 1) / 2;
  }
}

// cos/sin of pair k (axes of 16/56/56 channels = 8/28/28 pairs), angle
// p_axis * theta^(-2i/d) formed in FP64 and rounded once to FP32.
__device__ __forceinline__ void pair_cos_sin(int k, int p0, int p1, int p2, double theta,
                                             float& c, float& s) {
  int i, d, p;
  if (k < 8) { i = k; d = 16; p = p0; }
  else if (k < 36) { i = k - 8; d = 56; p = p1; }
  else { i = k - 36; d = 56; p = p2; }
  const double omega = pow(theta, -2.0 * (double)i / (double)d);
  const double phi = (double)p * omega;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

}  // namespace qi
