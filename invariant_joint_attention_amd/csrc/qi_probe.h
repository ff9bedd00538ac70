// qi_probe.h -- the strict-arithmetic probe: a kernel built with the
// library's own compiler flags, run once per device, whose results must
// equal the strict (IEEE, no fast math) values.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List",
// rule 4 (no fast math); [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Numerical
// requirements" (unsupported strict configurations fail closed); [PR 537]
// "[WS1][Qwen-Image][CUDA] AdaLN modulation projection
// (adaln_mod_projection)": a probe of the built arithmetic, verdict kept per
// device.
//
// Every check has an answer that a build with relaxed floating point
// changes: a flushed subnormal, an approximate division or square root, a
// contracted multiply-add (x*x - y is 2^-24 as an fma, 0 rounded twice), a
// NaN test folded away under finite-math assumptions.  The inputs arrive as
// kernel arguments, so the compiler cannot evaluate any of it ahead of time.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qi_common.h"

namespace qi {
namespace probe {

constexpr int kChecks = 7;
static __device__ uint32_t g_probe_out[8];

static __global__ void strict_probe_kernel(float sub, float three, float two, float tie1, float tie2, float zero,
                                           float x, float y, float nan_in) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  g_probe_out[0] = __float_as_uint(sub * 1.5f);   // subnormal survives (no flush)
  g_probe_out[1] = __float_as_uint(1.0f / three); // correctly rounded division
  g_probe_out[2] = __float_as_uint(sqrtf(two));   // correctly rounded square root
  g_probe_out[3] = pack_bf16x2(tie1, tie2);       // FP32 -> BF16 ties to even
  g_probe_out[4] = __float_as_uint(__builtin_amdgcn_exp2f(zero));  // exp2(0) == 1 exactly
  const float prod = x * x;                        // no contraction into an fma
  g_probe_out[5] = __float_as_uint(prod - y);
  g_probe_out[6] = (nan_in != nan_in) ? 1u : 0u;   // NaN compares unequal (no finite-math folding)
}

static inline uint32_t f2u(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// Runs the probe on the current device (default stream, synchronous read
// back).  Returns 0, or 6 (strict check failed) / 7 (HIP error) with a
// message in msg.
static inline int run(int dev, char* msg, size_t n) {
  const float sub = std::ldexp(1.0f, -140), three = 3.0f, two = 2.0f;
  const float tie1 = 1.0f + std::ldexp(1.0f, -8), tie2 = 1.0f + 3.0f * std::ldexp(1.0f, -8);
  const float x = 1.0f + std::ldexp(1.0f, -12), y = 1.0f + std::ldexp(1.0f, -11);
  uint32_t nan_bits = 0x7fc00000u;
  float nan_in;
  std::memcpy(&nan_in, &nan_bits, 4);
  hipLaunchKernelGGL(strict_probe_kernel, dim3(1), dim3(64), 0, 0, sub, three, two, tie1, tie2, 0.0f, x, y,
                     nan_in);
  if (hipGetLastError() != hipSuccess) {
    snprintf(msg, n, "strict probe launch failed on device %d", dev);
    return 7;
  }
  uint32_t out[8] = {0};
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_probe_out), sizeof out, 0, hipMemcpyDeviceToHost) != hipSuccess) {
    snprintf(msg, n, "strict probe readback failed on device %d", dev);
    return 7;
  }
  volatile float vthree = three, vtwo = two;
  const uint32_t want[kChecks] = {f2u(std::ldexp(3.0f, -141)), f2u(1.0f / vthree), f2u(std::sqrt(vtwo)),
                                  0x3F823F80u, f2u(1.0f), 0u, 1u};
  const char* what[kChecks] = {"subnormal multiply", "division rounding", "sqrt rounding", "bf16 RNE",
                               "exp2(0)", "no fma contraction", "NaN != NaN"};
  for (int i = 0; i < kChecks; ++i)
    if (out[i] != want[i]) {
      snprintf(msg, n, "strict probe failed on device %d: %s (got 0x%08x want 0x%08x)", dev, what[i], out[i],
               want[i]);
      return 6;
    }
  return 0;
}

}  // namespace probe
}  // namespace qi
