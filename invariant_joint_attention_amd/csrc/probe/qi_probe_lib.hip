// qi_probe_lib.hip -- the strict-arithmetic probe of qi_probe.h as a library
// of its own, so that the probe can be built with other compiler flags than
// the attention library.  The build compiles it with -ffast-math into
// libqi_probe_fastmath.so: on a GPU its verdict must be the strict failure
// code, which shows that the probe libqi.so runs at start-up detects a
// relaxed build ([Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel
// List", rule 4, no fast math; [PR 537] "[WS1][Qwen-Image][CUDA] AdaLN
// modulation projection (adaln_mod_projection)", a probe that flips under
// fast math).
#include "../qi_probe.h"

extern "C" {

// Runs the probe on `device`: 0 = strict arithmetic, 6 = a check failed,
// 7 = HIP error (msg receives the reason).
int qi_probe_standalone(int device, char* msg, int msg_bytes) {
  if (hipSetDevice(device) != hipSuccess) {
    snprintf(msg, (size_t)msg_bytes, "HIP device %d not available", device);
    return 7;
  }
  return qi::probe::run(device, msg, (size_t)msg_bytes);
}
}
