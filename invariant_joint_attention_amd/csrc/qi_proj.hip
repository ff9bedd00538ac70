// qi_proj.hip -- the projections around the attention on gfx950: the packed
// per-stream Q/K/V projection (3072 -> 3 x 3072 + bias at 24 heads) with the
// Q/K prologue (RMSNorm, gain, three-axis RoPE) fused into its epilogue, and
// the per-stream output projection (3072 -> 3072 + bias).
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// qkv_bias_gemm (one weight set per stream), qk_rmsnorm, multi_axis_rope and
// attn_out_bias_gemm; [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Model contract"
// row Streams (text and image tokens keep separate weights) and "Numerical
// requirements" (fixed reduction order, FP32 accumulation, no split-K, one
// cast at the declared output, fused kernels equal to the unfused result).
//
// Arithmetic (frozen):
//  * Y^T = W X^T with v_mfma_f32_32x32x16_bf16: A = 32 output channels (rows
//    of W), B = 32 tokens (rows of X); each output accumulates its K sum in
//    64-element steps in ascending order, 4 MFMAs of 16 per step, from zero,
//    so a row's bits depend on its own X row only (no split-K; the M and N
//    tiling is free).  Then y = acc + bias (FP32) and one RNE cast to BF16.
//  * Fused Q/K prologue: the BF16 y of a Q or K head row goes through the
//    prologue's arithmetic exactly: the sum of squares is formed per 8-channel
//    group in channel order and the 16 group sums are added in the prologue
//    kernel's butterfly order, r = 1/sqrt(sum/128 + eps), t = g (y r), then
//    the rotation with the same FP32 cos/sin (a table written by the
//    prologue's angle code).  The fused output therefore equals the
//    projection followed by qi_qknorm_rope byte for byte.
//
// Schedule (free): workgroup = 8 waves, tile 256 tokens x 256 channels; wave
// w computes 64 tokens (block w % 4) x 128 channels (block w / 4, one head) =
// 8 accumulators of 32x32.  X and W tiles of 64 K-elements sit in LDS as
// 128-byte rows (16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7): the
// fragment reads and the direct-load writes meet no bank conflict), double
// buffered, filled by direct global->LDS loads (waves 0-3 the X rows, waves
// 4-7 the W rows).  Rows past the valid tokens or channels repeat the last
// valid row; their results are not stored.  Tiles never straddle the text /
// image boundary (each stream segment is tiled from its own start).
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_lds.h"
#include "qi_rope.h"

namespace qi {

using namespace lds;

namespace {

constexpr int kPRowB = 128;                // bytes per LDS row: 64 K-elements
constexpr int kPTileB = kProjTile * kPRowB;  // 32 KiB: 256 rows
constexpr int kPStageB = 2 * kPTileB;       // X tile + W tile

// Fixed tree of the prologue's row sum: group sums s[0..15] (channels 8j ..
// 8j+7), then pairs j, j+8; j, j+4; j, j+2; j, j+1.
__device__ __forceinline__ float prologue_tree(const float (&s)[16]) {
  float a[8], b[4], c[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = s[j] + s[j + 8];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = a[j] + a[j + 4];
#pragma unroll
  for (int j = 0; j < 2; ++j) c[j] = b[j] + b[j + 2];
  return c[0] + c[1];
}

}  // namespace

__global__ __launch_bounds__(kProjWaves * 64, 1) void proj_gemm_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kPStageB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // tile: N fastest, then M tiles of the sample (text segment, image segment), then the sample
  int g = blockIdx.x;
  const int nt = g % a.n_nt;
  g /= a.n_nt;
  const int per_b = a.n_mt_txt + a.n_mt_img;
  const int mt = g % per_b, b = g / per_b;
  const bool txt = mt < a.n_mt_txt;
  const int tok0 = txt ? mt * kProjTile : a.T_txt + (mt - a.n_mt_txt) * kProjTile;
  const int tok_end = txt ? a.T_txt : a.S;
  const int stream = (txt || a.weight_streams == 1) ? 0 : 1;
  const int n0 = nt * kProjTile;

  // loader: waves 0-3 fill X rows 64w .. 64w+63, waves 4-7 W rows
  const int sub = wave & 3;
  const bool ldx = wave < 4;
  const int last = ldx ? tok_end - 1 : a.N - 1;
  const int row0 = (ldx ? tok0 : n0) + 64 * sub;
  const int base_row = min(row0, last);
  const int64_t stride = ldx ? a.x_ss : (int64_t)a.K;
  const uint16_t* const src0 =
      ldx ? a.x + (int64_t)b * a.x_sb + (int64_t)base_row * a.x_ss : a.w + ((int64_t)stream * a.N + base_row) * a.K;
  uint32_t off[8];  // load i, lane l: row 8i + l/8, logical chunk (l%8) ^ ((row >> 1) & 7)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int rel = min(row0 + r, last) - base_row;
    off[i] = (uint32_t)rel * (uint32_t)(stride * 2) + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  const uint32_t lds0 = addr_of(smem);
  const uint32_t dst0 = lds0 + (ldx ? 0u : (uint32_t)kPTileB) + (uint32_t)(64 * sub * kPRowB);
  auto load = [&](int ks) {
    const char* src = (const char*)src0 + (int64_t)ks * kProjTK * 2;
    const uint32_t dst = dst0 + (uint32_t)((ks & 1) * kPStageB);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(src, off[i], dst + 1024u * i);
  };

  // fragment bases: X rows 64*(w%4) + 32*tb2 + lr, W rows 128*(w/4) + 32*d + lr
  const int tbw = wave & 3, cbw = wave >> 2;
  const uint32_t xb0 = vt_base(lds0 + (uint32_t)(64 * tbw * kPRowB), lane);
  const uint32_t wb0 = vt_base(lds0 + (uint32_t)kPTileB + (uint32_t)(128 * cbw * kPRowB), lane);

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][d][r] = 0.f;

  const int ns = a.K / kProjTK;
  load(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  bar();
  for (int ks = 0; ks < ns; ++ks) {
    if (ks + 1 < ns) load(ks + 1);
    const uint32_t st = (uint32_t)((ks & 1) * kPStageB);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 f[6];
      const uint32_t xa = (xb0 + st) ^ (uint32_t)(kk << 5), wa = (wb0 + st) ^ (uint32_t)(kk << 5);
      f[0] = ds_b128<0>(xa);
      f[1] = ds_b128<32 * kPRowB>(xa);
      f[2] = ds_b128<0>(wa);
      f[3] = ds_b128<32 * kPRowB>(wa);
      f[4] = ds_b128<64 * kPRowB>(wa);
      f[5] = ds_b128<96 * kPRowB>(wa);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < 6; ++i) asm volatile("" : "+v"(f[i]));
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          acc[tb2][d] = mfma32(__builtin_bit_cast(bf16x8, f[2 + d]), __builtin_bit_cast(bf16x8, f[tb2]), acc[tb2][d]);
    }
    // next stage landed (every wave's loads); every wave is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bar();
  }

  // ---- epilogue: y = acc + bias, one RNE cast; Q/K heads optionally through the prologue
  const int ch_w = n0 + 128 * cbw;  // this wave's 128 channels: one head of one section
  if (ch_w >= a.N) return;
  const int section = ch_w / a.D, head = (ch_w - section * a.D) / kHeadDim;
  const float* const bias = a.bias + (int64_t)stream * a.N + ch_w;
  const View<uint16_t> out = a.out[section];
  const bool fused = a.fuse && section < 2;
  const float* gain = nullptr;
  if (fused) gain = (section == 0 ? a.gain_q : a.gain_k);
#pragma unroll
  for (int tb2 = 0; tb2 < 2; ++tb2) {
    const int tok = tok0 + 64 * tbw + 32 * tb2 + lr;
    // channel of register (d, 4g+e): 32d + 8g + 4hh + e
    float y[4][16];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 bv = *(const f32x4*)(bias + 32 * d + 8 * g4 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[tb2][d][4 * g4 + e] + bv[e];
          y[d][4 * g4 + e] = bf16_lo(pack_bf16x2(v, 0.f) & 0xffffu);  // BF16 value, widened
        }
      }
    if (fused) {
      // group sums of squares (group j = 4d + g4: channels 8j .. 8j+7, the
      // first four in half 0, the last four in half 1), in channel order
      float part[16];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float ss = y[d][4 * g4] * y[d][4 * g4];
#pragma unroll
          for (int e = 1; e < 4; ++e) {
            const float sq = y[d][4 * g4 + e] * y[d][4 * g4 + e];
            ss = ss + sq;
          }
          part[4 * d + g4] = ss;
        }
      float s16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float ss = __shfl_xor(part[j], 32);  // half 1 receives the first four channels' sum
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = j >> 2, g4 = j & 3;
          const float sq = y[d][4 * g4 + e] * y[d][4 * g4 + e];
          ss = ss + sq;
        }
        s16[j] = ss;
      }
      float r = 0.f;
      if (hh == 1) {
        const float ms = prologue_tree(s16) / 128.0f;
        r = 1.0f / sqrtf(ms + a.eps);
      }
      r = __shfl(r, lr + 32);  // both halves: the row's 1/rms from half 1
      const int s = tok < a.S ? tok : a.S - 1;
      const float* gp = gain + ((a.gain_streams == 2 && s >= a.T_txt) ? kHeadDim : 0);
      const float* cs = a.rope + (int64_t)s * 128;  // (cos, sin) of the 64 pairs
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c0 = 32 * d + 8 * g4 + 4 * hh;
          const f32x4 gv = *(const f32x4*)(gp + c0);
          const f32x4 rc = *(const f32x4*)(cs + c0);  // pairs c0/2, c0/2 + 1
          float t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xh = y[d][4 * g4 + e] * r;
            t[e] = gv[e] * xh;
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float c = rc[2 * u], sn = rc[2 * u + 1];
            const float q0 = t[2 * u] * c, q1 = t[2 * u + 1] * sn, q2 = t[2 * u] * sn, q3 = t[2 * u + 1] * c;
            y[d][4 * g4 + 2 * u] = q0 - q1;
            y[d][4 * g4 + 2 * u + 1] = q2 + q3;
          }
        }
    }
    if (tok < tok_end) {
      uint16_t* orow = out.row(b, tok, head);
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x2 ov = {pack_bf16x2(y[d][4 * g4], y[d][4 * g4 + 1]), pack_bf16x2(y[d][4 * g4 + 2], y[d][4 * g4 + 3])};
          *(u32x2*)(orow + 32 * d + 8 * g4 + 4 * hh) = ov;
        }
    }
  }
}

// cos/sin of the 64 rotation pairs of every token position: table[s][k] =
// (cos, sin), from the prologue's own angle code (FP64, rounded once).
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.S * 64) return;
  const int s = (int)(i >> 6), k = (int)(i & 63);
  int p0, p1, p2;
  token_position(s, a.T_txt, a.gh, a.gw, p0, p1, p2);
  float c, sn;
  pair_cos_sin(k, p0, p1, p2, a.theta, c, sn);
  a.table[2 * i] = c;
  a.table[2 * i + 1] = sn;
}

}  // namespace qi
