// qi_prologue.hip -- the Q/K prologue on gfx950: learned-gain per-head
// RMSNorm, three-axis rotary embedding and the single FP32->BF16 cast, plus
// its backward (inverse rotation, RMSNorm backward, gain-gradient partials).
//
// Pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
// ablation matrix and integration plan", "Model contract" rows Q/K
// preprocessing and RoPE; [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU
// Kernel List", rows qk_rmsnorm and multi_axis_rope; the learned-gain comment
// of [Roadmap] (gain of 128 entries, backward yields dx and the gain grad).
//
// Mapping: one wave per token.  Lane k (0..63) first forms the FP64 angle of
// rotation pair k at the token's position and rounds cos/sin once to FP32;
// then each group of 16 lanes takes one head row (16 B = 8 channels = 4
// pairs per lane), so a wave streams 4 rows (1 KiB contiguous for dense
// heads) per step.  The kernel is HBM-bound: it reads and writes each
// element once.  The row sum of squares is summed in a fixed tree: 8
// sequential terms per lane, then xor-butterflies over 8, 4, 2, 1 lanes
// (each lane ends with the same bits because FP addition is commutative).
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_rope.h"
#include "qi_vtiles.h"

namespace qi {

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

// Sum over the 16 lanes of a row group, fixed xor tree.
__device__ __forceinline__ float row16_sum(float v) {
  v = v + __shfl_xor(v, 8);
  v = v + __shfl_xor(v, 4);
  v = v + __shfl_xor(v, 2);
  v = v + __shfl_xor(v, 1);
  return v;
}

// 1/sqrt(mean(x^2) + eps) of one row: 8 squares per lane in order, then the
// 16-lane tree.  sqrtf and '/' compile to correctly rounded sequences.
__device__ __forceinline__ float row_rinv(const float* xf, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sq = xf[i] * xf[i];
    ss = ss + sq;
  }
  ss = row16_sum(ss);
  const float ms = ss / 128.0f;
  return 1.0f / sqrtf(ms + eps);
}

// Tokens 4 blk .. 4 blk + 3 of the launch, one per wave.  With kPre > 0
// the rows of the first kPre head groups are loaded before the token's
// angles are formed, so their loads are in flight during the FP64 rotation
// code (branch-free: lanes past the last head load its row and drop it).
// The loads' timing changes no bit.
template <int kPre>
__device__ __forceinline__ void prologue_body(const PrologueArgs& a, int64_t blk) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = blk * 4 + (threadIdx.x >> 6);
  if (tok >= (int64_t)a.B * a.S) return;  // wave-uniform; no block barrier follows
  const int b = (int)(tok / a.S), s = (int)(tok - (int64_t)b * a.S);

  const int j = lane & 15;  // channel group: channels 8j..8j+7, pairs 4j..4j+3
  const float* gp = a.gain + ((a.gain_streams == 2 && s >= a.T_txt) ? kHeadDim : 0) + 8 * j;
  const f32x4 g0 = *(const f32x4*)gp, g1 = *(const f32x4*)(gp + 4);
  const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
  u32x4 xpre[kPre > 0 ? kPre : 1];
#pragma unroll
  for (int gi = 0; gi < kPre; ++gi) {
    const int h = min(4 * gi + (lane >> 4), a.H - 1);
    xpre[gi] = *(const u32x4*)(a.x.row(b, s, h) + 8 * j);
  }

  int p0, p1, p2;
  token_position(s, a.T_txt, a.gh, a.gw, p0, p1, p2);
  float cl, sl;
  pair_cos_sin(lane, p0, p1, p2, a.theta, cl, sl);

  float c[4], sn[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    c[u] = __shfl(cl, 4 * j + u);
    sn[u] = __shfl(sl, 4 * j + u);
  }

  auto row = [&](int h0, const u32x4& xraw) {
    const int h = h0 + (lane >> 4);
    const bool active = h < a.H;
    const u32x4 xv = active ? xraw : u32x4{0u, 0u, 0u, 0u};
    float xf[8];
    unpack8(xv, xf);
    const float r = row_rinv(xf, a.eps);
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xh = xf[i] * r;
      t[i] = g[i] * xh;
    }
    float yo[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float y0 = t[2 * u], y1 = t[2 * u + 1];
      const float q0 = y0 * c[u], q1 = y1 * sn[u], q2 = y0 * sn[u], q3 = y1 * c[u];
      yo[2 * u] = q0 - q1;
      yo[2 * u + 1] = q2 + q3;
    }
    if (active) {
      u32x4 ov;
#pragma unroll
      for (int u = 0; u < 4; ++u) ov[u] = pack_bf16x2(yo[2 * u], yo[2 * u + 1]);
      *(u32x4*)(a.y.row(b, s, h) + 8 * j) = ov;
      if (a.yf) {
        float* dst = a.yf + (((int64_t)b * a.S + s) * a.H + h) * kHeadDim + 8 * j;
        *(f32x4*)dst = f32x4{yo[0], yo[1], yo[2], yo[3]};
        *(f32x4*)(dst + 4) = f32x4{yo[4], yo[5], yo[6], yo[7]};
      }
    }
  };
#pragma unroll
  for (int gi = 0; gi < kPre; ++gi)
    if (4 * gi < a.H) row(4 * gi, xpre[gi]);
  for (int h0 = 4 * kPre; h0 < a.H; h0 += 4) {
    const int h = h0 + (lane >> 4);
    u32x4 xv = {0u, 0u, 0u, 0u};
    if (h < a.H) xv = *(const u32x4*)(a.x.row(b, s, h) + 8 * j);
    row(h0, xv);
  }
}

// Alone, the kernel measured faster without the early loads (12.5 against
// 13.2 us at 1024^2); the one-launch preparation below, which runs the K rows
// and V tiles beside it, measured faster with them (25.8 against 27.2 us).
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(PrologueArgs a) { prologue_body<0>(a, blockIdx.x); }

// The Q and K prologues and the V tile conversion of a forward in one launch:
// blocks [0, nblk) take Q's tokens, [nblk, 2 nblk) K's, and the rest one V
// key tile each, (t, h, b) in row-major order.  Each part runs exactly the
// arithmetic of its own kernel, so every output byte is the same.
__global__ __launch_bounds__(256) void qkv_prologue_kernel(QkvPrologueArgs a) {
  const int64_t bx = blockIdx.x;
  if (bx < a.nblk) {
    prologue_body<8>(a.q, bx);
  } else if (bx < 2 * a.nblk) {
    prologue_body<8>(a.k, bx - a.nblk);
  } else {
    const int64_t r = bx - 2 * a.nblk;
    const int64_t th = r / a.v.nt_max;
    v_tile_body(a.v, (int)(r - th * a.v.nt_max), (int)(th % a.v.H), (int)(th / a.v.H));
  }
}

// Backward of the prologue, in place on the FP32 gradient buffer: dq' -> dq.
// One workgroup owns a chunk of kChunk consecutive tokens of one stream
// segment (text tokens [0,T_txt) and image tokens [T_txt,S) are chunked
// from their own starts), so its gain-gradient partial is a fixed sum that
// depends only on the sample's own rows: wave w takes tokens 4w..4w+3 of the
// chunk in order; inside a wave each lane accumulates its 8 channels over
// its rows, the four lane groups are combined by an xor tree (16, 32), and
// the four waves are added in order 0,1,2,3.
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(PrologueBwdPair p) {
  const PrologueBwdArgs a = blockIdx.z ? p.t[1] : p.t[0];  // Q's or K's gradient (uniform)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int chunk = blockIdx.x;  // 0 .. n_txt_chunks + n_img_chunks - 1
  int seg_start, seg_end, c0;
  if (chunk < a.n_txt_chunks) {
    seg_start = 0; seg_end = a.T_txt; c0 = chunk * kPrologueChunk;
  } else {
    seg_start = a.T_txt; seg_end = a.S; c0 = a.T_txt + (chunk - a.n_txt_chunks) * kPrologueChunk;
  }
  (void)seg_start;
  const int j = lane & 15;
  const int set = (a.gain_streams == 2 && c0 >= a.T_txt) ? 1 : 0;
  const float* gp = a.gain + set * kHeadDim + 8 * j;
  const f32x4 g0 = *(const f32x4*)gp, g1 = *(const f32x4*)(gp + 4);
  const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};

  float dg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dg[i] = 0.f;

  for (int it = 0; it < kPrologueChunk / 4; ++it) {
    const int s = c0 + 4 * wave + it;
    if (s >= seg_end) break;  // wave-uniform
    int p0, p1, p2;
    token_position(s, a.T_txt, a.gh, a.gw, p0, p1, p2);
    float cl, sl;
    pair_cos_sin(lane, p0, p1, p2, a.theta, cl, sl);
    float c[4], sn[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = __shfl(cl, 4 * j + u);
      sn[u] = __shfl(sl, 4 * j + u);
    }
    for (int h0 = 0; h0 < a.H; h0 += 4) {
      const int h = h0 + (lane >> 4);
      const bool active = h < a.H;
      u32x4 xv = {0u, 0u, 0u, 0u};
      f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
      float* gd = active ? a.dx.row(b, s, h) + 8 * j : nullptr;
      if (active) {
        xv = *(const u32x4*)(a.x.row(b, s, h) + 8 * j);
        d0 = *(const f32x4*)gd;
        d1 = *(const f32x4*)(gd + 4);
      }
      float xf[8];
      unpack8(xv, xf);
      const float r = row_rinv(xf, a.eps);
      const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      float u8[8], xh[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float e0 = dv[2 * u], e1 = dv[2 * u + 1];
        const float q0 = e0 * c[u], q1 = e1 * sn[u], q2 = e0 * sn[u], q3 = e1 * c[u];
        u8[2 * u] = q0 + q1;
        u8[2 * u + 1] = q3 - q2;
      }
      float dot = 0.f, dxh[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xh[i] = xf[i] * r;
        const float pr = u8[i] * xh[i];
        dg[i] = dg[i] + (active ? pr : 0.f);
        dxh[i] = u8[i] * g[i];
        const float pd = dxh[i] * xh[i];
        dot = dot + pd;
      }
      dot = row16_sum(dot);
      const float mean = dot / 128.0f;
      if (active) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float tt = xh[i] * mean;
          o[i] = r * (dxh[i] - tt);
        }
        *(f32x4*)gd = f32x4{o[0], o[1], o[2], o[3]};
        *(f32x4*)(gd + 4) = f32x4{o[4], o[5], o[6], o[7]};
      }
    }
  }
  // combine the four lane groups of this wave (same channels), fixed tree
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dg[i] = dg[i] + __shfl_xor(dg[i], 16);
    dg[i] = dg[i] + __shfl_xor(dg[i], 32);
  }
  __shared__ float part[4][kHeadDim];
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) part[wave][8 * j + i] = dg[i];
  }
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int cc = threadIdx.x;
    float v = part[0][cc];
    v = v + part[1][cc];
    v = v + part[2][cc];
    v = v + part[3][cc];
    a.partials[((int64_t)b * a.n_chunks + chunk) * kHeadDim + cc] = v;
  }
}

// Fold the chunk partials of each sample and gain set in ascending chunk
// order, then (one thread per channel and set) the per-sample results in
// ascending b.  Grid: (gain_streams, 2 gains); block: 4 x 128 threads.
// The adds are one thread per channel, in chunk order; all 512 threads load
// the partials into LDS 64 chunks at a time, and the next batch's loads are
// in flight while the current batch is added, so the chain waits on memory
// about once per sample instead of once per batch.
constexpr int kFoldBatch = 64;
constexpr int kFoldThreads = 4 * kHeadDim;
__global__ __launch_bounds__(kFoldThreads) void dgain_fold_kernel(DgainFoldPair p) {
  const DgainFoldArgs a = blockIdx.y ? p.t[1] : p.t[0];  // Q's or K's gain (uniform)
  const int set = blockIdx.x, tid = threadIdx.x, cc = tid & (kHeadDim - 1), grp = tid >> 7;
  __shared__ float buf[kFoldBatch][kHeadDim];
  int k0, k1;
  if (a.gain_streams == 2) {
    k0 = set == 0 ? 0 : a.n_txt_chunks;
    k1 = set == 0 ? a.n_txt_chunks : a.n_chunks;
  } else {
    k0 = 0;
    k1 = a.n_chunks;
  }
  float tot = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const float* src = a.partials + (int64_t)b * a.n_chunks * kHeadDim + cc;
    float x[kFoldBatch / 4];  // chunks base + 4j + grp of the batch this thread loads
    auto fetch = [&](int base) {
#pragma unroll
      for (int j = 0; j < kFoldBatch / 4; ++j) {
        const int k = base + 4 * j + grp;
        x[j] = k < k1 ? src[(int64_t)k * kHeadDim] : 0.f;
      }
    };
    fetch(k0);
    float v = 0.f;
    for (int base = k0; base < k1; base += kFoldBatch) {
      __syncthreads();  // the previous batch's adds are done with buf
#pragma unroll
      for (int j = 0; j < kFoldBatch / 4; ++j) buf[4 * j + grp][cc] = x[j];
      __syncthreads();
      if (base + kFoldBatch < k1) fetch(base + kFoldBatch);
      if (tid < kHeadDim) {  // the batch's reads all issued, then the adds in chunk order
        const int n = min(kFoldBatch, k1 - base);
        float y[kFoldBatch];
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j) y[j] = buf[j][cc];
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j)
          if (j < n) v = v + y[j];
      }
    }
    if (tid < kHeadDim) {
      a.dg_ps[((int64_t)b * a.gain_streams + set) * kHeadDim + cc] = v;
      tot = tot + v;
    }
  }
  if (tid < kHeadDim && a.dg) a.dg[set * kHeadDim + cc] = tot;
}

}  // namespace qi
