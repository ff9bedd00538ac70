// qi_attn_fwd.hip -- masked non-causal joint attention forward on gfx950.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// joint_attn_qk_gemm, joint_attn_softmax, joint_attn_av_gemm and
// joint_attention_fused; [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Model contract"
// rows Streams and Text input, and "Numerical requirements" (fixed reduction
// trees, FP32 accumulation, no split-KV, one output cast, batch invariance).
//
// Design (per workgroup: 4 waves x 32 query rows of one (b, h)):
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    A = a 32-key block of K read from LDS, B = the wave's Q rows, kept in
//    registers for the whole key loop.  Lane l then owns query l%32 and 16
//    keys per block, so the row max is an in-lane max plus one exchange with
//    lane l^32, and the softmax rescale factor is a per-lane scalar.
//  * O^T = V^T P^T accumulates in 4 blocks of 32x32 FP32 (64 registers).  P
//    is taken straight from the score accumulators and enters the MFMA as two
//    BF16 terms, hi = bf16(p) and lo = bf16(p - hi), accumulated hi then lo:
//    one BF16 rounding of P alone would move O by up to 2^-9 * sum_j p_j|v_j|,
//    which breaks the output tolerance where O cancels on few, peaked keys.
//    The MFMA reduction index is a permutation of the 16 keys of a chunk
//    (bits 2 and 3 of the key index swapped) that matches the accumulator
//    layout of P; the transposing V reads fetch the keys in that order.
//  * Keys are tiled LOGICALLY: ceil(L_b/64) text tiles starting at key 0,
//    then ceil(T_img/64) image tiles starting at key T_txt.  Masked keys are
//    never read (their LDS slots are zero) and get probability exactly 0, so
//    a row's arithmetic does not depend on T_txt, on the batch or on the
//    workgroup shape.  The key tile width 64 is frozen; rows per workgroup,
//    grid order and LDS layout are free.
//  * Online softmax in the exp2 domain with c = log2(e)/sqrt(128):
//    p = exp2(s*c - m*c) (one fma); the row sum l adds the FP32 p lane by lane
//    in register order, then the two half-waves (commutative, so both get the
//    same bits); O = acc / l and LSE = (m*c + log2 l) * ln 2.
//    The reference max m moves only when a tile max exceeds it by more than
//    8/c (so p <= 256): each lane decides from its own row alone, and the
//    rescale (factor exactly 1 where m did not move) is skipped when no lane
//    of the wave moved.
//  * K/V tiles are double-buffered in LDS and filled by direct global->LDS
//    loads (global_load_lds_dwordx4, no registers), issued for tile t+1
//    while tile t is multiplied.  Rows are unpadded 256-byte lines whose
//    16-byte chunks are XOR-swizzled by key, so the K fragment reads, the V
//    transposing reads and the loads' contiguous LDS writes avoid bank
//    conflicts.  V stays row-major: ds_read_b64_tr_b16 delivers the
//    transposed V^T fragment of the A*V product straight from LDS.
//  * Two waves per SIMD (at most 256 VGPRs), 4 waves x 32 rows per
//    workgroup; s_setprio raises the MFMA sections' priority so one wave's
//    softmax overlaps the other wave's matrix work.
#include "qi_common.h"
#include "qi_kernels.h"

namespace qi {

namespace {

constexpr int kRowB = 256;                   // bytes per K / V row in LDS (unpadded, chunk-swizzled)
constexpr int kTileB = kFwdBN * kRowB;       // 16384
constexpr int kBufBytes = 2 * kTileB;        // K tile then V tile
// log2(e) / sqrt(128), rounded once to FP32
constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);
constexpr float kLn2 = 0.69314718055994530942f;
// Threshold on raw scores for moving the reference max: 8 in the exp2 domain.
constexpr float kTauRaw = (float)(8.0 / (1.4426950408889634074 / 11.313708498984760390));

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;

// 16-byte chunk c of key row `key` lives at chunk c ^ swz(key): conflict-free
// for the K fragment reads (8 consecutive keys), the transposing V reads
// (4 consecutive keys x 2 chunks) and the contiguous direct-load writes.
__device__ __forceinline__ int swz(int key) {
  return ((key & 3) << 1) | ((key >> 2) & 1) | (key & 8);
}
__device__ __forceinline__ int lds_off(int key, int chunk) {
  return key * kRowB + 16 * (chunk ^ swz(key));
}

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

// Global -> LDS without registers (global_load_lds_dwordx4): wave w fills
// keys 16w..16w+15 of the K and V tiles, 4 keys (1 KiB) per instruction;
// lane l writes LDS slot l of the instruction's block, i.e. physical chunk
// l%16 of key 4i + l/16, so it fetches the logical chunk that the swizzle
// maps there.  Keys past the tile's valid count are not read; their slots
// are zero-filled so a masked key never contributes a NaN to P*V.
__device__ __forceinline__ void load_tile_async(const FwdArgs& a, char* buf, int b, int h, int key0,
                                                int nvalid, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kt = 16 * wave + 4 * i;           // first key of this 1 KiB block
    const int key = kt + (lane >> 4);
    const int chunk = (lane & 15) ^ swz(key);   // logical chunk stored in slot lane
    lds_char* kdst = (lds_char*)(buf + kt * kRowB);
    lds_char* vdst = (lds_char*)(buf + kTileB + kt * kRowB);
    if (key < nvalid) {
      __builtin_amdgcn_global_load_lds((const void*)(a.k.row(b, key0 + key, h) + 8 * chunk), (void __attribute__((address_space(3)))*)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(a.v.row(b, key0 + key, h) + 8 * chunk), (void __attribute__((address_space(3)))*)vdst, 16, 0, 0);
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(buf + kt * kRowB + 16 * lane) = z;
      *(u32x4*)(buf + kTileB + kt * kRowB + 16 * lane) = z;
    }
  }
}

// V^T fragment for the A operand of O^T += V^T P^T: two transposing LDS reads
// (ds_read_b64_tr_b16).  Within each 16-lane group the read hands lane j
// element (j & 3) of the 8-byte row piece addressed by lane 4t + (j >> 2) as
// its slot t; the addresses below make lane l receive channel 32*dblk + l%32
// of the 8 keys that the permuted reduction index assigns to its half-wave.
__device__ __forceinline__ bf16x8 load_vt(const char* vbuf, int dblk, int c2, int lane) {
  const int hh = lane >> 5, g = (lane >> 4) & 1, i = lane & 15, q = i & 3;
  const int row0 = 16 * c2 + 4 * hh + (i >> 2);
  const int chunk = 4 * dblk + 2 * g + (q >> 1);
  const char* p0 = vbuf + lds_off(row0, chunk) + 8 * (q & 1);
  const char* p1 = vbuf + lds_off(row0 + 8, chunk) + 8 * (q & 1);
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_char*)p0);
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_char*)p1);
  const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufBytes];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hh = lane >> 5;

  // workgroup -> (b, h, query tile); optionally keep a head's tiles on one XCD
  int bh, qt;
  const int g = blockIdx.x;
  if (a.xcd_remap) {
    const int xcd = g & 7, j = g >> 3;
    const int hl = j / a.n_qtiles;
    qt = j - hl * a.n_qtiles;
    bh = xcd + 8 * hl;
  } else {
    bh = g / a.n_qtiles;
    qt = g - bh * a.n_qtiles;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int L = a.txt_len[b];
  const int qrow = qt * (kFwdWaves * kFwdRowsPerWave) + wave * kFwdRowsPerWave + lr;
  const bool qvalid = qrow < a.S;

  bf16x8 qreg[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
    qreg[kk] = __builtin_bit_cast(bf16x8, z);
  }

  const int ntxt = (L + kFwdBN - 1) / kFwdBN;
  const int nt = ntxt + (a.T_img + kFwdBN - 1) / kFwdBN;

  f32x16 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_used = -INFINITY, l_lane = 0.f;

  int key0, nvalid;
  tile_bounds(0, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
  load_tile_async(a, smem, b, h, key0, nvalid, wave, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const char* buf = smem + (t & 1) * kBufBytes;
    const int cur_valid = nvalid;
    if (t + 1 < nt) {
      tile_bounds(t + 1, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
      load_tile_async(a, smem + ((t + 1) & 1) * kBufBytes, b, h, key0, nvalid, wave, lane);
    }

    // ---- S^T = K Q^T for two 32-key blocks
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kv = *(const bf16x8*)(buf + lds_off(32 * kb + lr, 2 * kk + hh));
        s[kb] = mfma32(kv, qreg[kk], s[kb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // key of register r in block kb: 32*kb + 8*(r/4) + 4*hh + r%4
    if (cur_valid < kFwdBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= cur_valid) s[kb][r] = -INFINITY;
        }
    }
    // ---- row max (exact, any order), lane-local reference-max update
    float mt = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool move = mt > m_used + kTauRaw;
    const float m_new = move ? mt : m_used;
    if (__any(move)) {
      const float alpha = (m_new == m_used) ? 1.0f : __builtin_amdgcn_exp2f((m_used - m_new) * kC);
      l_lane = l_lane * alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] = acc[d][r] * alpha;
      m_used = m_new;
    }
    const float mc = m_used * kC;

    // ---- p = exp2(s*c - m*c) in place; l sums p in FP32 in register order
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], kC, -mc));
        ts = ts + s[kb][r];
      }
    l_lane = l_lane + ts;

    // ---- O^T += V^T P_hi^T, then V^T P_lo^T, one 16-key chunk at a time;
    //      p is split into hi = bf16(p), lo = bf16(p - hi)
    const char* vt = buf + kTileB;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const int kb = c2 >> 1, r0 = 8 * (c2 & 1);
      u32x4 hw, lw;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = s[kb][r0 + 2 * w], p1 = s[kb][r0 + 2 * w + 1];
        const uint32_t u = pack_bf16x2(p0, p1);
        hw[w] = u;
        lw[w] = pack_bf16x2(p0 - bf16_lo(u), p1 - bf16_hi(u));
      }
      const bf16x8 pbh = __builtin_bit_cast(bf16x8, hw), pbl = __builtin_bit_cast(bf16x8, lw);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 vv = load_vt(vt, d, c2, lane);
        acc[d] = mfma32(vv, pbh, acc[d]);
        acc[d] = mfma32(vv, pbl, acc[d]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's direct loads of the next tile have landed
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, one RNE cast; LSE in natural log
  const float l_tot = l_lane + __shfl_xor(l_lane, 32);
  if (qvalid) {
    uint16_t* orow = a.o.row(b, qrow, h);
    float* frow = a.of ? a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim : nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        const float o0 = acc[d][4 * g4] / l_tot, o1 = acc[d][4 * g4 + 1] / l_tot;
        const float o2 = acc[d][4 * g4 + 2] / l_tot, o3 = acc[d][4 * g4 + 3] / l_tot;
        const u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)(orow + d0) = ov;
        if (frow) *(f32x4*)(frow + d0) = f32x4{o0, o1, o2, o3};
      }
    if (hh == 0) {
      const float lse2 = m_used * kC + log2f(l_tot);
      a.lse[((int64_t)b * a.H + h) * a.S + qrow] = lse2 * kLn2;
    }
  }
}

}  // namespace qi
