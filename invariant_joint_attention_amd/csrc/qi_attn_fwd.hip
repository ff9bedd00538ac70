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
//    The MFMA reduction index is a permutation of the 16 keys
//    of a chunk (bits 2 and 3 of the key index swapped); V^T is written to
//    LDS in that permuted order so one 16-byte LDS read feeds each operand.
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
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are
//    in flight while the current tile is multiplied.
#include "qi_common.h"
#include "qi_kernels.h"

namespace qi {

namespace {

constexpr int kKRow = 272;                 // bytes per K row in LDS (256 + 16 pad)
constexpr int kVtRow = 144;                // bytes per V^T row (64 keys * 2 + 16 pad)
constexpr int kKBytes = kFwdBN * kKRow;    // 17408
constexpr int kVtBytes = kHeadDim * kVtRow;  // 18432
constexpr int kBufBytes = kKBytes + kVtBytes;
// log2(e) / sqrt(128), rounded once to FP32
constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);
constexpr float kLn2 = 0.69314718055994530942f;
// Threshold on raw scores for moving the reference max: 8 in the exp2 domain.
constexpr float kTauRaw = (float)(8.0 / (1.4426950408889634074 / 11.313708498984760390));

struct TileRegs {
  u32x4 kr[4];
  u32x4 vr[4];
};

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

__device__ __forceinline__ void load_tile(const FwdArgs& a, int b, int h, int key0, int nvalid,
                                          TileRegs& t) {
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = (tid >> 4) + 16 * i;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (key < nvalid) z = *(const u32x4*)(a.k.row(b, key0 + key, h) + 8 * c16);
    t.kr[i] = z;
  }
  const int a4 = tid >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = 4 * a4 + r;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (key < nvalid) z = *(const u32x4*)(a.v.row(b, key0 + key, h) + 8 * c16);
    t.vr[r] = z;
  }
}

__device__ __forceinline__ void store_tile(char* buf, const TileRegs& t) {
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = (tid >> 4) + 16 * i;
    *(u32x4*)(buf + key * kKRow + c16 * 16) = t.kr[i];
  }
  // V^T: this thread holds keys 4*a4..4*a4+3, channels 8*c16..8*c16+7.
  const int a4 = tid >> 4;
  const int pos = 16 * (a4 >> 2) + 8 * (a4 & 1) + 4 * ((a4 >> 1) & 1);  // bits 2,3 swapped
  char* vt = buf + kKBytes;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x0 = t.vr[0][w], x1 = t.vr[1][w], x2 = t.vr[2][w], x3 = t.vr[3][w];
    u32x2 lo = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
    u32x2 hi = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
    *(u32x2*)(vt + (8 * c16 + 2 * w) * kVtRow + pos * 2) = lo;
    *(u32x2*)(vt + (8 * c16 + 2 * w + 1) * kVtRow + pos * 2) = hi;
  }
}

}  // namespace

__global__ __launch_bounds__(256) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];

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

  TileRegs tr;
  int key0, nvalid;
  tile_bounds(0, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
  load_tile(a, b, h, key0, nvalid, tr);
  store_tile(smem, tr);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const char* buf = smem + (t & 1) * kBufBytes;
    const int cur_valid = nvalid;
    if (t + 1 < nt) {
      tile_bounds(t + 1, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
      load_tile(a, b, h, key0, nvalid, tr);
    }

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kv = *(const bf16x8*)(buf + (32 * kb + lr) * kKRow + (16 * kk + 8 * hh) * 2);
        s[kb] = mfma32(kv, qreg[kk], s[kb]);
      }
    }
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

    // ---- p = exp2(s*c - m*c); l sums p in FP32 in register order; p is
    //      split into two BF16 terms hi = bf16(p), lo = bf16(p - hi)
    uint32_t ph[2][8], pl[2][8];
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * w], kC, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * w + 1], kC, -mc));
        ts = ts + p0;
        ts = ts + p1;
        const uint32_t u = pack_bf16x2(p0, p1);
        ph[kb][w] = u;
        pl[kb][w] = pack_bf16x2(p0 - bf16_lo(u), p1 - bf16_hi(u));
      }
    l_lane = l_lane + ts;

    // ---- O^T += V^T P_hi^T, then V^T P_lo^T
    const char* vt = buf + kKBytes;
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const int kb = c2 >> 1, half = c2 & 1;
      const u32x4 hw = {ph[kb][4 * half], ph[kb][4 * half + 1], ph[kb][4 * half + 2], ph[kb][4 * half + 3]};
      const u32x4 lw = {pl[kb][4 * half], pl[kb][4 * half + 1], pl[kb][4 * half + 2], pl[kb][4 * half + 3]};
      const bf16x8 pbh = __builtin_bit_cast(bf16x8, hw), pbl = __builtin_bit_cast(bf16x8, lw);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 vv = *(const bf16x8*)(vt + (32 * d + lr) * kVtRow + (16 * c2 + 8 * hh) * 2);
        acc[d] = mfma32(vv, pbh, acc[d]);
        acc[d] = mfma32(vv, pbl, acc[d]);
      }
    }

    if (t + 1 < nt) store_tile(smem + ((t + 1) & 1) * kBufBytes, tr);
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
