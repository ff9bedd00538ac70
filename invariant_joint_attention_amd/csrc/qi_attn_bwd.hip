// qi_attn_bwd.hip -- deterministic attention backward on gfx950.
//
// Pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
// ablation matrix and integration plan", "Work items" (every differentiable
// operator has a backward) and "Numerical requirements" (fixed reduction
// trees, FP32 accumulators, no atomics); [Kernel list] "[RFC] [Qwen-Image]
// WS1 Single-GPU Kernel List", rows joint_attn_* (forward and backward).
//
// Two passes, each output element written by exactly one lane, no atomics:
//  * dQ pass (query-tile-major, grid as the forward): per wave 32 queries.
//    D_i = dO_i . O_i is formed first (fixed order) from the forward's FP32
//    (pre-cast) O -- the BF16 O would move D by ~2^-9 |dO||O| sqrt(128), which
//    the gain gradients, sums of many cancelling rows, do not tolerate -- and
//    stored for the dK/dV pass.  Then over the key tiles in the forward's logical order:
//    S^T = K Q^T, dP^T = V dO^T, P = exp2(s*c - LSE*log2 e),
//    dS = P (dP - D), dQ^T += K^T dS^T with dS split into two BF16 terms
//    (hi = bf16(dS), lo = bf16(dS - hi)) accumulated hi then lo.
//  * dK/dV pass (key-tile-major): per wave 32 keys held in registers.  Query
//    tiles of 64 rows are visited in a frozen logical order -- valid text rows
//    from 0, image rows from T_txt, then padded text rows from L_b -- so the
//    sum over queries of a key never depends on the batch or the launch.
//    S = Q K^T, dP = dO V^T, then dV^T += dO^T (P_hi + P_lo) and
//    dK^T += Q^T (dS_hi + dS_lo), each operand split into two BF16 terms
//    and accumulated hi then lo.  Keys of the masked text range get exact
//    zeros.
// All MFMAs are v_mfma_f32_32x32x16_bf16; transposed operands are written to
// LDS with the reduction index permuted (bits 2 and 3 of the index in each
// 16-chunk swapped) to match the accumulator layout of the probabilities.
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_lds.h"

namespace qi {

namespace {

constexpr int kRow = 272;    // bytes per row-major 128-channel row in LDS
constexpr int kTRow = 144;   // bytes per transposed row (64 entries + pad)
constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);  // log2(e)/sqrt(128)
constexpr float kLog2e = 1.4426950408889634074f;
constexpr float kScale = (float)(1.0 / 11.313708498984760390);  // 1/sqrt(128)

__device__ __forceinline__ int swap23(int a4) {  // position of key 4*a4 (a4 = 0..15)
  return 16 * (a4 >> 2) + 8 * (a4 & 1) + 4 * ((a4 >> 1) & 1);
}

// 4 consecutive rows x 8 channels of a [rows,128] tile -> row-major LDS and
// transposed (permuted) LDS.
__device__ __forceinline__ void store_rows_and_t(char* rm, char* tr, const u32x4* x, int a4, int c16) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *(u32x4*)(rm + (4 * a4 + r) * kRow + c16 * 16) = x[r];
  if (tr) {
    const int pos = swap23(a4);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = x[0][w], x1 = x[1][w], x2 = x[2][w], x3 = x[3][w];
      u32x2 lo = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
      u32x2 hi = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
      *(u32x2*)(tr + (8 * c16 + 2 * w) * kTRow + pos * 2) = lo;
      *(u32x2*)(tr + (8 * c16 + 2 * w + 1) * kTRow + pos * 2) = hi;
    }
  }
}

__device__ __forceinline__ void split_pack(const float* v, uint32_t* hi, uint32_t* lo) {
  // v[0..7] -> hi[0..3], lo[0..3] packed BF16 pairs
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t h = pack_bf16x2(v[2 * w], v[2 * w + 1]);
    hi[w] = h;
    const float r0 = v[2 * w] - bf16_lo(h);
    const float r1 = v[2 * w + 1] - bf16_hi(h);
    lo[w] = pack_bf16x2(r0, r1);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t* w) {
  const u32x4 v = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void decode_bh(const BwdArgs& a, int ntiles, int& b, int& h, int& tile) {
  const int g = blockIdx.x;
  int bh;
  if (a.xcd_remap) {
    const int xcd = g & 7, j = g >> 3;
    const int hl = j / ntiles;
    tile = j - hl * ntiles;
    bh = xcd + 8 * hl;
  } else {
    bh = g / ntiles;
    tile = g - bh * ntiles;
  }
  b = bh / a.H;
  h = bh - b * a.H;
}

// ----------------------------------------------------------------- dQ pass
// Workgroup = 8 waves x 32 query rows of one (b, h); waves w and w+4 share a
// SIMD.  Group 0 (waves 0-3) and group 1 (waves 4-7) alternate, one barrier
// per phase, between a matrix phase (dQ^T += K_t^T dS_t^T with dS split
// hi/lo, then the scores and dP of tile t+1: 64 MFMAs) and a VALU phase
// (P, dS and its split for tile t+1).  K and V tiles are triple-buffered in
// LDS (96 KiB) and filled by direct loads: in its VALU phase of tile t group
// 0 loads V_{t+2} and group 1 K_{t+2}; each waits for its loads at the end
// of its next matrix phase.  The arithmetic is the frozen one of the pass
// (per accumulator: scores and dP over the 8 head-dim chunks in order, dQ
// over the 16-key chunks in key order, hi then lo).
using namespace lds;
static_assert(kTileRows == kBwdBN, "dQ key tile is one LDS tile");

struct DqState {
  f32x16 acc[4];       // dQ^T: 4 head-dim blocks x 32 queries
  f32x16 s[2], dp[2];  // S^T and dP^T of one tile (two 32-key blocks)
  u32x4 dh[4], dl[4];  // hi / lo BF16 dS^T of the four 16-key chunks
  bf16x8 q[8], o[8];   // Q and dO rows of the wave's 32 queries
  float lse2, D;
};

__device__ __forceinline__ void dq_bounds(int t, int ntxt, int L, int T_txt, int T_img, int& key0, int& nvalid) {
  if (t < ntxt) {
    key0 = t * kBwdBN;
    nvalid = min(kBwdBN, L - key0);
  } else {
    const int ti = t - ntxt;
    key0 = T_txt + ti * kBwdBN;
    nvalid = min(kBwdBN, T_img - ti * kBwdBN);
  }
}

// P = exp2(s*c - LSE*log2 e) (0 for masked keys), dS = P (dP - D), split
// into hi = bf16(dS), lo = bf16(dS - hi) per 16-key chunk.
__device__ __forceinline__ void dq_softmax(DqState& st, int cur_valid, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // key of register r in block kb: 32*kb + 8*(r/4) + 4*hh + r%4
      const int key = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float p = key < cur_valid ? __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[kb][r], kC, -st.lse2)) : 0.f;
      ds[r] = p * (st.dp[kb][r] - st.D);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t hi[4], lo[4];
      split_pack(ds + 8 * half, hi, lo);
      st.dh[2 * kb + half] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      st.dl[2 * kb + half] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
}

// Matrix phase, 4 LDS reads and 4 MFMAs per step, fragments read one step
// ahead.  dQ steps j = 0..7: chunk c2 = j/2, head-dim blocks 2(j%2) and
// 2(j%2)+1 from the transposed K_t tile.  Score steps j = 0..7: head-dim
// chunk kk = j of both 32-key blocks of S^T (K_{t+1}) and dP^T (V_{t+1}).
struct DqBases {
  uint32_t tk, rk, rv;  // K_t transposed, K_{t+1} rows, V_{t+1} rows
};
using Ring = bf16x8[2][4];

template <bool kDq, int k>
__device__ __forceinline__ void dq_issue(Ring& f, const DqBases& b) {
  constexpr int nsteps = (kDq ? 8 : 0) + 8;
  if constexpr (k < nsteps) {
    bf16x8* x = f[k & 1];
    if constexpr (kDq && k < 8) {
      constexpr int c2 = k >> 1, d0 = 2 * (k & 1), d1 = d0 + 1;
      x[0] = tr_frag<c2, d0>(b.tk);
      x[1] = tr_frag<c2, d1>(b.tk);
    } else {
      constexpr int kk = kDq ? k - 8 : k;
      x[0] = row_frag<kk, 0>(b.rk);
      x[1] = row_frag<kk, 0>(b.rv);
      x[2] = row_frag<kk, 1>(b.rk);
      x[3] = row_frag<kk, 1>(b.rv);
    }
  }
}

template <bool kDq, bool kS, int k>
__device__ __forceinline__ void dq_step(DqState& st, Ring& f, const DqBases& b) {
  constexpr int nsteps = (kDq ? 8 : 0) + (kS ? 8 : 0);
  if constexpr (k < nsteps) {
    if constexpr (!(kDq && !kS && k + 1 >= 8)) dq_issue<kDq, k + 1>(f, b);
    // LDS reads issued after this step's: the next step's 4
    constexpr int later = (k + 1 < nsteps) ? 4 : 0;
    bf16x8* x = f[k & 1];
    if constexpr (kDq && k < 8) {
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x[0]), "+v"(x[1]) : "i"(later));
      constexpr int c2 = k >> 1, d0 = 2 * (k & 1), d1 = d0 + 1;
      st.acc[d0] = mfma32(x[0], __builtin_bit_cast(bf16x8, st.dh[c2]), st.acc[d0]);
      st.acc[d1] = mfma32(x[1], __builtin_bit_cast(bf16x8, st.dh[c2]), st.acc[d1]);
      st.acc[d0] = mfma32(x[0], __builtin_bit_cast(bf16x8, st.dl[c2]), st.acc[d0]);
      st.acc[d1] = mfma32(x[1], __builtin_bit_cast(bf16x8, st.dl[c2]), st.acc[d1]);
    } else {
      asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : "i"(later));
      constexpr int kk = kDq ? k - 8 : k;
      st.s[0] = mfma32(x[0], st.q[kk], st.s[0]);
      st.dp[0] = mfma32(x[1], st.o[kk], st.dp[0]);
      st.s[1] = mfma32(x[2], st.q[kk], st.s[1]);
      st.dp[1] = mfma32(x[3], st.o[kk], st.dp[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    dq_step<kDq, kS, k + 1>(st, f, b);
  }
}

template <bool kDq, bool kS>
__device__ __forceinline__ void dq_matrix(DqState& st, DqBases b) {
  if (kS) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st.s[kb][r] = 0.f;
        st.dp[kb][r] = 0.f;
      }
  }
  Ring f;
  // opaque copies keep the per-step address XORs inside their steps
  asm volatile("" : "+v"(b.tk), "+v"(b.rk), "+v"(b.rv));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kDq)
    dq_issue<true, 0>(f, b);
  else
    dq_issue<false, 0>(f, b);
  __builtin_amdgcn_sched_barrier(0);
  dq_step<kDq, kS, 0>(st, f, b);
}

}  // namespace

__global__ __launch_bounds__(kBwdDqWaves * 64, 1) void attn_bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[6 * kTileB];  // K tiles [3], V tiles [3]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, sub = wave & 3;
  const int lr = lane & 31, hh = lane >> 5;
  int b, h, qt;
  decode_bh(a, a.n_qtiles, b, h, qt);
  const int L = a.txt_len[b];
  const int qrow = qt * (kBwdDqWaves * 32) + wave * 32 + lr;
  const bool qvalid = qrow < a.S;

  DqState st;
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    if (qvalid) {
      zq = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
      zd = *(const u32x4*)(a.dO.row(b, qrow, h) + 16 * kk + 8 * hh);
      const float* orow = a.o.row(b, qrow, h) + 16 * kk + 8 * hh;
      o0 = *(const f32x4*)orow;
      o1 = *(const f32x4*)(orow + 4);
    }
    st.q[kk] = __builtin_bit_cast(bf16x8, zq);
    st.o[kk] = __builtin_bit_cast(bf16x8, zd);
    // D_i = dO_i . O_i (FP32 pre-cast O), fixed order: chunk, then channel
    const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = bf16_lo(zd[w]) * ov[2 * w];
      dpart = dpart + p0;
      const float p1 = bf16_hi(zd[w]) * ov[2 * w + 1];
      dpart = dpart + p1;
    }
  }
  st.D = dpart + __shfl_xor(dpart, 32);
  st.lse2 = INFINITY;
  if (qvalid) {
    const int64_t li = ((int64_t)b * a.H + h) * a.S + qrow;
    st.lse2 = a.lse[li] * kLog2e;
    if (hh == 0) a.Dvec[li] = st.D;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[d][r] = 0.f;

  const int ntxt = (L + kBwdBN - 1) / kBwdBN;
  const int nt = ntxt + (a.T_img + kBwdBN - 1) / kBwdBN;
  char* const kbase = smem;
  char* const vbase = smem + 3 * kTileB;
  auto kbuf = [&](int j) { return kbase + (j % 3) * kTileB; };
  auto vbuf = [&](int j) { return vbase + (j % 3) * kTileB; };
  auto valid_of = [&](int j) {
    int k0, nv;
    dq_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    return nv;
  };
  const RowOff ko = row_offsets(a.k.ss, lane), vo = row_offsets(a.v.ss, lane);
  auto load_k = [&](int j) {
    int k0, nv;
    dq_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.k, ko, kbuf(j), b, h, k0, nv, sub, lane);
  };
  auto load_v = [&](int j) {
    int k0, nv;
    dq_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.v, vo, vbuf(j), b, h, k0, nv, sub, lane);
  };
  auto bases = [&](int t) {
    DqBases bb;
    bb.tk = tr_base(addr_of(kbuf(t)), lane);
    bb.rk = row_base(addr_of(kbuf(t + 1)), lane);
    bb.rv = row_base(addr_of(vbuf(t + 1)), lane);
    return bb;
  };

  // prologue: tiles 0 (group 0) and 1 (group 1)
  if (grp == 0) {
    load_k(0);
    load_v(0);
  } else if (nt > 1) {
    load_k(1);
    load_v(1);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  bar();

  // Both groups run the same sequence; group 1 starts one barrier later, so
  // the two groups alternate phases.  Each group runs 2*nt + 1 barriers.
  if (grp == 1) bar();
  {
    DqBases b0;
    b0.tk = 0;
    b0.rk = row_base(addr_of(kbuf(0)), lane);
    b0.rv = row_base(addr_of(vbuf(0)), lane);
    __builtin_amdgcn_s_setprio(1);
    dq_matrix<false, true>(st, b0);
    __builtin_amdgcn_s_setprio(0);
  }
  bar();
  for (int t = 0; t + 1 < nt; ++t) {
    if (t + 2 < nt) {
      if (grp == 0)
        load_v(t + 2);
      else
        load_k(t + 2);
    }
    dq_softmax(st, valid_of(t), hh);
    bar();
    __builtin_amdgcn_s_setprio(1);
    dq_matrix<true, true>(st, bases(t));
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0070);  // this group's loads have landed
    bar();
  }
  dq_softmax(st, valid_of(nt - 1), hh);
  bar();
  {
    DqBases bl;
    bl.tk = tr_base(addr_of(kbuf(nt - 1)), lane);
    bl.rk = 0;
    bl.rv = 0;
    __builtin_amdgcn_s_setprio(1);
    dq_matrix<true, false>(st, bl);
    __builtin_amdgcn_s_setprio(0);
  }
  if (grp == 0) bar();

  if (qvalid) {
    float* drow = a.dq.row(b, qrow, h);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        *(f32x4*)(drow + d0) = f32x4{st.acc[d][4 * g4] * kScale, st.acc[d][4 * g4 + 1] * kScale,
                                     st.acc[d][4 * g4 + 2] * kScale, st.acc[d][4 * g4 + 3] * kScale};
      }
  }
}

// --------------------------------------------------------------- dK/dV pass
namespace {
constexpr int kKQ = kBwdBM * kRow;       // Q row-major
constexpr int kKDO = kBwdBM * kRow;      // dO row-major
constexpr int kKQT = kHeadDim * kTRow;   // Q^T
constexpr int kKDOT = kHeadDim * kTRow;  // dO^T
constexpr int kKBuf = kKQ + kKDO + kKQT + kKDOT + 2 * kBwdBM * 4;  // + lse2, D
constexpr int kKeysPerWG = 128;
}  // namespace

__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kKBuf];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  int b, h, kt;
  decode_bh(a, a.n_ktiles, b, h, kt);
  const int L = a.txt_len[b];
  const int nkt_txt = (L + kKeysPerWG - 1) / kKeysPerWG;
  const int nkt_img = (a.T_img + kKeysPerWG - 1) / kKeysPerWG;
  const int nkt_pad = (a.T_txt - L + kKeysPerWG - 1) / kKeysPerWG;
  if (kt >= nkt_txt + nkt_img + nkt_pad) return;  // whole workgroup

  int kbase, kend;
  bool zero_only = false;
  if (kt < nkt_txt) { kbase = kt * kKeysPerWG; kend = L; }
  else if (kt < nkt_txt + nkt_img) { kbase = a.T_txt + (kt - nkt_txt) * kKeysPerWG; kend = a.S; }
  else { kbase = L + (kt - nkt_txt - nkt_img) * kKeysPerWG; kend = a.T_txt; zero_only = true; }
  const int key = kbase + 32 * wave + lr;
  const bool kvalid = key < kend;

  if (zero_only) {
    if (kvalid) {
      float* dkr = a.dk.row(b, key, h);
      float* dvr = a.dv.row(b, key, h);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        *(f32x4*)(dkr + 64 * hh + 4 * i) = z;
        *(f32x4*)(dvr + 64 * hh + 4 * i) = z;
      }
    }
    return;  // whole workgroup takes this branch
  }

  bf16x8 kreg[8], vreg[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (kvalid) {
      zk = *(const u32x4*)(a.k.row(b, key, h) + 16 * kk + 8 * hh);
      zv = *(const u32x4*)(a.v.row(b, key, h) + 16 * kk + 8 * hh);
    }
    kreg[kk] = __builtin_bit_cast(bf16x8, zk);
    vreg[kk] = __builtin_bit_cast(bf16x8, zv);
  }

  // frozen query order: valid text, image, padded text; tiles of 64 rows
  const int nq_txt = (L + kBwdBM - 1) / kBwdBM;
  const int nq_img = (a.T_img + kBwdBM - 1) / kBwdBM;
  const int nq_pad = (a.T_txt - L + kBwdBM - 1) / kBwdBM;
  const int nqt = nq_txt + nq_img + nq_pad;
  auto bounds = [&](int t, int& q0, int& nq) {
    if (t < nq_txt) { q0 = t * kBwdBM; nq = min(kBwdBM, L - q0); }
    else if (t < nq_txt + nq_img) { const int ti = t - nq_txt; q0 = a.T_txt + ti * kBwdBM; nq = min(kBwdBM, a.T_img - ti * kBwdBM); }
    else { const int ti = t - nq_txt - nq_img; q0 = L + ti * kBwdBM; nq = min(kBwdBM, a.T_txt - L - ti * kBwdBM); }
  };

  f32x16 adk[4], adv[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) { adk[d][r] = 0.f; adv[d][r] = 0.f; }

  const int tid = threadIdx.x, a4 = tid >> 4, c16 = tid & 15;
  u32x4 qr[4], dr[4];
  float l2v = INFINITY, dvv = 0.f;
  const int64_t lbase = ((int64_t)b * a.H + h) * a.S;
  auto load = [&](int q0, int nq) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = 4 * a4 + r;
      u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
      if (qi < nq) {
        zq = *(const u32x4*)(a.q.row(b, q0 + qi, h) + 8 * c16);
        zd = *(const u32x4*)(a.dO.row(b, q0 + qi, h) + 8 * c16);
      }
      qr[r] = zq;
      dr[r] = zd;
    }
    l2v = INFINITY;
    dvv = 0.f;
    if (tid < kBwdBM && tid < nq) {
      l2v = a.lse[lbase + q0 + tid] * kLog2e;
      dvv = a.Dvec[lbase + q0 + tid];
    }
  };
  auto store = [&](char* buf) {
    store_rows_and_t(buf, buf + kKQ + kKDO, qr, a4, c16);
    store_rows_and_t(buf + kKQ, buf + kKQ + kKDO + kKQT, dr, a4, c16);
    if (tid < kBwdBM) {
      float* f = (float*)(buf + kKQ + kKDO + kKQT + kKDOT);
      f[tid] = l2v;
      f[kBwdBM + tid] = dvv;
    }
  };

  int q0, nq;
  bounds(0, q0, nq);
  load(q0, nq);
  store(smem);
  __syncthreads();
  for (int t = 0; t < nqt; ++t) {
    const char* buf = smem + (t & 1) * kKBuf;
    if (t + 1 < nqt) {
      bounds(t + 1, q0, nq);
      load(q0, nq);
    }
    const float* l2s = (const float*)(buf + kKQ + kKDO + kKQT + kKDOT);
    const float* Ds = l2s + kBwdBM;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[qb][r] = 0.f; dp[qb][r] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int off = (32 * qb + lr) * kRow + (16 * kk + 8 * hh) * 2;
        s[qb] = mfma32(*(const bf16x8*)(buf + off), kreg[kk], s[qb]);
        dp[qb] = mfma32(*(const bf16x8*)(buf + kKQ + off), vreg[kk], dp[qb]);
      }
    // lane <-> key; register r of block qb <-> query 32qb + 8(r/4) + 4hh + r%4
    uint32_t phi[2][8], plo[2][8], hi[2][8], lo[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], kC, -l2s[qi]));
        ds[r] = p[r] * (dp[qb][r] - Ds[qi]);
      }
      split_pack(p, phi[qb], plo[qb]);
      split_pack(p + 8, phi[qb] + 4, plo[qb] + 4);
      split_pack(ds, hi[qb], lo[qb]);
      split_pack(ds + 8, hi[qb] + 4, lo[qb] + 4);
    }
    const char* qt_ = buf + kKQ + kKDO;
    const char* dot_ = qt_ + kKQT;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qb = c >> 1, half = c & 1;
      const bf16x8 ph_ = as_bf16x8(phi[qb] + 4 * half), pl_ = as_bf16x8(plo[qb] + 4 * half);
      const bf16x8 bh_ = as_bf16x8(hi[qb] + 4 * half), bl_ = as_bf16x8(lo[qb] + 4 * half);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int off = (32 * d + lr) * kTRow + (16 * c + 8 * hh) * 2;
        const bf16x8 da = *(const bf16x8*)(dot_ + off);
        adv[d] = mfma32(da, ph_, adv[d]);
        adv[d] = mfma32(da, pl_, adv[d]);
        const bf16x8 qa = *(const bf16x8*)(qt_ + off);
        adk[d] = mfma32(qa, bh_, adk[d]);
        adk[d] = mfma32(qa, bl_, adk[d]);
      }
    }
    if (t + 1 < nqt) store(smem + ((t + 1) & 1) * kKBuf);
    __syncthreads();
  }
  if (kvalid) {
    float* dkr = a.dk.row(b, key, h);
    float* dvr = a.dv.row(b, key, h);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        *(f32x4*)(dvr + d0) = f32x4{adv[d][4 * g4], adv[d][4 * g4 + 1], adv[d][4 * g4 + 2], adv[d][4 * g4 + 3]};
        *(f32x4*)(dkr + d0) = f32x4{adk[d][4 * g4] * kScale, adk[d][4 * g4 + 1] * kScale,
                                    adk[d][4 * g4 + 2] * kScale, adk[d][4 * g4 + 3] * kScale};
      }
  }
}

}  // namespace qi
