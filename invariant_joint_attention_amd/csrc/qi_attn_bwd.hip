// qi_attn_bwd.hip -- deterministic attention backward on gfx950.
//
// Pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
// ablation matrix and integration plan", "Work items" (every differentiable
// operator has a backward) and "Numerical requirements" (fixed reduction
// trees, FP32 accumulators, no atomics); [Kernel list] "[RFC] [Qwen-Image]
// WS1 Single-GPU Kernel List", rows joint_attn_* (forward and backward).
//
// A preparation kernel forms D_i = dO_i . O_i (fixed order) from the
// forward's FP32 (pre-cast) O -- the BF16 O would move D by
// ~2^-9 |dO||O| sqrt(128), which the gain gradients, sums of many cancelling
// rows, do not tolerate -- and records max |dO| per 32 rows.  Then three
// passes, each output element written by exactly one lane, no atomics, all
// in one grid (dK workgroups, then dQ, then dV):
//  * dQ pass (query-tile-major): per wave 32 queries, over the key tiles in
//    the forward's logical order: S^T = K Q^T, dP^T = V dO^T,
//    P = exp2(s*c - LSE*log2 e), dS = P (dP - D), dQ^T += K^T dS^T with dS
//    split into two BF16 terms (hi = bf16(dS), lo = bf16(dS - hi))
//    accumulated hi then lo.
//  * dK and dV passes (key-tile-major): per wave 32 keys held in registers.
//    Query tiles of 64 rows are visited in a frozen logical order -- valid
//    text rows from 0, image rows from T_txt, then padded text rows from
//    L_b -- so the sum over queries of a key never depends on the batch or
//    the launch.  Padded text query rows take part like every other row:
//    their dO should be zero (their outputs carry no gradient), and their
//    q, k, O and LSE must be finite.  S = Q K^T and, for dK, dP = dO V^T;
//    then dK^T += Q^T (dS_hi + dS_lo), accumulated hi then lo
//    (v_mfma_f32_32x32x16_bf16), and dV^T += dO16^T P16 with P rounded once
//    to FP16 and dO as FP16 of dO * 2^e, one power of two per (sample,
//    head) taken from the slice's largest |dO| (the preparation kernel
//    records the maxima, do_convert_kernel folds them and converts dO), one
//    v_mfma_f32_32x32x16_f16 per step; dV = acc * 2^-e.  Keys of the masked
//    text range get exact zeros.
// Scores, dP, dQ and dK use v_mfma_f32_32x32x16_bf16; dV the f16 form.  Per
// accumulator the order is: scores and dP over the 8 head-dim chunks in
// order; gradients over the 16-row chunks of the streamed side in its
// frozen order (hi then lo for dQ and dK).
//
// Schedule (bit-neutral): every pass runs 8-wave workgroups, waves w and
// w+4 on one SIMD, group 0 (waves 0-3) and group 1 (waves 4-7).  A wave
// alternates a VALU block (P, dS and the hi/lo split of tile t) and a
// matrix block (the gradient MFMAs of tile t, then the scores -- and dP --
// of tile t+1), with one workgroup barrier per tile that group 1 passes
// before its VALU block and group 0 between its VALU and matrix blocks.
// Streamed tiles sit in LDS rings of four, filled by direct global->LDS
// loads three tiles ahead; transposed operands come from ds_read_b64_tr_b16
// on row-major tiles (see qi_lds.h), except the dV pass's FP16 dO, which
// do_convert writes already transposed (one ds_read_b128 per fragment).
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_lds.h"
#include "qi_attn_contract.h"

namespace qi {

namespace {

using namespace lds;
static_assert(kTileRows == kBwdBN && kTileRows == kBwdBM, "backward tiles are LDS tiles");
static_assert(kVtileElems == kHeadDim * kBwdBM && kVtileElems * 2 == kTileB, "a transposed FP16 dO tile fills one LDS tile");

constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);  // log2(e)/sqrt(128)
constexpr float kLog2e = 1.4426950408889634074f;
constexpr float kScale = (float)(1.0 / 11.313708498984760390);  // 1/sqrt(128)

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

__device__ __forceinline__ void decode_bh(const BwdArgs& a, int ntiles, int g, int& b, int& h, int& tile) {
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

// One direct global -> LDS load of one dword per lane: lane l's 4 bytes land
// at LDS byte lds + 4*l (same M0 contract as dma16).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const char* base, uint32_t off32, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(off32), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Streamed tiles sit in rings of four and are loaded three tiles ahead.
constexpr int kRing = 4;

// Tile fill that always issues four loads per wave (so a wave's vmcnt
// arithmetic is exact): wave `sub` of a group fills rows 16*sub..16*sub+15,
// four rows per load; rows past `nvalid` repeat the last valid row.  Every
// consumer masks those rows (their P and dS are exact zeros), so their
// contents never reach an output, and a masked row of the tensor is never
// read.
__device__ __forceinline__ void load_rows_rep(const View<const uint16_t>& src, const RowOff& ro, char* dst, int b,
                                              int h, int row0, int nvalid, int sub, int lane) {
  const int r0 = 16 * sub;
  const uint32_t la = addr_of(dst + r0 * kRowB);
  if (nvalid >= r0 + 16) {
    const char* base = (const char*)(src.p + (int64_t)b * src.sb + (int64_t)h * src.sh + (int64_t)(row0 + r0) * src.ss);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(base, ro.o[i], la + 4 * i * kRowB);
  } else {
    const int rbase = r0 < nvalid ? r0 : nvalid - 1;  // a valid source row
    const char* base =
        (const char*)(src.p + (int64_t)b * src.sb + (int64_t)h * src.sh + (int64_t)(row0 + rbase) * src.ss);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kl = 4 * i + (lane >> 4);                // LDS row within the wave's 16
      const int srow = min(r0 + kl, nvalid - 1) - rbase;  // source row relative to the base, >= 0
      const int chunk = (lane & 15) ^ swz(kl);
      dma16(base, (uint32_t)(srow * (uint32_t)src.ss + 8 * chunk) * 2u, la + 4 * i * kRowB);
    }
  }
}

// Wait until at most n of this wave's vector-memory operations are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(n) : "memory");
}

// Group g's barrier: if this wave's group (wave-uniform, in an SGPR) is g,
// wait until at most n of its vector-memory operations are in flight, then
// s_barrier; other waves skip both.  One asm block, so the compiler sees no
// branch between the blocks around it (a branch there makes it spill the
// matrix-phase registers).
template <int g, int n>
__device__ __forceinline__ void group_barrier(int grp) {
  asm volatile("s_cmp_eq_u32 %0, %1\n\ts_cbranch_scc0 2\n\ts_waitcnt vmcnt(%2)\n\ts_barrier"
               :
               : "s"(grp), "i"(g), "i"(n)
               : "memory", "scc");
}

// ------------------------------------------------------ matrix phase (all passes)
// State of one wave: 32 rows of the fixed side (queries for dQ, keys for dK
// and dV) in registers, one tile of the streamed side in LDS.
struct GState {
  f32x16 acc[4];        // gradient^T: 4 head-dim blocks x 32 fixed rows
  f32x16 s[2], dp[2];   // scores and dP of one tile (two 32-row blocks)
  u32x4 dh[4], dl[4];   // hi / lo BF16 B operand of the gradient, four 16-row chunks
  bf16x8 b1[8], b2[8];  // fixed-side rows: B operands of the scores (b1) and dP (b2)
  float lse2, D;        // dQ pass: LSE*log2 e and D of the lane's query
};
struct GBases {
  uint32_t t, r1, r2;  // transposed tile (gradient), row tiles of the scores and of dP
};
// Steps: gradient steps j = 0..7 (chunk j/2, head-dim blocks 2(j%2) and
// 2(j%2)+1; two transposed fragments, 4 MFMAs), then score steps: with dP,
// j = 0..15 covers head-dim chunk j/2 of 32-row block j%2 (S and dP, two
// row fragments); without, j = 0..7 covers chunk j of both blocks (S only).
// Each step reads two fragments, A steps before its MFMAs (A = 2 in the dQ
// pass, whose registers are full; 3 in the dK and dV passes).
template <int A>
using Ring = bf16x8[A + 1][2];

// kF16 (dV pass): the gradient's A operand comes from a transposed FP16
// tile, one ds_read_b128 per fragment instead of two transposing reads.
template <bool kAcc, bool kS, bool kDp, bool kF16, int A>
struct Plan {
  static constexpr int nacc = kAcc ? 8 : 0;
  static constexpr int n = nacc + (kS ? (kDp ? 16 : 8) : 0);
  static constexpr int reads(int k) { return k < n ? (k < nacc ? (kF16 ? 2 : 4) : 2) : 0; }
  static constexpr int later(int k) {  // LDS reads issued after step k's own, before its MFMAs
    int r = 0;
    for (int i = 1; i <= A; ++i) r += reads(k + i);
    return r;
  }
};

template <bool kAcc, bool kS, bool kDp, bool kF16, int A, int k>
__device__ __forceinline__ void g_issue(Ring<A>& f, const GBases& b) {
  using P = Plan<kAcc, kS, kDp, kF16, A>;
  if constexpr (k < P::n) {
    bf16x8* x = f[k % (A + 1)];
    if constexpr (k < P::nacc) {
      constexpr int c2 = k >> 1, d0 = 2 * (k & 1), d1 = d0 + 1;
      if constexpr (kF16) {
        x[0] = __builtin_bit_cast(bf16x8, ds_b128<d0 * 32 * kVtRowB>(b.t ^ (uint32_t)(c2 << 5)));
        x[1] = __builtin_bit_cast(bf16x8, ds_b128<d1 * 32 * kVtRowB>(b.t ^ (uint32_t)(c2 << 5)));
      } else {
        x[0] = tr_frag<c2, d0>(b.t);
        x[1] = tr_frag<c2, d1>(b.t);
      }
    } else if constexpr (kDp) {
      constexpr int j = k - P::nacc, kk = j >> 1, kb = j & 1;
      x[0] = row_frag<kk, kb>(b.r1);
      x[1] = row_frag<kk, kb>(b.r2);
    } else {
      constexpr int kk = k - P::nacc;
      x[0] = row_frag<kk, 0>(b.r1);
      x[1] = row_frag<kk, 1>(b.r1);
    }
  }
}

template <bool kAcc, bool kS, bool kDp, bool kF16, int A, int k>
__device__ __forceinline__ void g_step(GState& st, Ring<A>& f, const GBases& b) {
  using P = Plan<kAcc, kS, kDp, kF16, A>;
  if constexpr (k < P::n) {
    g_issue<kAcc, kS, kDp, kF16, A, k + A>(f, b);
    constexpr int later = P::later(k);
    static_assert(later <= 15, "lgkmcnt holds at most 15");
    bf16x8* x = f[k % (A + 1)];
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x[0]), "+v"(x[1]) : "i"(later));
    if constexpr (k < P::nacc) {
      constexpr int c2 = k >> 1, d0 = 2 * (k & 1), d1 = d0 + 1;
      if constexpr (kF16) {  // FP16 operands, one product
        using attn::f16x8;
        st.acc[d0] = attn::mfma32h(__builtin_bit_cast(f16x8, x[0]), __builtin_bit_cast(f16x8, st.dh[c2]), st.acc[d0]);
        st.acc[d1] = attn::mfma32h(__builtin_bit_cast(f16x8, x[1]), __builtin_bit_cast(f16x8, st.dh[c2]), st.acc[d1]);
      } else {
        st.acc[d0] = mfma32(x[0], __builtin_bit_cast(bf16x8, st.dh[c2]), st.acc[d0]);
        st.acc[d1] = mfma32(x[1], __builtin_bit_cast(bf16x8, st.dh[c2]), st.acc[d1]);
        st.acc[d0] = mfma32(x[0], __builtin_bit_cast(bf16x8, st.dl[c2]), st.acc[d0]);
        st.acc[d1] = mfma32(x[1], __builtin_bit_cast(bf16x8, st.dl[c2]), st.acc[d1]);
      }
    } else if constexpr (kDp) {
      // the first chunk starts from a zero accumulator operand, so S and dP
      // are not live during the gradient steps before them
      constexpr int j = k - P::nacc, kk = j >> 1, kb = j & 1;
      const f32x16 z = {};
      st.s[kb] = mfma32(x[0], st.b1[kk], kk == 0 ? z : st.s[kb]);
      st.dp[kb] = mfma32(x[1], st.b2[kk], kk == 0 ? z : st.dp[kb]);
    } else {
      constexpr int kk = k - P::nacc;
      const f32x16 z = {};
      st.s[0] = mfma32(x[0], st.b1[kk], kk == 0 ? z : st.s[0]);
      st.s[1] = mfma32(x[1], st.b1[kk], kk == 0 ? z : st.s[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    g_step<kAcc, kS, kDp, kF16, A, k + 1>(st, f, b);
  }
}

template <bool kAcc, bool kS, bool kDp, bool kF16, int A, int k>
__device__ __forceinline__ void g_prefetch(Ring<A>& f, const GBases& b) {
  if constexpr (k < A) {
    g_issue<kAcc, kS, kDp, kF16, A, k>(f, b);
    g_prefetch<kAcc, kS, kDp, kF16, A, k + 1>(f, b);
  }
}

template <bool kAcc, bool kS, bool kDp, bool kF16 = false, int A = 2>
__device__ __forceinline__ void g_matrix(GState& st, GBases b) {
  Ring<A> f;
  // opaque copies keep the per-step address XORs inside their steps
  asm volatile("" : "+v"(b.t), "+v"(b.r1), "+v"(b.r2));
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  g_prefetch<kAcc, kS, kDp, kF16, A, 0>(f, b);
  __builtin_amdgcn_sched_barrier(0);
  g_step<kAcc, kS, kDp, kF16, A, 0>(st, f, b);
  __builtin_amdgcn_s_setprio(0);
}

// ----------------------------------------------------------------- dQ pass
// Key tiles in the forward's logical order.  Group 0 loads V_{t+2} and
// group 1 K_{t+2} in their VALU phase of tile t.
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
template <bool kMask>
__device__ __forceinline__ void dq_softmax_t(GState& st, int cur_valid, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // key of register r in block kb: 32*kb + 8*(r/4) + 4*hh + r%4
      const int key = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[kb][r], kC, -st.lse2));
      const float p = !kMask || key < cur_valid ? e : 0.f;
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
// Full tiles (every tile but the last of each key segment) skip the mask.
__device__ __forceinline__ void dq_softmax(GState& st, int cur_valid, int hh) {
  if (cur_valid >= kBwdBN)
    dq_softmax_t<false>(st, cur_valid, hh);
  else
    dq_softmax_t<true>(st, cur_valid, hh);
}

}  // namespace

// D_i = dO_i . O_i from the forward's FP32 (pre-cast) O, in a fixed order
// (per lane half: chunk, then channel; then the two halves), LSE_i * log2(e)
// for the key-side passes, and each wave's max |dO| for the dV operand's
// scale.  Rows as in the dQ pass.
__global__ __launch_bounds__(kBwdDqWaves * 64) void attn_bwd_prep_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  int b, h, qt;
  decode_bh(a, a.n_qtiles, blockIdx.x, b, h, qt);
  const int qrow = qt * (kBwdDqWaves * 32) + wave * 32 + lr;
  const bool qvalid = qrow < a.S;
  float dpart = 0.f;
  uint32_t amax = 0;  // max |dO| of this lane's values, as BF16 magnitude bits (ordered like the values)
  // All 24 loads first, branch-free (rows past S read row S-1, and a bit
  // mask turns their values into +0), so none of them waits for another.
  const int qr = qvalid ? qrow : a.S - 1;
  const uint32_t vm = qvalid ? ~0u : 0u;
  u32x4 zdv[8];
  f32x4 o0v[8], o1v[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    zdv[kk] = *(const u32x4*)(a.dO.row(b, qr, h) + 16 * kk + 8 * hh);
    const float* orow = a.o.row(b, qr, h) + 16 * kk + 8 * hh;
    o0v[kk] = *(const f32x4*)orow;
    o1v[kk] = *(const f32x4*)(orow + 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x4 zd = zdv[kk] & vm;
    const f32x4 o0 = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, o0v[kk]) & vm);
    const f32x4 o1 = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, o1v[kk]) & vm);
    const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = bf16_lo(zd[w]) * ov[2 * w];
      dpart = dpart + p0;
      const float p1 = bf16_hi(zd[w]) * ov[2 * w + 1];
      dpart = dpart + p1;
      amax = max(amax, max(zd[w] & 0x7fffu, (zd[w] >> 16) & 0x7fffu));
    }
  }
  const float D = dpart + __shfl_xor(dpart, 32);
  // this wave's max |dO| (order-free)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));
  if (lane == 0) a.do_amax[(((int64_t)b * a.H + h) * a.n_qtiles + qt) * kBwdDqWaves + wave] = amax;
  if (qvalid && hh == 0) {
    const int64_t li = ((int64_t)b * a.H + h) * a.S + qrow;
    a.Dvec[li] = D;
    a.lse2[li] = a.lse[li] * kLog2e;
  }
}

namespace {

__device__ __forceinline__ void dq_pass(const BwdArgs& a, char* smem, int g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, sub = wave & 3;
  const int lr = lane & 31, hh = lane >> 5;
  int b, h, qt;
  decode_bh(a, a.n_qtiles, g, b, h, qt);
  const int L = a.txt_len[b];
  const int qrow = qt * (kBwdDqWaves * 32) + wave * 32 + lr;
  const bool qvalid = qrow < a.S;

  GState st;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
    if (qvalid) {
      zq = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
      zd = *(const u32x4*)(a.dO.row(b, qrow, h) + 16 * kk + 8 * hh);
    }
    st.b1[kk] = __builtin_bit_cast(bf16x8, zq);
    st.b2[kk] = __builtin_bit_cast(bf16x8, zd);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[d][r] = 0.f;

  const int ntxt = (L + kBwdBN - 1) / kBwdBN;
  const int nt = ntxt + (a.T_img + kBwdBN - 1) / kBwdBN;
  char* const kbase = smem;
  char* const vbase = smem + kRing * kTileB;
  auto kbuf = [&](int j) { return kbase + (j % kRing) * kTileB; };
  auto vbuf = [&](int j) { return vbase + (j % kRing) * kTileB; };
  auto valid_of = [&](int j) {
    int k0, nv;
    dq_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    return nv;
  };
  const RowOff ko = row_offsets(a.k.ss, lane), vo = row_offsets(a.v.ss, lane);
  // Tile j into ring slot j % 4; for j >= nt the last tile again (a load
  // into a free slot that nothing reads, so every iteration issues the same
  // loads and the waits are fixed counts).
  auto load_k = [&](int j) {
    int k0, nv;
    dq_bounds(min(j, nt - 1), ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows_rep(a.k, ko, kbuf(j), b, h, k0, nv, sub, lane);
  };
  auto load_v = [&](int j) {
    int k0, nv;
    dq_bounds(min(j, nt - 1), ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows_rep(a.v, vo, vbuf(j), b, h, k0, nv, sub, lane);
  };
  auto bases = [&](int t) {
    GBases bb;
    bb.t = tr_base(addr_of(kbuf(t)), lane);
    bb.r1 = row_base(addr_of(kbuf(t + 1)), lane);
    bb.r2 = row_base(addr_of(vbuf(t + 1)), lane);
    return bb;
  };

  // Schedule: one barrier B_t per key tile.  A wave runs VALU(t) (P, dS,
  // hi/lo split of tile t) then MM(t) (dQ MFMAs of tile t, then S and dP of
  // tile t+1); group 1 passes B_t before VALU(t), group 0 between VALU(t)
  // and MM(t), so between B_t and B_{t+1} both groups run MM(t) and a group
  // that finishes its VALU block starts its MFMAs beside the other's.
  // MM(t) reads K tile t (transposed) and K, V tiles t+1; no VALU block
  // reads LDS.  Tiles 0-2 are loaded up front; then V tile t+3 by group 0
  // before B_t (V tile t-1, in its slot, was last read by MM(t-2)) and K
  // tile t+3 by group 1 after B_t (K tile t-1 was last read by MM(t-1)).
  // Each wave issues four loads per iteration, and at B_t it has landed
  // every load but its latest four (group 0: tile t+3, group 1: tile t+2),
  // so tile t+1 is visible to all after B_t.
  if (grp == 0) {
    for (int j = 0; j < 3 && j < nt; ++j) load_v(j);
  } else {
    for (int j = 0; j < 3 && j < nt; ++j) load_k(j);
  }
  // The row's LSE and D after the first tiles' loads, so that their wait
  // is the one before the first barrier (not a wait of its own before the
  // tile loads are issued).
  st.lse2 = INFINITY;
  st.D = 0.f;
  if (qvalid) {
    const int64_t li = ((int64_t)b * a.H + h) * a.S + qrow;
    st.lse2 = a.lse[li] * kLog2e;
    st.D = a.Dvec[li];
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  bar();
  {
    GBases b0;
    b0.t = 0;
    b0.r1 = row_base(addr_of(kbuf(0)), lane);
    b0.r2 = row_base(addr_of(vbuf(0)), lane);
    g_matrix<false, true, true>(st, b0);
  }
#pragma clang loop unroll(disable)
  for (int t = 0; t + 1 < nt; ++t) {
    group_barrier<1, 4>(grp);  // B_t for group 1
    if (grp == 1)
      load_k(t + 3);
    else
      load_v(t + 3);
    dq_softmax(st, valid_of(t), hh);
    group_barrier<0, 4>(grp);  // B_t for group 0
    g_matrix<true, true, true>(st, bases(t));
  }
  // the last tile
  group_barrier<1, 0>(grp);
  dq_softmax(st, valid_of(nt - 1), hh);
  group_barrier<0, 0>(grp);
  {
    GBases bl;
    bl.t = tr_base(addr_of(kbuf(nt - 1)), lane);
    bl.r1 = 0;
    bl.r2 = 0;
    g_matrix<true, false, true>(st, bl);
  }

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

// ------------------------------------------------------------ dK and dV passes

// Query tiles in the frozen order: valid text, image, padded text.
struct QTiles {
  int L, T_txt, T_img, nq_txt, nq_img, nq_pad;
  __device__ QTiles(int L_, int T_txt_, int T_img_) : L(L_), T_txt(T_txt_), T_img(T_img_) {
    nq_txt = (L + kBwdBM - 1) / kBwdBM;
    nq_img = (T_img + kBwdBM - 1) / kBwdBM;
    nq_pad = (T_txt - L + kBwdBM - 1) / kBwdBM;
  }
  __device__ int count() const { return nq_txt + nq_img + nq_pad; }
  __device__ void bounds(int t, int& q0, int& nq) const {
    if (t < nq_txt) {
      q0 = t * kBwdBM;
      nq = min(kBwdBM, L - q0);
    } else if (t < nq_txt + nq_img) {
      const int ti = t - nq_txt;
      q0 = T_txt + ti * kBwdBM;
      nq = min(kBwdBM, T_img - ti * kBwdBM);
    } else {
      const int ti = t - nq_txt - nq_img;
      q0 = L + ti * kBwdBM;
      nq = min(kBwdBM, T_txt - L - ti * kBwdBM);
    }
  }
};

// P = exp2(s*c - LSE*log2 e) and, for dK, dS = P (dP - D), per query row
// (register r of block qb holds query 32*qb + 8*(r/4) + 4*hh + r%4).  dS of
// rows past the tile's valid count is exactly 0.  P of those rows is not
// masked in the dV pass: their Q rows and LSE entries repeat the tile's last
// valid row, so P lies in [0, 1], and the dO^T columns it meets are zero.
// dS is split hi/lo per 16-row chunk; P (dV) is rounded once to FP16.
template <bool kDk, bool kMask>
__device__ __forceinline__ void kv_softmax_t(GState& st, const float* lse, const float* dd, int nq, int hh) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q0 = 32 * qb + 8 * j + 4 * hh;
      const f32x4 lv = *(const f32x4*)(lse + q0);
      f32x4 dv = {0.f, 0.f, 0.f, 0.f};
      if (kDk) dv = *(const f32x4*)(dd + q0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * j + u;
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[qb][r], kC, -lv[u]));  // lv: LSE * log2(e)
        if constexpr (kDk) {
          // row 32*qb + 8*j + u in lanes 0-31, 4 more in lanes 32-63: the
          // lane mask is uniform, so it is formed with scalar instructions
          const int rlo = 32 * qb + 8 * j + u;
          const uint64_t m = (rlo < nq ? 0x00000000ffffffffull : 0ull) | (rlo + 4 < nq ? 0xffffffff00000000ull : 0ull);
          const float v = e * (st.dp[qb][r] - dv[u]);
          float xm;
          asm("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(xm) : "v"(v), "s"(m));
          x[r] = xm;
        } else {
          x[r] = e;
        }
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if constexpr (kDk) {
        uint32_t hi[4], lo[4];
        split_pack(x + 8 * half, hi, lo);
        st.dh[2 * qb + half] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        st.dl[2 * qb + half] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      } else {  // dV: P in FP16 (RNE), one operand
        const float* v = x + 8 * half;
        st.dh[2 * qb + half] = u32x4{attn::pack_f16x2(v[0], v[1]), attn::pack_f16x2(v[2], v[3]),
                                     attn::pack_f16x2(v[4], v[5]), attn::pack_f16x2(v[6], v[7])};
      }
    }
  }
}
// The dV pass has no mask; the dK pass masks dS with lane masks built on
// the scalar unit (one v_cndmask per value, no vector compare).
template <bool kDk>
__device__ __forceinline__ void kv_softmax(GState& st, const float* lse, const float* dd, int nq, int hh) {
  kv_softmax_t<kDk, kDk>(st, lse, dd, nq, hh);
}

constexpr int kKvKeysPerWG = kBwdKvWaves * 32;
constexpr int kKvSmem = 2 * kRing * kTileB + 2 * kRing * kBwdBM * 4;  // Q, dO tile rings; LSE, D row rings

// kDk: dK pass (S, dP, dK^T += Q^T dS); else dV pass (S, dV^T += dO^T P).
// Loads two tiles ahead in the VALU phase of tile t -- dK: group 0 dO and D,
// group 1 Q and LSE; dV: group 0 Q and LSE, group 1 dO -- each group waiting
// for its loads at the end of its next matrix phase.
template <bool kDk>
__device__ __forceinline__ void kv_pass(const BwdArgs& a, char* smem, int g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, sub = wave & 3;
  const int lr = lane & 31, hh = lane >> 5;
  int b, h, kt;
  decode_bh(a, a.n_ktiles, g, b, h, kt);
  const int L = a.txt_len[b];
  const int nkt_txt = (L + kKvKeysPerWG - 1) / kKvKeysPerWG;
  const int nkt_img = (a.T_img + kKvKeysPerWG - 1) / kKvKeysPerWG;
  const int nkt_pad = (a.T_txt - L + kKvKeysPerWG - 1) / kKvKeysPerWG;
  if (kt >= nkt_txt + nkt_img + nkt_pad) return;  // whole workgroup

  int kbase, kend;
  bool zero_only = false;
  if (kt < nkt_txt) {
    kbase = kt * kKvKeysPerWG;
    kend = L;
  } else if (kt < nkt_txt + nkt_img) {
    kbase = a.T_txt + (kt - nkt_txt) * kKvKeysPerWG;
    kend = a.S;
  } else {
    kbase = L + (kt - nkt_txt - nkt_img) * kKvKeysPerWG;
    kend = a.T_txt;
    zero_only = true;
  }
  const int key = kbase + 32 * wave + lr;
  const bool kvalid = key < kend;
  float* const out = kvalid ? (kDk ? a.dk.row(b, key, h) : a.dv.row(b, key, h)) : nullptr;

  if (zero_only) {  // masked text keys: exact zeros (whole workgroup)
    if (kvalid) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) *(f32x4*)(out + 64 * hh + 4 * i) = z;
    }
    return;
  }

  GState st;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (kvalid) {
      zk = *(const u32x4*)(a.k.row(b, key, h) + 16 * kk + 8 * hh);
      if (kDk) zv = *(const u32x4*)(a.v.row(b, key, h) + 16 * kk + 8 * hh);
    }
    st.b1[kk] = __builtin_bit_cast(bf16x8, zk);
    st.b2[kk] = __builtin_bit_cast(bf16x8, zv);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[d][r] = 0.f;

  const QTiles qt(L, a.T_txt, a.T_img);
  const int nt = qt.count();
  char* const qbase = smem;
  char* const obase = smem + kRing * kTileB;
  float* const lbase = (float*)(smem + 2 * kRing * kTileB);
  float* const dbase = lbase + kRing * kBwdBM;
  auto qbuf = [&](int j) { return qbase + (j % kRing) * kTileB; };
  auto obuf = [&](int j) { return obase + (j % kRing) * kTileB; };
  auto lrow = [&](int j) { return lbase + (j % kRing) * kBwdBM; };
  auto drow = [&](int j) { return dbase + (j % kRing) * kBwdBM; };
  auto nq_of = [&](int j) {
    int q0, nq;
    qt.bounds(j, q0, nq);
    return nq;
  };
  // Group 0 loads the tensor read only as score-side rows (dK: dO for dP;
  // dV: Q for S); group 1 the tensor also read transposed by the gradient
  // (dK: Q; dV: FP16 dO * 2^e as transposed tiles written by do_convert)
  // with the tile's LSE (and, for dK, D) row.
  const RowOff ro = row_offsets((grp == 0) == kDk ? a.dO.ss : a.q.ss, lane);
  const VtOff vo = vt_offsets(lane);
  const uint16_t* const dot_bh = a.do16t + ((int64_t)b * a.H + h) * a.nt_do * kVtileElems;
  const int64_t hb = ((int64_t)b * a.H + h) * a.S;  // [b, h] row of LSE and D
  // Tile j into ring slot j % 4; for j >= nt the last tile again (a load
  // into a free slot that nothing reads, so every iteration issues the same
  // loads and the waits are fixed counts).
  auto load_g0 = [&](int j) {
    const int js = min(j, nt - 1);
    int q0, nq;
    qt.bounds(js, q0, nq);
    load_rows_rep(kDk ? a.dO : a.q, ro, kDk ? obuf(j) : qbuf(j), b, h, q0, nq, sub, lane);
  };
  // Group 1 also loads the tile's LSE (and D) row: wave `sub` its entries
  // 16*sub .. 16*sub+15, rows past the tile's valid count repeating its last
  // row (those entries are masked), so each wave issues 4 + 1 (+ 1) loads.
  auto load_g1 = [&](int j) {
    const int js = min(j, nt - 1);
    int q0, nq;
    qt.bounds(js, q0, nq);
    if constexpr (kDk)
      load_rows_rep(a.q, ro, qbuf(j), b, h, q0, nq, sub, lane);
    else
      load_vt(dot_bh + (int64_t)js * kVtileElems, vo, obuf(j), sub);
    if (lane < 16) {
      const uint32_t r = (uint32_t)min(16 * sub + lane, nq - 1);
      dma4((const char*)(a.lse2 + hb + q0), 4u * r, addr_of((const char*)(lrow(j) + 16 * sub)));
      if (kDk) dma4((const char*)(a.Dvec + hb + q0), 4u * r, addr_of((const char*)(drow(j) + 16 * sub)));
    }
  };
  auto bases = [&](int t, bool next) {
    GBases bb;
    bb.t = kDk ? tr_base(addr_of(qbuf(t)), lane) : vt_base(addr_of(obuf(t)), lane);
    bb.r1 = next ? row_base(addr_of(qbuf(t + 1)), lane) : 0;
    bb.r2 = next ? row_base(addr_of(obuf(t + 1)), lane) : 0;
    return bb;
  };
  constexpr int kG1Loads = kDk ? 6 : 5;  // group 1's loads per tile

  // Schedule as in the dQ pass: one barrier B_t per query tile; group 1
  // passes it before VALU(t) (P and, for dK, dS of tile t from the LSE and D
  // rows in LDS), group 0 between VALU(t) and MM(t) (the gradient MFMAs of
  // tile t, then S and dP of tile t+1).  Between B_t and B_{t+1} the LDS
  // reads are: tile t of group 1's tensor (transposed), tile t+1 of both
  // tensors (rows), and the LSE/D rows of tiles t and t+1.  Tiles 0-2 up
  // front; tile t+3 of group 0's tensor before B_t (its slot's previous
  // tile, t-1, was last read by MM(t-2)), of group 1's tensor and rows
  // after B_t (last read by MM(t-1) and VALU(t-1)).  At B_t each wave has
  // landed every load but its latest tile's, so tile t+1 is visible after
  // B_t.
  for (int j = 0; j < 3 && j < nt; ++j) {
    if (grp == 0)
      load_g0(j);
    else
      load_g1(j);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  bar();
  {
    GBases b0;
    b0.t = 0;
    b0.r1 = row_base(addr_of(qbuf(0)), lane);
    b0.r2 = row_base(addr_of(obuf(0)), lane);
    g_matrix<false, true, kDk, false, 3>(st, b0);
  }
#pragma clang loop unroll(disable)
  for (int t = 0; t + 1 < nt; ++t) {
    group_barrier<1, kG1Loads>(grp);  // B_t for group 1: tile t+2 may stay in flight
    if (grp == 1)
      load_g1(t + 3);
    else
      load_g0(t + 3);
    kv_softmax<kDk>(st, lrow(t), drow(t), nq_of(t), hh);
    group_barrier<0, 4>(grp);  // B_t for group 0: tile t+3, issued just now, may stay in flight
    g_matrix<true, true, kDk, !kDk, 3>(st, bases(t, true));
  }
  // the last tile
  group_barrier<1, 0>(grp);
  kv_softmax<kDk>(st, lrow(nt - 1), drow(nt - 1), nq_of(nt - 1), hh);
  group_barrier<0, 0>(grp);
  g_matrix<true, false, kDk, !kDk, 3>(st, bases(nt - 1, false));

  if (kvalid) {
    // dK: times 1/sqrt(128); dV: times 2^-e, undoing dO's power-of-two scale (exact)
    const float f = kDk ? kScale : a.do_inv_scale[(int64_t)b * a.H + h];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        *(f32x4*)(out + d0) = f32x4{st.acc[d][4 * g4] * f, st.acc[d][4 * g4 + 1] * f, st.acc[d][4 * g4 + 2] * f,
                                    st.acc[d][4 * g4 + 3] * f};
      }
  }
}

}  // namespace

// The three passes in one grid: dK workgroups first, then dQ, then dV (the
// shortest).  Each workgroup runs one pass body; nothing is shared between
// workgroups, so every output bit is what the pass computes on its own.  One
// grid instead of three leaves a single partly filled last round.
static_assert(kBwdKvWaves == kBwdDqWaves && kKvSmem >= 2 * kRing * kTileB, "one workgroup shape for the three passes");
__global__ __launch_bounds__(kBwdKvWaves * 64, 1) void attn_bwd_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kKvSmem];
  const int g = blockIdx.x;
  const int n_kv = a.B * a.H * a.n_ktiles, n_dq = a.B * a.H * a.n_qtiles;
  if (g < n_kv)
    kv_pass<true>(a, smem, g);
  else if (g < n_kv + n_dq)
    dq_pass(a, smem, g - n_kv);
  else
    kv_pass<false>(a, smem, g - n_kv - n_dq);
}

// dO for the dV product: FP16 of dO * 2^e with one power of two per (sample,
// head), chosen from that slice's max |dO| so that its largest element lands
// in [2^14, 2^15) (e at most 100).  The scaling is exact and the conversion
// rounds to nearest even: relative error <= 2^-11 for |dO| >= max|dO| * 2^-28,
// absolute error <= max|dO| * 2^-39 below (e under its cap).  The maximum is order-free and
// covers only the slice's own rows, so the scale, like every output bit,
// depends on nothing outside the (sample, head).
//
// One workgroup per query tile t of the dK/dV passes' frozen order (valid
// text, image, padded text) of one (b, h): the tile's rows are staged in LDS,
// then written as 128 channel rows of 64 FP16 values, the queries of each
// 16-row chunk in the dV product's reduction order (position p holds row p
// with bits 2 and 3 swapped) and zero past the tile's valid count -- the
// layout of the forward's V^T key tiles, so a fragment is one 16-byte read.
__global__ __launch_bounds__(256) void do_convert_kernel(DoPrepArgs a) {
  __shared__ uint32_t red[4];
  __shared__ uint32_t tl[kBwdBM][kHeadDim / 2 + 1];  // [query][channel pair]; one pad word per row
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + h;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < a.n_amax; i += 256) m = max(m, a.amax[bh * a.n_amax + i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  int e = 0;  // max |dO| = f * 2^E with f in [0.5, 1): scale by 2^(15 - E)
  if (m != 0u && m < 0x7f80u) {  // nonzero and finite
    int E;
    (void)frexpf(__uint_as_float(m << 16), &E);
    e = min(15 - E, 100);
  }
  if (t == 0 && threadIdx.x == 0) a.inv_scale[bh] = ldexpf(1.0f, -e);
  const QTiles qt(a.txt_len[b], a.T_txt, a.T_img);
  if (t >= qt.count()) return;  // whole workgroup
  int q0, nq;
  qt.bounds(t, q0, nq);
  for (int i = threadIdx.x; i < kBwdBM * 16; i += 256) {  // 16 chunks of 8 channels per row
    const int r = i >> 4, c = i & 15;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < nq) w = *(const u32x4*)(a.dO.row(b, q0 + r, h) + 8 * c);
#pragma unroll
    for (int k = 0; k < 4; ++k) tl[r][4 * c + k] = w[k];
  }
  __syncthreads();
  uint16_t* const out = a.out + (bh * a.nt_do + t) * kVtileElems;
  for (int i = threadIdx.x; i < kHeadDim * 8; i += 256) {
    const int d = i >> 3, j = i & 7;  // channel row, 8-query chunk of the row
    float f[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = 8 * (j & 1) + k;  // position within 16-row chunk j/2
      const int r = 16 * (j >> 1) + ((p & 3) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3));
      const uint32_t w = tl[r][d >> 1];
      f[k] = ldexpf((d & 1) ? bf16_hi(w) : bf16_lo(w), e);
    }
    const u32x4 o = {attn::pack_f16x2(f[0], f[1]), attn::pack_f16x2(f[2], f[3]), attn::pack_f16x2(f[4], f[5]),
                     attn::pack_f16x2(f[6], f[7])};
    *(u32x4*)(out + d * kBwdBM + 8 * j) = o;
  }
}

}  // namespace qi
