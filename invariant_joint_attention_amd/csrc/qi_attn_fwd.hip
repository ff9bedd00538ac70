// qi_attn_fwd.hip -- masked non-causal joint attention forward on gfx950.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// joint_attn_qk_gemm, joint_attn_softmax, joint_attn_av_gemm and
// joint_attention_fused; [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Model contract"
// rows Streams and Text input, and "Numerical requirements" (fixed reduction
// trees, FP32 accumulation, no split-KV, one output cast, batch invariance).
//
// Arithmetic (frozen; every launch shape gives the same bits):
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    A = a 32-key block of K, B = 32 query rows of Q held in registers for
//    the whole key loop.  Lane l owns query l%32 and 16 keys per block, so
//    the row max is an in-lane max plus one exchange with lane l^32, and the
//    softmax rescale factor is a per-lane scalar.  Each 32-key block
//    accumulates its 8 head-dim chunks in order.
//  * O^T = V^T P^T accumulates in 4 blocks of 32x32 FP32 with
//    v_mfma_f32_32x32x16_f16, one product per 16-key chunk in key order.
//    P enters as FP16 (RNE; p <= 256, and values below 2^-24 that flush to
//    zero weigh less than 2^-24 of a row whose largest p is at least 1), V
//    as FP16 of v * 2^-8, written by a conversion pass as transposed key
//    tiles (exact for 2^-6 <= |v| <= 65504 * 2^8; smaller |v| keep an absolute
//    error below 2^-17).  One BF16 rounding of P would move O by up to
//    2^-9 * sum_j p_j|v_j| / l, which breaks the output tolerance where O
//    cancels on few, peaked keys; FP16 P has 2^-12.  The MFMA reduction index
//    is a permutation of the 16 keys of a chunk (bits 2 and 3 of the key
//    index swapped) that matches the accumulator layout of P; the
//    conversion pass stores the keys of each chunk in that order.
//  * Keys are tiled LOGICALLY: ceil(L_b/64) text tiles starting at key 0,
//    then ceil(T_img/64) image tiles starting at key T_txt.  Masked keys are
//    never read (their LDS slots are zero) and get probability exactly 0, so
//    a row's arithmetic does not depend on T_txt, on the batch or on the
//    workgroup shape.  The key tile width 64 is frozen.
//  * Online softmax in the exp2 domain with c = log2(e)/sqrt(128):
//    p = exp2(s*c - m*c) (one fma); the row sum l adds the FP32 p lane by lane
//    in register order, then the two half-waves (commutative, so both get the
//    same bits); O = acc / (l * 2^-8) (exact rescaling of the V scale) and
//    LSE = (m*c + log2 l) * ln 2.
//    The reference max m moves only when a tile max exceeds it by more than
//    8/c (so p <= 256): each lane decides from its own row alone, and the
//    rescale (factor exactly 1 where m did not move) is skipped when no lane
//    of the wave moved.
//
// Schedule (free; does not change any bit):
//  * Workgroup = 8 waves x 32 query rows of one (b, h).  Waves w and w+4 run
//    on the same SIMD.  A wave alternates a softmax block (VALU only) and a
//    matrix block (P*V of tile t plus the scores of tile t+1, 32 MFMAs); group
//    0 (waves 0-3) and group 1 (waves 4-7) are half a tile apart, with one
//    workgroup barrier per tile, so each SIMD has one wave issuing MFMAs
//    while its partner runs the softmax; the switch in mid-tile is
//    self-timed (details at the schedule section below).
//  * LDS: K tiles and V^T tiles in rings of four (128 KiB).  K rows are
//    unpadded 256-byte lines whose 16-byte chunks are XOR-swizzled by key
//    (swizzle bits 2-3 from key bits 0-1, bits 0-1 from key bits 2-3); V^T
//    tiles are 128 channel lines of 128 bytes swizzled by channel/2.  The K
//    and V^T fragment reads (one ds_read_b128 each, 16 rows per 16-lane
//    group) and the contiguous direct-load writes meet no LDS bank conflict
//    on the 64 banks.  Tiles are filled by direct global->LDS loads
//    (global_load_lds_dwordx4), group 0 the K tiles and group 1 the V^T
//    tiles, at the start of a softmax block, three tiles ahead.
//  * The softmax block ends with P rounded to FP16, so one FP32 score buffer
//    suffices: the matrix block accumulates the next tile's scores into it.
//  * The matrix block issues its LDS reads as inline asm three steps ahead of
//    use and waits for each step's read with an exact lgkmcnt; the direct
//    loads are inline asm too, so the compiler neither inserts waits for
//    them before unrelated LDS reads nor keeps 64-bit addresses for them.
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_attn_contract.h"
#include "qi_lds.h"
#include "qi_vtiles.h"

#include <type_traits>

namespace qi {

namespace {

using namespace lds;
using namespace attn;
static_assert(kTileRows == kFwdBN, "forward key tile is one LDS tile");

// ---------------------------------------------------------------- schedule
// Workgroup = 8 waves x 32 query rows of one (b, h); waves w and w+4 share a
// SIMD and belong to group 0 (waves 0-3) and group 1 (waves 4-7).  A wave's
// work per tile alternates a matrix block MM(t) = P*V of tile t and the
// scores of tile t+1 (32 MFMAs) with a softmax block SM(t+1) (VALU only:
// mask, row max, lazy reference-max move and rescale, p = exp2, row sum,
// FP16 packing of P).  One workgroup barrier B_t per tile; between B_t and
// B_{t+1}
//   group 0 runs MM(t), then SM(t+1);
//   group 1 runs SM(t),  then MM(t);
// so on each SIMD one wave issues MFMAs while its partner runs the softmax,
// and the mid-tile switch is self-timed: a group that finishes its softmax
// early starts its matrix block beside the partner's, which keeps the MFMA
// pipe busy until the barrier as long as a softmax block is shorter than a
// matrix block.
//
// LDS: K tiles in a ring of four, V^T tiles in a ring of four (128 KiB).
// Between B_t and B_{t+1} both groups read V tile t and K tile t+1; tiles
// are loaded four (K) and three (V) tiles ahead and each wave has its own
// loads of the tile before landed by the next barrier, so every tile is
// visible one tile before it is read: a matrix block's first fragments are
// read at the end of the softmax block before it, across the barrier for
// group 0.
struct St {
  f32x16 acc[4];  // O^T [32-channel block], FP32 (V scaled by 2^-8)
  f32x16 s[2];    // scores [32-key block]
  u32x4 p[4];     // FP16 P [16-key chunk]
  bf16x8 q[8];    // Q [16-channel chunk]
  float m_used, l;
};

// Per-lane LDS fragment addresses relative to K buffer 0 / V buffer 0: eight
// K row-fragment bases (one per 16-channel chunk kk) and four V^T bases (one
// per 16-key chunk c2); the 32-key block / 32-channel block go into the
// reads' immediate offsets and each block adds its buffers' offsets (the XOR
// patterns touch address bits 4-6 only, below the 1 KiB-aligned buffers).
struct Addr {
  uint32_t k[8], v[4];
};

constexpr int kKRing = 4, kVRing = 4;  // LDS ring depth (tiles), K and V^T
constexpr uint32_t kVRingOfs = kKRing * kTileB;
constexpr int kAhead = 3;  // fragments read ahead of their step (ring of 4)

// this block's addresses: the bases plus its K and V^T buffer offsets
__device__ __forceinline__ Addr block_addr(const Addr& ad, uint32_t kofs, uint32_t vofs) {
  Addr a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.k[i] = ad.k[i] + kofs;
#pragma unroll
  for (int i = 0; i < 4; ++i) a.v[i] = ad.v[i] + vofs;
  return a;
}

// Matrix block step k.  With P*V (kPV) the block alternates P*V and score
// products: even k = P*V of chunk k/8, channel block (k/2)%4; odd k (and
// every k of a scores-only block) = scores of 32-key block kb, chunk kk.
// Fragment k of the block is the operand read for step k.
template <bool kPV, int k>
struct MmStep {
  static constexpr bool pv = kPV && (k & 1) == 0;
  static constexpr int c2 = k >> 3, d = (k >> 1) & 3;            // P*V step
  static constexpr int ks = kPV ? (k >> 1) : k;                  // score step index
  static constexpr int kb = ks >> 3, kk = ks & 7;                // score step
};
template <bool kPV, int k>
__device__ __forceinline__ u32x4 read_frag(const Addr& ad) {
  using M = MmStep<kPV, k>;
  if constexpr (M::pv)
    return ds_b128<M::d * 32 * kVtRowB>(ad.v[M::c2]);
  else
    return ds_b128<M::kb * 32 * kRowB>(ad.k[M::kk]);
}

// Issue the first kAhead reads of a matrix block (ring slots 0..kAhead-1).
template <bool kPV, int f>
__device__ __forceinline__ void mm_prefetch(u32x4 (&fr)[4], const Addr& ad) {
  if constexpr (f < kAhead) {
    fr[f] = read_frag<kPV, f>(ad);
    mm_prefetch<kPV, f + 1>(fr, ad);
  }
}

// Matrix block: NF steps (32 with P*V and scores, 16 with one of them); the
// first kAhead fragments were issued before; each step issues the read
// kAhead ahead and waits for its own with an exact lgkmcnt.
template <bool kPV, bool kS, int k>
__device__ __forceinline__ void mm_step(St& st, u32x4 (&fr)[4], const Addr& ad) {
  constexpr int NF = (kPV ? 16 : 0) + (kS ? 16 : 0);
  if constexpr (k < NF) {
    constexpr int fn = k + kAhead;
    if constexpr (fn < NF) fr[fn & 3] = read_frag<kPV && kS, fn>(ad);
    constexpr int issued_after = NF - 1 - k;
    constexpr int later = issued_after < kAhead ? issued_after : kAhead;
    u32x4& v = fr[k & 3];
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "i"(later));
    using M = MmStep<kPV && kS, k>;
    constexpr bool pv = kS ? M::pv : true;  // a P*V-only block: every step is P*V
    if constexpr (pv) {
      constexpr int c2 = kS ? M::c2 : (k >> 2), d = kS ? M::d : (k & 3);
      st.acc[d] = mfma32h(__builtin_bit_cast(f16x8, fr[k & 3]), __builtin_bit_cast(f16x8, st.p[c2]), st.acc[d]);
    } else {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, fr[k & 3]);
      if constexpr (M::kk == 0)
        st.s[M::kb] = mfma32(kf, st.q[M::kk], f32x16{});
      else
        st.s[M::kb] = mfma32(kf, st.q[M::kk], st.s[M::kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    mm_step<kPV, kS, k + 1>(st, fr, ad);
  }
}
template <bool kPV, bool kS>
__device__ __forceinline__ void mm_block(St& st, u32x4 (&fr)[4], const Addr& ad) {
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  mm_step<kPV, kS, 0>(st, fr, ad);
  __builtin_amdgcn_s_setprio(0);
}
// Softmax block of one tile: mask, row max, lazy reference-max move (and
// rescale of acc, which holds P*V of the tiles before), p = exp2, row sum;
// then P rounded to FP16 (RNE) for the P*V products.
__device__ __forceinline__ void sm_block(St& st, int cur_valid, int hh) {
  f32x16 (&sx)[2] = st.s;
  if (cur_valid < kFwdBN) {
    // key of register r in block kb: 32*kb + 8*(r/4) + 4*hh + r%4
    const int lim = cur_valid - 4 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) sx[kb][r] = -INFINITY;
  }
  float mt = sx[0][0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sx[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sx[1][r]);
  {
    const uint32_t u = __float_as_uint(mt);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const bool move = mt > st.m_used + kTauRaw;
  const float m_new = move ? mt : st.m_used;
  if (__any(move)) {
    const float alpha = (m_new == st.m_used) ? 1.0f : __builtin_amdgcn_exp2f((st.m_used - m_new) * kC);
    st.l = st.l * alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[d][r] = st.acc[d][r] * alpha;
    st.m_used = m_new;
  }
  const float mc = st.m_used * kC;
  float ts = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sx[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[kb][r], kC, -mc));
      ts = ts + sx[kb][r];
    }
  st.l = st.l + ts;
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int kb = c2 >> 1, r = 8 * (c2 & 1) + 2 * w;
      st.p[c2][w] = pack_f16x2(sx[kb][r], sx[kb][r + 1]);
    }
}

}  // namespace

// The forward over all key tiles of each row (kWhole), or over the tiles of
// one key block: from an empty state with the row state (acc, reference
// max, row sum) written out instead of O (kBlock), or continuing the state a
// previous block left (kCarry), then writing that state (acc, reference max
// and the two half-wave row sums, so that the next block continues exactly)
// or, after the last block, O and LSE.  A block's tiles are processed exactly
// as the whole row's: same order, same arithmetic per tile, so blocks carried
// over the keys in ascending order give the whole-row bytes.
enum { kWhole = 0, kBlock = 1, kCarry = 2 };
template <int kMode>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a) {
  constexpr bool kPartial = kMode != kWhole;
  __shared__ __attribute__((aligned(1024))) char smem[(kKRing + kVRing) * kTileB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2;
  const int lr = lane & 31, hh = lane >> 5;

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

  St st;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qrow < a.S) z = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
    st.q[kk] = __builtin_bit_cast(bf16x8, z);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[d][r] = 0.f;
  st.m_used = -INFINITY;
  st.l = 0.f;
  if constexpr (kMode == kCarry) {
    if (a.cin_acc && qrow < a.S) {  // the state the previous block left
      const int64_t row = ((int64_t)b * a.H + h) * a.S + qrow;
      const float* prow = a.cin_acc + row * kHeadDim;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 x = *(const f32x4*)(prow + 32 * d + 8 * g4 + 4 * hh);
#pragma unroll
          for (int e = 0; e < 4; ++e) st.acc[d][4 * g4 + e] = x[e];
        }
      st.m_used = a.cin_m[row];
      st.l = a.cin_l[2 * row + hh];
    }
  }

  const int ntxt = (L + kFwdBN - 1) / kFwdBN;
  // Tiles processed, in key order: u < ntb are text tiles u; the others are
  // image tiles from t_img0 on (all of them unless kPartial).
  const int nimg = (a.T_img + kFwdBN - 1) / kFwdBN;
  const int ntb = kPartial ? (a.blk_text ? ntxt : 0) : ntxt;
  const int t_img0 = kPartial ? min(a.blk_img_t0, nimg) : 0;
  const int nt = kPartial ? ntb + max(0, min(a.blk_img_t1, nimg) - t_img0) : ntxt + nimg;
  auto tix = [&](int u) {
    if constexpr (kPartial)
      return u < ntb ? u : ntxt + t_img0 + (u - ntb);
    else
      return u;
  };
  if constexpr (kMode == kBlock) {
    if (nt == 0) {  // no key of this row in the block (uniform over the workgroup)
      if (qrow < a.S) {
        const int64_t row = ((int64_t)b * a.H + h) * a.S + qrow;
        float* prow = a.pacc + row * kHeadDim;
        for (int c = 4 * hh; c < kHeadDim; c += 8) *(f32x4*)(prow + c) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (hh == 0) {
          a.pm[row] = -INFINITY;
          a.pl[row] = 0.f;
        }
      }
      return;
    }
  }
  if (kMode != kCarry || nt > 0) {  // a carried block without keys of this row keeps the state
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  auto kbuf = [&](int j) { return smem + (j % kKRing) * kTileB; };
  auto vbuf = [&](int j) { return smem + kVRingOfs + (j % kVRing) * kTileB; };
  auto kofs = [&](int j) { return (uint32_t)((j % kKRing) * kTileB); };
  auto vofs = [&](int j) { return (uint32_t)((j % kVRing) * kTileB); };
  auto valid_of = [&](int j) {
    int k0, nv;
    tile_bounds(tix(j), ntxt, L, a.T_txt, a.T_img, k0, nv);
    return nv;
  };
  // Group 0 loads whole K tiles, group 1 whole V^T tiles: wave `sub` of a
  // group fills 16 K rows (four loads of 4 rows) or 32 V^T channel rows
  // (four loads of 8 rows).  K rows past the tile's valid count repeat its
  // last valid row (their scores are masked), so every load is issued.
  const int sub = wave & 3;
  const RowOff ko = row_offsets(a.k.ss, lane);
  auto load_k = [&](int j) {
    int k0, nv;
    tile_bounds(tix(j), ntxt, L, a.T_txt, a.T_img, k0, nv);
    const int r0 = 16 * sub;
    const uint32_t la = addr_of(kbuf(j) + r0 * kRowB);
    if (nv >= r0 + 16) {
      const char* base = (const char*)(a.k.p + (int64_t)b * a.k.sb + (int64_t)h * a.k.sh + (int64_t)(k0 + r0) * a.k.ss);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(base, ko.o[i], la + 4 * i * kRowB);
    } else {
      const int rbase = r0 < nv ? r0 : nv - 1;  // a valid source row
      const char* base =
          (const char*)(a.k.p + (int64_t)b * a.k.sb + (int64_t)h * a.k.sh + (int64_t)(k0 + rbase) * a.k.ss);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = 4 * i + (lane >> 4);            // LDS row within the wave's 16
        const int src = min(r0 + kl, nv - 1) - rbase;  // source row relative to the base, >= 0
        const int chunk = (lane & 15) ^ swz(kl);
        dma16(base, (uint32_t)(src * (uint32_t)a.k.ss + 8 * chunk) * 2u, la + 4 * i * kRowB);
      }
    }
  };
  const VtOff vo = vt_offsets(lane);
  const uint16_t* const vt_bh = a.vt + ((int64_t)b * a.H + h) * a.nt_max * kVtileElems;
  auto load_v = [&](int j) { load_vt(vt_bh + (int64_t)tix(j) * kVtileElems, vo, vbuf(j), sub); };

  Addr ad;
  {
    const uint32_t rbase = row_base(lds0, lane), vbase = vt_base(lds0 + kVRingOfs, lane);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ad.k[kk] = rbase ^ (uint32_t)(kk << 5);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) ad.v[c2] = vbase ^ (uint32_t)(c2 << 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(ad.k[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ad.v[i]));
  }

  // Tiles 0..2 of K and V up front.  Then K tile j is loaded by group 0
  // between B_{j-4} and B_{j-3} (at the start of its softmax block SM(j-3),
  // beside group 1's matrix block) and V tile j by group 1 between B_{j-3}
  // and B_{j-2} (at the start of its SM(j-3), beside group 0's matrix
  // block).  At every barrier a wave has its loads issued before the
  // barrier before landed, so a tile is visible to every wave one barrier
  // interval before it is read, and a buffer is refilled only after the
  // interval that last read it.
  for (int j = 0; j < 3 && j < nt; ++j) {
    if (grp == 0) load_k(j);
    else load_v(j);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  bar();

  u32x4 fr[4];
  // scores of tile 0, both groups
  {
    const Addr a0 = block_addr(ad, kofs(0), 0);
    mm_prefetch<false, 0>(fr, a0);
    mm_block<false, true>(st, fr, a0);
  }
  // B_t: this wave's loads issued before B_{t-1} have landed (the four
  // issued since may still be in flight), then the barrier.
  auto barrier_at = [&](int t, bool issued_since) {
    if (issued_since)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bar();
  };
  // Each wave runs SM(t), MM(t) for t = 0 .. nt-1; group 1 passes B_t
  // before SM(t), group 0 between SM(t) and MM(t).
  for (int t = 0; t < nt; ++t) {
    if (grp == 1) {
      barrier_at(t, t > 0 && t + 2 < nt);  // V tile t+2 was issued after B_{t-1}
      if (t + 3 < nt) load_v(t + 3);
    } else {
      if (t + 3 < nt) load_k(t + 3);
    }
    sm_block(st, valid_of(t), hh);
    // MM(t) reads V tile t and K tile t+1 (for t = nt-1 a stale K buffer:
    // those scores are never used); its first fragments now
    const Addr am = block_addr(ad, kofs(t + 1), vofs(t));
    mm_prefetch<true, 0>(fr, am);
    if (grp == 0) barrier_at(t, t + 3 < nt);  // K tile t+3, issued just now
    mm_block<true, true>(st, fr, am);
  }

  }

  // ---- epilogue
  const uint32_t lu = __float_as_uint(st.l);
  const auto sw = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if constexpr (kMode == kCarry) {
    if (a.pacc) {  // not the last block: the state, with each half-wave's row sum
      if (qrow < a.S) {
        const int64_t row = ((int64_t)b * a.H + h) * a.S + qrow;
        float* prow = a.pacc + row * kHeadDim;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *(f32x4*)(prow + 32 * d + 8 * g4 + 4 * hh) =
                f32x4{st.acc[d][4 * g4], st.acc[d][4 * g4 + 1], st.acc[d][4 * g4 + 2], st.acc[d][4 * g4 + 3]};
        if (hh == 0) a.pm[row] = st.m_used;
        a.pl[2 * row + hh] = st.l;
      }
      return;
    }
  }
  if constexpr (kMode == kBlock) {
    // the row state: acc (sum_j p_j v_j 2^-8, FP32), reference max, row sum
    if (qrow < a.S) {
      const int64_t row = ((int64_t)b * a.H + h) * a.S + qrow;
      float* prow = a.pacc + row * kHeadDim;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)(prow + 32 * d + 8 * g4 + 4 * hh) =
              f32x4{st.acc[d][4 * g4], st.acc[d][4 * g4 + 1], st.acc[d][4 * g4 + 2], st.acc[d][4 * g4 + 3]};
      if (hh == 0) {
        a.pm[row] = st.m_used;
        a.pl[row] = l_tot;
      }
    }
    return;
  }
  // O = acc / l, one RNE cast; LSE in natural log
  // acc holds sum_j p_j v_j 2^-8: divide by l * 2^-8 (exact scaling)
  const float l_div = l_tot * kVScale;
  if (qrow < a.S) {
    uint16_t* orow = a.o.row(b, qrow, h);
    float* frow = a.of ? a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim : nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        const float o0 = st.acc[d][4 * g4] / l_div, o1 = st.acc[d][4 * g4 + 1] / l_div;
        const float o2 = st.acc[d][4 * g4 + 2] / l_div, o3 = st.acc[d][4 * g4 + 3] / l_div;
        const u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)(orow + d0) = ov;
        if (frow) *(f32x4*)(frow + d0) = f32x4{o0, o1, o2, o3};
      }
    if (hh == 0) {
      const float lse2 = st.m_used * kC + log2f(l_tot);
      a.lse[((int64_t)b * a.H + h) * a.S + qrow] = lse2 * kLn2;
    }
  }
}


__global__ __launch_bounds__(kFwdWaves * 64, 1) void attn_fwd_kernel(FwdArgs a) { attn_fwd_body<kWhole>(a); }
__global__ __launch_bounds__(kFwdWaves * 64, 1) void attn_fwd_partial_kernel(FwdArgs a) { attn_fwd_body<kBlock>(a); }
__global__ __launch_bounds__(kFwdWaves * 64, 1) void attn_fwd_carry_kernel(FwdArgs a) { attn_fwd_body<kCarry>(a); }

// V -> FP16 V^T key tiles, one workgroup per (logical key tile t, h, b).
__global__ __launch_bounds__(256) void v_tiles_kernel(VtileArgs a) {
  v_tile_body(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

}  // namespace qi
