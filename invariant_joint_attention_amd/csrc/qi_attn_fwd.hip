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
//    on the same SIMD.  Group 0 (waves 0-3) and group 1 (waves 4-7) alternate
//    between a matrix phase (P*V of tile t plus the scores of tile t+1, 32
//    MFMAs) and a softmax phase (VALU only), one workgroup barrier per phase,
//    so each SIMD has one wave issuing MFMAs while its partner runs the
//    softmax.  Group 1 starts one barrier later; both run 2*nt + 1 barriers.
//  * LDS: K tiles in kbuf[j % 3], V^T tiles in vbuf[j % 3], 96 KiB.  K rows
//    are unpadded 256-byte lines whose 16-byte chunks are XOR-swizzled by key
//    (swizzle bits 2-3 from key bits 0-1, bits 0-1 from key bits 2-3); V^T
//    tiles are 128 channel lines of 128 bytes swizzled by channel/2.  The K
//    and V^T fragment reads (one ds_read_b128 each, 16 rows per 16-lane
//    group) and the contiguous direct-load writes meet no LDS bank conflict
//    on the 64 banks.  Tiles are filled by direct global->LDS loads
//    (global_load_lds_dwordx4) issued in the softmax phase of tile t: group
//    0 loads V_{t+1}, group 1 loads K_{t+2}; each waits for its loads
//    (vmcnt) at the end of its next matrix phase, a barrier before the tile
//    is read.  Three buffers are needed because group 0's softmax phase runs
//    while group 1 still reads the tiles of tile t-1.
//  * The softmax phase ends with P rounded to FP16, so one FP32 score buffer
//    suffices: the matrix phase accumulates the next tile's scores into it.
//  * The matrix phase issues its LDS reads as inline asm two steps ahead of
//    use and waits for each step's reads with an exact lgkmcnt; the direct
//    loads are inline asm too, so the compiler neither inserts waits for
//    them before unrelated LDS reads nor keeps 64-bit addresses for them.
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_lds.h"

#include <type_traits>

namespace qi {

namespace {

using namespace lds;
static_assert(kTileRows == kFwdBN, "forward key tile is one LDS tile");
// log2(e) / sqrt(128), rounded once to FP32
constexpr float kC = (float)(1.4426950408889634074 / 11.313708498984760390);
constexpr float kLn2 = 0.69314718055994530942f;
// V enters P*V as FP16 of v * 2^-8; the epilogue divides by l * 2^-8.
constexpr float kVScale = 0x1p-8f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two FP32 values -> packed FP16 pair (lo = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Threshold on raw scores for moving the reference max: 8 in the exp2 domain.
constexpr float kTauRaw = (float)(8.0 / (1.4426950408889634074 / 11.313708498984760390));

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

// Per-lane LDS addresses of the matrix phase, relative to K buffer 0 and V
// buffer 0: eight K row-fragment bases (one per 16-channel chunk kk) and
// four V^T fragment bases (one per 16-key chunk c2).  The 32-key block and
// the 32-channel block go into the reads' immediate offsets and each matrix
// phase adds its buffers' offsets; the XOR patterns touch address bits 5-7
// only, below the 1 KiB-aligned buffer starts, so base ^ pattern + offset is
// exact.
struct Addr {
  uint32_t k[8], v[4];
};
__device__ __forceinline__ Addr make_addr(uint32_t lds0, int lane) {
  Addr a;
  const uint32_t rb = row_base(lds0, lane), tb = vt_base(lds0 + 3 * kTileB, lane);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) a.k[kk] = rb ^ (uint32_t)(kk << 5);
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) a.v[c2] = tb ^ (uint32_t)(c2 << 5);
  // opaque: the compiler keeps the twelve addresses instead of
  // re-deriving them with VALU work inside the loop
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(a.k[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(a.v[i]));
  return a;
}

// K fragment of score step k (block kb = k/8, chunk kk = k%8).
template <int k>
__device__ __forceinline__ bf16x8 kfrag(const Addr& ad) {
  constexpr int kk = k & 7, kb = k >> 3;
  return __builtin_bit_cast(bf16x8, ds_b128<kb * 32 * kRowB>(ad.k[kk]));
}
// V^T fragment of P*V step k (16-key chunk c2 = k/4, 32-channel block d = k%4):
// channel rows 32*d .. 32*d+31, one 16-byte read per lane.
template <int k>
__device__ __forceinline__ f16x8 vfrag(const Addr& ad) {
  constexpr int c2 = k >> 2, d = k & 3;
  return __builtin_bit_cast(f16x8, ds_b128<d * 32 * kVtRowB>(ad.v[c2]));
}

struct State {
  f32x16 acc[4];
  f32x16 s[2];   // scores of one 64-key tile (two 32-key blocks), FP32
  u32x4 ph[4];   // FP16 P of the tile's four 16-key chunks
  bf16x8 q[8];
  float m_used, l_lane;
};

// S^T = K Q^T for one 64-key tile (16 MFMAs, no P*V work).
__device__ __forceinline__ void s_only(State& st, const char* kbuf, int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.s[kb][r] = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int kk = k >> 1, kb = k & 1;
    const bf16x8 kv = *(const bf16x8*)(kbuf + off(32 * kb + (lane & 31), 2 * kk + (lane >> 5)));
    st.s[kb] = mfma32(kv, st.q[kk], st.s[kb]);
  }
}

// Softmax of one tile: mask, row max, lazy reference-max move, p = exp2, row
// sum; then P rounded to FP16 (RNE) for the P*V products.
__device__ __forceinline__ void softmax_tile(State& st, int cur_valid, int hh) {
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
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const bool move = mt > st.m_used + kTauRaw;
  const float m_new = move ? mt : st.m_used;
  if (__any(move)) {
    const float alpha = (m_new == st.m_used) ? 1.0f : __builtin_amdgcn_exp2f((st.m_used - m_new) * kC);
    st.l_lane = st.l_lane * alpha;
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
  st.l_lane = st.l_lane + ts;
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int kb = c2 >> 1, r = 8 * (c2 & 1) + 2 * w;
      st.ph[c2][w] = pack_f16x2(sx[kb][r], sx[kb][r + 1]);
    }
}

// Matrix phase: O^T += V^T P^T per 16-key chunk and, when kS, S^T of the
// next tile interleaved (16 + 16 MFMAs).  Step k's fragments are read kPre
// steps ahead; sched barriers pin that order and each step waits only for
// its own reads.  The first score MFMA of each 32-key block starts from a
// zero accumulator.
constexpr int kPre = 2;

template <bool kS, int k>
__device__ __forceinline__ void mm_issue(f16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < 16) {
    vr[k % (kPre + 1)] = vfrag<k>(ad);
    if constexpr (kS) kr[k % (kPre + 1)] = kfrag<k>(ad);
  }
}

template <bool kS, int k>
__device__ __forceinline__ void mm_step(State& st, f16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < 16) {
    mm_issue<kS, k + kPre>(vr, kr, ad);
    // reads issued after step k's own: those of steps k+1 .. k+kPre
    constexpr int per = kS ? 2 : 1;
    constexpr int ahead = (15 - k) < kPre ? (15 - k) : kPre;
    constexpr int later = per * ahead;
    f16x8& vv = vr[k % (kPre + 1)];
    bf16x8& kv = kr[k % (kPre + 1)];
    if constexpr (kS)
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vv), "+v"(kv) : "i"(later));
    else
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vv) : "i"(later));
    constexpr int c2 = k >> 2, d = k & 3;
    st.acc[d] = mfma32h(vv, __builtin_bit_cast(f16x8, st.ph[c2]), st.acc[d]);
    if constexpr (kS) {
      constexpr int kb = k >> 3, kk = k & 7;
      if constexpr (kk == 0)
        st.s[kb] = mfma32(kv, st.q[kk], f32x16{});
      else
        st.s[kb] = mfma32(kv, st.q[kk], st.s[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    mm_step<kS, k + 1>(st, vr, kr, ad);
  }
}

template <bool kS, int k>
__device__ __forceinline__ void mm_prefetch(f16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < kPre) {
    mm_issue<kS, k>(vr, kr, ad);
    mm_prefetch<kS, k + 1>(vr, kr, ad);
  }
}

// Matrix phase of tile t: V_t in V buffer t % 3, K_{t+1} in K buffer
// (t + 1) % 3; kofs / vofs are those buffers' byte offsets (wave-uniform).
template <bool kS>
__device__ __forceinline__ void mm_tile(State& st, const Addr& ad, uint32_t kofs, uint32_t vofs) {
  Addr a2;
#pragma unroll
  for (int i = 0; i < 8; ++i) a2.k[i] = ad.k[i] + kofs;
#pragma unroll
  for (int i = 0; i < 4; ++i) a2.v[i] = ad.v[i] + vofs;
  f16x8 vr[kPre + 1];
  bf16x8 kr[kPre + 1];
  __builtin_amdgcn_sched_barrier(0);
  mm_prefetch<kS, 0>(vr, kr, a2);
  __builtin_amdgcn_sched_barrier(0);
  mm_step<kS, 0>(st, vr, kr, a2);
}

}  // namespace

__global__ __launch_bounds__(kFwdWaves * 64, 1) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[6 * kTileB];
  char* const kbase = smem;
  char* const vbase = smem + 3 * kTileB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2, sub = wave & 3;
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
  const bool qvalid = qrow < a.S;

  State st;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qvalid) z = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
    st.q[kk] = __builtin_bit_cast(bf16x8, z);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[d][r] = 0.f;
  st.m_used = -INFINITY;
  st.l_lane = 0.f;

  const int ntxt = (L + kFwdBN - 1) / kFwdBN;
  const int nt = ntxt + (a.T_img + kFwdBN - 1) / kFwdBN;
  auto kbuf = [&](int j) { return kbase + (j % 3) * kTileB; };
  auto vbuf = [&](int j) { return vbase + (j % 3) * kTileB; };
  auto valid_of = [&](int j) {
    int k0, nv;
    tile_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    return nv;
  };
  const RowOff ko = row_offsets(a.k.ss, lane);
  const VtOff vo = vt_offsets(lane);
  const uint16_t* const vt_bh = a.vt + ((int64_t)b * a.H + h) * a.nt_max * kVtileElems;
  auto load_k = [&](int j) {
    int k0, nv;
    tile_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.k, ko, kbuf(j), b, h, k0, nv, sub, lane);
  };
  auto load_v = [&](int j) { load_vt(vt_bh + (int64_t)j * kVtileElems, vo, vbuf(j), sub); };

  // prologue: K_0, V_0 (group 0) and K_1 (group 1)
  if (grp == 0) {
    load_k(0);
    load_v(0);
  } else if (nt > 1) {
    load_k(1);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  bar();

  const Addr ad = make_addr((uint32_t)(uintptr_t)(lds_char*)smem, lane);
  // one tile with a successor: group 0 loads V_{t+1}, group 1 K_{t+2};
  // softmax; matrix phase; each group waits for its own loads
  auto tile = [&](int t) {
    if (grp == 1) {
      if (t + 2 < nt) load_k(t + 2);
    } else {
      load_v(t + 1);
    }
    softmax_tile(st, valid_of(t), hh);
    bar();
    __builtin_amdgcn_s_setprio(1);
    mm_tile<true>(st, ad, ((t + 1) % 3) * kTileB, (t % 3) * kTileB);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0070);  // this group's loads have landed
    bar();
  };

  // Both groups run the same sequence; group 1 starts one barrier later, so
  // the two groups alternate phases.  Each group runs 2*nt + 1 barriers.
  if (grp == 1) bar();
  __builtin_amdgcn_s_setprio(1);
  s_only(st, kbuf(0), lane);
  __builtin_amdgcn_s_setprio(0);
  bar();
  for (int t = 0; t + 1 < nt; ++t) tile(t);
  softmax_tile(st, valid_of(nt - 1), hh);
  bar();
  __builtin_amdgcn_s_setprio(1);
  mm_tile<false>(st, ad, 0, ((nt - 1) % 3) * kTileB);
  __builtin_amdgcn_s_setprio(0);
  if (grp == 0) bar();

  // ---- epilogue: O = acc / l, one RNE cast; LSE in natural log
  const float l_tot = st.l_lane + __shfl_xor(st.l_lane, 32);
  // acc holds sum_j p_j v_j 2^-8: divide by l * 2^-8 (exact scaling)
  const float l_div = l_tot * kVScale;
  if (qvalid) {
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


// V -> FP16 V^T key tiles.  One workgroup per (logical key tile t, h, b):
// the tile's valid key rows are staged in LDS as BF16, then written out as
// 128 channel rows of 64 FP16 values v * 2^-8 (the multiply is exact, the
// conversion rounds to nearest even), the keys of each 16-key chunk in the
// A.V reduction order (position p holds key p with bits 2 and 3 swapped).
// Keys past the tile's valid count are written as zero, so the attention
// kernel loads whole tiles and a masked key's V slot is exactly zero.
__global__ __launch_bounds__(256) void v_tiles_kernel(VtileArgs a) {
  __shared__ uint32_t tl[kFwdBN][kHeadDim / 2 + 1];  // [key][channel pair]; one pad word per row
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = a.txt_len[b];
  const int ntxt = (L + kFwdBN - 1) / kFwdBN;
  const int nt = ntxt + (a.T_img + kFwdBN - 1) / kFwdBN;
  if (t >= nt) return;
  int key0, nvalid;
  tile_bounds(t, ntxt, L, a.T_txt, a.T_img, key0, nvalid);
  for (int i = threadIdx.x; i < kFwdBN * 16; i += 256) {
    const int key = i >> 4, c = i & 15;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < nvalid) w = *(const u32x4*)(a.v.row(b, key0 + key, h) + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) tl[key][4 * c + e] = w[e];
  }
  __syncthreads();
  uint16_t* const out = a.out + (((int64_t)b * a.H + h) * a.nt_max + t) * kVtileElems;
  for (int i = threadIdx.x; i < kHeadDim * 8; i += 256) {
    const int d = i >> 3, j = i & 7;  // channel row, 8-key chunk of the row
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = 8 * (j & 1) + e;  // position within 16-key chunk j/2
      const int key = 16 * (j >> 1) + ((p & 3) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3));
      const uint32_t w = tl[key][d >> 1];
      f[e] = ((d & 1) ? bf16_hi(w) : bf16_lo(w)) * kVScale;
    }
    const u32x4 o = {pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7])};
    *(u32x4*)(out + d * kFwdBN + 8 * j) = o;
  }
}

}  // namespace qi
