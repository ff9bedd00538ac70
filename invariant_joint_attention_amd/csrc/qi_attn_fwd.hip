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
//  * O^T = V^T P^T accumulates in 4 blocks of 32x32 FP32.  P enters the MFMA
//    as two BF16 terms, hi = bf16(p) and lo = bf16(p - hi), accumulated hi
//    then lo for each 16-key chunk in key order: one BF16 rounding of P
//    alone would move O by up to 2^-9 * sum_j p_j|v_j|, which breaks the
//    output tolerance where O cancels on few, peaked keys.  The MFMA
//    reduction index is a permutation of the 16 keys of a chunk (bits 2 and
//    3 of the key index swapped) that matches the accumulator layout of P;
//    the transposing V reads fetch the keys in that order.
//  * Keys are tiled LOGICALLY: ceil(L_b/64) text tiles starting at key 0,
//    then ceil(T_img/64) image tiles starting at key T_txt.  Masked keys are
//    never read (their LDS slots are zero) and get probability exactly 0, so
//    a row's arithmetic does not depend on T_txt, on the batch or on the
//    workgroup shape.  The key tile width 64 is frozen.
//  * Online softmax in the exp2 domain with c = log2(e)/sqrt(128):
//    p = exp2(s*c - m*c) (one fma); the row sum l adds the FP32 p lane by lane
//    in register order, then the two half-waves (commutative, so both get the
//    same bits); O = acc / l and LSE = (m*c + log2 l) * ln 2.
//    The reference max m moves only when a tile max exceeds it by more than
//    8/c (so p <= 256): each lane decides from its own row alone, and the
//    rescale (factor exactly 1 where m did not move) is skipped when no lane
//    of the wave moved.
//
// Schedule (free; does not change any bit):
//  * Workgroup = 8 waves x 32 query rows of one (b, h).  Waves w and w+4 run
//    on the same SIMD.  Group 0 (waves 0-3) and group 1 (waves 4-7) alternate
//    between a matrix phase (P*V of tile t plus the scores of tile t+1, 48
//    MFMAs) and a softmax phase (VALU only), one workgroup barrier per phase,
//    so each SIMD has one wave issuing MFMAs while its partner runs the
//    softmax.  Group 1 starts one barrier later; both run 2*nt + 1 barriers.
//  * LDS: K tiles in kbuf[j % 3], V tiles in vbuf[j % 3], 96 KiB.  Rows are
//    unpadded 256-byte lines whose 16-byte chunks are XOR-swizzled by key
//    (swizzle bits 2-3 from key bits 0-1, bits 0-1 from key bits 2-3), so
//    the K fragment reads (16 keys per 16-lane group), the transposing V
//    reads (ds_read_b64_tr_b16, 4 keys x 4 chunks per 32-lane group, V
//    stays row-major) and the contiguous direct-load writes meet no LDS bank
//    conflict on the 64 banks.  Tiles are filled by direct global->LDS loads
//    (global_load_lds_dwordx4) issued in the softmax phase of tile t: group
//    0 loads V_{t+1}, group 1 loads K_{t+2}; each waits for its loads
//    (vmcnt) at the end of its next matrix phase, a barrier before the tile
//    is read.  Three buffers are needed because group 0's softmax phase runs
//    while group 1 still reads the tiles of tile t-1.
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

// Per-lane LDS bases of the matrix phase: K row fragments (scores) and V
// transposed fragments (P*V).
struct Addr {
  uint32_t ak, av;
};
__device__ __forceinline__ Addr make_addr(uint32_t lds0, int lane) {
  Addr a;
  a.ak = row_base(lds0, lane);
  a.av = tr_base(lds0 + 3 * kTileB, lane);
  return a;
}

// K fragment of score step k (block kb = k/8, kk = k%8): block 0 is finished
// in the first half of the matrix phase and block 1 is started in the
// second, when the first two P chunks are no longer live.
template <int k>
__device__ __forceinline__ bf16x8 kfrag(const Addr& ad) {
  constexpr int kk = k & 7, kb = k >> 3;
  return lds::row_frag<kk, kb>(ad.ak);
}
// V^T fragment of P*V step k (c2 = k/4, d = k%4).
template <int k>
__device__ __forceinline__ bf16x8 vfrag(const Addr& ad) {
  constexpr int c2 = k >> 2, d = k & 3;
  return lds::tr_frag<c2, d>(ad.av);
}

struct State {
  f32x16 acc[4];
  f32x16 s[2][2];      // two score / P buffers (tile parity), two 32-key blocks each
  u32x4 ph[2], pl[2];  // hi/lo BF16 P of two 16-key chunks (chunk parity)
  bf16x8 q[8];
  float m_used, l_lane;
};

// S^T = K Q^T for one 64-key tile (16 MFMAs, no P*V work).
__device__ __forceinline__ void s_only(State& st, const char* kbuf, int lane) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.s[0][kb][r] = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int kk = k >> 1, kb = k & 1;
    const bf16x8 kv = *(const bf16x8*)(kbuf + off(32 * kb + (lane & 31), 2 * kk + (lane >> 5)));
    st.s[0][kb] = mfma32(kv, st.q[kk], st.s[0][kb]);
  }
}

// hi/lo BF16 split of 16-key chunk c2 of the P in buffer X, into slot c2 % 2.
template <int X, int c2>
__device__ __forceinline__ void pack_chunk(State& st) {
  constexpr int kb = c2 >> 1, r0 = 8 * (c2 & 1);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float p0 = st.s[X][kb][r0 + 2 * w], p1 = st.s[X][kb][r0 + 2 * w + 1];
    const uint32_t u = pack_bf16x2(p0, p1);
    st.ph[c2 & 1][w] = u;
    st.pl[c2 & 1][w] = pack_bf16x2(p0 - bf16_lo(u), p1 - bf16_hi(u));
  }
}

// Softmax of one tile (scores in buffer X, replaced by P in place): mask, row
// max, lazy reference-max move, p = exp2, row sum; then the hi/lo split of
// the first 16-key chunk (the matrix phase splits the others one chunk ahead).
template <int X>
__device__ __forceinline__ void softmax_tile(State& st, int cur_valid, int hh) {
  f32x16 (&sx)[2] = st.s[X];
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
  pack_chunk<X, 0>(st);
}

// Matrix phase: O^T += V^T P_hi^T then V^T P_lo^T per 16-key chunk, and,
// when kS, S^T of the next tile interleaved (one score MFMA between the hi
// and lo products).  Step k's fragments are read kPre steps ahead; sched
// barriers pin that order and each step waits only for its own reads.
constexpr int kPre = 2;

template <bool kS, int k>
__device__ __forceinline__ void mm_issue(bf16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < 16) {
    vr[k % (kPre + 1)] = vfrag<k>(ad);
    if constexpr (kS) kr[k % (kPre + 1)] = kfrag<k>(ad);
  }
}

template <bool kS, int X, int k>
__device__ __forceinline__ void mm_step(State& st, bf16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < 16) {
    mm_issue<kS, k + kPre>(vr, kr, ad);
    // reads issued after step k's own: those of steps k+1 .. k+kPre
    constexpr int per = kS ? 3 : 2;
    constexpr int ahead = (15 - k) < kPre ? (15 - k) : kPre;
    constexpr int later = per * ahead;
    bf16x8& vv = vr[k % (kPre + 1)];
    bf16x8& kv = kr[k % (kPre + 1)];
    if constexpr (kS)
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vv), "+v"(kv) : "i"(later));
    else
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(vv) : "i"(later));
    constexpr int c2 = k >> 2, d = k & 3;
    st.acc[d] = mfma32(vv, __builtin_bit_cast(bf16x8, st.ph[c2 & 1]), st.acc[d]);
    if constexpr (kS) st.s[1 - X][k >> 3] = mfma32(kv, st.q[k & 7], st.s[1 - X][k >> 3]);
    st.acc[d] = mfma32(vv, __builtin_bit_cast(bf16x8, st.pl[c2 & 1]), st.acc[d]);
    // split the next chunk while this chunk's products run
    if constexpr ((k & 3) == 1 && c2 < 3) pack_chunk<X, c2 + 1>(st);
    __builtin_amdgcn_sched_barrier(0);
    mm_step<kS, X, k + 1>(st, vr, kr, ad);
  }
}

template <bool kS, int k>
__device__ __forceinline__ void mm_prefetch(bf16x8 (&vr)[kPre + 1], bf16x8 (&kr)[kPre + 1], const Addr& ad) {
  if constexpr (k < kPre) {
    mm_issue<kS, k>(vr, kr, ad);
    mm_prefetch<kS, k + 1>(vr, kr, ad);
  }
}

template <bool kS, int X>
__device__ __forceinline__ void mm_tile(State& st, const Addr& ad) {
  if (kS) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.s[1 - X][kb][r] = 0.f;
  }
  bf16x8 vr[kPre + 1], kr[kPre + 1];
  // opaque copies: keeps the per-step address XORs inside their steps
  Addr a2 = ad;
  asm volatile("" : "+v"(a2.ak), "+v"(a2.av));
  __builtin_amdgcn_sched_barrier(0);
  mm_prefetch<kS, 0>(vr, kr, a2);
  __builtin_amdgcn_sched_barrier(0);
  mm_step<kS, X, 0>(st, vr, kr, a2);
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
  const RowOff ko = row_offsets(a.k.ss, lane), vo = row_offsets(a.v.ss, lane);
  auto load_k = [&](int j) {
    int k0, nv;
    tile_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.k, ko, kbuf(j), b, h, k0, nv, sub, lane);
  };
  auto load_v = [&](int j) {
    int k0, nv;
    tile_bounds(j, ntxt, L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.v, vo, vbuf(j), b, h, k0, nv, sub, lane);
  };

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
  // matrix phase of tile t: V_t in vbuf[t % 3], K_{t+1} in kbuf[(t + 1) % 3];
  // P of tile t in score buffer t & 1, scores of tile t+1 into the other
  auto mm = [&](int t, auto par, auto ks) {
    constexpr int X = decltype(par)::value;
    constexpr bool S = decltype(ks)::value;
    Addr a2;
    a2.av = ad.av + (t % 3) * kTileB;
    a2.ak = ad.ak + ((t + 1) % 3) * kTileB;
    __builtin_amdgcn_s_setprio(1);
    mm_tile<S, X>(st, a2);
    __builtin_amdgcn_s_setprio(0);
  };
  using Yes = std::true_type;
  using No = std::false_type;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // one tile with a successor: group 0 loads V_{t+1}, group 1 K_{t+2};
  // softmax; matrix phase; each group waits for its own loads
  auto tile = [&](int t, auto par) {
    constexpr int X = decltype(par)::value;
    if (grp == 1) {
      if (t + 2 < nt) load_k(t + 2);
    } else {
      load_v(t + 1);
    }
    softmax_tile<X>(st, valid_of(t), hh);
    bar();
    mm(t, par, Yes{});
    __builtin_amdgcn_s_waitcnt(0x0070);  // this group's loads have landed
    bar();
  };
  auto last = [&](int t, auto par) {
    constexpr int X = decltype(par)::value;
    softmax_tile<X>(st, valid_of(t), hh);
    bar();
    mm(t, par, No{});
    if (grp == 0) bar();
  };

  // Both groups run the same sequence; group 1 starts one barrier later, so
  // the two groups alternate phases.  Each group runs 2*nt + 1 barriers.
  if (grp == 1) bar();
  __builtin_amdgcn_s_setprio(1);
  s_only(st, kbuf(0), lane);
  __builtin_amdgcn_s_setprio(0);
  bar();
  int t = 0;
  for (; t + 2 < nt; t += 2) {
    tile(t, B0{});
    tile(t + 1, B1{});
  }
  if (t + 1 < nt) {
    tile(t, B0{});
    last(t + 1, B1{});
  } else {
    last(t, B0{});
  }

  // ---- epilogue: O = acc / l, one RNE cast; LSE in natural log
  const float l_tot = st.l_lane + __shfl_xor(st.l_lane, 32);
  if (qvalid) {
    uint16_t* orow = a.o.row(b, qrow, h);
    float* frow = a.of ? a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim : nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        const float o0 = st.acc[d][4 * g4] / l_tot, o1 = st.acc[d][4 * g4 + 1] / l_tot;
        const float o2 = st.acc[d][4 * g4 + 2] / l_tot, o3 = st.acc[d][4 * g4 + 3] / l_tot;
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

}  // namespace qi
