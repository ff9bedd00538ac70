// qi_attn_unfused.hip -- the unfused attention forward on gfx950: the score
// GEMM, the masked softmax with fixed tiling, and the A.V GEMM as three
// separate operators with their intermediates in HBM.
//
// Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rows
// joint_attn_qk_gemm (Q K^T / sqrt(d) over the joint sequence),
// joint_attn_softmax (online softmax over the key sequence with a fixed
// tiling and reduction order), joint_attn_av_gemm (A.V), and
// joint_attention_fused, whose output must equal the composition of these
// three byte for byte; [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2
// kernel roadmap, ablation matrix and integration plan", "Numerical
// requirements" (fused kernels reproduce the unfused result byte for byte).
//
// Each operator performs, per query row, exactly the arithmetic that the
// fused kernel performs for that row, in the same order, with the same
// instructions and operand layouts:
//  * attn_qk_kernel: raw scores q'.k' of each 64-key logical tile, two
//    32-key blocks of v_mfma_f32_32x32x16_bf16 (S^T = K Q^T), the 8 head-dim
//    chunks of a block accumulated in order from zero.  The 1/sqrt(128)
//    scale is not applied here: it enters the softmax's exponent as the FP32
//    constant c = log2(e)/sqrt(128) (p = exp2(s*c - m*c), one fma), which is
//    how the fused kernel applies it.  Masked slots hold -inf.
//  * attn_softmax_kernel: per tile, the exact tile max (both half-rows), the
//    lazy reference max m (moved only when the tile max exceeds it by more
//    than 8/c), alpha = exp2((m_old - m_new) c) (1 where m did not move),
//    p = exp2(s c - m c), and the row sum kept as two half sums (keys
//    8g + 4hh + {0..3} of half hh, in register order) updated as
//    l_hh = l_hh * alpha + sum, then l = l_0 + l_1.  P is stored as FP16
//    (RNE), alpha per (row, tile), and LSE = (m c + log2 l) ln 2.
//  * attn_av_kernel: acc = alpha_t * acc + P_t V_t per tile with
//    v_mfma_f32_32x32x16_f16 on FP16 P and FP16 v * 2^-8 (the transposed key
//    tiles that v_tiles_kernel writes), 16-key chunks in key order; then
//    O = acc / (l 2^-8), one BF16 rounding.
// A factor of exactly 1 leaves a value unchanged, so multiplying every tile
// by alpha gives the bits of the fused kernel, which skips the rescale
// where no row of a wave moved its reference max.
//
// Launch shapes (free; no bit depends on them):
//  * scores: 8 waves x 32 query rows; K tiles are staged in LDS (direct
//    global->LDS loads, double buffered, the fused kernel's swizzled rows) and
//    shared by the workgroup; a wave's scores go to HBM as 16-byte stores.
//  * softmax: 4 waves x 32 rows; each wave stages its rows' score tile in LDS
//    (direct loads of whole 256-byte row pieces, double buffered), reads its
//    lanes' values back in the register order of the fused kernel, and writes
//    P through LDS as whole 128-byte row pieces.
//  * A.V: 8 waves x 32 rows; V^T tiles staged in LDS and shared (double
//    buffered); each wave stages its rows' P tile in LDS the same way.
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_attn_contract.h"
#include "qi_lds.h"

namespace qi {

using namespace attn;
using namespace lds;

namespace {

struct RowTiles {
  int L, ntxt, nt;
};
__device__ __forceinline__ RowTiles row_tiles(const int* txt_len, int b, int T_img) {
  RowTiles r;
  r.L = txt_len[b];
  r.ntxt = (r.L + kFwdBN - 1) / kFwdBN;
  r.nt = r.ntxt + (T_img + kFwdBN - 1) / kFwdBN;
  return r;
}

// Wait for this wave's LDS reads issued as inline asm, then pin the values
// behind the wait so that no use is scheduled above it.
template <int N>
__device__ __forceinline__ void lds_wait_pin(u32x4 (&f)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

// One direct global -> LDS load of 4 bytes per lane (lane l's bytes land at
// LDS byte lds + 4*l), with the conventions of dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const char* base, uint32_t off32, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(off32), "s"(base)
               : "memory", "m0");
}
// dma16 with the non-temporal hint: for the score and P streams, each byte
// of which is read once.
__device__ __forceinline__ void dma16_nt(const char* base, uint32_t off32, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds_addr), "v"(off32), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace

// Score staging per wave: 32 rows x 256 bytes, chunk c of row r at chunk
// c ^ (r & 15), so each store writes whole 256-byte row pieces.
constexpr int kQkStageB = 32 * 256;

__global__ __launch_bounds__(kQkWaves * 64) void attn_qk_kernel(QkArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileB + kQkWaves * kQkStageB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int qrow = blockIdx.x * (kQkWaves * 32) + wave * 32 + lr;
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;

  bf16x8 q[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qrow < a.S) z = *(const u32x4*)(a.q.row(b, qrow, h) + 16 * kk + 8 * hh);
    q[kk] = __builtin_bit_cast(bf16x8, z);
  }
  const int row0 = blockIdx.x * (kQkWaves * 32) + wave * 32;  // the wave's first row
  float* const srow0 = a.s + (((int64_t)b * a.H + h) * a.S + row0) * Kp;
  char* const stage = smem + 2 * kTileB + wave * kQkStageB;

  // Waves 0-3 fill the K tiles, 16 rows each; rows past a tile's valid count
  // are zero in LDS (their scores are masked).
  const RowOff ro = row_offsets(a.k.ss, lane);
  auto load = [&](int t) {
    int k0, nv;
    tile_bounds(t, rt.ntxt, rt.L, a.T_txt, a.T_img, k0, nv);
    load_rows(a.k, ro, smem + (t & 1) * kTileB, b, h, k0, nv, wave, lane);
  };
  const uint32_t rb0 = row_base(addr_of(smem), lane);
  if (wave < 4) load(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  bar();
  if (wave < 4 && rt.nt > 1) load(1);

  for (int t = 0; t < a.nt_max; ++t) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
    int nv = 0;
    if (t < rt.nt) {  // uniform over the workgroup
      int key0;
      tile_bounds(t, rt.ntxt, rt.L, a.T_txt, a.T_img, key0, nv);
      const uint32_t rb = rb0 + (uint32_t)((t & 1) * kTileB);
      u32x4 f[16];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        f[kk] = ds_b128<0>(rb ^ (uint32_t)(kk << 5));
        f[8 + kk] = ds_b128<32 * kRowB>(rb ^ (uint32_t)(kk << 5));
      }
      lds_wait_pin(f);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, f[8 * kb + kk]);
          if (kk == 0)
            s[kb] = mfma32(kf, q[0], f32x16{});
          else
            s[kb] = mfma32(kf, q[kk], s[kb]);
        }
      if (t + 1 < rt.nt) {
        // tile t+1 landed (loads and zero fills of waves 0-3); every wave is
        // done with buffer t&1, which then takes tile t+2
        if (wave < 4) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        bar();
        if (wave < 4 && t + 2 < rt.nt) load(t + 2);
      }
    }
    // this lane's keys 32kb + 8g + 4hh .. +3 of row lr are chunk 8kb + 2g + hh
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = score_key(kb, 4 * g + e, hh) < nv ? s[kb][4 * g + e] : -INFINITY;
        *(f32x4*)(stage + lr * 256 + 16 * ((8 * kb + 2 * g + hh) ^ (lr & 15))) = v;
      }
    // store i, lane l: row 4i + l/16, chunk l%16 (the rows' 256 bytes of tile t)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), c = lane & 15;
      const f32x4 v = *(const f32x4*)(stage + r * 256 + 16 * (c ^ (r & 15)));
      if (row0 + r < a.S) __builtin_nontemporal_store(v, (f32x4*)(srow0 + (int64_t)r * Kp + kFwdBN * t + 4 * c));
    }
  }
}

// Softmax LDS per wave: two score tiles of 32 rows x 256 bytes (chunk c of
// row r at chunk c ^ swz(r)) and one P tile of 32 rows x 128 bytes (chunk c
// of row r at chunk c ^ (r & 7)).
constexpr int kSmScoreB = 32 * 256, kSmPB = 32 * 128;
constexpr int kSmWaveB = 2 * kSmScoreB + kSmPB;

__global__ __launch_bounds__(kSoftmaxWaves * 64) void attn_softmax_kernel(SoftmaxArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kSoftmaxWaves * kSmWaveB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int row0 = blockIdx.x * (kSoftmaxWaves * 32) + wave * 32;  // the wave's first row
  const int qrow = row0 + lr;
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;
  const int64_t bh = (int64_t)b * a.H + h;
  const bool store = qrow < a.S;
  char* const wbuf = smem + wave * kSmWaveB;
  char* const pbuf = wbuf + 2 * kSmScoreB;

  // Rows past S read the last row (their results are not stored).
  const int base_row = min(row0, a.S - 1);
  const char* const sbase = (const char*)(a.s + (bh * a.S + base_row) * Kp);
  uint32_t soff[8];  // load i, lane l: row 4i + l/16, logical chunk (l%16) ^ swz(row)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int rr = min(row0 + r, a.S - 1) - base_row;
    soff[i] = (uint32_t)rr * (uint32_t)(Kp * 4) + 16u * (uint32_t)((lane & 15) ^ swz(r));
  }
  auto load_scores = [&](int t) {
    const char* src = sbase + (int64_t)t * kFwdBN * 4;
    const uint32_t dst = addr_of(wbuf + (t & 1) * kSmScoreB);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16_nt(src, soff[i], dst + 1024u * i);
  };
  // this lane's logical chunk 8kb + 2g + hh of row lr sits at chunk (8kb + 2g) ^ (hh ^ swz(lr))
  const uint32_t frag0 = addr_of(wbuf) + (uint32_t)(lr * 256 + 16 * (hh ^ swz(lr)));
  uint16_t* const prow0 = a.p + (bh * a.S + row0) * Kp;
  float* const acol = a.alpha + bh * a.nt_max * a.S + qrow;  // alpha of tile t at acol[t * S]

  float m_used = -INFINITY, l = 0.f;
  load_scores(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int t = 0; t < rt.nt; ++t) {
    if (t + 1 < rt.nt) load_scores(t + 1);
    u32x4 f[8];
    const uint32_t fb = frag0 + (uint32_t)((t & 1) * kSmScoreB);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = ds_b128<0>(fb ^ (uint32_t)(16 * (8 * (j >> 2) + 2 * (j & 3))));
    lds_wait_pin(f);
    f32x16 sx[2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sx[j >> 2][4 * (j & 3) + e] = __uint_as_float(f[j][e]);
    // exact tile max over the row's 64 slots: this half-row, then the other
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
    const bool move = mt > m_used + kTauRaw;
    const float m_new = move ? mt : m_used;
    const float alpha = (m_new == m_used) ? 1.0f : __builtin_amdgcn_exp2f((m_used - m_new) * kC);
    l = l * alpha;
    m_used = m_new;
    const float mc = m_used * kC;
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sx[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[kb][r], kC, -mc));
        ts = ts + sx[kb][r];
      }
    l = l + ts;
    // P (FP16) through LDS: keys 32kb + 8g + 4hh .. +3 are the 8-byte half hh
    // of chunk 4kb + g of the 128-byte row piece
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 pv = {pack_f16x2(sx[kb][4 * g], sx[kb][4 * g + 1]),
                          pack_f16x2(sx[kb][4 * g + 2], sx[kb][4 * g + 3])};
        *(u32x2*)(pbuf + lr * 128 + 16 * ((4 * kb + g) ^ (lr & 7)) + 8 * hh) = pv;
      }
    u32x4 po[4];  // store i, lane l: row 8i + l/8, physical chunk l%8
#pragma unroll
    for (int i = 0; i < 4; ++i) po[i] = *(const u32x4*)(pbuf + (8 * i + (lane >> 3)) * 128 + 16 * (lane & 7));
    // scores of tile t+1 landed; the stores of tile t-1 are done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      if (row0 + r < a.S) {
        const int c = (lane & 7) ^ (r & 7);
        __builtin_nontemporal_store(po[i], (u32x4*)(prow0 + (int64_t)r * Kp + kFwdBN * t + 8 * c));
      }
    }
    if (store && hh == 0) acol[(int64_t)t * a.S] = alpha;
  }
  // tiles past this row's count: P = 0, alpha = 1
  for (int t = rt.nt; t < a.nt_max; ++t) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      if (row0 + r < a.S) *(u32x4*)(prow0 + (int64_t)r * Kp + kFwdBN * t + 8 * (lane & 7)) = z;
    }
    if (store && hh == 0) acol[(int64_t)t * a.S] = 1.0f;
  }
  const uint32_t lu = __float_as_uint(l);
  const auto sw = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (store && hh == 0) {
    const int64_t row = bh * a.S + qrow;
    a.l[row] = l_tot;
    a.lse[row] = (m_used * kC + log2f(l_tot)) * kLn2;
  }
}

// A.V LDS: two V^T tiles (shared); per wave one P tile (32 rows x 128 bytes,
// chunk c of row r at chunk c ^ (r & 7)) and the tile's alpha of each lane's
// row (one word per lane).  Values that come from memory reach registers only
// through LDS reads issued and waited for within one tile step, so no
// register is written by a load still in flight across the loop.
constexpr int kAvPB = 32 * 128, kAvAB = 64 * 4;

__global__ __launch_bounds__(kAvWaves * 64) void attn_av_kernel(AvArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileB + kAvWaves * (kAvPB + kAvAB)];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int row0 = blockIdx.x * (kAvWaves * 32) + wave * 32;
  const int qrow = row0 + lr;
  const RowTiles rt = row_tiles(a.txt_len, b, a.T_img);
  const int64_t Kp = (int64_t)a.nt_max * kFwdBN;
  const int64_t bh = (int64_t)b * a.H + h;
  char* const pbuf = smem + 2 * kTileB + wave * kAvPB;
  char* const abuf = smem + 2 * kTileB + kAvWaves * kAvPB + wave * kAvAB;

  const int base_row = min(row0, a.S - 1);
  const char* const pbase = (const char*)(a.p + (bh * a.S + base_row) * Kp);
  uint32_t poff[4];  // load i, lane l: row 8i + l/8, logical chunk (l%8) ^ (row & 7)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int rr = min(row0 + r, a.S - 1) - base_row;
    poff[i] = (uint32_t)rr * (uint32_t)(Kp * 2) + 16u * (uint32_t)((lane & 7) ^ (r & 7));
  }
  // alpha of this lane's row in tile t: scalar base at the wave's first row of tile t
  const char* const abase = (const char*)(a.alpha + bh * a.nt_max * a.S + base_row);
  const uint32_t aoff = (uint32_t)(min(qrow, a.S - 1) - base_row) * 4u;
  auto load_p = [&](int t) {
    const char* src = pbase + (int64_t)t * kFwdBN * 2;
    const uint32_t dst = addr_of(pbuf);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_nt(src, poff[i], dst + 1024u * i);
    dma4(abase + (int64_t)t * a.S * 4, aoff, addr_of(abuf));
  };
  const uint16_t* const vt_bh = a.vt + bh * a.nt_max * kVtileElems;
  const VtOff vo = vt_offsets(lane);
  auto load_v = [&](int t) { load_vt(vt_bh + (int64_t)t * kVtileElems, vo, smem + (t & 1) * kTileB, wave - 4); };
  const uint32_t vb0 = vt_base(addr_of(smem), lane);
  // this lane's P operand: keys 16c2 + 4hh .. +3 (chunk 2c2, half hh) and
  // 16c2 + 8 + 4hh .. +3 (chunk 2c2 + 1, half hh) of row lr
  const uint32_t pr = addr_of(pbuf) + (uint32_t)(lr * 128 + 8 * hh);

  f32x16 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;

  if (wave >= 4) load_v(0);
  load_p(0);
  for (int t = 0; t < rt.nt; ++t) {
    // V^T tile t (waves 4-7), this wave's P tile t and alpha of tile t
    // landed; every wave is done with V^T buffer (t+1)&1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bar();
    if (wave >= 4 && t + 1 < rt.nt) load_v(t + 1);
    u32x2v pw[8];
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t ad = pr + (uint32_t)(16 * ((2 * c2 + j) ^ (lr & 7)));
        asm volatile("ds_read_b64 %0, %1" : "=v"(pw[2 * c2 + j]) : "v"(ad));
      }
    u32x4 vf[16];
    const uint32_t vb = vb0 + (uint32_t)((t & 1) * kTileB);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      vf[4 * c2 + 0] = ds_b128<0 * 32 * kVtRowB>(vb ^ (uint32_t)(c2 << 5));
      vf[4 * c2 + 1] = ds_b128<1 * 32 * kVtRowB>(vb ^ (uint32_t)(c2 << 5));
      vf[4 * c2 + 2] = ds_b128<2 * 32 * kVtRowB>(vb ^ (uint32_t)(c2 << 5));
      vf[4 * c2 + 3] = ds_b128<3 * 32 * kVtRowB>(vb ^ (uint32_t)(c2 << 5));
    }
    float al;
    asm volatile("ds_read_b32 %0, %1" : "=v"(al) : "v"(addr_of(abuf) + 4u * (uint32_t)lane));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(al) :: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(pw[i]));
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(vf[i]));
    if (t + 1 < rt.nt) load_p(t + 1);  // this wave's P and alpha reads are done
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = acc[d][r] * al;
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const u32x4 pq = {pw[2 * c2].x, pw[2 * c2].y, pw[2 * c2 + 1].x, pw[2 * c2 + 1].y};
      const f16x8 pf = __builtin_bit_cast(f16x8, pq);
#pragma unroll
      for (int d = 0; d < 4; ++d) acc[d] = mfma32h(__builtin_bit_cast(f16x8, vf[4 * c2 + d]), pf, acc[d]);
    }
  }
  // O = acc / (l * 2^-8), one RNE cast
  const float l_div = a.l[bh * a.S + min(qrow, a.S - 1)] * kVScale;
  if (qrow < a.S) {
    uint16_t* orow = a.o.row(b, qrow, h);
    float* frow = a.of ? a.of + (((int64_t)b * a.S + qrow) * a.H + h) * kHeadDim : nullptr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        const float o0 = acc[d][4 * g4] / l_div, o1 = acc[d][4 * g4 + 1] / l_div;
        const float o2 = acc[d][4 * g4 + 2] / l_div, o3 = acc[d][4 * g4 + 3] / l_div;
        const u32x2 ov = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        *(u32x2*)(orow + d0) = ov;
        if (frow) *(f32x4*)(frow + d0) = f32x4{o0, o1, o2, o3};
      }
  }
}

}  // namespace qi
