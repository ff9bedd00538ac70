// qi_lds.h -- LDS tiles of 64 rows x 128 BF16 channels on gfx950, shared by
// the attention forward and the dQ pass of the backward.
//
// A tile row is an unpadded 256-byte line; its 16-byte chunk c lives at
// chunk c ^ swz(row).  Tiles are filled by direct global->LDS loads
// (global_load_lds_dwordx4, no registers) and read in two ways:
//  * row fragments (ds_read_b128): the A operand of X.Y^T with the tile as X,
//    32 rows x 16 channels per v_mfma_f32_32x32x16_bf16;
//  * transposed fragments (ds_read_b64_tr_b16): the A operand of X^T.Z,
//    32 channels x 16 rows, with the 16 rows of a chunk in the permuted
//    order (bits 2 and 3 of the row index swapped) that matches the
//    accumulator layout of a 32x32 MFMA result used as the B operand.
// The matrix-phase reads and the loads are inline asm: their position and
// their waits (lgkmcnt / vmcnt) are explicit, so the compiler neither waits
// for the loads before unrelated LDS reads nor spills 64-bit addresses.
#pragma once

#include "qi_common.h"

namespace qi {
namespace lds {

constexpr int kRowB = 256;             // bytes per row
constexpr int kTileRows = 64;
constexpr int kTileB = kTileRows * kRowB;  // 16 KiB

typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// swz is a permutation of row % 16 (row reads: 16 consecutive rows hit 16
// distinct chunks) whose bits 2-3 take every value within each 4 consecutive
// rows (transposing reads: 4 rows x 4 chunks hit 16 distinct chunks), so
// neither read nor the contiguous load writes meet LDS bank conflicts.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int off(int row, int chunk) { return row * kRowB + 16 * (chunk ^ swz(row)); }

__device__ __forceinline__ uint32_t addr_of(const char* p) { return (uint32_t)(uintptr_t)(const lds_char*)p; }

// One direct global -> LDS load of 16 bytes per lane with a scalar base and
// a 32-bit lane offset: lane l's bytes land at LDS byte lds + 16*l.  M0 (the
// LDS destination) is written here; kernels that use it put nothing else in
// M0 (no LDS-DMA builtin, GWS or message send), so the clobber destroys no
// value the compiler keeps.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* base, uint32_t off32, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(off32), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Tile fill: wave `sub` (0..3) of a 4-wave group fills rows 16*sub..16*sub+15,
// 4 rows (1 KiB) per instruction; lane l writes LDS slot l of the block,
// i.e. physical chunk l%16 of row 4i + l/16, so it fetches the logical chunk
// that the swizzle maps there.  Rows past `nvalid` are not read and are
// zero-filled (plain LDS stores), so a masked row never carries a NaN.
struct RowOff {
  uint32_t o[4];
};
// Lane byte offsets for a source whose rows are `ss` elements apart
// (ss < 2^26, checked on the host).
__device__ __forceinline__ RowOff row_offsets(int64_t ss, int lane) {
  RowOff r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kl = 4 * i + (lane >> 4);       // row within a wave's 16
    const int chunk = (lane & 15) ^ swz(kl);  // swz depends on row % 16 only
    r.o[i] = (uint32_t)(kl * (uint32_t)ss + 8 * chunk) * 2u;
  }
  return r;
}
__device__ __forceinline__ void load_rows(const View<const uint16_t>& src, const RowOff& ro, char* dst, int b,
                                          int h, int row0, int nvalid, int sub, int lane) {
  const char* base = (const char*)(src.p + (int64_t)b * src.sb + (int64_t)h * src.sh +
                                   (int64_t)(row0 + 16 * sub) * src.ss);
  const uint32_t la = addr_of(dst + 16 * sub * kRowB);
  if (nvalid >= 16 * sub + 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(base, ro.o[i], la + 4 * i * kRowB);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (16 * sub + 4 * i + (lane >> 4) < nvalid) {
        dma16(base, ro.o[i], la + 4 * i * kRowB);
      } else {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4*)(dst + (16 * sub + 4 * i) * kRowB + 16 * lane) = z;
      }
    }
  }
}

template <int kOff>
__device__ __forceinline__ u32x2v ds_tr(uint32_t a) {
  u32x2v r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(kOff));
  return r;
}
template <int kOff>
__device__ __forceinline__ u32x4 ds_b128(uint32_t a) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(kOff));
  return r;
}

// Row fragment (rows 32*kb .. 32*kb+31, channels 16*kk .. 16*kk+15): lane l
// reads row 32*kb + l%32, logical chunk 2*kk + l/32.  With s = swz(l%32) the
// physical chunk is 2*(kk ^ s/2) + ((l/32) ^ s)%2, so the address is
// row_base ^ (kk << 5) plus the immediate kb * 32 rows.
__device__ __forceinline__ uint32_t row_base(uint32_t tile, int lane) {
  const int lr = lane & 31, hh = lane >> 5;
  const int s = swz(lr);
  return tile + lr * kRowB + 32 * (s >> 1) + 16 * ((hh ^ s) & 1);
}
template <int kk, int kb>
__device__ __forceinline__ bf16x8 row_frag(uint32_t rb) {
  return __builtin_bit_cast(bf16x8, ds_b128<kb * 32 * kRowB>(rb ^ (kk << 5)));
}

// Transposed fragment (channels 32*d .. 32*d+31, rows of chunk c2 = rows
// 16*c2 .. 16*c2+15): two reads, half r covering rows 16*c2 + 8*r + 4*hh +
// i/4 (i = lane % 16), logical chunk 4*d + 2*g + q/2 (g = bit 4 of the lane,
// q = i % 4).  The physical chunk is 4*(d ^ i/4) + ((2*g + q/2) ^ (2r + hh)),
// so the address is tr_base ^ (d << 6) ^ (r << 5) plus the immediate
// 16*c2 + 8*r rows.  Within each 16-lane group the read hands lane j element
// (j & 3) of the 8-byte piece addressed by lane 4t + (j >> 2) as its slot t,
// so lane l receives channel 32*d + l%32 of the 8 rows the permuted
// reduction index assigns to its half-wave.
__device__ __forceinline__ uint32_t tr_base(uint32_t tile, int lane) {
  const int hh = lane >> 5, g = (lane >> 4) & 1, i = lane & 15, q = i & 3;
  const int cl = 2 * g + (q >> 1);
  return tile + (4 * hh + (i >> 2)) * kRowB + 64 * (i >> 2) + 16 * (cl ^ hh) + 8 * (q & 1);
}
template <int c2, int d>
__device__ __forceinline__ bf16x8 tr_frag(uint32_t tb) {
  const u32x2v r0 = ds_tr<c2 * 16 * kRowB>(tb ^ (d << 6));
  const u32x2v r1 = ds_tr<c2 * 16 * kRowB + 8 * kRowB>(tb ^ (d << 6) ^ 32);
  const u32x4 v = {r0.x, r0.y, r1.x, r1.y};
  return __builtin_bit_cast(bf16x8, v);
}

// V^T tiles of the forward: 128 channel rows x 64 keys in FP16, one 128-byte
// line per channel, the keys of each 16-key chunk already in the A.V
// reduction order (written so by the conversion pass).  Logical 16-byte chunk
// j of row d (keys 8j .. 8j+7 of that order) lives at chunk j ^ ((d >> 1) & 7):
// a 16-lane group of fragment reads covers 16 consecutive rows at one logical
// chunk, i.e. 8 distinct chunks in each of two 128-byte row parities, which
// are the 64 banks once.
constexpr int kVtRowB = 128;

// Fragment of channel rows 32*db .. 32*db+31 and 16-key chunk c2: lane l
// reads row 32*db + l%32, logical chunk 2*c2 + l/32.  With s = ((l%32) >> 1) & 7
// the physical chunk is 2*(c2 ^ s/2) + ((l/32) ^ s)%2, so the address is
// vt_base ^ (c2 << 5) plus the immediate 32*db rows.
__device__ __forceinline__ uint32_t vt_base(uint32_t tile, int lane) {
  const int lr = lane & 31, hh = lane >> 5;
  const int s = (lr >> 1) & 7;
  return tile + lr * kVtRowB + 32 * (s >> 1) + 16 * ((hh ^ s) & 1);
}

// Tile fill from a contiguous 16 KiB source tile [128][64]: wave `sub` (0..3)
// fills channel rows 32*sub .. 32*sub+31, 8 rows (1 KiB) per instruction;
// lane l writes LDS slot l of the block, i.e. physical chunk l%8 of row
// 8i + l/8, and fetches the logical chunk the swizzle maps there, which
// depends on the lane and on i%2 only.
struct VtOff {
  uint32_t o[2];
};
__device__ __forceinline__ VtOff vt_offsets(int lane) {
  VtOff r;
#pragma unroll
  for (int p = 0; p < 2; ++p) r.o[p] = (uint32_t)((lane >> 3) * kVtRowB + 16 * ((lane & 7) ^ (4 * p + (lane >> 4))));
  return r;
}
__device__ __forceinline__ void load_vt(const uint16_t* src_tile, const VtOff& vo, char* dst, int sub) {
  const char* base = (const char*)src_tile + sub * 32 * kVtRowB;
  const uint32_t la = addr_of(dst + sub * 32 * kVtRowB);
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(base + i * 8 * kVtRowB, vo.o[i & 1], la + i * 8 * kVtRowB);
}

// Workgroup barrier without the memory fence of __syncthreads: callers wait
// for exactly the memory operations the next phase depends on.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace lds
}  // namespace qi
