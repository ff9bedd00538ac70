// qi_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "qi_common.h"

namespace qi {

constexpr int kPrologueChunk = 16;  // tokens per gain-gradient partial (frozen)

struct PrologueArgs {
  View<const uint16_t> x;
  View<uint16_t> y;
  float* yf;  // nullable dense [B,S,H,128]
  const float* gain;
  int gain_streams;
  int B, S, H, T_txt, gh, gw;
  double theta;
  float eps;
};

struct PrologueBwdArgs {
  View<const uint16_t> x;  // raw BF16 input of the prologue
  View<float> dx;          // in: dL/dy (pre-rotation gradient); out: dL/dx
  const float* gain;
  float* partials;  // [B][n_chunks][128]
  int gain_streams;
  int B, S, H, T_txt, gh, gw;
  int n_txt_chunks, n_chunks;
  double theta;
  float eps;
};

struct DgainFoldArgs {
  const float* partials;  // [B][n_chunks][128]
  float* dg_ps;           // [B][gain_streams][128]
  float* dg;              // nullable [gain_streams][128]
  int B, gain_streams, n_txt_chunks, n_chunks;
};

// Forward attention.  One launch covers up to kMaxBatchPerLaunch rows.
constexpr int kFwdBN = 64;        // key tile width (frozen: part of the arithmetic contract)
constexpr int kFwdWaves = 8;      // waves per workgroup, two per SIMD
constexpr int kFwdRowsPerWave = 32;
// Largest K/V sequence stride (elements) the forward's 32-bit row offsets cover.
constexpr int64_t kFwdMaxRowStride = int64_t(1) << 26;

struct FwdArgs {
  View<const uint16_t> q, k;
  const uint16_t* vt;  // FP16 V^T key tiles [B][H][nt_max][128][64] (B of this launch)
  View<uint16_t> o;
  float* lse;  // dense [B,H,S] (B of this launch)
  float* of;   // nullable dense [B,S,H,128]
  int B, S, H, T_txt, T_img;
  int nt_max;     // key tiles per (b, h) slot of vt
  int n_qtiles;   // ceil(S / rows per workgroup)
  int xcd_remap;  // 1: group the query tiles of a (b, h) on one XCD
  int txt_len[kMaxBatchPerLaunch];
  // partial forward only: the key block (text tiles when blk_text; image
  // tiles blk_img_t0 <= t < blk_img_t1) and the row-state outputs
  int blk_text, blk_img_t0, blk_img_t1;
  float* pacc;  // [B][H][S][128]: sum_j p_j v_j 2^-8 (B of this launch)
  float* pm;    // [B][H][S]: reference max of the raw scores
  float* pl;    // [B][H][S]: row sum of p; carried blocks: [B][H][S][2], one per half-wave
  // carried blocks only: the state the previous block left (all null: empty)
  const float* cin_acc;  // [B][H][S][128]
  const float* cin_m;    // [B][H][S]
  const float* cin_l;    // [B][H][S][2]
};

constexpr int kMaxMergeBlocks = 4096;  // key blocks one merge call folds

// Fixed-order merge of the row states of n key blocks (block k of every
// array at offset k * blk_stride elements, rows at 1 element / 128 for acc).
struct MergeArgs {
  const float* acc;  // [n][rows][128]
  const float* m;    // [n][rows]
  const float* l;    // [n][rows]
  int64_t rows;      // B * H * S
  View<uint16_t> o;
  float* lse;  // [B][H][S]
  float* of;   // nullable dense [B,S,H,128]
  int n, S, H;
};

// Backward attention.
constexpr int kBwdBN = 64;  // key tile of the dQ pass (= forward order)
constexpr int kBwdBM = 64;  // query tile of the dK/dV pass (frozen)
constexpr int kBwdDqWaves = 8;  // dQ pass: waves per workgroup (two alternating groups of 4)
constexpr int kBwdKvWaves = 8;  // dK and dV passes: waves (x 32 keys) per workgroup

struct BwdArgs {
  View<const uint16_t> q, k, v, dO;
  const uint16_t* do16t;       // FP16 dO * 2^e(b,h) as transposed query tiles [B][H][nt_do][128][64], for the dV product
  int nt_do;                   // query tiles per (b, h) in that buffer
  const float* do_inv_scale;   // [B][H]: 2^-e(b,h)
  uint32_t* do_amax;           // [B][H][n_qtiles][kBwdDqWaves]: max |dO| bits of each prep wave's rows
  View<const float> o;  // FP32 pre-cast forward output
  const float* lse;  // [B,H,S]
  float* Dvec;       // [B,H,S] workspace: rowsum(dO * O)
  float* lse2;       // [B,H,S] workspace: LSE * log2(e), for the key-side passes
  View<float> dq, dk, dv;
  int B, S, H, T_txt, T_img;
  int n_qtiles, n_ktiles;
  int xcd_remap;
  int txt_len[kMaxBatchPerLaunch];
};

__global__ void qknorm_rope_fwd_kernel(PrologueArgs a);
// The Q and K gradients go through one launch each: grid z (prologue
// backward) or y (fold) selects the tensor.
struct PrologueBwdPair {
  PrologueBwdArgs t[2];
};
struct DgainFoldPair {
  DgainFoldArgs t[2];
};
__global__ void qknorm_rope_bwd_kernel(PrologueBwdPair p);
__global__ void dgain_fold_kernel(DgainFoldPair p);
__global__ void attn_fwd_kernel(FwdArgs a);
__global__ void attn_fwd_partial_kernel(FwdArgs a);
__global__ void attn_fwd_carry_kernel(FwdArgs a);
__global__ void attn_merge_kernel(MergeArgs a);

// V -> FP16 (v * 2^-8) conversion pass of the forward: writes each logical
// key tile of 64 keys transposed, as 128 channel rows of 64 keys, the keys of
// every 16-key chunk in the A.V product's reduction order; keys past a tile's
// valid count are zero.
constexpr int kVtileElems = kHeadDim * kFwdBN;  // FP16 values per V^T tile
struct VtileArgs {
  View<const uint16_t> v;  // BF16 [B,S,H,128] (B of this launch)
  uint16_t* out;           // FP16 [B][H][nt_max][128][64]
  int H, T_txt, T_img, nt_max;
  int txt_len[kMaxBatchPerLaunch];
  // tiles converted: the text tiles when with_text, image tiles img_t0 <= t' < img_t1
  int with_text, img_t0, img_t1;
};
__global__ void v_tiles_kernel(VtileArgs a);

// The forward's Q and K prologues and its V tile conversion in one launch.
struct QkvPrologueArgs {
  PrologueArgs q, k;  // same token range (B of this launch)
  VtileArgs v;
  int64_t nblk;       // blocks per prologue: ceil(B * S / 4)
};
__global__ void qkv_prologue_kernel(QkvPrologueArgs a);

// Unfused forward: the three operators whose composition the fused kernel
// reproduces byte for byte.  Intermediates are dense per (b, h) row-major
// over the query rows, with Kp = 64 * nt_max key slots per row: slot 64*t + j
// is key j of logical key tile t (slots of keys past a tile's valid count,
// and of tiles past the row's tile count, hold the masked value).
constexpr int kQkWaves = 8;       // score operator: waves (x 32 query rows) per workgroup
constexpr int kSoftmaxWaves = 4;  // softmax operator
constexpr int kAvWaves = 8;       // A.V operator
struct QkArgs {
  View<const uint16_t> q, k;
  float* s;  // FP32 raw scores q'.k' [B][H][S][Kp] (B of this launch); masked = -inf
  int S, H, T_txt, T_img, nt_max;
  int txt_len[kMaxBatchPerLaunch];
};
struct SoftmaxArgs {
  const float* s;  // [B][H][S][Kp]
  uint16_t* p;     // FP16 P [B][H][S][Kp]; masked = 0
  float* alpha;    // FP32 rescale factor of tile t [B][H][nt_max][S] (tile-major); unused tiles = 1
  float* l;        // FP32 row sum [B][H][S]
  float* lse;      // FP32 [B][H][S]
  int S, H, T_txt, T_img, nt_max;
  int txt_len[kMaxBatchPerLaunch];
};
struct AvArgs {
  const uint16_t* p;
  const float* alpha;
  const float* l;
  const uint16_t* vt;  // FP16 V^T key tiles from v_tiles_kernel [B][H][nt_max][128][64]
  View<uint16_t> o;
  float* of;  // nullable dense [B,S,H,128]
  int S, H, T_txt, T_img, nt_max;
  int txt_len[kMaxBatchPerLaunch];
};
__global__ void attn_qk_kernel(QkArgs a);
__global__ void attn_softmax_kernel(SoftmaxArgs a);
__global__ void attn_av_kernel(AvArgs a);

// Projections around the attention (per-stream weights, Y = X W^T + bias).
constexpr int kProjTile = 256;  // tokens and channels per workgroup tile
constexpr int kProjTK = 64;     // K-elements per LDS stage
constexpr int kProjWaves = 8;
struct ProjArgs {
  const uint16_t* x;  // BF16 rows of K elements: token s of sample b at x + b*x_sb + s*x_ss
  int64_t x_sb, x_ss;
  const uint16_t* w;  // BF16 [weight_streams][N][K]
  const float* bias;  // FP32 [weight_streams][N]
  int weight_streams;
  int B, S, T_txt, K, N, D;  // N = sections * D output channels
  int n_mt_txt, n_mt_img, n_nt;
  View<uint16_t> out[3];  // section i (channels i*D .. i*D + D - 1) as [B,S,H,128]
  int fuse;               // 1: sections 0 and 1 (Q, K) go through the RMSNorm + gain + RoPE prologue
  const float* gain_q;
  const float* gain_k;  // FP32 [gain_streams][128]
  int gain_streams;
  float eps;
  const float* rope;  // FP32 [S][64][2]: (cos, sin) per token position and pair
};
struct RopeTableArgs {
  float* table;  // [S][64][2]
  int S, T_txt, gh, gw;
  double theta;
};
__global__ void proj_gemm_kernel(ProjArgs a);
__global__ void rope_table_kernel(RopeTableArgs a);

// dO -> FP16 dO * 2^e(b,h): one power of two per (sample, head), from the
// max |dO| that the prep kernel records per wave; written as transposed
// query tiles of the dK/dV passes' frozen order (grid: nt_do x H x B).
struct DoPrepArgs {
  View<const uint16_t> dO;  // BF16 [B,S,H,128] (B of this launch)
  uint16_t* out;            // FP16 transposed query tiles [B][H][nt_do][128][64]
  const uint32_t* amax;     // [B][H][n_amax]
  int n_amax;               // maxima per (b, h)
  float* inv_scale;         // [B][H]
  int S, H, T_txt, T_img, nt_do;
  int txt_len[kMaxBatchPerLaunch];
};
__global__ void do_convert_kernel(DoPrepArgs a);
// D and the max |dO| per wave (grid: B*H*n_qtiles workgroups of kBwdDqWaves
// waves), then the dK, dQ and dV passes in one grid of
// B*H*(2*n_ktiles + n_qtiles) workgroups.
__global__ void attn_bwd_prep_kernel(BwdArgs a);
__global__ void attn_bwd_kernel(BwdArgs a);

}  // namespace qi
