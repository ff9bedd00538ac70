/*
 * qi.h -- C ABI of the strict joint-attention library for AMD Instinct
 * MI355X (gfx950): learned-gain Q/K RMSNorm + three-axis RoPE, and masked
 * non-causal joint attention over [text, image] with a deterministic
 * backward.
 *
 * Pages cited (by title and section):
 *   [Roadmap]     "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
 *                 ablation matrix and integration plan" (issue 386).
 *   [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List".
 *   [PR 537]      "[WS1][Qwen-Image][CUDA] AdaLN modulation projection
 *                 (adaln_mod_projection)".
 *   [PR 507]      "[WS1][CUDA][Qwen3-Next] TP4 GDN, convolution and D=256
 *                 attention mixers on real weights".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory.  Every tensor pointer is a DEVICE pointer owned by the caller;
 *    `txt_len` in qi_geom is a HOST array.  The library never allocates,
 *    frees or retains a pointer after the call returns, and never writes an
 *    input.  Work is enqueued on `stream` (0 = the default stream); calls
 *    return without synchronising.
 *  - Activations are [B, S, H, 128] views (qi_bshd): the head-dim stride is 1
 *    and B, S, H strides are given in elements.  The sequence axis is the
 *    concatenation [text (T_txt, padded), image (grid_h * grid_w tokens,
 *    row-major)] ([Roadmap], "Model contract", row Streams).
 *  - Alignment: every data pointer 16-byte aligned and every stride a
 *    multiple of 16 bytes ([PR 537], the input-check rule of its kernel).
 *  - Status.  0 on success, else one of the QI_E_* codes; qi_last_error()
 *    then holds a message for the calling thread.  All arguments are
 *    validated before anything is launched: a failed call writes nothing.
 *    Configurations outside the strict contract fail closed ([Roadmap],
 *    "Numerical requirements"; [Kernel list], the rule against silent
 *    fallback): there is no other code path.
 *  - Determinism.  Fixed reduction trees, FP32 accumulation, no split-KV /
 *    Split-K / atomics; a row's output bytes do not depend on batch size,
 *    batch position, text padding, launch geometry or repetition
 *    ([Roadmap], "Numerical requirements"; [Kernel list], rules 1-6).
 */
#ifndef QI_H
#define QI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QI_HEAD_DIM 128

enum qi_status {
  QI_OK = 0,
  QI_E_INVALID = 1,     /* null pointer, bad size or geometry, txt_len out of range */
  QI_E_UNSUPPORTED = 2, /* D != 128, RoPE axes != {16,56,56}, no gfx950 device */
  QI_E_ALIGN = 3,       /* pointer or stride not 16-byte aligned */
  QI_E_ALIAS = 4,       /* an output overlaps an input or another output */
  QI_E_WORKSPACE = 5,   /* workspace null or smaller than qi_joint_attn_bwd_workspace() */
  QI_E_STRICT = 6,      /* strict-arithmetic probe failed on the device */
  QI_E_HIP = 7          /* a HIP runtime call or launch failed */
};

/* A [B, S, H, 128] view; element type given by the entry point. */
typedef struct {
  void* data;
  int64_t sb, ss, sh; /* strides in elements; the head-dim stride is 1 */
} qi_bshd;

/* Geometry of one call ([Roadmap], "Model contract": 24 heads x 128, text
 * length padded with a key mask, image grid of the reference shapes). */
typedef struct {
  int32_t B;              /* batch rows, >= 1 */
  int32_t H;              /* heads, >= 1 */
  int32_t D;              /* head dim; must be 128 */
  int32_t T_txt;          /* padded text length, >= 0 */
  int32_t grid_h, grid_w; /* image token grid, each >= 1; S = T_txt + grid_h*grid_w */
  const int32_t* txt_len; /* HOST [B]: valid text length of each row, 0..T_txt */
  int32_t rope_axes[3];   /* must be {16, 56, 56} */
  double rope_theta;      /* finite, > 1 (the model uses 10000) */
  float rms_eps;          /* finite, > 0 (the model uses 1e-6) */
  int32_t gain_streams;   /* 1: one [128] gain for all tokens; 2: [2][128],
                             set 0 for text tokens, set 1 for image tokens */
} qi_geom;

/*
 * qi_qknorm_rope -- prologue: per-head RMSNorm with a learned gain, then the
 * three-axis rotary embedding, then one FP32->BF16 rounding.
 *   [Roadmap] "Model contract", rows Q/K preprocessing (RMSNorm with learned
 *   gain, eps, before RoPE) and RoPE (axes 16/56/56, theta, centred image
 *   indices, text offset max(h/2, w/2)); [Kernel list] rows qk_rmsnorm and
 *   multi_axis_rope (text on the grid diagonal).
 * For each (b, s, h) row x of 128 BF16 values:
 *   r = 1/sqrt(mean(x^2) + eps);  t = gain ⊙ (x * r);
 *   y = bf16_rne(rotate(t)), pairs (2k, 2k+1) rotated by p_axis(k) * omega_k,
 *   positions: image token (row i, col j) -> (0, i - ceil(h/2), j - ceil(w/2)),
 *   text token j -> (o+j, o+j, o+j) with o = max(floor(h/2), floor(w/2)).
 * Arguments:
 *   x        BF16 [B,S,H,128] input (Q or K from the projection).
 *   gain     FP32 device [gain_streams][128].
 *   y        BF16 [B,S,H,128] output; must not overlap x or gain.
 *   y_f32    nullable FP32 dense [B,S,H,128] output of the pre-cast values.
 */
int qi_qknorm_rope(const qi_geom* geom, qi_bshd x, const float* gain, qi_bshd y,
                   float* y_f32, hipStream_t stream);

/* Bytes of device workspace qi_joint_attn_fwd needs for this geometry:
 * B*H*nt*64*128 FP16 values with nt = ceil(T_txt/64) + ceil(grid_h*grid_w/64)
 * key tiles, rounded up to 256 bytes; 0 for an invalid geometry. */
size_t qi_joint_attn_fwd_workspace(const qi_geom* geom);

/*
 * qi_joint_attn_fwd -- masked non-causal attention over [text, image].
 *   [Kernel list] rows joint_attn_qk_gemm, joint_attn_softmax,
 *   joint_attn_av_gemm and joint_attention_fused; [Roadmap] "Model
 *   contract", rows Streams and Text input (key mask for padded prompts).
 * Row b attends to keys j < txt_len[b] and T_txt <= j < S; every query row,
 * padded text rows included, is computed.
 *   O[b,i,h,:] = bf16_rne( sum_j softmax_j(q_i . k_j / sqrt(128)) v_j )
 *   lse[b,h,i] = ln sum_j exp(q_i . k_j / sqrt(128))   (FP32)
 * Arguments:
 *   q, k, v  BF16 [B,S,H,128] (q, k are the prologue outputs).
 *   o        BF16 [B,S,H,128] output.
 *   lse      FP32 dense [B,H,S] output (kept for the backward).
 *   o_f32    nullable FP32 dense [B,S,H,128] output of the pre-cast O; the
 *            backward needs it.
 *   workspace  device buffer of at least qi_joint_attn_fwd_workspace()
 *            bytes, 256-byte aligned, not overlapping any other argument;
 *            its contents are scratch (the call writes V there as FP16
 *            transposed key tiles).
 * The A.V product takes P and V in FP16: P rounded once (RNE), V as
 * v * 2^-8 rounded once, which is exact for 2^-6 <= |v| <= 65504 * 2^8
 * and keeps an absolute error below 2^-17 for smaller |v|; larger |v|
 * (and non-finite v) give non-finite outputs.  A single BF16 rounding of P
 * would break 1e-2*|ref| + 2e-3 where O cancels on a few peaked keys.
 * The row sum uses the FP32 p.
 * The sequence stride of k must stay below 2^26 elements (the kernel
 * addresses 16 key rows from one base with 32-bit offsets); larger strides
 * return QI_E_UNSUPPORTED.  A null, misaligned or short workspace returns
 * QI_E_WORKSPACE / QI_E_ALIGN before any launch.
 */
int qi_joint_attn_fwd(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd o,
                      float* lse, float* o_f32, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * qi_joint_attn_fwd_noalloc -- qi_joint_attn_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument, and the call
 * allocates and frees nothing.  The V tiles go to a static device array of
 * the library, 64 MiB (67108864 bytes) per GPU, held from the first call on
 * that GPU until the process ends.  Geometries whose
 * qi_joint_attn_fwd_workspace() exceeds 64 MiB (B * H * nt above 4096 key
 * tiles; the 1024^2 shape at 24 heads needs 1632 per row) return
 * QI_E_WORKSPACE before anything is launched.  O, LSE and O_f32 equal
 * qi_joint_attn_fwd's byte for byte; every other argument and error as there.
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (other streams, other threads) race and give undefined results; a
 * call may follow any earlier call on the same stream (each call rewrites
 * every tile it reads).
 */
int qi_joint_attn_fwd_noalloc(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd o,
                              float* lse, float* o_f32, hipStream_t stream);

/*
 * qi_qkv_prologue -- the forward's preparation in one launch: the Q and K
 * prologues of qi_qknorm_rope (same arithmetic, same bytes) and the V ->
 * FP16 key-tile conversion that qi_joint_attn_fwd otherwise runs first.
 * ([Kernel list] rows qk_rmsnorm, multi_axis_rope and joint_attn_av_gemm;
 * [Roadmap] "Numerical requirements": a fused kernel gives the bytes of the
 * unfused ones.)
 *   q_raw, k_raw  BF16 [B,S,H,128] inputs; v BF16 [B,S,H,128].
 *   gain_q, gain_k  FP32 device [gain_streams][128].
 *   q, k     BF16 [B,S,H,128] outputs q', k'.
 *   v_tiles  device buffer of at least qi_joint_attn_fwd_workspace() bytes,
 *            256-byte aligned: receives V as FP16 v * 2^-8 transposed key
 *            tiles, the format qi_joint_attn_fwd_vtiles reads.
 */
int qi_qkv_prologue(const qi_geom* geom, qi_bshd q_raw, qi_bshd k_raw, qi_bshd v,
                    const float* gain_q, const float* gain_k, qi_bshd q, qi_bshd k,
                    void* v_tiles, size_t v_tiles_bytes, hipStream_t stream);

/*
 * qi_joint_attn_fwd_vtiles -- qi_joint_attn_fwd with V already converted:
 * one attention launch over the key tiles that qi_qkv_prologue wrote for
 * the same geometry and V (the contents are not checked).  O, LSE and O_f32
 * equal qi_joint_attn_fwd's byte for byte.  Arguments and errors as for
 * qi_joint_attn_fwd, with v_tiles (read only) in place of v and workspace.
 */
int qi_joint_attn_fwd_vtiles(const qi_geom* geom, qi_bshd q, qi_bshd k, const void* v_tiles,
                             size_t v_tiles_bytes, qi_bshd o, float* lse, float* o_f32,
                             hipStream_t stream);

/*
 * Key-block forward and merge -- the ring-ready form of qi_joint_attn_fwd
 * ([Kernel list], row joint_attention_fused, which is marked for Ulysses /
 * Ring sequence parallelism; [Roadmap], "Numerical requirements": distributed
 * execution reproduces the single-device bytes).  The keys of each row are
 * split into blocks; every block yields a row state (acc, m, l) on its own,
 * in any order, on any device, and qi_joint_attn_merge folds the states in
 * the fixed block order k = 0, 1, ...:
 *   m = max_k m_k;  alpha_k = exp2((m_k - m) c);  acc = sum_k alpha_k acc_k;
 *   l = sum_k alpha_k l_k (both summed in ascending k);
 *   O = bf16(acc / (l 2^-8));  LSE = (m c + log2 l) ln 2,  c = log2(e)/sqrt(128).
 * One block holding every key gives O, LSE and O_f32 equal byte for byte to
 * qi_joint_attn_fwd.  With several blocks the bytes are fixed by the block
 * partition alone (not by the order, device or launch that produced each
 * state).
 *
 * A block: the text keys j < txt_len[b] of every row when include_text = 1,
 * plus the image keys T_txt + i with img_begin <= i < img_end; img_begin a
 * multiple of 64, img_end a multiple of 64 or grid_h * grid_w (the key tiles
 * of the whole-row forward stay whole).  The blocks passed to one merge must
 * cover every key of every row exactly once.
 */
typedef struct {
  int32_t include_text;
  int32_t img_begin, img_end;
} qi_key_block;

/*
 * qi_joint_attn_fwd_partial -- the forward over one key block: the row state
 * after the block's key tiles, in the whole-row kernel's arithmetic.
 *   q, k, v  as for qi_joint_attn_fwd.
 *   acc      FP32 dense [B][H][S][128] output: sum_j p_j v_j 2^-8 with
 *            p_j = exp2(s_j c - m c) (FP16 V operand of the forward).
 *   m        FP32 dense [B][H][S] output: the block's reference max m of the
 *            raw scores (-inf for a row without keys in the block).
 *   l        FP32 dense [B][H][S] output: sum_j p_j (0 without keys).
 *            m and l need 4-byte alignment only (so that stacked states of
 *            any B*H*S can be written block by block); acc 16 bytes.
 *   workspace  as for qi_joint_attn_fwd.
 * QI_E_INVALID for a block outside the image range, not tile-aligned, or
 * empty.
 */
int qi_joint_attn_fwd_partial(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v,
                              qi_key_block block, float* acc, float* m, float* l,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * qi_joint_attn_merge -- fold n_blocks row states in ascending block order.
 *   acc, m, l  stacks of n_blocks states, block k at acc + k*B*H*S*128,
 *            m + k*B*H*S, l + k*B*H*S (1 <= n_blocks <= 4096).
 *   o        BF16 [B,S,H,128] output; lse FP32 dense [B,H,S] output;
 *            o_f32 nullable FP32 dense [B,S,H,128] output.
 */
int qi_joint_attn_merge(const qi_geom* geom, int32_t n_blocks, const float* acc,
                        const float* m, const float* l, qi_bshd o, float* lse, float* o_f32,
                        hipStream_t stream);

/*
 * qi_joint_attn_fwd_carry -- the forward over one key block continuing the
 * row state a previous block left: the other ring form of the same rows
 * ([Kernel list], row joint_attention_fused, Ulysses / Ring sequence
 * parallelism; [Roadmap], "Numerical requirements").  Where the merge form
 * keeps every block's state and folds them at the end, here the state
 * travels from block to block (with the query rows it belongs to) and the
 * last block writes O and LSE.  The kernel runs the block's key tiles on
 * the carried (acc, reference max, per-half-wave row sums) exactly as the
 * whole-row kernel runs them after the tiles before, so a chain of blocks
 * that visits the keys in the whole call's order -- the text block first,
 * then image tiles ascending, each block starting where the previous ended
 * -- gives O, LSE and O_f32 equal byte for byte to qi_joint_attn_fwd, for
 * any such partition.  Another order gives the same attention within
 * rounding, not the same bytes.
 *   q, k, v  as for qi_joint_attn_fwd; block as for qi_joint_attn_fwd_partial.
 *   acc_in, m_in, l_in   the state to continue, read only: acc FP32 dense
 *            [B][H][S][128] (16-byte aligned), m FP32 [B][H][S], l FP32
 *            [B][H][S][2] (8-byte aligned; the two half-wave sums of each
 *            row).  All three null: the empty state (the first block).
 *   acc_out, m_out, l_out  the state after the block, same layouts, written;
 *            each may be the same buffer as its input (continued in place:
 *            every row reads its state before it writes it), and must not
 *            overlap anything else.  All three null: this is the last block.
 *   o, lse, o_f32  written by the last block only (as for
 *            qi_joint_attn_fwd); pass {NULL} / NULL / NULL otherwise.
 *   workspace  as for qi_joint_attn_fwd (V tiles of the block).
 * QI_E_INVALID for a bad block (as qi_joint_attn_fwd_partial), a state given
 * in part, o / lse / o_f32 on a block that is not the last, or a single
 * text-only block (no previous state) for a sample with txt_len = 0, whose
 * rows would have no key.  A chain whose rows saw no key at all writes NaN.
 */
int qi_joint_attn_fwd_carry(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v,
                            qi_key_block block, const float* acc_in, const float* m_in,
                            const float* l_in, float* acc_out, float* m_out, float* l_out,
                            qi_bshd o, float* lse, float* o_f32, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Unfused forward -- the three attention operators of [Kernel list], rows
 * joint_attn_qk_gemm, joint_attn_softmax and joint_attn_av_gemm, whose
 * composition qk_gemm -> softmax -> av_gemm gives O, LSE (and O_f32) equal
 * byte for byte to qi_joint_attn_fwd on the same inputs (row
 * joint_attention_fused; [Roadmap], "Numerical requirements": fused kernels
 * reproduce the unfused result byte for byte).  They hold the same per-row
 * arithmetic as the fused kernel with the intermediates in HBM.
 *
 * Scores and P are dense arrays indexed [b][h][i][slot] for query row i
 * (alpha is tile-major: [b][h][t][i]), with Kp = qi_joint_attn_key_slots()
 * slots per row:
 * Kp = 64 * nt with nt = ceil(T_txt/64) + ceil(grid_h*grid_w/64) logical key
 * tiles; slot 64*t + j is key j of tile t of row b, where row b's tiles are
 * ceil(txt_len[b]/64) text tiles (keys 64t ...) followed by the image tiles
 * (keys T_txt + 64t' ...).  Slots of keys past a tile's valid count, and
 * every slot of the tiles past row b's own tile count, are masked.
 */
/* Key slots per query row, Kp (0 for an invalid geometry). */
int64_t qi_joint_attn_key_slots(const qi_geom* geom);

/*
 * qi_joint_attn_qk_gemm -- raw scores s = q_i . k_j, FP32 accumulation of
 * BF16 products in a fixed order ([Kernel list], row joint_attn_qk_gemm).
 * The 1/sqrt(128) scale is applied by qi_joint_attn_softmax (inside the
 * exponent, as c = log2(e)/sqrt(128)), as the fused kernel applies it.
 *   q, k     BF16 [B,S,H,128].
 *   scores   FP32 dense [B][H][S][Kp] output; masked slots are -inf.
 */
int qi_joint_attn_qk_gemm(const qi_geom* geom, qi_bshd q, qi_bshd k, float* scores,
                          hipStream_t stream);

/*
 * qi_joint_attn_softmax -- masked online softmax over the key tiles in
 * order, fixed tiling of 64 keys ([Kernel list], row joint_attn_softmax).
 * Per row and tile t: m_t = m_{t-1}, or the tile max when that exceeds
 * m_{t-1} by more than 8/c; alpha_t = exp2((m_{t-1} - m_t) c) (exactly 1
 * where m did not move); p = exp2(s c - m_t c); l = alpha_t l + sum p, the
 * sum formed as two half sums over the keys 8g + 4h' + {0..3} (h' = 0, 1)
 * in ascending g, added at the end; LSE = (m c + log2 l) ln 2.
 *   scores   FP32 dense [B][H][S][Kp] from qi_joint_attn_qk_gemm.
 *   p        FP16 dense [B][H][S][Kp] output: p rounded to nearest even;
 *            masked slots 0.
 *   alpha    FP32 dense [B][H][Kp/64][S] output, tile-major (1 for unused
 *            tiles).
 *   l        FP32 dense [B][H][S] output: the row sum of the FP32 p.
 *   lse      FP32 dense [B][H][S] output.
 */
int qi_joint_attn_softmax(const qi_geom* geom, const float* scores, void* p, float* alpha,
                          float* l, float* lse, hipStream_t stream);

/*
 * qi_joint_attn_av_gemm -- O = (sum_t alpha-rescaled P_t V_t) / l
 * ([Kernel list], row joint_attn_av_gemm): acc = alpha_t acc + P_t V_t tile
 * by tile, FP16 P times FP16 v * 2^-8 with FP32 accumulation, then
 * O = acc / (l 2^-8) rounded once to BF16.
 *   p, alpha, l  outputs of qi_joint_attn_softmax.
 *   v        BF16 [B,S,H,128].
 *   o        BF16 [B,S,H,128] output; o_f32 nullable FP32 dense
 *            [B,S,H,128] output of the pre-cast O.
 *   workspace  as for qi_joint_attn_fwd (same size; scratch).
 */
int qi_joint_attn_av_gemm(const qi_geom* geom, const void* p, const float* alpha,
                          const float* l, qi_bshd v, qi_bshd o, float* o_f32, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Projections around the attention ([Kernel list], rows qkv_bias_gemm and
 * attn_out_bias_gemm; [Roadmap], "Model contract", row Streams: one weight
 * set per stream).  D = H * 128 model channels; x, o and y are [B,S,H,128]
 * views whose H * 128 channels of a token are contiguous (head stride 128).
 * Weights are BF16 [weight_streams][N][D] (a linear layer's [out][in]
 * layout), biases FP32 [weight_streams][N]; with weight_streams = 2, set 0
 * serves the text tokens s < T_txt and set 1 the image tokens.
 *   y[n] = bf16_rne( sum_k x[k] W[n][k] + bias[n] ),
 * FP32 accumulation over k ascending (fixed order, no split-K), so a token's
 * output bytes depend on its own row only.
 */
/* Bytes of workspace qi_qkv_proj needs with fuse_prologue = 1 (a table of
 * the rotation's cos/sin per token position: S*64*2 FP32, rounded up to 256
 * bytes); 0 for an invalid geometry. */
size_t qi_qkv_proj_workspace(const qi_geom* geom);

/*
 * qi_qkv_proj -- packed Q/K/V projection, N = 3D output channels: channels
 * 0..D-1 are Q (head h = channels 128h..128h+127), D..2D-1 K, 2D..3D-1 V.
 * With fuse_prologue = 1 the Q and K outputs are the prologue of
 * qi_qknorm_rope applied to the BF16 projections (gains gain_q, gain_k as
 * there); the bytes equal qi_qkv_proj with fuse_prologue = 0 followed by
 * qi_qknorm_rope on q and k, without their round trip through memory.
 *   x        BF16 [B,S,H,128] hidden states.
 *   q, k, v  BF16 [B,S,H,128] outputs.
 *   workspace  with fuse_prologue = 1: at least qi_qkv_proj_workspace()
 *            bytes, 256-byte aligned (scratch); else may be NULL.
 */
int qi_qkv_proj(const qi_geom* geom, qi_bshd x, const void* w, const float* bias,
                int32_t weight_streams, const float* gain_q, const float* gain_k,
                int32_t fuse_prologue, qi_bshd q, qi_bshd k, qi_bshd v, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * qi_attn_out_proj -- output projection, N = D: y = o W^T + bias.
 *   o        BF16 [B,S,H,128] attention output.
 *   y        BF16 [B,S,H,128] output.
 */
int qi_attn_out_proj(const qi_geom* geom, qi_bshd o, const void* w, const float* bias,
                     int32_t weight_streams, qi_bshd y, hipStream_t stream);

/* Bytes of device workspace qi_joint_attn_bwd needs for this geometry. */
size_t qi_joint_attn_bwd_workspace(const qi_geom* geom);

/*
 * qi_joint_attn_bwd -- gradients of the whole path (attention, rotation,
 * RMSNorm and gains) for upstream dO, with fixed-order tile sums and no
 * atomics ([Roadmap], "Work items": every differentiable operator has a
 * backward; "Numerical requirements"; the learned-gain comment of [Roadmap]
 * whose backward yields both dx and the gain gradient).
 *   dP = dO V^T;  D_i = dO_i . O_i;  dS = P ⊙ (dP - D);
 *   dq' = dS K / sqrt(128);  dk' = dS^T Q / sqrt(128);  dv = P^T dO;
 *   then for q (and likewise k): u = R^T dq';  dgain += u ⊙ xhat;
 *   dx = r (u ⊙ g - xhat * mean(u ⊙ g ⊙ xhat)).
 * Arguments:
 *   q_raw, k_raw   BF16 [B,S,H,128] prologue inputs.
 *   q, k, v        BF16 [B,S,H,128] prologue outputs and V.
 *   o_f32          FP32 [B,S,H,128]: the forward's pre-cast O (the o_f32
 *                  output of qi_joint_attn_fwd).  D_i is formed from it: the
 *                  BF16 O would shift D by ~2^-9 |dO||O| sqrt(128), more than
 *                  the gain gradients tolerate.
 *   lse            FP32 dense [B,H,S] from the forward.
 *   d_o            BF16 [B,S,H,128] upstream gradient.  The dv product
 *                  takes it as FP16 of dO * 2^e, one power of two per
 *                  (sample, head) that puts the slice's largest |dO| in
 *                  [2^14, 2^15): elements below 2^-28 of that maximum keep an
 *                  absolute error under 2^-39 of it; the scale is undone
 *                  exactly, so dv stays linear in power-of-two factors of dO.
 *   gain_q, gain_k FP32 device [gain_streams][128].
 *   dq, dk, dv     FP32 [B,S,H,128] outputs (dq, dk w.r.t. q_raw, k_raw).
 *                  Padded text query rows (txt_len[b] <= s < T_txt) are part
 *                  of the sums over queries of dk and dv like every other
 *                  row: give them dO = 0 (their outputs carry no gradient;
 *                  with dO = 0 they add exact zeros, so the valid rows'
 *                  gradients do not depend on T_txt), and keep their q_raw,
 *                  k_raw, q, k, o_f32 and lse finite.  Masked keys are never
 *                  read: their dk, dv rows are exact zeros.
 *   dgain_q_ps, dgain_k_ps   FP32 device [B][gain_streams][128]: gain
 *                  gradients of each sample alone.
 *   dgain_q, dgain_k  nullable FP32 device [gain_streams][128]: the
 *                  per-sample values summed in ascending b.
 *   workspace      device buffer of at least qi_joint_attn_bwd_workspace()
 *                  bytes, 256-byte aligned; its contents are scratch.
 * The sequence strides of q, k, v and d_o must stay below 2^26 elements, and
 * H at most 65535 (QI_E_UNSUPPORTED otherwise).
 */
int qi_joint_attn_bwd(const qi_geom* geom, qi_bshd q_raw, qi_bshd k_raw, qi_bshd q,
                      qi_bshd k, qi_bshd v, qi_bshd o_f32, const float* lse, qi_bshd d_o,
                      const float* gain_q, const float* gain_k, qi_bshd dq, qi_bshd dk,
                      qi_bshd dv, float* dgain_q_ps, float* dgain_k_ps, float* dgain_q,
                      float* dgain_k, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Measurement support (not part of the attention path).
 *
 * qi_clock_probe -- enqueue one launch of n_groups single-wave workgroups;
 * each reads the shader clock counter (s_memtime) and the constant-rate
 * wall clock (s_memrealtime), runs `iters` rounds of four BF16 MFMAs, reads
 * both again and writes out[3i] = shader-clock ticks, out[3i+1] = wall-clock
 * ticks elapsed in between (out[3i+2] keeps the MFMA result alive).
 * (ticks / wall ticks) * qi_wall_clock_khz() is the wave's average shader
 * clock in kHz while the chip carries a matrix load.
 *   out      device uint64 [n_groups][3], 8-byte aligned; 1 <= n_groups <= 65536,
 *            1 <= iters <= 2^20.
 * qi_wall_clock_khz -- rate of the wall clock of `device` in kHz (0 and
 * QI_E_HIP in qi_last_error() if it cannot be queried).
 */
int qi_clock_probe(uint64_t* out, int32_t n_groups, int32_t iters, hipStream_t stream);
int64_t qi_wall_clock_khz(int device);

/* Message for the calling thread's last nonzero status ("" if none). */
const char* qi_last_error(void);

/*
 * qi_strict_probe -- run the strict-arithmetic probe kernel on `device`:
 * an FP32 subnormal must survive a multiply, a division and a square root
 * must be correctly rounded, and the library's FP32->BF16 cast must round to
 * nearest even (cf. [PR 537], its probe of the built arithmetic).  The
 * verdict is cached per device id.  Returns QI_OK or QI_E_STRICT (or
 * QI_E_UNSUPPORTED / QI_E_HIP when the device cannot run it).
 */
int qi_strict_probe(int device);

/*
 * qi_trace -- JSON text describing the arithmetic contract the library was
 * built with: kernel names, frozen tile sizes, MFMA instructions, reduction
 * orders, accumulator precision, split-K / split-KV / atomics state, build
 * flags and target ([Kernel list], rule 7; [Roadmap], "Work items",
 * qwenimage_operator_trace).  The string is static; do not free it.
 */
const char* qi_trace(void);

#ifdef __cplusplus
}
#endif

#endif /* QI_H */
