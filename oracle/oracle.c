/*
 * oracle.c -- plain CPU oracle for the strict joint-attention path of a
 * Qwen-Image-style MMDiT block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no source with the GPU library.
 *
 * Pages followed (cited by title and section):
 *   [Roadmap]     "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
 *                 ablation matrix and integration plan" (issue 386): the
 *                 "Model contract" table (rows Streams, Text input, Q/K
 *                 preprocessing, RoPE) and "Numerical requirements".
 *   [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List": the
 *                 "Kernel table" rows qk_rmsnorm, multi_axis_rope,
 *                 joint_attn_qk_gemm, joint_attn_softmax, joint_attn_av_gemm.
 *   [Gain note]   the comment thread of [Roadmap]: the Q/K norm carries a
 *                 learned weight of 128 entries with eps 1e-6, so its
 *                 backward produces both dx and the weight gradient.
 *
 * What is computed is the plain mathematical definition, not a replica of any
 * tiling: RMSNorm with a learned gain, then a three-axis rotary embedding,
 * then masked softmax attention over the concatenated [text, image] sequence,
 * and the exact gradients of that composition.  Loops are sequential in
 * ascending index order with accumulators of type `real`; OpenMP only splits
 * independent rows, so results do not depend on the thread count.
 *
 * Build: ORACLE_REAL selects the arithmetic type.  `float` is the FP32 CPU
 * reference that [Roadmap] "Numerical requirements" asks for; `double` is the
 * same algorithm in FP64, used to pin it with finite differences.  Compile
 * without fast math and with -ffp-contract=off.
 *
 * Readings where the pages are silent (each one is also listed, with its
 * reason, in the repository's design notes):
 *   - a single FP32->BF16 rounding, after norm, gain and rotation (the pages
 *     allow one cast, at the kernel's declared output);
 *   - interleaved rotation pairs (2k, 2k+1); pair k belongs to axis 0 for
 *     k < 8, axis 1 for 8 <= k < 36, axis 2 otherwise;
 *   - image token (row r, col c) of an h x w grid sits at
 *     (0, r - ceil(h/2), c - ceil(w/2)); text token j sits at o+j on all three
 *     axes with o = max(floor(h/2), floor(w/2));
 *   - rotation angles are formed in FP64 and their cos/sin rounded once;
 *   - every query row (padded text rows too) is computed; the mask is on keys;
 *   - with two gain sets, set 0 is the text stream and set 1 the image stream.
 */
#include <math.h>
#include <tgmath.h> /* sqrt/exp/log follow the type of `real` */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#ifndef ORACLE_REAL
#define ORACLE_REAL float
#endif
typedef ORACLE_REAL real;

enum { HD = 128, NPAIR = 64 };

/* -------------------------------------------------------------------------
 * Precision conversions.  BF16 is the top half of an IEEE binary32.
 * ---------------------------------------------------------------------- */

/* BF16 -> real: exact (every BF16 value is representable in binary32). */
void oracle_bf16_widen(int64_t n, const uint16_t* in, real* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    out[i] = (real)f;
  }
}

/* real -> BF16 with round-to-nearest-even, one rounding of the real value.
 * Written from the definition: keep 8 significant bits of the binary value
 * (BF16 shares binary32's exponent range, so its subnormal spacing is
 * 2^-133), round the rest to nearest with ties to even, overflow to inf. */
static uint16_t bf16_rne(double x) {
  if (isnan(x)) return (uint16_t)0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e;
  (void)frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) */
  int ulp_exp = e - 8;           /* 8 significant bits */
  if (ulp_exp < -133) ulp_exp = -133;
  double q = ldexp(a, -ulp_exp); /* exact scaling */
  double fl = floor(q);
  double rem = q - fl;           /* exact */
  double rq = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) rq = fl + 1.0;
  double r = ldexp(rq, ulp_exp);
  if (r >= 0x1.0p128) return (uint16_t)(sign | 0x7F80); /* overflow */
  float f = (float)r;            /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void oracle_cast_bf16(int64_t n, const real* in, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne((double)in[i]);
}

void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_real_bytes(void) { return (int)sizeof(real); }

/* -------------------------------------------------------------------------
 * Positions  [Roadmap, "Model contract", row RoPE: image indices are centred
 * and text starts at max(h/2, w/2); Kernel list, row multi_axis_rope: text
 * tokens lie on the diagonal of the grid].
 * ---------------------------------------------------------------------- */
void oracle_positions(int T_txt, int gh, int gw, int32_t* pos /* [S][3] */) {
  int o = (gh / 2 > gw / 2) ? gh / 2 : gw / 2;
  int ch = (gh + 1) / 2, cw = (gw + 1) / 2;
  for (int j = 0; j < T_txt; ++j) {
    pos[3 * j + 0] = o + j;
    pos[3 * j + 1] = o + j;
    pos[3 * j + 2] = o + j;
  }
  for (int t = 0; t < gh * gw; ++t) {
    int row = t / gw, col = t % gw;
    int32_t* p = pos + 3 * (int64_t)(T_txt + t);
    p[0] = 0;
    p[1] = row - ch;
    p[2] = col - cw;
  }
}

/* -------------------------------------------------------------------------
 * Rotary embedding  [Roadmap, "Model contract", row RoPE: axes of 16, 56 and
 * 56 channels, theta 10000].  Pair k rotates by angle
 * p_axis * theta^(-2i/d_axis), i being the pair's index inside its axis.
 * ---------------------------------------------------------------------- */
static void pair_axis(int k, int* axis, int* i, int* d) {
  if (k < 8) { *axis = 0; *i = k; *d = 16; }
  else if (k < 36) { *axis = 1; *i = k - 8; *d = 56; }
  else { *axis = 2; *i = k - 36; *d = 56; }
}

/* cos/sin of every pair's angle for one position triple. */
static void rope_cos_sin(const int32_t* p, double theta, real* c, real* s) {
  for (int k = 0; k < NPAIR; ++k) {
    int axis, i, d;
    pair_axis(k, &axis, &i, &d);
    double omega = pow(theta, -2.0 * (double)i / (double)d);
    double phi = (double)p[axis] * omega;
    c[k] = (real)cos(phi);
    s[k] = (real)sin(phi);
  }
}

/* Rotate n_tok tokens x H heads of 128 by their positions (forward). */
void oracle_rope_apply(int64_t n_tok, int H, const int32_t* pos, double theta,
                       const real* y, real* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    real c[NPAIR], s[NPAIR];
    rope_cos_sin(pos + 3 * t, theta, c, s);
    for (int h = 0; h < H; ++h) {
      const real* a = y + (t * H + h) * HD;
      real* b = out + (t * H + h) * HD;
      for (int k = 0; k < NPAIR; ++k) {
        real y0 = a[2 * k], y1 = a[2 * k + 1];
        real p0 = y0 * c[k];
        real p1 = y1 * s[k];
        real p2 = y0 * s[k];
        real p3 = y1 * c[k];
        b[2 * k] = p0 - p1;
        b[2 * k + 1] = p2 + p3;
      }
    }
  }
}

/* -------------------------------------------------------------------------
 * RMSNorm with learned gain  [Roadmap, "Model contract", row Q/K
 * preprocessing: per-head RMSNorm with a learned gain, eps 1e-6, applied
 * before the rotation; Gain note].
 *   ms = (1/128) sum_c x_c^2 ;  r = 1/sqrt(ms + eps) ;  y_c = g_c * (x_c * r)
 * ---------------------------------------------------------------------- */
static real rms_rinv(const real* x, real eps) {
  real ss = 0;
  for (int c = 0; c < HD; ++c) {
    real sq = x[c] * x[c];
    ss = ss + sq;
  }
  real ms = ss / (real)HD;
  real den = sqrt(ms + eps);
  return (real)1 / den;
}

void oracle_rmsnorm(int64_t n_rows, const real* x, const real* gain, real eps,
                    real* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const real* a = x + r * HD;
    real rinv = rms_rinv(a, eps);
    for (int c = 0; c < HD; ++c) {
      real xh = a[c] * rinv;
      y[r * HD + c] = gain[c] * xh;
    }
  }
}

/* Gain set used by token s: set 0 = text stream, set 1 = image stream. */
static const real* gain_for(const real* gain, int gain_streams, int s, int T_txt) {
  return (gain_streams == 2 && s >= T_txt) ? gain + HD : gain;
}

/* Full prologue: y = rope(g * rmsnorm(x)), pre-cast.  x, y: [B][S][H][128]. */
void oracle_qknorm_rope(int B, int S, int H, int T_txt, int gh, int gw,
                        const real* x, const real* gain, int gain_streams,
                        double theta, real eps, real* y) {
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)S);
  oracle_positions(T_txt, gh, gw, pos);
  real* tmp = (real*)malloc(sizeof(real) * (size_t)S * H * HD);
  for (int b = 0; b < B; ++b) {
    const real* xb = x + (int64_t)b * S * H * HD;
    real* yb = y + (int64_t)b * S * H * HD;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
      const real* g = gain_for(gain, gain_streams, s, T_txt);
      for (int h = 0; h < H; ++h) {
        const real* a = xb + ((int64_t)s * H + h) * HD;
        real* t = tmp + ((int64_t)s * H + h) * HD;
        real rinv = rms_rinv(a, eps);
        for (int c = 0; c < HD; ++c) {
          real xh = a[c] * rinv;
          t[c] = g[c] * xh;
        }
      }
    }
    oracle_rope_apply(S, H, pos, theta, tmp, yb);
  }
  free(tmp);
  free(pos);
}

/* -------------------------------------------------------------------------
 * Attention  [Kernel list, rows joint_attn_qk_gemm (scores are Q K^T scaled
 * by 1/sqrt(d) over a sequence of T_txt + T_img tokens), joint_attn_softmax
 * (softmax over the keys), joint_attn_av_gemm (weights times V); Roadmap,
 * "Model contract", rows Streams (joint, non-causal, text before image) and
 * Text input (padded prompts need a key mask)].  Valid keys of a row with text
 * length L
 * are j < L and T_txt <= j < S.  Per (batch, head) slice; q, k, v are the
 * dense [S][128] rows of that slice.
 * ---------------------------------------------------------------------- */
/* A row's key set: the text keys j < L and the image keys T_txt + i with
 * img_lo <= i < img_hi.  The attention of a row uses all its image keys
 * (img_lo = 0, img_hi = S - T_txt); a key block of a split forward uses a
 * range of them, with or without the text keys. */
typedef struct { int T_txt, L, img_lo, img_hi; } keyset;
static keyset all_keys(int S, int T_txt, int L) {
  keyset ks = {T_txt, L, 0, S - T_txt};
  return ks;
}
static int key_valid(int j, keyset ks) {
  return j < ks.L || (j >= ks.T_txt + ks.img_lo && j < ks.T_txt + ks.img_hi);
}
static real softmax_scale(void) { return (real)(1.0 / sqrt((double)HD)); }

static void scores_row(int S, keyset ks, const real* qi, const real* k, real* srow) {
  real sc = softmax_scale();
  for (int j = 0; j < S; ++j) {
    if (!key_valid(j, ks)) { srow[j] = 0; continue; }
    const real* kj = k + (int64_t)j * HD;
    real dot = 0;
    for (int c = 0; c < HD; ++c) {
      real pr = qi[c] * kj[c];
      dot = dot + pr;
    }
    srow[j] = dot * sc;
  }
}

/* Softmax of one score row over the valid keys; returns the row max and
 * fills p (masked entries exactly 0) and *lse = m + log(sum exp(s - m)). */
static void softmax_row(int S, keyset ks, const real* srow, real* p, real* lse) {
  real m = -INFINITY;
  for (int j = 0; j < S; ++j)
    if (key_valid(j, ks) && srow[j] > m) m = srow[j];
  real l = 0;
  for (int j = 0; j < S; ++j) {
    if (!key_valid(j, ks)) { p[j] = 0; continue; }
    p[j] = exp(srow[j] - m);
    l = l + p[j];
  }
  for (int j = 0; j < S; ++j) p[j] = p[j] / l;
  *lse = m + log(l);
}

/* Forward of query rows [s0, s1) over the key set ks: o [s1-s0][128]
 * pre-cast, lse [s1-s0]. */
static void attn_fwd_keys(int S, keyset ks, const real* q, const real* k,
                          const real* v, int s0, int s1, real* o, real* lse) {
#pragma omp parallel
  {
    real* srow = (real*)malloc(sizeof(real) * (size_t)S);
    real* p = (real*)malloc(sizeof(real) * (size_t)S);
#pragma omp for schedule(static)
    for (int i = s0; i < s1; ++i) {
      scores_row(S, ks, q + (int64_t)i * HD, k, srow);
      softmax_row(S, ks, srow, p, &lse[i - s0]);
      real acc[HD];
      for (int c = 0; c < HD; ++c) acc[c] = 0;
      for (int j = 0; j < S; ++j) {
        if (!key_valid(j, ks)) continue;
        const real* vj = v + (int64_t)j * HD;
        for (int c = 0; c < HD; ++c) {
          real pr = p[j] * vj[c];
          acc[c] = acc[c] + pr;
        }
      }
      for (int c = 0; c < HD; ++c) o[(int64_t)(i - s0) * HD + c] = acc[c];
    }
    free(p);
    free(srow);
  }
}

/* Forward for query rows [s0, s1) over all keys of the row. */
void oracle_attn_fwd_bh(int S, int T_txt, int L, const real* q, const real* k,
                        const real* v, int s0, int s1, real* o, real* lse) {
  attn_fwd_keys(S, all_keys(S, T_txt, L), q, k, v, s0, s1, o, lse);
}

/* Forward over one key block [Kernel list, row joint_attention_fused: the
 * fused operator is marked for ring sequence parallelism, where each device
 * holds a block of the keys]: the text keys j < L when with_text, and the
 * image keys T_txt + i with img_lo <= i < img_hi.  o and lse describe
 * attention restricted to those keys. */
void oracle_attn_fwd_block_bh(int S, int T_txt, int L, int with_text, int img_lo,
                              int img_hi, const real* q, const real* k, const real* v,
                              int s0, int s1, real* o, real* lse) {
  keyset ks = {T_txt, with_text ? L : 0, img_lo, img_hi};
  attn_fwd_keys(S, ks, q, k, v, s0, s1, o, lse);
}

/* The three attention operators one at a time [Kernel list, rows
 * joint_attn_qk_gemm, joint_attn_softmax, joint_attn_av_gemm], for checking
 * each unfused operator on its own.
 *
 * Scaled scores of rows [s0, s1) over all S keys, [s1-s0][S]; masked keys 0. */
void oracle_attn_scores_bh(int S, int T_txt, int L, const real* q, const real* k,
                           int s0, int s1, real* s) {
#pragma omp parallel for schedule(static)
  for (int i = s0; i < s1; ++i)
    scores_row(S, all_keys(S, T_txt, L), q + (int64_t)i * HD, k, s + (int64_t)(i - s0) * S);
}

/* Softmax over the valid keys of n rows of scaled scores [n][S]: p [n][S]
 * (masked entries 0), lse [n]. */
void oracle_attn_softmax_rows(int n, int S, int T_txt, int L, const real* s, real* p,
                              real* lse) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i)
    softmax_row(S, all_keys(S, T_txt, L), s + (int64_t)i * S, p + (int64_t)i * S, &lse[i]);
}

/* The A.V operator of the online softmax [Kernel list, row joint_attn_av_gemm;
 * row joint_attn_softmax: the softmax runs over the key sequence in a fixed
 * tiling].  Keys of a row with text length L are split into logical tiles of
 * 64: ceil(L/64) tiles of text keys 64t .. (up to L), then the image keys
 * T_txt + 64u .. (up to S).  P[i][t][j] is the weight of key j of tile t and
 * alpha[i][t] the factor by which the operator rescales what the tiles
 * before t contributed, so tile t's contribution carries the product of the
 * factors of every later tile:
 *   o_i = ( sum_t w_t sum_j P[i][t][j] v_key(t,j) ) / l_i,
 *   w_t = prod_{u > t} alpha[i][u]   (w of the row's last tile = 1),
 * both sums in ascending t, j.  P [n][nt][64] and alpha [n][nt] for nt tile
 * slots (slots past the row's tiles, and past a tile's keys, are ignored);
 * l [n]; v [S][128]. */
void oracle_attn_av_rows(int n, int S, int T_txt, int L, int nt, const real* P,
                         const real* alpha, const real* l, const real* v, real* o) {
  const int T_img = S - T_txt;
  const int ntxt = (L + 63) / 64, nimg = (T_img + 63) / 64;
  const int ntile = ntxt + nimg < nt ? ntxt + nimg : nt;
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    real* w = (real*)malloc(sizeof(real) * (size_t)(ntile > 0 ? ntile : 1));
    for (int t = 0; t < ntile; ++t) {
      real prod = 1;
      for (int u = t + 1; u < ntile; ++u) prod = prod * alpha[(int64_t)i * nt + u];
      w[t] = prod;
    }
    real acc[HD];
    for (int c = 0; c < HD; ++c) acc[c] = 0;
    for (int t = 0; t < ntile; ++t) {
      const int first = t < ntxt ? 64 * t : T_txt + 64 * (t - ntxt);
      const int end = t < ntxt ? L : S;
      for (int j = 0; j < 64 && first + j < end; ++j) {
        const real wp = w[t] * P[((int64_t)i * nt + t) * 64 + j];
        const real* vj = v + (int64_t)(first + j) * HD;
        for (int c = 0; c < HD; ++c) {
          real pr = wp * vj[c];
          acc[c] = acc[c] + pr;
        }
      }
    }
    for (int c = 0; c < HD; ++c) o[(int64_t)i * HD + c] = acc[c] / l[i];
    free(w);
  }
}

/* Gradients of the attention slice for upstream dO ([S][128]):
 *   dP = dO V^T ; D_i = sum_c dO_ic O_ic ; dS = P o (dP - D) ;
 *   dq = dS K / sqrt(d) ; dk = dS^T Q / sqrt(d) ; dv = P^T dO.
 * O here is the oracle's own (pre-cast) output.  Masked keys get dk = dv = 0.
 * P and dS are materialised ([S][S] each) so both reductions use the same
 * values; columns are then summed in ascending query order. */
int oracle_attn_bwd_bh(int S, int T_txt, int L, const real* q, const real* k,
                       const real* v, const real* dO, real* dq, real* dk,
                       real* dv) {
  real* P = (real*)malloc(sizeof(real) * (size_t)S * S);
  real* dS = (real*)malloc(sizeof(real) * (size_t)S * S);
  if (!P || !dS) { free(P); free(dS); return 1; }
  real sc = softmax_scale();
  const keyset ks = all_keys(S, T_txt, L);
#pragma omp parallel
  {
    real* srow = (real*)malloc(sizeof(real) * (size_t)S);
#pragma omp for schedule(static)
    for (int i = 0; i < S; ++i) {
      real lse;
      real* p = P + (int64_t)i * S;
      scores_row(S, ks, q + (int64_t)i * HD, k, srow);
      softmax_row(S, ks, srow, p, &lse);
      real oi[HD];
      for (int c = 0; c < HD; ++c) oi[c] = 0;
      for (int j = 0; j < S; ++j) {
        if (!key_valid(j, ks)) continue;
        for (int c = 0; c < HD; ++c) {
          real pr = p[j] * v[(int64_t)j * HD + c];
          oi[c] = oi[c] + pr;
        }
      }
      const real* g = dO + (int64_t)i * HD;
      real Di = 0;
      for (int c = 0; c < HD; ++c) {
        real pr = g[c] * oi[c];
        Di = Di + pr;
      }
      real* ds = dS + (int64_t)i * S;
      for (int j = 0; j < S; ++j) {
        if (!key_valid(j, ks)) { ds[j] = 0; continue; }
        real dp = 0;
        for (int c = 0; c < HD; ++c) {
          real pr = g[c] * v[(int64_t)j * HD + c];
          dp = dp + pr;
        }
        ds[j] = p[j] * (dp - Di);
      }
      /* dq_ic = sum_j ds_j k_jc, each channel summed in ascending j */
      real acc[HD];
      for (int c = 0; c < HD; ++c) acc[c] = 0;
      for (int j = 0; j < S; ++j) {
        if (!key_valid(j, ks)) continue;
        for (int c = 0; c < HD; ++c) {
          real pr = ds[j] * k[(int64_t)j * HD + c];
          acc[c] = acc[c] + pr;
        }
      }
      for (int c = 0; c < HD; ++c) dq[(int64_t)i * HD + c] = acc[c] * sc;
    }
    free(srow);
  }
#pragma omp parallel for schedule(static)
  for (int j = 0; j < S; ++j) {
    real* dkj = dk + (int64_t)j * HD;
    real* dvj = dv + (int64_t)j * HD;
    if (!key_valid(j, ks)) {
      for (int c = 0; c < HD; ++c) { dkj[c] = 0; dvj[c] = 0; }
      continue;
    }
    /* dk_jc = sum_i dS_ij q_ic and dv_jc = sum_i P_ij dO_ic, each channel
     * summed in ascending query order i */
    real ak[HD], av[HD];
    for (int c = 0; c < HD; ++c) { ak[c] = 0; av[c] = 0; }
    for (int i = 0; i < S; ++i) {
      const real dsij = dS[(int64_t)i * S + j], pij = P[(int64_t)i * S + j];
      const real* qi = q + (int64_t)i * HD;
      const real* gi = dO + (int64_t)i * HD;
      for (int c = 0; c < HD; ++c) {
        real pk = dsij * qi[c];
        ak[c] = ak[c] + pk;
        real pv = pij * gi[c];
        av[c] = av[c] + pv;
      }
    }
    for (int c = 0; c < HD; ++c) {
      dkj[c] = ak[c] * sc;
      dvj[c] = av[c];
    }
  }
  free(P);
  free(dS);
  return 0;
}

/* -------------------------------------------------------------------------
 * Prologue backward  [Gain note; Roadmap, "Work items": every differentiable
 * operator comes with a forward and a backward].  For each row with upstream dy (gradient of the
 * rotated, pre-cast output; the single output cast is treated as identity):
 *   u = R^T dy ; dg += u o xhat ; dxhat = u o g ;
 *   dx = r * (dxhat - xhat * (1/128) sum_c dxhat_c xhat_c).
 * dg is per sample and per gain set: dg_per_sample [B][gain_streams][128],
 * each entry summed over (s, h) in ascending order.
 * ---------------------------------------------------------------------- */
void oracle_qknorm_rope_bwd(int B, int S, int H, int T_txt, int gh, int gw,
                            const real* x, const real* gain, int gain_streams,
                            double theta, real eps, const real* dy, real* dx,
                            real* dg_per_sample) {
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)S);
  oracle_positions(T_txt, gh, gw, pos);
  int64_t rows = (int64_t)S * H;
  real* U = (real*)malloc(sizeof(real) * (size_t)rows * HD);
  real* XH = (real*)malloc(sizeof(real) * (size_t)rows * HD);
  for (int b = 0; b < B; ++b) {
    const real* xb = x + (int64_t)b * rows * HD;
    const real* dyb = dy + (int64_t)b * rows * HD;
    real* dxb = dx + (int64_t)b * rows * HD;
#pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
      real c[NPAIR], sn[NPAIR];
      rope_cos_sin(pos + 3 * (int64_t)s, theta, c, sn);
      const real* g = gain_for(gain, gain_streams, s, T_txt);
      for (int h = 0; h < H; ++h) {
        int64_t r = (int64_t)s * H + h;
        const real* a = xb + r * HD;
        const real* d = dyb + r * HD;
        real* u = U + r * HD;
        real* xh = XH + r * HD;
        for (int k = 0; k < NPAIR; ++k) {
          real d0 = d[2 * k], d1 = d[2 * k + 1];
          real p0 = d0 * c[k];
          real p1 = d1 * sn[k];
          real p2 = d0 * sn[k];
          real p3 = d1 * c[k];
          u[2 * k] = p0 + p1;
          u[2 * k + 1] = p3 - p2;
        }
        real rinv = rms_rinv(a, eps);
        for (int cc = 0; cc < HD; ++cc) xh[cc] = a[cc] * rinv;
        real dot = 0;
        real dxh[HD];
        for (int cc = 0; cc < HD; ++cc) {
          dxh[cc] = u[cc] * g[cc];
          real pr = dxh[cc] * xh[cc];
          dot = dot + pr;
        }
        real mean = dot / (real)HD;
        for (int cc = 0; cc < HD; ++cc) {
          real t = xh[cc] * mean;
          dxb[r * HD + cc] = rinv * (dxh[cc] - t);
        }
      }
    }
    /* dg for this sample: ascending (s, h) per channel and gain set. */
    for (int st = 0; st < gain_streams; ++st) {
      real* dg = dg_per_sample + ((int64_t)b * gain_streams + st) * HD;
#pragma omp parallel for schedule(static)
      for (int cc = 0; cc < HD; ++cc) {
        real acc = 0;
        for (int s = 0; s < S; ++s) {
          int set = (gain_streams == 2 && s >= T_txt) ? 1 : 0;
          if (set != st) continue;
          for (int h = 0; h < H; ++h) {
            int64_t r = (int64_t)s * H + h;
            real pr = U[r * HD + cc] * XH[r * HD + cc];
            acc = acc + pr;
          }
        }
        dg[cc] = acc;
      }
    }
  }
  free(XH);
  free(U);
  free(pos);
}

/* -------------------------------------------------------------------------
 * Projections around the attention  [Kernel list, rows qkv_bias_gemm (the
 * packed Q/K/V projection, 3072 -> 3 x 3072 plus bias, one weight set per
 * stream) and attn_out_bias_gemm (the output projection 3072 -> 3072 plus
 * bias, per stream); Roadmap, "Model contract", row Streams: text and image
 * tokens keep separate weights].
 *
 * y[i][n] = sum_k x[i][k] W[n][k] + bias[n] for rows i of x [n_rows][K] and
 * W [N][K] (the layout of a linear layer's weight), the sum in ascending k.
 * ---------------------------------------------------------------------- */
void oracle_linear(int64_t n_rows, int K, int N, const real* x, const real* W,
                   const real* bias, real* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    const real* xi = x + i * K;
    for (int n = 0; n < N; ++n) {
      const real* wn = W + (int64_t)n * K;
      real acc = 0;
      for (int k = 0; k < K; ++k) {
        real pr = xi[k] * wn[k];
        acc = acc + pr;
      }
      y[i * N + n] = acc + bias[n];
    }
  }
}
