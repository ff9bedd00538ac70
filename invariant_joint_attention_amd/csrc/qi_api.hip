// qi_api.hip -- the C ABI declared in include/qi.h: argument validation, the
// per-device gfx950 / strict-arithmetic gate, launch configuration and the
// trace record.  No entry point allocates device memory.
//
// Pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
// ablation matrix and integration plan", "Numerical requirements" (strict
// configurations that are not supported fail closed) and "Work items"
// (qwenimage_operator_trace); [Kernel list] "[RFC] [Qwen-Image] WS1
// Single-GPU Kernel List", rules 4 and 7 (no fast math; trace records);
// [PR 537] "[WS1][Qwen-Image][CUDA] AdaLN modulation projection
// (adaln_mod_projection)": a probe kernel built with the library's own flags
// checks the arithmetic, and its verdict is kept per device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qi.h"
#include "qi_common.h"
#include "qi_kernels.h"
#include "qi_probe.h"

using namespace qi;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// ----------------------------------------------------------- validation
struct Extent {
  const char* name;
  uintptr_t lo, hi;  // byte range [lo, hi)
  bool output;
};

int check_geom(const qi_geom* g) {
  if (!g) return fail(QI_E_INVALID, "geom is null");
  if (g->D != kHeadDim) return fail(QI_E_UNSUPPORTED, "head dim %d unsupported (must be 128)", g->D);
  if (g->B < 1 || g->H < 1) return fail(QI_E_INVALID, "B=%d H=%d must be >= 1", g->B, g->H);
  if (g->T_txt < 0 || g->grid_h < 1 || g->grid_w < 1)
    return fail(QI_E_INVALID, "T_txt=%d grid=%dx%d invalid", g->T_txt, g->grid_h, g->grid_w);
  const int64_t S = (int64_t)g->T_txt + (int64_t)g->grid_h * g->grid_w;
  if (S > (1 << 24)) return fail(QI_E_INVALID, "sequence length %lld too large", (long long)S);
  if (g->rope_axes[0] != 16 || g->rope_axes[1] != 56 || g->rope_axes[2] != 56)
    return fail(QI_E_UNSUPPORTED, "rope axes {%d,%d,%d} unsupported (must be {16,56,56})", g->rope_axes[0],
                g->rope_axes[1], g->rope_axes[2]);
  if (!(std::isfinite(g->rope_theta) && g->rope_theta > 1.0))
    return fail(QI_E_INVALID, "rope_theta must be finite and > 1");
  if (!(std::isfinite(g->rms_eps) && g->rms_eps > 0.f)) return fail(QI_E_INVALID, "rms_eps must be finite and > 0");
  if (g->gain_streams != 1 && g->gain_streams != 2)
    return fail(QI_E_INVALID, "gain_streams=%d must be 1 or 2", g->gain_streams);
  if (!g->txt_len) return fail(QI_E_INVALID, "txt_len is null");
  for (int b = 0; b < g->B; ++b)
    if (g->txt_len[b] < 0 || g->txt_len[b] > g->T_txt)
      return fail(QI_E_INVALID, "txt_len[%d]=%d outside [0, %d]", b, g->txt_len[b], g->T_txt);
  return QI_OK;
}

int64_t seq_len(const qi_geom* g) { return (int64_t)g->T_txt + (int64_t)g->grid_h * g->grid_w; }

// A [B,S,H,128] view: alignment, non-negative strides, and for outputs an
// injective layout (no two elements share memory).
int check_view(const qi_geom* g, const qi_bshd& v, int elsize, bool output, const char* name,
               std::vector<Extent>& ext) {
  if (!v.data) return fail(QI_E_INVALID, "%s is null", name);
  if ((uintptr_t)v.data % 16) return fail(QI_E_ALIGN, "%s is not 16-byte aligned", name);
  const int64_t S = seq_len(g);
  const int64_t n[3] = {g->B, S, g->H};
  const int64_t st[3] = {v.sb, v.ss, v.sh};
  int64_t span = kHeadDim;  // elements reachable from the start
  for (int i = 0; i < 3; ++i) {
    if (n[i] == 1) continue;
    if (st[i] < 0) return fail(QI_E_INVALID, "%s has a negative stride", name);
    if ((st[i] * elsize) % 16) return fail(QI_E_ALIGN, "%s stride %lld is not a multiple of 16 bytes", name,
                                           (long long)st[i]);
    span += (n[i] - 1) * st[i];
  }
  if (output) {
    int idx[3] = {0, 1, 2};
    std::sort(idx, idx + 3, [&](int x, int y) { return st[x] < st[y]; });
    int64_t inner = kHeadDim;
    for (int k = 0; k < 3; ++k) {
      const int i = idx[k];
      if (n[i] == 1) continue;
      if (st[i] < inner) return fail(QI_E_ALIAS, "%s has overlapping elements (stride %lld)", name, (long long)st[i]);
      inner = st[i] * n[i];
    }
  }
  ext.push_back({name, (uintptr_t)v.data, (uintptr_t)v.data + (uintptr_t)(span * elsize), output});
  return QI_OK;
}

int check_dense(const void* p, int64_t bytes, bool output, const char* name, std::vector<Extent>& ext,
                bool nullable = false, int align = 16) {
  if (!p) return nullable ? QI_OK : fail(QI_E_INVALID, "%s is null", name);
  if ((uintptr_t)p % align) return fail(QI_E_ALIGN, "%s is not %d-byte aligned", name, align);
  ext.push_back({name, (uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, output});
  return QI_OK;
}

int check_alias(const std::vector<Extent>& ext) {
  for (size_t i = 0; i < ext.size(); ++i) {
    if (!ext[i].output) continue;
    for (size_t j = 0; j < ext.size(); ++j) {
      if (i == j || (j < i && ext[j].output)) continue;
      if (ext[i].lo < ext[j].hi && ext[j].lo < ext[i].hi)
        return fail(QI_E_ALIAS, "output %s overlaps %s", ext[i].name, ext[j].name);
    }
  }
  return QI_OK;
}

// ------------------------------------------------- device gate and probe
// Shader-clock probe for measurement: each single-wave workgroup reads the
// shader clock counter (s_memtime) and the constant-rate wall clock
// (s_memrealtime), runs `iters` rounds of four independent BF16 MFMAs (a
// matrix load like the attention kernel's), reads both again and writes
// the two differences.  Both readings of a pair come from the same wave, so
// counters of different XCDs are never subtracted from each other.
__global__ void clock_probe_kernel(unsigned long long* out, int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed * (float)(i - (int)threadIdx.x));
  }
  f32x16 acc[4] = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float sink = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) sink += acc[j][0];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    unsigned long long* o = out + 3 * (size_t)blockIdx.x;
    o[0] = t1 - t0;
    o[1] = r1 - r0;
    o[2] = (unsigned long long)__float_as_uint(sink);
  }
}

std::mutex g_mu;
std::map<int, int> g_dev_status;     // device id -> QI_OK / error code
std::map<int, std::string> g_dev_msg;

int run_probe(int dev) {
  char msg[256];
  const int rc = probe::run(dev, msg, sizeof msg);
  return rc ? fail(rc, "%s", msg) : QI_OK;
}

int gate_device(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev_status.find(dev);
  if (it != g_dev_status.end()) {
    if (it->second != QI_OK) g_err = g_dev_msg[dev];
    return it->second;
  }
  int st = QI_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    st = fail(QI_E_UNSUPPORTED, "cannot query HIP device %d", dev);
  } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    st = fail(QI_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  } else {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != dev) (void)hipSetDevice(dev);
    st = run_probe(dev);
    if (cur != dev && cur >= 0) (void)hipSetDevice(cur);
  }
  g_dev_status[dev] = st;
  g_dev_msg[dev] = st == QI_OK ? std::string() : g_err;
  return st;
}

int current_device_gate() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(QI_E_UNSUPPORTED, "no HIP device available");
  return gate_device(dev);
}

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QI_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return QI_OK;
}

template <typename T>
View<T> view_of(const qi_bshd& v, int64_t boff) {
  return View<T>{(T*)v.data + boff * v.sb, v.sb, v.ss, v.sh};
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t dvec, lse2, pq, pk, do16, amax, scale, total;
  int n_txt_chunks, n_chunks;
};

// Forward workspace: V as FP16 (v * 2^-8) transposed key tiles [B][H][nt_max][128][64].
// key tiles per (b, h) at the longest valid text: text tiles, then image tiles
int fwd_nt_max(const qi_geom* g) {
  return (int)(ceil_div(g->T_txt, kFwdBN) + ceil_div((int64_t)g->grid_h * g->grid_w, kFwdBN));
}

size_t fwd_workspace_bytes(const qi_geom* g) {
  return align256((size_t)g->B * g->H * fwd_nt_max(g) * kVtileElems * 2);
}

// The unfused operators launch a (query-row block, head, batch) grid.
int check_unfused_grid(const qi_geom* g) {
  if (g->H > 65535) return fail(QI_E_UNSUPPORTED, "H=%d above the 65535 heads the unfused operators launch", g->H);
  return QI_OK;
}
dim3 unfused_grid(const qi_geom* g, int nb, int waves) {
  return dim3((unsigned)ceil_div(seq_len(g), 32 * waves), (unsigned)g->H, (unsigned)nb);
}
void batch_txt_len(const qi_geom* g, int b0, int nb, int* dst) {
  for (int i = 0; i < kMaxBatchPerLaunch; ++i) dst[i] = i < nb ? g->txt_len[b0 + i] : 0;
}

// Projections: the input rows (a token's D = H*128 channels) must be
// contiguous, and the loads address 64 rows from one base with 32-bit
// offsets.
int check_proj_common(const qi_geom* g, qi_bshd x, const void* w, const float* bias, int32_t weight_streams,
                      int64_t N, std::vector<Extent>& ext) {
  int rc;
  if (weight_streams != 1 && weight_streams != 2)
    return fail(QI_E_INVALID, "weight_streams=%d must be 1 or 2", weight_streams);
  const int64_t D = (int64_t)g->H * kHeadDim;
  if ((rc = check_view(g, x, 2, false, "x", ext))) return rc;
  if (g->H > 1 && x.sh != kHeadDim)
    return fail(QI_E_UNSUPPORTED, "x head stride %lld: a token's %lld channels must be contiguous",
                (long long)x.sh, (long long)D);
  if (seq_len(g) > 1 && x.ss > (int64_t(1) << 25))
    return fail(QI_E_UNSUPPORTED, "x sequence stride above 2^25 elements");
  if (D > (int64_t(1) << 24)) return fail(QI_E_UNSUPPORTED, "model width %lld too large", (long long)D);
  if ((rc = check_dense(w, weight_streams * N * D * 2, false, "w", ext))) return rc;
  if ((rc = check_dense(bias, weight_streams * N * 4, false, "bias", ext))) return rc;
  return QI_OK;
}

int launch_proj(const qi_geom* g, qi_bshd x, const void* w, const float* bias, int weight_streams, int64_t N,
                int sections, const qi_bshd* outs, int fuse, const float* gain_q, const float* gain_k,
                float* rope, hipStream_t stream) {
  int rc;
  const int64_t S = seq_len(g);
  if (fuse) {
    RopeTableArgs t;
    t.table = rope;
    t.S = (int)S;
    t.T_txt = g->T_txt;
    t.gh = g->grid_h;
    t.gw = g->grid_w;
    t.theta = g->rope_theta;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)ceil_div(S * 64, 256)), dim3(256), 0, stream, t);
    if ((rc = launched("rope_table_kernel"))) return rc;
  }
  ProjArgs a;
  a.x = (const uint16_t*)x.data;
  a.x_sb = x.sb;
  a.x_ss = x.ss;
  a.w = (const uint16_t*)w;
  a.bias = bias;
  a.weight_streams = weight_streams;
  a.B = g->B;
  a.S = (int)S;
  a.T_txt = g->T_txt;
  a.K = g->H * kHeadDim;
  a.N = (int)N;
  a.D = g->H * kHeadDim;
  a.n_mt_txt = (int)ceil_div(g->T_txt, kProjTile);
  a.n_mt_img = (int)ceil_div((int64_t)g->grid_h * g->grid_w, kProjTile);
  a.n_nt = (int)ceil_div(N, kProjTile);
  for (int i = 0; i < 3; ++i) a.out[i] = view_of<uint16_t>(outs[i < sections ? i : 0], 0);
  a.fuse = fuse;
  a.gain_q = gain_q;
  a.gain_k = gain_k;
  a.gain_streams = g->gain_streams;
  a.eps = g->rms_eps;
  a.rope = rope;
  const int64_t grid = (int64_t)g->B * (a.n_mt_txt + a.n_mt_img) * a.n_nt;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)grid), dim3(kProjWaves * 64), 0, stream, a);
  return launched("proj_gemm_kernel");
}

// Query tiles per (b, h) of the dK/dV passes' frozen order (valid text,
// image, padded text; 64 rows each), at the sample that needs the most.
int bwd_nt_do(const qi_geom* g) {
  const int64_t T_img = (int64_t)g->grid_h * g->grid_w;
  int64_t n = 0;
  for (int b = 0; b < g->B; ++b) {
    const int64_t L = g->txt_len[b];
    n = std::max(n, ceil_div(L, kBwdBM) + ceil_div(T_img, kBwdBM) + ceil_div(g->T_txt - L, kBwdBM));
  }
  return (int)n;
}

BwdLayout bwd_layout(const qi_geom* g) {
  BwdLayout L;
  const int64_t S = seq_len(g);
  L.n_txt_chunks = (int)ceil_div(g->T_txt, kPrologueChunk);
  L.n_chunks = L.n_txt_chunks + (int)ceil_div((int64_t)g->grid_h * g->grid_w, kPrologueChunk);
  L.dvec = 0;
  L.lse2 = align256((size_t)g->B * g->H * S * 4);
  L.pq = L.lse2 + align256((size_t)g->B * g->H * S * 4);
  const size_t part = align256((size_t)g->B * L.n_chunks * kHeadDim * 4);
  L.pk = L.pq + part;
  L.do16 = L.pk + part;
  L.amax = L.do16 + align256((size_t)g->B * g->H * bwd_nt_do(g) * kVtileElems * 2);
  const size_t n_qtiles = (size_t)ceil_div(S, kBwdDqWaves * 32);
  L.scale = L.amax + align256((size_t)g->B * g->H * n_qtiles * kBwdDqWaves * 4);
  L.total = L.scale + align256((size_t)g->B * g->H * 4);
  return L;
}

// The state a carried key block starts from (all null: the empty state).
struct CarryIn {
  const float* acc;
  const float* m;
  const float* l;
};

// One forward call: the V tile pass and the attention kernel per batch chunk.
// With blk the partial kernel runs over that key block and writes the row
// state (acc, m, l) instead of O and LSE; with carry as well, the carried
// kernel continues the state carry holds over the block and writes the new
// state to (pacc, pm, pl), or O and LSE when pacc is null.
int launch_fwd(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd* o_p, float* lse, float* o_f32,
               uint16_t* vt, const qi_key_block* blk, float* pacc, float* pm, float* pl, hipStream_t stream,
               bool vt_ready = false, const CarryIn* carry = nullptr) {
  int rc;
  const int64_t S = seq_len(geom);
  // vt: FP16 V^T key tiles [B][H][nt_max][128][64] in the workspace
  const int nt_max = fwd_nt_max(geom);
  const int rows_per_wg = kFwdWaves * kFwdRowsPerWave;
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    FwdArgs a;
    a.q = view_of<const uint16_t>(q, b0);
    a.k = view_of<const uint16_t>(k, b0);
    a.vt = vt + (int64_t)b0 * geom->H * nt_max * kVtileElems;
    a.o = o_p ? view_of<uint16_t>(*o_p, b0) : View<uint16_t>{nullptr, 0, 0, 0};
    a.lse = lse ? lse + (int64_t)b0 * geom->H * S : nullptr;
    a.of = o_f32 ? o_f32 + (int64_t)b0 * S * geom->H * kHeadDim : nullptr;
    const int64_t r0 = (int64_t)b0 * geom->H * S;
    a.blk_text = blk ? blk->include_text : 1;
    a.blk_img_t0 = blk ? blk->img_begin / kFwdBN : 0;
    a.blk_img_t1 = blk ? (int)ceil_div(blk->img_end, kFwdBN) : 0;
    const int64_t l_words = carry ? 2 : 1;  // carried states keep a row sum per half-wave
    a.pacc = pacc ? pacc + r0 * kHeadDim : nullptr;
    a.pm = pm ? pm + r0 : nullptr;
    a.pl = pl ? pl + r0 * l_words : nullptr;
    const bool cin = carry && carry->acc;
    a.cin_acc = cin ? carry->acc + r0 * kHeadDim : nullptr;
    a.cin_m = cin ? carry->m + r0 : nullptr;
    a.cin_l = cin ? carry->l + r0 * 2 : nullptr;
    a.B = nb;
    a.S = (int)S;
    a.H = geom->H;
    a.T_txt = geom->T_txt;
    a.T_img = geom->grid_h * geom->grid_w;
    a.nt_max = nt_max;
    a.n_qtiles = (int)ceil_div(S, rows_per_wg);
    a.xcd_remap = ((nb * geom->H) % 8) == 0;
    for (int i = 0; i < kMaxBatchPerLaunch; ++i) a.txt_len[i] = i < nb ? geom->txt_len[b0 + i] : 0;

    VtileArgs c;
    c.v = view_of<const uint16_t>(v, b0);
    c.out = const_cast<uint16_t*>(a.vt);
    c.H = geom->H;
    c.T_txt = geom->T_txt;
    c.T_img = a.T_img;
    c.nt_max = nt_max;
    for (int i = 0; i < kMaxBatchPerLaunch; ++i) c.txt_len[i] = a.txt_len[i];
    c.with_text = a.blk_text;
    c.img_t0 = blk ? a.blk_img_t0 : 0;
    c.img_t1 = blk ? a.blk_img_t1 : nt_max;
    if (!vt_ready) {
      hipLaunchKernelGGL(v_tiles_kernel, dim3((unsigned)nt_max, (unsigned)geom->H, (unsigned)nb), dim3(256), 0,
                         stream, c);
      if ((rc = launched("v_tiles_kernel"))) return rc;
    }

    const int64_t grid = (int64_t)nb * geom->H * a.n_qtiles;
    if (carry) {
      hipLaunchKernelGGL(attn_fwd_carry_kernel, dim3((unsigned)grid), dim3(kFwdWaves * 64), 0, stream, a);
      if ((rc = launched("attn_fwd_carry_kernel"))) return rc;
    } else if (blk) {
      hipLaunchKernelGGL(attn_fwd_partial_kernel, dim3((unsigned)grid), dim3(kFwdWaves * 64), 0, stream, a);
      if ((rc = launched("attn_fwd_partial_kernel"))) return rc;
    } else {
      hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(kFwdWaves * 64), 0, stream, a);
      if ((rc = launched("attn_fwd_kernel"))) return rc;
    }
  }
  return QI_OK;
}

PrologueArgs prologue_args(const qi_geom* g, qi_bshd x, const float* gain, qi_bshd y, float* yf, int b0, int nb) {
  PrologueArgs a;
  a.x = view_of<const uint16_t>(x, b0);
  a.y = view_of<uint16_t>(y, b0);
  a.yf = yf;
  a.gain = gain;
  a.gain_streams = g->gain_streams;
  a.B = nb;
  a.S = (int)seq_len(g);
  a.H = g->H;
  a.T_txt = g->T_txt;
  a.gh = g->grid_h;
  a.gw = g->grid_w;
  a.theta = g->rope_theta;
  a.eps = g->rms_eps;
  return a;
}

int launch_prologue(const qi_geom* g, qi_bshd x, const float* gain, qi_bshd y, float* yf, hipStream_t st) {
  PrologueArgs a;
  a.x = view_of<const uint16_t>(x, 0);
  a.y = view_of<uint16_t>(y, 0);
  a.yf = yf;
  a.gain = gain;
  a.gain_streams = g->gain_streams;
  a.B = g->B;
  a.S = (int)seq_len(g);
  a.H = g->H;
  a.T_txt = g->T_txt;
  a.gh = g->grid_h;
  a.gw = g->grid_w;
  a.theta = g->rope_theta;
  a.eps = g->rms_eps;
  const int64_t tokens = (int64_t)a.B * a.S;
  hipLaunchKernelGGL(qknorm_rope_fwd_kernel, dim3((unsigned)ceil_div(tokens, 4)), dim3(256), 0, st, a);
  return launched("qknorm_rope_fwd_kernel");
}

// The prologue backward of both gradients (t = 0: q, 1: k) in one launch,
// then both gain folds in one launch.
int launch_prologue_bwd(const qi_geom* g, const qi_bshd x[2], const float* const gain[2], const qi_bshd dx[2],
                        float* const partials[2], float* const dg_ps[2], float* const dg[2], const BwdLayout& Lw,
                        hipStream_t st) {
  PrologueBwdPair pp;
  DgainFoldPair fp;
  for (int t = 0; t < 2; ++t) {
    PrologueBwdArgs& a = pp.t[t];
    a.x = view_of<const uint16_t>(x[t], 0);
    a.dx = view_of<float>(dx[t], 0);
    a.gain = gain[t];
    a.partials = partials[t];
    a.gain_streams = g->gain_streams;
    a.B = g->B;
    a.S = (int)seq_len(g);
    a.H = g->H;
    a.T_txt = g->T_txt;
    a.gh = g->grid_h;
    a.gw = g->grid_w;
    a.n_txt_chunks = Lw.n_txt_chunks;
    a.n_chunks = Lw.n_chunks;
    a.theta = g->rope_theta;
    a.eps = g->rms_eps;
    DgainFoldArgs& f = fp.t[t];
    f.partials = partials[t];
    f.dg_ps = dg_ps[t];
    f.dg = dg[t];
    f.B = g->B;
    f.gain_streams = g->gain_streams;
    f.n_txt_chunks = Lw.n_txt_chunks;
    f.n_chunks = Lw.n_chunks;
  }
  hipLaunchKernelGGL(qknorm_rope_bwd_kernel, dim3(Lw.n_chunks, g->B, 2), dim3(256), 0, st, pp);
  int rc = launched("qknorm_rope_bwd_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(dgain_fold_kernel, dim3(g->gain_streams, 2), dim3(4 * kHeadDim), 0, st, fp);
  return launched("dgain_fold_kernel");
}

// Argument checks shared by the two whole-row forward entry points.
int check_fwd_io(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd o, float* lse, float* o_f32,
                 std::vector<Extent>& ext) {
  int rc = check_geom(geom);
  if (rc) return rc;
  const int64_t S = seq_len(geom);
  const int64_t n = (int64_t)geom->B * S * geom->H * kHeadDim;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  if ((rc = check_view(geom, o, 2, true, "o", ext))) return rc;
  if ((rc = check_dense(lse, (int64_t)geom->B * geom->H * S * 4, true, "lse", ext))) return rc;
  if ((rc = check_dense(o_f32, n * 4, true, "o_f32", ext, true))) return rc;
  if (S > 1 && k.ss > kFwdMaxRowStride)
    return fail(QI_E_UNSUPPORTED, "k sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  return QI_OK;
}

// Static scratch of qi_joint_attn_fwd_noalloc: the V tiles the forward
// otherwise keeps in the caller's workspace.  Each device holds its own copy
// for the life of the process.  In host code `scratch` only names the
// symbol; its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is passed to
// kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::map<int, void*> g_scratch_ptr;  // device id -> device address of `scratch`

int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(QI_E_UNSUPPORTED, "no HIP device available");
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QI_E_HIP, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                  hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return QI_OK;
}

}  // namespace

// ================================================================ C ABI
extern "C" {

const char* qi_last_error(void) { return g_err.c_str(); }

int qi_strict_probe(int device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n)
    return fail(QI_E_UNSUPPORTED, "HIP device %d not available", device);
  return gate_device(device);
}

int qi_qknorm_rope(const qi_geom* geom, qi_bshd x, const float* gain, qi_bshd y, float* y_f32,
                   hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom);
  const int64_t n = (int64_t)geom->B * S * geom->H * kHeadDim;
  if ((rc = check_view(geom, x, 2, false, "x", ext))) return rc;
  if ((rc = check_dense(gain, (int64_t)geom->gain_streams * kHeadDim * 4, false, "gain", ext))) return rc;
  if ((rc = check_view(geom, y, 2, true, "y", ext))) return rc;
  if ((rc = check_dense(y_f32, n * 4, true, "y_f32", ext, true))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;
  return launch_prologue(geom, x, gain, y, y_f32, stream);
}

size_t qi_joint_attn_fwd_workspace(const qi_geom* geom) {
  if (check_geom(geom)) return 0;
  return fwd_workspace_bytes(geom);
}

int qi_joint_attn_fwd(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd o, float* lse,
                      float* o_f32, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  std::vector<Extent> ext;
  int rc = check_fwd_io(geom, q, k, v, o, lse, o_f32, ext);
  if (rc) return rc;
  const size_t ws_need = fwd_workspace_bytes(geom);
  if (!workspace) return fail(QI_E_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(QI_E_ALIGN, "workspace is not 256-byte aligned");
  if (workspace_bytes < ws_need)
    return fail(QI_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, ws_need);
  ext.push_back({"workspace", (uintptr_t)workspace, (uintptr_t)workspace + ws_need, true});
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;

  return launch_fwd(geom, q, k, v, &o, lse, o_f32, (uint16_t*)workspace, nullptr, nullptr, nullptr, nullptr, stream);
}

int qi_joint_attn_fwd_noalloc(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_bshd o, float* lse,
                              float* o_f32, hipStream_t stream) {
  std::vector<Extent> ext;
  int rc = check_fwd_io(geom, q, k, v, o, lse, o_f32, ext);
  if (rc) return rc;
  const size_t ws_need = fwd_workspace_bytes(geom);
  if (ws_need > kNoAllocScratchBytes)
    return fail(QI_E_WORKSPACE,
                "this geometry needs %zu bytes of V tiles, more than the %zu-byte static scratch of "
                "qi_joint_attn_fwd_noalloc; use qi_joint_attn_fwd with a workspace",
                ws_need, (size_t)kNoAllocScratchBytes);
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;
  void* scratch_dev = nullptr;
  if ((rc = noalloc_scratch(&scratch_dev))) return rc;
  return launch_fwd(geom, q, k, v, &o, lse, o_f32, (uint16_t*)scratch_dev, nullptr, nullptr, nullptr, nullptr, stream);
}

int qi_qkv_prologue(const qi_geom* geom, qi_bshd q_raw, qi_bshd k_raw, qi_bshd v, const float* gain_q,
                    const float* gain_k, qi_bshd q, qi_bshd k, void* v_tiles, size_t v_tiles_bytes,
                    hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom);
  const int64_t gbytes = (int64_t)geom->gain_streams * kHeadDim * 4;
  if ((rc = check_view(geom, q_raw, 2, false, "q_raw", ext))) return rc;
  if ((rc = check_view(geom, k_raw, 2, false, "k_raw", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  if ((rc = check_dense(gain_q, gbytes, false, "gain_q", ext))) return rc;
  if ((rc = check_dense(gain_k, gbytes, false, "gain_k", ext))) return rc;
  if ((rc = check_view(geom, q, 2, true, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, true, "k", ext))) return rc;
  const size_t vt_need = fwd_workspace_bytes(geom);
  if (!v_tiles) return fail(QI_E_WORKSPACE, "v_tiles is null");
  if ((uintptr_t)v_tiles % 256) return fail(QI_E_ALIGN, "v_tiles is not 256-byte aligned");
  if (v_tiles_bytes < vt_need)
    return fail(QI_E_WORKSPACE, "v_tiles of %zu bytes is smaller than the %zu required", v_tiles_bytes, vt_need);
  ext.push_back({"v_tiles", (uintptr_t)v_tiles, (uintptr_t)v_tiles + vt_need, true});
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;

  const int nt_max = fwd_nt_max(geom);
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    QkvPrologueArgs a;
    a.q = prologue_args(geom, q_raw, gain_q, q, nullptr, b0, nb);
    a.k = prologue_args(geom, k_raw, gain_k, k, nullptr, b0, nb);
    a.nblk = ceil_div((int64_t)nb * S, 4);
    a.v.v = view_of<const uint16_t>(v, b0);
    a.v.out = (uint16_t*)v_tiles + (int64_t)b0 * geom->H * nt_max * kVtileElems;
    a.v.H = geom->H;
    a.v.T_txt = geom->T_txt;
    a.v.T_img = geom->grid_h * geom->grid_w;
    a.v.nt_max = nt_max;
    for (int i = 0; i < kMaxBatchPerLaunch; ++i) a.v.txt_len[i] = i < nb ? geom->txt_len[b0 + i] : 0;
    a.v.with_text = 1;
    a.v.img_t0 = 0;
    a.v.img_t1 = nt_max;
    const int64_t grid = 2 * a.nblk + (int64_t)nt_max * geom->H * nb;
    if (grid > 0x7fffffff) return fail(QI_E_UNSUPPORTED, "%lld workgroups in one prologue launch", (long long)grid);
    hipLaunchKernelGGL(qkv_prologue_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    if ((rc = launched("qkv_prologue_kernel"))) return rc;
  }
  return QI_OK;
}

int qi_joint_attn_fwd_vtiles(const qi_geom* geom, qi_bshd q, qi_bshd k, const void* v_tiles, size_t v_tiles_bytes,
                             qi_bshd o, float* lse, float* o_f32, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom);
  const int64_t n = (int64_t)geom->B * S * geom->H * kHeadDim;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_view(geom, o, 2, true, "o", ext))) return rc;
  if ((rc = check_dense(lse, (int64_t)geom->B * geom->H * S * 4, true, "lse", ext))) return rc;
  if ((rc = check_dense(o_f32, n * 4, true, "o_f32", ext, true))) return rc;
  const size_t vt_need = fwd_workspace_bytes(geom);
  if (!v_tiles) return fail(QI_E_WORKSPACE, "v_tiles is null");
  if ((uintptr_t)v_tiles % 256) return fail(QI_E_ALIGN, "v_tiles is not 256-byte aligned");
  if (v_tiles_bytes < vt_need)
    return fail(QI_E_WORKSPACE, "v_tiles of %zu bytes is smaller than the %zu required", v_tiles_bytes, vt_need);
  ext.push_back({"v_tiles", (uintptr_t)v_tiles, (uintptr_t)v_tiles + vt_need, false});
  if ((rc = check_alias(ext))) return rc;
  if (S > 1 && k.ss > kFwdMaxRowStride)
    return fail(QI_E_UNSUPPORTED, "k sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  if ((rc = current_device_gate())) return rc;
  const qi_bshd no_v{nullptr, 0, 0, 0};
  return launch_fwd(geom, q, k, no_v, &o, lse, o_f32, (uint16_t*)v_tiles, nullptr, nullptr, nullptr, nullptr, stream,
                    true);
}

int check_key_block(const qi_geom* geom, const qi_key_block& blk) {
  const int64_t T_img = (int64_t)geom->grid_h * geom->grid_w;
  if (blk.include_text != 0 && blk.include_text != 1)
    return fail(QI_E_INVALID, "include_text=%d must be 0 or 1", blk.include_text);
  if (blk.img_begin < 0 || blk.img_begin > blk.img_end || blk.img_end > T_img)
    return fail(QI_E_INVALID, "image key range [%d, %d) outside [0, %lld]", blk.img_begin, blk.img_end,
                (long long)T_img);
  if (blk.img_begin % kFwdBN || (blk.img_end % kFwdBN && blk.img_end != T_img))
    return fail(QI_E_INVALID, "image key range [%d, %d) is not aligned to the 64-key tiles", blk.img_begin,
                blk.img_end);
  if (!blk.include_text && blk.img_begin == blk.img_end) return fail(QI_E_INVALID, "empty key block");
  return QI_OK;
}

int check_workspace(const qi_geom* geom, void* workspace, size_t workspace_bytes, std::vector<Extent>& ext) {
  const size_t ws_need = fwd_workspace_bytes(geom);
  if (!workspace) return fail(QI_E_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(QI_E_ALIGN, "workspace is not 256-byte aligned");
  if (workspace_bytes < ws_need)
    return fail(QI_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, ws_need);
  ext.push_back({"workspace", (uintptr_t)workspace, (uintptr_t)workspace + ws_need, true});
  return QI_OK;
}

int qi_joint_attn_fwd_partial(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_key_block blk, float* acc,
                              float* m, float* l, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  if ((rc = check_key_block(geom, blk))) return rc;
  const int64_t S = seq_len(geom);
  std::vector<Extent> ext;
  const int64_t rows = (int64_t)geom->B * geom->H * S;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  if ((rc = check_dense(acc, rows * kHeadDim * 4, true, "acc", ext))) return rc;
  if ((rc = check_dense(m, rows * 4, true, "m", ext, false, 4))) return rc;  // one word per row
  if ((rc = check_dense(l, rows * 4, true, "l", ext, false, 4))) return rc;
  if ((rc = check_workspace(geom, workspace, workspace_bytes, ext))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if (S > 1 && k.ss > kFwdMaxRowStride)
    return fail(QI_E_UNSUPPORTED, "k sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  if ((rc = current_device_gate())) return rc;
  return launch_fwd(geom, q, k, v, nullptr, nullptr, nullptr, (uint16_t*)workspace, &blk, acc, m, l, stream);
}

int qi_joint_attn_fwd_carry(const qi_geom* geom, qi_bshd q, qi_bshd k, qi_bshd v, qi_key_block blk,
                            const float* acc_in, const float* m_in, const float* l_in, float* acc_out, float* m_out,
                            float* l_out, qi_bshd o, float* lse, float* o_f32, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  if ((rc = check_key_block(geom, blk))) return rc;
  const int n_in = !!acc_in + !!m_in + !!l_in, n_out = !!acc_out + !!m_out + !!l_out;
  if (n_in % 3) return fail(QI_E_INVALID, "acc_in, m_in and l_in must be all null or all given");
  if (n_out % 3) return fail(QI_E_INVALID, "acc_out, m_out and l_out must be all null or all given");
  const bool last = n_out == 0;
  if (!last && (o.data || lse || o_f32))
    return fail(QI_E_INVALID, "o, lse and o_f32 are written by the last block only (acc_out null)");
  if (last && !n_in && blk.img_begin == blk.img_end)
    for (int b = 0; b < geom->B; ++b)
      if (geom->txt_len[b] == 0)
        return fail(QI_E_INVALID, "sample %d has no key in a single text-only block", b);
  const int64_t S = seq_len(geom);
  const int64_t rows = (int64_t)geom->B * geom->H * S;
  std::vector<Extent> ext;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  // A state may be continued in place (the same buffer in and out): each row
  // reads its own state before it writes it.
  const float* ins[3] = {acc_in, m_in, l_in};
  float* outs[3] = {acc_out, m_out, l_out};
  const int64_t bytes[3] = {rows * kHeadDim * 4, rows * 4, rows * 2 * 4};
  const char* in_names[3] = {"acc_in", "m_in", "l_in"};
  const char* out_names[3] = {"acc_out", "m_out", "l_out"};
  const int word[3] = {16, 4, 8};
  for (int i = 0; i < 3; ++i) {
    if (outs[i] && (rc = check_dense(outs[i], bytes[i], true, out_names[i], ext, false, word[i]))) return rc;
    if (ins[i] && ins[i] != outs[i] && (rc = check_dense(ins[i], bytes[i], false, in_names[i], ext, false, word[i])))
      return rc;
  }
  if (last) {
    if ((rc = check_view(geom, o, 2, true, "o", ext))) return rc;
    if ((rc = check_dense(lse, rows * 4, true, "lse", ext))) return rc;
    if ((rc = check_dense(o_f32, rows * kHeadDim * 4, true, "o_f32", ext, true))) return rc;
  }
  if ((rc = check_workspace(geom, workspace, workspace_bytes, ext))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if (S > 1 && k.ss > kFwdMaxRowStride)
    return fail(QI_E_UNSUPPORTED, "k sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  if ((rc = current_device_gate())) return rc;
  const CarryIn carry{acc_in, m_in, l_in};
  return launch_fwd(geom, q, k, v, last ? &o : nullptr, lse, o_f32, (uint16_t*)workspace, &blk, acc_out, m_out,
                    l_out, stream, false, &carry);
}

int qi_joint_attn_merge(const qi_geom* geom, int32_t n_blocks, const float* acc, const float* m, const float* l,
                        qi_bshd o, float* lse, float* o_f32, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  if (n_blocks < 1 || n_blocks > kMaxMergeBlocks)
    return fail(QI_E_INVALID, "n_blocks=%d outside [1, %d]", n_blocks, kMaxMergeBlocks);
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom);
  const int64_t rows = (int64_t)geom->B * geom->H * S;
  if ((rc = check_dense(acc, n_blocks * rows * kHeadDim * 4, false, "acc", ext))) return rc;
  if ((rc = check_dense(m, n_blocks * rows * 4, false, "m", ext, false, 4))) return rc;
  if ((rc = check_dense(l, n_blocks * rows * 4, false, "l", ext, false, 4))) return rc;
  if ((rc = check_view(geom, o, 2, true, "o", ext))) return rc;
  if ((rc = check_dense(lse, rows * 4, true, "lse", ext))) return rc;
  if ((rc = check_dense(o_f32, rows * kHeadDim * 4, true, "o_f32", ext, true))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;
  MergeArgs a;
  a.acc = acc;
  a.m = m;
  a.l = l;
  a.rows = rows;
  a.o = view_of<uint16_t>(o, 0);
  a.lse = lse;
  a.of = o_f32;
  a.n = n_blocks;
  a.S = (int)S;
  a.H = geom->H;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)ceil_div(rows, 8)), dim3(256), 0, stream, a);
  return launched("attn_merge_kernel");
}

size_t qi_qkv_proj_workspace(const qi_geom* geom) {
  if (check_geom(geom)) return 0;
  return align256((size_t)seq_len(geom) * 64 * 2 * 4);
}

int qi_qkv_proj(const qi_geom* geom, qi_bshd x, const void* w, const float* bias, int32_t weight_streams,
                const float* gain_q, const float* gain_k, int32_t fuse_prologue, qi_bshd q, qi_bshd k, qi_bshd v,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  if (fuse_prologue != 0 && fuse_prologue != 1)
    return fail(QI_E_INVALID, "fuse_prologue=%d must be 0 or 1", fuse_prologue);
  const int64_t D = (int64_t)geom->H * kHeadDim, N = 3 * D;
  std::vector<Extent> ext;
  if ((rc = check_proj_common(geom, x, w, bias, weight_streams, N, ext))) return rc;
  const int64_t gbytes = (int64_t)geom->gain_streams * kHeadDim * 4;
  if (fuse_prologue) {
    if ((rc = check_dense(gain_q, gbytes, false, "gain_q", ext))) return rc;
    if ((rc = check_dense(gain_k, gbytes, false, "gain_k", ext))) return rc;
  }
  if ((rc = check_view(geom, q, 2, true, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, true, "k", ext))) return rc;
  if ((rc = check_view(geom, v, 2, true, "v", ext))) return rc;
  const size_t ws_need = fuse_prologue ? qi_qkv_proj_workspace(geom) : 0;
  if (fuse_prologue) {
    if (!workspace) return fail(QI_E_WORKSPACE, "workspace is null");
    if ((uintptr_t)workspace % 256) return fail(QI_E_ALIGN, "workspace is not 256-byte aligned");
    if (workspace_bytes < ws_need)
      return fail(QI_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, ws_need);
    ext.push_back({"workspace", (uintptr_t)workspace, (uintptr_t)workspace + ws_need, true});
  }
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;
  const qi_bshd outs[3] = {q, k, v};
  return launch_proj(geom, x, w, bias, weight_streams, N, 3, outs, fuse_prologue, gain_q, gain_k,
                     (float*)workspace, stream);
}

int qi_attn_out_proj(const qi_geom* geom, qi_bshd o, const void* w, const float* bias, int32_t weight_streams,
                     qi_bshd y, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  const int64_t D = (int64_t)geom->H * kHeadDim;
  std::vector<Extent> ext;
  if ((rc = check_proj_common(geom, o, w, bias, weight_streams, D, ext))) return rc;
  if ((rc = check_view(geom, y, 2, true, "y", ext))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if ((rc = current_device_gate())) return rc;
  const qi_bshd outs[3] = {y, y, y};
  return launch_proj(geom, o, w, bias, weight_streams, D, 1, outs, 0, nullptr, nullptr, nullptr, stream);
}

int64_t qi_joint_attn_key_slots(const qi_geom* geom) {
  if (check_geom(geom)) return 0;
  return (int64_t)fwd_nt_max(geom) * kFwdBN;
}

int qi_joint_attn_qk_gemm(const qi_geom* geom, qi_bshd q, qi_bshd k, float* scores, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom), Kp = (int64_t)fwd_nt_max(geom) * kFwdBN;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_dense(scores, (int64_t)geom->B * geom->H * S * Kp * 4, true, "scores", ext))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if ((rc = check_unfused_grid(geom))) return rc;
  if (S > 1 && k.ss > kFwdMaxRowStride)
    return fail(QI_E_UNSUPPORTED, "k sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  if ((rc = current_device_gate())) return rc;
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    QkArgs a;
    a.q = view_of<const uint16_t>(q, b0);
    a.k = view_of<const uint16_t>(k, b0);
    a.s = scores + (int64_t)b0 * geom->H * S * Kp;
    a.S = (int)S;
    a.H = geom->H;
    a.T_txt = geom->T_txt;
    a.T_img = geom->grid_h * geom->grid_w;
    a.nt_max = fwd_nt_max(geom);
    batch_txt_len(geom, b0, nb, a.txt_len);
    hipLaunchKernelGGL(attn_qk_kernel, unfused_grid(geom, nb, kQkWaves), dim3(64 * kQkWaves), 0, stream, a);
    if ((rc = launched("attn_qk_kernel"))) return rc;
  }
  return QI_OK;
}

int qi_joint_attn_softmax(const qi_geom* geom, const float* scores, void* p, float* alpha, float* l, float* lse,
                          hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom), nt_max = fwd_nt_max(geom), Kp = nt_max * kFwdBN;
  const int64_t rows = (int64_t)geom->B * geom->H * S;
  if ((rc = check_dense(scores, rows * Kp * 4, false, "scores", ext))) return rc;
  if ((rc = check_dense(p, rows * Kp * 2, true, "p", ext))) return rc;
  if ((rc = check_dense(alpha, rows * nt_max * 4, true, "alpha", ext))) return rc;
  if ((rc = check_dense(l, rows * 4, true, "l", ext))) return rc;
  if ((rc = check_dense(lse, rows * 4, true, "lse", ext))) return rc;
  if ((rc = check_alias(ext))) return rc;
  if ((rc = check_unfused_grid(geom))) return rc;
  if ((rc = current_device_gate())) return rc;
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    const int64_t r0 = (int64_t)b0 * geom->H * S;
    SoftmaxArgs a;
    a.s = scores + r0 * Kp;
    a.p = (uint16_t*)p + r0 * Kp;
    a.alpha = alpha + r0 * nt_max;
    a.l = l + r0;
    a.lse = lse + r0;
    a.S = (int)S;
    a.H = geom->H;
    a.T_txt = geom->T_txt;
    a.T_img = geom->grid_h * geom->grid_w;
    a.nt_max = (int)nt_max;
    batch_txt_len(geom, b0, nb, a.txt_len);
    hipLaunchKernelGGL(attn_softmax_kernel, unfused_grid(geom, nb, kSoftmaxWaves), dim3(64 * kSoftmaxWaves), 0, stream,
                       a);
    if ((rc = launched("attn_softmax_kernel"))) return rc;
  }
  return QI_OK;
}

int qi_joint_attn_av_gemm(const qi_geom* geom, const void* p, const float* alpha, const float* l, qi_bshd v,
                          qi_bshd o, float* o_f32, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom), nt_max = fwd_nt_max(geom), Kp = nt_max * kFwdBN;
  const int64_t rows = (int64_t)geom->B * geom->H * S;
  const int64_t n = (int64_t)geom->B * S * geom->H * kHeadDim;
  if ((rc = check_dense(p, rows * Kp * 2, false, "p", ext))) return rc;
  if ((rc = check_dense(alpha, rows * nt_max * 4, false, "alpha", ext))) return rc;
  if ((rc = check_dense(l, rows * 4, false, "l", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  if ((rc = check_view(geom, o, 2, true, "o", ext))) return rc;
  if ((rc = check_dense(o_f32, n * 4, true, "o_f32", ext, true))) return rc;
  const size_t ws_need = fwd_workspace_bytes(geom);
  if (!workspace) return fail(QI_E_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(QI_E_ALIGN, "workspace is not 256-byte aligned");
  if (workspace_bytes < ws_need)
    return fail(QI_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, ws_need);
  ext.push_back({"workspace", (uintptr_t)workspace, (uintptr_t)workspace + ws_need, true});
  if ((rc = check_alias(ext))) return rc;
  if ((rc = check_unfused_grid(geom))) return rc;
  if ((rc = current_device_gate())) return rc;
  uint16_t* vt = (uint16_t*)workspace;
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    const int64_t r0 = (int64_t)b0 * geom->H * S;
    AvArgs a;
    a.p = (const uint16_t*)p + r0 * Kp;
    a.alpha = alpha + r0 * nt_max;
    a.l = l + r0;
    a.vt = vt + (int64_t)b0 * geom->H * nt_max * kVtileElems;
    a.o = view_of<uint16_t>(o, b0);
    a.of = o_f32 ? o_f32 + (int64_t)b0 * S * geom->H * kHeadDim : nullptr;
    a.S = (int)S;
    a.H = geom->H;
    a.T_txt = geom->T_txt;
    a.T_img = geom->grid_h * geom->grid_w;
    a.nt_max = (int)nt_max;
    batch_txt_len(geom, b0, nb, a.txt_len);

    VtileArgs c;
    c.v = view_of<const uint16_t>(v, b0);
    c.out = const_cast<uint16_t*>(a.vt);
    c.H = geom->H;
    c.T_txt = geom->T_txt;
    c.T_img = a.T_img;
    c.nt_max = (int)nt_max;
    for (int i = 0; i < kMaxBatchPerLaunch; ++i) c.txt_len[i] = a.txt_len[i];
    c.with_text = 1;
    c.img_t0 = 0;
    c.img_t1 = (int)nt_max;
    hipLaunchKernelGGL(v_tiles_kernel, dim3((unsigned)nt_max, (unsigned)geom->H, (unsigned)nb), dim3(256), 0, stream,
                       c);
    if ((rc = launched("v_tiles_kernel"))) return rc;
    hipLaunchKernelGGL(attn_av_kernel, unfused_grid(geom, nb, kAvWaves), dim3(64 * kAvWaves), 0, stream, a);
    if ((rc = launched("attn_av_kernel"))) return rc;
  }
  return QI_OK;
}

size_t qi_joint_attn_bwd_workspace(const qi_geom* geom) {
  if (check_geom(geom)) return 0;
  return bwd_layout(geom).total;
}

int qi_joint_attn_bwd(const qi_geom* geom, qi_bshd q_raw, qi_bshd k_raw, qi_bshd q, qi_bshd k, qi_bshd v,
                      qi_bshd o_f32, const float* lse, qi_bshd d_o, const float* gain_q, const float* gain_k,
                      qi_bshd dq, qi_bshd dk, qi_bshd dv, float* dgain_q_ps, float* dgain_k_ps,
                      float* dgain_q, float* dgain_k, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  int rc = check_geom(geom);
  if (rc) return rc;
  std::vector<Extent> ext;
  const int64_t S = seq_len(geom);
  const int64_t gbytes = (int64_t)geom->gain_streams * kHeadDim * 4;
  if ((rc = check_view(geom, q_raw, 2, false, "q_raw", ext))) return rc;
  if ((rc = check_view(geom, k_raw, 2, false, "k_raw", ext))) return rc;
  if ((rc = check_view(geom, q, 2, false, "q", ext))) return rc;
  if ((rc = check_view(geom, k, 2, false, "k", ext))) return rc;
  if ((rc = check_view(geom, v, 2, false, "v", ext))) return rc;
  if ((rc = check_view(geom, o_f32, 4, false, "o_f32", ext))) return rc;
  if ((rc = check_dense(lse, (int64_t)geom->B * geom->H * S * 4, false, "lse", ext))) return rc;
  if ((rc = check_view(geom, d_o, 2, false, "d_o", ext))) return rc;
  if ((rc = check_dense(gain_q, gbytes, false, "gain_q", ext))) return rc;
  if ((rc = check_dense(gain_k, gbytes, false, "gain_k", ext))) return rc;
  if ((rc = check_view(geom, dq, 4, true, "dq", ext))) return rc;
  if ((rc = check_view(geom, dk, 4, true, "dk", ext))) return rc;
  if ((rc = check_view(geom, dv, 4, true, "dv", ext))) return rc;
  if ((rc = check_dense(dgain_q_ps, geom->B * gbytes, true, "dgain_q_ps", ext))) return rc;
  if ((rc = check_dense(dgain_k_ps, geom->B * gbytes, true, "dgain_k_ps", ext))) return rc;
  if ((rc = check_dense(dgain_q, gbytes, true, "dgain_q", ext, true))) return rc;
  if ((rc = check_dense(dgain_k, gbytes, true, "dgain_k", ext, true))) return rc;
  const BwdLayout Lw = bwd_layout(geom);
  if (!workspace) return fail(QI_E_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(QI_E_ALIGN, "workspace is not 256-byte aligned");
  if (workspace_bytes < Lw.total)
    return fail(QI_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, Lw.total);
  ext.push_back({"workspace", (uintptr_t)workspace, (uintptr_t)workspace + Lw.total, true});
  if ((rc = check_alias(ext))) return rc;
  if (S > 1 && (k.ss > kFwdMaxRowStride || v.ss > kFwdMaxRowStride || q.ss > kFwdMaxRowStride ||
                d_o.ss > kFwdMaxRowStride))
    return fail(QI_E_UNSUPPORTED, "q/k/v/d_o sequence stride above %lld elements", (long long)kFwdMaxRowStride);
  if (geom->H > 65535) return fail(QI_E_UNSUPPORTED, "H=%d above the 65535 heads the backward launches", geom->H);
  if ((rc = current_device_gate())) return rc;

  char* ws = (char*)workspace;
  float* Dvec = (float*)(ws + Lw.dvec);
  float* lse2 = (float*)(ws + Lw.lse2);
  uint16_t* do16 = (uint16_t*)(ws + Lw.do16);
  uint32_t* amax = (uint32_t*)(ws + Lw.amax);
  float* inv_scale = (float*)(ws + Lw.scale);
  const int rows_per_wg = kBwdDqWaves * 32;
  const int keys_per_wg = kBwdKvWaves * 32;
  const int nt_do = bwd_nt_do(geom);
  int nk_max = 0;
  for (int b0 = 0; b0 < geom->B; b0 += kMaxBatchPerLaunch) {
    const int nb = std::min(kMaxBatchPerLaunch, geom->B - b0);
    BwdArgs a;
    a.q = view_of<const uint16_t>(q, b0);
    a.k = view_of<const uint16_t>(k, b0);
    a.v = view_of<const uint16_t>(v, b0);
    a.o = view_of<const float>(o_f32, b0);
    a.dO = view_of<const uint16_t>(d_o, b0);
    a.do16t = do16 + (int64_t)b0 * geom->H * nt_do * kVtileElems;
    a.nt_do = nt_do;
    a.do_inv_scale = inv_scale + (int64_t)b0 * geom->H;
    a.lse = lse + (int64_t)b0 * geom->H * S;
    a.Dvec = Dvec + (int64_t)b0 * geom->H * S;
    a.lse2 = lse2 + (int64_t)b0 * geom->H * S;
    a.dq = view_of<float>(dq, b0);
    a.dk = view_of<float>(dk, b0);
    a.dv = view_of<float>(dv, b0);
    a.B = nb;
    a.S = (int)S;
    a.H = geom->H;
    a.T_txt = geom->T_txt;
    a.T_img = geom->grid_h * geom->grid_w;
    a.n_qtiles = (int)ceil_div(S, rows_per_wg);
    a.do_amax = amax + (int64_t)b0 * geom->H * a.n_qtiles * kBwdDqWaves;
    nk_max = 0;
    for (int i = 0; i < nb; ++i) {
      const int L = geom->txt_len[b0 + i];
      const int nk = (int)(ceil_div(L, keys_per_wg) + ceil_div(a.T_img, keys_per_wg) +
                           ceil_div(geom->T_txt - L, keys_per_wg));
      nk_max = std::max(nk_max, nk);
    }
    a.n_ktiles = nk_max;
    a.xcd_remap = ((nb * geom->H) % 8) == 0;
    for (int i = 0; i < kMaxBatchPerLaunch; ++i) a.txt_len[i] = i < nb ? geom->txt_len[b0 + i] : 0;
    const int64_t n_dq = (int64_t)nb * geom->H * a.n_qtiles;
    hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)n_dq), dim3(kBwdDqWaves * 64), 0, stream, a);
    if ((rc = launched("attn_bwd_prep_kernel"))) return rc;
    {  // dO -> FP16 under the per-(b, h) scale, from the recorded maxima
      DoPrepArgs pa;
      pa.dO = a.dO;
      pa.out = const_cast<uint16_t*>(a.do16t);
      pa.amax = a.do_amax;
      pa.n_amax = a.n_qtiles * kBwdDqWaves;
      pa.inv_scale = inv_scale + (int64_t)b0 * geom->H;
      pa.S = (int)S;
      pa.H = geom->H;
      pa.T_txt = a.T_txt;
      pa.T_img = a.T_img;
      pa.nt_do = nt_do;
      for (int i = 0; i < kMaxBatchPerLaunch; ++i) pa.txt_len[i] = a.txt_len[i];
      hipLaunchKernelGGL(do_convert_kernel, dim3((unsigned)nt_do, (unsigned)geom->H, (unsigned)nb), dim3(256), 0,
                         stream, pa);
      if ((rc = launched("do_convert_kernel"))) return rc;
    }
    const int64_t n_kv = (int64_t)nb * geom->H * a.n_ktiles;
    hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)(2 * n_kv + n_dq)), dim3(kBwdKvWaves * 64), 0, stream, a);
    if ((rc = launched("attn_bwd_kernel"))) return rc;
  }
  const qi_bshd xs[2] = {q_raw, k_raw}, dxs[2] = {dq, dk};
  const float* const gains[2] = {gain_q, gain_k};
  float* const parts[2] = {(float*)(ws + Lw.pq), (float*)(ws + Lw.pk)};
  float* const dg_ps[2] = {dgain_q_ps, dgain_k_ps};
  float* const dg[2] = {dgain_q, dgain_k};
  return launch_prologue_bwd(geom, xs, gains, dxs, parts, dg_ps, dg, Lw, stream);
}

int qi_clock_probe(uint64_t* out, int32_t n_groups, int32_t iters, hipStream_t stream) {
  if (!out) return fail(QI_E_INVALID, "out is null");
  if ((uintptr_t)out % 8) return fail(QI_E_ALIGN, "out is not 8-byte aligned");
  if (n_groups < 1 || n_groups > 65536) return fail(QI_E_INVALID, "n_groups %d outside 1..65536", n_groups);
  if (iters < 1 || iters > (1 << 20)) return fail(QI_E_INVALID, "iters %d outside 1..2^20", iters);
  int rc = current_device_gate();
  if (rc) return rc;
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)n_groups), dim3(64), 0, stream, (unsigned long long*)out,
                     (int)iters, 1.0f / 1024.0f);
  return launched("clock_probe_kernel");
}

int64_t qi_wall_clock_khz(int device) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) {
    fail(QI_E_HIP, "cannot query the wall-clock rate of device %d", device);
    return 0;
  }
  return khz;
}

const char* qi_trace(void) {
  static const std::string s = [] {
    char buf[4096];
    snprintf(buf, sizeof buf,
             "{\"library\":\"qi\",\"target\":\"gfx950\",\"contract_version\":3,"
             "\"kernels\":{\"prologue\":\"qknorm_rope_fwd_kernel\",\"prologue_bwd\":\"qknorm_rope_bwd_kernel\","
             "\"dgain_fold\":\"dgain_fold_kernel\",\"attn_fwd_v_tiles\":\"v_tiles_kernel\","
             "\"qkv_prologue\":\"qkv_prologue_kernel\",\"attn_fwd\":\"attn_fwd_kernel\","
             "\"fwd_partial\":\"attn_fwd_partial_kernel\",\"fwd_carry\":\"attn_fwd_carry_kernel\","
             "\"merge\":\"attn_merge_kernel\","
             "\"qkv_proj\":\"proj_gemm_kernel\",\"out_proj\":\"proj_gemm_kernel\",\"rope_table\":\"rope_table_kernel\","
             "\"unfused_qk\":\"attn_qk_kernel\",\"unfused_softmax\":\"attn_softmax_kernel\",\"unfused_av\":\"attn_av_kernel\","
             "\"attn_bwd_prep\":\"attn_bwd_prep_kernel\",\"attn_bwd\":\"attn_bwd_kernel (dK, dQ, dV workgroups)\","
             "\"bwd_do_convert\":\"do_convert_kernel\"},"
             "\"mfma\":\"v_mfma_f32_32x32x16_bf16 (fwd P*V and bwd dV: v_mfma_f32_32x32x16_f16)\",\"accumulator\":\"fp32\","
             "\"frozen\":{\"fwd_key_tile\":%d,\"bwd_dq_key_tile\":%d,\"bwd_dkdv_query_tile\":%d,"
             "\"prologue_dgain_chunk\":%d,\"key_order\":\"text tiles from 0, image tiles from T_txt\","
             "\"bwd_query_order\":\"valid text, image, padded text\","
             "\"softmax\":\"exp2(fma(s,log2e/sqrt(128),-m*c)); l sums fp32 P in register order\","
             "\"fwd_pv_operands\":\"P fp16 RNE, V fp16 RNE of v*2^-8, O=acc/(l*2^-8)\","
             "\"bwd_D\":\"rowsum(dO*O) from the fp32 forward O\","
             "\"reference_max_threshold_log2\":8,"
             "\"ds_split\":\"hi=bf16(dS), lo=bf16(dS-hi), accumulated hi then lo (dQ, dK)\","
             "\"dv_operands\":\"P fp16 RNE, dO fp16 RNE of dO*2^e per (b,h) (e from its max|dO|, taken by the preparation kernel), dV=acc*2^-e\","
             "\"rms_sum_tree\":\"8 sequential per lane, xor 8,4,2,1\","
             "\"dgain_fold\":\"chunks ascending per sample, then samples ascending\"},"
             "\"free\":[\"rows per workgroup\",\"grid order / XCD mapping\",\"LDS layout\",\"prefetch depth\"],"
             "\"split_k\":false,\"split_kv\":false,\"stream_k\":false,\"atomics\":false,\"tf32\":false,"
             "\"fast_math\":false,\"fp_contract\":\"off\",\"fp32_denormals\":\"preserved\","
             "\"div_sqrt\":\"correctly rounded\",\"exp2\":\"v_exp_f32\","
             "\"rope_angles\":\"fp64, cos/sin rounded once to fp32\",\"output_cast\":\"fp32->bf16 RNE, once\","
             "\"hipcc\":\"%s\"}",
             kFwdBN, kBwdBN, kBwdBM, kPrologueChunk, __clang_version__);
    return std::string(buf);
  }();
  return s.c_str();
}

}  // extern "C"
