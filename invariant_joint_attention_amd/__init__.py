"""Strict joint attention for AMD Instinct MI355X (gfx950).

Python binding of ``libqi.so`` (declared in ``include/qi.h``).  It only
marshals arguments: every step of the path -- the learned-gain Q/K RMSNorm
with three-axis RoPE, the masked joint attention forward and its
deterministic backward -- runs in the library's HIP kernels.  torch supplies
device memory and the current stream.  A nonzero status raises ``QiError``;
there is no other code path, and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os

import torch

HEAD_DIM = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqi.so")

STATUS = {0: "QI_OK", 1: "QI_E_INVALID", 2: "QI_E_UNSUPPORTED", 3: "QI_E_ALIGN", 4: "QI_E_ALIAS",
          5: "QI_E_WORKSPACE", 6: "QI_E_STRICT", 7: "QI_E_HIP"}

# every entry point declared in include/qi.h
SYMBOLS = ("qi_qknorm_rope", "qi_joint_attn_fwd_workspace", "qi_joint_attn_fwd", "qi_joint_attn_fwd_noalloc",
           "qi_qkv_prologue",
           "qi_joint_attn_fwd_vtiles", "qi_joint_attn_fwd_partial",
           "qi_joint_attn_merge", "qi_joint_attn_fwd_carry", "qi_qkv_proj_workspace", "qi_qkv_proj", "qi_attn_out_proj",
           "qi_joint_attn_key_slots",
           "qi_joint_attn_qk_gemm", "qi_joint_attn_softmax", "qi_joint_attn_av_gemm", "qi_joint_attn_bwd_workspace",
           "qi_joint_attn_bwd", "qi_clock_probe", "qi_wall_clock_khz", "qi_last_error", "qi_strict_probe",
           "qi_trace")


class QiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class QiBshd(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("sb", ctypes.c_int64), ("ss", ctypes.c_int64), ("sh", ctypes.c_int64)]


class QiKeyBlock(ctypes.Structure):
    _fields_ = [("include_text", ctypes.c_int32), ("img_begin", ctypes.c_int32), ("img_end", ctypes.c_int32)]


class QiGeom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("T_txt", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("txt_len", ctypes.POINTER(ctypes.c_int32)), ("rope_axes", ctypes.c_int32 * 3),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float), ("gain_streams", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with invariant_joint_attention_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, G, S = ctypes.c_void_p, ctypes.POINTER(QiGeom), ctypes.c_void_p
        L.qi_qknorm_rope.argtypes = [G, QiBshd, P, QiBshd, P, S]
        L.qi_joint_attn_fwd_workspace.argtypes = [G]
        L.qi_joint_attn_fwd_workspace.restype = ctypes.c_size_t
        L.qi_joint_attn_fwd.argtypes = [G, QiBshd, QiBshd, QiBshd, QiBshd, P, P, P, ctypes.c_size_t, S]
        L.qi_joint_attn_fwd_noalloc.argtypes = [G, QiBshd, QiBshd, QiBshd, QiBshd, P, P, S]
        L.qi_qkv_prologue.argtypes = [G, QiBshd, QiBshd, QiBshd, P, P, QiBshd, QiBshd, P, ctypes.c_size_t, S]
        L.qi_joint_attn_fwd_vtiles.argtypes = [G, QiBshd, QiBshd, P, ctypes.c_size_t, QiBshd, P, P, S]
        L.qi_joint_attn_fwd_partial.argtypes = [G, QiBshd, QiBshd, QiBshd, QiKeyBlock, P, P, P, P, ctypes.c_size_t, S]
        L.qi_joint_attn_merge.argtypes = [G, ctypes.c_int32, P, P, P, QiBshd, P, P, S]
        L.qi_joint_attn_fwd_carry.argtypes = [G, QiBshd, QiBshd, QiBshd, QiKeyBlock, P, P, P, P, P, P, QiBshd, P, P,
                                              P, ctypes.c_size_t, S]
        L.qi_qkv_proj_workspace.argtypes = [G]
        L.qi_qkv_proj_workspace.restype = ctypes.c_size_t
        L.qi_qkv_proj.argtypes = [G, QiBshd, P, P, ctypes.c_int32, P, P, ctypes.c_int32, QiBshd, QiBshd, QiBshd, P,
                                  ctypes.c_size_t, S]
        L.qi_attn_out_proj.argtypes = [G, QiBshd, P, P, ctypes.c_int32, QiBshd, S]
        L.qi_joint_attn_key_slots.argtypes = [G]
        L.qi_joint_attn_key_slots.restype = ctypes.c_int64
        L.qi_joint_attn_qk_gemm.argtypes = [G, QiBshd, QiBshd, P, S]
        L.qi_joint_attn_softmax.argtypes = [G, P, P, P, P, P, S]
        L.qi_joint_attn_av_gemm.argtypes = [G, P, P, P, QiBshd, QiBshd, P, P, ctypes.c_size_t, S]
        L.qi_joint_attn_bwd_workspace.argtypes = [G]
        L.qi_joint_attn_bwd_workspace.restype = ctypes.c_size_t
        L.qi_joint_attn_bwd.argtypes = [G, QiBshd, QiBshd, QiBshd, QiBshd, QiBshd, QiBshd, P, QiBshd, P, P,
                                        QiBshd, QiBshd, QiBshd, P, P, P, P, P, ctypes.c_size_t, S]
        L.qi_clock_probe.argtypes = [P, ctypes.c_int32, ctypes.c_int32, S]
        L.qi_wall_clock_khz.argtypes = [ctypes.c_int]
        L.qi_wall_clock_khz.restype = ctypes.c_int64
        L.qi_last_error.restype = ctypes.c_char_p
        L.qi_strict_probe.argtypes = [ctypes.c_int]
        L.qi_trace.restype = ctypes.c_char_p
        for name in ("qi_qknorm_rope", "qi_joint_attn_fwd", "qi_joint_attn_fwd_noalloc", "qi_joint_attn_fwd_partial", "qi_joint_attn_merge",
                     "qi_joint_attn_fwd_carry", "qi_qkv_proj", "qi_attn_out_proj",
                     "qi_joint_attn_qk_gemm", "qi_joint_attn_softmax",
                     "qi_joint_attn_av_gemm", "qi_joint_attn_bwd", "qi_clock_probe", "qi_strict_probe"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise QiError(rc, lib().qi_last_error().decode())


class Geometry:
    """Geometry of one call (mirrors ``qi_geom``)."""

    def __init__(self, B, H, T_txt, grid_h, grid_w, txt_len, rope_theta=10000.0, rms_eps=1e-6, gain_streams=1,
                 D=HEAD_DIM, rope_axes=(16, 56, 56)):
        self.B, self.H, self.T_txt, self.grid_h, self.grid_w = int(B), int(H), int(T_txt), int(grid_h), int(grid_w)
        self.txt_len = [int(x) for x in txt_len]
        self.S = self.T_txt + self.grid_h * self.grid_w
        self._len = (ctypes.c_int32 * max(1, len(self.txt_len)))(*self.txt_len)
        self.c = QiGeom(self.B, self.H, int(D), self.T_txt, self.grid_h, self.grid_w,
                        ctypes.cast(self._len, ctypes.POINTER(ctypes.c_int32)),
                        (ctypes.c_int32 * 3)(*rope_axes), float(rope_theta), float(rms_eps), int(gain_streams))
        self.gain_streams = int(gain_streams)

    def ptr(self):
        return ctypes.byref(self.c)


def _bshd(t: torch.Tensor) -> QiBshd:
    if t.dim() != 4:
        raise ValueError("expected a [B, S, H, 128] tensor")
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if t.stride(3) != 1:
        raise ValueError("the head dimension must have stride 1")
    return QiBshd(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def qknorm_rope(x, gain, geom: Geometry, out=None, out_f32=None):
    """y = bf16(rope(gain * rmsnorm(x))) for a BF16 [B,S,H,128] tensor."""
    if out is None:
        out = _empty(x.shape, torch.bfloat16, x)
    _check(lib().qi_qknorm_rope(geom.ptr(), _bshd(x), _ptr(gain), _bshd(out), _ptr(out_f32), _stream()))
    return out


def fwd_workspace_bytes(geom: Geometry) -> int:
    return int(lib().qi_joint_attn_fwd_workspace(geom.ptr()))


def joint_attn_fwd(q, k, v, geom: Geometry, out=None, lse=None, out_f32=None, workspace=None):
    """Masked joint attention forward; returns (O BF16 [B,S,H,128], LSE FP32 [B,H,S]).
    ``workspace`` is a device byte tensor of at least ``fwd_workspace_bytes``
    (allocated here when omitted)."""
    if out is None:
        out = _empty(q.shape, torch.bfloat16, q)
    if lse is None:
        lse = _empty((geom.B, geom.H, geom.S), torch.float32, q)
    if workspace is None:
        workspace = _empty((max(1, fwd_workspace_bytes(geom)),), torch.uint8, q)
    _check(lib().qi_joint_attn_fwd(geom.ptr(), _bshd(q), _bshd(k), _bshd(v), _bshd(out), _ptr(lse),
                                   _ptr(out_f32), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream()))
    return out, lse


def joint_attn_fwd_noalloc(q, k, v, geom: Geometry, out, lse, out_f32=None):
    """qi_joint_attn_fwd_noalloc: the forward with the library's static
    scratch instead of a workspace; the caller passes every output (nothing
    is allocated here either)."""
    _check(lib().qi_joint_attn_fwd_noalloc(geom.ptr(), _bshd(q), _bshd(k), _bshd(v), _bshd(out), _ptr(lse),
                                           _ptr(out_f32), _stream()))
    return out, lse


def qkv_prologue(q_raw, k_raw, v, gain_q, gain_k, geom: Geometry, q=None, k=None, v_tiles=None):
    """Q and K prologues and the V tile conversion in one launch; returns
    (q', k', v_tiles) with v_tiles a device byte tensor of
    ``fwd_workspace_bytes`` holding V in the attention's FP16 tile format."""
    q = _empty(q_raw.shape, torch.bfloat16, q_raw) if q is None else q
    k = _empty(k_raw.shape, torch.bfloat16, k_raw) if k is None else k
    if v_tiles is None:
        v_tiles = _empty((max(1, fwd_workspace_bytes(geom)),), torch.uint8, q_raw)
    _check(lib().qi_qkv_prologue(geom.ptr(), _bshd(q_raw), _bshd(k_raw), _bshd(v), _ptr(gain_q), _ptr(gain_k),
                                 _bshd(q), _bshd(k), _ptr(v_tiles), v_tiles.numel() * v_tiles.element_size(),
                                 _stream()))
    return q, k, v_tiles


def joint_attn_fwd_vtiles(q, k, v_tiles, geom: Geometry, out=None, lse=None, out_f32=None):
    """Attention forward over the V tiles written by ``qkv_prologue``;
    returns (O, LSE) as ``joint_attn_fwd``."""
    if out is None:
        out = _empty(q.shape, torch.bfloat16, q)
    if lse is None:
        lse = _empty((geom.B, geom.H, geom.S), torch.float32, q)
    _check(lib().qi_joint_attn_fwd_vtiles(geom.ptr(), _bshd(q), _bshd(k), _ptr(v_tiles),
                                          v_tiles.numel() * v_tiles.element_size(), _bshd(out), _ptr(lse),
                                          _ptr(out_f32), _stream()))
    return out, lse


def joint_attn_fwd_partial(q, k, v, geom: Geometry, include_text: bool, img_begin: int, img_end: int,
                           acc=None, m=None, l=None, workspace=None):
    """Row state of one key block: (acc FP32 [B,H,S,128], m FP32 [B,H,S],
    l FP32 [B,H,S]); acc holds sum_j p_j v_j 2^-8."""
    B, H, S = geom.B, geom.H, geom.S
    acc = _empty((B, H, S, HEAD_DIM), torch.float32, q) if acc is None else acc
    m = _empty((B, H, S), torch.float32, q) if m is None else m
    l = _empty((B, H, S), torch.float32, q) if l is None else l
    if workspace is None:
        workspace = _empty((max(1, fwd_workspace_bytes(geom)),), torch.uint8, q)
    blk = QiKeyBlock(int(bool(include_text)), int(img_begin), int(img_end))
    _check(lib().qi_joint_attn_fwd_partial(geom.ptr(), _bshd(q), _bshd(k), _bshd(v), blk, _ptr(acc), _ptr(m), _ptr(l),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return acc, m, l


def joint_attn_fwd_carry(q, k, v, geom: Geometry, include_text: bool, img_begin: int, img_end: int,
                         state=None, last=False, state_out=None, out=None, lse=None, out_f32=None, workspace=None):
    """One key block continuing ``state`` = (acc [B,H,S,128], m [B,H,S],
    l [B,H,S,2]) FP32 (None: the first block).  Not last: returns the state
    after the block (written to ``state_out``, which may be ``state`` itself
    for an in-place chain); last: returns (O, LSE) as ``joint_attn_fwd``."""
    B, H, S = geom.B, geom.H, geom.S
    if workspace is None:
        workspace = _empty((max(1, fwd_workspace_bytes(geom)),), torch.uint8, q)
    blk = QiKeyBlock(int(bool(include_text)), int(img_begin), int(img_end))
    ins = (None, None, None) if state is None else state
    no_o = QiBshd(None, 0, 0, 0)
    if last:
        outs = (None, None, None)
        out = _empty(q.shape, torch.bfloat16, q) if out is None else out
        lse = _empty((B, H, S), torch.float32, q) if lse is None else lse
        o_arg = _bshd(out)
    else:
        outs = state_out if state_out is not None else (
            _empty((B, H, S, HEAD_DIM), torch.float32, q), _empty((B, H, S), torch.float32, q),
            _empty((B, H, S, 2), torch.float32, q))
        o_arg = no_o
    _check(lib().qi_joint_attn_fwd_carry(geom.ptr(), _bshd(q), _bshd(k), _bshd(v), blk,
                                         *[_ptr(t) for t in ins], *[_ptr(t) for t in outs], o_arg, _ptr(lse),
                                         _ptr(out_f32), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream()))
    return (out, lse) if last else outs


def joint_attn_merge(acc, m, l, geom: Geometry, out=None, lse=None, out_f32=None):
    """Fold stacked row states (acc [n,B,H,S,128], m and l [n,B,H,S]) in
    ascending block order; returns (O BF16 [B,S,H,128], LSE FP32 [B,H,S])."""
    n = acc.shape[0]
    if out is None:
        out = torch.empty((geom.B, geom.S, geom.H, HEAD_DIM), dtype=torch.bfloat16, device=acc.device)
    if lse is None:
        lse = _empty((geom.B, geom.H, geom.S), torch.float32, acc)
    _check(lib().qi_joint_attn_merge(geom.ptr(), int(n), _ptr(acc), _ptr(m), _ptr(l), _bshd(out), _ptr(lse),
                                     _ptr(out_f32), _stream()))
    return out, lse


def qkv_proj(x, w, bias, geom: Geometry, gain_q=None, gain_k=None, fuse_prologue=True, q=None, k=None, v=None,
             workspace=None):
    """Per-stream packed QKV projection of x [B,S,H,128] (BF16) with weights
    w [streams, 3D, D] (BF16) and bias [streams, 3D] (FP32).  With
    fuse_prologue the Q and K outputs are already RMS-normalised, scaled by
    the gains and rotated (the prologue).  Returns (q, k, v) BF16 [B,S,H,128]."""
    q = torch.empty_like(x) if q is None else q
    k = torch.empty_like(x) if k is None else k
    v = torch.empty_like(x) if v is None else v
    if fuse_prologue and workspace is None:
        workspace = _empty((max(1, int(lib().qi_qkv_proj_workspace(geom.ptr()))),), torch.uint8, x)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qi_qkv_proj(geom.ptr(), _bshd(x), _ptr(w), _ptr(bias), int(w.shape[0]), _ptr(gain_q), _ptr(gain_k),
                             int(bool(fuse_prologue)), _bshd(q), _bshd(k), _bshd(v), _ptr(workspace), nbytes,
                             _stream()))
    return q, k, v


def attn_out_proj(o, w, bias, geom: Geometry, y=None):
    """Per-stream output projection of o [B,S,H,128] (BF16): y = o W^T + b."""
    y = torch.empty_like(o) if y is None else y
    _check(lib().qi_attn_out_proj(geom.ptr(), _bshd(o), _ptr(w), _ptr(bias), int(w.shape[0]), _bshd(y), _stream()))
    return y


def key_slots(geom: Geometry) -> int:
    """Key slots per query row of the unfused intermediates (64 per logical key tile)."""
    return int(lib().qi_joint_attn_key_slots(geom.ptr()))


def joint_attn_qk_gemm(q, k, geom: Geometry, scores=None):
    """Raw scores q'.k' as FP32 [B, H, S, key_slots] (masked slots -inf)."""
    if scores is None:
        scores = _empty((geom.B, geom.H, geom.S, key_slots(geom)), torch.float32, q)
    _check(lib().qi_joint_attn_qk_gemm(geom.ptr(), _bshd(q), _bshd(k), _ptr(scores), _stream()))
    return scores


def joint_attn_softmax(scores, geom: Geometry, p=None, alpha=None, l=None, lse=None):
    """Online softmax over the key tiles of FP32 scores [B, H, S, key_slots].
    Returns (P FP16 [B,H,S,slots], alpha FP32 [B,H,slots/64,S] (tile-major),
    l FP32 [B,H,S], LSE FP32 [B,H,S])."""
    B, H, S, Kp = geom.B, geom.H, geom.S, key_slots(geom)
    p = _empty((B, H, S, Kp), torch.float16, scores) if p is None else p
    alpha = _empty((B, H, Kp // 64, S), torch.float32, scores) if alpha is None else alpha
    l = _empty((B, H, S), torch.float32, scores) if l is None else l
    lse = _empty((B, H, S), torch.float32, scores) if lse is None else lse
    _check(lib().qi_joint_attn_softmax(geom.ptr(), _ptr(scores), _ptr(p), _ptr(alpha), _ptr(l), _ptr(lse), _stream()))
    return p, alpha, l, lse


def joint_attn_av_gemm(p, alpha, l, v, geom: Geometry, out=None, out_f32=None, workspace=None):
    """O = (alpha-rescaled sum of P V over the key tiles) / l, BF16 [B,S,H,128]."""
    if out is None:
        out = _empty(v.shape, torch.bfloat16, v)
    if workspace is None:
        workspace = _empty((max(1, fwd_workspace_bytes(geom)),), torch.uint8, v)
    _check(lib().qi_joint_attn_av_gemm(geom.ptr(), _ptr(p), _ptr(alpha), _ptr(l), _bshd(v), _bshd(out),
                                       _ptr(out_f32), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream()))
    return out


def joint_attn_unfused(q, k, v, geom: Geometry, out_f32=None):
    """The composition qk_gemm -> softmax -> av_gemm; returns (O, LSE, dict of
    the intermediates).  Equal byte for byte to ``joint_attn_fwd``."""
    s = joint_attn_qk_gemm(q, k, geom)
    p, alpha, l, lse = joint_attn_softmax(s, geom)
    o = joint_attn_av_gemm(p, alpha, l, v, geom, out_f32=out_f32)
    return o, lse, dict(scores=s, p=p, alpha=alpha, l=l)


def bwd_workspace_bytes(geom: Geometry) -> int:
    return int(lib().qi_joint_attn_bwd_workspace(geom.ptr()))


def joint_attn_bwd(q_raw, k_raw, q, k, v, o_f32, lse, d_o, gain_q, gain_k, geom: Geometry, workspace=None,
                   dq=None, dk=None, dv=None, dgain_q_ps=None, dgain_k_ps=None, dgain_q=None, dgain_k=None):
    """Gradients of the whole path (o_f32: the forward's FP32 pre-cast O).
    Returns a dict with dq, dk, dv (FP32
    [B,S,H,128], w.r.t. the raw prologue inputs and V), dgain_q_ps /
    dgain_k_ps (FP32 [B, gain_streams, 128]) and dgain_q / dgain_k (their
    sums in ascending batch order)."""
    dev = q.device
    shp = q.shape
    dq = torch.empty(shp, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(shp, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(shp, dtype=torch.float32, device=dev) if dv is None else dv
    ns = geom.gain_streams
    def buf(t, shape):
        return torch.empty(shape, dtype=torch.float32, device=dev) if t is None else t

    dgq_ps, dgk_ps = buf(dgain_q_ps, (geom.B, ns, HEAD_DIM)), buf(dgain_k_ps, (geom.B, ns, HEAD_DIM))
    dgq, dgk = buf(dgain_q, (ns, HEAD_DIM)), buf(dgain_k, (ns, HEAD_DIM))
    nbytes = bwd_workspace_bytes(geom)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().qi_joint_attn_bwd(geom.ptr(), _bshd(q_raw), _bshd(k_raw), _bshd(q), _bshd(k), _bshd(v), _bshd(o_f32),
                                   _ptr(lse), _bshd(d_o), _ptr(gain_q), _ptr(gain_k), _bshd(dq), _bshd(dk),
                                   _bshd(dv), _ptr(dgq_ps), _ptr(dgk_ps), _ptr(dgq), _ptr(dgk),
                                   _ptr(workspace), workspace.numel(), _stream()))
    return dict(dq=dq, dk=dk, dv=dv, dgain_q_ps=dgq_ps, dgain_k_ps=dgk_ps, dgain_q=dgq, dgain_k=dgk)


def joint_attention(q_raw, k_raw, v, gain_q, gain_k, geom: Geometry, keep_f32=False):
    """The whole forward path: prologue on Q and K, then attention.
    Returns (q', k', O, LSE, O_f32) -- O_f32 (needed by the backward) only
    when keep_f32, else None."""
    q = qknorm_rope(q_raw, gain_q, geom)
    k = qknorm_rope(k_raw, gain_k, geom)
    of = torch.empty(q.shape, dtype=torch.float32, device=q.device) if keep_f32 else None
    o, lse = joint_attn_fwd(q, k, v, geom, out_f32=of)
    return q, k, o, lse, of


def strict_probe(device: int = 0) -> None:
    _check(lib().qi_strict_probe(int(device)))


def trace() -> str:
    return lib().qi_trace().decode()


def last_error() -> str:
    return lib().qi_last_error().decode()


def clock_probe(out: torch.Tensor, iters: int = 512) -> None:
    """Enqueue the shader-clock probe into ``out`` (int64 [n, 3] on the
    device): per single-wave workgroup the shader-clock and wall-clock ticks
    over `iters` rounds of four BF16 MFMAs."""
    assert out.dtype == torch.int64 and out.dim() == 2 and out.shape[1] == 3 and out.is_contiguous()
    _check(lib().qi_clock_probe(_ptr(out), int(out.shape[0]), int(iters), _stream()))


def wall_clock_khz(device: int = 0) -> int:
    khz = int(lib().qi_wall_clock_khz(int(device)))
    if khz <= 0:
        raise QiError(7, last_error())
    return khz
