"""NumPy-level wrapper around the C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only users.  Nothing here touches the
GPU library, and the GPU library never loads this module or its ``.so``.

Two builds of the same C source exist:
  * ``liboracle_f32.so`` -- the FP32 CPU reference (``real = float``);
  * ``liboracle_f64.so`` -- the same algorithm in FP64, used by the pins that
    need it (finite differences, comparisons against library routines).

Arrays follow the path's logical layout: activations ``[B, S, H, 128]`` with
the sequence ordered [text (T_txt, padded), image (h*w, row-major)].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
HD = 128

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas"]


def lib_path(precision: str) -> str:
    return os.path.join(HERE, f"liboracle_{precision}.so")


def build(verbose: bool = False) -> None:
    """Compile both precisions of the oracle with gcc (always recompiles)."""
    for prec, real in (("f32", "float"), ("f64", "double")):
        out = lib_path(prec)
        tmp = out + ".tmp"
        cmd = ["gcc", *_CFLAGS, f"-DORACLE_REAL={real}", SRC, "-o", tmp, "-lm"]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """Handle on one precision of the oracle library."""

    def __init__(self, precision: str = "f32"):
        if precision not in ("f32", "f64"):
            raise ValueError(precision)
        path = lib_path(precision)
        if not os.path.exists(path):
            build()
        self.precision = precision
        self.dtype = np.float32 if precision == "f32" else np.float64
        self.creal = ctypes.c_float if precision == "f32" else ctypes.c_double
        self.lib = ctypes.CDLL(path)
        assert self.lib.oracle_real_bytes() == np.dtype(self.dtype).itemsize

    # ------------------------------------------------------------------ util
    def _r(self, a) -> np.ndarray:
        return np.ascontiguousarray(a, dtype=self.dtype)

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(ctypes.c_int(n))

    def widen(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=self.dtype)
        self.lib.oracle_bf16_widen(ctypes.c_int64(bits.size), _ptr(bits, ctypes.c_uint16),
                                   _ptr(out, self.creal))
        return out

    def cast_bf16(self, x: np.ndarray) -> np.ndarray:
        x = self._r(x)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_cast_bf16(ctypes.c_int64(x.size), _ptr(x, self.creal),
                                  _ptr(out, ctypes.c_uint16))
        return out

    # -------------------------------------------------------------- prologue
    def positions(self, T_txt: int, h: int, w: int) -> np.ndarray:
        S = T_txt + h * w
        pos = np.empty((S, 3), dtype=np.int32)
        self.lib.oracle_positions(ctypes.c_int(T_txt), ctypes.c_int(h), ctypes.c_int(w),
                                  _ptr(pos, ctypes.c_int32))
        return pos

    def rope_apply(self, pos: np.ndarray, y: np.ndarray, theta: float = 10000.0) -> np.ndarray:
        """Rotate y [n_tok, H, 128] by integer position triples pos [n_tok, 3]."""
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        y = self._r(y)
        n_tok, H = y.shape[0], y.shape[1]
        assert y.shape == (n_tok, H, HD) and pos.shape == (n_tok, 3)
        out = np.empty_like(y)
        self.lib.oracle_rope_apply(ctypes.c_int64(n_tok), ctypes.c_int(H), _ptr(pos, ctypes.c_int32),
                                   ctypes.c_double(theta), _ptr(y, self.creal), _ptr(out, self.creal))
        return out

    def rmsnorm(self, x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
        x = self._r(x)
        g = self._r(gain)
        assert x.shape[-1] == HD and g.shape == (HD,)
        out = np.empty_like(x)
        self.lib.oracle_rmsnorm(ctypes.c_int64(x.size // HD), _ptr(x, self.creal), _ptr(g, self.creal),
                                self.creal(eps), _ptr(out, self.creal))
        return out

    def qknorm_rope(self, x, gain, T_txt, h, w, theta=10000.0, eps=1e-6) -> np.ndarray:
        """Pre-cast prologue output for x [B,S,H,128]; gain [streams,128]."""
        x = self._r(x)
        g = self._r(np.atleast_2d(gain))
        B, S, H, D = x.shape
        assert D == HD and S == T_txt + h * w and g.shape[0] in (1, 2)
        y = np.empty_like(x)
        self.lib.oracle_qknorm_rope(ctypes.c_int(B), ctypes.c_int(S), ctypes.c_int(H),
                                    ctypes.c_int(T_txt), ctypes.c_int(h), ctypes.c_int(w),
                                    _ptr(x, self.creal), _ptr(g, self.creal), ctypes.c_int(g.shape[0]),
                                    ctypes.c_double(theta), self.creal(eps), _ptr(y, self.creal))
        return y

    def qknorm_rope_bwd(self, x, gain, dy, T_txt, h, w, theta=10000.0, eps=1e-6):
        """Returns (dx [B,S,H,128], dg_per_sample [B, streams, 128])."""
        x = self._r(x)
        dy = self._r(dy)
        g = self._r(np.atleast_2d(gain))
        B, S, H, D = x.shape
        ns = g.shape[0]
        dx = np.empty_like(x)
        dg = np.empty((B, ns, HD), dtype=self.dtype)
        self.lib.oracle_qknorm_rope_bwd(ctypes.c_int(B), ctypes.c_int(S), ctypes.c_int(H),
                                        ctypes.c_int(T_txt), ctypes.c_int(h), ctypes.c_int(w),
                                        _ptr(x, self.creal), _ptr(g, self.creal), ctypes.c_int(ns),
                                        ctypes.c_double(theta), self.creal(eps), _ptr(dy, self.creal),
                                        _ptr(dx, self.creal), _ptr(dg, self.creal))
        return dx, dg

    # ------------------------------------------------------------- attention
    def attn_fwd_bh(self, q, k, v, T_txt, L, s0=0, s1=None):
        """One (batch, head) slice: q,k,v [S,128].  Rows [s0,s1)."""
        q, k, v = self._r(q), self._r(k), self._r(v)
        S = q.shape[0]
        s1 = S if s1 is None else s1
        o = np.empty((s1 - s0, HD), dtype=self.dtype)
        lse = np.empty((s1 - s0,), dtype=self.dtype)
        self.lib.oracle_attn_fwd_bh(ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(L),
                                    _ptr(q, self.creal), _ptr(k, self.creal), _ptr(v, self.creal),
                                    ctypes.c_int(s0), ctypes.c_int(s1), _ptr(o, self.creal),
                                    _ptr(lse, self.creal))
        return o, lse

    def attn_fwd_block_bh(self, q, k, v, T_txt, L, with_text, img_lo, img_hi, s0=0, s1=None):
        """One (batch, head) slice over one key block: the text keys j < L
        (when with_text) and the image keys T_txt + i, img_lo <= i < img_hi.
        Rows [s0, s1).  Returns o, lse of attention restricted to the block."""
        q, k, v = self._r(q), self._r(k), self._r(v)
        S = q.shape[0]
        s1 = S if s1 is None else s1
        o = np.empty((s1 - s0, HD), dtype=self.dtype)
        lse = np.empty((s1 - s0,), dtype=self.dtype)
        self.lib.oracle_attn_fwd_block_bh(ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(L),
                                          ctypes.c_int(int(bool(with_text))), ctypes.c_int(img_lo),
                                          ctypes.c_int(img_hi), _ptr(q, self.creal), _ptr(k, self.creal),
                                          _ptr(v, self.creal), ctypes.c_int(s0), ctypes.c_int(s1),
                                          _ptr(o, self.creal), _ptr(lse, self.creal))
        return o, lse

    def attn_fwd(self, q, k, v, txt_len, T_txt, heads=None):
        """q,k,v [B,S,H,128].  Returns o [B,S,H,128] and lse [B,H,S].

        ``heads``: optional list of (b, h) pairs to compute; the others are
        left as NaN (for sampled checks at full size)."""
        B, S, H, _ = q.shape
        o = np.full((B, S, H, HD), np.nan, dtype=self.dtype)
        lse = np.full((B, H, S), np.nan, dtype=self.dtype)
        pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
        for b, h in pairs:
            ob, lb = self.attn_fwd_bh(q[b, :, h], k[b, :, h], v[b, :, h], T_txt, int(txt_len[b]))
            o[b, :, h] = ob
            lse[b, h] = lb
        return o, lse

    def attn_scores_bh(self, q, k, T_txt, L, s0=0, s1=None):
        """Scaled scores q_i.k_j / sqrt(128) of one (batch, head) slice, rows
        [s0, s1) x all S keys; masked keys 0."""
        q, k = self._r(q), self._r(k)
        S = q.shape[0]
        s1 = S if s1 is None else s1
        s = np.empty((s1 - s0, S), dtype=self.dtype)
        self.lib.oracle_attn_scores_bh(ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(L), _ptr(q, self.creal),
                                       _ptr(k, self.creal), ctypes.c_int(s0), ctypes.c_int(s1), _ptr(s, self.creal))
        return s

    def attn_softmax_rows(self, s, T_txt, L):
        """Softmax over the valid keys of score rows s [n, S] (scaled).
        Returns p [n, S] (masked entries 0) and lse [n]."""
        s = self._r(s)
        n, S = s.shape
        p = np.empty((n, S), dtype=self.dtype)
        lse = np.empty((n,), dtype=self.dtype)
        self.lib.oracle_attn_softmax_rows(ctypes.c_int(n), ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(L),
                                          _ptr(s, self.creal), _ptr(p, self.creal), _ptr(lse, self.creal))
        return p, lse

    def attn_av_rows(self, P, alpha, l, v, T_txt, L):
        """The A.V operator over logical 64-key tiles, as its closed form
        o = sum_t (prod_{u>t} alpha_u) P_t V_t / l: P [n, nt, 64],
        alpha [n, nt], l [n], v [S, 128] -> o [n, 128]."""
        P, alpha, l, v = self._r(P), self._r(alpha), self._r(l), self._r(v)
        n, nt, _ = P.shape
        S = v.shape[0]
        o = np.empty((n, HD), dtype=self.dtype)
        self.lib.oracle_attn_av_rows(ctypes.c_int(n), ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(L),
                                     ctypes.c_int(nt), _ptr(P, self.creal), _ptr(alpha, self.creal),
                                     _ptr(l, self.creal), _ptr(v, self.creal), _ptr(o, self.creal))
        return o

    def attn_bwd(self, q, k, v, dO, txt_len, T_txt, heads=None):
        """Returns dq', dk', dv [B,S,H,128] (NaN outside ``heads``)."""
        B, S, H, _ = q.shape
        outs = [np.full((B, S, H, HD), np.nan, dtype=self.dtype) for _ in range(3)]
        pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
        for b, h in pairs:
            qs, ks, vs, gs = (self._r(t[b, :, h]) for t in (q, k, v, dO))
            dq, dk, dv = (np.empty((S, HD), dtype=self.dtype) for _ in range(3))
            rc = self.lib.oracle_attn_bwd_bh(ctypes.c_int(S), ctypes.c_int(T_txt), ctypes.c_int(int(txt_len[b])),
                                             _ptr(qs, self.creal), _ptr(ks, self.creal), _ptr(vs, self.creal),
                                             _ptr(gs, self.creal), _ptr(dq, self.creal), _ptr(dk, self.creal),
                                             _ptr(dv, self.creal))
            if rc != 0:
                raise MemoryError("oracle_attn_bwd_bh: allocation failed")
            outs[0][b, :, h], outs[1][b, :, h], outs[2][b, :, h] = dq, dk, dv
        return tuple(outs)


    # ----------------------------------------------------------- projections
    def linear(self, x, W, bias):
        """y = x W^T + bias for x [n, K], W [N, K], bias [N]; the sum over k
        ascending."""
        x, W, bias = self._r(x), self._r(W), self._r(bias)
        n, K = x.shape
        N = W.shape[0]
        assert W.shape == (N, K) and bias.shape == (N,)
        y = np.empty((n, N), dtype=self.dtype)
        self.lib.oracle_linear(ctypes.c_int64(n), ctypes.c_int(K), ctypes.c_int(N), _ptr(x, self.creal),
                               _ptr(W, self.creal), _ptr(bias, self.creal), _ptr(y, self.creal))
        return y

    def stream_linear(self, x, W, bias, T_txt):
        """Per-stream projection of x [B, S, K]: text rows s < T_txt use
        W[0], bias[0]; image rows use the last set (one set: shared)."""
        B, S, K = x.shape
        W, bias = np.asarray(W), np.asarray(bias)
        out = np.empty((B, S, W.shape[1]), dtype=self.dtype)
        for b in range(B):
            if T_txt:
                out[b, :T_txt] = self.linear(x[b, :T_txt], W[0], bias[0])
            out[b, T_txt:] = self.linear(x[b, T_txt:], W[-1], bias[-1])
        return out


def fold_batch(per_sample: np.ndarray) -> np.ndarray:
    """Sum per-sample partials over the batch in ascending order."""
    acc = np.zeros(per_sample.shape[1:], dtype=per_sample.dtype)
    for b in range(per_sample.shape[0]):
        acc = acc + per_sample[b]
    return acc


def forward_path(orc: Oracle, x_q, x_k, v, g_q, g_k, txt_len, T_txt, h, w, heads=None):
    """The whole forward path from raw BF16 bit patterns.

    x_q, x_k, v: uint16 BF16 bits [B,S,H,128]; g_q, g_k: float [streams,128].
    Returns a dict with the pre-cast prologue outputs, their BF16 casts, the
    pre-cast attention output, its BF16 cast and the LSE."""
    qp = orc.qknorm_rope(orc.widen(x_q), g_q, T_txt, h, w)
    kp = orc.qknorm_rope(orc.widen(x_k), g_k, T_txt, h, w)
    qb, kb = orc.cast_bf16(qp), orc.cast_bf16(kp)
    o, lse = orc.attn_fwd(orc.widen(qb), orc.widen(kb), orc.widen(v), txt_len, T_txt, heads=heads)
    ob = orc.cast_bf16(np.nan_to_num(o)) if heads is not None else orc.cast_bf16(o)
    return dict(q_pre=qp, k_pre=kp, q_bf16=qb, k_bf16=kb, o=o, o_bf16=ob, lse=lse)


def qkv_path(orc: Oracle, x, W, bias, g_q, g_k, T_txt, h, w):
    """The packed QKV projection and the Q/K prologue from BF16 bit patterns.

    x: uint16 [B, S, D] hidden states (D = H*128); W: uint16 [streams, 3D, D];
    bias: float [streams, 3D].  The projection output is rounded once to BF16
    (its declared output), then Q and K go through the prologue.  Returns the
    BF16 bit patterns of q', k', v and the projections q, k."""
    B, S, D = x.shape
    H = D // HD
    y = orc.stream_linear(orc.widen(x), orc.widen(W), bias, T_txt)
    yb = orc.cast_bf16(y)
    q, k, v = (yb[..., i * D:(i + 1) * D].reshape(B, S, H, HD) for i in range(3))
    qp = orc.cast_bf16(orc.qknorm_rope(orc.widen(q), g_q, T_txt, h, w))
    kp = orc.cast_bf16(orc.qknorm_rope(orc.widen(k), g_k, T_txt, h, w))
    return dict(q=q, k=k, v=v, q_prime=qp, k_prime=kp, y=y)
