"""A NumPy model of the GPU kernels' operand roundings, for choosing them.

Not a reference and not the oracle: it replays the attention forward and
backward with the roundings a kernel design applies (P in BF16 or FP16, V
scaled by 2^-8 into FP16, dS in BF16, split BF16 hi + lo or FP16 under a power
of two, D from the BF16 or the FP32 O) and everything else in FP32, so that
its error against exact arithmetic can be compared with the tolerance
1e-2 * |ref| + 2e-3 before a kernel is built.  FP32 matrix products stand in
for the MFMA's FP32 accumulation (their summation orders differ; both keep
FP32 rounding, ~1e-7 relative, far below the effects studied).
"""
from __future__ import annotations

import numpy as np
import torch

LOG2E = 1.4426950408889634074
INV_SQRT_D = 1.0 / 11.313708498984760390
C = np.float32(LOG2E * INV_SQRT_D)


def bf16(x) -> np.ndarray:
    """Round to BF16 (nearest even), returned as float32."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def fp16(x) -> np.ndarray:
    """Round to FP16 (nearest even, subnormals kept), returned as float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def pow2_scale(amax: float, top: int = 14) -> float:
    """2^e with amax * 2^e in [2^top, 2^(top+1)) (1 for amax = 0)."""
    if amax <= 0 or not np.isfinite(amax):
        return 1.0
    return float(2.0 ** (top - np.floor(np.log2(amax))))


def round_p(p, mode):
    if mode == "fp32":
        return p
    if mode == "bf16":
        return bf16(p)
    if mode == "fp16":
        return fp16(p)
    raise ValueError(mode)


def forward(q, k, v, keys, p_mode="fp16", v_mode="fp16_scaled"):
    """One (batch, head) slice: q, k, v float32 [S, 128] (already BF16
    values), keys = indices of the valid keys.  Returns (O before the BF16
    cast, O after it, LSE), all float64."""
    kv, vv = k[keys], v[keys]
    s = (q @ kv.T).astype(np.float32)
    m = s.max(axis=1, keepdims=True)
    p = np.exp2((s * C - m * C).astype(np.float32)).astype(np.float32)
    l = p.sum(axis=1, dtype=np.float32)
    pr = round_p(p, p_mode)
    if v_mode == "fp16_scaled":
        vr, vs = fp16(vv * np.float32(2.0 ** -8)), np.float32(2.0 ** -8)
    elif v_mode == "bf16":
        vr, vs = vv, np.float32(1.0)
    else:
        raise ValueError(v_mode)
    acc = (pr @ vr).astype(np.float32)
    o = (acc / (l * vs)[:, None]).astype(np.float32)
    lse = (m[:, 0] * C + np.log2(l)) * np.float32(np.log(2.0))
    return o.astype(np.float64), bf16(o).astype(np.float64), lse.astype(np.float64)


def backward(q, k, v, dO, lse, o_for_D, keys, ds_mode="hilo", dv_mode="fp16_scaled"):
    """Attention gradients of one slice with the kernel's roundings: returns
    dq', dk', dv (float64) for the valid keys (dk', dv rows of `keys`)."""
    kv, vv = k[keys], v[keys]
    s = (q @ kv.T).astype(np.float32)
    p = np.exp2((s * C - (lse.astype(np.float32) * np.float32(LOG2E))[:, None]).astype(np.float32))
    dp = (dO @ vv.T).astype(np.float32)
    D = (dO * o_for_D).sum(axis=1, dtype=np.float32)
    ds = (p * (dp - D[:, None])).astype(np.float32)
    if ds_mode == "fp32":
        dq = ds @ kv
        dk = ds.T @ q
    elif ds_mode == "bf16":
        h = bf16(ds)
        dq, dk = h @ kv, h.T @ q
    elif ds_mode == "hilo":
        h = bf16(ds)
        lo = bf16(ds - h)
        dq = (h @ kv).astype(np.float32) + (lo @ kv).astype(np.float32)
        dk = (h.T @ q).astype(np.float32) + (lo.T @ q).astype(np.float32)
    elif ds_mode == "fp16_scaled":
        e = pow2_scale(float(np.abs(ds).max()))
        h = fp16(ds * np.float32(e))
        dq = (h @ kv).astype(np.float32) / np.float32(e)
        dk = (h.T @ q).astype(np.float32) / np.float32(e)
    else:
        raise ValueError(ds_mode)
    if dv_mode == "fp16_scaled":
        e = pow2_scale(float(np.abs(dO).max()))
        dv = (fp16(p).T @ fp16(dO * np.float32(e))).astype(np.float32) / np.float32(e)
    elif dv_mode == "bf16":
        dv = bf16(p).T @ dO
    else:
        raise ValueError(dv_mode)
    f = lambda a: np.asarray(a, dtype=np.float64) * INV_SQRT_D  # noqa: E731
    return f(dq), f(dk), np.asarray(dv, dtype=np.float64)


def exact_forward(q, k, v, keys):
    """float64 softmax attention of one slice over the valid keys."""
    q, kv, vv = (np.asarray(t, dtype=np.float64) for t in (q, k[keys], v[keys]))
    s = q @ kv.T * INV_SQRT_D
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1)
    return (e @ vv) / l[:, None], m[:, 0] + np.log(l)


def exact_backward(q, k, v, dO, keys):
    """float64 gradients of one slice (O from the exact forward)."""
    q, kv, vv, g = (np.asarray(t, dtype=np.float64) for t in (q, k[keys], v[keys], dO))
    s = q @ kv.T * INV_SQRT_D
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ vv
    ds = p * (g @ vv.T - (g * o).sum(axis=1, keepdims=True))
    return ds @ kv * INV_SQRT_D, ds.T @ q * INV_SQRT_D, p.T @ g


def ratio(x, ref, rtol=1e-2, atol=2e-3) -> float:
    """max |x - ref| / (rtol |ref| + atol): above 1 means outside the bound."""
    return float(np.max(np.abs(np.asarray(x) - ref) / (rtol * np.abs(ref) + atol)))
