"""Shared helpers of the GPU tests: tolerance checks and tensor conversions.

The floating-point bound is the one the path is specified with:
|gpu - oracle| <= 1e-2 * |oracle| + 2e-3 elementwise for BF16 outputs and the
FP32 gradients, and <= 1e-4 absolute for the FP32 debug output of the prologue
and for the LSE (values that carry no BF16 operand rounding).
"""
import numpy as np
import torch

RTOL, ATOL = 1e-2, 2e-3
DEBUG_ATOL = 1e-4


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bytes of a tensor as an integer array (for bit-exact comparison)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    raise TypeError(t.dtype)


def mixed_check(gpu, ref, name, rtol=RTOL, atol=ATOL, mask=None):
    g, r = f64(gpu), f64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(r).all(), f"{name}: oracle not finite"
    err = np.abs(g - r)
    bound = rtol * np.abs(r) + atol
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), g.shape)
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements outside |d| <= {rtol}|ref|+{atol}; "
                             f"worst at {i}: gpu={g[i]!r} ref={r[i]!r} (max abs err {err.max():.3e})")
    return float(err.max()) if err.size else 0.0


def abs_check(gpu, ref, name, atol=DEBUG_ATOL, mask=None):
    g, r = f64(gpu), f64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    err = np.abs(g - r)
    if not (err <= atol).all():
        i = np.unravel_index(np.argmax(err), g.shape)
        raise AssertionError(f"{name}: max abs err {err.max():.3e} > {atol} at {i}: gpu={g[i]!r} ref={r[i]!r}")
    return float(err.max()) if err.size else 0.0


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
