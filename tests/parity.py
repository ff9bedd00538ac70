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


class ParityStats:
    """Parity statistics of one output over any number of checked slices:
    elements, failures, fraction within the bound, max abs error, max
    relative error (over elements where the relative term of the bound
    dominates, |ref| > atol / rtol), max error / bound, and where the worst
    element (by error / bound) lies.  The relative error is taken over
    |ref| > rel_floor: atol / rtol by default, 100 * atol for a purely
    absolute bound."""

    def __init__(self, name, rtol=RTOL, atol=ATOL, rel_floor=None):
        self.name, self.rtol, self.atol = name, rtol, atol
        self.rel_floor = rel_floor if rel_floor is not None else (atol / rtol if rtol > 0 else 100.0 * atol)
        self.n = self.bad = self.n_rel = 0
        self.max_abs = self.max_rel = self.max_ratio = 0.0
        self.worst = None

    def add(self, g, r, where=()):
        err = np.abs(g - r)
        bound = self.rtol * np.abs(r) + self.atol
        ratio = err / bound
        self.n += err.size
        self.bad += int((~(err <= bound)).sum())
        if err.size:
            self.max_abs = max(self.max_abs, float(err.max()))
            big = np.abs(r) > self.rel_floor
            self.n_rel += int(big.sum())
            if big.any():
                self.max_rel = max(self.max_rel, float((err[big] / np.abs(r[big])).max()))
            i = np.unravel_index(np.argmax(ratio), ratio.shape)
            if float(ratio[i]) >= self.max_ratio:
                self.max_ratio = float(ratio[i])
                self.worst = tuple(where) + tuple(int(x) for x in i)

    def line(self):
        frac = 100.0 * (self.n - self.bad) / max(self.n, 1)
        return (f"PARITY {self.name}: elements={self.n} within={frac:.4f}% failures={self.bad} "
                f"max_abs={self.max_abs:.3e} max_rel(|ref|>{self.rel_floor:g}, {self.n_rel} elements)={self.max_rel:.3e} max_err/bound={self.max_ratio:.4f} "
                f"worst={self.worst}")


def mixed_check(gpu, ref, name, rtol=RTOL, atol=ATOL, mask=None, stats=None, where=()):
    g, r = f64(gpu), f64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(r).all(), f"{name}: oracle not finite"
    if stats is not None:
        stats.add(g, r, where)
    err = np.abs(g - r)
    bound = rtol * np.abs(r) + atol
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), g.shape)
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements outside |d| <= {rtol}|ref|+{atol}; "
                             f"worst at {i}: gpu={g[i]!r} ref={r[i]!r} (max abs err {err.max():.3e})")
    return float(err.max()) if err.size else 0.0


def abs_check(gpu, ref, name, atol=DEBUG_ATOL, mask=None, stats=None, where=()):
    g, r = f64(gpu), f64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    if stats is not None:
        stats.add(g, r, where)
    err = np.abs(g - r)
    if not (err <= atol).all():
        i = np.unravel_index(np.argmax(err), g.shape)
        raise AssertionError(f"{name}: max abs err {err.max():.3e} > {atol} at {i}: gpu={g[i]!r} ref={r[i]!r}")
    return float(err.max()) if err.size else 0.0


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
