"""Strict arithmetic on the GPU: the probe that gates every device flips for
a fast-math build, and the exponential the softmax uses (the gfx950
instruction v_exp_f32 behind __builtin_amdgcn_exp2f) stays within its stated
accuracy, checked against float64 exp2 of the same FP32 argument.

Pages: [Kernel list] "[RFC] [Qwen-Image] WS1 Single-GPU Kernel List", rule 4
(no fast math, no fast exponential intrinsics); [PR 537] "[WS1][Qwen-Image]
[CUDA] AdaLN modulation projection (adaln_mod_projection)", a probe of the
built arithmetic that must flip under fast math.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FASTMATH_LIB = os.path.join(os.path.dirname(qi.LIB_PATH), "libqi_probe_fastmath.so")

# c = log2(e)/sqrt(128) rounded once to FP32, as the kernels hold it
KC = np.float32(1.4426950408889634074 / 11.313708498984760390)


def test_probe_passes_on_the_strict_build():
    qi.strict_probe(0)


def test_probe_fails_on_a_fast_math_build():
    """The same probe source built with -ffast-math (contraction, approximate
    division and square root, finite-math folding) reports QI_E_STRICT."""
    assert os.path.exists(FASTMATH_LIB), "build() writes libqi_probe_fastmath.so beside libqi.so"
    lib = ctypes.CDLL(FASTMATH_LIB)
    lib.qi_probe_standalone.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int]
    lib.qi_probe_standalone.restype = ctypes.c_int
    msg = ctypes.create_string_buffer(256)
    rc = lib.qi_probe_standalone(0, msg, 256)
    assert rc == 6, (rc, msg.value.decode())
    assert b"strict probe failed" in msg.value


def _ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of FP32 at |x| (2^-149 in the subnormal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 23)


def test_exp2_rescale_factor_accuracy():
    """alpha of the unfused softmax is one exp2 of an FP32 argument
    (m_old - m_new) * c.  Scores whose tile maxima climb by 63..1263 raw
    units per tile give arguments from -8 down to -161; alpha must be within
    1 ulp of float64 exp2 of the same FP32 argument where the result is a
    normal FP32 number, and +0 below 2^-126 (the instruction does not return
    subnormal results).  Tile 0 starts from an empty state: alpha = 0."""
    rows, tiles = 4096, 64
    geo = qi.Geometry(B=1, H=1, T_txt=0, grid_h=64, grid_w=64, txt_len=[0])
    assert qi.key_slots(geo) == 64 * tiles
    s = workloads.staircase_scores(rows, tiles, seed=11)
    _, alpha, _, _ = qi.joint_attn_softmax(s.to(DEV), geo)
    torch.cuda.synchronize()
    a = alpha[0, 0].cpu().numpy()  # [tiles, rows]
    assert (a[0] == 0).all()
    lv = s[0, 0, :, ::64].numpy()  # [rows, tiles] tile maxima (FP32)
    d = (lv[:, :-1] - lv[:, 1:]).astype(np.float32)  # FP32 subtraction, as on the GPU
    arg = (d * KC).astype(np.float32)  # FP32 product (no contraction)
    exact = np.exp2(arg.astype(np.float64))
    got = a[1:].T.astype(np.float64)
    assert arg.max() < -8 and arg.min() < -150
    normal = exact >= 2.0 ** -126
    err_ulp = np.abs(got - exact) / _ulp(exact)
    assert normal.sum() > 100000 and (~normal).sum() > 5000
    worst = float(err_ulp[normal].max())
    assert worst <= 1.0, f"exp2 error {worst:.3f} ulp on normal results"
    assert (got[~normal] == 0).all(), "results below 2^-126 come back as +0"
    assert not np.signbit(got).any()
