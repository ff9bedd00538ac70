"""Why the kernels round their MMA operands the way they do: a NumPy model of
each candidate rounding (tests/emulation.py) against exact float64
arithmetic, measured as the ratio of the error to the output tolerance
1e-2 * |ref| + 2e-3 (above 1 = the tolerance is broken).

Forward (A.V operands): one BF16 rounding of P and V breaks the bound on
few-key rows with peaked softmax (gains N(3, 0.3)); FP16 P with FP16 V*2^-8
stays at the level of the final BF16 cast of O alone.

Backward (dS operand of dQ' and dK', D term): the gain gradients sum the
gradients of all 4352 x 24 rows of the 1024^2 backward workload and cancel
to values as small as ~0.02, so they are the fragile output.  A single BF16
dS breaks their bound many times over and FP16 dS under a per-(sample, head)
power of two still breaks it; the split dS = bf16(dS) + bf16(dS - bf16(dS))
keeps them far inside, and so does D from the FP32 O.

The pages: [Roadmap] "[RFC][Qwen-Image][CUDA/ROCm] WS1/WS2 kernel roadmap,
ablation matrix and integration plan", "Numerical requirements" (FP32
accumulation, one output cast, declared tolerances); [Kernel list] "[RFC]
[Qwen-Image] WS1 Single-GPU Kernel List", rows joint_attn_av_gemm and the
backward of every operator.
"""
import numpy as np
import pytest

import emulation as E
import workloads
from oracle import Oracle


@pytest.fixture(scope="module")
def orc():
    return Oracle("f32")


def _prologue_bf16(orc, x, g, wl):
    return E.bf16(orc.qknorm_rope(orc.widen(workloads.bits(x)), g.numpy(), wl.T_txt, wl.h, wl.w))


def _keys(wl, b):
    return np.array([j for j in range(wl.S) if j < wl.txt_len[b] or j >= wl.T_txt])


def test_forward_av_operands(orc):
    """Ragged few-key shape (B=2, 16 heads, T_txt=7 with 0 and 7 valid text
    keys, 5x3 image grid) at gains N(3, 0.3)."""
    wl = workloads.custom("ragged16", 2, 16, 7, (0, 7), 5, 3, 5)
    inp = workloads.make_inputs(wl, gain_mean=3.0, gain_std=0.3)
    q = _prologue_bf16(orc, inp["q"], inp["g_q"], wl)
    k = _prologue_bf16(orc, inp["k"], inp["g_k"], wl)
    v = inp["v"].float().numpy()
    worst = {"bf16": 0.0, "fp16": 0.0, "fp32": 0.0}
    for b in range(wl.B):
        keys = _keys(wl, b)
        for h in range(wl.H):
            ex, _ = E.exact_forward(q[b, :, h], k[b, :, h], v[b, :, h], keys)
            for pm, vm in (("bf16", "bf16"), ("fp16", "fp16_scaled"), ("fp32", "bf16")):
                _, ob, _ = E.forward(q[b, :, h], k[b, :, h], v[b, :, h], keys, pm, vm)
                worst[pm] = max(worst[pm], E.ratio(ob, ex))
    assert worst["bf16"] > 1.1, worst       # BF16 P and V: outside the bound
    assert worst["fp16"] < 0.4, worst       # FP16 P, FP16 V*2^-8: inside
    assert worst["fp16"] <= worst["fp32"] * 1.01, worst  # no worse than exact P (the BF16 output cast dominates)


def test_backward_ds_operand_and_D_term(orc):
    """The 1024^2 backward workload (B=1, 24 heads, S=4352): gain gradients
    from the modelled dq', dk' through the oracle's prologue backward, against
    those from exact dq', dk'."""
    o64 = Oracle("f64")
    wl = workloads.WORKLOADS["1024sq_bwd"]
    inp = workloads.make_inputs(wl)
    q = _prologue_bf16(orc, inp["q"], inp["g_q"], wl)
    k = _prologue_bf16(orc, inp["k"], inp["g_k"], wl)
    v, dO = inp["v"].float().numpy(), inp["dO"].float().numpy()
    keys = _keys(wl, 0)
    modes = [("fp32", "hilo"), ("bf16", "hilo"), ("fp32", "bf16"), ("fp32", "fp16_scaled")]
    shape = (1, wl.S, wl.H, 128)
    ex = [np.zeros(shape), np.zeros(shape)]
    got = {m: [np.zeros(shape), np.zeros(shape)] for m in modes}
    elem = {m: 0.0 for m in modes}
    for h in range(wl.H):
        a, b, g = q[0, :, h], k[0, :, h], dO[0, :, h]
        dq, dk, _ = E.exact_backward(a, b, v[0, :, h], g, keys)
        ex[0][0, :, h], ex[1][0, keys, h] = dq, dk
        of, ob, lse = E.forward(a, b, v[0, :, h], keys, "fp16", "fp16_scaled")
        for m in modes:
            o_d = (of if m[0] == "fp32" else ob).astype(np.float32)
            mq, mk, _ = E.backward(a, b, v[0, :, h], g, lse.astype(np.float32), o_d, keys, ds_mode=m[1])
            got[m][0][0, :, h], got[m][1][0, keys, h] = mq, mk
            elem[m] = max(elem[m], E.ratio(mq, dq), E.ratio(mk, dk))
    xq, xk = o64.widen(workloads.bits(inp["q"])), o64.widen(workloads.bits(inp["k"]))
    dg = lambda x, g, d: o64.qknorm_rope_bwd(x, g.numpy(), d, wl.T_txt, wl.h, wl.w)[1]  # noqa: E731
    ref_q, ref_k = dg(xq, inp["g_q"], ex[0]), dg(xk, inp["g_k"], ex[1])
    r = {m: max(E.ratio(dg(xq, inp["g_q"], got[m][0]), ref_q), E.ratio(dg(xk, inp["g_k"], got[m][1]), ref_k))
         for m in modes}
    # elementwise dq', dk' pass with every candidate
    assert max(elem.values()) < 0.5, elem
    # gain gradients: only the hi/lo split (with either D) stays inside
    assert r[("fp32", "hilo")] < 0.25, r
    assert r[("bf16", "hilo")] < 1.0, r
    assert r[("fp32", "bf16")] > 4.0, r
    assert r[("fp32", "fp16_scaled")] > 1.0, r
