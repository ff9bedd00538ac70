"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small shapes are compared element by element over every output; the full
reference shapes are compared on sampled (batch, head, row-range) slices the
oracle computes one by one, in the same launch configuration bench.py times.
"""
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import Oracle, fold_batch
from parity import DEBUG_ATOL, ParityStats, abs_check, f64, mixed_check

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def orc():
    return Oracle("f32")


def gpu_inputs(wl, **kw):
    inp = workloads.make_inputs(wl, **kw)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return inp, g


def geom_of(wl, txt_len=None, gain_streams=1, B=None):
    return qi.Geometry(B=wl.B if B is None else B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w,
                       txt_len=list(wl.txt_len if txt_len is None else txt_len), gain_streams=gain_streams)


SMALL = [  # name, B, H, T_txt, txt_len, h, w
    ("tiny", 1, 2, 8, (5,), 4, 4),
    ("ragged_odd", 2, 3, 7, (0, 7), 5, 3),
    ("one_image_token", 2, 1, 3, (0, 2), 1, 1),
    ("no_text", 1, 2, 0, (0,), 6, 5),
    ("multi_tile", 2, 2, 100, (77, 3), 13, 11),
    ("wide", 1, 3, 70, (64,), 9, 20),
]


def small_wl(spec, seed=100, backward=False):
    name, B, H, T, Ls, h, w = spec
    return workloads.custom(name, B, H, T, Ls, h, w, seed, backward=backward)


def test_strict_probe():
    qi.strict_probe(0)


def test_trace_mentions_mfma():
    assert "v_mfma_f32_32x32x16_bf16" in qi.trace()


# ------------------------------------------------------------------ prologue
@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("streams", [1, 2])
def test_prologue_small(orc, spec, streams):
    wl = small_wl(spec)
    inp, g = gpu_inputs(wl, gain_streams=streams)
    geo = geom_of(wl, gain_streams=streams)
    for name, gain in (("q", "g_q"), ("k", "g_k")):
        yf = torch.empty(g[name].shape, dtype=torch.float32, device=DEV)
        y = qi.qknorm_rope(g[name], g[gain], geo, out_f32=yf)
        torch.cuda.synchronize()
        ref = orc.qknorm_rope(orc.widen(workloads.bits(inp[name])), inp[gain].numpy(), wl.T_txt, wl.h, wl.w)
        abs_check(yf, ref, f"{name}' fp32")
        mixed_check(y, ref, f"{name}' bf16")
        # the BF16 output is the single RNE cast of the FP32 value
        assert torch.equal(y.cpu(), yf.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("cfg", ["1024sq", "1328sq_cfg", "1664x928"])
def test_prologue_full(orc, cfg):
    wl = workloads.WORKLOADS[cfg]
    inp, g = gpu_inputs(wl)
    geo = geom_of(wl)
    yf = torch.empty(g["q"].shape, dtype=torch.float32, device=DEV)
    y = qi.qknorm_rope(g["q"], g["g_q"], geo, out_f32=yf)
    torch.cuda.synchronize()
    ref = orc.qknorm_rope(orc.widen(workloads.bits(inp["q"])), inp["g_q"].numpy(), wl.T_txt, wl.h, wl.w)
    s32 = ParityStats(f"{cfg} q' (FP32)", rtol=0.0, atol=DEBUG_ATOL)
    s16 = ParityStats(f"{cfg} q' (BF16)")
    abs_check(yf, ref, "q' fp32", stats=s32)
    mixed_check(y, ref, "q' bf16", stats=s16)
    print(s32.line(), flush=True)
    print(s16.line(), flush=True)


# ------------------------------------------------------------------- forward
def _fwd_all(g, geo, with_f32=False):
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV) if with_f32 else None
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of)
    torch.cuda.synchronize()
    return q, k, o, lse, of


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small(orc, spec):
    wl = small_wl(spec)
    inp, g = gpu_inputs(wl)
    geo = geom_of(wl)
    q, k, o, lse, of = _fwd_all(g, geo, with_f32=True)
    # isolation: the oracle attends over the GPU's own q', k'
    ro, rl = orc.attn_fwd(f64(q), f64(k), f64(inp["v"].float()), wl.txt_len, wl.T_txt)
    mixed_check(o, ro, "O bf16")
    mixed_check(of, ro, "O fp32")
    abs_check(lse, rl, "LSE")
    # end to end from the raw inputs
    from oracle import forward_path
    fw = forward_path(orc, workloads.bits(inp["q"]), workloads.bits(inp["k"]), workloads.bits(inp["v"]),
                      inp["g_q"].numpy(), inp["g_k"].numpy(), wl.txt_len, wl.T_txt, wl.h, wl.w)
    mixed_check(o, fw["o"], "O end-to-end")
    abs_check(lse, fw["lse"], "LSE end-to-end", atol=2e-3)


@pytest.mark.parametrize("cfg", ["1024sq", "1328sq_cfg", "1664x928"])
def test_forward_full_every_element(orc, cfg):
    """O and LSE of every row of every head of every sample at the full
    reference shapes, against the oracle over the GPU's own q', k' (the
    launch configuration the benchmark times)."""
    wl = workloads.WORKLOADS[cfg]
    inp, g = gpu_inputs(wl)
    geo = geom_of(wl)
    q, k, o, lse, _ = _fwd_all(g, geo)
    qn, kn, on, ln = f64(q), f64(k), f64(o), f64(lse)
    vn = f64(inp["v"].float())
    so, sl = ParityStats(f"{cfg} O (BF16)"), ParityStats(f"{cfg} LSE (FP32)", rtol=0.0, atol=DEBUG_ATOL)
    for b in range(wl.B):
        for h in range(wl.H):
            ro, rl = orc.attn_fwd_bh(qn[b, :, h], kn[b, :, h], vn[b, :, h], wl.T_txt, wl.txt_len[b], 0, wl.S)
            mixed_check(on[b, :, h], ro, f"O b{b} h{h}", stats=so, where=(b, h))
            abs_check(ln[b, h], rl, f"LSE b{b} h{h}", stats=sl, where=(b, h))
        print(f"{cfg}: sample {b}, {wl.H} heads x {wl.S} rows checked", flush=True)
    print(so.line(), flush=True)
    print(sl.line(), flush=True)


def test_forward_constant_v_and_scaling():
    """V enters A.V as FP16 of v * 2^-8, which is exact for BF16 values of
    magnitude 2^-9 and above (multiples of 2^-16 after the scale); with such
    a V the weights' exact normalisation returns a constant V bit for bit and
    doubling V doubles O and leaves LSE alone.  Smaller |v| keep an absolute
    error below 2^-17 before the output cast."""
    wl = small_wl(("c", 1, 2, 40, (29,), 9, 7), seed=5)
    inp, g = gpu_inputs(wl)
    geo = geom_of(wl)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    tiny = g["v"].abs() < 2.0 ** -9
    v = torch.where(tiny, torch.zeros_like(g["v"]), g["v"])
    vc = v[:, :1].expand_as(v).contiguous()
    oc, _ = qi.joint_attn_fwd(q, k, vc, geo)
    assert torch.equal(oc, vc), "constant V must be returned exactly"
    o1, l1 = qi.joint_attn_fwd(q, k, v, geo)
    o2, l2 = qi.joint_attn_fwd(q, k, (v.float() * 2).to(torch.bfloat16), geo)
    assert torch.equal(o2, (o1.float() * 2).to(torch.bfloat16)) and torch.equal(l1, l2)
    # large magnitudes (beyond FP16's own range, within the 2^-8 scale's)
    o3, _ = qi.joint_attn_fwd(q, k, (v.float() * 2.0 ** 14).to(torch.bfloat16), geo)
    assert torch.equal(o3, (o1.float() * 2.0 ** 14).to(torch.bfloat16))
    # tiny magnitudes: a constant V of values below 2^-9 comes back within the FP16 quantum
    vt = (g["v"][:, :1] * 2.0 ** -12).to(torch.bfloat16).expand_as(v).contiguous()
    ot, _ = qi.joint_attn_fwd(q, k, vt, geo)
    err = (ot.float() - vt.float()).abs().max().item()
    assert err <= 2.0 ** -16, err


# ------------------------------------------------------------------ backward
def _bwd_all(g, geo):
    q, k, o, lse, of = _fwd_all(g, geo, with_f32=True)
    r = qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    return q, k, o, lse, r


BWD_SMALL = [s for s in SMALL if s[0] != "wide"] + [("wide", 1, 3, 70, (64,), 9, 20)]


@pytest.mark.parametrize("spec", BWD_SMALL, ids=[s[0] for s in BWD_SMALL])
@pytest.mark.parametrize("streams", [1, 2])
def test_backward_small(orc, spec, streams):
    wl = small_wl(spec, backward=True)
    inp, g = gpu_inputs(wl, gain_streams=streams)
    geo = geom_of(wl, gain_streams=streams)
    q, k, o, lse, r = _bwd_all(g, geo)
    # oracle: attention gradients at the GPU's q', k' (isolation), then the
    # prologue backward from the raw inputs
    dqp, dkp, dv = orc.attn_bwd(f64(q), f64(k), f64(inp["v"].float()), f64(inp["dO"].float()), wl.txt_len, wl.T_txt)
    dq, dgq = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["q"])), inp["g_q"].numpy(), dqp, wl.T_txt, wl.h, wl.w)
    dk, dgk = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["k"])), inp["g_k"].numpy(), dkp, wl.T_txt, wl.h, wl.w)
    mixed_check(r["dv"], dv, "dv")
    mixed_check(r["dq"], dq, "dq")
    mixed_check(r["dk"], dk, "dk")
    mixed_check(r["dgain_q_ps"], dgq, "dgain_q per sample")
    mixed_check(r["dgain_k_ps"], dgk, "dgain_k per sample")
    mixed_check(r["dgain_q"], fold_batch(dgq), "dgain_q")
    mixed_check(r["dgain_k"], fold_batch(dgk), "dgain_k")
    # masked keys receive exactly zero
    for b in range(wl.B):
        L = wl.txt_len[b]
        assert not r["dv"][b, L:wl.T_txt].any() and not r["dk"][b, L:wl.T_txt].any()


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def test_backward_exactly_linear_in_dO():
    """Every gradient is linear in dO, and the path's arithmetic keeps that
    exact for power-of-two factors: gradients of dO * 2^k are the gradients
    of dO times 2^k, bit for bit (k = -16 and +12 move dO far from unit
    scale; the dV operand's internal scaling must follow).  dO = 0 gives
    exactly zero everywhere."""
    wl = small_wl(BWD_SMALL[4], backward=True)  # multi_tile
    inp, g = gpu_inputs(wl, gain_streams=2)
    geo = geom_of(wl, gain_streams=2)
    q, k, o, lse, r0 = _bwd_all(g, geo)
    for kexp in (-16, 12):
        gs = dict(g, dO=(g["dO"].float() * 2.0 ** kexp).to(torch.bfloat16))
        _, _, _, _, rs = _bwd_all(gs, geo)
        for name, t in r0.items():
            assert _bits_equal(rs[name], t * 2.0 ** kexp), f"{name} at dO * 2^{kexp}"
    gz = dict(g, dO=torch.zeros_like(g["dO"]))
    _, _, _, _, rz = _bwd_all(gz, geo)
    for name, t in rz.items():
        assert not t.any(), f"{name} with dO = 0"
    # one (sample, head) slice of dO scaled by 2^-24: that slice's dq, dk, dv
    # scale exactly, and every other slice keeps its bits
    d1 = g["dO"].clone()
    d1[1, :, 0] = (d1[1, :, 0].float() * 2.0 ** -24).to(torch.bfloat16)
    _, _, _, _, r1 = _bwd_all(dict(g, dO=d1), geo)
    for name in ("dq", "dk", "dv"):
        a, ref = r1[name], r0[name]
        assert _bits_equal(a[1, :, 0], ref[1, :, 0] * 2.0 ** -24), f"{name} of the scaled slice"
        assert _bits_equal(a[0], ref[0]) and _bits_equal(a[1, :, 1:], ref[1, :, 1:]), f"{name} of other slices"


def test_backward_wide_channel_range_dv(orc):
    """dO channels spread over 2^-12 .. 2^12: each dV channel, divided by its
    channel's factor, stays within the bound of the oracle's (the dV operand
    shares one scale per (sample, head), set by that slice's largest
    element)."""
    wl = small_wl(BWD_SMALL[4], seed=105, backward=True)
    inp, g = gpu_inputs(wl)
    geo = geom_of(wl)
    s = 2.0 ** torch.linspace(-12, 12, 128).round()
    dO = (inp["dO"].float() * s).to(torch.bfloat16)
    q, k, o, lse, r = _bwd_all(dict(g, dO=dO.to(DEV)), geo)
    dqp, dkp, dv = orc.attn_bwd(f64(q), f64(k), f64(inp["v"].float()), f64(dO.float()), wl.txt_len, wl.T_txt)
    sn = s.double().numpy()
    mixed_check(f64(r["dv"]) / sn, dv / sn, "dv per channel")


def test_backward_full_config_every_element(orc):
    """The deterministic backward at 1024^2 (B=2: the workload's sample, then
    one more drawn next, both with 219 valid text tokens; 24 heads): every
    element of dq, dk, dv of both samples and the per-sample and folded gain
    gradients against the FP32 oracle.  The attention gradients are taken at
    the GPU's own q', k' (the values the backward consumes); the prologue
    backward runs from the raw inputs."""
    wl = workloads.WORKLOADS["1024sq_bwd"]
    inp, g = gpu_inputs(wl, extra_samples=1)
    txt_len = inp["txt_len"]
    geo = geom_of(wl, txt_len=txt_len, B=2)
    q, k, o, lse, r = _bwd_all(g, geo)
    orc.set_threads(min(16, os.cpu_count() or 1))
    dqp, dkp, dv = orc.attn_bwd(f64(q), f64(k), f64(inp["v"].float()), f64(inp["dO"].float()), txt_len, wl.T_txt)
    dq, dgq = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["q"])), inp["g_q"].numpy(), dqp, wl.T_txt, wl.h, wl.w)
    dk, dgk = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["k"])), inp["g_k"].numpy(), dkp, wl.T_txt, wl.h, wl.w)
    st = {n: ParityStats(f"1024sq_bwd B=2 {n} (FP32)") for n in ("dv", "dq", "dk", "dgain_q", "dgain_k")}
    for b in range(2):
        mixed_check(r["dv"][b], dv[b], f"dv sample {b}", stats=st["dv"], where=(b,))
        mixed_check(r["dq"][b], dq[b], f"dq sample {b}", stats=st["dq"], where=(b,))
        mixed_check(r["dk"][b], dk[b], f"dk sample {b}", stats=st["dk"], where=(b,))
    mixed_check(r["dgain_q_ps"], dgq, "dgain_q per sample", stats=st["dgain_q"])
    mixed_check(r["dgain_k_ps"], dgk, "dgain_k per sample", stats=st["dgain_k"])
    mixed_check(r["dgain_q"], fold_batch(dgq), "dgain_q folded")
    mixed_check(r["dgain_k"], fold_batch(dgk), "dgain_k folded")
    for v in st.values():
        print(v.line(), flush=True)
