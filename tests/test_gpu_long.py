"""GPU tests at sizes beyond the reference shapes: a long sequence (26,112
tokens, 25,600 image keys and a padded text of 512), many heads (40 x 128),
and a long backward (6,400 tokens).  Sampled rows against the oracle, and
every row's bytes against its run alone."""
import numpy as np
import pytest
import torch

import workloads
from oracle import Oracle
from parity import abs_check, f64, mixed_check

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(wl, **kw):
    inp = workloads.make_inputs(wl, **kw)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    return inp, g, geo


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("spec", [
    ("long_seq", 2, 2, 512, (300, 0), 160, 160),  # S = 26112
    ("many_heads", 1, 40, 96, (77,), 24, 30),     # 40 x 128 channels per token
], ids=["long_seq", "many_heads"])
def test_forward_beyond_reference_shapes(spec):
    name, B, H, T, Ls, h, w = spec
    print(f"forward: {spec}", flush=True)
    wl = workloads.custom(name, B, H, T, Ls, h, w, 900)
    inp, g, geo = _inputs(wl)
    q, k, vt = qi.qkv_prologue(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo)
    o, lse = qi.joint_attn_fwd_vtiles(q, k, vt, geo)
    torch.cuda.synchronize()
    orc = Oracle("f32")
    S = wl.S
    qn, kn, vn = f64(q), f64(k), f64(inp["v"].float())
    rows = [(0, 64), (max(0, T - 32), T + 32), (S // 2, S // 2 + 64), (S - 64, S)]
    for b in range(B):
        for hh in (0, H - 1):
            for s0, s1 in rows:
                ro, rl = orc.attn_fwd_bh(qn[b, :, hh], kn[b, :, hh], vn[b, :, hh], T, wl.txt_len[b], s0, s1)
                mixed_check(o[b, s0:s1, hh], ro, f"O b{b} h{hh} rows {s0}:{s1}")
                abs_check(lse[b, hh, s0:s1], rl, f"LSE b{b} h{hh} rows {s0}:{s1}")
    # each row alone gives the same bytes
    for b in range(B):
        g1 = qi.Geometry(B=1, H=H, T_txt=T, grid_h=h, grid_w=w, txt_len=[wl.txt_len[b]])
        q1, k1, vt1 = qi.qkv_prologue(g["q"][b:b + 1].contiguous(), g["k"][b:b + 1].contiguous(),
                                      g["v"][b:b + 1].contiguous(), g["g_q"], g["g_k"], g1)
        o1, l1 = qi.joint_attn_fwd_vtiles(q1, k1, vt1, g1)
        torch.cuda.synchronize()
        assert _same(o1, o[b:b + 1]) and _same(l1, lse[b:b + 1]), f"row {b} alone"


def test_backward_long_sequence():
    wl = workloads.custom("long_bwd", 1, 1, 256, (200,), 64, 96, 901, backward=True)  # S = 6400
    print("backward: S = 6400", flush=True)
    inp, g, geo = _inputs(wl)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of)
    r = qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    orc = Oracle("f32")
    dqp, dkp, dv = orc.attn_bwd(f64(q), f64(k), f64(inp["v"].float()), f64(inp["dO"].float()), wl.txt_len, wl.T_txt)
    dq, dgq = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["q"])), inp["g_q"].numpy(), dqp, wl.T_txt, wl.h, wl.w)
    dk, dgk = orc.qknorm_rope_bwd(orc.widen(workloads.bits(inp["k"])), inp["g_k"].numpy(), dkp, wl.T_txt, wl.h, wl.w)
    mixed_check(r["dv"], dv, "dv")
    mixed_check(r["dq"], dq, "dq")
    mixed_check(r["dk"], dk, "dk")
    mixed_check(r["dgain_q_ps"], dgq, "dgain_q")
    mixed_check(r["dgain_k_ps"], dgk, "dgain_k")
    L = wl.txt_len[0]
    assert not r["dv"][0, L:wl.T_txt].any() and not r["dk"][0, L:wl.T_txt].any()
