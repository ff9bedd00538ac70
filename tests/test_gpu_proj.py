"""GPU tests of the projections around the attention: the per-stream packed
QKV projection (with and without the fused Q/K prologue) and the per-stream
output projection.

* Projections against the oracle's per-stream linear layer (BF16 outputs,
  the path's mixed bound), on ragged small shapes and on sampled rows of the
  1024^2 shape.
* The fused Q/K prologue equals the unfused projection followed by
  qi_qknorm_rope byte for byte (small shapes and the full 1024^2 shape), and
  the fused q', k' are within the bound of the oracle's projection ->
  BF16 -> prologue.
* A row's bytes do not depend on the batch it was computed in.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import Oracle, qkv_path
from parity import f64, mixed_check

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HD = 128

SMALL = [  # name, B, H, T_txt, txt_len, h, w, weight streams, gain streams
    ("tiny", 1, 2, 8, (5,), 4, 4, 2, 1),
    ("ragged_h3", 2, 3, 130, (0, 130), 9, 11, 2, 2),
    ("one_stream", 1, 2, 0, (0,), 15, 20, 1, 1),
    ("wide_text", 2, 4, 300, (17, 300), 3, 5, 2, 2),
]


def _case(spec, seed=600):
    name, B, H, T, Ls, h, w, ws, gs = spec
    wl = workloads.custom(name, B, H, T, Ls, h, w, seed)
    geo = qi.Geometry(B=B, H=H, T_txt=T, grid_h=h, grid_w=w, txt_len=list(Ls), gain_streams=gs)
    p = workloads.proj_inputs(wl, streams=ws)
    p["g_q"], p["g_k"] = p["g_q"][:gs].contiguous(), p["g_k"][:gs].contiguous()
    return wl, geo, p


def _dev(p):
    return {k: v.to(DEV) for k, v in p.items()}


def _bits(t):
    return workloads.bits(t.cpu())


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _view4(t, H):
    B, S, D = t.shape
    return t.view(B, S, H, HD)


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_qkv_proj_against_oracle(spec):
    wl, geo, p = _case(spec)
    print(f"qkv projection: {spec}", flush=True)
    d = _dev(p)
    x = _view4(d["x"], wl.H)
    q, k, v = qi.qkv_proj(x, d["w_qkv"], d["b_qkv"], geo, fuse_prologue=False)
    qf, kf, vf = qi.qkv_proj(x, d["w_qkv"], d["b_qkv"], geo, gain_q=d["g_q"], gain_k=d["g_k"], fuse_prologue=True)
    qp = qi.qknorm_rope(q, d["g_q"], geo)
    kp = qi.qknorm_rope(k, d["g_k"], geo)
    torch.cuda.synchronize()
    # fused == projection, then the prologue
    assert _same(qf, qp) and _same(kf, kp) and _same(vf, v)
    orc = Oracle("f32")
    ref = qkv_path(orc, _bits(p["x"]), _bits(p["w_qkv"]), p["b_qkv"].numpy(), p["g_q"].numpy(), p["g_k"].numpy(),
                   wl.T_txt, wl.h, wl.w)
    y = ref["y"]
    D = wl.H * HD
    for i, t in enumerate((q, k, v)):
        mixed_check(t, y[..., i * D:(i + 1) * D].reshape(t.shape), f"section {i}")
    mixed_check(qf, orc.widen(ref["q_prime"]), "q'")
    mixed_check(kf, orc.widen(ref["k_prime"]), "k'")


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_out_proj_against_oracle(spec):
    wl, geo, p = _case(spec, seed=601)
    d = _dev(p)
    o = _view4(d["o"], wl.H)
    y = qi.attn_out_proj(o, d["w_o"], d["b_o"], geo)
    torch.cuda.synchronize()
    orc = Oracle("f32")
    ref = orc.stream_linear(orc.widen(_bits(p["o"])), orc.widen(_bits(p["w_o"])), p["b_o"].numpy(), wl.T_txt)
    mixed_check(y, ref.reshape(y.shape), "y")


def test_projection_rows_independent_of_batch():
    spec = SMALL[3]
    wl, geo, p = _case(spec, seed=602)
    d = _dev(p)
    x = _view4(d["x"], wl.H)
    o = _view4(d["o"], wl.H)
    full = qi.qkv_proj(x, d["w_qkv"], d["b_qkv"], geo, gain_q=d["g_q"], gain_k=d["g_k"])
    yo = qi.attn_out_proj(o, d["w_o"], d["b_o"], geo)
    for b in range(wl.B):
        g1 = qi.Geometry(B=1, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=[wl.txt_len[b]],
                         gain_streams=geo.gain_streams)
        one = qi.qkv_proj(x[b:b + 1].contiguous(), d["w_qkv"], d["b_qkv"], g1, gain_q=d["g_q"], gain_k=d["g_k"])
        y1 = qi.attn_out_proj(o[b:b + 1].contiguous(), d["w_o"], d["b_o"], g1)
        torch.cuda.synchronize()
        for a_, b_ in zip(one, full):
            assert _same(a_, b_[b:b + 1])
        assert _same(y1, yo[b:b + 1])


def test_projections_full_1024sq():
    """The 1024^2 shape (24 heads, D = 3072, two weight streams): fused ==
    unfused + prologue over every element; sampled token rows against the
    oracle."""
    wl = workloads.WORKLOADS["1024sq"]
    geo = qi.Geometry(B=1, H=24, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len),
                      gain_streams=2)
    print("projections at 1024^2", flush=True)
    p = workloads.proj_inputs(wl, streams=2)
    d = _dev(p)
    x = _view4(d["x"], 24)
    o = _view4(d["o"], 24)
    q, k, v = qi.qkv_proj(x, d["w_qkv"], d["b_qkv"], geo, fuse_prologue=False)
    qf, kf, vf = qi.qkv_proj(x, d["w_qkv"], d["b_qkv"], geo, gain_q=d["g_q"], gain_k=d["g_k"])
    qp = qi.qknorm_rope(q, d["g_q"], geo)
    kp = qi.qknorm_rope(k, d["g_k"], geo)
    y = qi.attn_out_proj(o, d["w_o"], d["b_o"], geo)
    torch.cuda.synchronize()
    assert _same(qf, qp) and _same(kf, kp) and _same(vf, v)
    orc = Oracle("f32")
    D = 24 * HD
    rows = np.r_[0:40, 250:262, 2000:2040, wl.S - 40:wl.S]
    xw = orc.widen(_bits(p["x"][0, rows]))
    W = orc.widen(_bits(p["w_qkv"]))
    Wo = orc.widen(_bits(p["w_o"]))
    ow = orc.widen(_bits(p["o"][0, rows]))
    txt = rows < wl.T_txt
    for sel, st in ((txt, 0), (~txt, 1)):
        ref = orc.linear(xw[sel], W[st], p["b_qkv"][st].numpy())
        for i, t in enumerate((q, k, v)):
            mixed_check(t[0, rows[sel]].reshape(-1, D), ref[:, i * D:(i + 1) * D], f"qkv section {i} stream {st}")
        refo = orc.linear(ow[sel], Wo[st], p["b_o"][st].numpy())
        mixed_check(y[0, rows[sel]].reshape(-1, D), refo, f"out stream {st}")
