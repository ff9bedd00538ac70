"""qi_joint_attn_fwd_noalloc -- the forward with the library's static
scratch (for callers that cannot allocate) -- against qi_joint_attn_fwd
with a caller workspace: O, LSE and O_f32 byte for byte, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
tiles; the second must read only its own)."""
import pytest
import torch

import workloads
from parity import bits

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(wl):
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    return geo, q, k, g["v"]


def _outputs(geo, like):
    o = torch.empty(like.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((geo.B, geo.H, geo.S), dtype=torch.float32, device=DEV)
    of = torch.empty(like.shape, dtype=torch.float32, device=DEV)
    return o, lse, of


def test_noalloc_forward_equals_workspace_forward():
    cases = [workloads.WORKLOADS["1024sq"],
             workloads.custom("smaller", 2, 2, 100, (77, 3), 13, 11, 41)]
    for wl in cases:  # the second call is the smaller one
        geo, q, k, v = _case(wl)
        o1, l1, f1 = _outputs(geo, q)
        qi.joint_attn_fwd(q, k, v, geo, out=o1, lse=l1, out_f32=f1)
        o2, l2, f2 = _outputs(geo, q)
        for t in (o2, l2, f2):
            t.fill_(float("nan"))
        qi.joint_attn_fwd_noalloc(q, k, v, geo, out=o2, lse=l2, out_f32=f2)
        torch.cuda.synchronize()
        for name, a, b in (("O", o1, o2), ("LSE", l1, l2), ("O_f32", f1, f2)):
            assert (bits(a) == bits(b)).all(), f"{name} differs at {wl.name}"


def test_noalloc_forward_refuses_geometries_beyond_its_scratch():
    wl = workloads.WORKLOADS["1664x928"]  # 4 x 24 x 103 key tiles: 155 MiB of V tiles
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    x = torch.zeros((wl.B, wl.S, wl.H, 128), dtype=torch.bfloat16, device=DEV)
    o, lse, of = _outputs(geo, x)
    with pytest.raises(qi.QiError) as e:
        qi.joint_attn_fwd_noalloc(x, x, x, geo, out=o, lse=lse, out_f32=of)
    assert e.value.code == 5 and "static scratch" in str(e.value)
