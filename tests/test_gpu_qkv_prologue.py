"""GPU tests of the one-launch forward preparation (qi_qkv_prologue: the Q
and K prologues plus the V tile conversion) and of the forward over those
tiles (qi_joint_attn_fwd_vtiles).  Both must give the bytes of the separate
calls -- qi_qknorm_rope twice, then qi_joint_attn_fwd -- on ragged small
shapes, both gain layouts, and the three full reference shapes."""
import pytest
import torch

import workloads

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SMALL = [  # name, B, H, T_txt, txt_len, h, w
    ("tiny", 1, 2, 8, (5,), 4, 4),
    ("ragged_odd", 2, 3, 7, (0, 7), 5, 3),
    ("one_image_token", 2, 1, 3, (0, 2), 1, 1),
    ("no_text", 1, 2, 0, (0,), 6, 5),
    ("multi_tile", 3, 2, 100, (77, 3, 100), 13, 11),
]


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check(wl, streams):
    inp = workloads.make_inputs(wl, gain_streams=streams)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len),
                      gain_streams=streams)
    nbytes = qi.fwd_workspace_bytes(geo)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    vt = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of, workspace=ws)
    qf, kf, _ = qi.qkv_prologue(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, v_tiles=vt)
    of2 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o2, lse2 = qi.joint_attn_fwd_vtiles(qf, kf, vt, geo, out_f32=of2)
    torch.cuda.synchronize()
    assert _same(qf, q), "q'"
    assert _same(kf, k), "k'"
    assert _same(vt, ws), "V tiles"
    assert _same(o2, o), "O"
    assert _same(lse2, lse), "LSE"
    assert _same(of2, of), "O_f32"


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("streams", [1, 2])
def test_fused_prologue_path_small(spec, streams):
    name, B, H, T, Ls, h, w = spec
    print(f"fused prologue path: {spec} streams={streams}", flush=True)
    _check(workloads.custom(name, B, H, T, Ls, h, w, 800), streams)


@pytest.mark.parametrize("cfg", ["1024sq", "1328sq_cfg", "1664x928"])
def test_fused_prologue_path_full(cfg):
    print(f"fused prologue path: {cfg}", flush=True)
    _check(workloads.WORKLOADS[cfg], 2)
