"""The library's calls captured in a HIP graph (they allocate nothing and do
not synchronise) replay to the eager bytes: several replays, with eager work
and host synchronisation between them, each compared with the eager result."""
import pytest
import torch

import workloads

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("fused_prologue", [False, True], ids=["separate_prologue", "qkv_prologue"])
@pytest.mark.parametrize("name", ["ragged", "1024sq_bwd"])
def test_graph_replay_matches_eager(name, fused_prologue):
    if name == "ragged":
        wl = workloads.custom("ragged", 3, 2, 130, (0, 67, 130), 9, 11, 500, backward=True)
    else:
        wl = workloads.WORKLOADS[name]
    print(f"graph replay: {wl.name} fused_prologue={fused_prologue}", flush=True)
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    shp = g["q"].shape

    def buffers():
        return dict(qp=torch.empty(shp, dtype=torch.bfloat16, device=DEV),
                    kp=torch.empty(shp, dtype=torch.bfloat16, device=DEV),
                    o=torch.empty(shp, dtype=torch.bfloat16, device=DEV),
                    of=torch.empty(shp, dtype=torch.float32, device=DEV),
                    lse=torch.empty((wl.B, wl.H, wl.S), dtype=torch.float32, device=DEV),
                    fws=torch.empty(qi.fwd_workspace_bytes(geo), dtype=torch.uint8, device=DEV),
                    bws=torch.empty(qi.bwd_workspace_bytes(geo), dtype=torch.uint8, device=DEV),
                    dq=torch.empty(shp, dtype=torch.float32, device=DEV),
                    dk=torch.empty(shp, dtype=torch.float32, device=DEV),
                    dv=torch.empty(shp, dtype=torch.float32, device=DEV))

    def step(b):
        if fused_prologue:
            qi.qkv_prologue(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, q=b["qp"], k=b["kp"], v_tiles=b["fws"])
            qi.joint_attn_fwd_vtiles(b["qp"], b["kp"], b["fws"], geo, out=b["o"], lse=b["lse"], out_f32=b["of"])
        else:
            qi.qknorm_rope(g["q"], g["g_q"], geo, out=b["qp"])
            qi.qknorm_rope(g["k"], g["g_k"], geo, out=b["kp"])
            qi.joint_attn_fwd(b["qp"], b["kp"], g["v"], geo, out=b["o"], lse=b["lse"], out_f32=b["of"],
                              workspace=b["fws"])
        r = qi.joint_attn_bwd(g["q"], g["k"], b["qp"], b["kp"], g["v"], b["of"], b["lse"], g["dO"], g["g_q"], g["g_k"],
                              geo, workspace=b["bws"], dq=b["dq"], dk=b["dk"], dv=b["dv"])
        return r

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    keys = ("qp", "kp", "o", "of", "lse", "dq", "dk", "dv")
    ref = {k: eager[k].clone() for k in keys}

    gb = buffers()
    step(gb)  # first call outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb)
    for rep in range(3):
        for k in keys:
            gb[k].zero_()
        torch.cuda.synchronize()
        graph.replay()
        step(eager)  # eager work on other buffers between replays
        torch.cuda.synchronize()
        for k in keys:
            assert _same(gb[k], ref[k]), f"replay {rep}: {k}"
