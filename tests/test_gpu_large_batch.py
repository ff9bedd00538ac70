"""Batches larger than one launch holds (64 rows: the per-row text lengths
travel in the kernel arguments): the library splits them into launches of up
to 64 rows, and every row's bytes equal its run alone -- forward, backward,
the key-block forward with merge, the carried key-block chain, the unfused
operators and the projections."""
import pytest
import torch

import workloads

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
B = 67  # two launches: 64 + 3 rows


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.fixture(scope="module")
def case():
    T, h, w = 8, 4, 4
    lens = [(7 * b) % (T + 1) for b in range(B)]  # every length 0..8, in a fixed pattern
    wl = workloads.custom("large_batch", B, 2, T, lens, h, w, seed=700, backward=True)
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=B, H=2, T_txt=T, grid_h=h, grid_w=w, txt_len=lens)
    return wl, g, geo


def _one(wl, b):
    return qi.Geometry(B=1, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=[wl.txt_len[b]])


def _rows(t, b):
    return t[b:b + 1].contiguous()


def test_forward_backward_rows_equal_alone(case):
    wl, g, geo = case
    print("large batch: forward and backward", flush=True)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of)
    r = qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    for b in (0, 1, 63, 64, 65, 66):
        g1 = _one(wl, b)
        of1 = torch.empty((1,) + tuple(q.shape[1:]), dtype=torch.float32, device=DEV)
        o1, l1 = qi.joint_attn_fwd(_rows(q, b), _rows(k, b), _rows(g["v"], b), g1, out_f32=of1)
        r1 = qi.joint_attn_bwd(_rows(g["q"], b), _rows(g["k"], b), _rows(q, b), _rows(k, b), _rows(g["v"], b), of1, l1,
                               _rows(g["dO"], b), g["g_q"], g["g_k"], g1)
        torch.cuda.synchronize()
        assert _same(o1, o[b:b + 1]) and _same(l1, lse[b:b + 1]) and _same(of1, of[b:b + 1]), f"forward row {b}"
        for n in ("dq", "dk", "dv"):
            assert _same(r1[n], r[n][b:b + 1]), f"{n} row {b}"
        assert _same(r1["dgain_q_ps"], r["dgain_q_ps"][b:b + 1]) and _same(r1["dgain_k_ps"], r["dgain_k_ps"][b:b + 1])


def test_blocks_unfused_projections_rows_equal_alone(case):
    wl, g, geo = case
    print("large batch: blocks, unfused, projections", flush=True)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo)
    ou, lu, _ = qi.joint_attn_unfused(q, k, g["v"], geo)
    # two key blocks: text + first image tile (64 keys: all 16 here), then nothing else -> use text / image split
    acc = torch.empty((2, B, 2, wl.S, 128), dtype=torch.float32, device=DEV)
    m = torch.empty((2, B, 2, wl.S), dtype=torch.float32, device=DEV)
    l = torch.empty((2, B, 2, wl.S), dtype=torch.float32, device=DEV)
    qi.joint_attn_fwd_partial(q, k, g["v"], geo, True, 0, 0, acc=acc[0], m=m[0], l=l[0])
    qi.joint_attn_fwd_partial(q, k, g["v"], geo, False, 0, wl.T_img, acc=acc[1], m=m[1], l=l[1])
    om, lm = qi.joint_attn_merge(acc, m, l, geo)
    p = {n: t.to(DEV) for n, t in workloads.proj_inputs(wl, streams=2).items()}
    x = p["x"].view(B, wl.S, 2, 128)
    pq, pk, pv = qi.qkv_proj(x, p["w_qkv"], p["b_qkv"], geo, gain_q=p["g_q"][:1].contiguous(),
                             gain_k=p["g_k"][:1].contiguous())
    y = qi.attn_out_proj(x, p["w_o"], p["b_o"], geo)
    torch.cuda.synchronize()
    assert _same(ou, o) and _same(lu, lse)  # unfused composition == fused, all 67 rows
    for b in (0, 63, 64, 66):
        g1 = _one(wl, b)
        o1, l1 = qi.joint_attn_fwd(_rows(q, b), _rows(k, b), _rows(g["v"], b), g1)
        a1 = torch.empty((2, 1, 2, wl.S, 128), dtype=torch.float32, device=DEV)
        m1 = torch.empty((2, 1, 2, wl.S), dtype=torch.float32, device=DEV)
        l1b = torch.empty((2, 1, 2, wl.S), dtype=torch.float32, device=DEV)
        qi.joint_attn_fwd_partial(_rows(q, b), _rows(k, b), _rows(g["v"], b), g1, True, 0, 0, acc=a1[0], m=m1[0], l=l1b[0])
        qi.joint_attn_fwd_partial(_rows(q, b), _rows(k, b), _rows(g["v"], b), g1, False, 0, wl.T_img, acc=a1[1], m=m1[1],
                                  l=l1b[1])
        om1, lm1 = qi.joint_attn_merge(a1, m1, l1b, g1)
        pq1, pk1, pv1 = qi.qkv_proj(_rows(x, b), p["w_qkv"], p["b_qkv"], g1, gain_q=p["g_q"][:1].contiguous(),
                                    gain_k=p["g_k"][:1].contiguous())
        y1 = qi.attn_out_proj(_rows(x, b), p["w_o"], p["b_o"], g1)
        torch.cuda.synchronize()
        assert _same(o1, o[b:b + 1]) and _same(l1, lse[b:b + 1]), f"forward row {b}"
        assert _same(om1, om[b:b + 1]) and _same(lm1, lm[b:b + 1]), f"merged row {b}"
        for t1, t in ((pq1, pq), (pk1, pk), (pv1, pv), (y1, y)):
            assert _same(t1, t[b:b + 1]), f"projection row {b}"


def test_qkv_prologue_path_equals_separate_calls(case):
    """The one-launch Q/K/V prologue and the forward over its tiles, at a
    batch of two launches: the same bytes as the separate prologues and
    the forward call."""
    wl, g, geo = case
    print("large batch: fused prologue path", flush=True)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo)
    qf, kf, vt = qi.qkv_prologue(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo)
    of_, lf = qi.joint_attn_fwd_vtiles(qf, kf, vt, geo)
    torch.cuda.synchronize()
    assert _same(qf, q) and _same(kf, k)
    assert _same(of_, o) and _same(lf, lse)


def test_carried_chain_over_two_launches(case):
    """The carried key-block forward at a batch of two launches: text block,
    then the image keys in two tile-aligned blocks, the state continued in
    place; every row equals the whole-row forward byte for byte (the state
    offsets of the second launch included)."""
    wl, g, geo = case
    print("large batch: carried chain", flush=True)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of)
    st = (torch.full((B, 2, wl.S, 128), float("nan"), dtype=torch.float32, device=DEV),
          torch.full((B, 2, wl.S), float("nan"), dtype=torch.float32, device=DEV),
          torch.full((B, 2, wl.S, 2), float("nan"), dtype=torch.float32, device=DEV))
    assert wl.T_img == 16  # one image tile: split it as [0, 16) after the text block
    st = qi.joint_attn_fwd_carry(q, k, g["v"], geo, True, 0, 0, state_out=st)
    of_c = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o_c, lse_c = qi.joint_attn_fwd_carry(q, k, g["v"], geo, False, 0, wl.T_img, state=st, last=True, out_f32=of_c)
    torch.cuda.synchronize()
    assert _same(o_c, o) and _same(lse_c, lse) and _same(of_c, of)
