"""GPU bit-exactness: replay, batch size, batch position, reversal, text
padding and poisoned masked keys must leave a logical row's bytes unchanged
(the pages' batch-invariance rule: a row's bytes depend on nothing but the
row)."""
import pytest
import torch

import workloads
from parity import bits

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def geom(B, H, T, Ls, h, w):
    return qi.Geometry(B=B, H=H, T_txt=T, grid_h=h, grid_w=w, txt_len=list(Ls))


def forward(g, geo):
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo)
    torch.cuda.synchronize()
    return q, k, o, lse


def sub(g, idx):
    out = dict(g)
    for n in ("q", "k", "v", "dO"):
        if g.get(n) is not None:
            out[n] = g[n][idx].contiguous()
    return out


def test_forward_replay_bitexact():
    wl = workloads.WORKLOADS["1024sq"]
    g = to_dev(workloads.make_inputs(wl))
    geo = geom(wl.B, wl.H, wl.T_txt, wl.txt_len, wl.h, wl.w)
    ref = [bits(t) for t in forward(g, geo)]
    for _ in range(3):
        cur = [bits(t) for t in forward(g, geo)]
        for a, b in zip(ref, cur):
            assert (a == b).all()


def _rows_equal(full, part, rows_full, name):
    for i, j in rows_full:
        assert (bits(full[i]) == bits(part[j])).all(), f"{name}: row {i} != row {j} of the other run"


@pytest.mark.parametrize("cfg", ["1664x928", "1328sq_cfg"])
def test_batch_invariance(cfg):
    wl = workloads.WORKLOADS[cfg]
    g = to_dev(workloads.make_inputs(wl))
    B = wl.B
    geo = geom(B, wl.H, wl.T_txt, wl.txt_len, wl.h, wl.w)
    full = forward(g, geo)
    # each row alone
    for b in range(B):
        one = forward(sub(g, slice(b, b + 1)), geom(1, wl.H, wl.T_txt, [wl.txt_len[b]], wl.h, wl.w))
        for name, fa, fb in zip(("q'", "k'", "O", "LSE"), full, one):
            _rows_equal(fa, fb, [(b, 0)], f"{name} alone")
    # reversed order
    rev = list(range(B))[::-1]
    r = forward(sub(g, rev), geom(B, wl.H, wl.T_txt, [wl.txt_len[i] for i in rev], wl.h, wl.w))
    for name, fa, fb in zip(("q'", "k'", "O", "LSE"), full, r):
        _rows_equal(fa, fb, [(rev[j], j) for j in range(B)], f"{name} reversed")
    # prefixes B = 1, 2 (and the full batch above)
    for nb in (1, 2):
        if nb >= B:
            continue
        p = forward(sub(g, slice(0, nb)), geom(nb, wl.H, wl.T_txt, wl.txt_len[:nb], wl.h, wl.w))
        for name, fa, fb in zip(("q'", "k'", "O", "LSE"), full, p):
            _rows_equal(fa, fb, [(j, j) for j in range(nb)], f"{name} B={nb}")


def _repad(t, L, T_old, T_new, fill):
    """Move the text segment of t [B,S,H,D] to a padded length T_new keeping
    the first L rows and the image rows; new pad rows come from `fill`."""
    B, S, H, D = t.shape
    img = t[:, T_old:]
    pad = fill[:, : T_new - L] if T_new > L else t[:, :0]
    return torch.cat([t[:, :L], pad, img], 1).contiguous()


def test_padding_invariance():
    wl = workloads.WORKLOADS["1024sq"]
    g = to_dev(workloads.make_inputs(wl))
    L = wl.txt_len[0]
    base = forward(g, geom(1, wl.H, wl.T_txt, [L], wl.h, wl.w))
    filler = to_dev(workloads.make_inputs(workloads.custom("fill", 1, wl.H, 512, [0], 1, 1, 77)))
    for T_new in (L, 512, 300):
        gn = dict(g)
        for n in ("q", "k", "v"):
            gn[n] = _repad(g[n], L, wl.T_txt, T_new, filler[n])
        out = forward(gn, geom(1, wl.H, T_new, [L], wl.h, wl.w))
        T_img = wl.h * wl.w
        for name, fa, fb in zip(("q'", "k'", "O"), base[:3], out[:3]):
            assert (bits(fa[:, :L]) == bits(fb[:, :L])).all(), f"{name} text rows, T_txt={T_new}"
            assert (bits(fa[:, wl.T_txt:]) == bits(fb[:, T_new:T_new + T_img])).all(), f"{name} image rows, T_txt={T_new}"
        la, lb = base[3], out[3]
        assert (bits(la[:, :, :L]) == bits(lb[:, :, :L])).all()
        assert (bits(la[:, :, wl.T_txt:]) == bits(lb[:, :, T_new:])).all()


def test_masked_keys_poisoned():
    wl = workloads.WORKLOADS["1664x928"]
    g = to_dev(workloads.make_inputs(wl))
    geo = geom(wl.B, wl.H, wl.T_txt, wl.txt_len, wl.h, wl.w)
    q, k, o, lse = forward(g, geo)
    kp, vp = k.clone(), g["v"].clone()
    for b, L in enumerate(wl.txt_len):
        kp[b, L:wl.T_txt] = float("nan")
        vp[b, L:wl.T_txt] = float("inf")
    o2, l2 = qi.joint_attn_fwd(q, kp, vp, geo)
    torch.cuda.synchronize()
    assert (bits(o2) == bits(o)).all() and (bits(l2) == bits(lse)).all()


def backward(g, geo):
    q, k, o, lse, of = qi.joint_attention(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, keep_f32=True)
    r = qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    return r


def test_backward_replay_and_batch():
    wl = workloads.WORKLOADS["1024sq_bwd"]
    inp2 = workloads.make_inputs(wl, extra_samples=1)  # B = 2: the config's sample, then one more
    g2 = to_dev(inp2)
    g1 = sub(g2, slice(0, 1))
    geo1 = geom(1, wl.H, wl.T_txt, wl.txt_len, wl.h, wl.w)
    geo2 = geom(2, wl.H, wl.T_txt, inp2["txt_len"], wl.h, wl.w)
    names = ("dq", "dk", "dv", "dgain_q_ps", "dgain_k_ps", "dgain_q", "dgain_k")
    ref = backward(g1, geo1)
    ref_bits = {n: bits(ref[n]) for n in names}
    for _ in range(4):
        cur = backward(g1, geo1)
        for n in names:
            assert (bits(cur[n]) == ref_bits[n]).all(), f"{n} replay"
    two = backward(g2, geo2)
    for n in ("dq", "dk", "dv", "dgain_q_ps", "dgain_k_ps"):
        assert (bits(two[n][:1]) == ref_bits[n]).all(), f"{n}: sample 0 at B=2 differs from B=1"


def _bwd_from(g, geo, q=None, k=None):
    """Forward (prologues + attention, keeping the FP32 O) and backward; q, k
    replace the prologue outputs the backward consumes when given."""
    q0, k0, o, lse, of = qi.joint_attention(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, keep_f32=True)
    q = q0 if q is None else q
    k = k0 if k is None else k
    r = qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    return (q0, k0), r


def test_backward_padding_invariance():
    """Re-padding the text to T_txt = 219, 300 and 512 (new pad rows drawn from
    another seed, dO = 0 on every padded query row) leaves dq, dk, dv of the
    valid text rows and of the image rows, and the per-sample gain
    gradients, bit for bit unchanged: padded queries add exact zeros."""
    wl = workloads.WORKLOADS["1024sq_bwd"]
    g = to_dev(workloads.make_inputs(wl))
    L, T, T_img = wl.txt_len[0], wl.T_txt, wl.h * wl.w
    g["dO"] = g["dO"].clone()
    g["dO"][:, L:T] = 0
    _, base = _bwd_from(g, geom(1, wl.H, T, [L], wl.h, wl.w))
    filler = to_dev(workloads.make_inputs(workloads.custom("fill", 1, wl.H, 512, [0], 1, 1, 78, backward=True)))
    filler["dO"] = torch.zeros_like(filler["dO"])
    for T_new in (L, 300, 512):
        gn = dict(g)
        for n in ("q", "k", "v", "dO"):
            gn[n] = _repad(g[n], L, T, T_new, filler[n])
        _, r = _bwd_from(gn, geom(1, wl.H, T_new, [L], wl.h, wl.w))
        for n in ("dq", "dk", "dv"):
            a, b = base[n], r[n]
            assert (bits(a[:, :L]) == bits(b[:, :L])).all(), f"{n} text rows, T_txt={T_new}"
            assert (bits(a[:, T:]) == bits(b[:, T_new:T_new + T_img])).all(), f"{n} image rows, T_txt={T_new}"
        for n in ("dgain_q_ps", "dgain_k_ps", "dgain_q", "dgain_k"):
            assert (bits(base[n]) == bits(r[n])).all(), f"{n}, T_txt={T_new}"


def test_backward_masked_keys_poisoned():
    """NaN in the masked text keys of k' and Inf in those rows of V leave every
    gradient byte unchanged (masked keys are never read by the backward)."""
    wl = workloads.WORKLOADS["1664x928"]
    B = 2
    inp = workloads.make_inputs(workloads.custom("poison_bwd", B, 8, wl.T_txt, wl.txt_len[:B], wl.h, wl.w,
                                                 31, backward=True))
    g = to_dev(inp)
    geo = geom(B, 8, wl.T_txt, wl.txt_len[:B], wl.h, wl.w)
    (q, k), clean = _bwd_from(g, geo)
    kp, vp = k.clone(), g["v"].clone()
    for b, L in enumerate(wl.txt_len[:B]):
        kp[b, L:wl.T_txt] = float("nan")
        vp[b, L:wl.T_txt] = float("inf")
    q0, k0, o, lse, of = qi.joint_attention(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, keep_f32=True)
    r = qi.joint_attn_bwd(g["q"], g["k"], q0, kp, vp, of, lse, g["dO"], g["g_q"], g["g_k"], geo)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dgain_q_ps", "dgain_k_ps", "dgain_q", "dgain_k"):
        assert (bits(clean[n]) == bits(r[n])).all(), n
