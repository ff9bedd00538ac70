"""GPU tests of the unfused forward: the score GEMM, the tiled softmax and the
A.V GEMM as three operators.

* The composition qk_gemm -> softmax -> av_gemm equals the fused forward byte
  for byte (O, LSE and the FP32 pre-cast O) on ragged small shapes and on the
  full reference shapes.
* Each operator on its own against the oracle: scores against the oracle's
  scaled scores; the softmax (fed seeded raw scores) against the oracle's
  softmax of the same scores, with the probabilities rebuilt from P, the tile
  factors alpha and l; the A.V operator (fed seeded P, alpha, l) against the
  oracle's tile recurrence.
* The contents of masked and unused slots are what the interface fixes.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import Oracle
from parity import f64, mixed_check

qi = pytest.importorskip("invariant_joint_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HD = 128


@pytest.fixture(scope="module")
def o64():
    return Oracle("f64")


SMALL = [  # name, B, H, T_txt, txt_len, h, w
    ("tiny", 1, 2, 8, (5,), 4, 4),
    ("ragged", 3, 2, 130, (0, 67, 130), 9, 11),
    ("one_image_token", 2, 1, 3, (0, 2), 1, 1),
    ("no_text", 1, 2, 0, (0,), 6, 5),
    ("tile_edges", 2, 3, 64, (64, 1), 8, 8),
]


def _wl(spec, seed=300):
    name, B, H, T, Ls, h, w = spec
    return workloads.custom(name, B, H, T, Ls, h, w, seed)


def _geom(wl):
    return qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))


def _prologue_inputs(wl):
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = _geom(wl)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    return geo, q, k, g["v"]


def _tiles(T, L, S):
    """(first key, valid count) of each logical 64-key tile of a row."""
    t = [(k0, min(64, L - k0)) for k0 in range(0, L, 64)]
    t += [(k0, min(64, S - k0)) for k0 in range(T, S, 64)]
    return t


def _slot_keys(T, L, S, Kp):
    """Key of each slot (-1 for a masked or unused slot)."""
    key = np.full(Kp, -1, dtype=np.int64)
    for t, (k0, nv) in enumerate(_tiles(T, L, S)):
        key[64 * t:64 * t + nv] = np.arange(k0, k0 + nv)
    return key


def _same_bytes(a, b, name):
    assert a.shape == b.shape and a.dtype == b.dtype, name
    x, y = a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)
    if not torch.equal(x, y):
        n = int((a.contiguous().view(-1).view(torch.int16 if a.element_size() == 2 else torch.int32) !=
                 b.contiguous().view(-1).view(torch.int16 if b.element_size() == 2 else torch.int32)).sum())
        raise AssertionError(f"{name}: {n} elements differ between the fused and the unfused forward")


def _compare_fused_unfused(geo, q, k, v):
    of_f = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    of_u = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o_f, lse_f = qi.joint_attn_fwd(q, k, v, geo, out_f32=of_f)
    o_u, lse_u, mid = qi.joint_attn_unfused(q, k, v, geo, out_f32=of_u)
    torch.cuda.synchronize()
    _same_bytes(o_u, o_f, "O")
    _same_bytes(lse_u, lse_f, "LSE")
    _same_bytes(of_u, of_f, "O_f32")
    return mid


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_composition_equals_fused_small(spec):
    wl = _wl(spec)
    print(f"composition vs fused: {spec}", flush=True)
    geo, q, k, v = _prologue_inputs(wl)
    mid = _compare_fused_unfused(geo, q, k, v)
    # masked / unused slot contents
    Kp = qi.key_slots(geo)
    s, p, alpha = (mid[n].cpu() for n in ("scores", "p", "alpha"))
    for b in range(wl.B):
        key = _slot_keys(wl.T_txt, wl.txt_len[b], wl.S, Kp)
        masked = torch.from_numpy(key < 0)
        assert torch.isneginf(s[b][..., masked]).all()
        assert torch.isfinite(s[b][..., ~masked]).all()
        assert (p[b][..., masked] == 0).all()
        n_b = len(_tiles(wl.T_txt, wl.txt_len[b], wl.S))
        ab = alpha[b]  # [H, tiles, S]
        assert (ab[:, n_b:] == 1).all()
        assert (ab[:, 0] == 0).all()  # nothing accumulated before the first tile
        assert ((ab[:, :n_b] >= 0) & (ab[:, :n_b] <= 1)).all()


@pytest.mark.parametrize("cfg", ["1024sq", "1328sq_cfg", "1664x928"])
def test_composition_equals_fused_full(cfg):
    """At the reference shapes, in the launch configuration the benchmark
    times, over every output element."""
    wl = workloads.WORKLOADS[cfg]
    print(f"composition vs fused: {cfg}", flush=True)
    geo, q, k, v = _prologue_inputs(wl)
    _compare_fused_unfused(geo, q, k, v)


def _q_k_bf16_f64(q, k, b, h):
    return f64(q[b, :, h]), f64(k[b, :, h])


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_qk_gemm_against_oracle(o64, spec):
    """Raw scores / sqrt(128) against the oracle's scaled scores of the same
    BF16 q', k'; the bound is the FP32 accumulation of 128 exact products."""
    wl = _wl(spec, seed=301)
    geo, q, k, v = _prologue_inputs(wl)
    s = qi.joint_attn_qk_gemm(q, k, geo)
    torch.cuda.synchronize()
    Kp = qi.key_slots(geo)
    sc = 1 / math.sqrt(HD)
    for b in range(wl.B):
        key = _slot_keys(wl.T_txt, wl.txt_len[b], wl.S, Kp)
        live = key >= 0
        for h in range(wl.H):
            qs, ks = _q_k_bf16_f64(q, k, b, h)
            ref = o64.attn_scores_bh(qs, ks, wl.T_txt, wl.txt_len[b])[:, key[live]]
            mag = (np.abs(qs) @ np.abs(ks).T)[:, key[live]] * sc
            got = f64(s[b, h])[:, live] * sc
            err = np.abs(got - ref)
            assert (err <= 2.0 ** -16 * mag + 1e-30).all(), f"b={b} h={h}: max err {err.max():.3e}"


def test_qk_gemm_full_sampled(o64):
    wl = workloads.WORKLOADS["1024sq"]
    geo, q, k, v = _prologue_inputs(wl)
    s = qi.joint_attn_qk_gemm(q, k, geo)
    torch.cuda.synchronize()
    Kp = qi.key_slots(geo)
    key = _slot_keys(wl.T_txt, wl.txt_len[0], wl.S, Kp)
    live = key >= 0
    sc = 1 / math.sqrt(HD)
    for h, r0 in ((0, 0), (13, 2100), (23, wl.S - 70)):
        qs, ks = _q_k_bf16_f64(q, k, 0, h)
        ref = o64.attn_scores_bh(qs, ks, wl.T_txt, wl.txt_len[0], r0, r0 + 70)[:, key[live]]
        mag = (np.abs(qs[r0:r0 + 70]) @ np.abs(ks).T)[:, key[live]] * sc
        got = f64(s[0, h, r0:r0 + 70])[:, live] * sc
        assert (np.abs(got - ref) <= 2.0 ** -16 * mag + 1e-30).all()
        assert torch.isneginf(s[0, h, r0:r0 + 70][:, torch.from_numpy(~live).to(DEV)]).all()


def _softmax_case(wl, seed):
    geo = _geom(wl)
    Kp = qi.key_slots(geo)
    raw = workloads.score_operands(wl.B, wl.H, wl.S, Kp, seed)
    for b in range(wl.B):  # the interface's masked value
        key = _slot_keys(wl.T_txt, wl.txt_len[b], wl.S, Kp)
        raw[b][..., torch.from_numpy(key < 0)] = -math.inf
    return geo, Kp, raw


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_softmax_against_oracle(o64, spec):
    """Seeded raw scores through the softmax operator.  The probability of
    key j in tile t is rebuilt as P_j * prod_{u>t} alpha_u / l and compared
    with the oracle's softmax of the scaled scores; LSE likewise."""
    wl = _wl(spec)
    geo, Kp, raw = _softmax_case(wl, seed=302)
    p, alpha, l, lse = qi.joint_attn_softmax(raw.to(DEV), geo)
    torch.cuda.synchronize()
    p, alpha, l, lse = f64(p), f64(alpha), f64(l), f64(lse)
    sc = 1 / math.sqrt(HD)
    moved = 0
    for b in range(wl.B):
        L = wl.txt_len[b]
        key = _slot_keys(wl.T_txt, L, wl.S, Kp)
        live = key >= 0
        nt = len(_tiles(wl.T_txt, L, wl.S))
        for h in range(wl.H):
            s_keys = np.zeros((wl.S, wl.S))
            s_keys[:, key[live]] = raw[b, h].double().numpy()[:, live] * sc
            p_ref, lse_ref = o64.attn_softmax_rows(s_keys, wl.T_txt, L)
            a = alpha[b, h].T  # [S, tiles]
            # weight of tile t in the final sum: product of the later tiles' factors
            later = np.ones((wl.S, Kp // 64))
            for t in range(nt - 2, -1, -1):
                later[:, t] = later[:, t + 1] * a[:, t + 1]
            w = np.repeat(later, 64, axis=1)
            prob = p[b, h] * w / l[b, h][:, None]
            got, ref = prob[:, live], p_ref[:, key[live]]
            err = np.abs(got - ref)
            assert (err <= 2.0 ** -10 * ref + 2.0 ** -24).all(), f"b={b} h={h}: max err {err.max():.3e}"
            assert np.abs(lse[b, h] - lse_ref).max() <= 1e-5 * max(1.0, np.abs(lse_ref).max())
            moved += int((a[:, 1:nt] < 1).sum())
    if spec[0] in ("tiny", "ragged", "tile_edges"):
        assert moved > 0  # the seeded drift makes the reference max move


def _av_case(wl, seed):
    geo = _geom(wl)
    Kp = qi.key_slots(geo)
    ops = workloads.av_operands(wl.B, wl.H, wl.S, Kp, seed)
    for b in range(wl.B):  # the interface's masked value of P
        key = _slot_keys(wl.T_txt, wl.txt_len[b], wl.S, Kp)
        ops["p"][b][..., torch.from_numpy(key < 0)] = 0
    return geo, Kp, ops


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_av_gemm_against_oracle(o64, spec):
    """Seeded P, alpha, l and V through the A.V operator against the oracle's
    tile recurrence acc <- alpha acc + P_t V_t, O = acc / l.  Bound: FP32
    accumulation over at most 16 products per MFMA plus 4 accumulations per
    tile, and V in FP16 as v * 2^-8 (exact above 2^-6, abs error <= 2^-17
    below)."""
    wl = _wl(spec)
    geo, Kp, ops = _av_case(wl, seed=303)
    v = workloads.make_inputs(wl)["v"]
    of = torch.empty((wl.B, wl.S, wl.H, HD), dtype=torch.float32, device=DEV)
    o = qi.joint_attn_av_gemm(ops["p"].to(DEV), ops["alpha"].to(DEV), ops["l"].to(DEV), v.to(DEV), geo, out_f32=of)
    torch.cuda.synchronize()
    for b in range(wl.B):
        L = wl.txt_len[b]
        nt_b = len(_tiles(wl.T_txt, L, wl.S))
        n_adds = 16 + 4 * nt_b
        for h in range(wl.H):
            P = f64(ops["p"][b, h]).reshape(wl.S, Kp // 64, 64)
            al, lv = f64(ops["alpha"][b, h]).T.copy(), f64(ops["l"][b, h])
            vb = f64(v[b, :, h])
            ref = o64.attn_av_rows(P, al, lv, vb, wl.T_txt, L)
            mag = o64.attn_av_rows(P, al, lv, np.abs(vb), wl.T_txt, L)
            wsum = o64.attn_av_rows(P, al, lv, np.ones_like(vb), wl.T_txt, L)
            tol = 2.0 * n_adds * 2.0 ** -24 * mag + 2.0 ** -17 * wsum + 1e-30
            got = f64(of[b, :, h])
            err = np.abs(got - ref)
            assert (err <= tol).all(), f"b={b} h={h}: max err {err.max():.3e}"
            mixed_check(o[b, :, h], ref, f"O b={b} h={h}")


def test_composition_against_oracle_attention():
    """End to end on a ragged shape: the composed O and LSE against the
    oracle's plain attention of the same BF16 q', k' and V."""
    wl = _wl(SMALL[1], seed=304)
    geo, q, k, v = _prologue_inputs(wl)
    o, lse, _ = qi.joint_attn_unfused(q, k, v, geo)
    torch.cuda.synchronize()
    orc = Oracle("f32")
    ro, rl = orc.attn_fwd(f64(q), f64(k), f64(v), list(wl.txt_len), wl.T_txt)
    mixed_check(o, ro, "O")
    assert np.abs(f64(lse) - rl).max() <= 1e-4


def test_row_independent_of_batch():
    """A row's composed outputs do not depend on the other rows of the batch:
    sample 1 alone equals sample 1 of the batch."""
    wl = _wl(SMALL[1], seed=305)
    geo, q, k, v = _prologue_inputs(wl)
    o, lse, _ = qi.joint_attn_unfused(q, k, v, geo)
    g1 = qi.Geometry(B=1, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=[wl.txt_len[1]])
    o1, lse1, _ = qi.joint_attn_unfused(q[1:2].contiguous(), k[1:2].contiguous(), v[1:2].contiguous(), g1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o[1:2].view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse[1:2].view(torch.int32))
