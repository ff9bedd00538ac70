"""GPU tests of the key-block forward and the fixed-order merge.

* One block holding every key, merged, equals the whole-row forward byte for
  byte (O, LSE, O_f32), on ragged small shapes and at two full reference
  shapes.
* With the image keys split into tile-aligned blocks, the merged bytes do not
  depend on the order in which the block states were computed, on the
  buffers, or on which other samples shared the launch.
* Each block's state describes attention restricted to that block's keys
  (checked against the oracle's block attention), and the merged output is
  within the path's tolerance of the oracle's full attention.
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
LN2 = math.log(2.0)
C = (1.0 / math.log(2.0)) / math.sqrt(HD)  # log2(e)/sqrt(128), the exponent scale of the row state

SMALL = [  # name, B, H, T_txt, txt_len, h, w, image block size (keys)
    ("tiny", 1, 2, 8, (5,), 4, 4, 64),
    ("ragged", 3, 2, 130, (0, 67, 130), 13, 11, 64),
    ("no_text", 1, 2, 0, (0,), 15, 9, 64),
    ("chunks_128", 2, 3, 64, (64, 1), 16, 16, 128),
]


def _wl(spec, seed=400):
    name, B, H, T, Ls, h, w, _ = spec
    return workloads.custom(name, B, H, T, Ls, h, w, seed)


def _geom(wl, B=None, txt_len=None):
    return qi.Geometry(B=wl.B if B is None else B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w,
                       txt_len=list(wl.txt_len if txt_len is None else txt_len))


def _inputs(wl):
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = _geom(wl)
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    return geo, q, k, g["v"]


def _blocks(T_img, size):
    """Block 0: the text keys and the first image chunk; then one block per chunk."""
    edges = list(range(0, T_img, size)) + [T_img]
    return [(k == 0, edges[k], edges[k + 1]) for k in range(len(edges) - 1)]


def _states(q, k, v, geo, blocks, order):
    n = len(blocks)
    B, H, S = geo.B, geo.H, geo.S
    acc = torch.empty((n, B, H, S, HD), dtype=torch.float32, device=DEV)
    m = torch.empty((n, B, H, S), dtype=torch.float32, device=DEV)
    l = torch.empty((n, B, H, S), dtype=torch.float32, device=DEV)
    for i in order:
        wt, lo, hi = blocks[i]
        qi.joint_attn_fwd_partial(q, k, v, geo, wt, lo, hi, acc=acc[i], m=m[i], l=l[i])
    return acc, m, l


def _bytes_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check_one_block(geo, q, k, v):
    T_img = geo.grid_h * geo.grid_w
    of_f = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o_f, lse_f = qi.joint_attn_fwd(q, k, v, geo, out_f32=of_f)
    acc, m, l = _states(q, k, v, geo, [(True, 0, T_img)], [0])
    of_m = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o_m, lse_m = qi.joint_attn_merge(acc, m, l, geo, out_f32=of_m)
    torch.cuda.synchronize()
    assert _bytes_equal(o_m, o_f), "O"
    assert _bytes_equal(lse_m, lse_f), "LSE"
    assert _bytes_equal(of_m, of_f), "O_f32"


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_one_block_equals_whole_row_forward(spec):
    print(f"one block vs fused: {spec}", flush=True)
    geo, q, k, v = _inputs(_wl(spec))
    _check_one_block(geo, q, k, v)


@pytest.mark.parametrize("cfg", ["1024sq", "1328sq_cfg"])
def test_one_block_equals_whole_row_forward_full(cfg):
    print(f"one block vs fused: {cfg}", flush=True)
    geo, q, k, v = _inputs(workloads.WORKLOADS[cfg])
    _check_one_block(geo, q, k, v)


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_split_merge_independent_of_order_and_batch(spec):
    wl = _wl(spec, seed=401)
    print(f"split blocks: {spec}", flush=True)
    geo, q, k, v = _inputs(wl)
    blocks = _blocks(wl.T_img, spec[7])
    n = len(blocks)
    o1, l1 = qi.joint_attn_merge(*_states(q, k, v, geo, blocks, range(n)), geo)
    o2, l2 = qi.joint_attn_merge(*_states(q, k, v, geo, blocks, reversed(range(n))), geo)
    torch.cuda.synchronize()
    assert _bytes_equal(o1, o2) and _bytes_equal(l1, l2)
    # each sample alone (its own launches and buffers)
    for b in range(wl.B):
        g1 = _geom(wl, B=1, txt_len=[wl.txt_len[b]])
        sl = (slice(b, b + 1),)
        ob, lb = qi.joint_attn_merge(*_states(q[sl].contiguous(), k[sl].contiguous(), v[sl].contiguous(), g1, blocks,
                                              range(n)), g1)
        torch.cuda.synchronize()
        assert _bytes_equal(ob, o1[sl]) and _bytes_equal(lb, l1[sl]), f"sample {b}"


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_block_states_and_merge_against_oracle(spec):
    wl = _wl(spec, seed=402)
    geo, q, k, v = _inputs(wl)
    blocks = _blocks(wl.T_img, spec[7])
    acc, m, l = _states(q, k, v, geo, blocks, range(len(blocks)))
    o, lse = qi.joint_attn_merge(acc, m, l, geo)
    torch.cuda.synchronize()
    orc = Oracle("f32")
    qf, kf, vf = f64(q), f64(k), f64(v)
    for b in range(wl.B):
        L = wl.txt_len[b]
        for h in range(wl.H):
            for i, (wt, lo, hi) in enumerate(blocks):
                has_keys = (wt and L > 0) or hi > lo
                mi, li, ai = f64(m[i, b, h]), f64(l[i, b, h]), f64(acc[i, b, h])
                if not has_keys:
                    assert np.all(mi == -np.inf) and np.all(li == 0) and np.all(ai == 0)
                    continue
                ro, rl = orc.attn_fwd_block_bh(qf[b, :, h], kf[b, :, h], vf[b, :, h], wl.T_txt, L, wt, lo, hi)
                ob = ai / (li[:, None] * 2.0 ** -8)
                mixed_check(ob, ro, f"block {i} O b={b} h={h}")
                lse_b = (mi * C + np.log2(li)) * LN2
                assert np.abs(lse_b - rl).max() <= 1e-4, f"block {i} LSE b={b} h={h}"
    ro, rl = orc.attn_fwd(qf, kf, vf, list(wl.txt_len), wl.T_txt)
    mixed_check(o, ro, "merged O")
    assert np.abs(f64(lse) - rl).max() <= 1e-4


def test_split_merge_full_1024sq():
    """The 1024^2 shape with the image keys in 8 blocks of 512 (a sequence-
    parallel split over 8 devices): order independence, and sampled rows of
    the merged output against the oracle."""
    wl = workloads.WORKLOADS["1024sq"]
    geo, q, k, v = _inputs(wl)
    blocks = _blocks(wl.T_img, 512)
    assert len(blocks) == 8
    o1, l1 = qi.joint_attn_merge(*_states(q, k, v, geo, blocks, range(8)), geo)
    o2, l2 = qi.joint_attn_merge(*_states(q, k, v, geo, blocks, [3, 7, 0, 5, 1, 6, 2, 4]), geo)
    torch.cuda.synchronize()
    assert _bytes_equal(o1, o2) and _bytes_equal(l1, l2)
    orc = Oracle("f32")
    for h, r0 in ((0, 0), (11, 2048), (23, wl.S - 64)):
        ro, rl = orc.attn_fwd_bh(f64(q[0, :, h]), f64(k[0, :, h]), f64(v[0, :, h]), wl.T_txt, wl.txt_len[0],
                                 r0, r0 + 64)
        mixed_check(o1[0, r0:r0 + 64, h], ro, f"merged O h={h}")
        assert np.abs(f64(l1[0, h, r0:r0 + 64]) - rl).max() <= 1e-4
