"""GPU tests of the carried key-block forward (the state travels from block to
block, the last block writes O and LSE).

* A chain over tile-aligned blocks in the whole call's key order (text block
  first, image tiles ascending) gives O, LSE and O_f32 equal byte for byte to
  the whole-row forward, for even and uneven partitions, with the state in
  separate buffers or continued in place, at small ragged shapes and at two
  full reference shapes (1024^2 in 8 blocks, 1328^2 with a ragged last
  block).
* A chain in another order is still the attention of every key: within the
  path's tolerance of the oracle.
* The state after a block is the block-restricted attention of the keys seen
  so far (checked against the oracle on one small shape).
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
C = (1.0 / math.log(2.0)) / math.sqrt(HD)

SMALL = [  # name, B, H, T_txt, txt_len, h, w
    ("tiny", 1, 2, 8, (5,), 4, 4),
    ("ragged", 3, 2, 130, (0, 67, 130), 13, 11),
    ("no_text", 1, 2, 0, (0,), 15, 9),
    ("wide", 2, 3, 64, (64, 1), 16, 16),
]


def _inputs(wl):
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    return geo, q, k, g["v"]


def _bytes_equal(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _chain(q, k, v, geo, blocks, in_place=False):
    """Run the blocks in the given order; returns (O, LSE, O_f32)."""
    state = None
    if in_place:
        B, H, S = geo.B, geo.H, geo.S
        buf = (torch.empty((B, H, S, HD), dtype=torch.float32, device=DEV),
               torch.empty((B, H, S), dtype=torch.float32, device=DEV),
               torch.empty((B, H, S, 2), dtype=torch.float32, device=DEV))
    for i, (wt, lo, hi) in enumerate(blocks):
        if i + 1 < len(blocks):
            out = buf if in_place else None
            state = qi.joint_attn_fwd_carry(q, k, v, geo, wt, lo, hi, state=state, state_out=out)
        else:
            of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
            o, lse = qi.joint_attn_fwd_carry(q, k, v, geo, wt, lo, hi, state=state, last=True, out_f32=of)
            return o, lse, of


def _fused(q, k, v, geo):
    of = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    o, lse = qi.joint_attn_fwd(q, k, v, geo, out_f32=of)
    return o, lse, of


def _even(T_img, size):
    """Text keys with the first image chunk, then one block per chunk."""
    edges = list(range(0, T_img, size)) + [T_img]
    return [(j == 0, edges[j], edges[j + 1]) for j in range(len(edges) - 1)]


def _uneven(T_img, seed):
    """Text keys alone, then image blocks of 1..5 tiles, the last one ragged."""
    rng = np.random.default_rng(seed)
    edges, e = [0], 0
    while e < T_img:
        e = min(T_img, e + 64 * int(rng.integers(1, 6)))
        edges.append(e)
    return [(True, 0, 0)] + [(False, edges[j], edges[j + 1]) for j in range(len(edges) - 1)]


def _assert_same(got, ref, what):
    for name, a, b in zip(("O", "LSE", "O_f32"), got, ref):
        assert _bytes_equal(a, b), f"{what}: {name} differs from the whole-row forward"


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_chain_equals_whole_row_forward(spec):
    name, B, H, T, Ls, h, w = spec
    wl = workloads.custom(name, B, H, T, Ls, h, w, 410)
    print(f"carried chains vs fused: {spec}", flush=True)
    geo, q, k, v = _inputs(wl)
    ref = _fused(q, k, v, geo)
    for blocks, what in ((_even(wl.T_img, 64), "64-key blocks"), (_even(wl.T_img, 128), "128-key blocks"),
                         (_uneven(wl.T_img, 5), "uneven blocks"), ([(True, 0, wl.T_img)], "one block")):
        for in_place in (False, True):
            got = _chain(q, k, v, geo, blocks, in_place)
            torch.cuda.synchronize()
            _assert_same(got, ref, f"{what}, in place={in_place}")


@pytest.mark.parametrize("cfg,size", [("1024sq", 512), ("1328sq_cfg", 512)])
def test_chain_equals_whole_row_forward_full(cfg, size):
    """8 blocks of 512 image keys at 1024^2 (a ring over 8 devices); at
    1328^2 the last of 14 blocks ends at T_img = 6889, inside a tile; and an
    uneven partition with the text keys alone."""
    wl = workloads.WORKLOADS[cfg]
    print(f"carried chains vs fused: {cfg}", flush=True)
    geo, q, k, v = _inputs(wl)
    ref = _fused(q, k, v, geo)
    blocks = _even(wl.T_img, size)
    assert len(blocks) == -(-wl.T_img // size)
    _assert_same(_chain(q, k, v, geo, blocks), ref, f"{cfg} even")
    _assert_same(_chain(q, k, v, geo, _uneven(wl.T_img, 6), in_place=True), ref, f"{cfg} uneven, in place")
    torch.cuda.synchronize()


@pytest.mark.parametrize("spec", SMALL[1:3], ids=[s[0] for s in SMALL[1:3]])
def test_chain_in_another_order_against_oracle(spec):
    """Image blocks descending, the text block last: not the whole call's
    bytes, but the same attention within the path's tolerance."""
    name, B, H, T, Ls, h, w = spec
    wl = workloads.custom(name, B, H, T, Ls, h, w, 411)
    geo, q, k, v = _inputs(wl)
    blocks = [(False, lo, hi) for (_, lo, hi) in reversed(_even(wl.T_img, 64))] + [(True, 0, 0)]
    o, lse, _ = _chain(q, k, v, geo, blocks)
    torch.cuda.synchronize()
    ro, rl = Oracle("f32").attn_fwd(f64(q), f64(k), f64(v), list(wl.txt_len), wl.T_txt)
    mixed_check(o, ro, "O of a reordered chain")
    assert np.abs(f64(lse) - rl).max() <= 1e-4


def test_intermediate_state_against_oracle():
    """After the text block and the first image blocks, the state is the
    attention restricted to the keys seen so far."""
    wl = workloads.custom("ragged", 3, 2, 130, (0, 67, 130), 13, 11, 412)
    geo, q, k, v = _inputs(wl)
    state = qi.joint_attn_fwd_carry(q, k, v, geo, True, 0, 64)
    state = qi.joint_attn_fwd_carry(q, k, v, geo, False, 64, 128, state=state)
    acc, m, l = state
    torch.cuda.synchronize()
    orc = Oracle("f32")
    qf, kf, vf = f64(q), f64(k), f64(v)
    lsum = f64(l).sum(axis=-1)
    for b in range(wl.B):
        for h in range(wl.H):
            ro, rl = orc.attn_fwd_block_bh(qf[b, :, h], kf[b, :, h], vf[b, :, h], wl.T_txt, wl.txt_len[b], True, 0, 128)
            ob = f64(acc[b, h]) / (lsum[b, h][:, None] * 2.0 ** -8)
            mixed_check(ob, ro, f"state O b={b} h={h}")
            lse_b = (f64(m[b, h]) * C + np.log2(lsum[b, h])) * LN2
            assert np.abs(lse_b - rl).max() <= 1e-4, f"state LSE b={b} h={h}"
