"""Pins of the CPU oracle against things other than itself.

Every check here ties the oracle to a closed form, an invariant, a hand-written
fixture, a library routine (torch float64 RMSNorm / SDPA / autograd, numpy
complex arithmetic, scipy logsumexp) or finite differences.  None calls the
GPU library.  A plausible slip in the oracle -- a dropped term, a wrong sign
or index, a transposed operand, the wrong pairing or centring -- fails at
least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import workloads
from oracle import Oracle, fold_batch, forward_path, qkv_path

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HD = 128


@pytest.fixture(scope="module")
def o32():
    return Oracle("f32")


@pytest.fixture(scope="module")
def o64():
    return Oracle("f64")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------- conversions
def test_bf16_cast_matches_torch_rne(o32):
    """The oracle's FP32->BF16 rounding equals torch's RNE conversion on
    random bit patterns (normal, subnormal, overflow-adjacent values)."""
    rng = _rng(0)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ties = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-130, 3 * 2**-134,
                     3.3895314e38, 3.3961775e38, 0.0, -0.0], dtype=np.float32)
    f = np.concatenate([f, ties])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o32.cast_bf16(f)
    assert np.array_equal(got, ref)


def test_bf16_cast_hand_values(o32, o64):
    # ties go to even: 1+2^-8 -> 1.0 ; 1+3*2^-8 -> 1+2^-6
    assert o32.cast_bf16(np.array([1 + 2**-8], np.float32))[0] == 0x3F80
    assert o32.cast_bf16(np.array([1 + 3 * 2**-8], np.float32))[0] == 0x3F82
    # one rounding of the double value: just above the tie rounds up, whereas
    # a detour through float32 would land exactly on the tie and round down.
    assert o64.cast_bf16(np.array([1 + 2**-8 + 2**-30], np.float64))[0] == 0x3F81
    assert o64.cast_bf16(np.array([-(1 + 2**-8 + 2**-30)], np.float64))[0] == 0xBF81
    assert o64.cast_bf16(np.array([np.inf, -np.inf], np.float64)).tolist() == [0x7F80, 0xFF80]


def test_bf16_widen_exact(o32, o64):
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    w = o32.widen(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(o64.widen(bits)[fin], ref[fin].astype(np.float64))


# ------------------------------------------------------------------ positions
@pytest.mark.parametrize("name,T,h,w", [("positions_t8_h4_w4.txt", 8, 4, 4),
                                         ("positions_t3_h5_w3.txt", 3, 5, 3)])
def test_positions_golden(o32, name, T, h, w):
    g = _golden(name)
    pos = o32.positions(T, h, w)
    assert np.array_equal(g[:, 0].astype(int), np.arange(T + h * w))
    assert np.array_equal(pos, g[:, 1:].astype(np.int32))


@pytest.mark.parametrize("T,h,w", [(256, 64, 64), (512, 83, 83), (512, 104, 58), (512, 58, 104), (0, 1, 1)])
def test_positions_structure(o32, T, h, w):
    """Image indices are centred (each axis spans ceil/floor halves), text is
    on the diagonal and strictly past every image index."""
    pos = o32.positions(T, h, w)
    img = pos[T:]
    assert (img[:, 0] == 0).all()
    assert img[:, 1].min() == -((h + 1) // 2) and img[:, 1].max() == h // 2 - 1
    assert img[:, 2].min() == -((w + 1) // 2) and img[:, 2].max() == w // 2 - 1
    txt = pos[:T]
    assert (txt[:, 0] == txt[:, 1]).all() and (txt[:, 1] == txt[:, 2]).all()
    if T:
        assert txt[0, 0] == max(h // 2, w // 2)
        assert np.array_equal(np.diff(txt[:, 0]), np.ones(T - 1))
        assert txt[0, 0] > img[:, 1:].max()


# ----------------------------------------------------------------------- RoPE
def test_rope_frequencies_closed_form(o64):
    """Angle recovered from the rotation of a unit pair equals p * omega with
    omega from the hand-evaluated closed forms."""
    g = _golden("rope_frequencies.txt")
    for p in (1, 3, -7, 41):
        for k, axis, omega in g:
            k, axis = int(k), int(axis)
            pos = np.zeros((1, 3), np.int32)
            pos[0, axis] = p
            y = np.zeros((1, 1, HD))
            y[0, 0, 2 * k] = 1.0
            out = o64.rope_apply(pos, y)
            phi = p * omega
            assert abs(out[0, 0, 2 * k] - math.cos(phi)) < 1e-15
            assert abs(out[0, 0, 2 * k + 1] - math.sin(phi)) < 1e-15
            # every other channel stays zero
            rest = np.delete(out[0, 0], [2 * k, 2 * k + 1])
            assert not rest.any()


def _rope_complex_ref(pos, y, theta=10000.0):
    """Textbook form: pair k as the complex number y[2k] + i y[2k+1],
    multiplied by exp(i * p_axis(k) * omega_k)."""
    dims = [16, 56, 56]
    omegas, axes = [], []
    for a, d in enumerate(dims):
        for i in range(d // 2):
            omegas.append(theta ** (-2.0 * i / d))
            axes.append(a)
    omegas, axes = np.array(omegas), np.array(axes)
    phi = pos[:, axes].astype(np.float64) * omegas[None, :]          # [n, 64]
    z = y[..., 0::2] + 1j * y[..., 1::2]                             # [n, H, 64]
    r = z * np.exp(1j * phi)[:, None, :]
    out = np.empty_like(y)
    out[..., 0::2], out[..., 1::2] = r.real, r.imag
    return out


def test_rope_matches_complex_multiplication(o64, o32):
    rng = _rng(1)
    pos = rng.integers(-60, 600, size=(50, 3)).astype(np.int32)
    y = rng.standard_normal((50, 3, HD))
    ref = _rope_complex_ref(pos, y)
    assert np.abs(o64.rope_apply(pos, y) - ref).max() < 1e-12
    assert np.abs(o32.rope_apply(pos, y.astype(np.float32)) - ref).max() < 5e-6
    # the pin is sensitive to the pairing: half-split pairs give other values
    half = np.concatenate([y[..., :64, None], y[..., 64:, None]], -1).reshape(y.shape)
    ref_half = _rope_complex_ref(pos, half)
    ref_half = np.concatenate([ref_half[..., 0::2], ref_half[..., 1::2]], -1)
    assert np.abs(ref_half - ref).max() > 0.1


def test_rope_preserves_pair_norm_and_identity(o32):
    rng = _rng(2)
    pos = rng.integers(-60, 600, size=(64, 3)).astype(np.int32)
    y = rng.standard_normal((64, 2, HD)).astype(np.float32)
    out = o32.rope_apply(pos, y)
    n_in = np.hypot(y[..., 0::2].astype(np.float64), y[..., 1::2])
    n_out = np.hypot(out[..., 0::2].astype(np.float64), out[..., 1::2])
    assert np.abs(n_out - n_in).max() <= 4 * 2**-24 * n_in.max()
    zero = np.zeros((4, 3), np.int32)
    ident = o32.rope_apply(zero, y[:4])
    assert np.array_equal(ident, y[:4])


def test_rope_relative_position(o64):
    """<R_p a, R_q b> depends on q - p only: a common shift of every axis
    leaves all pairwise scores unchanged."""
    rng = _rng(3)
    pos = rng.integers(-50, 300, size=(20, 3)).astype(np.int32)
    a = rng.standard_normal((20, 1, HD))
    b = rng.standard_normal((20, 1, HD))
    s0 = o64.rope_apply(pos, a)[:, 0] @ o64.rope_apply(pos, b)[:, 0].T
    for delta in (1, 17, -40, 555):
        s1 = o64.rope_apply(pos + delta, a)[:, 0] @ o64.rope_apply(pos + delta, b)[:, 0].T
        assert np.abs(s1 - s0).max() < 1e-10
    # and a shift of a single axis is not neutral (the axes really act)
    p2 = pos.copy()
    p2[:, 1] += 7
    p2[0, 1] += 1
    s2 = o64.rope_apply(p2, a)[:, 0] @ o64.rope_apply(p2, b)[:, 0].T
    assert np.abs(s2 - s0).max() > 1e-3


# -------------------------------------------------------------------- RMSNorm
def test_rmsnorm_matches_torch(o64, o32):
    rng = _rng(4)
    x = rng.standard_normal((300, HD)) * rng.uniform(0.01, 30, size=(300, 1))
    g = 1 + 0.1 * rng.standard_normal(HD)
    ref = F.rms_norm(torch.from_numpy(x), (HD,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.abs(o64.rmsnorm(x, g) - ref).max() < 1e-13 * np.abs(ref).max()
    got32 = o32.rmsnorm(x.astype(np.float32), g.astype(np.float32))
    assert np.abs(got32 - ref).max() < 2e-6 * np.abs(ref).max()


def test_rmsnorm_closed_forms(o64):
    for c in (1e-4, 0.5, 3.0, -7.0):
        x = np.full((1, HD), c)
        y = o64.rmsnorm(x, np.ones(HD))
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    rng = _rng(5)
    x = rng.standard_normal((10, HD))
    g = rng.standard_normal(HD)
    # homogeneity: x -> a*x with eps -> a^2*eps leaves the output unchanged
    assert np.abs(o64.rmsnorm(1e4 * x, g, eps=1e-6 * 1e8) - o64.rmsnorm(x, g)).max() < 1e-14
    # eps really enters: without the rescaling the outputs move by ~eps/ms
    assert np.abs(o64.rmsnorm(1e4 * x, g) - o64.rmsnorm(x, g)).max() > 1e-8
    assert np.abs(o64.rmsnorm(x, 2 * g) - 2 * o64.rmsnorm(x, g)).max() < 1e-15


# -------------------------------------------------------------- full prologue
def _torch_prologue(x, g, T, h, w, pos_fixture=None):
    """Library composition in float64: torch RMSNorm, then numpy complex
    rotation at the hand-written positions."""
    B, S, H, _ = x.shape
    out = np.empty_like(x)
    for b in range(B):
        gs = g if g.ndim == 1 else None
        for s in range(S):
            gg = gs if gs is not None else (g[0] if (g.shape[0] == 1 or s < T) else g[1])
            out[b, s] = F.rms_norm(torch.from_numpy(x[b, s]), (HD,), weight=torch.from_numpy(gg), eps=1e-6).numpy()
        out[b] = _rope_complex_ref(pos_fixture, out[b])
    return out


@pytest.mark.parametrize("streams", [1, 2])
def test_prologue_matches_library_composition(o64, o32, streams):
    rng = _rng(6)
    T, h, w = 8, 4, 4
    pos = _golden("positions_t8_h4_w4.txt")[:, 1:].astype(np.int32)
    x = rng.standard_normal((2, T + h * w, 3, HD))
    g = 1 + 0.1 * rng.standard_normal((streams, HD))
    ref = _torch_prologue(x, g, T, h, w, pos)
    assert np.abs(o64.qknorm_rope(x, g, T, h, w) - ref).max() < 1e-12
    got32 = o32.qknorm_rope(x.astype(np.float32), g.astype(np.float32), T, h, w)
    assert np.abs(got32 - ref).max() < 1e-5
    # image tokens (frame 0) leave channels 0..15 unrotated: exactly g * xhat
    y32 = got32[:, T:, :, :16]
    gi = g[-1].astype(np.float32)
    xr = x.astype(np.float32)[:, T:]
    direct = o32.rmsnorm(xr.reshape(-1, HD), gi).reshape(xr.shape)[..., :16]
    assert np.array_equal(y32, direct)


# ------------------------------------------------------------------ attention
def _sdpa_ref(q, k, v, txt_len, T):
    """torch scaled_dot_product_attention in float64 with a boolean key mask,
    plus LSE from scipy's logsumexp of torch-matmul scores."""
    B, S, H, _ = q.shape
    o = np.empty((B, S, H, HD))
    lse = np.empty((B, H, S))
    for b in range(B):
        valid = np.array([j < txt_len[b] or j >= T for j in range(S)])
        qt = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))
        kt = torch.from_numpy(np.ascontiguousarray(k[b].transpose(1, 0, 2)))
        vt = torch.from_numpy(np.ascontiguousarray(v[b].transpose(1, 0, 2)))
        mask = torch.from_numpy(valid)[None, None, :].expand(H, S, S)
        ot = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        o[b] = ot.numpy().transpose(1, 0, 2)
        sc = (qt @ kt.transpose(1, 2)).numpy() / math.sqrt(HD)
        lse[b] = logsumexp(np.where(valid[None, None, :], sc, -np.inf), axis=-1)
    return o, lse


ATTN_SHAPES = [  # (B, H, T_txt, txt_len, h, w)
    (1, 2, 8, (5,), 4, 4),
    (2, 2, 7, (0, 7), 3, 5),
    (2, 1, 11, (3, 10), 5, 3),
    (1, 1, 3, (0,), 1, 1),
]


@pytest.mark.parametrize("shape", ATTN_SHAPES)
def test_attention_matches_sdpa(o64, o32, shape):
    B, H, T, Ls, h, w = shape
    S = T + h * w
    rng = _rng(7)
    q, k, v = (rng.standard_normal((B, S, H, HD)) for _ in range(3))
    ref_o, ref_l = _sdpa_ref(q, k, v, Ls, T)
    o, l = o64.attn_fwd(q, k, v, Ls, T)
    assert np.abs(o - ref_o).max() < 1e-12 and np.abs(l - ref_l).max() < 1e-12
    o, l = o32.attn_fwd(*(t.astype(np.float32) for t in (q, k, v)), Ls, T)
    assert np.abs(o - ref_o).max() < 2e-5 and np.abs(l - ref_l).max() < 2e-5


def test_attention_invariants(o32):
    B, H, T, Ls, h, w = 2, 2, 8, (5, 0), 4, 4
    S = T + h * w
    rng = _rng(8)
    q, k, v = (rng.standard_normal((B, S, H, HD)).astype(np.float32) for _ in range(3))
    o, l = o32.attn_fwd(q, k, v, Ls, T)
    # V * 2 -> O * 2 bit for bit (scaling by 2 is exact at every step)
    o2, l2 = o32.attn_fwd(q, k, 2 * v, Ls, T)
    assert np.array_equal(o2, 2 * o) and np.array_equal(l2, l)
    # constant V returns V
    vc = np.broadcast_to(rng.standard_normal(HD).astype(np.float32), v.shape).copy()
    oc, _ = o32.attn_fwd(q, k, vc, Ls, T)
    assert np.abs(oc - vc).max() <= 1e-6 * np.abs(vc).max()
    # Q = 0 -> uniform weights -> mean of the valid V rows
    oz, lz = o32.attn_fwd(np.zeros_like(q), k, v, Ls, T)
    for b in range(B):
        valid = [j for j in range(S) if j < Ls[b] or j >= T]
        mean = v[b, valid].astype(np.float64).mean(0)
        assert np.abs(oz[b] - mean[None]).max() < 1e-6
        assert np.allclose(lz[b], math.log(len(valid)), rtol=0, atol=1e-6)
    # masked keys contribute exactly nothing: poison them
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        kp[b, Ls[b]:T] = np.nan
        vp[b, Ls[b]:T] = 1e30
    op, lp = o32.attn_fwd(q, kp, vp, Ls, T)
    assert np.array_equal(op, o) and np.array_equal(lp, l)
    # batch permutation permutes the outputs bit for bit
    orev, lrev = o32.attn_fwd(q[::-1], k[::-1], v[::-1], Ls[::-1], T)
    assert np.array_equal(orev, o[::-1]) and np.array_equal(lrev, l[::-1])


def test_softmax_rows_sum_to_one(o32):
    """With V = identity rows, O_i[j] is the attention weight p_ij."""
    T, L, h, w = 8, 5, 4, 4
    S = T + h * w
    rng = _rng(9)
    q = (2 * rng.standard_normal((1, S, 1, HD))).astype(np.float32)
    k = (2 * rng.standard_normal((1, S, 1, HD))).astype(np.float32)
    v = np.zeros((1, S, 1, HD), np.float32)
    for j in range(S):
        v[0, j, 0, j] = 1
    o, _ = o32.attn_fwd(q, k, v, [L], T)
    p = o[0, :, 0, :S]
    assert np.abs(p.sum(1) - 1).max() < 1e-6
    assert not p[:, L:T].any()                 # masked keys have weight 0
    assert (p[:, list(range(L)) + list(range(T, S))] > 0).all()


def test_single_key(o32):
    """h = w = 1 and no text: one key; every row returns it, LSE = its score."""
    T, h, w = 3, 1, 1
    rng = _rng(10)
    q, k, v = (rng.standard_normal((1, 4, 1, HD)).astype(np.float32) for _ in range(3))
    o, l = o32.attn_fwd(q, k, v, [0], T)
    assert np.array_equal(o[0, :, 0], np.broadcast_to(v[0, 3, 0], (4, HD)))
    s = (q[0, :, 0].astype(np.float64) @ k[0, 3, 0].astype(np.float64)) / math.sqrt(HD)
    assert np.abs(l[0, 0] - s).max() < 1e-5


def test_oracle_thread_count_independent(o32):
    B, H, T, Ls, h, w = 1, 2, 8, (5,), 6, 6
    S = T + h * w
    rng = _rng(11)
    q, k, v, d = (rng.standard_normal((B, S, H, HD)).astype(np.float32) for _ in range(4))
    try:
        o32.set_threads(1)
        a = o32.attn_fwd(q, k, v, Ls, T)
        ab = o32.attn_bwd(q, k, v, d, Ls, T)
        o32.set_threads(8)
        c = o32.attn_fwd(q, k, v, Ls, T)
        cb = o32.attn_bwd(q, k, v, d, Ls, T)
    finally:
        o32.set_threads(os.cpu_count() or 1)
    assert all(np.array_equal(x, y) for x, y in zip(a, c))
    assert all(np.array_equal(x, y) for x, y in zip(ab, cb))


# ------------------------------------------------------------------- backward
def _chain_f64(o64, xq, xk, v, gq, gk, Ls, T, h, w):
    yq = o64.qknorm_rope(xq, gq, T, h, w)
    yk = o64.qknorm_rope(xk, gk, T, h, w)
    o, _ = o64.attn_fwd(yq, yk, v, Ls, T)
    return yq, yk, o


def _chain_grads(o64, xq, xk, v, gq, gk, dO, Ls, T, h, w):
    yq, yk, _ = _chain_f64(o64, xq, xk, v, gq, gk, Ls, T, h, w)
    dqp, dkp, dv = o64.attn_bwd(yq, yk, v, dO, Ls, T)
    dxq, dgq = o64.qknorm_rope_bwd(xq, gq, dqp, T, h, w)
    dxk, dgk = o64.qknorm_rope_bwd(xk, gk, dkp, T, h, w)
    return dict(xq=dxq, xk=dxk, v=dv, gq=fold_batch(dgq), gk=fold_batch(dgk), dqp=dqp, dkp=dkp)


@pytest.mark.parametrize("streams", [1, 2])
def test_backward_matches_torch_autograd(o64, streams):
    """Whole-chain gradients vs torch autograd through library ops in
    float64 (F.rms_norm with weight, complex rotation, SDPA with a mask)."""
    B, H, T, Ls, h, w = 2, 2, 8, (5, 2), 4, 4
    S = T + h * w
    rng = _rng(12)
    xq, xk, v, dO = (rng.standard_normal((B, S, H, HD)) for _ in range(4))
    gq = 1 + 0.1 * rng.standard_normal((streams, HD))
    gk = 1 + 0.1 * rng.standard_normal((streams, HD))
    got = _chain_grads(o64, xq, xk, v, gq, gk, dO, Ls, T, h, w)

    pos = torch.from_numpy(_golden("positions_t8_h4_w4.txt")[:, 1:])
    dims = [16, 56, 56]
    om, ax = [], []
    for a, d in enumerate(dims):
        for i in range(d // 2):
            om.append(10000.0 ** (-2.0 * i / d))
            ax.append(a)
    phi = pos[:, ax].double() * torch.tensor(om, dtype=torch.float64)[None]
    rot = torch.polar(torch.ones_like(phi), phi)                        # [S, 64]

    T_ = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    txq, txk, tv, tgq, tgk = T_(xq), T_(xk), T_(v), T_(gq), T_(gk)

    def prologue(x, g):
        parts = []
        for s in range(S):
            gg = g[0] if (g.shape[0] == 1 or s < T) else g[1]
            parts.append(F.rms_norm(x[:, s], (HD,), weight=gg, eps=1e-6))
        y = torch.stack(parts, 1)                                        # [B,S,H,128]
        z = torch.view_as_complex(y.reshape(B, S, H, 64, 2).contiguous())
        return torch.view_as_real(z * rot[None, :, None, :]).reshape(B, S, H, HD)

    yq, yk = prologue(txq, tgq), prologue(txk, tgk)
    outs = []
    for b in range(B):
        valid = torch.tensor([j < Ls[b] or j >= T for j in range(S)])
        mask = valid[None, None, :].expand(H, S, S)
        ob = F.scaled_dot_product_attention(yq[b].transpose(0, 1), yk[b].transpose(0, 1),
                                            tv[b].transpose(0, 1), attn_mask=mask)
        outs.append(ob.transpose(0, 1))
    o = torch.stack(outs)
    (o * torch.from_numpy(dO)).sum().backward()
    for name, t in (("xq", txq), ("xk", txk), ("v", tv), ("gq", tgq), ("gk", tgk)):
        ref = t.grad.numpy()
        assert np.abs(got[name] - ref).max() < 1e-10 * max(1.0, np.abs(ref).max()), name


def test_backward_finite_differences(o64):
    """Central differences of L = sum(dO * O) through the whole chain."""
    B, H, T, Ls, h, w = 1, 2, 8, (5,), 4, 4
    S = T + h * w
    rng = _rng(13)
    xq, xk, v, dO = (rng.standard_normal((B, S, H, HD)) for _ in range(4))
    gq = 1 + 0.1 * rng.standard_normal((1, HD))
    gk = 1 + 0.1 * rng.standard_normal((1, HD))
    got = _chain_grads(o64, xq, xk, v, gq, gk, dO, Ls, T, h, w)
    args = dict(xq=xq, xk=xk, v=v, gq=gq, gk=gk)

    def loss(a):
        _, _, o = _chain_f64(o64, a["xq"], a["xk"], a["v"], a["gq"], a["gk"], Ls, T, h, w)
        return float((o * dO).sum())

    eps = 1e-5
    for name in args:
        flat_idx = rng.choice(args[name].size, size=6, replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, args[name].shape)
            a_p = {k_: v_.copy() for k_, v_ in args.items()}
            a_m = {k_: v_.copy() for k_, v_ in args.items()}
            a_p[name][idx] += eps
            a_m[name][idx] -= eps
            fd = (loss(a_p) - loss(a_m)) / (2 * eps)
            assert abs(fd - got[name][idx]) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, got[name][idx])


def test_backward_attention_identities(o32):
    B, H, T, Ls, h, w = 2, 2, 8, (5, 0), 4, 4
    S = T + h * w
    rng = _rng(14)
    q, k, v, dO = (rng.standard_normal((B, S, H, HD)).astype(np.float32) for _ in range(4))
    dq, dk, dv = o32.attn_bwd(q, k, v, dO, Ls, T)
    for b in range(B):
        # masked keys receive exactly zero gradient
        assert not dk[b, Ls[b]:T].any() and not dv[b, Ls[b]:T].any()
        # shift invariance of softmax: sum over keys of dk' vanishes
        assert np.abs(dk[b].astype(np.float64).sum(0)).max() < 1e-4
        # dv = P^T dO with P from torch's float64 softmax
        for hh in range(H):
            valid = torch.tensor([j < Ls[b] or j >= T for j in range(S)])
            sc = torch.from_numpy(q[b, :, hh].astype(np.float64)) @ torch.from_numpy(k[b, :, hh].astype(np.float64)).T
            sc = (sc / math.sqrt(HD)).masked_fill(~valid[None, :], -math.inf)
            P = torch.softmax(sc, -1).numpy()
            ref = P.T @ dO[b, :, hh].astype(np.float64)
            assert np.abs(dv[b, :, hh] - ref).max() < 1e-5


def test_forward_path_against_library_composition(o32):
    """forward_path (prologue, one BF16 cast, attention on the cast values)
    against an independent float64 composition: torch RMSNorm and numpy
    complex rotation at the hand-written positions, torch's BF16 cast, then
    torch SDPA with the boolean key mask."""
    wl = workloads.WORKLOADS["tiny"]
    inp = workloads.make_inputs(wl)
    bq, bk, bv = (workloads.bits(inp[n]) for n in ("q", "k", "v"))
    gq, gk = inp["g_q"].numpy(), inp["g_k"].numpy()
    fw = forward_path(o32, bq, bk, bv, gq, gk, inp["txt_len"], wl.T_txt, wl.h, wl.w)
    pos = _golden("positions_t8_h4_w4.txt")[:, 1:].astype(np.int32)
    ref_bits = {}
    for n, x, g in (("q", inp["q"], gq), ("k", inp["k"], gk)):
        pre = _torch_prologue(x.double().numpy(), g.astype(np.float64), wl.T_txt, wl.h, wl.w, pos)
        assert np.abs(fw[f"{n}_pre"] - pre).max() < 2e-5
        rb = torch.from_numpy(pre).to(torch.bfloat16)
        ref_bits[n] = rb.view(torch.int16).numpy().view(np.uint16)
        got = fw[f"{n}_bf16"]
        # one RNE cast of values that agree to ~1e-6: equal bits except where
        # a value sits on a rounding boundary (then one BF16 step apart)
        same = got == ref_bits[n]
        assert same.mean() > 0.99
        gv = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.all(np.abs(gv - rb.double().numpy()) <= 2.0 ** -7 * np.abs(rb.double().numpy()) + 1e-30)
    widen = lambda u: torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).double().numpy()  # noqa: E731
    ref_o, ref_l = _sdpa_ref(widen(fw["q_bf16"]), widen(fw["k_bf16"]), widen(bv), inp["txt_len"], wl.T_txt)
    assert np.abs(fw["o"] - ref_o).max() < 2e-5 and np.abs(fw["lse"] - ref_l).max() < 2e-5
    ob = torch.from_numpy(fw["o"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fw["o_bf16"], ob)
    assert fw["o_bf16"].shape == (1, 24, 2, HD)


def test_qkv_path_against_numpy_composition(o64):
    """qkv_path against numpy float64: the per-stream projection x W^T + b
    (text rows with set 0, image rows with set 1), torch's BF16 cast, the
    packed layout written out index by index (Q channels 0..D-1, K D..2D-1, V
    2D..3D-1, head h at 128h), then the prologue of the float64 library
    composition on Q and K."""
    rng = _rng(23)
    B, H, T, h, w = 2, 2, 8, 4, 4
    S, D = T + h * w, H * HD
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    ub = lambda t: t.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    x = bf(rng.standard_normal((B, S, D)))
    W = bf(rng.standard_normal((2, 3 * D, D)) / math.sqrt(D))
    bias = 0.02 * rng.standard_normal((2, 3 * D))
    gq, gk = 1 + 0.1 * rng.standard_normal((1, HD)), 1 + 0.1 * rng.standard_normal((1, HD))
    got = qkv_path(o64, ub(x), ub(W), bias, gq, gk, T, h, w)
    xd, Wd = x.double().numpy(), W.double().numpy()
    y = np.empty((B, S, 3 * D))
    y[:, :T] = xd[:, :T] @ Wd[0].T + bias[0]
    y[:, T:] = xd[:, T:] @ Wd[1].T + bias[1]
    assert np.abs(got["y"] - y).max() < 1e-12
    yb = ub(torch.from_numpy(y).to(torch.bfloat16))
    for i, n in enumerate(("q", "k", "v")):
        ref = np.empty((B, S, H, HD), dtype=np.uint16)
        for hh in range(H):
            for c in range(HD):
                ref[:, :, hh, c] = yb[:, :, i * D + 128 * hh + c]
        assert np.array_equal(got[n], ref), n
    pos = _golden("positions_t8_h4_w4.txt")[:, 1:].astype(np.int32)
    for n, g in (("q", gq), ("k", gk)):
        xin = torch.from_numpy(got[n].view(np.int16)).view(torch.bfloat16).double().numpy()
        pre = _torch_prologue(xin, g[0], T, h, w, pos)
        rb = ub(torch.from_numpy(pre).to(torch.bfloat16))
        assert (got[f"{n}_prime"] == rb).mean() > 0.99


# ------------------------------------------------- attention, one operator at a time
def _tile_keys(T, L, S):
    """Keys of each logical 64-key tile of a row with text length L: text
    tiles from key 0, then image tiles from key T (the key tiling of the
    online softmax)."""
    tiles = [list(range(t, min(t + 64, L))) for t in range(0, L, 64)]
    tiles += [list(range(t, min(t + 64, S))) for t in range(T, S, 64)]
    return tiles


OPERATOR_SHAPES = [  # (T_txt, L, h, w)
    (8, 5, 4, 4),
    (70, 67, 9, 9),
    (0, 0, 13, 11),
    (130, 130, 3, 2),
]


@pytest.mark.parametrize("shape", OPERATOR_SHAPES)
def test_operator_scores_and_softmax_match_library(o64, shape):
    """Scaled scores equal a float64 torch matmul over the valid keys (0 on
    masked keys); the softmax rows equal scipy's softmax / logsumexp."""
    T, L, h, w = shape
    S = T + h * w
    rng = _rng(11)
    q, k = rng.standard_normal((S, HD)), rng.standard_normal((S, HD))
    valid = np.array([j < L or j >= T for j in range(S)])
    ref = (torch.from_numpy(q) @ torch.from_numpy(k).T).numpy() / math.sqrt(HD)
    s = o64.attn_scores_bh(q, k, T, L)
    assert np.abs(s[:, valid] - ref[:, valid]).max() < 1e-12
    assert (s[:, ~valid] == 0).all()
    s2 = o64.attn_scores_bh(q, k, T, L, 3, min(S, 9))
    assert np.array_equal(s2, s[3:min(S, 9)])
    sm = np.where(valid[None], 5 * s, -np.inf)
    lse_ref = logsumexp(sm, axis=-1)
    p, lse = o64.attn_softmax_rows(5 * s, T, L)
    assert np.abs(p - np.exp(sm - lse_ref[:, None])).max() < 1e-14
    assert np.abs(lse - lse_ref).max() < 1e-12
    assert (p[:, ~valid] == 0).all()


@pytest.mark.parametrize("shape", OPERATOR_SHAPES)
def test_operator_av_recurrence(o64, shape):
    """The A.V recurrence over logical tiles (1) with factors from a running
    maximum reproduces softmax(s) v from torch SDPA, and (2) for arbitrary
    P, alpha, l equals the closed form sum_t (prod_{u>t} alpha_u) P_t V_t / l."""
    T, L, h, w = shape
    S = T + h * w
    rng = _rng(12)
    q, k, v = (rng.standard_normal((S, HD)) for _ in range(3))
    tiles = _tile_keys(T, L, S)
    nt = len(tiles) + 1  # one unused slot past the row's tiles
    s = o64.attn_scores_bh(q, k, T, L)
    n = S
    P = np.full((n, nt, 64), np.nan)  # unused slots must be ignored
    alpha = np.full((n, nt), np.nan)
    l = np.zeros(n)
    m = np.full(n, -np.inf)
    for t, keys in enumerate(tiles):
        st = s[:, keys]
        m_new = np.maximum(m, st.max(axis=1))
        alpha[:, t] = np.exp(m - m_new)
        P[:, t, :len(keys)] = np.exp(st - m_new[:, None])
        l = alpha[:, t] * l + P[:, t, :len(keys)].sum(axis=1)
        m = m_new
    o = o64.attn_av_rows(P, alpha, l, v, T, L)
    valid = torch.tensor([j < L or j >= T for j in range(S)])
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], attn_mask=valid[None, None, :].expand(1, S, S))
    assert np.abs(o - ref[0].numpy()).max() < 1e-12

    # (2) arbitrary P, alpha, l: the operator's recurrence acc <- alpha_t acc
    # + P_t V_t, O = acc / l, run tile by tile in float64 (the route the
    # operator is specified by; the oracle evaluates the closed form)
    Pr = rng.uniform(0, 2, (n, nt, 64))
    ar = rng.uniform(0.25, 1, (n, nt))
    lr = rng.uniform(1, 64, n)
    o = o64.attn_av_rows(Pr, ar, lr, v, T, L)
    acc = np.zeros((n, HD))
    for t, keys in enumerate(tiles):
        acc = ar[:, t:t + 1] * acc + Pr[:, t, :len(keys)] @ v[keys]
    assert np.abs(o - acc / lr[:, None]).max() < 1e-12
    # a factor of 0 at tile t erases every tile before it
    if len(tiles) > 1:
        az = ar.copy()
        az[:, 1] = 0.0
        oz = o64.attn_av_rows(Pr, az, lr, v, T, L)
        ref = np.zeros((n, HD))
        for t, keys in enumerate(tiles[1:], start=1):
            ref = az[:, t:t + 1] * ref + Pr[:, t, :len(keys)] @ v[keys]
        assert np.abs(oz - ref / lr[:, None]).max() < 1e-12


BLOCK_CASES = [  # (T_txt, L, h, w, with_text, img_lo, img_hi)
    (8, 5, 4, 4, True, 0, 0),
    (8, 5, 4, 4, False, 0, 16),
    (70, 67, 13, 11, True, 64, 128),
    (70, 67, 13, 11, False, 128, 143),
    (3, 0, 5, 5, True, 0, 25),
]


@pytest.mark.parametrize("case", BLOCK_CASES)
def test_block_attention_matches_sdpa(o64, case):
    """Attention restricted to one key block equals torch SDPA with the
    block's boolean key mask; rows of a block without keys are not asked
    for.  The full block (text + all image keys) equals the plain forward."""
    T, L, h, w, with_text, lo, hi = case
    S = T + h * w
    rng = _rng(13)
    q, k, v = (rng.standard_normal((S, HD)) for _ in range(3))
    keys = [j for j in range(S) if (with_text and j < L) or (T + lo <= j < T + hi)]
    if not keys:
        pytest.skip("block without keys")
    mask = torch.zeros(S, dtype=torch.bool)
    mask[keys] = True
    qt, kt, vt = (torch.from_numpy(t)[None] for t in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None, :].expand(1, S, S))[0].numpy()
    sc = (q @ k.T) / math.sqrt(HD)
    ref_lse = logsumexp(np.where(mask.numpy()[None, :], sc, -np.inf), axis=-1)
    o, lse = o64.attn_fwd_block_bh(q, k, v, T, L, with_text, lo, hi)
    assert np.abs(o - ref).max() < 1e-12 and np.abs(lse - ref_lse).max() < 1e-12
    of, lf = o64.attn_fwd_block_bh(q, k, v, T, L, True, 0, h * w)
    o_all, l_all = o64.attn_fwd_bh(q, k, v, T, L)
    assert np.array_equal(of, o_all) and np.array_equal(lf, l_all)


# ------------------------------------------------------------ projections
def test_linear_matches_numpy(o64):
    """y = x W^T + b against numpy's float64 matmul, on shapes with odd K, N."""
    rng = _rng(21)
    for n, K, N in ((1, 1, 1), (7, 130, 33), (64, 256, 384)):
        x, W, b = rng.standard_normal((n, K)), rng.standard_normal((N, K)), rng.standard_normal(N)
        y = o64.linear(x, W, b)
        assert np.abs(y - (x @ W.T + b)).max() <= 1e-12 * max(1.0, np.abs(x @ W.T).max())


def test_stream_linear_selects_weights_by_segment(o64):
    """Text rows use weight set 0, image rows the last set: with W_img = 0 the
    image rows equal the image bias exactly, and with one set both agree."""
    rng = _rng(22)
    B, T, S, K, N = 2, 5, 12, 16, 8
    x = rng.standard_normal((B, S, K))
    W = np.stack([rng.standard_normal((N, K)), np.zeros((N, K))])
    b = rng.standard_normal((2, N))
    y = o64.stream_linear(x, W, b, T)
    assert np.array_equal(y[:, T:], np.broadcast_to(b[1], (B, S - T, N)))
    assert np.abs(y[:, :T] - (x[:, :T] @ W[0].T + b[0])).max() < 1e-12
    y1 = o64.stream_linear(x, W[:1], b[:1], T)
    assert np.abs(y1 - (x @ W[0].T + b[0])).max() < 1e-12
    y0 = o64.stream_linear(x, W, b, 0)  # no text rows
    assert np.array_equal(y0, np.broadcast_to(b[1], (B, S, N)))
