"""CPU-side checks of the C ABI: the library loads, exports every entry point
that include/qi.h declares, rejects invalid arguments before touching a device
(no compute is launched here: there is no GPU), and reports its contract."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import invariant_joint_attention_amd as qi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qi.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qi.LIB_PATH), reason="libqi.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qi_[a-z0-9_]+)\s*\(", text)))


def test_header_lists_the_binding_symbols():
    assert declared_symbols() == sorted(qi.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = qi.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (qi_\w+)", out))
    assert set(declared_symbols()) <= exported


def test_trace_is_json_with_the_frozen_contract():
    t = json.loads(qi.trace())
    assert t["target"] == "gfx950"
    assert t["split_k"] is False and t["split_kv"] is False and t["atomics"] is False
    assert t["fast_math"] is False and t["fp_contract"] == "off"
    assert t["frozen"]["fwd_key_tile"] == 64
    # every kernel the trace names is one the library defines (the entry points' launches)
    for name in ("attn_fwd_kernel", "attn_fwd_partial_kernel", "attn_fwd_carry_kernel", "attn_merge_kernel"):
        assert name in t["kernels"].values()


# Fake, never-dereferenced device addresses (validation only looks at them).
BASE = 0x7F0000000000


def fake_bshd(addr, B, S, H, sb=None, ss=None, sh=None):
    sh = 128 if sh is None else sh
    ss = H * sh if ss is None else ss
    sb = S * ss if sb is None else sb
    return qi.QiBshd(addr, sb, ss, sh)


def region(i):
    return BASE + i * (1 << 32)


def fwd_call(geom, q=None, k=None, v=None, o=None, lse=None, of=None, ws=None, ws_bytes=None):
    g = geom
    q = q or fake_bshd(region(0), g.B, g.S, g.H)
    k = k or fake_bshd(region(1), g.B, g.S, g.H)
    v = v or fake_bshd(region(2), g.B, g.S, g.H)
    o = o or fake_bshd(region(3), g.B, g.S, g.H)
    lse = region(4) if lse is None else lse
    ws = region(5) if ws is None else ws
    if ws_bytes is None:
        ws_bytes = qi.lib().qi_joint_attn_fwd_workspace(g.ptr())
    return qi.lib().qi_joint_attn_fwd(g.ptr(), q, k, v, o, lse, of, ws, ws_bytes, None)


def geom(**kw):
    args = dict(B=1, H=2, T_txt=8, grid_h=4, grid_w=4, txt_len=[5])
    args.update(kw)
    return qi.Geometry(**args)


def code(name):
    return {v: k for k, v in qi.STATUS.items()}[name]


@pytest.mark.parametrize("kw,expect", [
    (dict(D=64), "QI_E_UNSUPPORTED"),
    (dict(rope_axes=(16, 48, 64)), "QI_E_UNSUPPORTED"),
    (dict(B=0, txt_len=[]), "QI_E_INVALID"),
    (dict(H=0), "QI_E_INVALID"),
    (dict(grid_h=0), "QI_E_INVALID"),
    (dict(T_txt=-1), "QI_E_INVALID"),
    (dict(txt_len=[9]), "QI_E_INVALID"),
    (dict(txt_len=[-1]), "QI_E_INVALID"),
    (dict(rms_eps=0.0), "QI_E_INVALID"),
    (dict(rms_eps=float("nan")), "QI_E_INVALID"),
    (dict(rope_theta=float("inf")), "QI_E_INVALID"),
    (dict(gain_streams=3), "QI_E_INVALID"),
])
def test_invalid_geometry_fails_closed(kw, expect):
    g = geom(**kw)
    assert fwd_call(g, ws_bytes=1 << 20) == code(expect)
    assert qi.last_error() != ""
    assert qi.lib().qi_joint_attn_bwd_workspace(g.ptr()) == 0
    assert qi.lib().qi_joint_attn_fwd_workspace(g.ptr()) == 0


def test_null_and_misaligned_pointers():
    g = geom()
    assert fwd_call(g, q=qi.QiBshd(0, 0, 0, 0)) == code("QI_E_INVALID")
    assert fwd_call(g, q=fake_bshd(region(0) + 8, g.B, g.S, g.H)) == code("QI_E_ALIGN")
    assert fwd_call(g, lse=region(4) + 4) == code("QI_E_ALIGN")
    # a stride that is not a multiple of 16 bytes
    assert fwd_call(g, k=fake_bshd(region(1), g.B, g.S, g.H, sh=132)) == code("QI_E_ALIGN")
    assert fwd_call(g, k=fake_bshd(region(1), g.B, g.S, g.H, sh=-128)) == code("QI_E_INVALID")


def test_forward_workspace_validation():
    g = geom()
    L = qi.lib()
    ws = L.qi_joint_attn_fwd_workspace(g.ptr())
    # B*H*nt FP16 tiles of 64 keys x 128 channels, nt = ceil(T_txt/64) + ceil(h*w/64), rounded up to 256 bytes
    nt = -(-g.T_txt // 64) + -(-(g.grid_h * g.grid_w) // 64)
    assert ws == -(-(g.B * g.H * nt * 64 * 128 * 2) // 256) * 256
    assert fwd_call(g, ws=0) == code("QI_E_WORKSPACE")
    assert fwd_call(g, ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    assert fwd_call(g, ws=region(5) + 16) == code("QI_E_ALIGN")
    # the workspace may overlap nothing else, inputs included
    assert fwd_call(g, ws=region(2)) == code("QI_E_ALIAS")
    assert fwd_call(g, ws=region(3) + 256) == code("QI_E_ALIAS")
    assert fwd_call(g) == code("QI_E_UNSUPPORTED")  # valid: stops at the device gate


def test_aliasing_is_rejected():
    g = geom()
    # output equal to an input
    assert fwd_call(g, o=fake_bshd(region(0), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    # output overlapping the LSE buffer
    assert fwd_call(g, lse=region(3) + 256) == code("QI_E_ALIAS")
    # an output view whose elements overlap each other (head stride 64 < 128)
    assert fwd_call(g, o=fake_bshd(region(3), g.B, g.S, g.H, sh=64)) == code("QI_E_ALIAS")
    # inputs may alias each other (q = k) -- only outputs are exclusive
    rc = fwd_call(g, k=fake_bshd(region(0), g.B, g.S, g.H))
    assert rc != code("QI_E_ALIAS")


def test_valid_call_without_gpu_reports_no_device():
    """All arguments valid: the only failure left on a GPU-less host is the
    device gate, and nothing is launched."""
    g = geom()
    rc = fwd_call(g)
    assert rc == code("QI_E_UNSUPPORTED"), qi.last_error()


def test_prologue_and_backward_validation():
    g = geom()
    L = qi.lib()
    x = fake_bshd(region(0), g.B, g.S, g.H)
    y = fake_bshd(region(1), g.B, g.S, g.H)
    assert L.qi_qknorm_rope(g.ptr(), x, region(2), x, None, None) == code("QI_E_ALIAS")
    assert L.qi_qknorm_rope(g.ptr(), x, None, y, None, None) == code("QI_E_INVALID")
    assert L.qi_qknorm_rope(g.ptr(), x, region(2), y, region(3) + 4, None) == code("QI_E_ALIGN")
    ws = L.qi_joint_attn_bwd_workspace(g.ptr())
    assert ws > 0 and ws % 256 == 0
    views = [fake_bshd(region(i), g.B, g.S, g.H) for i in range(6)]
    dout = fake_bshd(region(7), g.B, g.S, g.H)
    grads = [fake_bshd(region(10 + i), g.B, g.S, g.H, sh=128) for i in range(3)]

    def bwd(ws_ptr=region(20), ws_bytes=ws, dq=None):
        return L.qi_joint_attn_bwd(g.ptr(), *views, region(6), dout, region(8), region(9),
                                   dq or grads[0], grads[1], grads[2], region(14), region(15), None, None,
                                   ws_ptr, ws_bytes, None)

    assert bwd(ws_ptr=None) == code("QI_E_WORKSPACE")
    assert bwd(ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    assert bwd(ws_ptr=region(20) + 16) == code("QI_E_ALIGN")
    assert bwd(dq=fake_bshd(region(0), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    assert bwd() == code("QI_E_UNSUPPORTED")


def test_strict_probe_without_gpu():
    assert qi.lib().qi_strict_probe(0) == code("QI_E_UNSUPPORTED")


def test_row_strides_beyond_32_bit_lane_offsets_are_refused():
    """The attention kernels address 16 rows of K, V (and Q, dO in the
    backward) from one scalar base with 32-bit lane offsets; a sequence
    stride of 2^26 elements or more is refused before any device work."""
    g = geom()
    big = (1 << 26) + 128
    rc = fwd_call(g, k=fake_bshd(region(1), g.B, g.S, g.H, ss=big, sb=g.S * big))
    assert rc == code("QI_E_UNSUPPORTED") and "stride" in qi.last_error()
    # v is read by a conversion pass with 64-bit addressing, so its stride is free
    rc = fwd_call(g, v=fake_bshd(region(2), g.B, g.S, g.H, ss=big, sb=g.S * big))
    assert rc == code("QI_E_UNSUPPORTED") and "stride" not in qi.last_error()
    # at the limit itself the call passes validation (and stops at the device gate)
    ok = 1 << 26
    rc = fwd_call(g, k=fake_bshd(region(1), g.B, g.S, g.H, ss=ok, sb=g.S * ok))
    assert rc == code("QI_E_UNSUPPORTED") and "stride" not in qi.last_error()

    L = qi.lib()
    ws = L.qi_joint_attn_bwd_workspace(g.ptr())
    for bad in (0, 3):  # q_raw is not addressed by the attention passes; q and d_o are
        views = [fake_bshd(region(i), g.B, g.S, g.H) for i in range(6)]
        dout = fake_bshd(region(7), g.B, g.S, g.H)
        if bad == 0:
            dout = fake_bshd(region(7), g.B, g.S, g.H, ss=big, sb=g.S * big)
        else:
            views[2] = fake_bshd(region(2), g.B, g.S, g.H, ss=big, sb=g.S * big)  # q
        grads = [fake_bshd(region(10 + i), g.B, g.S, g.H) for i in range(3)]
        rc = L.qi_joint_attn_bwd(g.ptr(), *views, region(6), dout, region(8), region(9), *grads,
                                 region(14), region(15), None, None, region(20), ws, None)
        assert rc == code("QI_E_UNSUPPORTED") and "stride" in qi.last_error(), qi.last_error()


def test_unfused_operators_validation():
    """The three unfused operators: key-slot count, argument checks before any
    launch, and the device gate for valid calls."""
    g = geom()
    L = qi.lib()
    nt = -(-g.T_txt // 64) + -(-(g.grid_h * g.grid_w) // 64)
    assert L.qi_joint_attn_key_slots(g.ptr()) == 64 * nt
    assert L.qi_joint_attn_key_slots(geom(D=64).ptr()) == 0
    q = fake_bshd(region(0), g.B, g.S, g.H)
    k = fake_bshd(region(1), g.B, g.S, g.H)
    v = fake_bshd(region(2), g.B, g.S, g.H)
    o = fake_bshd(region(3), g.B, g.S, g.H)
    # scores
    assert L.qi_joint_attn_qk_gemm(g.ptr(), q, k, region(4), None) == code("QI_E_UNSUPPORTED")
    assert L.qi_joint_attn_qk_gemm(g.ptr(), q, k, None, None) == code("QI_E_INVALID")
    assert L.qi_joint_attn_qk_gemm(g.ptr(), q, k, region(4) + 8, None) == code("QI_E_ALIGN")
    assert L.qi_joint_attn_qk_gemm(g.ptr(), q, k, region(1), None) == code("QI_E_ALIAS")
    assert L.qi_joint_attn_qk_gemm(geom(H=70000).ptr(), q, k, region(4), None) == code("QI_E_UNSUPPORTED")
    # softmax: p, alpha, l, lse are outputs and may overlap nothing
    sm = lambda s=region(4), p=region(5), a=region(6), l=region(7), e=region(8): \
        L.qi_joint_attn_softmax(g.ptr(), s, p, a, l, e, None)  # noqa: E731
    assert sm() == code("QI_E_UNSUPPORTED")
    assert sm(p=None) == code("QI_E_INVALID")
    assert sm(a=region(6) + 4) == code("QI_E_ALIGN")
    assert sm(l=region(8)) == code("QI_E_ALIAS")
    assert sm(p=region(4)) == code("QI_E_ALIAS")
    # A.V
    ws = L.qi_joint_attn_fwd_workspace(g.ptr())
    av = lambda o=o, ws_ptr=region(9), ws_bytes=ws, of=None: \
        L.qi_joint_attn_av_gemm(g.ptr(), region(5), region(6), region(7), v, o, of, ws_ptr, ws_bytes, None)  # noqa: E731
    assert av() == code("QI_E_UNSUPPORTED")
    assert av(ws_ptr=None) == code("QI_E_WORKSPACE")
    assert av(ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    assert av(ws_ptr=region(9) + 16) == code("QI_E_ALIGN")
    assert av(o=fake_bshd(region(5), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    assert av(of=region(7)) == code("QI_E_ALIAS")


def test_block_forward_and_merge_validation():
    """Key-block forward and merge: block ranges, outputs, workspace and
    n_blocks are checked before any launch."""
    g = geom()  # T_img = 16
    L = qi.lib()
    q = fake_bshd(region(0), g.B, g.S, g.H)
    k = fake_bshd(region(1), g.B, g.S, g.H)
    v = fake_bshd(region(2), g.B, g.S, g.H)
    ws = L.qi_joint_attn_fwd_workspace(g.ptr())

    def part(blk=(1, 0, 16), acc=region(4), m=region(5), l=region(6), ws_ptr=region(9), ws_bytes=ws):
        return L.qi_joint_attn_fwd_partial(g.ptr(), q, k, v, qi.QiKeyBlock(*blk), acc, m, l, ws_ptr, ws_bytes, None)

    assert part() == code("QI_E_UNSUPPORTED")  # valid: stops at the device gate
    assert part(blk=(1, 0, 0)) == code("QI_E_UNSUPPORTED")  # text keys only
    assert part(blk=(0, 0, 16)) == code("QI_E_UNSUPPORTED")  # image keys only
    assert part(blk=(0, 0, 0)) == code("QI_E_INVALID")  # empty
    assert part(blk=(2, 0, 16)) == code("QI_E_INVALID")
    assert part(blk=(1, 0, 17)) == code("QI_E_INVALID")  # past the image keys
    assert part(blk=(1, 8, 16)) == code("QI_E_INVALID")  # not tile-aligned
    assert part(blk=(1, 16, 8)) == code("QI_E_INVALID")
    assert part(acc=None) == code("QI_E_INVALID")
    assert part(m=region(5) + 2) == code("QI_E_ALIGN")
    assert part(m=region(5) + 4) == code("QI_E_UNSUPPORTED")  # one word per row: 4-byte alignment
    assert part(acc=region(4) + 4) == code("QI_E_ALIGN")
    assert part(l=region(5)) == code("QI_E_ALIAS")
    assert part(acc=region(1)) == code("QI_E_ALIAS")
    assert part(ws_ptr=None) == code("QI_E_WORKSPACE")
    assert part(ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    g2 = geom(grid_h=16, grid_w=9)  # T_img = 144: a block may end at T_img
    assert L.qi_joint_attn_fwd_partial(g2.ptr(), fake_bshd(region(0), g2.B, g2.S, g2.H),
                                       fake_bshd(region(1), g2.B, g2.S, g2.H), fake_bshd(region(2), g2.B, g2.S, g2.H),
                                       qi.QiKeyBlock(0, 128, 144), region(4), region(5), region(6), region(9),
                                       L.qi_joint_attn_fwd_workspace(g2.ptr()), None) == code("QI_E_UNSUPPORTED")

    o = fake_bshd(region(3), g.B, g.S, g.H)

    def merge(n=2, acc=region(4), m=region(5), l=region(6), o=o, lse=region(7), of=None):
        return L.qi_joint_attn_merge(g.ptr(), n, acc, m, l, o, lse, of, None)

    assert merge() == code("QI_E_UNSUPPORTED")
    assert merge(n=0) == code("QI_E_INVALID")
    assert merge(n=4097) == code("QI_E_INVALID")
    assert merge(m=None) == code("QI_E_INVALID")
    assert merge(lse=region(5)) == code("QI_E_ALIAS")
    assert merge(o=fake_bshd(region(4), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    assert merge(of=region(6) + 16) == code("QI_E_ALIAS")


def test_carried_block_forward_validation():
    """Carried key-block forward: the state is given whole or not at all, it
    may be continued in place but overlap nothing else, O and LSE belong to
    the last block only, and a single text-only block is refused for a
    sample without text keys."""
    g = geom()  # T_img = 16
    L = qi.lib()
    q = fake_bshd(region(0), g.B, g.S, g.H)
    k = fake_bshd(region(1), g.B, g.S, g.H)
    v = fake_bshd(region(2), g.B, g.S, g.H)
    o = fake_bshd(region(3), g.B, g.S, g.H)
    no_o = qi.QiBshd(None, 0, 0, 0)
    ws = L.qi_joint_attn_fwd_workspace(g.ptr())
    st_in = (region(4), region(5), region(6))
    st_out = (region(7), region(8), region(10))

    def carry(blk=(1, 0, 16), sin=st_in, sout=st_out, o=no_o, lse=None, of=None, ws_ptr=region(9), ws_bytes=ws,
              gm=g):
        return L.qi_joint_attn_fwd_carry(gm.ptr(), q, k, v, qi.QiKeyBlock(*blk), *sin, *sout, o, lse, of, ws_ptr,
                                         ws_bytes, None)

    none3 = (None, None, None)
    assert carry() == code("QI_E_UNSUPPORTED")  # valid: stops at the device gate
    assert carry(sin=none3) == code("QI_E_UNSUPPORTED")  # the first block
    assert carry(sin=st_in, sout=st_in) == code("QI_E_UNSUPPORTED")  # continued in place
    assert carry(sout=none3, o=o, lse=region(11)) == code("QI_E_UNSUPPORTED")  # the last block
    assert carry(sin=none3, sout=none3, o=o, lse=region(11)) == code("QI_E_UNSUPPORTED")  # one block for all
    assert carry(blk=(0, 0, 0)) == code("QI_E_INVALID")  # empty
    assert carry(blk=(1, 8, 16)) == code("QI_E_INVALID")  # not tile-aligned
    assert carry(sin=(region(4), None, region(6))) == code("QI_E_INVALID")
    assert carry(sout=(region(7), region(8), None)) == code("QI_E_INVALID")
    assert carry(o=o) == code("QI_E_INVALID")  # O on a block that is not the last
    assert carry(lse=region(11)) == code("QI_E_INVALID")
    assert carry(sout=none3, o=o, lse=None) == code("QI_E_INVALID")  # the last block needs LSE
    assert carry(sout=(region(7), region(8), region(10) + 4)) == code("QI_E_ALIGN")  # two words per row
    assert carry(sin=(region(4) + 8, region(5), region(6))) == code("QI_E_ALIGN")
    assert carry(sin=(region(7) + 16, region(5), region(6))) == code("QI_E_ALIAS")  # overlaps acc_out, not equal
    assert carry(sout=(region(7), region(1), region(10))) == code("QI_E_ALIAS")  # m_out over k
    assert carry(sin=st_in, sout=(region(4), region(6), region(10))) == code("QI_E_ALIAS")  # m_out over l_in
    assert carry(sout=none3, o=o, lse=region(4)) == code("QI_E_ALIAS")  # lse over the input state
    assert carry(ws_ptr=None) == code("QI_E_WORKSPACE")
    assert carry(ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    g0 = geom(B=2, txt_len=[5, 0])
    last_alone = dict(sin=none3, sout=none3, o=fake_bshd(region(3), g0.B, g0.S, g0.H), lse=region(11), gm=g0,
                      ws_bytes=L.qi_joint_attn_fwd_workspace(g0.ptr()))
    assert carry(blk=(1, 0, 0), **last_alone) == code("QI_E_INVALID")  # sample 1 would have no key
    assert carry(blk=(1, 0, 16), **last_alone) == code("QI_E_UNSUPPORTED")


def test_projection_validation():
    """QKV and output projections: weights, streams, contiguity of a token's
    channels, outputs and workspace are checked before any launch."""
    g = geom()  # H = 2: D = 256
    L = qi.lib()
    D = 256
    x = fake_bshd(region(0), g.B, g.S, g.H)
    outs = [fake_bshd(region(3 + i), g.B, g.S, g.H) for i in range(3)]
    ws = L.qi_qkv_proj_workspace(g.ptr())
    assert ws == -(-(g.S * 64 * 2 * 4) // 256) * 256

    def qkv(x=x, w=region(1), bias=region(2), streams=2, gq=region(7), gk=region(8), fuse=1, outs=outs,
            ws_ptr=region(9), ws_bytes=ws):
        return L.qi_qkv_proj(g.ptr(), x, w, bias, streams, gq, gk, fuse, *outs, ws_ptr, ws_bytes, None)

    assert qkv() == code("QI_E_UNSUPPORTED")  # valid: stops at the device gate
    assert qkv(fuse=0, gq=None, gk=None, ws_ptr=None, ws_bytes=0) == code("QI_E_UNSUPPORTED")
    assert qkv(streams=3) == code("QI_E_INVALID")
    assert qkv(fuse=2) == code("QI_E_INVALID")
    assert qkv(w=None) == code("QI_E_INVALID")
    assert qkv(gq=None) == code("QI_E_INVALID")
    assert qkv(ws_ptr=None) == code("QI_E_WORKSPACE")
    assert qkv(ws_bytes=ws - 1) == code("QI_E_WORKSPACE")
    assert qkv(bias=region(2) + 4) == code("QI_E_ALIGN")
    # a token's channels must be contiguous (head stride 128)
    assert qkv(x=fake_bshd(region(0), g.B, g.S, g.H, sh=256, ss=512)) == code("QI_E_UNSUPPORTED")
    # outputs may not overlap the weights or each other
    assert qkv(outs=[fake_bshd(region(1), g.B, g.S, g.H)] + outs[1:]) == code("QI_E_ALIAS")
    assert qkv(outs=[outs[0], outs[0], outs[2]]) == code("QI_E_ALIAS")
    # the weight array spans streams * 3D * D BF16 values: an output right after its start overlaps
    assert qkv(outs=[fake_bshd(region(1) + 2 * 3 * D * D, g.B, g.S, g.H)] + outs[1:]) == code("QI_E_ALIAS")

    def out(o=x, w=region(1), bias=region(2), streams=1, y=outs[0]):
        return L.qi_attn_out_proj(g.ptr(), o, w, bias, streams, y, None)

    assert out() == code("QI_E_UNSUPPORTED")
    assert out(streams=0) == code("QI_E_INVALID")
    assert out(y=fake_bshd(region(0), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    assert out(bias=None) == code("QI_E_INVALID")


def test_qkv_prologue_and_pretiled_forward_validation():
    g = geom()
    L = qi.lib()
    vt_bytes = L.qi_joint_attn_fwd_workspace(g.ptr())
    qr, kr, v = (fake_bshd(region(i), g.B, g.S, g.H) for i in range(3))
    q, k = fake_bshd(region(3), g.B, g.S, g.H), fake_bshd(region(4), g.B, g.S, g.H)
    gq, gk, vt = region(5), region(6), region(7)

    def pro(**kw):
        a = dict(qr=qr, kr=kr, v=v, gq=gq, gk=gk, q=q, k=k, vt=vt, n=vt_bytes)
        a.update(kw)
        return L.qi_qkv_prologue(g.ptr(), a["qr"], a["kr"], a["v"], a["gq"], a["gk"], a["q"], a["k"], a["vt"],
                                 a["n"], None)

    assert pro() == code("QI_E_UNSUPPORTED")  # valid: stops at the device gate
    assert pro(vt=0) == code("QI_E_WORKSPACE")
    assert pro(n=vt_bytes - 1) == code("QI_E_WORKSPACE")
    assert pro(vt=vt + 16) == code("QI_E_ALIGN")
    assert pro(gk=None) == code("QI_E_INVALID")
    assert pro(k=q) == code("QI_E_ALIAS")                      # two outputs on one buffer
    assert pro(vt=region(2)) == code("QI_E_ALIAS")             # tiles over the V input
    assert pro(q=fake_bshd(region(0), g.B, g.S, g.H)) == code("QI_E_ALIAS")  # q' over q_raw

    o = fake_bshd(region(8), g.B, g.S, g.H)
    lse = region(9)

    def fwd(**kw):
        a = dict(q=q, k=k, vt=vt, n=vt_bytes, o=o, lse=lse, of=None)
        a.update(kw)
        return L.qi_joint_attn_fwd_vtiles(g.ptr(), a["q"], a["k"], a["vt"], a["n"], a["o"], a["lse"], a["of"], None)

    assert fwd() == code("QI_E_UNSUPPORTED")
    assert fwd(vt=0) == code("QI_E_WORKSPACE")
    assert fwd(n=vt_bytes - 1) == code("QI_E_WORKSPACE")
    assert fwd(vt=vt + 16) == code("QI_E_ALIGN")
    assert fwd(o=fake_bshd(vt, g.B, g.S, g.H)) == code("QI_E_ALIAS")  # output over the tiles
    assert fwd(vt=region(0)) != code("QI_E_ALIAS")                     # the tiles are read only
    assert fwd(lse=region(9) + 2) == code("QI_E_ALIGN")


def test_backward_head_limit_and_workspace_parts():
    """The backward's workspace holds at least D (FP32 per row) and the FP16
    copy of dO; a head count beyond the 65,535 its launches address is
    refused before the device gate."""
    L = qi.lib()
    g = geom()
    ws = L.qi_joint_attn_bwd_workspace(g.ptr())
    assert ws >= g.B * g.H * g.S * 4 + g.B * g.S * g.H * 128 * 2
    g = geom(H=65536)
    ws = L.qi_joint_attn_bwd_workspace(g.ptr())
    views = [fake_bshd(region(i), g.B, g.S, g.H) for i in range(6)]
    grads = [fake_bshd(region(10 + i), g.B, g.S, g.H) for i in range(3)]
    rc = L.qi_joint_attn_bwd(g.ptr(), *views, region(6), fake_bshd(region(7), g.B, g.S, g.H), region(8), region(9),
                             *grads, region(14), region(15), None, None, region(20), ws, None)
    assert rc == code("QI_E_UNSUPPORTED") and "65535" in qi.last_error(), qi.last_error()


def test_clock_probe_validation():
    L = qi.lib()
    assert L.qi_clock_probe(None, 4, 8, None) == code("QI_E_INVALID")
    assert L.qi_clock_probe(region(0) + 4, 4, 8, None) == code("QI_E_ALIGN")
    assert L.qi_clock_probe(region(0), 0, 8, None) == code("QI_E_INVALID")
    assert L.qi_clock_probe(region(0), 4, 0, None) == code("QI_E_INVALID")
    assert L.qi_clock_probe(region(0), 4, 8, None) == code("QI_E_UNSUPPORTED")  # no device here


def test_fast_math_probe_library_is_built_beside_the_library():
    """build() also writes the probe alone compiled with -ffast-math; the GPU
    tests expect its verdict to be the strict failure."""
    path = os.path.join(os.path.dirname(qi.LIB_PATH), "libqi_probe_fastmath.so")
    assert os.path.exists(path)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert re.search(r"\bT qi_probe_standalone\b", out)


def test_noalloc_forward_validation():
    """The no-allocation forward validates like qi_joint_attn_fwd, and a
    geometry whose V tiles exceed its 64 MiB static scratch is refused
    before the device gate."""
    L = qi.lib()

    def call(g, o=None):
        views = [fake_bshd(region(i), g.B, g.S, g.H) for i in range(3)]
        o = o or fake_bshd(region(3), g.B, g.S, g.H)
        return L.qi_joint_attn_fwd_noalloc(g.ptr(), *views, o, region(4), None, None)

    g = geom()
    assert call(g) == code("QI_E_UNSUPPORTED")  # valid: only the device gate is left
    assert call(g, o=fake_bshd(region(0), g.B, g.S, g.H)) == code("QI_E_ALIAS")
    big = qi.Geometry(B=4, H=24, T_txt=512, grid_h=104, grid_w=58, txt_len=[7, 64, 200, 511])
    assert call(big) == code("QI_E_WORKSPACE")
    assert "static scratch" in qi.last_error()
    ok = qi.Geometry(B=1, H=24, T_txt=256, grid_h=64, grid_w=64, txt_len=[219])
    assert call(ok) == code("QI_E_UNSUPPORTED")
