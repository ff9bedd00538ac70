"""Seeded synthetic workloads for the strict joint-attention path.

This module holds the workload shapes and the seeded input generators shared
by the GPU tests, the oracle tests and the benchmark.  It performs none of the
method's arithmetic: it only draws random tensors and describes geometry.

Shapes follow the pages' reference resolutions (the "Model contract" table of
the Qwen-Image roadmap RFC, row "Reference shapes": 1024x1024, 1328x1328 and
1664x928 pixels, i.e. 64x64, 83x83 and 104x58 image tokens after the 16x
reduction of the latent packing) with 24 heads of 128 channels.  The pages use
checkpoint activations; none are available, so Q, K, V and dO are standard
normal BF16 draws and the RMSNorm gains are FP32 draws around 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T_txt: int
    txt_len: tuple
    h: int
    w: int
    seed: int
    backward: bool = False
    note: str = ""

    @property
    def T_img(self) -> int:
        return self.h * self.w

    @property
    def S(self) -> int:
        return self.T_txt + self.h * self.w

    def valid_keys(self) -> list:
        return [L + self.T_img for L in self.txt_len]

    def fwd_flops(self) -> float:
        """Algorithmic forward FLOPs: 2 GEMMs of 2*S*K*D per (b, h)."""
        return float(sum(4 * HEAD_DIM * self.H * self.S * K for K in self.valid_keys()))

    def bwd_flops(self) -> float:
        """Algorithmic backward FLOPs: 5 GEMMs of 2*S*K*D per (b, h)."""
        return float(sum(10 * HEAD_DIM * self.H * self.S * K for K in self.valid_keys()))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 8, (5,), 4, 4, 0, note="B=1, 2x128, T_txt=8 (5 valid), 4x4 grid"),
    "1024sq": Workload("1024sq", 1, 24, 256, (219,), 64, 64, 1, note="1024^2 image, single sample"),
    "1328sq_cfg": Workload("1328sq_cfg", 2, 24, 512, (301, 12), 83, 83, 2, note="1328^2 CFG pair"),
    "1664x928": Workload("1664x928", 4, 24, 512, (7, 64, 200, 511), 104, 58, 3,
                         note="1664x928 batch-invariance sweep"),
    "1024sq_bwd": Workload("1024sq_bwd", 1, 24, 256, (219,), 64, 64, 4, backward=True,
                           note="deterministic backward at 1024^2"),
}


def make_inputs(wl: Workload, extra_samples: int = 0, gain_mean: float = 1.0, gain_std: float = 0.1,
                gain_streams: int = 1) -> dict:
    """Draw the workload's inputs on the CPU from its seed.

    Draw order: Q, K, V as N(0,1) rounded to BF16, then g_q and g_k as
    gain_mean + gain_std * N(0,1) in FP32, then dO (backward workloads).
    ``extra_samples`` appends further batch rows drawn next from the same
    generator (same shapes, text length of the last row)."""
    g = torch.Generator("cpu").manual_seed(wl.seed)
    B, S, H = wl.B, wl.S, wl.H

    def bf16(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)

    q, k, v = bf16(B, S, H, HEAD_DIM), bf16(B, S, H, HEAD_DIM), bf16(B, S, H, HEAD_DIM)
    gq = gain_mean + gain_std * torch.randn(gain_streams, HEAD_DIM, generator=g, dtype=torch.float32)
    gk = gain_mean + gain_std * torch.randn(gain_streams, HEAD_DIM, generator=g, dtype=torch.float32)
    dO = bf16(B, S, H, HEAD_DIM) if wl.backward else None
    txt_len = list(wl.txt_len)
    if extra_samples:
        qs, ks, vs, ds = [q], [k], [v], [dO]
        for _ in range(extra_samples):
            qs.append(bf16(1, S, H, HEAD_DIM))
            ks.append(bf16(1, S, H, HEAD_DIM))
            vs.append(bf16(1, S, H, HEAD_DIM))
            if wl.backward:
                ds.append(bf16(1, S, H, HEAD_DIM))
            txt_len.append(txt_len[-1])
        q, k, v = torch.cat(qs), torch.cat(ks), torch.cat(vs)
        dO = torch.cat(ds) if wl.backward else None
    return dict(q=q, k=k, v=v, g_q=gq, g_k=gk, dO=dO, txt_len=txt_len, T_txt=wl.T_txt, h=wl.h, w=wl.w)


def custom(name: str, B: int, H: int, T_txt: int, txt_len, h: int, w: int, seed: int,
           backward: bool = False) -> Workload:
    """A workload with explicit geometry (tests of ragged and edge shapes)."""
    return Workload(name, B, H, T_txt, tuple(txt_len), h, w, seed, backward)


def bits(t: torch.Tensor):
    """BF16 tensor -> numpy uint16 bit patterns (a view, no arithmetic)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def score_operands(B: int, H: int, S: int, key_slots: int, seed: int) -> torch.Tensor:
    """Raw FP32 scores [B, H, S, key_slots] for exercising the softmax operator
    on its own: row i of tile t is sigma_i * N(0,1) + drift_i * t, with
    sigma_i uniform in [4, 40) and drift_i uniform in [-80, 80) (raw units,
    before the 1/sqrt(128) scale), so rows both keep and move their running
    maximum from tile to tile."""
    g = torch.Generator("cpu").manual_seed(seed)
    sig = 4 + 36 * torch.rand(B, H, S, 1, generator=g)
    drift = -80 + 160 * torch.rand(B, H, S, 1, generator=g)
    tile = (torch.arange(key_slots) // 64).to(torch.float32)
    return sig * torch.randn(B, H, S, key_slots, generator=g) + drift * tile


def av_operands(B: int, H: int, S: int, key_slots: int, seed: int) -> dict:
    """Operands of the A.V operator on its own: P FP16 uniform in [0, 2)
    [B, H, S, key_slots], alpha FP32 uniform in [1/4, 1] [B, H, key_slots/64, S]
    (tile-major), l FP32 uniform in [1, 64) [B, H, S]."""
    g = torch.Generator("cpu").manual_seed(seed)
    p = (2 * torch.rand(B, H, S, key_slots, generator=g)).to(torch.float16)
    alpha = 0.25 + 0.75 * torch.rand(B, H, key_slots // 64, S, generator=g)
    l = 1 + 63 * torch.rand(B, H, S, generator=g)
    return dict(p=p, alpha=alpha, l=l)


def proj_inputs(wl: Workload, streams: int = 2, seed_offset: int = 1000) -> dict:
    """Inputs of the projections around the attention (the model's packed QKV
    projection and output projection, D = H*128 channels), drawn on the CPU:
    hidden states x ~ N(0,1) and attention output o ~ N(0,1) in BF16
    [B, S, D]; per-stream weights W_qkv [streams, 3D, D] and W_o [streams, D,
    D] ~ N(0, 1/D) in BF16 (outputs of unit scale), biases b_qkv [streams, 3D]
    and b_o [streams, D] ~ N(0, 0.02^2) in FP32; RMSNorm gains g_q, g_k
    [streams, 128] ~ 1 + 0.1 N(0,1).  Draw order as listed."""
    g = torch.Generator("cpu").manual_seed(wl.seed + seed_offset)
    B, S, D = wl.B, wl.S, wl.H * HEAD_DIM

    def bf16(*shape, std=1.0):
        return (std * torch.randn(*shape, generator=g, dtype=torch.float32)).to(torch.bfloat16)

    x = bf16(B, S, D)
    o = bf16(B, S, D)
    w_qkv = bf16(streams, 3 * D, D, std=D ** -0.5)
    w_o = bf16(streams, D, D, std=D ** -0.5)
    b_qkv = 0.02 * torch.randn(streams, 3 * D, generator=g, dtype=torch.float32)
    b_o = 0.02 * torch.randn(streams, D, generator=g, dtype=torch.float32)
    gq = 1.0 + 0.1 * torch.randn(streams, HEAD_DIM, generator=g, dtype=torch.float32)
    gk = 1.0 + 0.1 * torch.randn(streams, HEAD_DIM, generator=g, dtype=torch.float32)
    return dict(x=x, o=o, w_qkv=w_qkv, w_o=w_o, b_qkv=b_qkv, b_o=b_o, g_q=gq, g_k=gk)


def staircase_scores(rows: int, tiles: int, seed: int, jump_lo: float = 63.0, jump_hi: float = 1263.0) -> torch.Tensor:
    """Raw FP32 scores [1, 1, rows, 64 * tiles] whose tile maxima climb: every
    key of tile 0 is 0 and every key of tile t > 0 equals the previous tile's
    value plus a jump drawn uniformly from [jump_lo, jump_hi) (raw units), so
    every tile moves the running maximum of its row by one drawn jump."""
    g = torch.Generator("cpu").manual_seed(seed)
    jumps = jump_lo + (jump_hi - jump_lo) * torch.rand(rows, tiles, generator=g, dtype=torch.float64)
    jumps[:, 0] = 0.0
    level = torch.cumsum(jumps, dim=1).to(torch.float32)  # [rows, tiles]
    return level.repeat_interleave(64, dim=1).reshape(1, 1, rows, 64 * tiles).contiguous()
