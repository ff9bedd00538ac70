"""Benchmark of the strict joint-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1024sq]

A step is one pass of the path over one batch of synthetic input that is
already resident in HBM: the Q and K prologues (RMSNorm + gain + RoPE), the
conversion of V to the attention's FP16 key tiles, and the attention
forward; for a backward workload the step also runs the backward (attention
+ prologue gradients).  Prints ONE JSON line.

By default a step is two library calls: qi_qkv_prologue (Q and K prologues
and the V conversion in one launch) and qi_joint_attn_fwd_vtiles (the
attention kernel alone); --separate-prologue runs qi_qknorm_rope twice and
qi_joint_attn_fwd (V conversion + attention) instead.  Both give the same
bytes.

By default every call is launched from the host each step; --graph captures
each part of a step (prologues, forward call, backward call) once as a HIP
graph and replays it (same kernels, arguments and buffers).  The default
warmup is long on purpose: the GPU clock under MFMA load settles only after
a few hundred calls, and a short warmup measures the ramp.

value = algorithmic forward FLOPs per step / wall time per step (TFLOP/s),
with the algorithmic count 4 * D * H * sum_b S * K_b (K_b = valid keys).  For
a backward workload `fwd_bwd_step` adds the backward's 10 * D * H * sum_b S * K_b
to the count over the same step time.
The K timed steps run back to back between one pair of HIP events and the
host clock (no event inside the region).  The attention-forward call is then
timed alone on the launch stream: max(K, 100) back-to-back calls between one
event pair, five repeats (by default one launch of the attention kernel; with
--separate-prologue the V tile pass and the attention kernel); that time
gives the roofline fraction against the MI355X dense BF16 MFMA peak
(2.5 PFLOP/s).  The other measurements of the line (the 1024^2 backward, the
key-block forward, the projections, the unfused operators) run before the
headline loop.  The shader clock is sampled with the library's clock probe
just before and just after the timed steps.  The CPU oracle is timed on a
bounded sample of the same workload on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~0.1 s of untimed load first (the clock under MFMA load settles
    # over the first few hundred calls), then ~0.1 s timed
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="1024sq")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--separate-prologue", action="store_true",
                    help="run the step as qi_qknorm_rope twice + qi_joint_attn_fwd (V converted inside the forward "
                         "call) instead of qi_qkv_prologue + qi_joint_attn_fwd_vtiles")
    ap.add_argument("--graph", action="store_true",
                    help="replay each part of a step from a captured HIP graph instead of launching every call")
    ap.add_argument("--proj-steps", type=int, default=50,
                    help="also time the QKV and output projections this many times (0: skip)")
    ap.add_argument("--block-steps", type=int, default=20,
                    help="also time the key-block forward (image keys in blocks of 512) and the merge (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=100,
                    help="also time the backward of the 1024^2 backward workload this many times (0: skip)")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="also time the attention call this many times with the caches flushed first (0: skip)")
    ap.add_argument("--unfused-steps", type=int, default=10,
                    help="also time the unfused forward (scores -> softmax -> A.V) this many times (0: skip)")
    return ap.parse_args()


def source_hash(name: str) -> str:
    p = os.path.join(ROOT, "invariant_joint_attention_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profile(kernel: str, src: str, workload: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_hash(src):
        return None
    return float(m_b.group(1))


def host_env(torch):
    """The machine the numbers come from (GPU, software, host CPU)."""
    props = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count, "hbm_gib": round(props.total_memory / 2**30, 1),
            "rocm_hip": torch.version.hip, "torch": torch.__version__, "host_cpu": cpu,
            "host_threads": os.cpu_count()}


def sha256_of(*tensors) -> str:
    """SHA-256 over the raw bytes of the tensors, in order."""
    import torch

    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().cpu().view(-1).view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


class ClockProbe:
    """Shader clock under a matrix load, sampled by the library's clock probe:
    one wave per SIMD runs MFMAs for ~30 us and times them against the
    constant-rate wall clock (both counters read by the same wave)."""

    def __init__(self, qi, torch, groups=1024, iters=512, samples=2):
        self.qi, self.iters = qi, iters
        self.bufs = [torch.zeros((groups, 3), dtype=torch.int64, device="cuda:0") for _ in range(samples)]
        self.khz = qi.wall_clock_khz(0)

    def sample(self, i):
        self.qi.clock_probe(self.bufs[i], self.iters)

    def mhz(self, i):
        a = self.bufs[i].cpu().numpy().astype("float64")
        ticks, wall = a[:, 0], a[:, 1]
        ok = wall > 0
        if not ok.any():
            return None
        per = ticks[ok] / wall[ok] * self.khz / 1e3
        return {"mean_mhz": round(float(ticks[ok].sum() / wall[ok].sum() * self.khz / 1e3), 1),
                "min_mhz": round(float(per.min()), 1), "max_mhz": round(float(per.max()), 1),
                "waves": int(ok.sum())}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path shards over (batch, head) with no exchange, "
              "and the benchmark measures one GPU's share; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import invariant_joint_attention_amd as qi
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = workloads.make_inputs(wl)
    in_sha = sha256_of(*(inp[n] for n in ("q", "k", "v", "g_q", "g_k") + (("dO",) if wl.backward else ())))
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    qi.strict_probe(0)
    env = host_env(torch)

    # preallocated outputs: the timed region launches kernels only
    shp = g["q"].shape
    qp = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    kp = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    o = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.B, wl.H, wl.S), dtype=torch.float32, device=dev)
    of = torch.empty(shp, dtype=torch.float32, device=dev) if wl.backward else None
    fws = torch.empty(qi.fwd_workspace_bytes(geo), dtype=torch.uint8, device=dev)
    if wl.backward:
        ws = torch.empty(qi.bwd_workspace_bytes(geo), dtype=torch.uint8, device=dev)
        grads = {n: torch.empty(shp, dtype=torch.float32, device=dev) for n in ("dq", "dk", "dv")}

    # the parts of a step, each a fixed sequence of library calls
    if args.separate_prologue:
        def pro():
            qi.qknorm_rope(g["q"], g["g_q"], geo, out=qp)
            qi.qknorm_rope(g["k"], g["g_k"], geo, out=kp)

        def fwd():
            qi.joint_attn_fwd(qp, kp, g["v"], geo, out=o, lse=lse, out_f32=of, workspace=fws)
    else:
        # one launch for the Q/K prologues and the V tile conversion, then the attention kernel alone
        def pro():
            qi.qkv_prologue(g["q"], g["k"], g["v"], g["g_q"], g["g_k"], geo, q=qp, k=kp, v_tiles=fws)

        def fwd():
            qi.joint_attn_fwd_vtiles(qp, kp, fws, geo, out=o, lse=lse, out_f32=of)

    def bwd():
        qi.joint_attn_bwd(g["q"], g["k"], qp, kp, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo,
                          workspace=ws, **grads)

    names = ["pro", "fwd"] + (["bwd"] if wl.backward else [])
    parts = [pro, fwd] + ([bwd] if wl.backward else [])
    for p in parts:  # eager once (device gate, first-launch costs)
        p()
    torch.cuda.synchronize()

    out = {}
    # ---- the other measurements of the line come first: each is real work
    # of the path (not the headline step), and together they run the GPU
    # long enough for its clock under matrix load to settle before the
    # headline loop starts
    aux = {}
    # the backward's inputs first; its timed loop runs last, right before the
    # headline warmup, so the timed steps follow ~0.1 s of continuous load
    bwd_case = prepare_bwd(qi, torch, workloads) if args.bwd_steps > 0 and not wl.backward else None
    if args.block_steps > 0:
        aux["blocks"] = bench_blocks(qi, torch, np, wl, geo, qp, kp, g["v"], args.block_steps)
    if args.proj_steps > 0:
        aux["projections"] = bench_proj(qi, torch, np, workloads, wl, args.proj_steps)
    if args.unfused_steps > 0:
        aux["unfused_fwd"] = bench_unfused(qi, torch, np, wl, geo, qp, kp, g["v"], args.unfused_steps)
    bwd_report = bench_bwd(torch, np, bwd_case, args.bwd_steps) if bwd_case is not None else None

    if not args.graph:
        runs = parts
    else:
        # Each part captured once as a HIP graph and replayed: the launches
        # of a step reach the GPU without per-call host overhead, so no part
        # waits for the host between kernels (the kernels, their arguments
        # and buffers are the eager ones; the library allocates nothing).
        graphs = []
        for p in parts:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                p()
            graphs.append(gr)
        runs = [gr.replay for gr in graphs]
    # The timed steps carry no events of their own: an event record between
    # two kernels costs the stream several microseconds and has slowed the
    # kernel after it, so the K steps run back to back between one event pair.
    clock = ClockProbe(qi, torch)

    def step():
        for r in runs:
            r()

    def region(fn, n):
        """GPU time per call of `fn` over n back-to-back calls (one event pair)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(args.warmup):
        step()
    clock.sample(0)
    torch.cuda.synchronize()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record()
    for _ in range(args.steps):
        step()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step_ms = e_start.elapsed_time(e_end) / args.steps
    clock.sample(1)
    ms_step = wall * 1e3 / args.steps

    # The dominant kernel alone, right after the timed steps: the attention
    # call launched back to back K times between one event pair, five such
    # repeats (mean of the repeats for the roofline; median and min beside
    # it); the prologue (and backward) the same way.
    j_fwd = names.index("fwd")
    n_alone = max(args.steps, 100)  # at least 100 back-to-back calls per repeat, whatever K is
    fwd_rep = [region(runs[j_fwd], n_alone) for _ in range(5)]
    fwd_ms = float(np.mean(fwd_rep))
    fwd_t = fwd_rep
    pro_ms = region(runs[names.index("pro")], n_alone)
    bwd_ms = region(runs[names.index("bwd")], max(1, args.steps // 4)) if wl.backward else 0.0
    torch.cuda.synchronize()
    clock_before, clock_after = clock.mhz(0), clock.mhz(1)
    out_sha = sha256_of(o, lse)
    if bwd_report is not None:
        aux["attn_bwd"] = bwd_report()
        aux["attn_bwd"]["sha256_outputs"] = sha256_of(*bwd_case["outputs"])
    fwd_flops = wl.fwd_flops()
    value = fwd_flops / (ms_step * 1e-3) / 1e12
    attn_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    pro_bytes = 2 * 2 * 2 * wl.B * wl.S * wl.H * 128  # Q and K, read + write BF16
    if not args.separate_prologue:
        # + the valid V rows read and the FP16 key tiles written (64 keys x 128 channels x 2 B each)
        for L in wl.txt_len:
            pro_bytes += (L + wl.T_img) * wl.H * 128 * 2 + (-(-L // 64) + -(-wl.T_img // 64)) * wl.H * 64 * 128 * 2

    if args.separate_prologue:
        # one forward call = v_tiles_kernel (V to FP16 key tiles) + attn_fwd_kernel, timed together
        traffic = traffic_from_profile("attn_fwd_call", "qi_attn_fwd.hip", args.workload)
        kernel = "attn_fwd_kernel (+ v_tiles_kernel: one forward call)"
    else:
        traffic = traffic_from_profile("attn_fwd_kernel", "qi_attn_fwd.hip", args.workload)
        kernel = "attn_fwd_kernel (one qi_joint_attn_fwd_vtiles call)"
    roofline = {"bound": "mfma", "kernel": kernel,
                "achieved": round(attn_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "flops_per_launch": fwd_flops, "avg_launch_ms": round(fwd_ms, 4)}

    # the attention call again with the caches flushed before each launch
    # (inputs read from HBM, not from the 256 MB last-level cache)
    flushed = None
    if args.flush_steps > 0:
        junk = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev)
        fe = []
        for _ in range(args.flush_steps):
            junk.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fwd()
            e1.record()
            fe.append((e0, e1))
        torch.cuda.synchronize()
        ft = [a.elapsed_time(b) for a, b in fe]
        flushed = {"steps": args.flush_steps, "median_ms": round(float(np.median(ft)), 4),
                   "min_ms": round(float(np.min(ft)), 4),
                   "tflops_median": round(fwd_flops / (float(np.median(ft)) * 1e-3) / 1e12, 1)}
        del junk

    out.update({
        "metric": "joint-attn fwd TFLOP/s and % BF16 MFMA peak at 1024^2 (S=4096+256), 24x128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp16",
        "dtype_detail": "QK^T on BF16 MFMA (v_mfma_f32_32x32x16_bf16); P.V on FP16 MFMA "
                        "(v_mfma_f32_32x32x16_f16, FP16 P and FP16 V*2^-8); FP32 accumulation; "
                        "prologue FP32 with one BF16 output cast",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.note}", "B": wl.B, "heads": wl.H, "head_dim": 128,
                   "T_txt": wl.T_txt, "txt_len": list(wl.txt_len), "grid": [wl.h, wl.w], "S": wl.S,
                   "backward": wl.backward},
        "env": env,
        "sha256": {"inputs": in_sha, "outputs_o_lse": out_sha},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "attn_fwd": {"timed": f"5 repeats of {n_alone} back-to-back calls, one event pair each, after the "
                              "timed steps",
                     "ms": round(fwd_ms, 4), "median_ms": round(float(np.median(fwd_t)), 4),
                     "min_ms": round(float(np.min(fwd_t)), 4), "max_ms": round(float(np.max(fwd_t)), 4),
                     "tflops": round(attn_tflops, 2),
                     "pct_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
                     "pct_peak_median": round(100 * fwd_flops / (float(np.median(fwd_t)) * 1e-3) / 1e12
                                              / PEAK_BF16_TFLOPS, 2),
                     "cache_flushed": flushed},
        "step_gpu_ms": round(gpu_step_ms, 4),
        "shader_clock": {"before_timed_steps": clock_before, "after_timed_steps": clock_after,
                         "how": "per wave: s_memtime ticks / s_memrealtime ticks x wall-clock rate, one wave "
                                "per SIMD running BF16 MFMAs for ~30 us, sampled just before and just after "
                                "the timed steps"},
        "prologue": {"calls": "qi_qknorm_rope x 2" if args.separate_prologue else "qi_qkv_prologue (Q, K, V tiles)",
                     "timed": f"{n_alone} back-to-back calls after the timed steps", "ms": round(pro_ms, 4), "bytes": pro_bytes, "gbps": round(pro_bytes / (pro_ms * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(pro_bytes / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        "roofline": roofline,
        "launch": "hip_graph_replay" if args.graph else "eager",
    })
    if wl.backward:
        bflops = wl.bwd_flops()
        out["attn_bwd"] = {"ms": round(bwd_ms, 4), "tflops": round(bflops / (bwd_ms * 1e-3) / 1e12, 2),
                           "algorithmic_flops": bflops}
        # the whole step (prologues, forward, backward) against forward + backward FLOPs
        out["fwd_bwd_step"] = {"ms": round(ms_step, 4), "flops": fwd_flops + bflops,
                               "tflops": round((fwd_flops + bflops) / (ms_step * 1e-3) / 1e12, 2)}
    for k_, v_ in aux.items():
        if isinstance(v_, dict) and "ms" in v_ and k_ in ("blocks", "unfused_fwd"):
            v_["vs_fused"] = round(v_["ms"] / fwd_ms, 3)
            if "carried" in v_:
                v_["carried"]["vs_fused"] = round(v_["carried"]["ms"] / fwd_ms, 3)
        out[k_] = v_
    out["order"] = ("the other measurements (" + ", ".join(aux) + ") ran before the headline loop, the "
                    "backward last, so that the warmup and the timed steps follow continuous load; then "
                    "the attention call alone and the prologue alone") if aux else "warmup, then the timed steps"

    # ---------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, qp, kp, o, lse, args.cpu_seconds)

    print(json.dumps(out), flush=True)


def prepare_bwd(qi, torch, workloads):
    """Inputs, forward state and buffers of the 1024^2 backward workload
    (same shapes as the forward workload, its own seed, plus dO): the
    prologues and the forward (keeping the FP32 O) run once here."""
    dev = "cuda:0"
    wl = workloads.WORKLOADS["1024sq_bwd"]
    inp = workloads.make_inputs(wl)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len))
    q = qi.qknorm_rope(g["q"], g["g_q"], geo)
    k = qi.qknorm_rope(g["k"], g["g_k"], geo)
    of = torch.empty(q.shape, dtype=torch.float32, device=dev)
    o, lse = qi.joint_attn_fwd(q, k, g["v"], geo, out_f32=of)
    ws = torch.empty(qi.bwd_workspace_bytes(geo), dtype=torch.uint8, device=dev)
    grads = {n: torch.empty(q.shape, dtype=torch.float32, device=dev) for n in ("dq", "dk", "dv")}
    dg = {n: torch.empty(shape, dtype=torch.float32, device=dev)
          for n, shape in (("dgain_q_ps", (wl.B, 1, 128)), ("dgain_k_ps", (wl.B, 1, 128)),
                           ("dgain_q", (1, 128)), ("dgain_k", (1, 128)))}

    def run():
        qi.joint_attn_bwd(g["q"], g["k"], q, k, g["v"], of, lse, g["dO"], g["g_q"], g["g_k"], geo, workspace=ws,
                          **grads, **dg)

    run()
    torch.cuda.synchronize()
    return {"wl": wl, "run": run, "outputs": [grads["dq"], grads["dk"], grads["dv"], dg["dgain_q_ps"],
                                             dg["dgain_k_ps"]]}


def bench_bwd(torch, np, case, steps):
    """The deterministic backward (qi_joint_attn_bwd) of the prepared 1024^2
    backward workload, `steps` calls each bracketed by HIP events on the
    launch stream.  Returns a function that reads the events out later (each
    read synchronises, so it waits until the headline loop is done) and
    reports against the dense BF16 MFMA peak on the algorithmic count
    10 * D * H * S * K."""
    wl, run = case["wl"], case["run"]
    ev = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        ev.append((e0, e1))

    def report():
        t = [a.elapsed_time(b) for a, b in ev]
        flops = wl.bwd_flops()
        ms = float(np.mean(t))
        return {"workload": f"{wl.name}: {wl.note}", "steps": steps, "calls": "qi_joint_attn_bwd",
                "ms": round(ms, 4), "median_ms": round(float(np.median(t)), 4), "min_ms": round(float(np.min(t)), 4),
                "algorithmic_flops": flops, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma"}

    return report


def bench_blocks(qi, torch, np, wl, geo, q, k, v, steps, block=512):
    """The key-block forward as a sequence-parallel split would run it: the
    image keys in blocks of `block` keys (the text keys in block 0), one
    partial call per block, then the fixed-order merge; each timed with HIP
    events on the launch stream.  The partial calls together perform the
    whole forward's algorithmic FLOPs; the merge is HBM-bound (it reads n row
    states of 520 bytes and writes O).  The carried form runs the same blocks
    as one chain (the state continued in place, the last block writing O
    and LSE), the ring in which the state travels with the query rows."""
    dev = q.device
    B, H, S, T_img = wl.B, wl.H, wl.S, wl.T_img
    edges = list(range(0, T_img, block)) + [T_img]
    blocks = [(i == 0, edges[i], edges[i + 1]) for i in range(len(edges) - 1)]
    n = len(blocks)
    acc = torch.empty((n, B, H, S, 128), dtype=torch.float32, device=dev)
    m = torch.empty((n, B, H, S), dtype=torch.float32, device=dev)
    l = torch.empty((n, B, H, S), dtype=torch.float32, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ws = torch.empty(qi.fwd_workspace_bytes(geo), dtype=torch.uint8, device=dev)
    ev = {"partials": [], "merge": [], "carried": []}
    st = (torch.empty((B, H, S, 128), dtype=torch.float32, device=dev),
          torch.empty((B, H, S), dtype=torch.float32, device=dev),
          torch.empty((B, H, S, 2), dtype=torch.float32, device=dev))
    o_c = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse_c = torch.empty((B, H, S), dtype=torch.float32, device=dev)

    def chain(timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if timed else None
        if timed:
            e[0].record()
        for i, (wt, lo, hi) in enumerate(blocks):
            if i + 1 < n:
                qi.joint_attn_fwd_carry(q, k, v, geo, wt, lo, hi, state=st if i else None, state_out=st,
                                        workspace=ws)
            else:
                qi.joint_attn_fwd_carry(q, k, v, geo, wt, lo, hi, state=st if i else None, last=True, out=o_c,
                                        lse=lse_c, workspace=ws)
        if timed:
            e[1].record()
            ev["carried"].append((e[0], e[1]))

    def run(timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record()
        for i, (wt, lo, hi) in enumerate(blocks):
            qi.joint_attn_fwd_partial(q, k, v, geo, wt, lo, hi, acc=acc[i], m=m[i], l=l[i], workspace=ws)
        if timed:
            e[1].record()
        qi.joint_attn_merge(acc, m, l, geo, out=o, lse=lse)
        if timed:
            e[2].record()
            ev["partials"].append((e[0], e[1]))
            ev["merge"].append((e[1], e[2]))

    for _ in range(steps):
        run(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        run(True)
    torch.cuda.synchronize()
    for _ in range(steps):
        chain(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        chain(True)
    torch.cuda.synchronize()
    p_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["partials"]]))
    m_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["merge"]]))
    c_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["carried"]]))
    flops = wl.fwd_flops()
    rows = B * H * S
    m_bytes = n * rows * (128 * 4 + 8) + rows * 128 * 2 + rows * 4
    return {"steps": steps, "block_keys": block, "n_blocks": n,
            "partials": {"ms": round(p_ms, 4), "tflops": round(flops / (p_ms * 1e-3) / 1e12, 1),
                         "frac": round(flops / (p_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma"},
            "merge": {"ms": round(m_ms, 4), "bytes": m_bytes, "gbps": round(m_bytes / (m_ms * 1e-3) / 1e9, 1),
                      "frac": round(m_bytes / (m_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4), "bound": "hbm"},
            "ms": round(p_ms + m_ms, 4),
            "carried": {"ms": round(c_ms, 4), "tflops": round(flops / (c_ms * 1e-3) / 1e12, 1),
                        "frac": round(flops / (c_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma",
                        "state_bytes_per_block": B * H * S * (128 + 3) * 4}}


def bench_proj(qi, torch, np, workloads, wl, steps):
    """The projections around the attention on the same shape (synthetic
    per-stream weights): the packed QKV projection with the fused Q/K
    prologue and the output projection, each timed with HIP events on the
    launch stream against the dense BF16 MFMA peak (2 * tokens * N * D
    FLOPs)."""
    dev = "cuda:0"
    geo = qi.Geometry(B=wl.B, H=wl.H, T_txt=wl.T_txt, grid_h=wl.h, grid_w=wl.w, txt_len=list(wl.txt_len),
                      gain_streams=2)
    p = {k: v.to(dev) for k, v in workloads.proj_inputs(wl, streams=2).items()}
    D = wl.H * 128
    x = p["x"].view(wl.B, wl.S, wl.H, 128)
    o = p["o"].view(wl.B, wl.S, wl.H, 128)
    q, k, v, y = (torch.empty_like(x) for _ in range(4))
    ws = torch.empty(int(qi.lib().qi_qkv_proj_workspace(geo.ptr())), dtype=torch.uint8, device=dev)
    tokens = wl.B * wl.S
    flops = {"qkv_proj": 2.0 * tokens * 3 * D * D, "out_proj": 2.0 * tokens * D * D}
    ev = {n: [] for n in flops}

    def run(timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record()
        qi.qkv_proj(x, p["w_qkv"], p["b_qkv"], geo, gain_q=p["g_q"], gain_k=p["g_k"], q=q, k=k, v=v, workspace=ws)
        if timed:
            e[1].record()
        qi.attn_out_proj(o, p["w_o"], p["b_o"], geo, y=y)
        if timed:
            e[2].record()
            ev["qkv_proj"].append((e[0], e[1]))
            ev["out_proj"].append((e[1], e[2]))

    for _ in range(steps):
        run(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        run(True)
    torch.cuda.synchronize()
    res = {"steps": steps, "bound": "mfma", "peak_tflops": PEAK_BF16_TFLOPS, "weight_streams": 2,
           "d_model": D, "tokens": tokens}
    for n, f in flops.items():
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
        tf = f / (ms * 1e-3) / 1e12
        res[n] = {"ms": round(ms, 4), "flops": f, "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return res


def bench_unfused(qi, torch, np, wl, geo, q, k, v, steps):
    """The three unfused operators on the same inputs, each timed with HIP
    events on the launch stream, against the HBM roofline of the arrays each
    one reads and writes (scores FP32 and P FP16 over all key slots, the tile
    factors, V through its FP16 tile pass, O)."""
    dev = q.device
    B, H, S = wl.B, wl.H, wl.S
    Kp = qi.key_slots(geo)
    nt = Kp // 64
    s = torch.empty((B, H, S, Kp), dtype=torch.float32, device=dev)
    p = torch.empty((B, H, S, Kp), dtype=torch.float16, device=dev)
    alpha = torch.empty((B, H, nt, S), dtype=torch.float32, device=dev)
    l = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qi.fwd_workspace_bytes(geo), dtype=torch.uint8, device=dev)
    act = 2 * B * S * H * 128  # one BF16 [B,S,H,128] tensor
    rows = B * H * S
    nbytes = {
        "qk_gemm": 2 * act + 4 * rows * Kp,
        "softmax": 4 * rows * Kp + 2 * rows * Kp + 4 * rows * nt + 8 * rows,
        "av_gemm": 2 * rows * Kp + 4 * rows * nt + 4 * rows + act + 2 * 2 * B * H * nt * 64 * 128 + act,
    }
    ev = {n: [] for n in nbytes}

    def run(timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if timed:
            e[0].record()
        qi.joint_attn_qk_gemm(q, k, geo, scores=s)
        if timed:
            e[1].record()
        qi.joint_attn_softmax(s, geo, p=p, alpha=alpha, l=l, lse=lse)
        if timed:
            e[2].record()
        qi.joint_attn_av_gemm(p, alpha, l, v, geo, out=o, workspace=ws)
        if timed:
            e[3].record()
            for i, n in enumerate(nbytes):
                ev[n].append((e[i], e[i + 1]))

    run(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        run(True)
    torch.cuda.synchronize()
    res = {"steps": steps, "bound": "hbm", "peak_gbps": PEAK_HBM_GBPS}
    total = 0.0
    for n, nb in nbytes.items():
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
        total += ms
        gbps = nb / (ms * 1e-3) / 1e9
        res[n] = {"ms": round(ms, 4), "bytes": nb, "gbps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    res["ms"] = round(total, 4)
    return res


def cpu_baseline(wl, inp, qp, kp, o, lse, target_s):
    """Time the oracle (as it stands) on the same workload on all host
    threads: the Q and K prologues and then the attention of every (b, h)
    slice, until about ``target_s`` seconds are spent (the whole forward of
    the 1024^2 workload takes a few seconds).  Every element the oracle
    produces is also compared with the GPU output."""
    import numpy as np

    import workloads
    from oracle import Oracle

    orc = Oracle("f32")
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    orc.set_threads(threads)
    f = lambda t: t.detach().float().cpu().numpy()  # noqa: E731
    on, ln = f(o), f(lse)
    t0 = time.perf_counter()
    qpre = orc.qknorm_rope(orc.widen(workloads.bits(inp["q"])), inp["g_q"].numpy(), wl.T_txt, wl.h, wl.w)
    kpre = orc.qknorm_rope(orc.widen(workloads.bits(inp["k"])), inp["g_k"].numpy(), wl.T_txt, wl.h, wl.w)
    qb, kb = orc.widen(orc.cast_bf16(qpre)), orc.widen(orc.cast_bf16(kpre))
    vn = orc.widen(workloads.bits(inp["v"]))
    t_pro = time.perf_counter() - t0
    flops, worst_o, worst_l, done = 0.0, 0.0, 0.0, 0
    t_att = 0.0
    for b in range(wl.B):
        K = wl.valid_keys()[b]
        for h in range(wl.H):
            t = time.perf_counter()
            ro, rl = orc.attn_fwd_bh(qb[b, :, h], kb[b, :, h], vn[b, :, h], wl.T_txt, wl.txt_len[b])
            t_att += time.perf_counter() - t
            flops += 4.0 * 128 * wl.S * K
            done += 1
            worst_o = max(worst_o, float(np.max(np.abs(on[b, :, h] - ro) / (1e-2 * np.abs(ro) + 2e-3))))
            worst_l = max(worst_l, float(np.max(np.abs(ln[b, h] - rl))))
            if t_pro + t_att > target_s:
                break
        if t_pro + t_att > target_s:
            break
    secs = t_pro + t_att
    whole = done == wl.B * wl.H
    what = "the whole forward step" if whole else f"the prologues and {done} of {wl.B * wl.H} (b, h) slices"
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of the same workload (Q/K RMSNorm+RoPE on all rows, then masked attention over "
                      f"all valid keys), FP32 C oracle with OpenMP, {secs:.1f} s",
            "seconds": round(secs, 2),
            "gpu_vs_oracle": {"elements": "every O and LSE element computed",
                              "O_max_ratio_to_bound": round(worst_o, 4), "LSE_max_abs_err": float(f"{worst_l:.3g}")}}


if __name__ == "__main__":
    main()
