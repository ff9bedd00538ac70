"""Host-side checks of bench.py (no GPU): the one-GPU guard and the reading
of the committed HBM counter summaries."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_is_used_only_for_its_own_kernel_source():
    # the committed attention-kernel summary names its source file and hash;
    # read against another source file (another hash) it is ignored
    path = os.path.join(ROOT, "profiles", "attn_fwd_kernel_1024sq_hbm_traffic.txt")
    assert os.path.exists(path)
    assert bench.traffic_from_profile("attn_fwd_kernel", "qi_prologue.hip", "1024sq") is None
    assert bench.traffic_from_profile("no_such_kernel", "qi_attn_fwd.hip", "1024sq") is None
    v = bench.traffic_from_profile("attn_fwd_kernel", "qi_attn_fwd.hip", "1024sq")
    assert v is None or abs(v - 1.2529e8) < 1e3
