"""Host logic of bench.py, without a GPU: the one-GPU guard, the algorithmic bytes per
kernel launch against the packed layout's sizes, and the reading of the committed
HBM counter summary."""
import json
import os
import subprocess
import sys

import bench
import quantized_expert_matvec_amd as qem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in rec and rec["requested_gpus"] == 2


def test_phase_bytes_follow_the_layout():
    H, I, E, K = 4096, 1024, 512, 4
    eb = qem.fmoe_expert_bytes(4, H, I)
    gub = eb - H * (I // 64) * 36  # gate/up rows: everything but the down rows
    assert (eb, gub) == (7077888, 4718592)
    xd = (H // 64) * 52 * 4  # x in digit form
    # router: fp32 rows + gate vector + x in, logits + sigma + digit form out
    assert bench.phase_bytes(1, 4, eb, gub, E, H, I, K, 4) == E * H * 4 + H * 4 + H * 4 + E * 4 + 4 + xd
    # gate/up: 4 distinct routed experts + the shared one, and the activations
    p2 = bench.phase_bytes(2, 4, eb, gub, E, H, I, K, 4)
    assert p2 == 5 * gub + xd + E * 4 + K * I * 4 + I * 4 == 23628800
    # down + combine: 5 down regions, h in, residual in, out
    p3 = bench.phase_bytes(4, 4, eb, gub, E, H, I, K, 4)
    assert p3 == 5 * (eb - gub) + K * I * 4 + I * 4 + H * 4 + 4 + H * 4 == 11849732
    # fewer distinct experts (repeated choices) move fewer bytes
    assert bench.phase_bytes(2, 3, eb, gub, E, H, I, K, 4) == p2 - gub


def test_counter_summary_is_read_only_for_known_kernels():
    assert bench.counter_traffic("no_such_kernel") is None
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()
    t = bench.counter_traffic("k_phase2")
    if t is not None:  # the summary matches the current sources
        assert 23628800 <= t <= 1.1 * 23628800
