"""Benchmark: µs per MoE decode layer (top-4 + shared, 4-bit, B=1) and weight GB/s.

Workload: a stack of MoE layers resident in HBM, each with 512 routed experts + 1
shared expert (hidden 4096, inter 1024, group-64 4-bit codes with bf16 scale and
bias), an fp32 512x4096 router and an fp32 shared-expert gate vector; RMS scaling
between layers; every layer has its own weights (60 layers = 218 GB at 4 bits), so
no layer's bytes can be served from the 256 MB Infinity Cache. A step is one
decode token (B tokens) through the whole stack: router, softmax top-4, the five
experts' gate/up + SwiGLU, down + weighted combine + residual + sigmoid-gated
shared expert, RMS scaling. Inputs are synthetic and seeded (no trained weights
exist here): codes ~ U{0..15}, scale ~ U(0.002, 0.02), bias = -8 scale (1 + U(-0.1, 0.1)),
router and gate vector ~ N(0, 0.02), fresh hidden states ~ N(0, 1) per step.

Besides the timed stack, the JSON line carries
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average duration, timed with HIP events on its own stream;
  cpu_baseline  the fp64 CPU oracle timed on one MoE layer of the same workload;
  parity        layer 0 of the first step checked against that oracle.

`--calibrate-copy` instead runs a plain 1 GiB device copy (for scaling the HBM
byte counters of a profiler run) and prints its size.

Prints one JSON line. With --gpus N > 1 it exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["layer_kernels.h", "device.h", "kernels.h", "layout.h", "kernels_q4.hip"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "moe_layer_q4_B1_hbm_counters.txt")
PHASE_NAMES = {1: "router + shared gate (k_phase1)", 2: "routing + routed and shared gate/up (k_phase2)",
               4: "routed and shared down + combine (k_phase3)"}
# the grouped layer's launches per phase (B > 1): the router and token preparation;
# the gate/up of the distinct experts (above 8 tokens after the routing kernels);
# the down projections and the combine
GROUP_PHASE_NAMES = {1: "router + token preparation (k_g1 / k_g1t)",
                     2: "gate/up of the distinct routed and shared experts (k_g2; k_topk + k_group above 8 tokens)",
                     4: "down projections + combine (k_g3 + k_g4)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=60)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--bits", type=int, default=4)
    p.add_argument("--experts", type=int, default=512)
    p.add_argument("--hidden", type=int, default=4096)
    p.add_argument("--inter", type=int, default=1024)
    p.add_argument("--topk", type=int, default=4)
    p.add_argument("--seed", type=int, default=42)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=5,
                   help="passes over the layers when timing one kernel (0: no per-kernel timing, so that a "
                        "counter run sees only the stack's own dispatches)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-verify", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--forms", action="store_true",
                   help="time the standalone matvec (1024 and 16384 x 4096) and the whole 4096/1024 SwiGLU "
                        "expert in each form of the per-weight dequant arithmetic (q4 and q2) instead of the stack")
    p.add_argument("--tier-slots", type=str, default=None,
                   help="time the host-memory expert tier instead of the resident stack: comma-separated HBM cache "
                        "sizes in expert slots ('pages' = the pages' page-cache share of the bank, 35 of 209 GB); "
                        "one JSON line each, plus one for a repeated token (every expert a hit)")
    p.add_argument("--tier-layers", type=int, default=8, help="layers whose routed banks sit in pinned host memory")
    p.add_argument("--tier-policy", choices=["host", "device", "both"], default="both",
                   help="where the host-memory tier's cache policy runs")
    p.add_argument("--timeline", action="store_true",
                   help="print device-clock stamps of a few layers' kernels inside the graph-captured stack "
                        "instead of timing")
    return p.parse_args()


class Filler:
    """Device generation (bit-identical to the host generator) + the library's device packer."""

    def __init__(self, torch, synth, qem, hidden, inter, dev):
        self.t, self.synth, self.qem = torch, synth, qem
        self.hidden, self.inter = hidden, inter
        n = hidden * inter
        self.codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(3)]
        self.scale = [torch.empty(n // 64, dtype=torch.int16, device=dev) for _ in range(3)]
        self.bias = [torch.empty(n // 64, dtype=torch.int16, device=dev) for _ in range(3)]

    def expert(self, seed, layer, expert_id, bits, blob_out):
        H, I, s = self.hidden, self.inter, self.synth
        st = self.t.cuda.current_stream().cuda_stream
        for j, (tid, r, c) in enumerate([(s.T_GATE, I, H), (s.T_UP, I, H), (s.T_DOWN, H, I)]):
            s.dev_qmat(seed, layer, expert_id, tid, bits, r, c, self.codes[j], self.scale[j], self.bias[j], st)
        self.qem.fmoe_pack_expert_device(bits, H, I, self.codes, self.scale, self.bias, blob_out)


def tier(a):
    """The host-memory expert tier: the routed banks of --tier-layers layers in pinned host
    memory, an HBM cache of expert slots shared by the layers. A step runs the layers in
    order (RMS scaling, then the tiered layer call: routing on the GPU, one read-back,
    copies of the misses, the experts from their slots). Fresh synthetic tokens every
    step (uniform routing: the hit rate is about the cache's share of the bank); the last
    line repeats one token (every expert a hit after the first step), the call's floor."""
    import numpy as np
    import psutil
    import torch

    import synth
    import quantized_expert_matvec_amd as qem

    dev = torch.device("cuda:0")
    H, I, E, K, B, bits = a.hidden, a.inter, a.experts, a.topk, a.batch, a.bits
    eb = qem.fmoe_expert_bytes(bits, H, I)
    bank_bytes = E * eb
    avail = psutil.virtual_memory().available
    n_layers = max(1, min(a.tier_layers, int(0.4 * avail // bank_bytes)))
    if n_layers < a.tier_layers:
        log(f"bench: tier with {n_layers} layers ({avail / 2**30:.0f} GiB host memory available)")
    log(f"bench: filling {n_layers} host banks x {bank_bytes / 1e9:.2f} GB (pinned)")
    t0 = time.time()
    filler = Filler(torch, synth, qem, H, I, dev)
    stage = torch.empty(bank_bytes, dtype=torch.uint8, device=dev)
    layers, keep = [], []
    for l in range(n_layers):
        for e in range(E):
            filler.expert(a.seed, l, e, bits, stage[e * eb:(e + 1) * eb])
        host = torch.empty(bank_bytes, dtype=torch.uint8, pin_memory=True)
        host.copy_(stage)
        sh = torch.empty(eb, dtype=torch.uint8, device=dev)
        filler.expert(a.seed, l, synth.SHARED_EXPERT, bits, sh)
        R = torch.from_numpy(synth.router(a.seed, l, E, H)).to(dev)
        g = torch.from_numpy(synth.shared_gate(a.seed, l, H)).to(dev)
        keep.append((host, sh, R, g))
        layers.append(qem.Layer(R, g, host, sh, E, K, H, I, bits))
    torch.cuda.synchronize()
    del stage, filler
    log(f"bench: fill done in {time.time() - t0:.1f} s")

    # host-to-device rate of one expert blob at a time (the tier's unit of transfer)
    probe = torch.empty(4 * eb, dtype=torch.uint8, device=dev)
    src = keep[0][0]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep_ in range(2):
        e0.record()
        for r in range(16):
            for j in range(4):
                probe[j * eb:(j + 1) * eb].copy_(src[((4 * r + j) * 37 % E) * eb:][:eb], non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
    h2d_gbps = 64 * eb / (e0.elapsed_time(e1) * 1e6)
    del probe

    h = torch.empty((B, H), dtype=torch.float32, device=dev)
    h2 = torch.empty_like(h)
    x = torch.empty_like(h)
    ws = torch.empty(qem.fmoe_tiered_workspace_bytes(layers[0], B), dtype=torch.uint8, device=dev)

    def tokens(i):
        return torch.from_numpy(synth.activations(a.seed, synth.T_H0, i, B, H)).to(dev)

    def step(cache, h0):
        nonlocal h, h2
        h.copy_(h0)
        for l in range(n_layers):
            qem.fmoe_rms_scale(h, x)
            qem.fmoe_moe_layer_tiered(cache, l, layers[l], x, h, out=h2, ws=ws)
            h, h2 = h2, h
        torch.cuda.synchronize()

    # the policy on the GPU: the layers' calls need no host synchronisation, so a step is
    # captured once in a graph (after an eager step that initialises the cache's state)
    # and replayed; a step copies its tokens into the graph's input first
    hin = torch.empty_like(h)
    hbuf = [torch.empty_like(h) for _ in range(2)]

    def dev_calls(cache):
        cur = hin
        for l in range(n_layers):
            qem.fmoe_rms_scale(cur, x)
            nxt = hbuf[l & 1]
            qem.fmoe_moe_layer_tiered_device(cache, l, layers[l], x, cur, out=nxt, ws=ws)
            cur = nxt

    graphs = {}

    def step_dev(cache, h0):
        hin.copy_(h0)
        g = graphs.get(id(cache))
        if g is None:
            dev_calls(cache)  # eager (the first call of each layer initialises or warms)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dev_calls(cache)
            graphs[id(cache)] = g
            hin.copy_(h0)
        g.replay()
        torch.cuda.synchronize()

    total_slots = n_layers * E
    sizes = []
    for t in a.tier_slots.split(","):
        t = t.strip()
        sizes.append(max(K * B, round(total_slots * 35 / 209)) if t == "pages" else int(t))
    policies = ["host", "device"] if a.tier_policy == "both" else [a.tier_policy]
    for policy, n_slots, repeat in [(p, n, False) for p in policies for n in sizes] + \
                                   [(p, max(sizes), True) for p in policies]:
        buf_bytes = qem.fmoe_cache_device_bytes(bits, H, I, E, n_slots)
        cache = qem.ExpertCache(bits, H, I, E, n_slots, dev)
        run_step = step if policy == "host" else step_dev
        warm = a.warmup + (1 if repeat else int(np.ceil(2 * n_slots / (K * B * n_layers))))
        log(f"bench: tier ({policy} policy) {n_slots} slots{' (repeated token)' if repeat else ''}: "
            f"{warm} warm-up steps")
        tok = 0
        for s in range(warm):
            run_step(cache, tokens(0 if repeat else tok))
            tok += 1
        st0 = cache.stats()
        times = []
        for s in range(a.steps):
            h0 = tokens(0 if repeat else tok)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            run_step(cache, h0)
            times.append(time.perf_counter() - t1)
            tok += 1
        st1 = cache.stats()
        hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
        copied = st1["bytes_copied"] - st0["bytes_copied"]
        per_layer = np.array(times) * 1e6 / n_layers
        us_layer = float(np.sum(times) * 1e6 / (a.steps * n_layers))
        rec = {
            "metric": f"µs per MoE layer, routed experts in host memory behind an HBM cache "
                      f"(top-{K} + shared, {bits}-bit, B={B}, policy on the {policy})",
            "value": round(us_layer, 2), "unit": "us/layer", "higher_is_better": False,
            "steps": a.steps, "warmup": warm,
            "config": {"workload": f"moe_stack_q{bits}_B{B}_host_tier", "layers": n_layers, "batch": B,
                       "experts": E, "top_k": K, "hidden": H, "inter": I, "group": 64,
                       "policy": "host (one read-back per layer)" if policy == "host"
                       else "device (no host synchronisation; a step is one graph replay)",
                       "cache_slots": n_slots, "cache_share_of_bank": round(n_slots / total_slots, 4),
                       "cache_GB": round(buf_bytes / 1e9, 2), "host_bank_GB": round(n_layers * bank_bytes / 1e9, 2),
                       "tokens": "one token repeated" if repeat else "fresh synthetic tokens each step"},
            "us_per_layer_p10_p50_p90": [round(float(v), 1) for v in np.percentile(per_layer, [10, 50, 90])],
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "distinct_experts_per_layer": round((hits + misses) / (a.steps * n_layers), 3),
            "misses_per_layer": round(misses / (a.steps * n_layers), 3),
            "copied_MB_per_layer": round(copied / (a.steps * n_layers) / 1e6, 2),
            "h2d_GBps_one_expert_copies": round(h2d_gbps, 1),
            "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        }
        print(json.dumps(rec, ensure_ascii=False), flush=True)
        graphs.pop(id(cache), None)
        cache.close()
        del cache
        torch.cuda.empty_cache()


def calibrate_copy():
    """A plain device-to-device copy of known size, for the profiler's byte counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)   # one elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise int32 bitwise_not, 1 GiB in, 1 GiB out",
                      "bytes_read": n, "bytes_written": n}), flush=True)


def timeline(torch, np, qem, layers, c_layers, h_in, h0_all, ws, n_layers):
    """Per-workgroup device-clock stamps (100 MHz) of the kernels of a few layers,
    each inside the graph-captured stack, summarised per kernel: when the workgroups
    start, have their inputs in LDS, know the routing, and end (one token), or finish
    their work items (the grouped layer's persistent gate/up kernel)."""
    B = h_in.shape[0]
    tr = torch.zeros((3, qem.TRACE_BLOCKS, qem.TRACE_SLOTS), dtype=torch.int64, device=h_in.device)
    h_out = torch.empty_like(h_in)
    picks = sorted({n_layers // 4, n_layers // 2, (3 * n_layers) // 4})
    names = ("k_phase1 (router, x digits, gate)", "k_phase2 (routing, gate/up)", "k_phase3 (down, combine)")
    print(f"device-clock stamps of one layer's kernels inside the graph-captured stack (B={B}); "
          "µs from the first router workgroup's start; min / median / p90 / max over workgroups", flush=True)
    for lt in picks:
        def call():
            qem.fmoe_moe_stack_trace(layers, h_in, tr, lt, h_out=h_out, ws=ws, c_layers=c_layers)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for s in range(3):
            h_in.copy_(h0_all[s % h0_all.shape[0]])
            g.replay()
        torch.cuda.synchronize()
        tr.zero_()
        h_in.copy_(h0_all[3 % h0_all.shape[0]])
        g.replay()
        torch.cuda.synchronize()
        del g
        t = tr.cpu().numpy()
        rec = [t[k][t[k, :, 0] > 0] for k in range(3)]
        t0 = rec[0][:, 0].min()
        us = lambda v: (v - t0) / 100.0
        q = lambda v: "/".join(f"{x:5.2f}" for x in np.percentile(us(v), [0, 50, 90, 100]))
        print(f"layer {lt}:", flush=True)
        if B > 1:
            timeline_grouped(np, rec, us, q)
            continue
        for k in range(3):
            r = rec[k]
            if k == 0:
                groups = [("router", r[r[:, 1] > 0]), ("x digits, gate", r[r[:, 1] == 0])]
            elif k == 1:
                groups = [("routed", r[r[:, 2] > 0]), ("shared", r[r[:, 2] == 0])]
            else:
                groups = [("all", r)]
            for gname, gr in groups:
                if len(gr) == 0:
                    continue
                line = f"  {names[k]:34s} {gname:14s} {len(gr):4d} wg  start {q(gr[:, 0])}"
                if (gr[:, 1] > 0).all():
                    line += f"  inputs {q(gr[:, 1])}"
                if (gr[:, 2] > 0).all():
                    line += f"  routing {q(gr[:, 2])}"
                line += f"  end {q(gr[:, 3])}"
                print(line, flush=True)
        gaps = [us(rec[k + 1][:, 0].min()) - us(rec[k][:, 3].max()) for k in range(2)]
        print(f"  last end -> next kernel's first start: k_phase1 -> k_phase2 {gaps[0]:.2f}, "
              f"k_phase2 -> k_phase3 {gaps[1]:.2f}; first start -> last end of the layer "
              f"{us(rec[2][:, 3].max()):.2f}", flush=True)


def timeline_grouped(np, rec, us, q):
    """Summary of the grouped layer's stamps: router + token preparation; the persistent
    gate/up workgroups (start, routing derived, each item's end, end; items per workgroup
    and the time per item); the down workgroups."""
    names = ("router + token preparation", "gate/up (persistent)", "down")
    r = rec[0]
    print(f"  {names[0]:28s} {len(r):4d} wg  start {q(r[:, 0])}  end {q(r[:, 3])}", flush=True)
    r = rec[1]
    line = f"  {names[1]:28s} {len(r):4d} wg  start {q(r[:, 0])}"
    routed = r[r[:, 1] > 0]
    if len(routed):
        line += f"  routing {q(routed[:, 1])}"
    line += f"  first item end {q(r[r[:, 2] > 0][:, 2])}  end {q(r[:, 7])}"
    print(line, flush=True)
    items = (r[:, 2:7] > 0).sum(axis=1)
    hist = {int(k): int(v) for k, v in zip(*np.unique(items, return_counts=True))}
    durs = []
    for row in r:
        prev = row[1] if row[1] > 0 and row[1] < row[2] else row[0]
        for i in range(5):
            if row[2 + i] > 0:
                durs.append((row[2 + i] - prev) / 100.0)
                prev = row[2 + i]
    d = np.array(durs)
    print(f"  {'':28s} items per workgroup {hist} (5 = five or more); time per item "
          f"{'/'.join(f'{x:5.2f}' for x in np.percentile(d, [0, 50, 90, 100]))} µs", flush=True)
    r = rec[2]
    print(f"  {names[2]:28s} {len(r):4d} wg  start {q(r[:, 0])}  end {q(r[:, 3])}", flush=True)
    gaps = [us(rec[k + 1][:, 0].min()) - us(rec[k][:, 3 if k == 0 else 7].max()) for k in range(2)]
    print(f"  last end -> next kernel's first start: router -> gate/up {gaps[0]:.2f} (the top-K "
          f"kernel between them above 8 tokens, and the grouping kernel above 64 slots), gate/up -> down {gaps[1]:.2f}; first start -> last down end "
          f"{us(rec[2][:, 3].max()):.2f} (the combine follows)", flush=True)


FORM_NAMES = {0: "naive (c*s+b)*x", 1: "recast fma(c, s*x, b*x)", 2: "group-factored s*sum(c*x)+b*sum(x)",
              3: "table of c*s+b in LDS"}


def forms(a):
    """The standalone dequantized matvec W [rows][4096] (rows 1024, and 16384 where the
    per-weight arithmetic weighs more than the launch) in each form of the per-weight
    arithmetic (fmoe_qmatvec_form) and the library's own call, q4 and q2; then the whole
    SwiGLU expert (hidden 4096, inter 1024: fmoe_expert_ffn against fmoe_expert_ffn_form
    in each form); then the one-token MoE layer (fmoe_moe_layer against
    fmoe_moe_layer_form). Each is a graph of one call per copy (per layer) over enough
    independent copies of the weights and x that they exceed the 256 MB Infinity Cache.
    Each form's output of copy 0 is compared with the library call's (the tests check
    every form against the oracle)."""
    import numpy as np
    import torch

    import synth
    import quantized_expert_matvec_amd as qem
    dev = torch.device("cuda:0")
    cols = 4096
    st = torch.cuda.current_stream().cuda_stream
    recs = []
    for rows, bits in ((1024, 4), (1024, 2), (16384, 4), (16384, 2)):
        nb = qem.fmoe_qmat_bytes(bits, rows, cols)
        stride = (nb + 255) // 256 * 256
        copies = max(8, -(-(450 << 20) // stride))
        bank = torch.empty(copies * stride, dtype=torch.uint8, device=dev)
        codes = torch.empty(rows * cols, dtype=torch.uint8, device=dev)
        scale = torch.empty(rows * cols // 64, dtype=torch.int16, device=dev)
        bias = torch.empty(rows * cols // 64, dtype=torch.int16, device=dev)
        for k in range(copies):
            synth.dev_qmat(a.seed, synth.STANDALONE_LAYER, k, synth.T_MATRIX, bits, rows, cols, codes, scale, bias, st)
            qem.fmoe_pack_qmat_device(bits, rows, cols, codes, scale, bias, bank[k * stride:(k + 1) * stride])
        xs = torch.from_numpy(np.stack([synth.activations(a.seed, synth.T_X, k, 1, cols)[0]
                                        for k in range(copies)])).to(dev)
        ys = torch.empty((copies, rows), dtype=torch.float32, device=dev)
        cq = [qem.QMat(bank[k * stride:(k + 1) * stride], rows, cols, bits).c() for k in range(copies)]
        lib_fn = qem.lib().fmoe_q4_matvec if bits == 4 else qem.lib().fmoe_q2_matvec
        variants = [(None, f"library call fmoe_q{bits}_matvec")] + [(f, FORM_NAMES[f]) for f in range(4)]
        ref = None
        for form, name in variants:
            def call():
                for k in range(copies):
                    if form is None:
                        lib_fn(cq[k], xs[k].data_ptr(), ys[k].data_ptr(), torch.cuda.current_stream().cuda_stream)
                    else:
                        qem.lib().fmoe_qmatvec_form(cq[k], xs[k].data_ptr(), ys[k].data_ptr(), form,
                                                    torch.cuda.current_stream().cuda_stream)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            y0 = ys[0].cpu().numpy().astype(np.float64)
            if ref is None:
                ref = y0
            max_rel = float(np.max(np.abs(y0 - ref)) / np.max(np.abs(ref)))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / (5 * copies)
            algo = nb + cols * 4 + rows * 4
            recs.append({"rows": rows, "cols": cols, "bits": bits, "form": form, "name": name,
                         "us_per_matvec": round(us, 3),
                         "GBps": round(algo / (us * 1e3), 1), "algorithmic_bytes": algo, "copies": copies,
                         "max_rel_vs_library_call": max_rel})
            print(json.dumps(recs[-1]), flush=True)
            del g
        del bank, xs, ys
    # the whole SwiGLU expert (hidden 4096, inter 1024) in each form: the library's
    # fmoe_expert_ffn and fmoe_expert_ffn_form(0..3), a graph of one call per copy
    H, I = cols, 1024
    filler = Filler(torch, synth, qem, H, I, dev)
    for bits in (4, 2):
        eb = qem.fmoe_expert_bytes(bits, H, I)
        copies = max(8, -(-(450 << 20) // eb))
        bank = torch.empty(copies * eb, dtype=torch.uint8, device=dev)
        for k in range(copies):
            filler.expert(a.seed, synth.STANDALONE_LAYER, k, bits, bank[k * eb:(k + 1) * eb])
        xs = torch.from_numpy(np.stack([synth.activations(a.seed, synth.T_X, k, 1, H)[0]
                                        for k in range(copies)])).to(dev)
        ys = torch.empty((copies, H), dtype=torch.float32, device=dev)
        Es = [qem.Expert(bank[k * eb:(k + 1) * eb], H, I, bits) for k in range(copies)]
        ce = [E.c() for E in Es]
        need = qem.fmoe_expert_workspace_bytes(Es[0])
        ws = torch.empty((copies, (need + 255) // 256 * 256), dtype=torch.uint8, device=dev)
        ref = None
        for form, name in [(None, "library call fmoe_expert_ffn")] + [(f, FORM_NAMES[f]) for f in range(4)]:
            def call():
                stn = torch.cuda.current_stream().cuda_stream
                for k in range(copies):
                    if form is None:
                        qem.lib().fmoe_expert_ffn(ce[k], xs[k].data_ptr(), ys[k].data_ptr(), ws[k].data_ptr(),
                                                  ws.shape[1], stn)
                    else:
                        qem.lib().fmoe_expert_ffn_form(ce[k], xs[k].data_ptr(), ys[k].data_ptr(), ws[k].data_ptr(),
                                                       ws.shape[1], form, stn)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            y0 = ys[0].cpu().numpy().astype(np.float64)
            if ref is None:
                ref = y0
            max_rel = float(np.max(np.abs(y0 - ref)) / np.max(np.abs(ref)))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / (5 * copies)
            algo = eb + 2 * H * 4 + I * 4 * 2
            recs.append({"expert": f"{H}/{I}", "bits": bits, "form": form, "name": name,
                         "us_per_expert": round(us, 3), "GBps": round(algo / (us * 1e3), 1),
                         "algorithmic_bytes": algo, "copies": copies, "max_rel_vs_library_call": max_rel})
            print(json.dumps(recs[-1]), flush=True)
            del g
        del bank, xs, ys, ws
    # the one-token MoE layer (512 experts + shared, hidden 4096, inter 1024, top-4) with
    # every expert projection in each form: fmoe_moe_layer against fmoe_moe_layer_form,
    # a graph of one call per layer over 8 layers (350 MB of chosen weights at q4)
    E, K, NL = 512, 4, 8
    for bits in (4, 2):
        eb = qem.fmoe_expert_bytes(bits, H, I)
        keep, layers = [], []
        for l in range(NL):
            bank = torch.empty((E + 1) * eb, dtype=torch.uint8, device=dev)
            for e in range(E):
                filler.expert(a.seed, 200 + l, e, bits, bank[e * eb:(e + 1) * eb])
            filler.expert(a.seed, 200 + l, synth.SHARED_EXPERT, bits, bank[E * eb:])
            R = torch.from_numpy(synth.router(a.seed, 200 + l, E, H)).to(dev)
            gv = torch.from_numpy(synth.shared_gate(a.seed, 200 + l, H)).to(dev)
            keep.append((bank, R, gv))
            layers.append(qem.Layer(R, gv, bank[:E * eb], bank[E * eb:], E, K, H, I, bits))
        cl = [L.c() for L in layers]
        x = torch.from_numpy(synth.activations(a.seed, synth.T_X, 77, 1, H)).to(dev)
        res = torch.from_numpy(synth.activations(a.seed, synth.T_RESIDUAL, 77, 1, H)).to(dev)
        outs = torch.empty((NL, 1, H), dtype=torch.float32, device=dev)
        need = qem.fmoe_workspace_bytes(layers[0], 1)
        ws = torch.empty((NL, (need + 255) // 256 * 256), dtype=torch.uint8, device=dev)
        ref = None
        for form, name in [(None, "library call fmoe_moe_layer")] + [(f, FORM_NAMES[f]) for f in range(4)]:
            def call():
                stn = torch.cuda.current_stream().cuda_stream
                for l in range(NL):
                    if form is None:
                        qem.lib().fmoe_moe_layer(cl[l], 1, x.data_ptr(), res.data_ptr(), outs[l].data_ptr(), None,
                                                 None, ws[l].data_ptr(), ws.shape[1], stn)
                    else:
                        qem.lib().fmoe_moe_layer_form(cl[l], x.data_ptr(), res.data_ptr(), outs[l].data_ptr(), None,
                                                      None, ws[l].data_ptr(), ws.shape[1], form, stn)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            y0 = (outs[0] - res).cpu().numpy().astype(np.float64)
            if ref is None:
                ref = y0
            max_rel = float(np.max(np.abs(y0 - ref)) / np.max(np.abs(ref)))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / (10 * NL)
            algo = (K + 1) * eb + E * H * 4 + H * 4
            recs.append({"layer": f"{E}+1 experts, {H}/{I}, top-{K}", "bits": bits, "form": form, "name": name,
                         "us_per_layer": round(us, 3), "GBps": round(algo / (us * 1e3), 1),
                         "algorithmic_bytes": algo, "layers": NL, "max_rel_vs_library_call": max_rel})
            print(json.dumps(recs[-1]), flush=True)
            del g
        del keep, layers, outs, ws


def read_ceiling(torch, qem, dev):
    """The HBM read rate this GPU reaches (the library's streaming-read kernel over a
    4 GiB buffer, 12 passes in a graph), and the time per launch of an empty kernel in a
    graph of 180 (the floor of a kernel boundary)."""
    free = torch.cuda.mem_get_info()[0]
    nb = min(4 << 30, (free - (1 << 30)) // (1 << 20) * (1 << 20))
    if nb < (256 << 20):
        return None, None  # no room for a buffer well beyond the caches
    buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    res = []
    for calls, src in ((4, buf), (180, None)):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            qem.fmoe_read_xor(src, out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(calls):
                qem.fmoe_read_xor(src, out)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1000.0 / (3 * calls))  # µs per launch
        del g
    del buf
    return ({"GBps": round(nb / (res[0] * 1e3), 1), "bytes": int(nb),
             "kernel": "fmoe_read_xor (16-byte non-temporal loads, 8 in flight per thread)"}, round(res[1], 3))


def burst_floor(torch, qem, dev, sizes, rounds=60):
    """How long plain streaming kernels with the given byte counts take back to back: the
    library's streaming-read kernel (every thread's loads requested at once: one burst per
    launch) on `rounds` rounds of distinct buffers, one launch per size per round, in a
    graph replayed 3 times. Returns µs per round and, per size, µs per launch alone."""
    sizes = [(n + 15) // 16 * 16 for n in sizes]
    need = rounds * sum(sizes)
    if torch.cuda.mem_get_info()[0] < need + (1 << 30):
        return None
    buf = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    offs = [sum(sizes[:i]) for i in range(len(sizes))]

    def timed(which):
        def call():
            for r in range(rounds):
                base = r * sum(sizes)
                for i in which:
                    qem.fmoe_read_xor(buf[base + offs[i]:base + offs[i] + sizes[i]], out)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1000.0 / (3 * rounds)

    chain = timed(list(range(len(sizes))))
    alone = [timed([i]) for i in range(len(sizes))]
    del buf
    return round(chain, 3), [round(t, 3) for t in alone]


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model/stepping numbers."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                info.setdefault(k.strip(), v.strip())
    except OSError:
        return None
    name = info.get("model name")
    if name is None:
        return None
    ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({ids})" if ids else name


def host_threads():
    """Hardware threads this process may run on (what std::thread::hardware_concurrency reports,
    within the CPU set the process is allowed)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count()


def versions(torch):
    v = {"torch": torch.__version__, "hip": torch.version.hip,
         "gpu": torch.cuda.get_device_properties(0).gcnArchName}
    for key, path in (("rocm", "/opt/rocm/.info/version"), ("amdgpu_driver", "/sys/module/amdgpu/version")):
        try:
            v[key] = open(path).read().strip()
        except OSError:
            v[key] = None
    return v


def kernels_per_layer(B, K):
    """Launches of one layer: 3 for one token; grouped, 4, plus the top-K kernel above 8
    tokens (or 128 slots), plus the grouping kernel above 64 slots."""
    if B == 1:
        return 3
    if B <= 8 and B * K <= 128:
        return 4
    return 5 if B * K <= 64 else 6


def group_phase_bytes(phase, d_routed, eb, gub, E, H, I, K, B):
    """Algorithmic bytes of one grouped phase: every weight row once, plus activations."""
    if phase == 1:   # router + gate vector; x in; logits, x in integer form out
        return E * H * 4 + H * 4 + B * H * 4 + B * E * 4 + 3 * B * H
    if phase == 2:   # distinct routed + shared gate/up halves; logits, x (integer form) in
        return (d_routed + 1) * gub + B * E * 4 + 3 * B * H
    if phase == 4:   # distinct routed + shared down halves; partials, residual, shared output, out
        return (d_routed + 1) * (eb - gub) + B * (K + 2) * H * 4
    raise ValueError(phase)


def phase_bytes(phase, d_routed, eb, gub, E, H, I, K, bits):
    """Algorithmic bytes one launch of a layer kernel moves (B=1): the weights it must
    stream once plus its activation reads and writes."""
    down = eb - gub
    xd = (H // 64) * 52 * 4  # x in digit form: 52 words per 64-column group
    if phase == 1:   # router rows + gate vector; x in; logits, sigma, x in digit form out
        return E * H * 4 + H * 4 + H * 4 + E * 4 + 4 + xd
    if phase == 2:   # distinct routed gate/up + shared gate/up; x (digit form), logits in; h_routed, h_shared out
        return d_routed * gub + gub + xd + E * 4 + K * I * 4 + I * 4
    if phase == 4:   # distinct routed down + shared down; h_routed, h_shared, residual, sigma in; out
        return d_routed * down + down + K * I * 4 + I * 4 + H * 4 + 4 + H * 4
    raise ValueError(phase)


def kernel_source_hash():
    """sha256 over the sources of the one-token layer kernels (q4 instantiation)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_expert_matvec_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(tag):
    """HBM bytes per launch of kernel `tag` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by the copy calibration), or None when there is
    none or the kernel sources changed since the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    h = kernel_source_hash()
    with open(COUNTERS_FILE) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 8 and f[0] == "counters" and f[1] == tag and f[7] == h:
                return int(f[3]) + int(f[5])
    return None


def cpu_baseline(a, synth, oracle, R0, g0, h0, budget_s):
    """Time the fp64 oracle on MoE layer 0 for one token; also returns its output for parity."""
    H, I, E, K, bits = a.hidden, a.inter, a.experts, a.topk, a.bits
    x0 = oracle.rms_scale(h0)
    idx, _, _ = oracle.route(oracle.router_logits(R0, x0), K)
    experts = {int(e): synth.expert(a.seed, 0, int(e), bits, H, I) for e in idx}
    shared = synth.expert(a.seed, 0, synth.SHARED_EXPERT, bits, H, I)
    reps, t_total, res = 0, 0.0, None
    while reps == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        res = oracle.moe_layer(R0, g0, experts, shared, x0, h0, K)
        t_total += time.perf_counter() - t0
        reps += 1
    return t_total / reps, reps, t_total, res


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "requested_gpus": a.gpus}))
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.forms:
        forms(a)
        return
    if a.tier_slots:
        tier(a)
        return
    import numpy as np
    import torch

    import synth
    import quantized_expert_matvec_amd as qem

    dev = torch.device("cuda:0")
    H, I, E, K, B, bits = a.hidden, a.inter, a.experts, a.topk, a.batch, a.bits
    eb = qem.fmoe_expert_bytes(bits, H, I)
    gub = eb - H * (I // 64) * (bits * 8 + 4)
    layer_bytes = (E + 1) * eb + E * H * 4 + H * 4
    free, total = torch.cuda.mem_get_info()
    n_layers = min(a.layers, int((free - 8 * 2 ** 30) // layer_bytes))
    if n_layers < a.layers:
        log(f"bench: only {n_layers} of {a.layers} layers fit ({free / 2**30:.1f} GiB free)")
    log(f"bench: filling {n_layers} layers x {layer_bytes / 1e9:.2f} GB")
    t0 = time.time()
    filler = Filler(torch, synth, qem, H, I, dev)
    layers, keep = [], []
    for l in range(n_layers):
        bank = torch.empty((E + 1) * eb, dtype=torch.uint8, device=dev)
        for e in range(E):
            filler.expert(a.seed, l, e, bits, bank[e * eb:(e + 1) * eb])
        filler.expert(a.seed, l, synth.SHARED_EXPERT, bits, bank[E * eb:])
        R = torch.from_numpy(synth.router(a.seed, l, E, H)).to(dev)
        g = torch.from_numpy(synth.shared_gate(a.seed, l, H)).to(dev)
        keep.append((bank, R, g))
        layers.append(qem.Layer(R, g, bank[:E * eb], bank[E * eb:], E, K, H, I, bits))
        if l % 10 == 9:
            torch.cuda.synchronize()
            log(f"bench: filled {l + 1} layers ({time.time() - t0:.1f} s)")
    del filler
    torch.cuda.synchronize()
    log(f"bench: fill done in {time.time() - t0:.1f} s")

    steps = a.warmup + a.steps
    h0_host = np.stack([synth.activations(a.seed, synth.T_H0, s, B, H) for s in range(steps)])
    h0_all = torch.from_numpy(h0_host).to(dev)
    c_layers = (qem.fmoe_layer * n_layers)(*[L.c() for L in layers])
    h_in = torch.empty((B, H), dtype=torch.float32, device=dev)
    h_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    idx = torch.empty((n_layers, B, K), dtype=torch.int32, device=dev)
    ws = torch.empty(qem.fmoe_stack_workspace_bytes(layers[0], B), dtype=torch.uint8, device=dev)

    def step_call():
        qem.fmoe_moe_stack(layers, h_in, h_out=h_out, topk_idx=idx, ws=ws, c_layers=c_layers)

    h_in.copy_(h0_all[0])
    step_call()
    torch.cuda.synchronize()
    graph = None
    if not a.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_call()
        torch.cuda.synchronize()

    if a.timeline:
        timeline(torch, np, qem, layers, c_layers, h_in, h0_all, ws, n_layers)
        return

    def run(s):
        h_in.copy_(h0_all[s])
        if graph is not None:
            graph.replay()
        else:
            step_call()

    log("bench: timing the stack")
    for s in range(a.warmup):
        run(s)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    evs[0].record()
    for j, s in enumerate(range(a.warmup, steps)):
        run(s)
        evs[j + 1].record()
    torch.cuda.synchronize()
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_step = ms_total / a.steps
    us_layer = ms_step * 1000.0 / n_layers
    per_step = np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(a.steps)]) * 1000.0 / n_layers
    spread = [round(float(v), 3) for v in np.percentile(per_step, [10, 50, 90])]

    # ---- the measured read ceiling and the empty-kernel gap inside a graph
    log("bench: streaming-read ceiling and empty-kernel gap")
    ceiling, gap = read_ceiling(torch, qem, dev)

    # algorithmic bytes: the distinct experts each layer-step touches (replayed untimed)
    distinct = []
    for s in range(a.warmup, steps):
        run(s)
        torch.cuda.synchronize()
        ii = idx.cpu().numpy()
        distinct.append(np.mean([len(set(ii[l].ravel().tolist())) for l in range(n_layers)]))
    d_mean = float(np.mean(distinct))
    w_bytes_layer = (d_mean + 1) * eb + E * H * 4 + H * 4
    act_bytes_layer = 3 * B * H * 4
    weight_gbps = w_bytes_layer / (us_layer * 1e3)

    # ---- per-kernel (B=1) or per-phase (grouped) durations, HIP events on the launching stream
    roofline, kernels = None, {}
    if a.kernel_reps > 0:
        log("bench: timing each layer kernel")
        kstream = torch.cuda.Stream()
        xs = torch.from_numpy(np.stack([synth.activations(a.seed, synth.T_X, l, B, H)
                                        for l in range(n_layers)])).to(dev)
        outs = torch.empty((n_layers, B, H), dtype=torch.float32, device=dev)
        lws_bytes = qem.fmoe_workspace_bytes(layers[0], B)
        lws = torch.empty((n_layers, (lws_bytes + 255) // 256 * 256), dtype=torch.uint8, device=dev)
        kp = (B * K + 3) // 4 * 4  # (rows 16-byte aligned)
        kidx = torch.empty((n_layers, kp), dtype=torch.int32, device=dev)
        with torch.cuda.stream(kstream):
            for l in range(n_layers):   # full layers first: every kernel's inputs are then in place
                qem.fmoe_moe_layer_phases(layers[l], xs[l], xs[l], outs[l], 7, lws[l],
                                          topk_idx=kidx[l, :B * K], stream=kstream, c_layer=c_layers[l])
        kstream.synchronize()
        kd = float(np.mean([len(set(r[:B * K].tolist())) for r in kidx.cpu().numpy()]))
        names = PHASE_NAMES if B == 1 else GROUP_PHASE_NAMES
        for ph in (1, 2, 4):
            # n_layers launches of one phase, captured once and replayed on kstream
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=kstream):
                for l in range(n_layers):
                    qem.fmoe_moe_layer_phases(layers[l], xs[l], xs[l], outs[l], ph, lws[l], c_layer=c_layers[l])
            with torch.cuda.stream(kstream):
                g.replay()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(kstream)
                for _ in range(a.kernel_reps):
                    g.replay()
                e1.record(kstream)
            kstream.synchronize()
            del g
            us = e0.elapsed_time(e1) * 1000.0 / (a.kernel_reps * n_layers)
            nbytes = (phase_bytes(ph, kd, eb, gub, E, H, I, K, bits) if B == 1
                      else group_phase_bytes(ph, kd, eb, gub, E, H, I, K, B))
            kernels[names[ph]] = {"avg_us": round(us, 3), "algorithmic_bytes": int(nbytes),
                                  "GBps": round(nbytes / (us * 1e3), 1)}
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        kk = kernels[dom]
        tag = dom.split("(")[-1].rstrip(")")
        traffic = (counter_traffic(tag) if (B == 1 and bits == 4 and (H, I, E, K) == (4096, 1024, 512, 4))
                   else None)
        roofline = {"bound": "hbm", "achieved": kk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(kk["GBps"] / HBM_PEAK_GBPS, 4), "traffic": traffic, "traffic_unit": "bytes/launch",
                    "kernel": dom, "avg_us": kk["avg_us"], "algorithmic_bytes_per_launch": kk["algorithmic_bytes"]}
        del lws, outs, xs

    # ---- one token: how long three plain streaming kernels with the layer kernels' bytes take
    chain_floor = None
    if B == 1 and kernels:
        log("bench: streaming bursts with the layer kernels' bytes")
        names1 = list(kernels)
        bf = burst_floor(torch, qem, dev, [kernels[n]["algorithmic_bytes"] for n in names1])
        if bf is not None:
            chain_floor = {"three_bursts_us_per_layer": bf[0],
                           "burst_alone_us": {n: t for n, t in zip(names1, bf[1])},
                           "kernel": "fmoe_read_xor (each thread's loads requested at once: one burst per launch)",
                           "layer_us": round(us_layer, 3)}

    # ---- parity of layer 0, step 0 against the oracle, and the oracle's CPU time
    parity, cpu = None, None
    need_oracle = B == 1 and (not a.no_verify or not a.no_cpu_baseline)
    if need_oracle:
        import oracle
        R0 = synth.router(a.seed, 0, E, H)
        g0 = synth.shared_gate(a.seed, 0, H)
        h0 = h0_host[0][0].astype(np.float64)
        budget = 0.0 if a.no_cpu_baseline else a.cpu_seconds
        log(f"bench: oracle on layer 0 ({budget:.0f} s budget)")
        t_layer, reps, t_total, (o_out, o_idx, o_w, _) = cpu_baseline(a, synth, oracle, R0, g0, h0, budget)
        if not a.no_cpu_baseline:
            n_threads = oracle.get_threads()
            oracle.set_threads(1)
            t1, reps1, t_total1, _ = cpu_baseline(a, synth, oracle, R0, g0, h0, budget / 2)
            oracle.set_threads(n_threads)
            cpu = {"value": round(t_layer * 1e6, 1), "unit": "us/layer", "cores": n_threads,
                   "host_threads": host_threads(),
                   "value_1core": round(t1 * 1e6, 1), "cpu_model": cpu_model(),
                   "kind": "oracle",
                   "sample": f"fp64 oracle, one MoE layer (512-expert router, softmax top-{K}, {K} routed + shared "
                             f"SwiGLU experts, q{bits}) for one token, run {reps}x in {t_total:.1f} s; "
                             f"expert generation excluded"}
        if not a.no_verify:
            h_all = torch.empty((n_layers, 1, H), dtype=torch.float32, device=dev)
            h_in.copy_(h0_all[0])
            qem.fmoe_moe_stack(layers, h_in, h_out=h_out, h_all=h_all, topk_idx=idx, ws=ws, c_layers=c_layers)
            torch.cuda.synchronize()
            y = h_all[0, 0].cpu().numpy().astype(np.float64)
            d = y - o_out
            parity = {"layer": 0, "step": 0,
                      "routing_exact": bool(list(idx[0, 0].cpu().numpy()) == list(o_idx)),
                      "max_rel": float(np.max(np.abs(d)) / np.max(np.abs(o_out))),
                      "l2_rel": float(np.linalg.norm(d) / np.linalg.norm(o_out))}
            parity["pass"] = bool(parity["routing_exact"] and parity["max_rel"] <= 2e-3 and parity["l2_rel"] <= 1e-4)
            # near-ties: gaps among the oracle's top K+1 logits below the fp32 rounding
            # allowance 1e-5 * sum_i |R_ei x_i| of the two logits
            x0 = oracle.rms_scale(h0)
            lg = oracle.router_logits(R0, x0)
            tau = 1e-5 * np.abs(R0.astype(np.float64) * x0[None, :]).sum(axis=1)
            order = np.argsort(-lg, kind="stable")
            parity["near_ties"] = int(sum(lg[order[j]] - lg[order[j + 1]] < max(tau[order[j]], tau[order[j + 1]])
                                          for j in range(K)))

    # the layer's floor on this GPU: its weight bytes streamed at the measured read rate,
    # plus one empty-kernel launch per kernel of the layer
    floor = None
    if ceiling and gap is not None:
        n_k = kernels_per_layer(B, K)
        stream_us = w_bytes_layer / (ceiling["GBps"] * 1e3)
        floor = {"stream_at_read_ceiling_us": round(stream_us, 3), "launch_gaps_us": round(n_k * gap, 3),
                 "total_us": round(stream_us + n_k * gap, 3)}
    rec = {
        "metric": f"µs per MoE layer (top-{K} + shared, {bits}-bit, B={B}) and weight GB/s vs HBM peak",
        "value": round(us_layer, 4),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"u{bits} codes, bf16 scale/bias; gate/up as exact int4 dot products with x in per-64-group "
                  f"block fixed point (2^-22 of the group max); router, down and combine fp32" if B == 1 else
                  f"u{bits} codes, bf16 scale/bias; experts as exact int8 MFMA with x and h in per-64-group block "
                  f"fixed point (2^-22 of the group max); router fp32"),
        "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        "config": {"workload": f"moe_stack_q{bits}_B{B}", "layers": n_layers, "batch": B, "experts": E,
                   "top_k": K, "hidden": H, "inter": I, "group": 64, "graph": graph is not None,
                   "seed": a.seed},
        "us_per_layer_p10_p50_p90": spread,
        "kernels_per_layer": kernels_per_layer(B, K),
        "floor_us": floor,
        "chain_floor": chain_floor,
        "weight_GBps": round(weight_gbps, 1),
        "frac_hbm_peak": round(weight_gbps / HBM_PEAK_GBPS, 4),
        "read_ceiling_GBps": ceiling,
        "frac_read_ceiling": round(weight_gbps / ceiling["GBps"], 4) if ceiling else None,
        "empty_kernel_gap_us": gap,
        "algorithmic_bytes_per_layer": int(w_bytes_layer + act_bytes_layer),
        "distinct_routed_experts_per_layer": round(d_mean, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "parity": parity,
        "versions": versions(torch),
    }
    print(json.dumps(rec, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
