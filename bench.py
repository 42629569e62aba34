"""Benchmark: µs per MoE decode layer (top-4 + shared expert, 4-bit, B=1) and weight GB/s.

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
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--verify", type=int, default=1, help="tokens checked against the oracle after timing")
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


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "requested_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import quantized_expert_matvec_amd as qem

    dev = torch.device("cuda:0")
    H, I, E, K, B, bits = a.hidden, a.inter, a.experts, a.topk, a.batch, a.bits
    eb = qem.fmoe_expert_bytes(bits, H, I)
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
    h0_all = torch.from_numpy(np.stack([synth.activations(a.seed, synth.T_H0, s, B, H) for s in range(steps)])).to(dev)
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

    def run(s):
        h_in.copy_(h0_all[s])
        if graph is not None:
            graph.replay()
        else:
            step_call()

    for s in range(a.warmup):
        run(s)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    routed = []
    ev0.record()
    for s in range(a.warmup, steps):
        run(s)
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / a.steps
    us_layer = ms_step * 1000.0 / n_layers

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
    rec = {
        "metric": "us per MoE layer (top-4 + shared, 4-bit, B=1) and weight GB/s vs HBM peak",
        "value": round(us_layer, 4),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes x fp32" if bits == 4 else "u2 codes x fp32",
        "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        "config": {"workload": f"moe_stack_q{bits}", "layers": n_layers, "batch": B, "experts": E,
                   "top_k": K, "hidden": H, "inter": I, "group": 64, "graph": graph is not None},
        "weight_GBps": round(weight_gbps, 1),
        "frac_hbm_peak": round(weight_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_layer": int(w_bytes_layer + act_bytes_layer),
        "distinct_routed_experts_per_layer": round(d_mean, 3),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
