"""Shared helpers for the GPU tests: build device-resident weights from the seeded
generator (host pack for small cases, device generator + device pack for the
multi-GB banks), and compare GPU results with the oracle to the acceptance bar:
max-relative error (norm-wise, max|d| / max|ref|) <= 2e-3 and L2-relative error
per token <= 1e-4; routing indices identical; routing weights within 1e-5."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import quantized_expert_matvec_amd as qem

MAX_REL = 2e-3
L2_REL = 1e-4
W_REL = 1e-5


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    mx = np.abs(d).max() / max(np.abs(ref).max(), 1e-300)
    l2 = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    return mx, l2


def assert_close(got, ref, what=""):
    mx, l2 = errors(got, ref)
    print(f"  {what}: max-rel {mx:.3e}  l2-rel {l2:.3e}", flush=True)
    assert mx <= MAX_REL and l2 <= L2_REL, (what, mx, l2)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host_qmat(bits, q, dev):
    blob = qem.fmoe_pack_qmat(bits, q.codes, q.scale, q.bias)
    return qem.QMat(to_dev(blob, dev), q.rows, q.cols, bits)


def host_expert(bits, e, dev):
    blob = qem.fmoe_pack_expert(bits, e["gate"], e["up"], e["down"])
    return qem.Expert(to_dev(blob, dev), e["gate"].cols, e["gate"].rows, bits)


class DeviceFiller:
    """Generates canonical codes/scale/bias on the device (bit-identical to the host
    generator) and packs them with the library's device packer."""

    def __init__(self, hidden, inter, dev):
        self.hidden, self.inter, self.dev = hidden, inter, dev
        n = hidden * inter
        self.codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(3)]
        self.scale = [torch.empty(n // 64, dtype=torch.int16, device=dev) for _ in range(3)]
        self.bias = [torch.empty(n // 64, dtype=torch.int16, device=dev) for _ in range(3)]

    def expert(self, seed, layer, expert_id, bits, blob_out):
        H, I = self.hidden, self.inter
        shapes = [(synth.T_GATE, I, H), (synth.T_UP, I, H), (synth.T_DOWN, H, I)]
        for j, (t, r, c) in enumerate(shapes):
            synth.dev_qmat(seed, layer, expert_id, t, bits, r, c, self.codes[j], self.scale[j], self.bias[j],
                           torch.cuda.current_stream().cuda_stream)
        qem.fmoe_pack_expert_device(bits, H, I, self.codes, self.scale, self.bias, blob_out)


def device_layer(seed, layer, bits, n_exp, k, hidden, inter, dev, shared=True, filler=None, bank=None,
                 shared_blob=None):
    """A layer whose bank is generated and packed on the device."""
    eb = qem.fmoe_expert_bytes(bits, hidden, inter)
    filler = filler or DeviceFiller(hidden, inter, dev)
    if bank is None:
        bank = torch.empty(n_exp * eb, dtype=torch.uint8, device=dev)
    for e in range(n_exp):
        filler.expert(seed, layer, e, bits, bank[e * eb:(e + 1) * eb])
    sh = None
    if shared:
        sh = shared_blob if shared_blob is not None else torch.empty(eb, dtype=torch.uint8, device=dev)
        filler.expert(seed, layer, synth.SHARED_EXPERT, bits, sh)
    R = to_dev(synth.router(seed, layer, n_exp, hidden), dev)
    g = to_dev(synth.shared_gate(seed, layer, hidden), dev) if shared else None
    return qem.Layer(R, g, bank, sh, n_exp, k, hidden, inter, bits)


def host_layer(seed, layer, bits, n_exp, k, hidden, inter, dev, shared=True):
    eb = qem.fmoe_expert_bytes(bits, hidden, inter)
    bank = np.empty(n_exp * eb, np.uint8)
    for e in range(n_exp):
        ex = synth.expert(seed, layer, e, bits, hidden, inter)
        bank[e * eb:(e + 1) * eb] = qem.fmoe_pack_expert(bits, ex["gate"], ex["up"], ex["down"])
    sh = None
    if shared:
        ex = synth.expert(seed, layer, synth.SHARED_EXPERT, bits, hidden, inter)
        sh = to_dev(qem.fmoe_pack_expert(bits, ex["gate"], ex["up"], ex["down"]), dev)
    R = to_dev(synth.router(seed, layer, n_exp, hidden), dev)
    g = to_dev(synth.shared_gate(seed, layer, hidden), dev) if shared else None
    return qem.Layer(R, g, to_dev(bank, dev), sh, n_exp, k, hidden, inter, bits)


class OracleLayer:
    """The oracle's view of a generated layer: regenerates only the experts it touches."""

    ZERO_SHARED = None

    def __init__(self, seed, layer, bits, n_exp, k, hidden, inter, shared=True):
        self.seed, self.layer, self.bits = seed, layer, bits
        self.n_exp, self.k, self.hidden, self.inter = n_exp, k, hidden, inter
        self.R = synth.router(seed, layer, n_exp, hidden)
        self.shared = shared
        self.g = synth.shared_gate(seed, layer, hidden) if shared else np.zeros(hidden, np.float32)
        self.cache = {}

    def expert(self, e):
        if e not in self.cache:
            self.cache[e] = synth.expert(self.seed, self.layer, e, self.bits, self.hidden, self.inter)
        return self.cache[e]

    def zero_expert(self):
        z = synth.QMat(self.bits, np.zeros((self.inter, self.hidden), np.uint8),
                       np.zeros((self.inter, self.hidden // 64), np.uint16),
                       np.zeros((self.inter, self.hidden // 64), np.uint16))
        zd = synth.QMat(self.bits, np.zeros((self.hidden, self.inter), np.uint8),
                        np.zeros((self.hidden, self.inter // 64), np.uint16),
                        np.zeros((self.hidden, self.inter // 64), np.uint16))
        return {"gate": z, "up": z, "down": zd}

    def forward(self, x, residual):
        """Returns (out, idx, w, logits) for one token."""
        logits = oracle.router_logits(self.R, x)
        idx, w, _ = oracle.route(logits, self.k)
        experts = {int(e): self.expert(int(e)) for e in idx}
        sh = self.expert(synth.SHARED_EXPERT) if self.shared else self.zero_expert()
        out, idx2, w2, sig = oracle.moe_layer(self.R, self.g, experts, sh, x, residual, self.k)
        assert list(idx2) == list(idx)
        return out, idx, w, logits


def forward_with_routing(OL, x, residual, idx):
    """The oracle's layer for one token on a given routing: the oracle's softmax
    probabilities of the chosen experts renormalised, the oracle's expert outputs,
    shared gate and combine (out = residual + sum_k w_k E_k(x) + sigma E_shared(x)).
    Used where a near-tie lets the GPU choose differently from the oracle."""
    logits = oracle.router_logits(OL.R, x)
    _, _, p = oracle.route(logits, OL.k)
    idx = [int(e) for e in idx]
    w = np.array([p[e] for e in idx], dtype=np.float64)
    w = w / w.sum()
    out = np.asarray(residual, dtype=np.float64).copy()
    for wk, e in zip(w, idx):
        out += wk * oracle.expert(OL.expert(e), x)[1]
    if OL.shared:
        out += oracle.shared_gate(OL.g, x) * oracle.expert(OL.expert(synth.SHARED_EXPERT), x)[1]
    return out, w


def near_tie(logits, R, x, k, idx_gpu):
    """True when the oracle's ranking of the top k+1 logits has a gap below the
    rounding allowance tau_e = 1e-5 * sum_i |R_ei x_i| and the GPU's choice is
    consistent with the oracle's logits up to that allowance."""
    order = np.argsort(-logits, kind="stable")
    tau = 1e-5 * np.abs(R.astype(np.float64) * np.asarray(x, np.float64)[None, :]).sum(axis=1)
    gaps = [logits[order[j]] - logits[order[j + 1]] for j in range(k)]
    taus = [max(tau[order[j]], tau[order[j + 1]]) for j in range(k)]
    tied = any(gp < t for gp, t in zip(gaps, taus))
    if not tied:
        return False
    kth = logits[order[k - 1]]
    ok = all(logits[int(e)] >= kth - 2 * tau.max() for e in idx_gpu)
    ok = ok and all(logits[int(idx_gpu[j])] >= logits[int(idx_gpu[j + 1])] - 2 * tau.max() for j in range(k - 1))
    return ok
