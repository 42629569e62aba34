"""GPU parity for wider routing and larger batches: top_k up to 16 (10 is the model
family's native K) through the one-token and grouped kernels, and batches of up to
256 tokens, which the routing kernels (top-K per token, then the grouping of all
(token, choice) slots by expert) route before the grouped gate/up reads their table.
Every token against the fp64 oracle, to the bar of tests/test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_matvec_amd as qem
from tests._fixtures import (OracleLayer, assert_close, device_layer, forward_with_routing, host_layer, near_tie,
                             to_dev, W_REL)

pytestmark = pytest.mark.gpu


def _x(seed, idx, n, B=1):
    return synth.activations(seed, synth.T_X, idx, B, n)


def _check(device, OL, L, X, RES, what):
    B = X.shape[0]
    idx = torch.full((B, OL.k), -1, dtype=torch.int32, device=device)
    w = torch.zeros((B, OL.k), dtype=torch.float32, device=device)
    out = qem.fmoe_moe_layer(L, to_dev(X, device), to_dev(RES, device), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    got, gi, gw = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ties = 0
    for t in range(B):
        ref, ri, rw, logits = OL.forward(X[t], RES[t])
        if list(gi[t]) != list(ri):
            assert near_tie(logits, OL.R, X[t], OL.k, gi[t]), (t, gi[t], ri)
            ties += 1
            ref, rw = forward_with_routing(OL, X[t], RES[t], gi[t])
        assert np.abs(gw[t] - rw).max() <= W_REL * np.abs(rw).max(), (t, gw[t], rw)
        mx = np.abs(got[t] - ref).max() / np.abs(ref).max()
        l2 = np.linalg.norm(got[t] - ref) / np.linalg.norm(ref)
        assert mx <= 2e-3 and l2 <= 1e-4, (what, t, mx, l2)
    print(f"  {what}: {B} tokens checked, near-ties {ties}", flush=True)
    return ties


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter,k", [(1024, 512, 9), (1024, 512, 10), (1024, 1024, 16), (2048, 256, 10),
                                            (768, 2048, 12), (1024, 1024, 9), (512, 1024, 12), (1024, 2048, 10)])
def test_wide_topk_small(device, bits, hidden, inter, k):
    """top_k 9..16: the one-token kernels (12 or 16 slots per down lane group) token by
    token, then the same tokens grouped (routed inside the gate/up kernel)."""
    n_exp = 48
    print(f"wide top-k q{bits} hidden={hidden} inter={inter} k={k}", flush=True)
    L = host_layer(71, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(71, 0, bits, n_exp, k, hidden, inter)
    X = _x(71, k + hidden, hidden, 5)
    RES = synth.activations(71, synth.T_RESIDUAL, k, 5, hidden)
    for t in range(3):
        _check(device, OL, L, X[t:t + 1], RES[t:t + 1], f"k={k} one token {t}")
    _check(device, OL, L, X, RES, f"k={k} grouped B=5")


@pytest.mark.parametrize("bits", [4, 2])
def test_topk10_full_size(device, bits):
    """top_k 10 at the workload's size (512 experts + shared, hidden 4096, inter 1024),
    one token at a time and as a batch of 8 (80 slots)."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 10
    print(f"top-10 full size q{bits}", flush=True)
    L = device_layer(synth.SEED, 20, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 20, bits, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 8000 + bits, hidden, 8)
    RES = synth.activations(synth.SEED, synth.T_RESIDUAL, 8000 + bits, 8, hidden)
    for t in range(2):
        _check(device, OL, L, X[t:t + 1], RES[t:t + 1], f"top-10 q{bits} one token {t}")
    _check(device, OL, L, X, RES, f"top-10 q{bits} B=8")
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,k", [(65, 4), (128, 4), (256, 4), (64, 10), (200, 16)])
def test_large_batch_small_layer(device, B, k):
    """Batches past the gate/up kernel's own routing (more than 8 tokens or 512 slots):
    the routing kernels' top-K and grouping, then the grouped kernels, every token."""
    hidden, inter, n_exp, bits = 1024, 512, 64, 4
    print(f"large batch B={B} k={k}", flush=True)
    L = host_layer(72, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(72, 0, bits, n_exp, k, hidden, inter)
    X = _x(72, B * 10 + k, hidden, B)
    RES = synth.activations(72, synth.T_RESIDUAL, B, B, hidden)
    _check(device, OL, L, X, RES, f"B={B} k={k}")


def test_large_batch_forced_collisions(device):
    """256 tokens in 4 groups of identical inputs: every expert a group picks receives 64
    tokens (16 token blocks of one expert), and the results equal the one-token results."""
    hidden, inter, n_exp, k, bits = 512, 256, 32, 4, 4
    L = host_layer(73, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(73, 0, bits, n_exp, k, hidden, inter)
    base = _x(73, 1, hidden, 4)
    X = np.repeat(base, 64, axis=0)
    _check(device, OL, L, X, X, "collisions B=256")


@pytest.mark.parametrize("B", [128, 256])
def test_large_batch_full_size(device, B):
    """B = 128 and 256 decode tokens at the workload's size (q4, 512 experts + shared,
    hidden 4096, inter 1024, top-4): about 430 distinct experts at B = 256, each read once."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    print(f"large batch full size B={B}", flush=True)
    L = device_layer(synth.SEED, 30, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 30, 4, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 9000 + B, hidden, B)
    RES = synth.activations(synth.SEED, synth.T_RESIDUAL, 9000 + B, B, hidden)
    _check(device, OL, L, X, RES, f"full size B={B}")
    del L
    torch.cuda.empty_cache()


def test_large_batch_stack(device):
    """A 3-layer q4 stack at B = 128 (RMS scaling between layers): every layer's output
    and routing against the oracle's own chain, per token."""
    hidden, inter, n_exp, k, n_layers, B = 1024, 256, 64, 4, 3, 128
    layers = [host_layer(74, l, 4, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    OLs = [OracleLayer(74, l, 4, n_exp, k, hidden, inter) for l in range(n_layers)]
    h0 = synth.activations(74, synth.T_H0, 3, B, hidden)
    h_all = torch.empty((n_layers, B, hidden), dtype=torch.float32, device=device)
    idx = torch.empty((n_layers, B, k), dtype=torch.int32, device=device)
    qem.fmoe_moe_stack(layers, to_dev(h0, device), h_all=h_all, topk_idx=idx)
    torch.cuda.synchronize()
    ha, gi = h_all.cpu().numpy(), idx.cpu().numpy()
    for t in range(B):
        h = h0[t].astype(np.float64)
        for l in range(n_layers):
            x = oracle.rms_scale(h)
            ref, ri, rw, logits = OLs[l].forward(x, h)
            if list(gi[l, t]) != list(ri):
                assert near_tie(logits, OLs[l].R, x, k, gi[l, t]), (l, t)
                ref, _ = forward_with_routing(OLs[l], x, h, gi[l, t])
            mx = np.abs(ha[l, t] - ref).max() / np.abs(ref).max()
            l2 = np.linalg.norm(ha[l, t] - ref) / np.linalg.norm(ref)
            assert mx <= 2e-3 and l2 <= 1e-4, (l, t, mx, l2)
            h = ref


@pytest.mark.parametrize("n_exp,B,hidden,inter,k", [(40, 33, 768, 256, 4), (13, 35, 1280, 256, 3),
                                                    (64, 48, 2304, 512, 8), (24, 47, 256, 768, 2)])
def test_router_tiles_ragged(device, n_exp, B, hidden, inter, k):
    """From 32 tokens the router runs as 16 x 16 tiles on the matrix cores: expert and
    token counts that are not multiples of 16 (clamped tile edges), expert tile counts
    that are not multiples of 8 (the plain tile order), and several widths."""
    print(f"router tiles E={n_exp} B={B} hidden={hidden}", flush=True)
    L = host_layer(75, 0, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(75, 0, 4, n_exp, k, hidden, inter)
    X = _x(75, B + n_exp, hidden, B)
    RES = synth.activations(75, synth.T_RESIDUAL, B, B, hidden)
    _check(device, OL, L, X, RES, f"router tiles E={n_exp} B={B}")


@pytest.mark.parametrize("bits", [4, 2])
def test_router_tiles_full_size(device, bits):
    """32 and 40 tokens at the workload's size (512 experts: 32 expert tiles, placed by
    XCD), every token against the oracle."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    L = device_layer(synth.SEED, 31, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 31, bits, n_exp, k, hidden, inter)
    for B in (32, 40):
        print(f"router tiles full size q{bits} B={B}", flush=True)
        X = _x(synth.SEED, 9500 + B, hidden, B)
        RES = synth.activations(synth.SEED, synth.T_RESIDUAL, 9500 + B, B, hidden)
        _check(device, OL, L, X, RES, f"router tiles full size q{bits} B={B}")
    del L
    torch.cuda.empty_cache()
