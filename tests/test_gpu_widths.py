"""GPU parity at hidden and inter widths that are multiples of 256 but not powers of
two (a row's groups then fill only part of its lane segment): the matvec, the dequant
forms, the expert, the one-token and grouped layers and the stack, each against the
fp64 oracle on the same seeded inputs, to the same bar as tests/test_gpu_parity.py
(routing exact, max-relative 2e-3, per-token L2-relative 1e-4), and one-hot columns
bit-exact (which pins the packed layout at these widths)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_matvec_amd as qem
from tests._fixtures import (OracleLayer, assert_close, device_layer, forward_with_routing, host_expert,
                             host_layer, host_qmat, near_tie, to_dev, W_REL)

pytestmark = pytest.mark.gpu


def _x(seed, idx, n, B=1):
    return synth.activations(seed, synth.T_X, idx, B, n)


def _check(device, OL, L, X, RES, what):
    """Every token against the oracle (near-ties: against the oracle's layer on the GPU's
    routing); returns the number of near-ties."""
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
        assert np.abs(gw[t] - rw).max() <= W_REL * np.abs(rw).max(), (gw[t], rw)
        assert_close(got[t], ref, f"{what} token {t}")
    return ties


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", [(333, 768), (1024, 1280), (77, 1792), (1000, 2304), (1024, 3072),
                                       (129, 3840), (20000, 3072)])
def test_matvec_widths_vs_oracle(device, bits, rows, cols):
    print(f"matvec width q{bits} {rows}x{cols}", flush=True)
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, rows + 7, synth.T_MATRIX, bits, rows, cols)
    W = host_qmat(bits, q, device)
    x = _x(synth.SEED, rows + cols + 1, cols)[0]
    fn = qem.fmoe_q4_matvec if bits == 4 else qem.fmoe_q2_matvec
    y = fn(W, to_dev(x, device))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.qmatvec(q, x), f"q{bits} {rows}x{cols}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("cols", [768, 3072])
def test_matvec_widths_one_hot_columns(device, bits, cols):
    """x = e_j: y = code[:, j] * scale + bias exactly, for columns in the first, middle and
    last groups (the last real group is the one the lanes past the row's groups re-read)."""
    rows = 200
    q = synth.qmat(6, 1, cols, synth.T_UP, bits, rows, cols)
    W = host_qmat(bits, q, device)
    Wd = oracle.dequant(q)
    fn = qem.fmoe_q4_matvec if bits == 4 else qem.fmoe_q2_matvec
    for j in (0, 5, 63, 64, cols // 2 + 3, cols - 65, cols - 64, cols - 1):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y = fn(W, to_dev(x, device)).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, Wd[:, j]), (cols, j)


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("bits", [4, 2])
def test_matvec_forms_widths(device, form, bits):
    rows, cols = 301, 2304
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, 9, synth.T_MATRIX, bits, rows, cols)
    W = host_qmat(bits, q, device)
    x = _x(synth.SEED, 11, cols)[0]
    y = qem.fmoe_qmatvec_form(W, to_dev(x, device), form)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.qmatvec(q, x), f"form {form} q{bits} {rows}x{cols}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter", [(3072, 768), (768, 1280), (1280, 3840)])
def test_expert_widths_vs_oracle(device, bits, hidden, inter):
    print(f"expert width q{bits} {hidden}/{inter}", flush=True)
    e = synth.expert(synth.SEED, synth.STANDALONE_LAYER, 5000 + hidden + inter, bits, hidden, inter)
    E = host_expert(bits, e, device)
    x = _x(synth.SEED, 17, hidden)[0]
    out = qem.fmoe_expert_ffn(E, to_dev(x, device))
    torch.cuda.synchronize()
    _, ref = oracle.expert(e, x)
    assert_close(out.cpu().numpy(), ref, f"expert q{bits} {hidden}/{inter}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter,k", [(768, 256, 4), (256, 768, 8), (1280, 2304, 4), (2304, 1280, 2),
                                            (3840, 768, 3)])
def test_layer_widths_small(device, bits, hidden, inter, k):
    """Each padding class of the hidden and inter widths, one token at a time and as a
    grouped batch of 6 (two token blocks per expert for the shared expert)."""
    n_exp = 24
    print(f"layer width q{bits} hidden={hidden} inter={inter} k={k}", flush=True)
    L = host_layer(61, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(61, 0, bits, n_exp, k, hidden, inter)
    X = _x(61, hidden + inter + k, hidden, 6)
    RES = synth.activations(61, synth.T_RESIDUAL, k, 6, hidden)
    ties = 0
    for t in range(3):
        ties += _check(device, OL, L, X[t:t + 1], RES[t:t + 1], f"width one token {t}")
    ties += _check(device, OL, L, X, RES, "width grouped")
    print(f"  near-ties: {ties}", flush=True)


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_3072_768_vs_oracle(device, bits):
    """hidden 3072, inter 768 (another size of the model family), 256 experts + shared,
    top-4, generated and packed on the device: three tokens through the one-token kernels,
    then batches of 5 and 16 through the grouped kernels."""
    hidden, inter, n_exp, k = 3072, 768, 256, 4
    print(f"layer 3072/768 q{bits}", flush=True)
    L = device_layer(synth.SEED, 5, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 5, bits, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 7000 + bits, hidden, 16)
    RES = synth.activations(synth.SEED, synth.T_RESIDUAL, 7000 + bits, 16, hidden)
    ties = 0
    for t in range(3):
        ties += _check(device, OL, L, X[t:t + 1], RES[t:t + 1], f"3072/768 q{bits} one token {t}")
    ties += _check(device, OL, L, X[:5], RES[:5], f"3072/768 q{bits} B=5")
    ties += _check(device, OL, L, X, RES, f"3072/768 q{bits} B=16")
    print(f"  near-ties: {ties}", flush=True)
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 4])
def test_stack_3072_768_vs_oracle(device, B):
    """A 3-layer q4 stack at hidden 3072, inter 768 (RMS scaling between layers), every
    layer's output and routing against the oracle's own chain."""
    hidden, inter, n_exp, k, n_layers, bits = 3072, 768, 64, 4, 3, 4
    print(f"stack 3072/768 B={B}", flush=True)
    layers = [device_layer(62, l, bits, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    OLs = [OracleLayer(62, l, bits, n_exp, k, hidden, inter) for l in range(n_layers)]
    h0 = synth.activations(62, synth.T_H0, B, B, hidden)
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
            assert_close(ha[l, t], ref, f"stack 3072/768 layer {l} token {t}")
            h = ref
