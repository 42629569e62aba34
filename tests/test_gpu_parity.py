"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs. Bar: routing indices identical (near-ties of the oracle's logits
excepted, and then the GPU's choice must be consistent with them), routing
weights within 1e-5 relative, outputs within max-relative 2e-3 and per-token
L2-relative 1e-4; byte work (packing, generation) bit-exact."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_expert_matvec_amd as qem
from tests._fixtures import (DeviceFiller, OracleLayer, assert_close, device_layer, errors, forward_with_routing,
                             host_expert, host_layer, host_qmat, near_tie, to_dev, W_REL)

pytestmark = pytest.mark.gpu


def _x(seed, idx, n, B=1):
    return synth.activations(seed, synth.T_X, idx, B, n)


# --------------------------------------------------------------------------- matvec

@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", [(1024, 4096), (1, 256), (37, 512), (1000, 4096), (4096, 1024),
                                       (5, 2048), (513, 1024), (20000, 4096)])
def test_matvec_vs_oracle(device, bits, rows, cols):
    print(f"matvec bits={bits} rows={rows} cols={cols}", flush=True)
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, rows, synth.T_MATRIX, bits, rows, cols)
    W = host_qmat(bits, q, device)
    x = _x(synth.SEED, rows + cols, cols)[0]
    fn = qem.fmoe_q4_matvec if bits == 4 else qem.fmoe_q2_matvec
    y = fn(W, to_dev(x, device))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.qmatvec(q, x), f"q{bits} {rows}x{cols}")


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", [(1024, 4096), (37, 512), (5, 256), (5000, 4096), (20000, 4096)])
def test_matvec_forms_vs_oracle(device, form, bits, rows, cols):
    """Each form of the per-weight arithmetic (naive, fma recast, group-factored, table)
    against the oracle's dequantize-then-multiply, at one, two and four rows per
    wavefront."""
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, rows, synth.T_MATRIX, bits, rows, cols)
    W = host_qmat(bits, q, device)
    x = _x(synth.SEED, rows + cols, cols)[0]
    y = qem.fmoe_qmatvec_form(W, to_dev(x, device), form)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.qmatvec(q, x), f"form {form} q{bits} {rows}x{cols}")


@pytest.mark.parametrize("bits", [4, 2])
def test_matvec_one_hot_extracts_columns_exactly(device, bits):
    """x = e_j: y = code[:, j]*scale + bias, exactly (fp32 holds it); checks the packed layout."""
    rows, cols = 300, 1024
    q = synth.qmat(5, 1, 1, synth.T_UP, bits, rows, cols)
    W = host_qmat(bits, q, device)
    Wd = oracle.dequant(q)
    fn = qem.fmoe_q4_matvec if bits == 4 else qem.fmoe_q2_matvec
    for j in (0, 1, 4, 7, 31, 32, 63, 64, 100, 517, 1023):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y = fn(W, to_dev(x, device)).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, Wd[:, j]), j


def test_matvec_deterministic(device):
    q = synth.qmat(2, 0, 0, synth.T_MATRIX, 4, 1024, 4096)
    W = host_qmat(4, q, device)
    x = to_dev(_x(2, 0, 4096)[0], device)
    a = qem.fmoe_q4_matvec(W, x)
    b = qem.fmoe_q4_matvec(W, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------- packing / generation

@pytest.mark.parametrize("bits", [4, 2])
def test_device_generator_and_packer_match_host(device, bits):
    hidden, inter = 1024, 512
    f = DeviceFiller(hidden, inter, device)
    eb = qem.fmoe_expert_bytes(bits, hidden, inter)
    blob = torch.empty(eb, dtype=torch.uint8, device=device)
    f.expert(17, 3, 11, bits, blob)
    e = synth.expert(17, 3, 11, bits, hidden, inter)
    assert np.array_equal(f.codes[0].cpu().numpy().reshape(inter, hidden), e["gate"].codes)
    assert np.array_equal(f.scale[2].cpu().numpy().view(np.uint16).reshape(hidden, inter // 64), e["down"].scale)
    assert np.array_equal(f.bias[1].cpu().numpy().view(np.uint16).reshape(inter, hidden // 64), e["up"].bias)
    host = qem.fmoe_pack_expert(bits, e["gate"], e["up"], e["down"])
    assert np.array_equal(blob.cpu().numpy(), host)


# --------------------------------------------------------------------------- expert

@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter", [(4096, 1024), (512, 256), (1024, 2048), (256, 4096)])
def test_expert_ffn_vs_oracle(device, bits, hidden, inter):
    print(f"expert bits={bits} hidden={hidden} inter={inter}", flush=True)
    e = synth.expert(synth.SEED, synth.STANDALONE_LAYER, hidden + inter, bits, hidden, inter)
    E = host_expert(bits, e, device)
    x = _x(synth.SEED, 7, hidden)[0]
    out = qem.fmoe_expert_ffn(E, to_dev(x, device))
    torch.cuda.synchronize()
    _, ref = oracle.expert(e, x)
    assert_close(out.cpu().numpy(), ref, f"expert q{bits} {hidden}/{inter}")


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter", [(4096, 1024), (512, 256)])
def test_expert_ffn_forms_vs_oracle(device, form, bits, hidden, inter):
    """The whole expert with the per-weight arithmetic in each form (naive, fma recast,
    group-factored, table) against the oracle's dequantize-then-multiply expert."""
    e = synth.expert(synth.SEED, synth.STANDALONE_LAYER, hidden + inter + 1, bits, hidden, inter)
    E = host_expert(bits, e, device)
    x = _x(synth.SEED, 8, hidden)[0]
    out = qem.fmoe_expert_ffn_form(E, to_dev(x, device), form)
    torch.cuda.synchronize()
    _, ref = oracle.expert(e, x)
    assert_close(out.cpu().numpy(), ref, f"expert form {form} q{bits} {hidden}/{inter}")


# --------------------------------------------------------------------------- layer

def _check_layer(device, OL, L, X, RES, what, in_place=False, form=None):
    xd = to_dev(X, device)
    rd = to_dev(RES, device)
    B = X.shape[0]
    idx = torch.full((B, OL.k), -1, dtype=torch.int32, device=device)
    w = torch.zeros((B, OL.k), dtype=torch.float32, device=device)
    if form is not None:
        assert B == 1
        out = qem.fmoe_moe_layer_form(L, xd, rd, form, topk_idx=idx, topk_w=w)
    elif in_place:
        out = qem.fmoe_moe_layer(L, xd, rd, out=rd, topk_idx=idx, topk_w=w)
        assert out.data_ptr() == rd.data_ptr()
    else:
        out = qem.fmoe_moe_layer(L, xd, rd, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    got, gi, gw = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ties = 0
    for t in range(B):
        ref, ri, rw, logits = OL.forward(X[t], RES[t])
        if list(gi[t]) != list(ri):
            # a near-tie: the GPU's choice must be consistent with the oracle's logits, and
            # its output must match the oracle's layer evaluated on that choice
            assert near_tie(logits, OL.R, X[t], OL.k, gi[t]), (t, gi[t], ri)
            ties += 1
            ref, rw = forward_with_routing(OL, X[t], RES[t], gi[t])
        assert np.abs(gw[t] - rw).max() <= W_REL * np.abs(rw).max(), (gw[t], rw)
        assert_close(got[t], ref, f"{what} token {t}")
    return ties


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("k", [4, 1, 2, 3, 8])
def test_layer_small_vs_oracle(device, bits, k):
    hidden, inter, n_exp = 1024, 512, 64
    print(f"layer small bits={bits} k={k}", flush=True)
    L = host_layer(31, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(31, 0, bits, n_exp, k, hidden, inter)
    X = _x(31, 100 + k, hidden, 3)
    RES = synth.activations(31, synth.T_RESIDUAL, k, 3, hidden)
    assert _check_layer(device, OL, L, X, RES, f"layer q{bits} k={k}") == 0


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_without_shared_expert(device, bits):
    hidden, inter, n_exp, k = 512, 256, 16, 4
    L = host_layer(8, 0, bits, n_exp, k, hidden, inter, device, shared=False)
    OL = OracleLayer(8, 0, bits, n_exp, k, hidden, inter, shared=False)
    X = _x(8, 0, hidden, 2)
    assert _check_layer(device, OL, L, X, X, "no-shared") == 0


def test_layer_in_place_residual(device):
    hidden, inter, n_exp, k = 2048, 256, 32, 4
    L = host_layer(12, 1, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(12, 1, 4, n_exp, k, hidden, inter)
    X = _x(12, 1, hidden, 2)
    RES = synth.activations(12, synth.T_RESIDUAL, 1, 2, hidden)
    assert _check_layer(device, OL, L, X, RES, "in-place", in_place=True) == 0


def test_layer_deterministic(device):
    hidden, inter, n_exp, k = 1024, 512, 64, 4
    L = host_layer(3, 0, 4, n_exp, k, hidden, inter, device)
    xd = to_dev(_x(3, 0, hidden, 2), device)
    a = qem.fmoe_moe_layer(L, xd, xd)
    b = qem.fmoe_moe_layer(L, xd, xd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_full_size_vs_oracle(device, bits):
    """One decode layer at the workload's size: 512 experts + 1 shared, hidden 4096, inter 1024,
    top-4, residual = x (q4: 3.6 GB bank; q2: 2.0 GB), generated and packed on the device."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    print(f"layer full size bits={bits}", flush=True)
    L = device_layer(synth.SEED, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 0, bits, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 1000 + bits, hidden, 4)
    ties = _check_layer(device, OL, L, X, X, f"full q{bits}")
    print(f"  near-ties: {ties}", flush=True)
    del L
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- one token (B = 1)

def _one_token(device, OL, L, X, RES, what):
    """Every token through the one-token kernels (one call per token) against the oracle."""
    return sum(_check_layer(device, OL, L, X[t:t + 1], RES[t:t + 1], f"{what} token {t}") for t in range(X.shape[0]))


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter,k,n_exp", [(1024, 512, 4, 64), (256, 256, 1, 64), (512, 1024, 2, 32),
                                                  (2048, 256, 3, 32), (4096, 256, 8, 16), (1024, 4096, 4, 8),
                                                  (1024, 4096, 8, 16)])
def test_one_token_layer_vs_oracle(device, bits, hidden, inter, k, n_exp):
    """The one-token kernels (router + digit form of x, routing + gate/up, down + combine)
    over the supported widths, every top_k class of the down kernel and both code widths."""
    print(f"one token q{bits} hidden={hidden} inter={inter} k={k} experts={n_exp}", flush=True)
    L = host_layer(41, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(41, 0, bits, n_exp, k, hidden, inter)
    X = _x(41, 200 + k, hidden, 2)
    RES = synth.activations(41, synth.T_RESIDUAL, 200 + k, 2, hidden)
    assert _one_token(device, OL, L, X, RES, f"one token q{bits}") == 0


_FORM_LAYERS = {}


@pytest.mark.parametrize("form", [0, 1, 2, 3])
@pytest.mark.parametrize("bits", [4, 2])
def test_layer_forms_vs_oracle(device, form, bits):
    """The one-token layer with the expert projections' per-weight arithmetic in each form
    (naive, fma recast, group-factored, table; fmoe_moe_layer_form) against the oracle:
    16 experts + shared, hidden 4096, inter 1024, top-4, two tokens."""
    hidden, inter, n_exp, k = 4096, 1024, 16, 4
    if bits not in _FORM_LAYERS:
        _FORM_LAYERS[bits] = (host_layer(45, 0, bits, n_exp, k, hidden, inter, device),
                              OracleLayer(45, 0, bits, n_exp, k, hidden, inter))
    L, OL = _FORM_LAYERS[bits]
    X = _x(45, 300 + bits, hidden, 2)
    RES = synth.activations(45, synth.T_RESIDUAL, 300 + bits, 2, hidden)
    ties = sum(_check_layer(device, OL, L, X[t:t + 1], RES[t:t + 1], f"layer form {form} q{bits} token {t}", form=form)
               for t in range(2))
    assert ties == 0


@pytest.mark.parametrize("bits", [4, 2])
def test_one_token_full_size_vs_oracle(device, bits):
    """The benchmarked configuration: one decode token through the one-token kernels, 512
    experts + 1 shared, hidden 4096, inter 1024, top-4, generated and packed on the device."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    print(f"one token full size q{bits}", flush=True)
    L = device_layer(synth.SEED, 2, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 2, bits, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 3000 + bits, hidden, 3)
    RES = synth.activations(synth.SEED, synth.T_RESIDUAL, 3000 + bits, 3, hidden)
    ties = _one_token(device, OL, L, X, RES, f"one token full q{bits}")
    print(f"  near-ties: {ties}", flush=True)
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("case", ["zero_group", "all_zero", "small", "large", "one_large_per_group", "integers"])
def test_one_token_input_magnitudes(device, bits, case):
    """Inputs that stress the digit form of x (per 64-column group: integers scaled below
    2^22 from the group's largest magnitude): a group of zeros, x = 0 (every expert ties:
    the lowest indices win), x scaled by 1e-6 and 1e6, one element 1e4 times the rest in
    every group, and small integers (held exactly); then the same tokens through the grouped
    kernels. The residual is 0, so the output is the experts' contribution alone."""
    hidden, inter, n_exp, k = 1024, 512, 32, 4
    print(f"input magnitudes q{bits} {case}", flush=True)
    L = host_layer(43, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(43, 0, bits, n_exp, k, hidden, inter)
    X = _x(43, 0, hidden, 2).astype(np.float64)
    if case == "zero_group":
        X[:, 64:128] = 0.0
    elif case == "all_zero":
        X[:] = 0.0
    elif case == "small":
        X *= 1e-6
    elif case == "large":
        X *= 1e6
    elif case == "one_large_per_group":
        X[:, ::64] *= 1e4
    else:
        X = np.round(X * 8.0)
    X = X.astype(np.float32)
    RES = np.zeros_like(X)
    assert _one_token(device, OL, L, X, RES, f"magnitudes q{bits} {case}") == 0
    # the same tokens together (the grouped kernels: x as three bf16 parts)
    assert _check_layer(device, OL, L, X, RES, f"magnitudes q{bits} {case} grouped") == 0


@pytest.mark.parametrize("n_exp,k", [(5, 4), (513, 4), (1024, 8)])
def test_layer_expert_counts(device, n_exp, k):
    """Expert counts around the routing's layouts: 5 (logit rows padded to a multiple of 4,
    lanes past the end), 513 and 1024 (the most experts: 16 logits per lane, and the
    one-token kernel's routing through LDS). One token at a time, then grouped."""
    hidden, inter, bits = 256, 256, 4
    print(f"expert count {n_exp} k={k}", flush=True)
    L = device_layer(44, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(44, 0, bits, n_exp, k, hidden, inter)
    X = _x(44, n_exp, hidden, 3)
    RES = synth.activations(44, synth.T_RESIDUAL, n_exp, 3, hidden)
    ties = _one_token(device, OL, L, X, RES, f"experts {n_exp} one token")
    ties += _check_layer(device, OL, L, X, RES, f"experts {n_exp} grouped")
    assert ties == 0


def test_stack_one_token_q2(device):
    """A 4-layer 2-bit stack for one token, RMS scaling between layers, against the oracle's
    own chain."""
    hidden, inter, n_exp, k, n_layers, bits = 1024, 256, 32, 4, 4, 2
    layers = [host_layer(51, l, bits, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    OLs = [OracleLayer(51, l, bits, n_exp, k, hidden, inter) for l in range(n_layers)]
    h0 = synth.activations(51, synth.T_H0, 1, 1, hidden)
    h_all = torch.empty((n_layers, 1, hidden), dtype=torch.float32, device=device)
    idx = torch.empty((n_layers, 1, k), dtype=torch.int32, device=device)
    qem.fmoe_moe_stack(layers, to_dev(h0, device), h_all=h_all, topk_idx=idx)
    torch.cuda.synchronize()
    ha, gi = h_all.cpu().numpy(), idx.cpu().numpy()
    h = h0[0].astype(np.float64)
    for l in range(n_layers):
        ref, ri, rw, logits = OLs[l].forward(oracle.rms_scale(h), h)
        assert list(gi[l, 0]) == list(ri), l
        assert_close(ha[l, 0], ref, f"stack q2 layer {l}")
        h = ref


def test_stack_trace_equals_stack(device):
    """The stamped form of the stack gives fmoe_moe_stack's output bit for bit; every recorded
    workgroup's stamps are ordered, and each kernel of the traced layer starts after the
    previous one's workgroups end (within 0.5 µs of clock skew)."""
    hidden, inter, n_exp, k, n_layers, bits = 1024, 256, 32, 4, 3, 4
    layers = [host_layer(52, l, bits, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    h0 = to_dev(synth.activations(52, synth.T_H0, 1, 1, hidden), device)
    ref = qem.fmoe_moe_stack(layers, h0)
    tr = torch.zeros((3, qem.TRACE_BLOCKS, qem.TRACE_SLOTS), dtype=torch.int64, device=device)
    out = qem.fmoe_moe_stack_trace(layers, h0, tr, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    t = tr.cpu().numpy()
    rec = [t[kk][t[kk, :, 0] > 0] for kk in range(3)]
    for r in rec:
        assert len(r) > 0
        assert (r[:, 3] >= r[:, 0]).all()
        has = r[:, 1] > 0
        assert has.any() and ((r[has, 1] >= r[has, 0]) & (r[has, 3] >= r[has, 1])).all()
    assert (rec[1][:, 2] > 0).any()  # routed workgroups of the gate/up kernel
    for kk in range(2):
        assert rec[kk + 1][:, 0].min() + 50 >= rec[kk][:, 3].max()


@pytest.mark.parametrize("B", [4, 16])
def test_stack_trace_grouped_equals_stack(device, B):
    """The stamped form of the grouped stack gives fmoe_moe_stack's output bit for bit;
    every persistent gate/up workgroup's item ends are ordered and lie between its start
    and end, and the down kernel starts after the gate/up kernel's workgroups end."""
    hidden, inter, n_exp, k, n_layers, bits = 1024, 256, 32, 4, 3, 4
    layers = [host_layer(53, l, bits, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    h0 = to_dev(synth.activations(53, synth.T_H0, 2, B, hidden), device)
    ref = qem.fmoe_moe_stack(layers, h0)
    tr = torch.zeros((3, qem.TRACE_BLOCKS, qem.TRACE_SLOTS), dtype=torch.int64, device=device)
    out = qem.fmoe_moe_stack_trace(layers, h0, tr, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    t = tr.cpu().numpy()
    rec = [t[kk][t[kk, :, 0] > 0] for kk in range(3)]
    for kk in (0, 2):
        assert len(rec[kk]) > 0 and (rec[kk][:, 3] >= rec[kk][:, 0]).all()
    g2 = rec[1]
    assert len(g2) > 0 and (g2[:, 7] >= g2[:, 0]).all()
    for row in g2:
        ends = [v for v in row[2:7] if v > 0]
        assert ends == sorted(ends) and all(row[0] <= v <= row[7] for v in ends)
    assert (g2[:, 1] > 0).any()  # workgroups that derived the routing
    assert rec[2][:, 0].min() + 50 >= g2[:, 7].max()


def test_read_xor(device):
    """The streaming-read measurement kernel: the XOR of a buffer's 32-bit words (several
    grid-stride rounds and a ragged tail) equals numpy's; calls accumulate; an empty call
    changes nothing."""
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=4 * (2048 * 256 * 8 * 2 + 12345), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(device)
    out = torch.zeros(1, dtype=torch.int32, device=device)
    qem.fmoe_read_xor(buf, out)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(words))
    assert int(out.cpu().numpy().view(np.uint32)[0]) == want
    qem.fmoe_read_xor(None, out)  # empty kernel
    qem.fmoe_read_xor(buf, out, nbytes=16 * 1000)
    torch.cuda.synchronize()
    want ^= int(np.bitwise_xor.reduce(words[:4 * 1000]))
    assert int(out.cpu().numpy().view(np.uint32)[0]) == want


# --------------------------------------------------------------------------- grouped (B > 1)

@pytest.mark.parametrize("bits,B", [(4, 16), (2, 16), (4, 8)])
def test_grouped_layer_forced_collisions(device, bits, B):
    """B tokens in 4 groups of identical x (so every chosen expert serves several tokens and the
    staging chunks of the grouped kernels loop), on 8 experts; each token against the oracle
    (8 tokens: routed inside the gate/up kernel; 16: by the routing kernels)."""
    hidden, inter, n_exp, k = 1024, 512, 8, 4
    L = host_layer(61, 0, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(61, 0, bits, n_exp, k, hidden, inter)
    base = _x(61, 7, hidden, 4)
    X = np.ascontiguousarray(base[np.arange(B) % 4])
    RES = synth.activations(61, synth.T_RESIDUAL, 7, B, hidden)
    assert _check_layer(device, OL, L, X, RES, f"collisions q{bits} B={B}") == 0


@pytest.mark.parametrize("B,k,n_exp", [(4, 16, 32), (3, 4, 8), (2, 8, 8), (4, 1, 4)])
def test_grouped_small_batch_routing(device, B, k, n_exp):
    """Batches of at most four tokens, grouped by one wavefront inside the gate/up kernel: up
    to 64 slots (4 tokens x top-16), tokens in pairs of identical x so that chosen experts
    serve two to four slots; every token against the oracle."""
    hidden, inter = 1024, 256
    L = host_layer(65, 0, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(65, 0, 4, n_exp, k, hidden, inter)
    base = _x(65, 11, hidden, 2)
    X = np.ascontiguousarray(base[np.arange(B) % 2])
    RES = synth.activations(65, synth.T_RESIDUAL, 11, B, hidden)
    assert _check_layer(device, OL, L, X, RES, f"small batch B={B} top-{k} of {n_exp}") == 0


def test_grouped_layer_max_slots(device):
    """64 tokens with top-8 of 16 experts: 512 slots, every expert shared by many tokens;
    inter 4096 (the smallest staging chunk)."""
    hidden, inter, n_exp, k, B = 256, 4096, 16, 8, 64
    L = host_layer(62, 0, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(62, 0, 4, n_exp, k, hidden, inter)
    X = _x(62, 3, hidden, B)
    assert _check_layer(device, OL, L, X, X, "max slots") == 0


def test_grouped_layer_in_kernel_routing_max(device):
    """The largest batch the gate/up kernel routes for itself: 8 tokens with top-16 of 32
    experts (128 slots, each expert chosen by several tokens), every token against the oracle."""
    hidden, inter, n_exp, k, B = 1024, 256, 32, 16, 8
    L = host_layer(64, 0, 4, n_exp, k, hidden, inter, device)
    OL = OracleLayer(64, 0, 4, n_exp, k, hidden, inter)
    X = _x(64, 5, hidden, B)
    assert _check_layer(device, OL, L, X, X, "in-kernel routing, 128 slots") == 0


def test_grouped_equals_one_token_routing(device):
    """The grouped kernels route every token exactly as the one-token kernels do (same logits
    arithmetic), and their outputs agree to the acceptance bar."""
    hidden, inter, n_exp, k, B = 2048, 512, 64, 4, 6
    L = host_layer(63, 0, 4, n_exp, k, hidden, inter, device)
    X = _x(63, 0, hidden, B)
    xd = to_dev(X, device)
    ig = torch.empty((B, k), dtype=torch.int32, device=device)
    og = qem.fmoe_moe_layer(L, xd, xd, topk_idx=ig)
    singles, i1 = [], torch.empty((B, k), dtype=torch.int32, device=device)
    for t in range(B):
        singles.append(qem.fmoe_moe_layer(L, xd[t:t + 1], xd[t:t + 1], topk_idx=i1[t:t + 1]))
    torch.cuda.synchronize()
    assert torch.equal(ig, i1)
    for t in range(B):
        assert_close(og[t].cpu().numpy(), singles[t][0].cpu().numpy(), f"grouped vs single token {t}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("B", [4, 16])
def test_grouped_full_size(device, B, bits):
    """The batched decode workload's layer: 4 or 16 tokens (x staged once per workgroup and
    one down tile per workgroup at 4; staged per item, ahead, and two tiles at 16), 512
    experts + shared, hidden 4096, inter 1024, q4 and q2, generated and packed on the
    device; every token against the oracle."""
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    print(f"grouped full size B={B} q{bits}", flush=True)
    L = device_layer(synth.SEED, 1, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 1, bits, n_exp, k, hidden, inter)
    X = _x(synth.SEED, 2016 + B, hidden, B)
    ties = _check_layer(device, OL, L, X, X, f"full B={B} q{bits}")
    print(f"  near-ties: {ties}", flush=True)
    del L
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- RMS + stack

def test_rms_scale_vs_oracle(device):
    h = synth.activations(4, synth.T_H0, 0, 5, 4096) * 3.0
    x = qem.fmoe_rms_scale(to_dev(h, device)).cpu().numpy()
    for t in range(5):
        assert_close(x[t], oracle.rms_scale(h[t].astype(np.float64)), f"rms token {t}")


@pytest.mark.parametrize("B", [1, 4, 16])
def test_stack_vs_oracle(device, B):
    """A 4-layer stack with RMS scaling between layers, every layer's output compared with the
    oracle's own chain (the oracle never sees a GPU value)."""
    hidden, inter, n_exp, k, n_layers, bits = 1024, 256, 32, 4, 4, 4
    layers = [host_layer(50, l, bits, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    OLs = [OracleLayer(50, l, bits, n_exp, k, hidden, inter) for l in range(n_layers)]
    h0 = synth.activations(50, synth.T_H0, B, B, hidden)
    h_all = torch.empty((n_layers, B, hidden), dtype=torch.float32, device=device)
    idx = torch.empty((n_layers, B, k), dtype=torch.int32, device=device)
    h_out = qem.fmoe_moe_stack(layers, to_dev(h0, device), h_all=h_all, topk_idx=idx)
    torch.cuda.synchronize()
    ha, gi = h_all.cpu().numpy(), idx.cpu().numpy()
    assert torch.equal(h_out, h_all[-1])
    for t in range(B):
        h = h0[t].astype(np.float64)
        for l in range(n_layers):
            x = oracle.rms_scale(h)
            ref, ri, rw, logits = OLs[l].forward(x, h)
            assert list(gi[l, t]) == list(ri), (l, t)
            assert_close(ha[l, t], ref, f"stack B={B} token {t} layer {l}")
            h = ref


@pytest.mark.parametrize("B", [1, 4, 16])
def test_stack_graph_replays_equal_eager(device, B):
    """The stack captured once in a HIP graph (as the benchmark times it) and replayed on three
    inputs in turn, with eager stack calls and synchronisations between the replays: every
    replay's output and routing equal, bit for bit, those of an eager call on the same input."""
    hidden, inter, n_exp, k, n_layers = 1024, 256, 32, 4, 3
    print(f"stack graph replays B={B}", flush=True)
    layers = [host_layer(70, l, 4, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    inputs = [to_dev(synth.activations(70, synth.T_H0, 300 + 17 * r + B, B, hidden), device) for r in range(3)]
    refs, ref_idx = [], []
    for x in inputs:
        idx = torch.empty((n_layers, B, k), dtype=torch.int32, device=device)
        refs.append(qem.fmoe_moe_stack(layers, x, topk_idx=idx))
        ref_idx.append(idx)
    torch.cuda.synchronize()
    h_in = torch.empty_like(inputs[0])
    h_out = torch.empty_like(inputs[0])
    g_idx = torch.empty((n_layers, B, k), dtype=torch.int32, device=device)
    need = int(qem.lib().fmoe_stack_workspace_bytes(ctypes.byref(layers[0].c()), B))
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    h_in.copy_(inputs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qem.fmoe_moe_stack(layers, h_in, h_out=h_out, topk_idx=g_idx, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qem.fmoe_moe_stack(layers, h_in, h_out=h_out, topk_idx=g_idx, ws=ws)
    for r in (1, 0, 2, 1):
        h_out.fill_(float("nan"))
        g_idx.fill_(-1)
        h_in.copy_(inputs[r])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h_out, refs[r]), (B, r)
        assert torch.equal(g_idx, ref_idx[r]), (B, r)
        other = qem.fmoe_moe_stack(layers, inputs[(r + 1) % 3])  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, refs[(r + 1) % 3])
    del g


@pytest.mark.parametrize("B", [1, 4, 16])
def test_stack_full_size(device, B):
    """Two full-size q4 layers (512 experts + shared, hidden 4096, inter 1024, generated and
    packed on the device) as a stack, RMS scaling folded into each layer's kernels, every
    layer's output and routing against the oracle's own chain."""
    hidden, inter, n_exp, k, n_layers = 4096, 1024, 512, 4, 2
    print(f"stack full size B={B}", flush=True)
    layers = [device_layer(synth.SEED, 10 + l, 4, n_exp, k, hidden, inter, device) for l in range(n_layers)]
    OLs = [OracleLayer(synth.SEED, 10 + l, 4, n_exp, k, hidden, inter) for l in range(n_layers)]
    h0 = synth.activations(synth.SEED, synth.T_H0, 100 + B, B, hidden)
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
                # a near-tie: checked against the oracle's layer on the GPU's routing
                assert near_tie(logits, OLs[l].R, x, k, gi[l, t]), (l, t, gi[l, t], ri)
                ref, _ = forward_with_routing(OLs[l], x, h, gi[l, t])
            assert_close(ha[l, t], ref, f"full stack B={B} token {t} layer {l}")
            h = ref
    del layers
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- routing edge cases

def _steered_router(seed, n_exp, hidden, x0, rows):
    """The generated router with some rows replaced by c * u, u = x0 / (x0 . x0): for a
    token near x0 the logit of such a row is about c, far above the random rows
    (std 0.02 * sqrt(hidden)); rows given the same c are identical, an exact tie."""
    R = synth.router(seed, 0, n_exp, hidden).copy()
    u = x0.astype(np.float64) / float(np.dot(x0.astype(np.float64), x0.astype(np.float64)))
    for e, c in rows.items():
        R[e] = (c * u).astype(np.float32)
    return R


@pytest.mark.parametrize("case", ["same_lane_pair", "spread"])
def test_routing_exact_ties_and_same_lane_pairs(device, case):
    """Top-K edge cases, one-token and grouped paths, against the oracle exactly:
    an exact tie of two identical router rows (lower index first, equal weights), and
    (same_lane_pair) the two best experts among the same 8 consecutive logits, which
    the lane-maxima fast path of the top-K cannot answer alone."""
    hidden, inter, n_exp, bits = 1024, 512, 512, 4
    if case == "same_lane_pair":
        k, rows, want = 4, {5: 6.0, 6: 5.9, 100: 5.0, 300: 5.0}, [5, 6, 100, 300]
    else:
        k, rows, want = 3, {9: 6.0, 100: 5.0, 300: 5.0}, [9, 100, 300]
    print(f"routing edge case {case}", flush=True)
    x0 = _x(77, 0, hidden)[0]
    noise = _x(77, 1, hidden, 3)
    X = (x0[None, :] + 0.3 * noise).astype(np.float32)  # tokens near x0
    R = _steered_router(77, n_exp, hidden, x0, rows)
    L = device_layer(77, 0, bits, n_exp, k, hidden, inter, device)
    L = qem.Layer(to_dev(R, device), L.shared_gate, L.bank, L.shared, n_exp, k, hidden, inter, bits)
    OL = OracleLayer(77, 0, bits, n_exp, k, hidden, inter)
    OL.R = R
    for t in range(X.shape[0]):
        _, ri, rw, _ = OL.forward(X[t], X[t])
        assert list(ri) == want, (t, ri)
    # one token at a time (one-token kernels), then all tokens grouped
    for t in range(X.shape[0]):
        assert _check_layer(device, OL, L, X[t:t + 1], X[t:t + 1], f"{case} token {t} alone") == 0
    assert _check_layer(device, OL, L, X, X, f"{case} grouped") == 0
