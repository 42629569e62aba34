"""Pins for the fp64 oracle.

Each test ties one oracle function to something other than itself: exact
rational brute force on tiny inputs (``fractions.Fraction``), closed forms and
special cases, algebraic identities (the naive and the FMA-recast forms of the
dequantized product), an independent library GEMV (numpy), exact round trips,
and invariants (thread-count determinism). A plausible slip in the oracle -- a
dropped bias term, a wrong sign, a group index taken from the wrong axis, a
transposed operand, a softmax over the wrong set, a tie broken the wrong way --
fails at least one of them.

Sources: the Flash-MoE pages. The dequantized product and its FMA recast follow
"397B MoE en MacBook: Motor Flash-MoE a 4,4 t/s", section "2. Kernel de
desquantizacion optimizado con FMA", and the German page "Flash-MoE: Ausfuehren
eines 397B-Parameter-Qwen-Modells auf dem MacBook Pro mit reinem C/Metal",
section "FMA-optimierter Dequant-Kernel"; routing, SwiGLU, the fused combine and
RMS scaling follow that German page's sections "Pipeline-Leistung" and
"Metal-Compute-Shader".
"""
import itertools
import math
import struct
import subprocess
import sys
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
import synth


class Q:
    def __init__(self, codes, scale, bias, group):
        self.codes = np.ascontiguousarray(codes, dtype=np.uint8)
        self.scale = np.ascontiguousarray(scale, dtype=np.uint16)
        self.bias = np.ascontiguousarray(bias, dtype=np.uint16)
        self.group = group


def bf16_of(v: float) -> int:
    """bf16 bit pattern of a value that bf16 holds exactly (asserted)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0, f"{v} is not exactly representable in bf16"
    return u >> 16


def frac_bf16(bits: int) -> Fr:
    return Fr(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


def exact_matvec(q, x):
    """Exact rational y = sum_c (code*scale + bias) * x."""
    rows, cols = q.codes.shape
    ng = cols // q.group
    xs = [Fr(float(v)) for v in x]
    out = []
    for r in range(rows):
        acc = Fr(0)
        for c in range(cols):
            s = frac_bf16(q.scale[r, c // q.group])
            b = frac_bf16(q.bias[r, c // q.group])
            acc += (int(q.codes[r, c]) * s + b) * xs[c]
        out.append(acc)
    assert ng * q.group == cols
    return out


# --------------------------------------------------------------------------- S1 brute force

DYADIC_S = [2.0 ** -7, 3 * 2.0 ** -8, 5 * 2.0 ** -9, 2.0 ** -6]
DYADIC_B = [-(3 * 2.0 ** -5), 2.0 ** -4, -(7 * 2.0 ** -8), 0.0]


@pytest.mark.parametrize("bits,cols,group", [(2, 4, 1), (2, 4, 2), (2, 4, 4), (4, 2, 1), (4, 2, 2)])
def test_s1_every_code_pattern_exact(bits, cols, group):
    """All (2^bits)^cols code patterns (256), one per row; the oracle equals the
    exact rational value bit for bit (every fp64 step is exact on dyadic inputs)."""
    levels = 1 << bits
    pats = np.array(list(itertools.product(range(levels), repeat=cols)), dtype=np.uint8)
    rows, ng = pats.shape[0], cols // group
    scale = np.array([[bf16_of(DYADIC_S[(r + g) % 4]) for g in range(ng)] for r in range(rows)], np.uint16)
    bias = np.array([[bf16_of(DYADIC_B[(r * 3 + g) % 4]) for g in range(ng)] for r in range(rows)], np.uint16)
    x = np.array([k * 2.0 ** -4 for k in (3, -5, 7, -1)][:cols])
    q = Q(pats, scale, bias, group)
    y = oracle.qmatvec(q, x)
    ex = exact_matvec(q, x)
    for r in range(rows):
        assert Fr(float(y[r])) == ex[r], (r, pats[r])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("cols,group", [(64, 1), (64, 2), (128, 64), (64, 64)])
def test_s1_random_small_exact(bits, cols, group):
    """Generated bf16 scale/bias, x = k/16: still exact in fp64, so equality is bit for bit."""
    rows = 3
    key = synth.stream(7, bits, cols, group)
    c = synth.codes(key, bits, rows, cols)
    s, b = synth.scale_bias(key ^ 1, bits, rows, cols // group)
    rng = np.random.default_rng(cols * 10 + group + bits)
    x = rng.integers(-64, 65, size=cols) / 16.0
    q = Q(c, s, b, group)
    y = oracle.qmatvec(q, x)
    ex = exact_matvec(q, x)
    assert all(Fr(float(y[r])) == ex[r] for r in range(rows))


# --------------------------------------------------------------------------- S2 identity

def _fma_form(q, x):
    """The recast of the pages: sum_j fma(code, scale*x_j, bias*x_j), per element."""
    W_s = oracle.bf16_to_f64(q.scale)
    W_b = oracle.bf16_to_f64(q.bias)
    rows, cols = q.codes.shape
    g = np.arange(cols) // q.group
    sx = W_s[:, g] * x[None, :]
    bx = W_b[:, g] * x[None, :]
    return (q.codes.astype(np.float64) * sx + bx).sum(axis=1)


def _group_factored(q, x):
    """scale * sum_{j in g} code_j x_j + bias * sum_{j in g} x_j, per group."""
    rows, cols = q.codes.shape
    ng = cols // q.group
    cx = (q.codes.astype(np.float64) * x[None, :]).reshape(rows, ng, q.group).sum(axis=2)
    X = x.reshape(ng, q.group).sum(axis=1)
    return (oracle.bf16_to_f64(q.scale) * cx + oracle.bf16_to_f64(q.bias) * X[None, :]).sum(axis=1)


def test_s2_identity_exact_on_dyadic():
    rng = np.random.default_rng(2)
    rows, cols, group = 5, 128, 64
    c = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    s = np.array([[bf16_of(DYADIC_S[(r + g) % 4]) for g in range(2)] for r in range(rows)], np.uint16)
    b = np.array([[bf16_of(DYADIC_B[(r + 2 * g) % 4]) for g in range(2)] for r in range(rows)], np.uint16)
    x = rng.integers(-32, 33, size=cols) / 8.0
    q = Q(c, s, b, group)
    y = oracle.qmatvec(q, x)
    assert np.array_equal(y, _fma_form(q, x))
    assert np.array_equal(y, _group_factored(q, x))


@pytest.mark.parametrize("bits", [4, 2])
def test_s2_identity_on_workload_matrix(bits):
    """1024 x 4096, group 64, the workload's distributions: naive (oracle), FMA form and
    group-factored form agree to 1e-12 relative (only rounding order differs)."""
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, 0, synth.T_MATRIX, bits, 1024, 4096)
    x = synth.activations(synth.SEED, synth.T_X, 0, 1, 4096)[0].astype(np.float64)
    y = oracle.qmatvec(q, x)
    scale = np.abs(y).max()
    assert np.abs(y - _fma_form(q, x)).max() <= 1e-12 * scale
    assert np.abs(y - _group_factored(q, x)).max() <= 1e-12 * scale


# --------------------------------------------------------------------------- S3 round trips

def test_s3_bf16_decode_all_patterns():
    """Every non-NaN bf16 pattern decodes (C and numpy paths agree) and re-encodes to itself."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    dec = oracle.bf16_to_f64(pats)
    lib = oracle._L()
    for p in range(0, 65536, 97):  # the C decoder on a spread of patterns incl. signs/exponents
        v = lib.orc_bf16(p)
        assert (math.isnan(v) and math.isnan(dec[p])) or v == dec[p]
    finite = ~np.isnan(dec)
    f32 = dec[finite].astype(np.float32)
    back = (f32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(back, pats[finite])
    assert np.all((f32.view(np.uint32) & 0xFFFF) == 0)


@pytest.mark.parametrize("bits,rows,cols", [(4, 1024, 4096), (4, 4096, 1024), (2, 1024, 4096), (2, 4096, 1024)])
def test_s3_requantize_recovers_codes(bits, rows, cols):
    """dequant is exact, so code = (W - bias) / scale recovers every code (workload shapes)."""
    q = synth.qmat(synth.SEED, 3, 5, synth.T_DOWN if rows > cols else synth.T_GATE, bits, rows, cols)
    W = oracle.dequant(q)
    g = np.arange(cols) // 64
    s = oracle.bf16_to_f64(q.scale)[:, g]
    b = oracle.bf16_to_f64(q.bias)[:, g]
    rec = (W - b) / s
    assert np.array_equal(rec, np.rint(rec))
    assert np.array_equal(rec.astype(np.int64), q.codes.astype(np.int64))


# --------------------------------------------------------------------------- S4 closed forms

@pytest.fixture(scope="module")
def q4small():
    return synth.qmat(11, 1, 2, synth.T_UP, 4, 96, 256)


def test_s4_one_hot_extracts_column(q4small):
    W = oracle.dequant(q4small)
    for j in (0, 1, 63, 64, 127, 255):
        e = np.zeros(256)
        e[j] = 1.0
        assert np.array_equal(oracle.qmatvec(q4small, e), W[:, j])


def test_s4_one_hot_column_is_code_times_scale_plus_bias(q4small):
    """Column j of W read through the matvec equals code[:, j]*scale[:, j//64] + bias[:, j//64]
    evaluated with exact rationals (catches a transposed operand or a group index on the wrong axis)."""
    for j in (5, 70, 200):
        e = np.zeros(256)
        e[j] = 1.0
        y = oracle.qmatvec(q4small, e)
        for r in (0, 37, 95):
            exp = int(q4small.codes[r, j]) * frac_bf16(q4small.scale[r, j // 64]) + frac_bf16(q4small.bias[r, j // 64])
            assert Fr(float(y[r])) == exp


def test_s4_all_ones_gives_integer_code_sums(q4small):
    """x = 1: y_r = sum_g (scale_rg * sum_{j in g} code_rj + 64 * bias_rg)."""
    y = oracle.qmatvec(q4small, np.ones(256))
    csum = q4small.codes.astype(np.int64).reshape(96, 4, 64).sum(axis=2)
    for r in range(0, 96, 7):
        exp = sum(int(csum[r, g]) * frac_bf16(q4small.scale[r, g]) + 64 * frac_bf16(q4small.bias[r, g])
                  for g in range(4))
        assert Fr(float(y[r])) == exp


def test_s4_unit_scale_zero_bias_integer_matvec():
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, size=(40, 192)).astype(np.uint8)
    one, zero = bf16_of(1.0), bf16_of(0.0)
    q = Q(c, np.full((40, 3), one, np.uint16), np.full((40, 3), zero, np.uint16), 64)
    x = rng.integers(-1000, 1000, size=192)
    y = oracle.qmatvec(q, x.astype(np.float64))
    assert np.array_equal(y, (c.astype(np.int64) @ x).astype(np.float64))


@pytest.mark.parametrize("c0", [0, 3, 15])
def test_s4_bias_cancels_code(c0):
    """All codes c0 with bias = -c0*scale: W = 0, so y = 0 exactly for any x."""
    s = 2.0 ** -6
    q = Q(np.full((8, 128), c0, np.uint8), np.full((8, 2), bf16_of(s), np.uint16),
          np.full((8, 2), bf16_of(-c0 * s), np.uint16), 64)
    x = synth.activations(1, synth.T_X, 9, 1, 128)[0]
    assert np.array_equal(oracle.qmatvec(q, x), np.zeros(8))


# --------------------------------------------------------------------------- S5 library GEMV

@pytest.mark.parametrize("bits", [4, 2])
def test_s5_matches_numpy_dense_gemv(bits):
    q = synth.qmat(synth.SEED, synth.STANDALONE_LAYER, 1, synth.T_MATRIX, bits, 1024, 4096)
    x = synth.activations(synth.SEED, synth.T_X, 1, 1, 4096)[0].astype(np.float64)
    y = oracle.qmatvec(q, x)
    ref = oracle.dequant(q) @ x
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # the batched form is the per-token form
    X = synth.activations(synth.SEED, synth.T_X, 2, 3, 4096).astype(np.float64)
    Y = oracle.qmatvec(q, X)
    assert np.array_equal(Y[1], oracle.qmatvec(q, X[1]))


# --------------------------------------------------------------------------- S6 routing

def test_s6_known_ranking():
    logits = np.array([0.1, 2.0, -1.0, 1.5, 3.0, 0.0, 1.5001, -2.0])
    idx, w, p = oracle.route(logits, 4)
    assert list(idx) == [4, 1, 6, 3]
    assert abs(p.sum() - 1.0) < 1e-15
    assert np.all(np.diff(w) <= 0) and abs(w.sum() - 1.0) < 1e-15


def test_s6_ties_lower_index_first_and_equal_weights():
    logits = np.array([0.5, 1.0, 0.2, 1.0, 1.0, 1.0, 0.9])
    idx, w, _ = oracle.route(logits, 4)
    assert list(idx) == [1, 3, 4, 5]
    assert np.all(w == 0.25)
    # a tie that straddles the cut: rank 3 and rank 4 equal -> the lower index is kept
    idx, w, _ = oracle.route(np.array([3.0, 1.0, 2.0, 1.0, 0.0]), 3)
    assert list(idx) == [0, 2, 1]


def test_s6_renormalised_equals_softmax_over_chosen_logits():
    rng = np.random.default_rng(6)
    for _ in range(20):
        lg = rng.normal(0, 1.3, size=512)
        idx, w, _ = oracle.route(lg, 4)
        t = lg[idx]
        direct = np.exp(t - t.max()) / np.exp(t - t.max()).sum()
        assert np.abs(w - direct).max() <= 1e-15


def test_s6_bruteforce_subset_maximises_mass():
    rng = np.random.default_rng(60)
    for _ in range(50):
        lg = rng.normal(0, 1.0, size=8)
        idx, w, p = oracle.route(lg, 4)
        best = max(itertools.combinations(range(8), 4), key=lambda S: sum(p[list(S)]))
        assert set(idx) == set(best)
        assert list(idx) == sorted(best, key=lambda e: (-p[e], e))


def test_s6_extreme_spread_ranks_as_exact_softmax():
    """Logits thousands apart: in fp64 every probability below the largest rounds to 0,
    but the exact softmax still orders them as the logits (log-probabilities
    l_i - logsumexp(l) are finite and strictly ordered like l). The top K and their order
    follow the log-probabilities; the weights are the renormalised exact values (here 1
    and underflowing zeros)."""
    rng = np.random.default_rng(61)
    for _ in range(20):
        lg = rng.normal(0, 3e5, size=64)
        idx, w, _ = oracle.route(lg, 4)
        m = lg.max()
        logp = lg - (m + np.log(np.exp(lg - m).sum()))
        want = sorted(range(64), key=lambda e: (-logp[e], e))[:4]
        assert list(idx) == want
        t = logp[want]
        assert np.array_equal(w, np.exp(t - t.max()) / np.exp(t - t.max()).sum())
    idx, _, _ = oracle.route(np.array([0.0, -1000.0, -2000.0, -800.0, -3000.0]), 3)
    assert list(idx) == [0, 3, 1]


def test_s6_nan_logit_ranks_last():
    idx, w, _ = oracle.route(np.array([np.nan, 0.5, 2.0, 1.0]), 3)
    assert list(idx) == [2, 3, 1]
    assert np.all(np.isfinite(w)) and abs(w.sum() - 1.0) < 1e-15


# --------------------------------------------------------------------------- S7 SwiGLU

def test_s7_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for z in (41.0, 60.0, 700.0):
        assert oracle.silu(z) == z
    for z in (-41.0, -60.0, -700.0):
        assert abs(oracle.silu(z)) < 1e-15
    for z in (0.3, 1.7, 5.0, 12.5):
        assert abs(oracle.silu(-z) - (oracle.silu(z) - z)) <= 1e-15 * max(1.0, z)
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16


def test_s7_expert_is_composition_of_matvecs():
    """orc_expert = down( silu(gate x) * (up x) ), against numpy dense products of dequantized
    weights with an independent silu (tanh form: silu(z) = z * (1 + tanh(z/2)) / 2)."""
    e = synth.expert(5, 0, 1, 4, 512, 256)
    x = synth.activations(5, synth.T_X, 3, 1, 512)[0].astype(np.float64)
    h, out = oracle.expert(e, x)
    g = oracle.dequant(e["gate"]) @ x
    u = oracle.dequant(e["up"]) @ x
    h_ref = g * (1.0 + np.tanh(g / 2.0)) / 2.0 * u
    out_ref = oracle.dequant(e["down"]) @ h_ref
    assert np.abs(h - h_ref).max() <= 1e-12 * np.abs(h_ref).max()
    assert np.abs(out - out_ref).max() <= 1e-12 * np.abs(out_ref).max()


# --------------------------------------------------------------------------- S8 combine / layer

def _small_layer(seed, n_exp, hidden, inter, bits):
    R = synth.router(seed, 0, n_exp, hidden)
    g = synth.shared_gate(seed, 0, hidden)
    experts = {e: synth.expert(seed, 0, e, bits, hidden, inter) for e in range(n_exp)}
    shared = synth.expert(seed, 0, synth.SHARED_EXPERT, bits, hidden, inter)
    return R, g, experts, shared


def test_s8_sigmoid_of_zero_is_half():
    assert oracle.shared_gate(np.zeros(64, np.float32), np.ones(64)) == 0.5
    assert oracle.sigmoid(0.0) == 0.5


def test_s8_zero_weights_pass_residual_through():
    hidden, inter, n_exp = 128, 64, 8
    zero = lambda r, c: Q(np.zeros((r, c), np.uint8), np.full((r, c // 64), bf16_of(0.5), np.uint16),
                          np.zeros((r, c // 64), np.uint16), 64)
    ex = {"gate": zero(inter, hidden), "up": zero(inter, hidden), "down": zero(hidden, inter)}
    R = synth.router(1, 0, n_exp, hidden)
    g = synth.shared_gate(1, 0, hidden)
    x = synth.activations(1, synth.T_X, 0, 1, hidden)[0]
    res = synth.activations(1, synth.T_RESIDUAL, 0, 1, hidden)[0]
    out, idx, w, sig = oracle.moe_layer(R, g, {e: ex for e in range(n_exp)}, ex, x, res, 4)
    assert np.array_equal(out, res.astype(np.float64))


@pytest.mark.parametrize("bits", [4, 2])
def test_s8_layer_matches_numpy_composition(bits):
    """The whole layer against an independent numpy composition: dense GEMVs of dequantized weights,
    softmax by numpy, top-k by lexsort, sigmoid via tanh, combine as residual + sum w E + sigma E_s."""
    hidden, inter, n_exp, k = 256, 128, 16, 4
    R, g, experts, shared = _small_layer(21, n_exp, hidden, inter, bits)
    for t in range(3):
        x = synth.activations(21, synth.T_X, t, 1, hidden)[0].astype(np.float64)
        res = synth.activations(21, synth.T_RESIDUAL, t, 1, hidden)[0].astype(np.float64)
        out, idx, w, sig = oracle.moe_layer(R, g, experts, shared, x, res, k)
        lg = R.astype(np.float64) @ x
        p = np.exp(lg - lg.max())
        p /= p.sum()
        order = np.lexsort((np.arange(n_exp), -p))[:k]
        w_ref = p[order] / p[order].sum()
        assert list(idx) == list(order)
        assert np.abs(w - w_ref).max() <= 1e-14

        def E(ex):
            gg = oracle.dequant(ex["gate"]) @ x
            uu = oracle.dequant(ex["up"]) @ x
            return oracle.dequant(ex["down"]) @ (gg * (1.0 + np.tanh(gg / 2.0)) / 2.0 * uu)

        sig_ref = (1.0 + math.tanh(float(g.astype(np.float64) @ x) / 2.0)) / 2.0
        ref = res + sum(w_ref[j] * E(experts[int(order[j])]) for j in range(k)) + sig_ref * E(shared)
        assert abs(sig - sig_ref) <= 1e-15
        assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


def test_s8_single_expert_unit_weight():
    """k = 1: the chosen expert gets weight exactly 1."""
    hidden, inter, n_exp = 128, 64, 4
    R, g, experts, shared = _small_layer(3, n_exp, hidden, inter, 4)
    x = synth.activations(3, synth.T_X, 0, 1, hidden)[0].astype(np.float64)
    res = np.zeros(hidden)
    out, idx, w, sig = oracle.moe_layer(R, g, experts, shared, x, res, 1)
    assert w[0] == 1.0
    _, e_out = oracle.expert(experts[int(idx[0])], x)
    _, s_out = oracle.expert(shared, x)
    assert np.abs(out - (e_out + sig * s_out)).max() <= 1e-13 * np.abs(out).max()


# --------------------------------------------------------------------------- S9 RMS scaling

def test_s9_rms_constant_vector():
    for c in (0.5, -3.0, 1e-3):
        h = np.full(4096, c)
        x = oracle.rms_scale(h, 1e-6)
        # a serial sum of 4096 equal squares carries ~n ulp of rounding
        assert np.abs(x - c / math.sqrt(c * c + 1e-6)).max() <= 1e-12 * abs(x[0])
        assert np.all(x == x[0])


def test_s9_rms_scale_invariance():
    h = synth.activations(9, synth.T_H0, 0, 1, 4096)[0].astype(np.float64)
    x1 = oracle.rms_scale(h, 0.0)
    for a in (2.0, -0.125, 1000.0):
        xa = oracle.rms_scale(a * h, 0.0)
        assert np.abs(xa - math.copysign(1.0, a) * x1).max() <= 1e-14
    assert abs(np.mean(x1 ** 2) - 1.0) <= 1e-14


# --------------------------------------------------------------------------- S10 determinism

def test_s10_bitwise_identical_across_thread_counts():
    q = synth.qmat(synth.SEED, 2, 2, synth.T_GATE, 4, 1024, 4096)
    x = synth.activations(synth.SEED, synth.T_X, 4, 1, 4096)[0]
    before = oracle.get_threads()
    try:
        oracle.set_threads(1)
        y1 = oracle.qmatvec(q, x)
        oracle.set_threads(max(2, before))
        y8 = oracle.qmatvec(q, x)
    finally:
        oracle.set_threads(before)
    assert np.array_equal(y1, y8)


def test_forward_with_routing_reproduces_the_oracle_layer():
    """The near-tie reference of the GPU tests (the oracle's layer on a given routing)
    equals oracle.moe_layer when given the oracle's own routing, and moves by exactly one
    expert's weighted output when one chosen expert is swapped."""
    from tests._fixtures import OracleLayer, forward_with_routing
    OL = OracleLayer(5, 0, 4, 16, 4, 256, 256)
    x = synth.activations(5, synth.T_X, 3, 1, 256)[0].astype(np.float64)
    res = synth.activations(5, synth.T_RESIDUAL, 3, 1, 256)[0].astype(np.float64)
    ref, idx, w, _ = OL.forward(x, res)
    got, gw = forward_with_routing(OL, x, res, idx)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    assert np.allclose(gw, w, rtol=1e-14)
    swapped = list(idx[:-1]) + [next(e for e in range(16) if e not in idx)]
    got2, w2 = forward_with_routing(OL, x, res, swapped)
    logits = oracle.router_logits(OL.R, x)
    _, _, p = oracle.route(logits, 4)
    assert np.allclose(w2, p[swapped] / p[swapped].sum(), rtol=1e-14)
    assert not np.allclose(got2, ref)
