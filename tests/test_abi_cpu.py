"""The C ABI without a GPU: the library loads and exports every function that
include/fmoe.h declares; sizes; host pack/unpack round trips and the documented
packed layout; and every validation error, each of which returns before any
device call (the arguments are fake device addresses that are never touched)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import synth
import quantized_expert_matvec_amd as qem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "fmoe.h")


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fmoe_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(qem.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding wraps every one of them under the same name
    assert all(hasattr(qem, n) for n in names)


def test_status_strings():
    for s in range(10):
        assert qem.fmoe_status_string(s) and qem.fmoe_status_string(s) != "unknown status"
    assert qem.fmoe_status_string(77) == "unknown status"


def test_sizes_match_page_facts():
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))
    mib = facts["expert_size_mb_4bit"]["value"]
    assert qem.fmoe_expert_bytes(4, facts["hidden"]["value"], 1024) == int(mib * 2 ** 20)
    assert qem.fmoe_qmat_bytes(4, 1024, 4096) == 1024 * 4096 // 2 + 1024 * 64 * 4
    assert qem.fmoe_qmat_bytes(2, 1024, 4096) == 1024 * 4096 // 4 + 1024 * 64 * 4
    assert qem.fmoe_expert_bytes(2, 4096, 1024) == 3 * (1024 * 4096 // 4 + 1024 * 64 * 4)


@pytest.mark.parametrize("args", [(3, 4096, 1024), (4, 4096, 640), (4, 100, 1024), (4, 8192, 1024), (4, 4352, 1024),
                                  (2, 4096, 128), (4, 0, 1024)])
def test_unsupported_sizes_are_zero(args):
    assert qem.fmoe_expert_bytes(*args) == 0


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("hidden,inter", [(4096, 768), (3072, 1024), (3072, 768), (1280, 2816), (256, 3840),
                                          (4096, 4096)])
def test_multiples_of_256_are_supported(bits, hidden, inter):
    """hidden and inter may be any multiple of 256 from 256 to 4096: an expert is the
    sum of its three matrices' row records (36 or 20 bytes per 64-column group), each
    region padded to 256 bytes."""
    gb = 36 if bits == 4 else 20
    up = lambda v: (v + 255) // 256 * 256
    want = up(2 * inter * (hidden // 64) * gb) + up(hidden * (inter // 64) * gb)
    assert qem.fmoe_expert_bytes(bits, hidden, inter) == want
    assert qem.fmoe_qmat_bytes(bits, 7, hidden) == up(7 * (hidden // 64) * gb)


def test_unsupported_group_is_zero():
    assert qem.fmoe_qmat_bytes(4, 16, 4096, 32) == 0
    assert qem.fmoe_qmat_bytes(4, 0, 4096) == 0


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rows,cols", [(1, 256), (37, 512), (1024, 4096), (4096, 1024), (5, 2048), (3, 768),
                                       (9, 3072), (2, 1280), (4, 3840)])
def test_pack_unpack_round_trip(bits, rows, cols):
    q = synth.qmat(3, 0, rows, synth.T_MATRIX, bits, rows, cols)
    blob = qem.fmoe_pack_qmat(bits, q.codes, q.scale, q.bias)
    assert blob.size == qem.fmoe_qmat_bytes(bits, rows, cols)
    c, s, b = qem.fmoe_unpack_qmat(bits, rows, cols, blob)
    assert np.array_equal(c, q.codes) and np.array_equal(s, q.scale) and np.array_equal(b, q.bias)


def _layout_reference(bits, codes, scale, bias):
    """The layout as include/fmoe.h describes it, written out independently with numpy."""
    rows, cols = codes.shape
    ng = cols // 64
    recs = []
    for r in range(rows):
        c = codes[r].astype(np.uint32).reshape(ng, 64)
        if bits == 4:
            halves = []
            for h in range(2):
                part = c[:, 32 * h:32 * h + 32].reshape(ng, 4, 8)       # [g][w][8 columns]
                byte = part[:, :, 0:4] | (part[:, :, 4:8] << 4)           # [g][w][k]
                halves.append(byte.astype(np.uint8).reshape(-1))
            codes_b = np.concatenate(halves)
        else:
            part = c.reshape(ng, 4, 4, 4)                                 # [g][w][q][k]
            byte = sum(part[:, :, q, :] << (2 * q) for q in range(4))     # [g][w][k]
            codes_b = byte.astype(np.uint8).reshape(-1)
        words = (scale[r].astype(np.uint32) << 16) | bias[r].astype(np.uint32)
        recs.append(np.concatenate([codes_b, words.astype("<u4").view(np.uint8)]))
    return np.concatenate(recs)


@pytest.mark.parametrize("bits", [4, 2])
def test_packed_layout_is_the_documented_one(bits):
    for cols in (512, 768, 1280):
        q = synth.qmat(9, 1, cols, synth.T_UP, bits, 6, cols)
        blob = qem.fmoe_pack_qmat(bits, q.codes, q.scale, q.bias)
        ref = _layout_reference(bits, q.codes, q.scale, q.bias)
        assert np.array_equal(blob[:ref.size], ref), cols


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_expert_interleaves_gate_and_up(bits):
    hidden, inter = 512, 256
    e = synth.expert(4, 0, 1, bits, hidden, inter)
    blob = qem.fmoe_pack_expert(bits, e["gate"], e["up"], e["down"])
    assert blob.size == qem.fmoe_expert_bytes(bits, hidden, inter)
    rb = (hidden // 64) * (36 if bits == 4 else 20)
    g1 = qem.fmoe_pack_qmat(bits, e["gate"].codes[1:2], e["gate"].scale[1:2], e["gate"].bias[1:2])
    u1 = qem.fmoe_pack_qmat(bits, e["up"].codes[1:2], e["up"].scale[1:2], e["up"].bias[1:2])
    assert np.array_equal(blob[2 * rb:3 * rb], g1[:rb]) and np.array_equal(blob[3 * rb:4 * rb], u1[:rb])
    back = qem.fmoe_unpack_expert(bits, hidden, inter, blob)
    for (c, s, b), key in zip(back, ("gate", "up", "down")):
        assert np.array_equal(c, e[key].codes) and np.array_equal(s, e[key].scale)
        assert np.array_equal(b, e[key].bias)


def test_pack_rejects_out_of_range_codes():
    q = synth.qmat(1, 0, 0, synth.T_MATRIX, 2, 4, 256)
    bad = q.codes.copy()
    bad[2, 7] = 4
    with pytest.raises(qem.FmoeError) as ei:
        qem.fmoe_pack_qmat(2, bad, q.scale, q.bias)
    assert ei.value.status == 2


# --------------------------------------------------------------------------- validation
# Fake device addresses: aligned values that are never dereferenced because each
# call below fails validation first.
A = 1 << 40          # 256-B aligned
B = A + (1 << 30)
C = A + (2 << 30)
WS = A + (3 << 30)
L = qem.lib()
NULL = None


def qm(blob=A, rows=1024, cols=4096, bits=4, group=64):
    return ctypes.byref(qem.fmoe_qmat(blob, rows, cols, bits, group))


@pytest.mark.parametrize("call,status", [
    (lambda: L.fmoe_q4_matvec(None, B, C, None), 1),
    (lambda: L.fmoe_q4_matvec(qm(blob=None), B, C, None), 1),
    (lambda: L.fmoe_q4_matvec(qm(), None, C, None), 1),
    (lambda: L.fmoe_q4_matvec(qm(bits=2), B, C, None), 4),
    (lambda: L.fmoe_q2_matvec(qm(bits=4), B, C, None), 4),
    (lambda: L.fmoe_q4_matvec(qm(cols=1000), B, C, None), 2),
    (lambda: L.fmoe_q4_matvec(qm(cols=640), B, C, None), 2),
    (lambda: L.fmoe_q4_matvec(qm(cols=8192), B, C, None), 2),
    (lambda: L.fmoe_q4_matvec(qm(rows=0), B, C, None), 2),
    (lambda: L.fmoe_q4_matvec(qm(group=32), B, C, None), 2),
    (lambda: L.fmoe_q4_matvec(qm(blob=A + 16), B, C, None), 3),
    (lambda: L.fmoe_q4_matvec(qm(), B + 4, C, None), 3),
    (lambda: L.fmoe_q4_matvec(qm(), B, B + 64, None), 9),
    (lambda: L.fmoe_qmatvec_form(qm(), B, C, 4, None), 2),
    (lambda: L.fmoe_qmatvec_form(qm(), B, C, -1, None), 2),
    (lambda: L.fmoe_qmatvec_form(None, B, C, 0, None), 1),
    (lambda: L.fmoe_qmatvec_form(qm(bits=3), B, C, 0, None), 4),
    (lambda: L.fmoe_qmatvec_form(qm(cols=1000), B, C, 1, None), 2),
    (lambda: L.fmoe_qmatvec_form(qm(), B + 4, C, 2, None), 3),
    (lambda: L.fmoe_qmatvec_form(qm(bits=2), B, B + 64, 3, None), 9),
])
def test_matvec_validation(call, status):
    assert call() == status


def ex(blob=A, hidden=4096, inter=1024, bits=4, group=64):
    return ctypes.byref(qem.fmoe_expert(blob, hidden, inter, bits, group))


def test_expert_validation():
    need = L.fmoe_expert_workspace_bytes(ex())
    assert need == 4096
    assert L.fmoe_expert_ffn(ex(), B, C, WS, need - 1, None) == 7
    assert L.fmoe_expert_ffn(ex(), B, C, None, need, None) == 7
    assert L.fmoe_expert_ffn(ex(bits=3), B, C, WS, need, None) == 4
    assert L.fmoe_expert_ffn(ex(inter=100), B, C, WS, need, None) == 2
    assert L.fmoe_expert_ffn(ex(), B, B, WS, need, None) == 9
    assert L.fmoe_expert_ffn(ex(), B, C, C, need, None) == 9
    assert L.fmoe_expert_ffn(ex(), B, C, WS + 16, need, None) == 3


def test_expert_form_validation():
    need = L.fmoe_expert_workspace_bytes(ex())
    call = lambda form=0, e=None, x=B, out=C, ws=WS, nb=need: L.fmoe_expert_ffn_form(e or ex(), x, out, ws, nb, form, None)
    assert call(form=-1) == 2 and call(form=4) == 2
    assert call(x=None) == 1 and call(out=None) == 1
    assert call(nb=need - 1) == 7 and call(ws=None) == 7
    assert call(e=ex(bits=3)) == 4
    assert call(e=ex(inter=100)) == 2
    assert call(out=B) == 9
    assert call(ws=WS + 16) == 3


def lay(**kw):
    d = dict(router=A, shared_gate=B, bank=C, shared=WS + (1 << 29), n_experts=512, top_k=4, hidden=4096,
             inter=1024, bits=4, group=64)
    d.update(kw)
    return qem.fmoe_layer(*d.values())


X, RES, OUT, WSL = A + (5 << 30), A + (6 << 30), A + (7 << 30), A + (8 << 30)


def test_layer_validation():
    L0 = lay()
    need = L.fmoe_workspace_bytes(ctypes.byref(L0), 1)
    assert need > 0
    call = lambda Lx, n=1, x=X, r=RES, o=OUT, i=None, w=None, ws=WSL, nb=need: L.fmoe_moe_layer(
        ctypes.byref(Lx), n, x, r, o, i, w, ws, nb, None)
    assert call(lay(router=None)) == 1
    assert call(lay(bank=None)) == 1
    assert call(lay(shared_gate=None)) == 1          # a shared expert needs its gate vector
    assert call(lay(top_k=0)) == 5
    assert call(lay(top_k=17)) == 5
    assert call(lay(n_experts=3)) == 5
    assert call(lay(n_experts=2000)) == 5
    assert call(lay(bits=8)) == 4
    assert call(lay(hidden=3000)) == 2
    assert call(L0, n=0) == 6
    assert call(L0, n=257) == 6
    assert call(L0, nb=need - 1) == 7
    assert call(L0, ws=None) == 7
    assert call(L0, x=None) == 1
    assert call(L0, o=X) == 9                          # out overlaps x
    assert call(L0, o=WSL) == 9                        # out overlaps the workspace
    assert call(L0, x=X + 8) == 3
    assert call(lay(bank=C + 64)) == 3
    # NaN-free pointer checks pass through to a launch only when everything is valid; not exercised here


def test_layer_form_validation():
    L0 = lay()
    need = L.fmoe_workspace_bytes(ctypes.byref(L0), 1)
    call = lambda Lx=L0, form=0, x=X, r=RES, o=OUT, ws=WSL, nb=need: L.fmoe_moe_layer_form(
        ctypes.byref(Lx), x, r, o, None, None, ws, nb, form, None)
    assert call(form=-1) == 2 and call(form=4) == 2
    assert call(lay(hidden=2048)) == 2                 # the form builds take hidden 4096, inter 1024
    assert call(lay(inter=512)) == 2
    L1000 = lay(n_experts=1000)
    assert call(L1000, nb=L.fmoe_workspace_bytes(ctypes.byref(L1000), 1)) == 2
    assert call(lay(top_k=2)) == 5
    assert call(lay(router=None)) == 1                 # fmoe_moe_layer's own checks
    assert call(nb=need - 1) == 7
    assert call(o=X) == 9
    assert call(x=X + 8) == 3


def test_layer_alias_validation():
    L0 = lay()
    need = L.fmoe_workspace_bytes(ctypes.byref(L0), 2)
    call = lambda x=X, r=RES, o=OUT, i=None, w=None: L.fmoe_moe_layer(
        ctypes.byref(L0), 2, x, r, o, i, w, WSL, need, None)
    IW = A + (11 << 30)
    assert call(o=RES + 16) == 9                       # out partly overlaps the residual
    assert call(r=OUT - 16) == 9
    assert call(i=RES + 64) == 9                       # routing outputs inside the residual
    assert call(w=RES + 64) == 9
    assert call(i=X + 64) == 9                         # ... inside x
    assert call(w=X) == 9
    assert call(i=OUT + 64) == 9                       # ... inside out
    assert call(i=IW, w=IW + 16) == 9                  # idx [2][4] and w overlap
    assert call(i=WSL + 256) == 9                      # ... inside the workspace


def test_stack_alias_validation():
    L0 = lay()
    arr = (qem.fmoe_layer * 2)(L0, L0)
    need = L.fmoe_stack_workspace_bytes(ctypes.byref(L0), 1)
    HA, IW = A + (11 << 30), A + (12 << 30)
    call = lambda h0=X, ho=OUT, ha=None, i=None, w=None: L.fmoe_moe_stack(
        arr, 2, 1, h0, ho, ha, i, w, 1e-6, WSL, need, None)
    assert call(i=X + 64) == 9                         # routing outputs inside h0
    assert call(w=OUT) == 9                            # ... inside h_out
    assert call(ha=HA, i=HA + 4096 * 4) == 9           # ... inside h_all (second layer's rows)
    assert call(ha=HA, w=HA) == 9
    assert call(i=IW, w=IW + 16) == 9
    assert call(ha=HA, h0=HA + 64) == 9                # h_all overlaps h0


def test_stack_validation():
    L0 = lay()
    arr = (qem.fmoe_layer * 2)(L0, lay(inter=512))
    need = L.fmoe_stack_workspace_bytes(ctypes.byref(L0), 1)
    assert need > L.fmoe_workspace_bytes(ctypes.byref(L0), 1)
    assert L.fmoe_moe_stack(arr, 2, 1, X, OUT, None, None, None, 1e-6, WSL, need, None) == 2
    arr = (qem.fmoe_layer * 2)(L0, L0)
    assert L.fmoe_moe_stack(arr, 0, 1, X, OUT, None, None, None, 1e-6, WSL, need, None) == 6
    assert L.fmoe_moe_stack(arr, 2, 1, X, OUT, None, None, None, 1e-6, WSL, need - 1, None) == 7
    assert L.fmoe_moe_stack(arr, 2, 1, None, OUT, None, None, None, 1e-6, WSL, need, None) == 1


def test_stack_trace_validation():
    L0 = lay()
    arr = (qem.fmoe_layer * 2)(L0, L0)
    need = L.fmoe_stack_workspace_bytes(ctypes.byref(L0), 1)
    TR = A + (9 << 30)
    call = lambda n_tokens=1, trace=TR, layer=1, ws_bytes=need, h0=X: L.fmoe_moe_stack_trace(
        arr, 2, n_tokens, h0, OUT, 1e-6, WSL, ws_bytes, trace, layer, None)
    assert call(trace=None) == 1
    assert call(n_tokens=0) == 6 and call(n_tokens=257) == 6
    assert call(layer=2) == 6 and call(layer=-1) == 6
    assert call(trace=TR + 4) == 3
    assert call(trace=WSL + 256) == 9
    # the stack's own checks still apply
    assert call(ws_bytes=need - 1) == 7
    assert call(h0=None) == 1


def test_read_xor_validation():
    OUTW = A + (10 << 30)
    assert L.fmoe_read_xor(A, 64, None, None) == 1
    assert L.fmoe_read_xor(None, 64, OUTW, None) == 1
    assert L.fmoe_read_xor(A, 8, OUTW, None) == 3
    assert L.fmoe_read_xor(A + 4, 64, OUTW, None) == 3
    assert L.fmoe_read_xor(A, 64, OUTW + 2, None) == 3
    assert L.fmoe_read_xor(A, 64, A + 32, None) == 9


def test_rms_validation():
    assert L.fmoe_rms_scale(None, B, 1, 4096, 1e-6, None) == 1
    assert L.fmoe_rms_scale(A, B, 0, 4096, 1e-6, None) == 6
    assert L.fmoe_rms_scale(A, B, 1, 0, 1e-6, None) == 2
    assert L.fmoe_rms_scale(A, A + 64, 1, 4096, 1e-6, None) == 9


def test_noalloc_validation():
    """The static-workspace variant validates like fmoe_moe_layer and rejects batches whose
    workspace exceeds its array before touching the device."""
    L0 = lay()
    call = lambda Lx=L0, n=1, x=X, r=RES, o=OUT: L.fmoe_moe_layer_noalloc(ctypes.byref(Lx), n, x, r, o, None, None,
                                                                          None)
    assert L.fmoe_workspace_bytes(ctypes.byref(L0), 64) > qem.NOALLOC_SCRATCH_BYTES
    assert call(n=64) == 7
    assert call(n=0) == 6
    assert call(x=None) == 1
    assert call(lay(top_k=17)) == 5
    assert call(lay(hidden=3000)) == 2
