"""fmoe_moe_layer_noalloc (the static per-GPU workspace) against fmoe_moe_layer
(a caller's workspace), through the C ABI: the same kernels, so outputs and
routing must be identical, bit for bit, on two calls in a row, the second with
fewer tokens (the array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import quantized_expert_matvec_amd as qem
from tests._fixtures import host_layer, to_dev

pytestmark = pytest.mark.gpu


def _ref(L, X, k, dev):
    xd = to_dev(X, dev)
    idx = torch.full((X.shape[0], k), -1, dtype=torch.int32, device=dev)
    w = torch.zeros((X.shape[0], k), dtype=torch.float32, device=dev)
    out = qem.fmoe_moe_layer(L, xd, xd, topk_idx=idx, topk_w=w)
    return out, idx, w


def _noalloc(L, X, k, dev):
    xd = to_dev(X, dev)
    B = X.shape[0]
    out = torch.full((B, X.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((B, k), -1, dtype=torch.int32, device=dev)
    w = torch.zeros((B, k), dtype=torch.float32, device=dev)
    st = qem.lib().fmoe_moe_layer_noalloc(ctypes.byref(L.c()), B, xd.data_ptr(), xd.data_ptr(), out.data_ptr(),
                                         idx.data_ptr(), w.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, qem.fmoe_status_string(st)
    return out, idx, w


@pytest.mark.parametrize("bits", [4, 2])
def test_noalloc_matches_layer_two_calls(device, bits):
    hidden, inter, n_exp, k = 1024, 512, 64, 4
    print(f"noalloc bits={bits}: B=16 then B=3 then B=1", flush=True)
    L = host_layer(77, 0, bits, n_exp, k, hidden, inter, device)
    for B, seed_idx in ((16, 0), (3, 1), (1, 2)):
        X = synth.activations(77, synth.T_X, 500 + seed_idx, B, hidden)
        ro, ri, rw = _ref(L, X, k, device)
        no, ni, nw = _noalloc(L, X, k, device)
        torch.cuda.synchronize()
        assert torch.equal(ni, ri), (B, ni, ri)
        assert torch.equal(nw, rw), B
        assert torch.equal(no, ro), (B, (no - ro).abs().max().item())


def test_noalloc_rejects_oversized_batch(device):
    hidden, inter, n_exp, k = 4096, 1024, 512, 4
    L = qem.Layer(torch.empty(1, device=device), torch.empty(1, device=device), torch.empty(256, dtype=torch.uint8,
                  device=device), torch.empty(256, dtype=torch.uint8, device=device), n_exp, k, hidden, inter, 4)
    need = qem.fmoe_workspace_bytes(L, 64)
    assert need > qem.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((64, hidden), dtype=torch.float32, device=device)
    out = torch.empty_like(x)
    st = qem.lib().fmoe_moe_layer_noalloc(ctypes.byref(L.c()), 64, x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                         None, None, torch.cuda.current_stream().cuda_stream)
    assert st == 7
