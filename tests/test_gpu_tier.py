"""GPU parity of the host-memory expert tier: the routed expert bank in pinned host
memory, an HBM cache of fewer slots than experts, fmoe_moe_layer_tiered against the
fp64 oracle token by token, and the cache's counters against the documented policy
replayed on the routing the GPU chose."""
import numpy as np
import pytest
import torch

import synth
import quantized_expert_matvec_amd as qem
from tests._fixtures import OracleLayer, forward_with_routing, near_tie, to_dev, W_REL
from tests.test_cache_cpu import Model

pytestmark = pytest.mark.gpu


def tiered_layer(seed, layer, bits, n_exp, k, hidden, inter, dev):
    """A layer whose routed bank is a pinned host tensor (router, gate vector and shared
    expert on the device)."""
    eb = qem.fmoe_expert_bytes(bits, hidden, inter)
    bank = np.empty(n_exp * eb, np.uint8)
    for e in range(n_exp):
        ex = synth.expert(seed, layer, e, bits, hidden, inter)
        bank[e * eb:(e + 1) * eb] = qem.fmoe_pack_expert(bits, ex["gate"], ex["up"], ex["down"])
    ex = synth.expert(seed, layer, synth.SHARED_EXPERT, bits, hidden, inter)
    sh = to_dev(qem.fmoe_pack_expert(bits, ex["gate"], ex["up"], ex["down"]), dev)
    R = to_dev(synth.router(seed, layer, n_exp, hidden), dev)
    g = to_dev(synth.shared_gate(seed, layer, hidden), dev)
    host_bank = torch.from_numpy(bank).pin_memory()
    return qem.Layer(R, g, host_bank, sh, n_exp, k, hidden, inter, bits)


def run_and_check(device, cache, layer_id, L, OL, X, what, fn=qem.fmoe_moe_layer_tiered):
    B = X.shape[0]
    idx = torch.full((B, OL.k), -1, dtype=torch.int32, device=device)
    w = torch.zeros((B, OL.k), dtype=torch.float32, device=device)
    out = fn(cache, layer_id, L, to_dev(X, device), to_dev(X, device), topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    got, gi, gw = out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    for t in range(B):
        ref, ri, rw, logits = OL.forward(X[t], X[t])
        if list(gi[t]) != list(ri):
            assert near_tie(logits, OL.R, X[t], OL.k, gi[t]), (t, gi[t], ri)
            ref, rw = forward_with_routing(OL, X[t], X[t], gi[t])
        assert np.abs(gw[t] - rw).max() <= W_REL * np.abs(rw).max()
        mx = np.abs(got[t] - ref).max() / np.abs(ref).max()
        l2 = np.linalg.norm(got[t] - ref) / np.linalg.norm(ref)
        assert mx <= 2e-3 and l2 <= 1e-4, (what, t, mx, l2)
    return sorted(set(gi.ravel().tolist()))


@pytest.mark.parametrize("bits", [4, 2])
def test_tiered_layer_vs_oracle_and_policy(device, bits):
    """Two layers sharing one cache of 10 slots (32 experts each): single tokens and
    batches of 2, every output against the oracle; the hit and miss counts equal the
    policy replayed on the distinct experts each call chose."""
    hidden, inter, n_exp, k, n_slots = 1024, 512, 32, 4, 10
    print(f"tiered q{bits}", flush=True)
    layers = [tiered_layer(81, l, bits, n_exp, k, hidden, inter, device) for l in range(2)]
    OLs = [OracleLayer(81, l, bits, n_exp, k, hidden, inter) for l in range(2)]
    cache = qem.ExpertCache(bits, hidden, inter, n_exp, n_slots, device)
    model = Model(n_slots)
    hits = misses = 0
    # (layer, tokens, activation index): call 1 repeats call 0's token (all hits); the
    # batches of 2 then overflow the 10 slots and evict the least recently used
    calls = [(0, 1, 0), (0, 1, 0), (1, 1, 1), (0, 2, 2), (1, 2, 3), (1, 1, 4), (0, 1, 2), (0, 1, 5)]
    for c, (layer_id, B, xi) in enumerate(calls):
        X = synth.activations(81, synth.T_X, xi, B, hidden)
        experts = run_and_check(device, cache, layer_id, layers[layer_id], OLs[layer_id], X, f"call {c}")
        _, m = model.plan(layer_id, experts)
        misses += sum(m)
        hits += len(m) - sum(m)
        st = cache.stats()
        assert st["hits"] == hits and st["misses"] == misses, (c, st, hits, misses)
        if c == 1:
            assert sum(m) == 0 and len(m) == k
    assert st["bytes_copied"] == misses * qem.fmoe_expert_bytes(bits, hidden, inter)
    assert st["lookups"] == hits + misses
    cache.close()


def test_tiered_full_size(device):
    """The workload's layer (q4, 512 experts of 6.75 MiB in pinned host memory, hidden
    4096, inter 1024, top-4) through a 64-slot cache: three tokens, one at a time, then
    the first again (all hits)."""
    hidden, inter, n_exp, k, bits = 4096, 1024, 512, 4, 4
    L = tiered_layer(synth.SEED, 40, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 40, bits, n_exp, k, hidden, inter)
    cache = qem.ExpertCache(bits, hidden, inter, n_exp, 64, device)
    X = synth.activations(synth.SEED, synth.T_X, 9100, 3, hidden)
    for t in range(3):
        run_and_check(device, cache, 0, L, OL, X[t:t + 1], f"full size token {t}")
    before = cache.stats()
    run_and_check(device, cache, 0, L, OL, X[0:1], "full size token 0 again")
    after = cache.stats()
    assert after["misses"] == before["misses"] and after["hits"] == before["hits"] + k
    cache.close()


def test_tiered_too_many_experts_for_the_slots(device):
    """A batch whose distinct experts exceed the slots is refused after the routing."""
    hidden, inter, n_exp, k, bits = 512, 256, 16, 4, 4
    L = tiered_layer(82, 0, bits, n_exp, k, hidden, inter, device)
    cache = qem.ExpertCache(bits, hidden, inter, n_exp, 4, device)
    X = to_dev(synth.activations(82, synth.T_X, 0, 8, hidden), device)
    with pytest.raises(qem.FmoeError) as ei:
        qem.fmoe_moe_layer_tiered(cache, 0, L, X, X)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    cache.close()


# --------------------------------------------------------------------------- the policy on the GPU

@pytest.mark.parametrize("bits", [4, 2])
def test_tiered_device_equals_host_policy(device, bits):
    """The same calls through two caches, one planned on the host and one on the GPU (no
    host synchronisation): the routing equal, the outputs equal bit for bit for batches
    (the same grouped kernels) and to rounding for one token (the device-planned call
    takes the one-token kernels), the counters equal after every call, and the
    device-planned outputs against the oracle."""
    hidden, inter, n_exp, k, n_slots = 1024, 512, 32, 4, 10
    print(f"tiered device policy q{bits}", flush=True)
    layers = [tiered_layer(81, l, bits, n_exp, k, hidden, inter, device) for l in range(2)]
    OLs = [OracleLayer(81, l, bits, n_exp, k, hidden, inter) for l in range(2)]
    host = qem.ExpertCache(bits, hidden, inter, n_exp, n_slots, device)
    dev = qem.ExpertCache(bits, hidden, inter, n_exp, n_slots, device)
    calls = [(0, 1, 0), (0, 1, 0), (1, 1, 1), (0, 2, 2), (1, 2, 3), (1, 1, 4), (0, 1, 2), (0, 1, 5), (1, 2, 6)]
    for c, (layer_id, B, xi) in enumerate(calls):
        X = to_dev(synth.activations(81, synth.T_X, xi, B, hidden), device)
        ih = torch.full((B, k), -1, dtype=torch.int32, device=device)
        idv = torch.full((B, k), -1, dtype=torch.int32, device=device)
        oh = qem.fmoe_moe_layer_tiered(host, layer_id, layers[layer_id], X, X, topk_idx=ih)
        od = qem.fmoe_moe_layer_tiered_device(dev, layer_id, layers[layer_id], X, X, topk_idx=idv)
        torch.cuda.synchronize()
        assert torch.equal(ih, idv), c
        if B > 1:
            assert torch.equal(oh, od), c
        else:
            a, b = oh.cpu().numpy().astype(np.float64), od.cpu().numpy().astype(np.float64)
            assert np.abs(a - b).max() <= 1e-5 * np.abs(a).max(), c
        assert host.stats() == dev.stats(), (c, host.stats(), dev.stats())
    for B in (1, 2):
        run_and_check(device, dev, 0, layers[0], OLs[0], synth.activations(81, synth.T_X, 7, B, hidden),
                      f"device policy B={B}", fn=qem.fmoe_moe_layer_tiered_device)
    # a cache is driven by one policy
    with pytest.raises(qem.FmoeError) as ei:
        qem.fmoe_moe_layer_tiered(dev, 0, layers[0], X, X)
    assert ei.value.status == 2
    with pytest.raises(qem.FmoeError) as ei:
        qem.fmoe_moe_layer_tiered_device(host, 0, layers[0], X, X)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    host.close()
    dev.close()


def test_tiered_device_full_size(device):
    """The workload's layer (q4, 512 experts of 6.75 MiB in pinned host memory) through a
    64-slot cache planned on the GPU: three tokens, then the first again (all hits), each
    against the oracle."""
    hidden, inter, n_exp, k, bits = 4096, 1024, 512, 4, 4
    L = tiered_layer(synth.SEED, 40, bits, n_exp, k, hidden, inter, device)
    OL = OracleLayer(synth.SEED, 40, bits, n_exp, k, hidden, inter)
    cache = qem.ExpertCache(bits, hidden, inter, n_exp, 64, device)
    X = synth.activations(synth.SEED, synth.T_X, 9100, 3, hidden)
    fn = qem.fmoe_moe_layer_tiered_device
    for t in range(3):
        run_and_check(device, cache, 0, L, OL, X[t:t + 1], f"device policy, full size token {t}", fn=fn)
    before = cache.stats()
    run_and_check(device, cache, 0, L, OL, X[0:1], "device policy, full size token 0 again", fn=fn)
    after = cache.stats()
    assert after["misses"] == before["misses"] and after["hits"] == before["hits"] + k
    assert after["bytes_copied"] == after["misses"] * qem.fmoe_expert_bytes(bits, hidden, inter)
    cache.close()


def test_tiered_device_graph_replays(device):
    """Two tiered layers planned on the GPU, captured once in a HIP graph after an eager
    first call, replayed on new tokens with eager work between the replays: every replay's
    outputs and the counters equal those of the same calls made eagerly on a twin cache
    (the cache's state lives on the device and carries over from replay to replay)."""
    hidden, inter, n_exp, k, bits, n_slots = 1024, 256, 32, 4, 4, 8
    layers = [tiered_layer(83, l, bits, n_exp, k, hidden, inter, device) for l in range(2)]
    xs = [to_dev(synth.activations(83, synth.T_X, i, 1, hidden), device) for i in range(4)]
    A = qem.ExpertCache(bits, hidden, inter, n_exp, n_slots, device)
    T = qem.ExpertCache(bits, hidden, inter, n_exp, n_slots, device)
    ws = [torch.empty(qem.fmoe_tiered_workspace_bytes(layers[0], 1), dtype=torch.uint8, device=device)
          for _ in range(2)]
    x_in = torch.empty_like(xs[0])
    outs = [torch.empty_like(xs[0]) for _ in range(2)]
    refs = [torch.empty_like(xs[0]) for _ in range(2)]

    def calls(cache, x, o):
        for l in range(2):
            qem.fmoe_moe_layer_tiered_device(cache, l, layers[l], x, x, out=o[l], ws=ws[l])

    x_in.copy_(xs[0])
    calls(A, x_in, outs)  # eager: initialises A's state
    calls(T, xs[0], refs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(A, x_in, outs)
    for r in (1, 2, 1, 3):
        for o in outs:
            o.fill_(float("nan"))
        x_in.copy_(xs[r])
        g.replay()
        torch.cuda.synchronize()
        calls(T, xs[r], refs)
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(outs[l], refs[l]), (r, l)
        assert A.stats() == T.stats(), (r, A.stats(), T.stats())
    del g
    A.close()
    T.close()
