"""The host-memory expert tier's cache policy, on the host: fmoe_cache_plan against a
plain model of the documented rule (a hit refreshes its slot; a miss takes the first
empty slot, else the least recently used slot the call does not need, ties to the
lower slot), and its errors. The device buffer is a fake address: planning never
touches it."""
import ctypes
import random

import numpy as np
import pytest

import quantized_expert_matvec_amd as qem

A = 1 << 40  # fake, 256-B aligned device address
L = qem.lib()


def make(n_slots, n_experts=64):
    nb = qem.fmoe_cache_device_bytes(4, 512, 256, n_experts, n_slots)
    assert nb > n_slots * qem.fmoe_expert_bytes(4, 512, 256)
    h = ctypes.c_void_p()
    assert L.fmoe_cache_create(4, 512, 256, 64, n_experts, n_slots, A, nb, ctypes.byref(h)) == 0
    return h


class Model:
    """The policy as the header states it, written out plainly."""

    def __init__(self, n):
        self.key = [None] * n
        self.last = [0] * n
        self.clock = 0

    def plan(self, layer, experts):
        held = {self.key.index((layer, e)) for e in experts if (layer, e) in self.key}
        slots, miss = [], []
        for e in experts:
            k = (layer, e)
            if k in self.key:
                s = self.key.index(k)
                miss.append(0)
            else:
                empty = [s for s in range(len(self.key)) if self.key[s] is None]
                if empty:
                    s = empty[0]
                else:
                    cand = [s for s in range(len(self.key)) if s not in held]
                    s = min(cand, key=lambda s: (self.last[s], s))
                self.key[s] = k
                held.add(s)
                miss.append(1)
            self.clock += 1
            self.last[s] = self.clock
            slots.append(s)
        return slots, miss


def test_plan_fills_hits_and_evicts_lru():
    h = make(4)
    s, m = qem.fmoe_cache_plan(h, 0, [3, 7])
    assert list(s) == [0, 1] and list(m) == [1, 1]
    s, m = qem.fmoe_cache_plan(h, 0, [7, 9, 11])
    assert list(s) == [1, 2, 3] and list(m) == [0, 1, 1]
    # full: expert 3 (slot 0) is the least recently used, then 7 (slot 1)
    s, m = qem.fmoe_cache_plan(h, 0, [12])
    assert list(s) == [0] and list(m) == [1]
    # the same expert id of another layer is another key
    s, m = qem.fmoe_cache_plan(h, 1, [9])
    assert list(m) == [1] and s[0] == 1
    st = qem.fmoe_cache_get_stats(h)
    assert st["hits"] == 1 and st["misses"] == 6 and st["lookups"] == 7 and st["bytes_copied"] == 0
    qem.fmoe_cache_destroy(h)


def test_plan_never_evicts_what_the_call_needs():
    h = make(3)
    qem.fmoe_cache_plan(h, 0, [1, 2, 3])
    # 1 is the least recently used but the call needs it: 2 goes instead
    s, m = qem.fmoe_cache_plan(h, 0, [4, 1, 3])
    assert list(m) == [1, 0, 0] and s[0] == 1
    qem.fmoe_cache_destroy(h)


def test_plan_errors_change_nothing():
    h = make(2, n_experts=8)
    slots = np.empty(3, np.int32)
    miss = np.empty(3, np.int32)
    call = lambda e: L.fmoe_cache_plan(h, 0, np.array(e, np.int32).ctypes.data, len(e), slots.ctypes.data,
                                       miss.ctypes.data)
    assert call([1, 2, 3]) == 7      # more experts than slots
    assert call([1, 1]) == 5         # a repeated expert
    assert call([8]) == 5            # outside the layer's experts
    assert call([-1]) == 5
    assert qem.fmoe_cache_get_stats(h)["lookups"] == 0
    s, m = qem.fmoe_cache_plan(h, 0, [5, 6])
    assert list(m) == [1, 1]
    qem.fmoe_cache_destroy(h)


def test_cache_create_validation():
    h = ctypes.c_void_p()
    nb = qem.fmoe_cache_device_bytes(4, 512, 256, 16, 4)
    assert L.fmoe_cache_create(4, 512, 256, 64, 16, 4, A, nb - 1, ctypes.byref(h)) == 7
    assert L.fmoe_cache_create(4, 512, 256, 64, 16, 0, A, nb, ctypes.byref(h)) == 7
    assert L.fmoe_cache_create(4, 512, 256, 64, 0, 4, A, nb, ctypes.byref(h)) == 5
    assert L.fmoe_cache_create(4, 500, 256, 64, 16, 4, A, nb, ctypes.byref(h)) == 2
    assert L.fmoe_cache_create(4, 512, 256, 64, 16, 4, A + 16, nb, ctypes.byref(h)) == 3
    assert L.fmoe_cache_create(4, 512, 256, 64, 16, 4, None, nb, ctypes.byref(h)) == 1
    assert qem.fmoe_cache_device_bytes(4, 512, 256, 16, 0) == 0


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_the_policy_model(seed):
    rng = random.Random(seed)
    n_slots, n_exp = rng.choice([4, 8, 16]), 32
    h = make(n_slots, n_exp)
    model = Model(n_slots)
    for _ in range(300):
        layer = rng.randrange(3)
        n = rng.randint(1, min(n_slots, 6))
        experts = rng.sample(range(n_exp), n)
        s, m = qem.fmoe_cache_plan(h, layer, experts)
        ms, mm = model.plan(layer, experts)
        assert list(s) == ms and list(m) == mm
    st = qem.fmoe_cache_get_stats(h)
    assert st["hits"] + st["misses"] == st["lookups"]
    qem.fmoe_cache_destroy(h)
