"""Seeded synthetic inputs for the quantized MoE expert forward.

This package draws numbers and nothing else: it holds none of the method's
arithmetic (no dequantization, no products, no routing). The fp64 oracle and the
GPU library both consume what it produces, in the canonical layout:

* codes: ``uint8 [rows, cols]``, one unsigned code in ``[0, 2**bits)`` per weight
* scale, bias: ``uint16 [rows, cols // group]`` bf16 bit patterns
* dense tensors (router, shared-expert gate vector, activations): ``float32``

Distributions follow the workloads the method is measured on (shapes from the
Flash-MoE pages: hidden 4096, 512 experts per layer, 4 routed + 1 shared, expert
intermediate 1024, 60 layers; value ranges as stated for each workload):

* 4-bit: code ~ U{0..15}, scale ~ U(0.002, 0.02), bias = -8 * scale * (1 + U(-0.1, 0.1))
* 2-bit: code ~ U{0..3},  scale ~ U(0.01, 0.05),  bias = -1.5 * scale * (1 + U(-0.1, 0.1))
* router and shared-expert gate vector ~ N(0, 0.02) (standard deviation), fp32
* activations ~ N(0, 1), fp32

The host generator is ``synth.c`` (splitmix64, counter based); ``synth_dev.hip``
is its device twin for bulk fills of resident expert banks (codes and scale/bias
only) and matches it bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SO = os.path.join(_HERE, "libsynth.so")
_DEV_SO = os.path.join(_HERE, "libsynth_dev.so")

SEED = 42
GROUP = 64

# Tensor ids inside a (layer, expert) pair. Scale/bias streams use id + SB_OFFSET.
T_GATE, T_UP, T_DOWN, T_MATRIX = 1, 2, 3, 4
SB_OFFSET = 16
T_ROUTER, T_SHARED_GATE, T_X, T_RESIDUAL, T_H0 = 32, 33, 34, 35, 36
SHARED_EXPERT = 0xFFFF  # expert id of the shared expert
STANDALONE_LAYER = 0xFFFE  # layer id used for standalone matrices / experts

# bits -> (scale lo, scale hi, bias multiplier, bias spread)
DIST = {4: (0.002, 0.02, 8.0, 0.1), 2: (0.01, 0.05, 1.5, 0.1)}


def build(verbose: bool = False) -> None:
    """Compile the host generator (gcc) and its device twin (hipcc, gfx950)."""
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", src, "-o", _HOST_SO, "-lm"]
    _run(cmd, verbose)
    dsrc = os.path.join(_HERE, "synth_dev.hip")
    dcmd = ["hipcc", "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-ffp-contract=off",
            "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            dsrc, "-o", _DEV_SO]
    _run(dcmd, verbose)


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}")


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(_HOST_SO):
            build()
        lib = ctypes.CDLL(_HOST_SO)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_void_p)
        lib.syn_word.argtypes = [u64, u64]
        lib.syn_word.restype = u64
        lib.syn_stream.argtypes = [u64, u64, u64, u64]
        lib.syn_stream.restype = u64
        lib.syn_codes.argtypes = [u64, i32, i64, vp]
        lib.syn_codes.restype = i32
        lib.syn_scale_bias.argtypes = [u64, i64, dbl, dbl, dbl, dbl, vp, vp]
        lib.syn_scale_bias.restype = i32
        lib.syn_normal.argtypes = [u64, i64, dbl, vp]
        lib.syn_normal.restype = i32
        lib.syn_uniform.argtypes = [u64, i64, dbl, dbl, vp]
        lib.syn_uniform.restype = i32
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (binds the HIP runtime torch already loaded)
        if not os.path.exists(_DEV_SO):
            build()
        lib = ctypes.CDLL(_DEV_SO)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_void_p)
        lib.synd_codes.argtypes = [u64, i32, i64, vp, vp]
        lib.synd_codes.restype = i32
        lib.synd_scale_bias.argtypes = [u64, i64, dbl, dbl, dbl, dbl, vp, vp, vp]
        lib.synd_scale_bias.restype = i32
        _dev = lib
    return _dev


# ----------------------------------------------------------------------------- primitives

def word(key: int, n: int) -> int:
    return int(_host_lib().syn_word(key, n))


def stream(seed: int, a: int, b: int, c: int) -> int:
    return int(_host_lib().syn_stream(seed, a, b, c))


def codes(key: int, bits: int, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint8)
    rc = _host_lib().syn_codes(key, bits, rows * cols, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"syn_codes: bits={bits}")
    return out


def scale_bias(key: int, bits: int, rows: int, ngroups: int):
    lo, hi, bmul, spread = DIST[bits]
    s = np.empty((rows, ngroups), dtype=np.uint16)
    b = np.empty((rows, ngroups), dtype=np.uint16)
    _host_lib().syn_scale_bias(key, rows * ngroups, lo, hi, bmul, spread, s.ctypes.data, b.ctypes.data)
    return s, b


def normal(key: int, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host_lib().syn_normal(key, n, std, out.ctypes.data)
    return out


def uniform(key: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host_lib().syn_uniform(key, n, lo, hi, out.ctypes.data)
    return out


# ----------------------------------------------------------------------------- tensors

@dataclass
class QMat:
    """One group-affine quantized matrix in canonical layout."""
    bits: int
    codes: np.ndarray  # uint8 [rows, cols]
    scale: np.ndarray  # uint16 bf16 [rows, cols // group]
    bias: np.ndarray   # uint16 bf16 [rows, cols // group]
    group: int = GROUP

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1]


def qmat(seed: int, layer: int, expert: int, tensor: int, bits: int, rows: int, cols: int,
         group: int = GROUP) -> QMat:
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    c = codes(stream(seed, layer, expert, tensor), bits, rows, cols)
    s, b = scale_bias(stream(seed, layer, expert, tensor + SB_OFFSET), bits, rows, cols // group)
    return QMat(bits, c, s, b, group)


def expert(seed: int, layer: int, expert_id: int, bits: int, hidden: int, inter: int,
           group: int = GROUP) -> dict:
    """gate and up are [inter, hidden]; down is [hidden, inter]."""
    return {
        "gate": qmat(seed, layer, expert_id, T_GATE, bits, inter, hidden, group),
        "up": qmat(seed, layer, expert_id, T_UP, bits, inter, hidden, group),
        "down": qmat(seed, layer, expert_id, T_DOWN, bits, hidden, inter, group),
    }


def router(seed: int, layer: int, n_experts: int, hidden: int) -> np.ndarray:
    return normal(stream(seed, layer, 0, T_ROUTER), n_experts * hidden, 0.02).reshape(n_experts, hidden)


def shared_gate(seed: int, layer: int, hidden: int) -> np.ndarray:
    return normal(stream(seed, layer, 0, T_SHARED_GATE), hidden, 0.02)


def activations(seed: int, tensor: int, index: int, n_tokens: int, hidden: int, std: float = 1.0):
    """[n_tokens, hidden] fp32 ~ N(0, std); `index` selects an independent draw (step, layer...)."""
    return normal(stream(seed, STANDALONE_LAYER, index, tensor), n_tokens * hidden, std).reshape(
        n_tokens, hidden)


# ----------------------------------------------------------------------------- device twin

def dev_qmat(seed: int, layer: int, expert: int, tensor: int, bits: int, rows: int, cols: int,
             codes_out, scale_out, bias_out, stream_ptr: int = 0, group: int = GROUP) -> None:
    """Fill canonical device tensors (torch, on the GPU) with the same draws as :func:`qmat`."""
    lib = _dev_lib()
    n = rows * cols
    ng = rows * (cols // group)
    if codes_out.numel() < n or scale_out.numel() < ng or bias_out.numel() < ng:
        raise ValueError("device output tensors too small")
    rc = lib.synd_codes(stream(seed, layer, expert, tensor), bits, n, codes_out.data_ptr(), stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synd_codes failed ({rc})")
    lo, hi, bmul, spread = DIST[bits]
    rc = lib.synd_scale_bias(stream(seed, layer, expert, tensor + SB_OFFSET), ng, lo, hi, bmul, spread,
                             scale_out.data_ptr(), bias_out.data_ptr(), stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synd_scale_bias failed ({rc})")
