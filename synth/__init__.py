"""Seeded synthetic inputs for the DFlash hot path (test and benchmark
infrastructure; no drafter arithmetic lives here).

The generator is counter-based (SplitMix64 -> Box-Muller, see synth.c), so a
tensor is a pure function of (seed, tensor name, element index).  Tensor
names map to 64-bit stream ids through FNV-1a.

`configs` describes the five drafter shapes that parity tests and the
benchmark run; `recipes` turns a shape into weights, hidden states, context
caches and planted verification inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
# DFLASH_SYNTH_LIB points the loader at another build (the sanitizer test's)
_LIB = os.environ.get("DFLASH_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
_lib = None
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile libsynth.so next to its source (gcc, OpenMP); with sanitize, an
    AddressSanitizer + UndefinedBehaviorSanitizer build at `out`."""
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared"] +
                              (SANITIZE if sanitize else []) + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
        lib.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, i64, vp]
        lib.synth_uniform_f64.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_plant_target.argtypes = [u64, u64, i32, i32, i32, vp, vp, dbl, i32, vp]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_uniform_int,
                  lib.synth_uniform_f64, lib.synth_plant_target):
            f.restype = None
        _lib = lib
    return _lib


def stream_id(name: str) -> int:
    """FNV-1a 64-bit hash of a tensor name."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


class Gen:
    """All draws for one seed.  dtype 'bf16' returns uint16 bit patterns."""

    def __init__(self, seed: int):
        self.seed = int(seed)

    def normal(self, name, shape, std=1.0, mean=0.0, dtype="f32", offset=0):
        lib = _load()
        shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
        n = int(np.prod(shape)) if shape else 1
        if dtype == "bf16":
            out = np.empty(shape, dtype=np.uint16)
            lib.synth_normal_bf16(self.seed, stream_id(name), offset, n, mean, std, _ptr(out))
        elif dtype == "f32":
            out = np.empty(shape, dtype=np.float32)
            lib.synth_normal_f32(self.seed, stream_id(name), offset, n, mean, std, _ptr(out))
        else:
            raise ValueError(dtype)
        return out

    def uniform_int(self, name, n, lo, hi, offset=0):
        out = np.empty(int(n), dtype=np.int64)
        _load().synth_uniform_int(self.seed, stream_id(name), offset, int(n), int(lo), int(hi),
                                  _ptr(out))
        return out

    def uniform(self, name, n, offset=0):
        out = np.empty(int(n), dtype=np.float64)
        _load().synth_uniform_f64(self.seed, stream_id(name), offset, int(n), _ptr(out))
        return out

    def plant_target(self, name, blocks, tau_star, vocab, dtype="f32", margin=1.0):
        """Target scores [n_seq][gamma][vocab] whose greedy verification of
        `blocks` [n_seq][gamma] accepts exactly tau_star[s] tokens."""
        blocks = np.ascontiguousarray(blocks, dtype=np.int32)
        tau_star = np.ascontiguousarray(tau_star, dtype=np.int32)
        n_seq, gamma = blocks.shape
        assert tau_star.shape == (n_seq,)
        assert np.all(tau_star >= 1) and np.all(tau_star <= gamma)
        np_dt = np.uint16 if dtype == "bf16" else np.float32
        out = np.empty((n_seq, gamma, vocab), dtype=np_dt)
        _load().synth_plant_target(self.seed, stream_id(name), n_seq, gamma, vocab,
                                   _ptr(blocks), _ptr(tau_star), float(margin),
                                   1 if dtype == "bf16" else 0, _ptr(out))
        return out
