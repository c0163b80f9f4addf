"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package draws inputs only: it holds none of the Dual-Flow arithmetic.
Every element is a pure function of (seed, stream id, index), computed by the
counter-based generator in ``gen.c`` (host) and its bit-identical device twin
in ``gen_dev.hip``. The oracle takes its inputs from the host generator; the
GPU path may fill device memory with the device twin, and tests check that the
two agree bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_gen.so")
_lib = None

M64 = (1 << 64) - 1
G64 = 0x9E3779B97F4A7C15


def build_host(force: bool = False) -> str:
    """Compile gen.c into _gen.so with gcc + OpenMP."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build_host()
        lib = ctypes.CDLL(_SO)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_words.argtypes = [vp, i64, u64, i64]
        lib.synth_normal_f32.argtypes = [vp, i64, u64, u64, i64, dbl]
        lib.synth_normal_bf16.argtypes = [vp, i64, u64, u64, i64, dbl]
        lib.synth_normal_bf16_streams.argtypes = [vp, i64, i64, i64, u64, vp, dbl]
        lib.synth_normal_f32_streams.argtypes = [vp, i64, i64, i64, u64, vp, dbl]
        lib.synth_uniform_i32.argtypes = [vp, i64, u64, u64, i64, ctypes.c_int32, ctypes.c_int32]
        _lib = lib
    return _lib


def _mix64(z: int) -> int:
    z &= M64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M64
    z ^= z >> 31
    return z


def stream_id(name: str, *idx: int) -> int:
    """64-bit stream id of a named tensor (FNV-1a of the name, then each index
    folded in through the SplitMix64 finaliser)."""
    h = 0xCBF29CE484222325
    for ch in name.encode():
        h ^= ch
        h = (h * 0x100000001B3) & M64
    for i in idx:
        h = _mix64(h ^ (((int(i) + 1) * G64) & M64))
    return h


def key(seed: int, stream: int) -> int:
    return int(_load().synth_key(seed & M64, stream & M64))


def words(key_: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_words(out.ctypes.data, n, key_ & M64, offset)
    return out


def normal(shape, seed: int, stream: int, sigma: float, dtype: str = "bf16", offset: int = 0) -> np.ndarray:
    """Irwin-Hall(4) approximate N(0, sigma^2) values. dtype 'bf16' returns the
    raw uint16 bit patterns; 'f32' returns float32."""
    n = int(np.prod(shape)) if len(shape) else 1
    lib = _load()
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_normal_bf16(out.ctypes.data, n, seed & M64, stream & M64, offset, float(sigma))
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_normal_f32(out.ctypes.data, n, seed & M64, stream & M64, offset, float(sigma))
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def normal_streams(streams, n_per: int, seed: int, sigma: float, dtype: str = "bf16") -> np.ndarray:
    """One row of n_per values per stream id: returns [len(streams), n_per]."""
    st = np.ascontiguousarray(np.asarray(streams, dtype=np.uint64))
    ns = st.shape[0]
    lib = _load()
    if dtype == "bf16":
        out = np.empty((ns, n_per), dtype=np.uint16)
        lib.synth_normal_bf16_streams(out.ctypes.data, ns, n_per, n_per, seed & M64, st.ctypes.data, float(sigma))
    elif dtype == "f32":
        out = np.empty((ns, n_per), dtype=np.float32)
        lib.synth_normal_f32_streams(out.ctypes.data, ns, n_per, n_per, seed & M64, st.ctypes.data, float(sigma))
    else:
        raise ValueError(dtype)
    return out


def uniform_int(n: int, seed: int, stream: int, lo: int, hi: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_i32(out.ctypes.data, n, seed & M64, stream & M64, offset, int(lo), int(hi))
    return out


def permutation(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    """A seeded permutation of range(n): stable argsort of n 64-bit words."""
    w = words(key(seed, stream), n, offset)
    return np.argsort(w, kind="stable").astype(np.int32)
