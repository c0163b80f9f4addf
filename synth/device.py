"""Device fill with the seeded generator (the HIP twin of gen.c).

Fills torch device tensors with exactly the values the host generator gives
for the same (seed, stream, index); used to place large synthetic inputs on
the GPU without a host round trip.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_gen_dev.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is missing; build with `python -m dual_flow_transformer_amd.build`")
        L = ctypes.CDLL(_SO)
        L.synth_dev_normal_streams.restype = ctypes.c_int
        L.synth_dev_normal_streams.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int,
                                               ctypes.c_void_p]
        _lib = L
    return _lib


def normal_streams(dst, streams, n_per: int, pitch: int, seed: int, sigma: float, bf16: bool, offset_elems: int = 0):
    """dst: torch device tensor (int16 storage for bf16, float32 otherwise).
    Stream s fills n_per elements at dst[offset + s*pitch]."""
    import torch
    st = torch.from_numpy(np.asarray(streams, dtype=np.uint64).view(np.int64)).to(dst.device)
    esz = dst.element_size()
    ptr = dst.data_ptr() + offset_elems * esz
    for c0 in range(0, len(streams), 65535):
        c1 = min(len(streams), c0 + 65535)
        rc = _load().synth_dev_normal_streams(ptr + c0 * pitch * esz, c1 - c0, n_per, pitch, seed & ((1 << 64) - 1),
                                              st.data_ptr() + c0 * 8, float(sigma), int(bf16),
                                              torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"device fill failed ({rc})")
    torch.cuda.current_stream().synchronize()   # keep `st` alive until the fill ran
