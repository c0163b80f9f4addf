"""Helpers of the GPU parity tests (host side only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import dualflow as odf


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(arr_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr_u16).view(np.int16)).cuda()


def bits_to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype == "bf16":
        return odf.decode_bf16(a.view(np.uint16))
    return a.astype(np.float64)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def argmax_agrees(p_gpu: np.ndarray, p_ref: np.ndarray, tok_gpu: int, margin: float = 1e-6) -> bool:
    """The GPU's argmax must be the oracle's, unless the oracle's top two are
    within `margin` (then any of the near-tied ids is valid)."""
    order = np.argsort(-p_ref, kind="stable")
    best = p_ref[order[0]]
    near = set(int(i) for i in np.nonzero(p_ref >= best - margin)[0])
    return int(tok_gpu) in near and int(tok_gpu) == int(np.argmax(p_gpu))
