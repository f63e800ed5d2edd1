"""Move synthetic cases (numpy bit patterns) into torch tensors on a device.

Pure data movement: raw fp16/bf16 bits are reinterpreted, never converted.
"""
from __future__ import annotations

import numpy as np


def _t():
    import torch
    return torch


def x_tensor(x_raw: np.ndarray, x_dtype: str, device="cuda"):
    torch = _t()
    if x_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x_raw, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(x_raw).view(np.int16))
    return t.view(torch.float16 if x_dtype == "f16" else torch.bfloat16).to(device)


def words_tensor(words: np.ndarray, device="cuda"):
    torch = _t()
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


def f16_tensor(bits: np.ndarray, device="cuda"):
    torch = _t()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(device)


def case_tensors(case, M: int, device="cuda"):
    """(x, words, scales, biases-or-None) of a synthetic Case as device tensors."""
    x = x_tensor(case.x(M), case.x_dtype, device)
    w = words_tensor(case.words, device)
    s = f16_tensor(case.scales, device)
    b = None if case.biases is None else f16_tensor(case.biases, device)
    return x, w, s, b
