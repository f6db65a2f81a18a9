"""Dequantisation written independently of the oracle, for pinning it.

E2M1 values come from the golden table (the bit layout the pages state); scale
bytes are decoded with torch's float8_e8m0fnu / float8_e4m3fn dtypes, a
library routine the oracle does not use.
"""
import json
import os

import numpy as np
import torch

_GOLD = os.path.join(os.path.dirname(__file__), "golden", "e2m1.json")
with open(_GOLD) as _f:
    E2M1 = np.array(json.load(_f)["values"], np.float64)


def scale_values(scales: np.ndarray, fmt: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(scales, np.uint8))
    dt = torch.float8_e8m0fnu if fmt == 0 else torch.float8_e4m3fn
    return t.view(dt).to(torch.float64).numpy()


def dequant(codes: np.ndarray, scales: np.ndarray, group: int, fmt: int) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    lo = E2M1[codes & 15]
    hi = E2M1[codes >> 4]
    vals = np.stack([lo, hi], -1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    sv = np.repeat(scale_values(scales, fmt), group, axis=-1)
    return vals * sv


def bf16_to_f64(bits) -> np.ndarray:
    t = torch.as_tensor(np.ascontiguousarray(bits)).view(torch.int16)
    return t.view(torch.bfloat16).to(torch.float64).numpy()
