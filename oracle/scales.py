"""CPU oracle of corrupted scale detection — TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the GPU library never does.

"LLM Quantization: GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)", §Quantized Artifact Security
(Runtime) lists corrupted scale detection among the checks of a loaded quantized model.
What counts as corrupted follows from how a scale is made ("LLM Quantization ... (7/10)",
§Asymmetric: s = (x_max - x_min) / (q_max - q_min); §Symmetric: s = max|x| / q_max;
§Group Scale Overhead: one fp16 scale per group): every stored scale is an fp16 value that
is a group's range over 15 or its largest magnitude over 7, so it is finite and not below
zero (0 for a group of zeros).  A stored scale is therefore corrupted when, read as an
IEEE 754 binary16 number, it is not finite, or it is finite and less than zero (-0 is not
less than zero).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def check_scales(scales: np.ndarray) -> Tuple[int, int, int]:
    """(number of non-finite scales, number of finite scales below zero, flat index of the
    first scale of either kind in row-major order, or -1).  scales: fp16 values or their
    uint16 bit patterns, any shape."""
    v = np.ascontiguousarray(scales).reshape(-1)
    if v.dtype != np.float16:
        v = v.astype(np.uint16).view(np.float16)
    x = v.astype(np.float64)
    nonfinite = ~np.isfinite(x)
    negative = np.isfinite(x) & (x < 0.0)
    bad = np.nonzero(nonfinite | negative)[0]
    return int(nonfinite.sum()), int(negative.sum()), int(bad[0]) if bad.size else -1
