"""Corrupted scale detection on the CPU: the oracle against IEEE 754 binary16 bit patterns
classified by hand, and the C ABI's argument rules (checked before anything is launched,
so no GPU is needed)."""
import ctypes

import numpy as np

from oracle import scales as oscales
import w4a16_group_wise_q4_amd as q4

# (bits, class): binary16 is sign | 5-bit exponent | 10-bit fraction; exponent 31 is Inf
# (fraction 0) or NaN, anything else with the sign set and a nonzero magnitude is below zero
PATTERNS = [
    (0x3C00, "ok"),        # 1.0
    (0x0000, "ok"),        # +0
    (0x8000, "ok"),        # -0: not below zero
    (0x0001, "ok"),        # 2^-24, the smallest subnormal
    (0x03FF, "ok"),        # the largest subnormal
    (0x7BFF, "ok"),        # 65504, the largest finite
    (0x7C00, "nonfinite"),  # +Inf
    (0xFC00, "nonfinite"),  # -Inf
    (0x7E00, "nonfinite"),  # a quiet NaN
    (0xFE01, "nonfinite"),  # a NaN with the sign set: not finite, so not counted as negative
    (0x7C01, "nonfinite"),  # a signalling NaN
    (0xBC00, "negative"),  # -1.0
    (0x8001, "negative"),  # -2^-24
    (0xFBFF, "negative"),  # -65504
]


def test_oracle_classifies_binary16_patterns():
    for bits, cls in PATTERNS:
        nf, neg, first = oscales.check_scales(np.array([bits], dtype=np.uint16))
        assert (nf, neg) == {"ok": (0, 0), "nonfinite": (1, 0), "negative": (0, 1)}[cls], hex(bits)
        assert first == (-1 if cls == "ok" else 0), hex(bits)


def test_oracle_counts_and_first_index():
    rng = np.random.default_rng(5)
    ok = np.array([b for b, c in PATTERNS if c == "ok"], dtype=np.uint16)
    a = rng.choice(ok, size=(37, 11))
    assert oscales.check_scales(a) == (0, 0, -1)
    a[3, 4] = 0xBC00   # flat 3 * 11 + 4 = 37
    a[20, 0] = 0x7E00  # 220
    a[36, 10] = 0xFC00  # 406
    a[2, 9] = 0x8001   # 31: the first
    assert oscales.check_scales(a) == (2, 2, 31)
    # fp16 arrays read the same as their bit patterns
    assert oscales.check_scales(a.view(np.float16)) == (2, 2, 31)


def test_abi_rules_before_launch():
    lib = q4.lib()
    A = ctypes.c_void_p(1 << 20)     # aligned, never dereferenced: every case fails a rule
    res = ctypes.c_void_p(1 << 21)
    OK, NULL, SHAPE, GROUP, ALIGN = 0, 1, 2, 3, 5
    assert lib.q4_check_scales(None, 16, 256, 128, res, None) == NULL
    assert lib.q4_check_scales(A, 16, 256, 128, None, None) == NULL
    assert lib.q4_check_scales(ctypes.c_void_p((1 << 20) + 1), 16, 256, 128, res, None) == ALIGN
    assert lib.q4_check_scales(A, 16, 256, 128, ctypes.c_void_p((1 << 21) + 4), None) == ALIGN
    assert lib.q4_check_scales(A, 16, 256, 48, res, None) == GROUP
    assert lib.q4_check_scales(A, 16, 200, 128, res, None) == SHAPE
    assert lib.q4_check_scales(A, 0, 256, 128, res, None) == SHAPE
    assert q4.q4_last_kernel() == ""
