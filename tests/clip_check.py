"""Validity check for a clip-search result produced by another implementation.

The clip search ("Quantization Algorithms 단권화", §MSE-optimal: argmin ||x - x_dq||^2 over
the candidate clip ratios) is decided by fp64 sums of squares.  Two implementations that
add the same g terms in different orders can round a near-tie the other way, so a
different ratio is still a correct answer when its error is within the rounding of the
sums of the smallest one.  A result is valid when, per group:
  * its bits (codes, fp16 scale, zero point) are the oracle's quantization at one of the
    eleven clip ratios, and
  * that ratio's error, as the oracle sums it, is at most E_min * (1 + 5 (g + 2) 2^-53),
    E_min the oracle's smallest error of the group.
The bound: any order of adding g non-negative terms, each a rounded square of a rounded
difference, is within a factor (1 +- eps), eps = (g + 2) 2^-53, of the exact sum; a
candidate the other side ranks first is then within (1 + eps)^2 / (1 - eps)^2 of the
oracle's minimum, which 1 + 5 eps covers for any g here.
"""
from __future__ import annotations

import numpy as np

import pins

RATIOS = pins.MSE_CANDIDATES


def clip_choice_report(o, w, g: int, sym: bool, qweight, scales, zeros):
    """(ratio index per group or -1 where no ratio reproduces the bits, error at that
    ratio, the oracle's minimum, the bound) for a result of W [n, k] (a float32/f16
    array, or a (uint16 bits, dtype code) pair, as the oracle takes it)."""
    n, k = (w[0] if isinstance(w, tuple) else w).shape
    G = k // g
    errs = o.mse_errors(w, g, sym)
    codes = pins.unpack_codes(np.asarray(qweight).view(np.uint32), k).reshape(n, G, g)
    s16 = np.asarray(scales).view(np.uint16)
    zz = None if sym else pins.unpack_zeros(np.asarray(zeros).view(np.uint32), G)
    ratio = np.full((n, G), -1, dtype=np.int64)
    for i in range(RATIOS):
        qi, si, zi = o.quantize_pack_clip(w, g, sym, i)
        same = (pins.unpack_codes(qi, k).reshape(n, G, g) == codes).all(axis=2) & (si == s16)
        if not sym:
            same &= pins.unpack_zeros(zi, G) == zz
        ratio[(ratio < 0) & same] = i
    err_at = np.take_along_axis(errs, np.maximum(ratio, 0)[..., None], axis=2)[..., 0]
    emin = errs.min(axis=2)
    bound = emin * (1.0 + 5.0 * (g + 2) * 2.0 ** -53)
    return ratio, err_at, emin, bound


def check_clip_choice(o, w, g: int, sym: bool, qweight, scales, zeros) -> float:
    """Assert the result is valid (see the module note); returns the fraction of groups
    whose ratio is the oracle's own choice."""
    ratio, err_at, emin, bound = clip_choice_report(o, w, g, sym, qweight, scales, zeros)
    bad = np.argwhere(ratio < 0)
    assert bad.size == 0, f"bits of group(s) {bad[:4].tolist()} are no clip ratio's quantization"
    worse = np.argwhere(err_at > bound)
    assert worse.size == 0, (f"group(s) {worse[:4].tolist()} chose an error above the bound: "
                             f"{err_at[tuple(worse[0])]!r} > {bound[tuple(worse[0])]!r}")
    _, _, _, choice = o.quantize_pack_mse(w, g, sym, with_choice=True)
    return float((ratio == choice).mean())
