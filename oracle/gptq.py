"""CPU oracle for GPTQ-style error-feedback quantization into the packed INT4 format —
TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the CPU-baseline leg
of the benchmark; the GPU library never uses it).

Follows "Quantization Algorithms 단권화", GPTQ chapter (§Hessian 정의, §OBQ single-step 수식,
§GPTQ block-wise, §알고리즘 개요, §설정 grid), in fp64 with numpy:

  1. H = 2 X^T X over the calibration tokens X [T][k] (k input features), dampened;
  2. L = the upper Cholesky factor of H^-1 (H^-1 = L^T L);
  3. for each block of 128 columns, for each column j of it: quantize column j, take
     err = (w_j - w_hat_j) / L[j, j], subtract err * L[j, j+1 : block end] from the block's
     later columns; after the block, subtract Err_block * L[block, rest] from the columns
     after it.

Readings where the pages leave a step open (listed with the others in the design notes):
  G1 the quantizer of every group is the RTN one of the original weights (scale, zero
     point, code range and rounding of q4_oracle.c's orc_quantize_pack), fixed before the
     sweep ("static groups"): the packed format fixes groups of g consecutive columns, and
     the outline quantizes each column against a given quantizer;
  G2 columns are swept in natural order, or, with act-order (§설정 grid: columns with the
     largest |X|^2 first), in the order of descending sum_t x_ti^2 (fp64), equal sums by
     the lower column index; a never-active feature sums to 0 and comes last.  The static
     group quantizers of G1 stay tied to the column's own position, so act-order changes
     only the order in which codes are chosen and errors carried, not the format;
  G3 dampening H_ii <- H_ii + lambda * H_ii with lambda = 0.01, as the Hessian section
     writes it;
  G4 a feature that is never active (H_ii = 0) gets H_ii = 1 before dampening, so H stays
     positive definite; its column then takes no error from the others.
"""
from __future__ import annotations

import numpy as np

from . import default as _default

BLOCK = 128
DAMP = 0.01


def hessian(x, damp: float = DAMP) -> np.ndarray:
    """H = 2 X^T X (fp64) with G4 and G3 applied; x is [T][k] (any float dtype)."""
    x64 = np.asarray(x, dtype=np.float64)
    h = 2.0 * (x64.T @ x64)
    d = np.diag(h).copy()
    d[d == 0.0] = 1.0                      # G4
    h[np.diag_indices_from(h)] = d + damp * d  # G3
    return h


def act_order(x) -> np.ndarray:
    """The act-order sweep order (G2): column indices by descending sum_t x_ti^2 in fp64,
    ties by the lower index; x is [T][k] (any float dtype)."""
    x64 = np.asarray(x, dtype=np.float64)
    energy = np.sum(x64 * x64, axis=0)
    return np.argsort(-energy, kind="stable")


def _codes_of(qweight: np.ndarray, k: int) -> np.ndarray:
    shifts = 4 * np.arange(8, dtype=np.uint32)
    nib = (qweight[:, :, None] >> shifts[None, None, :]) & np.uint32(0xF)
    return nib.reshape(qweight.shape[0], k).astype(np.int64)


def _zeros_of(zeros: np.ndarray, groups: int) -> np.ndarray:
    shifts = 4 * np.arange(8, dtype=np.uint32)
    nib = (zeros[:, :, None] >> shifts[None, None, :]) & np.uint32(0xF)
    return nib.reshape(zeros.shape[0], -1)[:, :groups].astype(np.int64)


def _pack(codes: np.ndarray) -> np.ndarray:
    n, k = codes.shape
    c = codes.astype(np.uint32).reshape(n, k // 8, 8)
    shifts = 4 * np.arange(8, dtype=np.uint32)
    return np.bitwise_or.reduce(c << shifts[None, None, :], axis=2).astype(np.uint32)


def gptq_quantize(w, h: np.ndarray, group_size: int, symmetric: bool, block: int = BLOCK,
                  oracle=None, order=None):
    """GPTQ of W [n][k] (an input as the oracle's quantize_pack takes: float32/float16
    array, or (uint16 bits, dtype code)) against the fp64 Hessian h [k][k].  ``order``
    (a permutation of the k columns, e.g. act_order(x)) is the sweep order; None is the
    natural order.  Returns (qweight, scales, zeros) in the packed format; scales and zeros
    are those of the RTN quantizer (G1)."""
    o = oracle if oracle is not None else _default()
    _, scales, zeros = o.quantize_pack(w, group_size, symmetric)        # G1
    if isinstance(w, tuple):                                            # exact widenings
        bits, code = w
        bits = np.asarray(bits, dtype=np.uint16)
        if code == 2:
            wf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        else:
            wf = bits.view(np.float16).astype(np.float64)
    else:
        wf = np.asarray(w, dtype=np.float64)
    n, k = wf.shape
    g = group_size
    s = scales.view(np.float16).astype(np.float64)                      # [n][G], exact
    z = np.full(s.shape, 8, dtype=np.int64) if symmetric else _zeros_of(zeros, k // g)
    q_lo, q_hi = (0, 15)                                                # stored codes u
    # G2: sweep position p takes column order[p]; H and W follow the same order, and each
    # column keeps its own group's quantizer
    order = np.arange(k) if order is None else np.asarray(order, dtype=np.int64)
    if sorted(order.tolist()) != list(range(k)):
        raise ValueError("order must be a permutation of the columns")
    h = np.asarray(h, dtype=np.float64)[np.ix_(order, order)]
    wf = wf[:, order]
    # step 2: upper Cholesky factor of H^-1 (H^-1 = L^T L)
    hinv = np.linalg.inv(h)
    lo = np.linalg.cholesky(hinv)                                       # hinv = lo lo^T
    L = lo.T
    W = wf.copy()
    codes = np.zeros((n, k), dtype=np.int64)
    for b0 in range(0, k, block):
        b1 = min(b0 + block, k)
        err_block = np.zeros((n, b1 - b0))
        for j in range(b0, b1):
            gj = order[j] // g
            # quantize column j against its group's quantizer: u = clamp(round(w/S) + z)
            u = np.clip(np.rint(W[:, j] / s[:, gj]) + z[:, gj], q_lo, q_hi).astype(np.int64)
            codes[:, j] = u
            w_hat = s[:, gj] * (u - z[:, gj])
            err = (W[:, j] - w_hat) / L[j, j]
            W[:, j + 1:b1] -= np.outer(err, L[j, j + 1:b1])
            err_block[:, j - b0] = err
        W[:, b1:] -= err_block @ L[b0:b1, b1:]
    placed = np.zeros_like(codes)
    placed[:, order] = codes                                            # back to column order
    return _pack(placed), scales, zeros


def layer_error(w, w_hat, x) -> float:
    """The layer-output objective ||X (W - W_hat)^T||_F^2 in fp64 (the quantity GPTQ
    lowers; [QA1] GPTQ chapter, §Layer-wise objective)."""
    d = np.asarray(w, dtype=np.float64) - np.asarray(w_hat, dtype=np.float64)
    y = np.asarray(x, dtype=np.float64) @ d.T
    return float(np.sum(y * y))
