"""Shared helpers of the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synthetic
import w4a16_group_wise_q4_amd as q4

DEV = torch.device("cuda:0")
SENTINEL_F32 = float("nan")
SENTINEL_I32 = -0x21524111  # 0xDEADBEEF as int32


def note(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives output capture)."""
    sys.__stderr__.write(f"  [gpu] {msg}\n")
    sys.__stderr__.flush()


def host_input(w: torch.Tensor):
    """A CPU tensor as the oracle's input (float32 array or (uint16 bits, dtype code))."""
    if w.dtype == torch.float32:
        return w.numpy()
    code = oracle.BF16 if w.dtype == torch.bfloat16 else oracle.F16
    return (synthetic.as_u16(w), code)


def guarded(shape, dtype, sentinel, guard=256):
    """An output tensor that is a view into a larger buffer filled with a sentinel, so
    stores outside the tensor can be detected afterwards."""
    numel = int(np.prod(shape))
    buf = torch.full((guard + numel + guard,), sentinel, dtype=dtype, device=DEV)
    return buf, buf[guard:guard + numel].view(*shape)


def guard_intact(buf, guard=256, sentinel=None):
    head = buf[:guard].cpu()
    tail = buf[-guard:].cpu()
    if sentinel is None or (isinstance(sentinel, float) and np.isnan(sentinel)):
        return bool(torch.isnan(head).all() and torch.isnan(tail).all())
    return bool((head == sentinel).all() and (tail == sentinel).all())


def pack_guarded(w_dev: torch.Tensor, g: int, sym: bool):
    """Quantize on the GPU into guarded output buffers; returns (packed, buffers)."""
    n, k = w_dev.shape
    G = k // g
    qb, qv = guarded((n, k // 8), torch.int32, SENTINEL_I32)
    sb, sv = guarded((n, G), torch.int16, -1)
    zb, zv = (None, None) if sym else guarded((n, (G + 7) // 8), torch.int32, SENTINEL_I32)
    p = q4.PackedWeight(qweight=qv, scales=sv.view(torch.float16), zeros=zv, n=n, k=k,
                        group_size=g, symmetric=sym)
    q4.q4_quantize_pack(w_dev, g, sym, out=p)
    return p, (qb, sb, zb)


def assert_pack_exact(p: q4.PackedWeight, w_host, g: int, sym: bool, rows=None):
    """Packed codes, scales and zero points equal the oracle's, bit for bit."""
    qo, so, zo = oracle.quantize_pack(w_host, g, sym)
    qg = p.qweight.cpu().numpy().view(np.uint32)
    sg = p.scales.cpu().numpy().view(np.uint16)
    if rows is not None:
        qg, sg = qg[rows], sg[rows]
    assert np.array_equal(qg, qo), f"qweight differs in {int((qg != qo).sum())} words"
    assert np.array_equal(sg, so), f"scales differ in {int((sg != so).sum())} groups"
    if not sym:
        zg = p.zeros.cpu().numpy().view(np.uint32)
        if rows is not None:
            zg = zg[rows]
        assert np.array_equal(zg, zo), f"zeros differ in {int((zg != zo).sum())} words"
    return qo, so, zo


def assert_linear_close(y_gpu: np.ndarray, x_host, packed_host, n, k, g, sym, rows=None,
                        cols=None, what=""):
    qo, so, zo = packed_host
    yr, ya = oracle.linear(x_host, qo, so, zo, n, k, g, sym, rows=rows, cols=cols)
    yg = y_gpu
    if rows is not None:
        yg = yg[np.asarray(rows)]
    if cols is not None:
        yg = yg[:, np.asarray(cols)]
    ok = oracle.within_tolerance(yg, yr, ya)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        det = [(int(i), int(j), float(yg[i, j]), float(yr[i, j]), float(ya[i, j])) for i, j in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())}/{ok.size} outside "
                             f"1e-3*|x||w|+1e-5; first (row, col, gpu, oracle, |x||w|): {det}")
    err = np.abs(yg - yr) / (ya + 1e-30)
    return float(err.max())
