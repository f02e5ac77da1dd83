"""CPU oracle for group-wise affine INT4 (W4A16) — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this package
imports nothing from it.

The arithmetic lives in ``q4_oracle.c`` (plain C, gcc -O2 -ffp-contract=off, no
fast-math); this module only builds it and marshals numpy arrays through ctypes.
Page citations and the readings taken where the pages are silent are in the C sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_q4.so")

F32, F16, BF16 = 0, 1, 2

GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra"]


def compile_source(src: str, out: str, include_dir: str = _HERE, compiler: str = "gcc",
                   extra: Tuple[str, ...] = ()) -> str:
    """Compile one oracle C source into a shared library with the oracle's flags (extra
    flags after them, e.g. sanitizers for a debug copy)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([compiler, *GCC_FLAGS, *extra, "-I", include_dir, "-o", tmp, src, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle (called by the build entry point every time)."""
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(w) -> Tuple[np.ndarray, int]:
    """numpy float32 / float16, or a (uint16 bit-pattern array, dtype code) tuple."""
    if isinstance(w, tuple):
        arr, code = w
        return np.ascontiguousarray(arr, dtype=np.uint16), int(code)
    if w.dtype == np.float32:
        return np.ascontiguousarray(w), F32
    if w.dtype == np.float16:
        return np.ascontiguousarray(w).view(np.uint16), F16
    raise TypeError("oracle input must be float32, float16 or (uint16 bits, code)")


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        c_i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.orc_f32_to_f16_rne.argtypes = [ctypes.c_float]
        lib.orc_f32_to_f16_rne.restype = ctypes.c_uint16
        lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_f32.restype = ctypes.c_float
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_quantize_pack.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_int, vp, vp, vp, vp]
        lib.orc_quantize_pack.restype = c_int
        lib.orc_quantize_pack_mse.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_int, vp, vp, vp, vp]
        lib.orc_quantize_pack_mse.restype = c_int
        lib.orc_quantize_pack_clip.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_int, vp, vp, vp, vp]
        lib.orc_quantize_pack_clip.restype = c_int
        lib.orc_mse_errors.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_int, vp]
        lib.orc_mse_errors.restype = c_int
        lib.orc_dequant_f64.argtypes = [vp, vp, vp, c_i64, c_i64, c_i64, c_int, vp]
        lib.orc_dequant_f64.restype = c_int
        lib.orc_linear_f64.argtypes = [vp, c_int, c_i64, vp, c_i64, vp, vp, vp,
                                       c_i64, c_i64, c_i64, c_int, vp, c_i64, vp, vp]
        lib.orc_linear_f64.restype = c_int
        lib.orc_kv_quantize.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_i64, c_int, c_i64, c_i64,
                                        vp, vp, vp]
        lib.orc_kv_quantize.restype = c_int
        lib.orc_kv_attention_f64.argtypes = [vp, c_int, c_i64, c_i64, c_i64, c_i64, vp, vp, vp,
                                             vp, vp, vp, c_i64, c_int, ctypes.c_double, vp, vp, vp]
        lib.orc_kv_attention_f64.restype = c_int
        lib.orc_qweight_words.argtypes = [c_i64, c_i64]
        lib.orc_qweight_words.restype = c_i64
        lib.orc_scale_count.argtypes = [c_i64, c_i64, c_i64]
        lib.orc_scale_count.restype = c_i64
        lib.orc_zero_words.argtypes = [c_i64, c_i64, c_i64]
        lib.orc_zero_words.restype = c_i64
        self.lib = lib
        self.path = path

    # ------------------------------------------------------------ conversions
    def f32_to_f16_bits(self, f: float) -> int:
        return int(self.lib.orc_f32_to_f16_rne(ctypes.c_float(f)))

    def f16_bits_to_f32(self, h: int) -> float:
        return float(self.lib.orc_f16_to_f32(ctypes.c_uint16(int(h))))

    def bf16_bits_to_f32(self, b: int) -> float:
        return float(self.lib.orc_bf16_to_f32(ctypes.c_uint16(int(b))))

    # ------------------------------------------------------------ the method
    def quantize_pack(self, w, group_size: int, symmetric: bool, with_diag: bool = False):
        """RTN quantize + pack of W [n, k]: (qweight u32 [n, k/8], scales u16 [n, G],
        zeros u32 [n, ceil(G/8)]) and, with ``with_diag``, per-group one-sided flags."""
        arr, code = _as_input(w)
        n, k = arr.shape
        G = k // group_size
        qweight = np.zeros((n, k // 8), dtype=np.uint32)
        scales = np.zeros((n, G), dtype=np.uint16)
        zeros = np.zeros((n, (G + 7) // 8), dtype=np.uint32)
        onesided = np.zeros((n, G), dtype=np.uint8)
        rc = self.lib.orc_quantize_pack(_ptr(arr), code, n, k, group_size,
                                        int(bool(symmetric)), _ptr(qweight), _ptr(scales),
                                        _ptr(zeros), _ptr(onesided))
        if rc != 0:
            raise ValueError("oracle quantize_pack rejected the arguments")
        if with_diag:
            return qweight, scales, zeros, onesided
        return qweight, scales, zeros

    def quantize_pack_mse(self, w, group_size: int, symmetric: bool, with_choice: bool = False):
        """MSE-optimal clip search + pack of W [n, k]: (qweight, scales, zeros) as
        quantize_pack, and with ``with_choice`` the chosen ratio index per group (alpha =
        (20 - i) / 20)."""
        arr, code = _as_input(w)
        n, k = arr.shape
        G = k // group_size
        qweight = np.zeros((n, k // 8), dtype=np.uint32)
        scales = np.zeros((n, G), dtype=np.uint16)
        zeros = np.zeros((n, (G + 7) // 8), dtype=np.uint32)
        choice = np.zeros((n, G), dtype=np.uint8)
        rc = self.lib.orc_quantize_pack_mse(_ptr(arr), code, n, k, group_size,
                                            int(bool(symmetric)), _ptr(qweight), _ptr(scales),
                                            _ptr(zeros), _ptr(choice))
        if rc != 0:
            raise ValueError("oracle quantize_pack_mse rejected the arguments")
        if with_choice:
            return qweight, scales, zeros, choice
        return qweight, scales, zeros

    def quantize_pack_clip(self, w, group_size: int, symmetric: bool, ratio):
        """Quantize + pack of W [n, k] with group (row, j) clipped at alpha = (20 - i) / 20,
        i = ratio[row, j] (an int, or an [n, G] array): (qweight, scales, zeros)."""
        arr, code = _as_input(w)
        n, k = arr.shape
        G = k // group_size
        idx = np.ascontiguousarray(np.broadcast_to(np.asarray(ratio, dtype=np.uint8), (n, G)))
        qweight = np.zeros((n, k // 8), dtype=np.uint32)
        scales = np.zeros((n, G), dtype=np.uint16)
        zeros = np.zeros((n, (G + 7) // 8), dtype=np.uint32)
        rc = self.lib.orc_quantize_pack_clip(_ptr(arr), code, n, k, group_size,
                                             int(bool(symmetric)), _ptr(idx), _ptr(qweight),
                                             _ptr(scales), _ptr(zeros))
        if rc != 0:
            raise ValueError("oracle quantize_pack_clip rejected the arguments")
        return qweight, scales, zeros

    def mse_errors(self, w, group_size: int, symmetric: bool) -> np.ndarray:
        """Every clip candidate's squared error, float64 [n, G, 11] (ratio index last)."""
        arr, code = _as_input(w)
        n, k = arr.shape
        out = np.zeros((n, k // group_size, 11), dtype=np.float64)
        rc = self.lib.orc_mse_errors(_ptr(arr), code, n, k, group_size, int(bool(symmetric)),
                                     _ptr(out))
        if rc != 0:
            raise ValueError("oracle mse_errors rejected the arguments")
        return out

    def dequant(self, qweight, scales, zeros, n: int, k: int, group_size: int,
                symmetric: bool) -> np.ndarray:
        """x_hat [n, k] in float64 (exact)."""
        out = np.zeros((n, k), dtype=np.float64)
        q, s, z = (np.ascontiguousarray(a) for a in (qweight, scales, zeros))
        rc = self.lib.orc_dequant_f64(_ptr(q), _ptr(s), _ptr(z), n, k, group_size,
                                      int(bool(symmetric)), _ptr(out))
        if rc != 0:
            raise ValueError("oracle dequant rejected the arguments")
        return out

    def linear(self, x, qweight, scales, zeros, n: int, k: int, group_size: int,
               symmetric: bool, rows=None, cols=None):
        """(y, yabs): y = x · x_hat^T in float64 and sum |x||x_hat| per element.
        ``rows``/``cols`` pick a sample of (m, n): y has shape [len(rows), len(cols)]."""
        xa, code = _as_input(x)
        m = xa.shape[0]
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
        nr = m if r is None else r.size
        nc = n if c is None else c.size
        y = np.zeros((nr, nc), dtype=np.float64)
        yabs = np.zeros((nr, nc), dtype=np.float64)
        q, s, z = (np.ascontiguousarray(a) for a in (qweight, scales, zeros))
        rc = self.lib.orc_linear_f64(_ptr(xa), code, m, _ptr(r), nr, _ptr(q), _ptr(s), _ptr(z),
                                     n, k, group_size, int(bool(symmetric)), _ptr(c), nc,
                                     _ptr(y), _ptr(yabs))
        if rc != 0:
            raise ValueError("oracle linear rejected the arguments")
        return y, yabs

    # ------------------------------------------------------------ KV cache
    def kv_cache(self, heads: int, t_cap: int, d: int, group_size: int):
        """An empty head-major cache (qcache, scache, zcache) of heads * t_cap rows."""
        return (np.zeros((heads * t_cap, d // 8), dtype=np.uint32),
                np.zeros((heads * t_cap, d // group_size), dtype=np.uint16),
                np.zeros((heads * t_cap, (d // group_size + 7) // 8), dtype=np.uint32))

    def kv_quantize(self, kv, group_size: int, symmetric: bool, cache, t0: int):
        """Quantize kv [t_new, heads, d] (an input as ``quantize_pack`` takes) into rows h * t_cap + t0 + t of ``cache`` (the
        arrays of ``kv_cache``), in place."""
        arr, code = _as_input(kv)
        t_new, heads, d = arr.shape
        qc, sc, zc = cache
        t_cap = qc.shape[0] // heads
        rc = self.lib.orc_kv_quantize(_ptr(arr), code, t_new, heads, d, group_size,
                                      int(bool(symmetric)), t_cap, t0, _ptr(qc), _ptr(sc),
                                      _ptr(zc))
        if rc != 0:
            raise ValueError("oracle kv_quantize rejected the arguments")
        return cache

    def kv_attention(self, q, kcache, vcache, n_tok: int, group_size: int, symmetric: bool,
                     scale: float):
        """(out [heads, d], score_abs [heads], v_abs [heads, d]) in float64 for queries
        q [heads, d] over the first n_tok tokens of the head-major caches."""
        qa, code = _as_input(q)
        heads, d = qa.shape
        kq, ks, kz = (np.ascontiguousarray(a) for a in kcache)
        vq, vs, vz = (np.ascontiguousarray(a) for a in vcache)
        t_cap = kq.shape[0] // heads
        out = np.zeros((heads, d), dtype=np.float64)
        sabs = np.zeros(heads, dtype=np.float64)
        vabs = np.zeros((heads, d), dtype=np.float64)
        rc = self.lib.orc_kv_attention_f64(_ptr(qa), code, heads, d, n_tok, t_cap, _ptr(kq),
                                           _ptr(ks), _ptr(kz), _ptr(vq), _ptr(vs), _ptr(vz),
                                           group_size, int(bool(symmetric)), float(scale),
                                           _ptr(out), _ptr(sabs), _ptr(vabs))
        if rc != 0:
            raise ValueError("oracle kv_attention rejected the arguments")
        return out, sabs, vabs

    def sizes(self, n: int, k: int, group_size: int) -> Tuple[int, int, int]:
        """Element counts of (qweight words, scales, zero words)."""
        return (int(self.lib.orc_qweight_words(n, k)),
                int(self.lib.orc_scale_count(n, k, group_size)),
                int(self.lib.orc_zero_words(n, k, group_size)))


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def quantize_pack(*a, **kw):
    return default().quantize_pack(*a, **kw)


def quantize_pack_mse(*a, **kw):
    return default().quantize_pack_mse(*a, **kw)


def quantize_pack_clip(*a, **kw):
    return default().quantize_pack_clip(*a, **kw)


def mse_errors(*a, **kw):
    return default().mse_errors(*a, **kw)


def dequant(*a, **kw):
    return default().dequant(*a, **kw)


def linear(*a, **kw):
    return default().linear(*a, **kw)


def within_tolerance(y_test, y_ref, yabs, rel: float = 1e-3, abs_: float = 1e-5) -> np.ndarray:
    """Elementwise |y_test - y_ref| <= rel * (|x| . |x_hat|^T) + abs_ (the matmul bound)."""
    return np.abs(np.asarray(y_test, dtype=np.float64) - y_ref) <= rel * yabs + abs_
