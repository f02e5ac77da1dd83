"""Python binding of libq4, the MI355X (gfx950) group-wise INT4 weight-only library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
(include/q4.h).  torch supplies device memory and the current stream.  There is no
CPU path: if the shared library is missing and cannot be built, importing the binding
raises.

Entry points (same names as the C ABI):
    q4_quantize_pack(w, group_size, symmetric)          -> PackedWeight
    q4_dequant(packed, out_dtype)                       -> W_hat [n, k]
    q4_w4a16_gemm(x, packed)                            -> y [m, n] fp32
    q4_w4a16_gemm_grouped(xs, packs)                    -> [y_i], one launch when m <= 16
    q4_kv_quantize(kv, cache, t0)                       -> appends tokens to a KvCache
    q4_kv_attention(q, kcache, vcache, n_tok, scale)    -> out [heads, d] fp32
    q4_gptq_quantize(w, x, group_size, symmetric)       -> PackedWeight (GPTQ codes;
                                                           act_order=True for act-order)
    q4_last_kernel()                                    -> name of the last kernel run
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _build

__all__ = ["PackedWeight", "q4_quantize_pack", "q4_quantize_pack_grouped", "q4_quantize_pack_mse",
           "q4_dequant", "q4_check_scales",
           "q4_w4a16_gemm",
           "q4_w4a16_gemm_grouped", "q4_last_kernel", "q4_last_kernels", "q4_last_launch_count",
           "q4_source_digest", "StaleLibraryError", "KvCache", "empty_kv_cache",
           "q4_kv_quantize", "q4_kv_attention", "q4_kv_attention_workspace",
           "q4_kv_attention_noalloc",
           "q4_gptq_quantize", "q4_gptq_workspace", "q4_gptq_act_order_workspace",
           "q4_qweight_words", "q4_scale_count", "q4_zero_words", "q4_layout_version",
           "library_path", "Q4Error"]

Q4_F32, Q4_F16, Q4_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: Q4_F32, torch.float16: Q4_F16, torch.bfloat16: Q4_BF16}

EXPORTED = ("q4_quantize_pack", "q4_quantize_pack_grouped", "q4_quantize_pack_mse", "q4_dequant",
            "q4_w4a16_gemm", "q4_w4a16_gemm_out", "q4_w4a16_gemm_ws", "q4_w4a16_gemm_workspace",
            "q4_w4a16_gemm_grouped", "q4_w4a16_gemm_grouped_out", "q4_kv_quantize", "q4_kv_attention",
            "q4_kv_attention_workspace", "q4_kv_attention_noalloc",
            "q4_kv_attention_noalloc_max_bytes", "q4_gptq_quantize", "q4_gptq_workspace",
            "q4_gptq_quantize_act_order", "q4_gptq_act_order_workspace", "q4_qweight_words",
            "q4_scale_count", "q4_zero_words", "q4_check_scales", "q4_status_str", "q4_last_kernel",
            "q4_last_kernels", "q4_last_launch_count", "q4_layout_version", "q4_source_digest")


class GemmProblem(ctypes.Structure):
    """q4_gemm_problem of the C ABI."""
    _fields_ = [("x", ctypes.c_void_p), ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("n", ctypes.c_int64), ("y", ctypes.c_void_p)]


class QuantProblem(ctypes.Structure):
    """q4_quant_problem of the C ABI."""
    _fields_ = [("w", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p)]


MAX_GROUP = 8


class Q4Error(RuntimeError):
    """A non-OK q4_status returned by the library."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"q4 status {code}: {msg}")
        self.code = code


_lib = None


def library_path() -> str:
    """The library the binding loads: $Q4_LIBRARY if set (another build of the same
    sources, e.g. the host-sanitized one), else the in-tree libq4.so."""
    return os.environ.get("Q4_LIBRARY") or _build.LIBRARY


class StaleLibraryError(RuntimeError):
    """libq4.so was built from sources other than the ones next to it."""


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if path == _build.LIBRARY and not os.path.exists(path):
        _build.build()  # raises if hipcc fails: there is no fallback
    lib = ctypes.CDLL(path)
    lib.q4_source_digest.argtypes = []
    lib.q4_source_digest.restype = ctypes.c_char_p
    built, here = lib.q4_source_digest().decode(), _build.source_digest()
    if built != here:
        raise StaleLibraryError(
            f"{path} was built from sources with digest {built}, but the sources "
            f"here digest to {here}: rebuild it (__graft_entry__.build())")
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.q4_quantize_pack.argtypes = [vp, ctypes.c_int, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.q4_quantize_pack.restype = ctypes.c_int
    lib.q4_quantize_pack_mse.argtypes = [vp, ctypes.c_int, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.q4_quantize_pack_mse.restype = ctypes.c_int
    lib.q4_quantize_pack_grouped.argtypes = [ctypes.POINTER(QuantProblem), i32, ctypes.c_int, i32,
                                             i32, vp]
    lib.q4_quantize_pack_grouped.restype = ctypes.c_int
    lib.q4_dequant.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, vp]
    lib.q4_dequant.restype = ctypes.c_int
    lib.q4_check_scales.argtypes = [vp, i64, i64, i32, vp, vp]
    lib.q4_check_scales.restype = ctypes.c_int
    lib.q4_w4a16_gemm.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp]
    lib.q4_w4a16_gemm.restype = ctypes.c_int
    lib.q4_w4a16_gemm_out.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp,
                                      ctypes.c_int, vp]
    lib.q4_w4a16_gemm_out.restype = ctypes.c_int
    lib.q4_w4a16_gemm_ws.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp,
                                     ctypes.c_int, vp, i64, vp]
    lib.q4_w4a16_gemm_ws.restype = ctypes.c_int
    lib.q4_w4a16_gemm_workspace.argtypes = [i64, i64, i64, i32]
    lib.q4_w4a16_gemm_workspace.restype = i64
    lib.q4_w4a16_gemm_grouped.argtypes = [ctypes.POINTER(GemmProblem), i32, ctypes.c_int, i64, i64,
                                          i32, i32, vp]
    lib.q4_w4a16_gemm_grouped.restype = ctypes.c_int
    lib.q4_w4a16_gemm_grouped_out.argtypes = [ctypes.POINTER(GemmProblem), i32, ctypes.c_int, i64, i64,
                                              i32, i32, ctypes.c_int, vp]
    lib.q4_w4a16_gemm_grouped_out.restype = ctypes.c_int
    lib.q4_kv_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, i32, i32, i64, i64, vp, vp, vp,
                                   vp]
    lib.q4_kv_quantize.restype = ctypes.c_int
    lib.q4_kv_attention_workspace.argtypes = [i64, i64, i64]
    lib.q4_kv_attention_workspace.restype = i64
    lib.q4_kv_attention.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                    i32, i32, ctypes.c_float, vp, vp, i64, vp]
    lib.q4_kv_attention.restype = ctypes.c_int
    lib.q4_kv_attention_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, vp, vp,
                                            vp, i32, i32, ctypes.c_float, vp, vp]
    lib.q4_kv_attention_noalloc.restype = ctypes.c_int
    lib.q4_kv_attention_noalloc_max_bytes.argtypes = []
    lib.q4_kv_attention_noalloc_max_bytes.restype = i64
    lib.q4_gptq_workspace.argtypes = [i64, i64, i32]
    lib.q4_gptq_workspace.restype = i64
    lib.q4_gptq_quantize.argtypes = [vp, ctypes.c_int, i64, i64, vp, ctypes.c_int, i64, i32, i32,
                                     ctypes.c_float, vp, vp, vp, vp, i64, vp]
    lib.q4_gptq_act_order_workspace.argtypes = [i64, i64, i32]
    lib.q4_gptq_act_order_workspace.restype = i64
    lib.q4_gptq_quantize_act_order.argtypes = lib.q4_gptq_quantize.argtypes
    lib.q4_gptq_quantize_act_order.restype = ctypes.c_int
    lib.q4_gptq_quantize.restype = ctypes.c_int
    lib.q4_qweight_words.argtypes = [i64, i64]
    lib.q4_qweight_words.restype = i64
    lib.q4_scale_count.argtypes = [i64, i64, i32]
    lib.q4_scale_count.restype = i64
    lib.q4_zero_words.argtypes = [i64, i64, i32]
    lib.q4_zero_words.restype = i64
    lib.q4_status_str.argtypes = [ctypes.c_int]
    lib.q4_status_str.restype = ctypes.c_char_p
    lib.q4_last_kernel.argtypes = []
    lib.q4_last_kernel.restype = ctypes.c_char_p
    lib.q4_last_kernels.argtypes = []
    lib.q4_last_kernels.restype = ctypes.c_char_p
    lib.q4_last_launch_count.argtypes = []
    lib.q4_last_launch_count.restype = i64
    lib.q4_layout_version.argtypes = []
    lib.q4_layout_version.restype = i32
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raw C ABI)."""
    return _load()


def _check(code: int):
    if code != 0:
        raise Q4Error(code, _load().q4_status_str(code).decode())


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev_ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(name: str, t: torch.Tensor, device=None):
    """t is a contiguous tensor on the current GPU (and on ``device`` when given)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the library has no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's other tensors on {device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not the current device "
                         f"cuda:{torch.cuda.current_device()} the kernels launch on")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need(name: str, t: torch.Tensor, shape, dtypes, device):
    """A device tensor of exactly this shape and one of these dtypes: a shorter buffer would
    let a kernel write (or read) past its end."""
    _need_cuda(name, t, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {sorted(map(str, dtypes))}")


def _layout_ok(n: int, k: int, g: int) -> bool:
    """Sizes for which the packed shapes are defined (others are refused by the C ABI)."""
    return g in (32, 64, 128) and n >= 1 and k >= 1 and k % g == 0


def _check_packed(p: "PackedWeight", device, n=None, k=None, group_size=None, symmetric=None):
    """The packed weight's tensors against its own n, k, group size and mode (and against
    the call's, when given): qweight int32 [n, k/8], scales fp16 [n, k/g], zeros int32
    [n, ceil(k/g/8)] unless symmetric."""
    if not isinstance(p, PackedWeight):
        raise TypeError("expected a PackedWeight")
    for nm, want, have in (("n", n, p.n), ("k", k, p.k), ("group_size", group_size, p.group_size),
                           ("symmetric", symmetric, p.symmetric)):
        if want is not None and want != have:
            raise ValueError(f"packed weight has {nm}={have}, the call needs {want}")
    if not _layout_ok(p.n, p.k, p.group_size):
        return  # the C ABI refuses these sizes before touching any memory
    G = p.k // p.group_size
    _need("qweight", p.qweight, (p.n, p.k // 8), (torch.int32,), device)
    _need("scales", p.scales, (p.n, G), (torch.float16,), device)
    if p.symmetric:
        if p.zeros is not None:
            _need("zeros", p.zeros, (p.n, (G + 7) // 8), (torch.int32,), device)
    else:
        if p.zeros is None:
            raise ValueError("an asymmetric packed weight needs zeros")
        _need("zeros", p.zeros, (p.n, (G + 7) // 8), (torch.int32,), device)


def _check_cache(name: str, c: "KvCache", device):
    """A KV cache's tensors against its heads, t_cap, head_dim, group size and mode."""
    if not isinstance(c, KvCache):
        raise TypeError(f"{name} must be a KvCache")
    if c.heads < 1 or c.t_cap < 1 or not _layout_ok(c.heads * c.t_cap, c.head_dim, c.group_size):
        return  # refused by the C ABI
    rows, G = c.heads * c.t_cap, c.head_dim // c.group_size
    _need(f"{name}.qcache", c.qcache, (rows, c.head_dim // 8), (torch.int32,), device)
    _need(f"{name}.scache", c.scache, (rows, G), (torch.float16,), device)
    if not c.symmetric:
        if c.zcache is None:
            raise ValueError(f"{name}: an asymmetric cache needs zcache")
        _need(f"{name}.zcache", c.zcache, (rows, (G + 7) // 8), (torch.int32,), device)


def _need_workspace(name: str, t: torch.Tensor, device):
    _need_cuda(name, t, device)


@dataclass
class PackedWeight:
    """Canonical packed INT4 weight: qweight int32 [n, k/8] (uint32 bit patterns),
    scales float16 [n, k/g], zeros int32 [n, ceil(k/g/8)] or None when symmetric."""
    qweight: torch.Tensor
    scales: torch.Tensor
    zeros: Optional[torch.Tensor]
    n: int
    k: int
    group_size: int
    symmetric: bool


def q4_qweight_words(n: int, k: int) -> int:
    return int(_load().q4_qweight_words(n, k))


def q4_scale_count(n: int, k: int, group_size: int) -> int:
    return int(_load().q4_scale_count(n, k, group_size))


def q4_zero_words(n: int, k: int, group_size: int) -> int:
    return int(_load().q4_zero_words(n, k, group_size))


def q4_layout_version() -> int:
    return int(_load().q4_layout_version())


def q4_last_kernel() -> str:
    return _load().q4_last_kernel().decode()


def q4_last_kernels() -> list:
    """Every kernel the last successful call on this thread enqueued (distinct names, in
    launch order)."""
    s = _load().q4_last_kernels().decode()
    return s.split(",") if s else []


def q4_last_launch_count() -> int:
    """How many kernel launches the last successful call on this thread enqueued."""
    return int(_load().q4_last_launch_count())


def q4_source_digest() -> str:
    return _load().q4_source_digest().decode()


def empty_packed(n: int, k: int, group_size: int, symmetric: bool, device) -> PackedWeight:
    G = k // group_size
    return PackedWeight(
        qweight=torch.empty((n, k // 8), dtype=torch.int32, device=device),
        scales=torch.empty((n, G), dtype=torch.float16, device=device),
        zeros=None if symmetric else torch.empty((n, (G + 7) // 8), dtype=torch.int32, device=device),
        n=n, k=k, group_size=group_size, symmetric=bool(symmetric))


def q4_quantize_pack(w: torch.Tensor, group_size: int = 128, symmetric: bool = False,
                     out: Optional[PackedWeight] = None) -> PackedWeight:
    """RTN quantize-and-pack W [n, k] (fp32 / fp16 / bf16, on the GPU)."""
    _need_cuda("w", w)
    if w.dim() != 2 or w.dtype not in _DTYPE_CODE:
        raise ValueError("w must be a 2-D fp32, fp16 or bf16 tensor")
    n, k = w.shape
    p = out if out is not None else empty_packed(n, k, group_size, symmetric, w.device)
    _check_packed(p, w.device, n, k, group_size, bool(symmetric))
    _check(_load().q4_quantize_pack(_dev_ptr(w), _DTYPE_CODE[w.dtype], n, k, group_size,
                                    int(bool(symmetric)), _dev_ptr(p.qweight),
                                    _dev_ptr(p.scales), _dev_ptr(p.zeros), _stream(w)))
    return p


def q4_quantize_pack_mse(w: torch.Tensor, group_size: int = 128, symmetric: bool = False,
                         out: Optional[PackedWeight] = None) -> PackedWeight:
    """Quantize-and-pack W [n, k] with the per-group clipping ratio that minimizes the
    squared reconstruction error (ratios (20 - i)/20, i = 0..10); same packed format."""
    _need_cuda("w", w)
    if w.dim() != 2 or w.dtype not in _DTYPE_CODE:
        raise ValueError("w must be a 2-D fp32, fp16 or bf16 tensor")
    n, k = w.shape
    p = out if out is not None else empty_packed(n, k, group_size, symmetric, w.device)
    _check_packed(p, w.device, n, k, group_size, bool(symmetric))
    _check(_load().q4_quantize_pack_mse(_dev_ptr(w), _DTYPE_CODE[w.dtype], n, k, group_size,
                                        int(bool(symmetric)), _dev_ptr(p.qweight),
                                        _dev_ptr(p.scales), _dev_ptr(p.zeros), _stream(w)))
    return p


def q4_quantize_pack_grouped(ws, group_size: int = 128, symmetric: bool = False, outs=None):
    """Quantize/pack up to 8 matrices (same dtype, group size and mode; each its own shape)
    in one launch; the same bits as one q4_quantize_pack call per matrix."""
    ws = list(ws)
    count = len(ws)
    if not 1 <= count <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} matrices per call")
    for w in ws:
        _need_cuda("w", w, ws[0].device)
        if w.dim() != 2 or w.dtype not in _DTYPE_CODE or w.dtype != ws[0].dtype:
            raise ValueError("matrices must be 2-D fp32, fp16 or bf16 tensors of one dtype")
    ps = list(outs) if outs is not None else [
        empty_packed(w.shape[0], w.shape[1], group_size, symmetric, w.device) for w in ws]
    if len(ps) != count:
        raise ValueError("one output per matrix")
    for w, pk in zip(ws, ps):
        _check_packed(pk, ws[0].device, w.shape[0], w.shape[1], group_size, bool(symmetric))
    arr = (QuantProblem * count)()
    for i, (w, p) in enumerate(zip(ws, ps)):
        arr[i] = QuantProblem(w.data_ptr(), w.shape[0], w.shape[1], p.qweight.data_ptr(),
                              p.scales.data_ptr(), None if p.zeros is None else p.zeros.data_ptr())
    _check(_load().q4_quantize_pack_grouped(arr, count, _DTYPE_CODE[ws[0].dtype], group_size,
                                            int(bool(symmetric)), _stream(ws[0])))
    return ps


def q4_dequant(p: PackedWeight, out_dtype: torch.dtype = torch.float32,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Full dequantization S * (u - z) -> [n, k] in out_dtype (fp32 exact)."""
    _need_cuda("qweight", p.qweight)
    _check_packed(p, p.qweight.device)
    o = out if out is not None else torch.empty((p.n, p.k), dtype=out_dtype,
                                                device=p.qweight.device)
    _need("out", o, (p.n, p.k), tuple(_DTYPE_CODE), p.qweight.device)
    _check(_load().q4_dequant(_dev_ptr(p.qweight), _dev_ptr(p.scales), _dev_ptr(p.zeros),
                              p.n, p.k, p.group_size, int(p.symmetric), _dev_ptr(o),
                              _DTYPE_CODE[o.dtype], _stream(o)))
    return o


def q4_check_scales(p: PackedWeight) -> Tuple[int, int, int]:
    """Corrupted scale detection: (number of non-finite scales, number of negative scales,
    flat index of the first such scale or -1) over p's fp16 scales (q4_check_scales)."""
    _need_cuda("scales", p.scales)
    _check_packed(p, p.scales.device)
    res = torch.empty(3, dtype=torch.int64, device=p.scales.device)
    _check(_load().q4_check_scales(_dev_ptr(p.scales), p.n, p.k, p.group_size, _dev_ptr(res),
                                   _stream(res)))
    nonfinite, negative, first = (int(v) for v in res.cpu().tolist())
    return nonfinite, negative, first


def q4_w4a16_gemm_workspace(m: int, n: int, k: int, group_size: int) -> int:
    """Bytes of workspace q4_w4a16_gemm_ws uses to split this product's K range (0: none)."""
    return int(_load().q4_w4a16_gemm_workspace(m, n, k, group_size))


def q4_w4a16_gemm(x: torch.Tensor, p: PackedWeight,
                  out: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.float32,
                  workspace: Optional[torch.Tensor] = None, split: bool = True) -> torch.Tensor:
    """y = x · (S (u - z))^T, x [m, k] fp16/bf16, y [m, n] fp32, or fp16 / bf16 rounded from
    the fp32 sums in the kernel's epilogue (q4_w4a16_gemm_ws).  A product that would leave
    compute units idle splits its K range into a workspace: ``workspace`` (a contiguous
    device tensor of at least q4_w4a16_gemm_workspace bytes), allocated here when needed
    and not given; ``split=False`` runs every product unsplit (q4_w4a16_gemm_out)."""
    _need_cuda("x", x)
    if x.dim() != 2 or x.dtype not in (torch.float16, torch.bfloat16) or x.shape[1] != p.k:
        raise ValueError("x must be [m, k] fp16 or bf16 with k matching the packed weight")
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("the output is fp32, fp16 or bf16")
    m = x.shape[0]
    _check_packed(p, x.device)
    y = out if out is not None else torch.empty((m, p.n), dtype=out_dtype, device=x.device)
    _need("out", y, (m, p.n), tuple(_DTYPE_CODE), x.device)
    if not split:
        workspace = None
    elif workspace is None:
        need = q4_w4a16_gemm_workspace(m, p.n, p.k, p.group_size)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0
    if workspace is not None:
        _need_workspace("workspace", workspace, x.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_load().q4_w4a16_gemm_ws(_dev_ptr(x), _DTYPE_CODE[x.dtype], m, _dev_ptr(p.qweight),
                                    _dev_ptr(p.scales), _dev_ptr(p.zeros), p.n, p.k,
                                    p.group_size, int(p.symmetric), _dev_ptr(y),
                                    _DTYPE_CODE[out_dtype], _dev_ptr(workspace) if workspace is not None
                                    else None, ws_bytes, _stream(x)))
    return y


def q4_w4a16_gemm_grouped(xs, packs, outs=None, out_dtype=torch.float32):
    """y_i = x_i · (S_i (u_i - z_i))^T for up to 8 problems sharing m, k, group size,
    symmetry and activation dtype; with m <= 16 they run in one launch.  xs may be a
    single tensor (shared by all problems) or one tensor per problem.  The outputs are
    out_dtype (fp32, or fp16 / bf16 rounded in the epilogue), or that of outs."""
    packs = list(packs)
    count = len(packs)
    if not 1 <= count <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} problems per call")
    xs = [xs] * count if isinstance(xs, torch.Tensor) else list(xs)
    if len(xs) != count:
        raise ValueError("one activation tensor per problem (or one shared)")
    p0, x0 = packs[0], xs[0]
    for x, p in zip(xs, packs):
        _need_cuda("x", x, xs[0].device)
        _check_packed(p, xs[0].device)
        if (x.shape != x0.shape or x.dtype != x0.dtype or x.dim() != 2 or p.k != p0.k
                or p.group_size != p0.group_size or p.symmetric != p0.symmetric or x.shape[1] != p.k):
            raise ValueError("problems must share m, k, group size, symmetry and dtype")
    if x0.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("activations must be fp16 or bf16")
    m = x0.shape[0]
    if outs is not None:
        outs = list(outs)
        out_dtype = outs[0].dtype
        if any(o.dtype != out_dtype for o in outs):
            raise ValueError("every output of a grouped call has one dtype")
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("the output is fp32, fp16 or bf16")
    ys = outs if outs is not None else [
        torch.empty((m, p.n), dtype=out_dtype, device=x0.device) for p in packs]
    if len(ys) != count:
        raise ValueError("one output per problem")
    for y, p in zip(ys, packs):
        _need("out", y, (m, p.n), (out_dtype,), x0.device)
    arr = (GemmProblem * count)()
    for i, (x, p, y) in enumerate(zip(xs, packs, ys)):
        arr[i] = GemmProblem(x.data_ptr(), p.qweight.data_ptr(), p.scales.data_ptr(),
                             None if p.zeros is None else p.zeros.data_ptr(), p.n, y.data_ptr())
    if out_dtype == torch.float32:
        _check(_load().q4_w4a16_gemm_grouped(arr, count, _DTYPE_CODE[x0.dtype], m, p0.k,
                                             p0.group_size, int(p0.symmetric), _stream(x0)))
    else:
        _check(_load().q4_w4a16_gemm_grouped_out(arr, count, _DTYPE_CODE[x0.dtype], m, p0.k,
                                                 p0.group_size, int(p0.symmetric),
                                                 _DTYPE_CODE[out_dtype], _stream(x0)))
    return ys


# ------------------------------------------------------------------ INT4 KV cache

@dataclass
class KvCache:
    """One layer's head-major INT4 K (or V) cache: token t of head h is row h * t_cap + t
    of the packed format with k = head_dim: qcache int32 [heads*t_cap, d/8], scache
    float16 [heads*t_cap, d/g], zcache int32 [heads*t_cap, ceil(d/g/8)] or None when
    symmetric."""
    qcache: torch.Tensor
    scache: torch.Tensor
    zcache: Optional[torch.Tensor]
    heads: int
    t_cap: int
    head_dim: int
    group_size: int
    symmetric: bool


def empty_kv_cache(heads: int, t_cap: int, head_dim: int, group_size: int = 32,
                   symmetric: bool = False, device="cuda") -> KvCache:
    p = empty_packed(heads * t_cap, head_dim, group_size, symmetric, device)
    return KvCache(p.qweight, p.scales, p.zeros, heads, t_cap, head_dim, group_size,
                   bool(symmetric))


def q4_kv_quantize(kv: torch.Tensor, cache: KvCache, t0: int) -> KvCache:
    """Quantize kv [t_new, heads, head_dim] (fp32 / fp16 / bf16) into token positions
    t0 .. t0 + t_new - 1 of ``cache``."""
    _need_cuda("kv", kv)
    if kv.dim() != 3 or kv.dtype not in _DTYPE_CODE:
        raise ValueError("kv must be a 3-D fp32, fp16 or bf16 tensor [t_new, heads, head_dim]")
    t_new, heads, d = kv.shape
    if heads != cache.heads or d != cache.head_dim:
        raise ValueError("kv does not match the cache's heads / head_dim")
    _check_cache("cache", cache, kv.device)
    _check(_load().q4_kv_quantize(_dev_ptr(kv), _DTYPE_CODE[kv.dtype], t_new, heads, d,
                                  cache.group_size, int(cache.symmetric), cache.t_cap, t0,
                                  _dev_ptr(cache.qcache), _dev_ptr(cache.scache),
                                  _dev_ptr(cache.zcache), _stream(kv)))
    return cache


def q4_kv_attention_workspace(heads: int, head_dim: int, n_tok: int) -> int:
    return int(_load().q4_kv_attention_workspace(heads, head_dim, n_tok))


def q4_kv_attention(q: torch.Tensor, kcache: KvCache, vcache: KvCache, n_tok: int,
                    scale: float, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention of q [heads, head_dim] (fp16 / bf16) over tokens 0 .. n_tok-1 of
    the INT4 caches; returns out [heads, head_dim] fp32.  A ``workspace`` passed in is
    sized with q4_kv_attention_workspace for the largest n_tok it will serve."""
    _need_cuda("q", q)
    if q.dim() != 2 or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be a 2-D fp16 or bf16 tensor [heads, head_dim]")
    heads, d = q.shape
    for c in (kcache, vcache):
        if (c.heads, c.head_dim) != (heads, d):
            raise ValueError("q does not match the caches' heads / head_dim")
    if (kcache.group_size, kcache.symmetric, kcache.t_cap) != \
            (vcache.group_size, vcache.symmetric, vcache.t_cap):
        raise ValueError("K and V caches must share group_size, symmetry and t_cap")
    _check_cache("kcache", kcache, q.device)
    _check_cache("vcache", vcache, q.device)
    if out is None:
        out = torch.empty((heads, d), dtype=torch.float32, device=q.device)
    _need("out", out, (heads, d), (torch.float32,), q.device)
    need = q4_kv_attention_workspace(heads, d, n_tok)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need_workspace("workspace", workspace, q.device)
    _check(_load().q4_kv_attention(
        _dev_ptr(q), _DTYPE_CODE[q.dtype], heads, d, n_tok, kcache.t_cap,
        _dev_ptr(kcache.qcache), _dev_ptr(kcache.scache), _dev_ptr(kcache.zcache),
        _dev_ptr(vcache.qcache), _dev_ptr(vcache.scache), _dev_ptr(vcache.zcache),
        kcache.group_size, int(kcache.symmetric), float(scale), _dev_ptr(out),
        _dev_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return out


def q4_kv_attention_noalloc(q: torch.Tensor, kcache: KvCache, vcache: KvCache, n_tok: int,
                            scale: float, out: torch.Tensor) -> torch.Tensor:
    """q4_kv_attention without a workspace, for callers that cannot allocate (HIP graph
    capture, serving loops): the partials go to the library's fixed per-GPU scratch, so
    ``out`` [heads, head_dim] fp32 must be passed in.  Calls on one GPU share that scratch
    and must not overlap."""
    _need_cuda("q", q)
    if q.dim() != 2 or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be a 2-D fp16 or bf16 tensor [heads, head_dim]")
    _need("out", out, tuple(q.shape), (torch.float32,), q.device)
    _check_cache("kcache", kcache, q.device)
    _check_cache("vcache", vcache, q.device)
    heads, d = q.shape
    for c in (kcache, vcache):
        if (c.heads, c.head_dim) != (heads, d):
            raise ValueError("q does not match the caches' heads / head_dim")
    if (kcache.group_size, kcache.symmetric, kcache.t_cap) != \
            (vcache.group_size, vcache.symmetric, vcache.t_cap):
        raise ValueError("K and V caches must share group_size, symmetry and t_cap")
    _check(_load().q4_kv_attention_noalloc(
        _dev_ptr(q), _DTYPE_CODE[q.dtype], heads, d, n_tok, kcache.t_cap,
        _dev_ptr(kcache.qcache), _dev_ptr(kcache.scache), _dev_ptr(kcache.zcache),
        _dev_ptr(vcache.qcache), _dev_ptr(vcache.scache), _dev_ptr(vcache.zcache),
        kcache.group_size, int(kcache.symmetric), float(scale), _dev_ptr(out), _stream(q)))
    return out


# ------------------------------------------------------------------ GPTQ

def q4_gptq_workspace(n: int, k: int, group_size: int) -> int:
    return int(_load().q4_gptq_workspace(n, k, group_size))


def q4_gptq_act_order_workspace(n: int, k: int, group_size: int) -> int:
    return int(_load().q4_gptq_act_order_workspace(n, k, group_size))


def q4_gptq_quantize(w: torch.Tensor, x: torch.Tensor, group_size: int = 128,
                     symmetric: bool = False, damp: float = 0.01,
                     out: Optional[PackedWeight] = None,
                     workspace: Optional[torch.Tensor] = None,
                     act_order: bool = False) -> PackedWeight:
    """GPTQ-quantize W [n, k] (fp32 / fp16 / bf16) against calibration activations
    x [tokens, k] (fp16 / bf16); same packed format, RTN's group scales and zero points.
    With ``act_order`` the columns are swept by descending activation energy
    (q4_gptq_quantize_act_order)."""
    _need_cuda("w", w)
    _need_cuda("x", x, w.device)
    if w.dim() != 2 or w.dtype not in _DTYPE_CODE:
        raise ValueError("w must be a 2-D fp32, fp16 or bf16 tensor")
    if x.dim() != 2 or x.dtype not in (torch.float16, torch.bfloat16) or x.shape[1] != w.shape[1]:
        raise ValueError("x must be a 2-D fp16 or bf16 tensor [tokens, k]")
    n, k = w.shape
    p = out if out is not None else empty_packed(n, k, group_size, symmetric, w.device)
    _check_packed(p, w.device, n, k, group_size, bool(symmetric))
    need = (q4_gptq_act_order_workspace if act_order else q4_gptq_workspace)(n, k, group_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=w.device)
    _need_workspace("workspace", workspace, w.device)
    entry = _load().q4_gptq_quantize_act_order if act_order else _load().q4_gptq_quantize
    _check(entry(_dev_ptr(w), _DTYPE_CODE[w.dtype], n, k, _dev_ptr(x), _DTYPE_CODE[x.dtype],
                 x.shape[0], group_size, int(bool(symmetric)), float(damp), _dev_ptr(p.qweight),
                 _dev_ptr(p.scales), _dev_ptr(p.zeros), _dev_ptr(workspace),
                 workspace.numel() * workspace.element_size(), _stream(w)))
    return p
