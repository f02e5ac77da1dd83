"""The Python binding checks every tensor against the sizes it passes to the C ABI, on the
CPU, before any kernel could run: a too-short output, a packed weight whose tensors
disagree with its n / k / group size, a wrong dtype, a missing zero-point tensor, a
non-contiguous view or tensors on different devices raise ValueError (or TypeError).  A
kernel would otherwise write past a buffer.

No GPU is used: tensors live on torch's "meta" device and the device-placement check is
replaced by one that accepts it.  Calls that pass validation reach the C ABI with NULL
pointers (meta tensors have no storage), which refuses them with Q4_ERR_NULL before
anything is enqueued; that status shows the binding let them through.  The library's
source digest and the stale-library refusal are checked here too."""
import pytest
import torch

import w4a16_group_wise_q4_amd as q4
from w4a16_group_wise_q4_amd import _build

META = torch.device("meta")
NULL = 1


@pytest.fixture(autouse=True)
def meta_tensors_pass_placement(monkeypatch):
    def need(name, t, device=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if device is not None and t.device != device:
            raise ValueError(f"{name} on another device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    monkeypatch.setattr(q4, "_need_cuda", need)
    monkeypatch.setattr(q4, "_stream", lambda t: None)


def packed(n=48, k=512, g=128, sym=False, **over):
    G = k // g
    t = dict(qweight=torch.empty((n, k // 8), dtype=torch.int32, device=META),
             scales=torch.empty((n, G), dtype=torch.float16, device=META),
             zeros=None if sym else torch.empty((n, (G + 7) // 8), dtype=torch.int32, device=META))
    t.update(over)
    return q4.PackedWeight(n=n, k=k, group_size=g, symmetric=sym, **t)


def x16(m=3, k=512, dtype=torch.bfloat16):
    return torch.empty((m, k), dtype=dtype, device=META)


def refused_by_c(fn):
    with pytest.raises(q4.Q4Error) as e:
        fn()
    assert e.value.code == NULL


# ------------------------------------------------------------------ matmul

def test_gemm_valid_reaches_the_c_abi():
    refused_by_c(lambda: q4.q4_w4a16_gemm(x16(), packed()))
    refused_by_c(lambda: q4.q4_w4a16_gemm(x16(), packed(sym=True)))
    refused_by_c(lambda: q4.q4_w4a16_gemm(x16(), packed(),
                                          out=torch.empty((3, 48), dtype=torch.float16, device=META)))


@pytest.mark.parametrize("make", [
    lambda: packed(qweight=torch.empty((48, 63), dtype=torch.int32, device=META)),     # short rows
    lambda: packed(qweight=torch.empty((47, 64), dtype=torch.int32, device=META)),     # short n
    lambda: packed(qweight=torch.empty((48, 64), dtype=torch.int64, device=META)),     # dtype
    lambda: packed(scales=torch.empty((48, 4), dtype=torch.float32, device=META)),
    lambda: packed(scales=torch.empty((48, 3), dtype=torch.float16, device=META)),
    lambda: packed(zeros=None),                                                        # asym needs zeros
    lambda: packed(zeros=torch.empty((48, 2), dtype=torch.int32, device=META)),
    lambda: packed(sym=True, zeros=torch.empty((1, 1), dtype=torch.int32, device=META)),
    lambda: packed(scales=torch.empty((4, 48), dtype=torch.float16, device=META).t()),  # not contiguous
    lambda: packed(qweight=torch.empty((48, 64), dtype=torch.int32)),                  # another device
])
def test_gemm_refuses_bad_packed_weight(make):
    with pytest.raises((ValueError, TypeError)):
        q4.q4_w4a16_gemm(x16(), make())


@pytest.mark.parametrize("out", [
    lambda: torch.empty((3, 47), dtype=torch.float32, device=META),   # one column short
    lambda: torch.empty((2, 48), dtype=torch.float32, device=META),
    lambda: torch.empty((3 * 48,), dtype=torch.float32, device=META),
    lambda: torch.empty((3, 48), dtype=torch.float64, device=META),
    lambda: torch.empty((48, 3), dtype=torch.float32, device=META).t(),
    lambda: torch.empty((3, 48), dtype=torch.float32),
])
def test_gemm_refuses_bad_output(out):
    with pytest.raises(ValueError):
        q4.q4_w4a16_gemm(x16(), packed(), out=out())


def test_gemm_refuses_mismatched_k():
    with pytest.raises(ValueError):
        q4.q4_w4a16_gemm(x16(k=256), packed())


def test_grouped_checks_every_problem():
    refused_by_c(lambda: q4.q4_w4a16_gemm_grouped(x16(), [packed(), packed(n=17)]))
    with pytest.raises(ValueError):
        q4.q4_w4a16_gemm_grouped(x16(), [packed(), packed(n=17, scales=torch.empty(
            (16, 4), dtype=torch.float16, device=META))])
    outs = [torch.empty((3, 48), dtype=torch.float32, device=META),
            torch.empty((3, 16), dtype=torch.float32, device=META)]
    with pytest.raises(ValueError):
        q4.q4_w4a16_gemm_grouped(x16(), [packed(), packed(n=17)], outs=outs)
    with pytest.raises(ValueError):
        q4.q4_w4a16_gemm_grouped(x16(), [packed(), packed(n=17)], outs=outs[:1])


# ------------------------------------------------------------------ quantize, dequant

def test_quantize_checks_the_output():
    w = torch.empty((48, 512), dtype=torch.bfloat16, device=META)
    refused_by_c(lambda: q4.q4_quantize_pack(w, 128, False, out=packed()))
    for bad in (packed(n=40, qweight=torch.empty((40, 64), dtype=torch.int32, device=META),
                       scales=torch.empty((40, 4), dtype=torch.float16, device=META),
                       zeros=torch.empty((40, 1), dtype=torch.int32, device=META)),
                packed(g=64, scales=torch.empty((48, 8), dtype=torch.float16, device=META)),
                packed(sym=True),
                packed(zeros=torch.empty((48, 1), dtype=torch.int16, device=META))):
        with pytest.raises(ValueError):
            q4.q4_quantize_pack(w, 128, False, out=bad)
        with pytest.raises(ValueError):
            q4.q4_quantize_pack_mse(w, 128, False, out=bad)
    with pytest.raises(ValueError):
        q4.q4_quantize_pack_grouped([w, w], 128, False, outs=[packed(), packed(sym=True)])


def test_dequant_checks_the_output():
    refused_by_c(lambda: q4.q4_dequant(packed(), out=torch.empty((48, 512), dtype=torch.bfloat16,
                                                                 device=META)))
    for bad in (torch.empty((48, 511), dtype=torch.float32, device=META),
                torch.empty((48, 512), dtype=torch.int32, device=META),
                torch.empty((512, 48), dtype=torch.float32, device=META).t()):
        with pytest.raises(ValueError):
            q4.q4_dequant(packed(), out=bad)


# ------------------------------------------------------------------ KV cache, GPTQ

def cache(heads=4, t_cap=64, d=128, g=32, sym=False, **over):
    p = packed(n=heads * t_cap, k=d, g=g, sym=sym)
    t = dict(qcache=p.qweight, scache=p.scales, zcache=p.zeros)
    t.update(over)
    return q4.KvCache(heads=heads, t_cap=t_cap, head_dim=d, group_size=g, symmetric=sym, **t)


def test_kv_calls_check_caches_outputs_and_workspace():
    q = torch.empty((4, 128), dtype=torch.bfloat16, device=META)
    kv = torch.empty((2, 4, 128), dtype=torch.bfloat16, device=META)
    ws = torch.empty((1 << 16,), dtype=torch.uint8, device=META)
    refused_by_c(lambda: q4.q4_kv_quantize(kv, cache(), 0))
    refused_by_c(lambda: q4.q4_kv_attention(q, cache(), cache(), 10, 0.1, workspace=ws))
    out = torch.empty((4, 128), dtype=torch.float32, device=META)
    refused_by_c(lambda: q4.q4_kv_attention_noalloc(q, cache(), cache(), 10, 0.1, out))
    short = cache(qcache=torch.empty((4 * 64 - 1, 16), dtype=torch.int32, device=META))
    nozero = cache(zcache=None)
    for bad in (short, nozero):
        with pytest.raises(ValueError):
            q4.q4_kv_quantize(kv, bad, 0)
        with pytest.raises(ValueError):
            q4.q4_kv_attention(q, cache(), bad, 10, 0.1, workspace=ws)
        with pytest.raises(ValueError):
            q4.q4_kv_attention_noalloc(q, bad, cache(), 10, 0.1, out)
    for bad_out in (torch.empty((4, 127), dtype=torch.float32, device=META),
                    torch.empty((4, 128), dtype=torch.float16, device=META)):
        with pytest.raises(ValueError):
            q4.q4_kv_attention(q, cache(), cache(), 10, 0.1, out=bad_out, workspace=ws)
        with pytest.raises(ValueError):
            q4.q4_kv_attention_noalloc(q, cache(), cache(), 10, 0.1, bad_out)
    with pytest.raises(ValueError):
        q4.q4_kv_attention(q, cache(), cache(), 10, 0.1, workspace=torch.empty((1 << 16,), dtype=torch.uint8))


def test_gptq_checks_its_tensors():
    w = torch.empty((48, 512), dtype=torch.bfloat16, device=META)
    x = torch.empty((64, 512), dtype=torch.bfloat16, device=META)
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device=META)
    refused_by_c(lambda: q4.q4_gptq_quantize(w, x, 128, False, out=packed(), workspace=ws))
    with pytest.raises(ValueError):
        q4.q4_gptq_quantize(w, x, 128, False, out=packed(n=47, qweight=torch.empty(
            (47, 64), dtype=torch.int32, device=META)), workspace=ws)
    with pytest.raises(ValueError):
        q4.q4_gptq_quantize(w, torch.empty((64, 512), dtype=torch.bfloat16), 128, False,
                            out=packed(), workspace=ws)


# ------------------------------------------------------------------ the library itself

def test_library_digest_matches_its_sources():
    assert q4.q4_source_digest() == _build.source_digest()
    assert len(q4.q4_source_digest()) == 16


def test_stale_library_is_refused(monkeypatch):
    monkeypatch.setattr(q4, "_lib", None)
    monkeypatch.setattr(_build, "source_digest", lambda: "0" * 16)
    with pytest.raises(q4.StaleLibraryError):
        q4.lib()


def test_launch_record_before_any_call():
    assert q4.q4_last_kernels() == []
    assert q4.q4_last_launch_count() == 0
