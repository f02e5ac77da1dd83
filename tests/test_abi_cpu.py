"""The C ABI on the CPU: the library loads, exports every function include/q4.h
declares, and rejects bad arguments on the host before any device work (so these
calls are safe without a GPU).  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import w4a16_group_wise_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")

OK, NULL, SHAPE, GROUP, DTYPE, ALIGN = 0, 1, 2, 3, 4, 5
A16 = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = q4.lib()
    names = declared_functions()
    assert set(names) == set(q4.EXPORTED), names
    for nm in names:
        assert hasattr(lib, nm), nm


def test_layout_version_and_initial_state():
    assert q4.q4_layout_version() == 1
    assert q4.q4_last_kernel() == ""


def test_status_strings():
    lib = q4.lib()
    for code in range(8):
        s = lib.q4_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.q4_status_str(99).decode() == "unknown status"


def test_size_helpers_match_oracle_and_pages(orc):
    for (n, k, g) in [(256, 512, 128), (4096, 4096, 128), (11008, 4096, 32), (4096, 11008, 128),
                      (28672, 8192, 128), (3, 96, 32), (1, 64, 64)]:
        assert (q4.q4_qweight_words(n, k), q4.q4_scale_count(n, k, g),
                q4.q4_zero_words(n, k, g)) == orc.sizes(n, k, g)
    # fp16 scale per 128 weights: 0.015625 bytes per weight
    assert q4.q4_scale_count(4096, 4096, 128) * 2 / 4096 ** 2 == 0.015625
    # symmetric group 32: 4.5 bits per weight (32 codes + one fp16 scale)
    n, k = 64, 4096
    assert (q4.q4_qweight_words(n, k) * 32 + q4.q4_scale_count(n, k, 32) * 16) / (n * k) == 4.5
    # rejected layouts report -1
    assert q4.q4_scale_count(4, 100, 32) == -1
    assert q4.q4_zero_words(4, 128, 16) == -1
    assert q4.q4_qweight_words(0, 8) == -1


def _qp(w=A16, dt=BF16, n=16, k=256, g=128, sym=0, qw=A16, sc=A16, zr=A16):
    return q4.lib().q4_quantize_pack(w, dt, n, k, g, sym, qw, sc, zr, None)


def _dq(qw=A16, sc=A16, zr=A16, n=16, k=256, g=128, sym=0, out=A16, od=F32):
    return q4.lib().q4_dequant(qw, sc, zr, n, k, g, sym, out, od, None)


def _mm(x=A16, xd=BF16, m=1, qw=A16, sc=A16, zr=A16, n=16, k=256, g=128, sym=0, y=A16):
    return q4.lib().q4_w4a16_gemm(x, xd, m, qw, sc, zr, n, k, g, sym, y, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _qp(g=16), GROUP), (lambda: _qp(g=256), GROUP), (lambda: _qp(k=96, g=64), SHAPE),
    (lambda: _qp(n=0), SHAPE), (lambda: _qp(k=0), SHAPE), (lambda: _qp(n=-1), SHAPE),
    (lambda: _qp(n=1 << 31), SHAPE), (lambda: _qp(n=1 << 30, k=1 << 20), SHAPE),
    (lambda: _qp(dt=7), DTYPE), (lambda: _qp(w=None), NULL), (lambda: _qp(qw=None), NULL),
    (lambda: _qp(sc=None), NULL), (lambda: _qp(zr=None), NULL),
    (lambda: _qp(w=A16 + 8), ALIGN), (lambda: _qp(qw=A16 + 4), ALIGN),
    (lambda: _qp(sc=A16 + 1), ALIGN), (lambda: _qp(zr=A16 + 2), ALIGN),
    (lambda: _dq(g=48), GROUP), (lambda: _dq(k=200), SHAPE), (lambda: _dq(od=5), DTYPE),
    (lambda: _dq(out=None), NULL), (lambda: _dq(zr=None), NULL), (lambda: _dq(out=A16 + 4), ALIGN),
    (lambda: _mm(m=0), SHAPE), (lambda: _mm(m=-3), SHAPE), (lambda: _mm(xd=F32), DTYPE),
    (lambda: _mm(x=None), NULL), (lambda: _mm(y=None), NULL), (lambda: _mm(zr=None), NULL),
    (lambda: _mm(x=A16 + 2), ALIGN), (lambda: _mm(y=A16 + 2), ALIGN), (lambda: _mm(g=100), GROUP),
    (lambda: _mm(k=320, g=128), SHAPE), (lambda: _mm(k=(1 << 22) + 128), SHAPE),
    (lambda: _mm(m=1 << 20, n=(1 << 18) + 1), SHAPE), (lambda: _mm(n=(1 << 25) + 1, k=128), SHAPE),
])
def test_host_validation_rejects_before_launch(call, code):
    assert call() == code
    assert q4.q4_last_kernel() == ""  # nothing was launched


def _mmo(yd=BF16, y=A16, m=1, **kw):
    a = dict(x=A16, xd=BF16, qw=A16, sc=A16, zr=A16, n=16, k=256, g=128, sym=0)
    a.update(kw)
    return q4.lib().q4_w4a16_gemm_out(a["x"], a["xd"], m, a["qw"], a["sc"], a["zr"], a["n"], a["k"],
                                      a["g"], a["sym"], y, yd, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _mmo(yd=3), DTYPE), (lambda: _mmo(yd=-1), DTYPE), (lambda: _mmo(y=None), NULL),
    (lambda: _mmo(yd=F32, y=A16 + 2), ALIGN), (lambda: _mmo(yd=BF16, y=A16 + 1), ALIGN),
    (lambda: _mmo(yd=F16, y=A16 + 1), ALIGN), (lambda: _mmo(m=0), SHAPE),
    (lambda: _mmo(xd=F32), DTYPE),
])
def test_output_dtype_validation_rejects_before_launch(call, code):
    """The output-dtype entry point: y_dtype is fp32, fp16 or bf16; a 16-bit y needs only
    2-byte alignment (checked here by a y 2 bytes past a 16-byte boundary passing the
    alignment rule and failing later on m)."""
    assert call() == code
    assert q4.q4_last_kernel() == ""


def test_output_dtype_16bit_alignment_is_two_bytes():
    assert _mmo(yd=BF16, y=A16 + 2, m=0) == SHAPE  # alignment passed, shape rejected
    assert _mmo(yd=F32, y=A16 + 2, m=0) == SHAPE   # shape is checked first
    arr = (q4.GemmProblem * 2)()
    arr[0] = q4.GemmProblem(A16, A16, A16, A16, 16, A16 + 2)
    arr[1] = q4.GemmProblem(A16, A16, A16, A16, 16, A16)
    assert q4.lib().q4_w4a16_gemm_grouped_out(arr, 2, BF16, 1, 256, 128, 0, 4, None) == DTYPE
    assert q4.lib().q4_w4a16_gemm_grouped_out(arr, 2, BF16, 1, 256, 128, 0, F32, None) == ALIGN


def test_symmetric_accepts_null_zeros_in_validation():
    # symmetric mode needs no zero points; with a bad group the call still fails on the
    # group (validated first), proving the NULL zeros pointer itself is accepted
    assert _qp(sym=1, zr=None, g=16) == GROUP
    assert _mm(sym=1, zr=None, m=0) == SHAPE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        q4.q4_quantize_pack(torch.zeros(4, 128), 128, False)


def _grouped(probs, count=None, xd=BF16, m=1, k=256, g=128, sym=0):
    arr = (q4.GemmProblem * max(1, len(probs)))()
    for i, pr in enumerate(probs):
        arr[i] = pr
    return q4.lib().q4_w4a16_gemm_grouped(arr if probs else None, len(probs) if count is None else count,
                                          xd, m, k, g, sym, None)


def _prob(x=A16, qw=A16, sc=A16, zr=A16, n=16, y=A16):
    return q4.GemmProblem(x, qw, sc, zr, n, y)


@pytest.mark.parametrize("call,code", [
    (lambda: _grouped([]), NULL),
    (lambda: _grouped([_prob()], count=0), SHAPE),
    (lambda: _grouped([_prob()] * 9), SHAPE),
    (lambda: _grouped([_prob(), _prob(n=0)]), SHAPE),
    (lambda: _grouped([_prob(), _prob(y=None)]), NULL),
    (lambda: _grouped([_prob(), _prob(zr=None)]), NULL),
    (lambda: _grouped([_prob(x=A16 + 2), _prob()]), ALIGN),
    (lambda: _grouped([_prob(), _prob()], g=100), GROUP),
    (lambda: _grouped([_prob(), _prob()], xd=F32), DTYPE),
    (lambda: _grouped([_prob(), _prob()], m=0), SHAPE),
    (lambda: _grouped([_prob(), _prob()], k=(1 << 22) + 128), SHAPE),
])
def test_grouped_validation_rejects_before_launch(call, code):
    """Every entry is checked before anything is enqueued; the first failure is returned."""
    assert call() == code
    assert q4.q4_last_kernel() == ""


def test_grouped_symmetric_accepts_null_zeros_in_validation():
    # a bad group size is reported although every zeros pointer is NULL: NULL is accepted
    assert _grouped([_prob(zr=None), _prob(zr=None)], g=16, sym=1) == GROUP


def _qgrouped(probs, count=None, wd=BF16, g=128, sym=0):
    arr = (q4.QuantProblem * max(1, len(probs)))()
    for i, pr in enumerate(probs):
        arr[i] = pr
    return q4.lib().q4_quantize_pack_grouped(arr if probs else None,
                                             len(probs) if count is None else count, wd, g, sym, None)


def _qprob(w=A16, n=16, k=256, qw=A16, sc=A16, zr=A16):
    return q4.QuantProblem(w, n, k, qw, sc, zr)


@pytest.mark.parametrize("call,code", [
    (lambda: _qgrouped([]), NULL),
    (lambda: _qgrouped([_qprob()], count=0), SHAPE),
    (lambda: _qgrouped([_qprob()] * 9), SHAPE),
    (lambda: _qgrouped([_qprob(), _qprob(n=0)]), SHAPE),
    (lambda: _qgrouped([_qprob(), _qprob(k=200)]), SHAPE),
    (lambda: _qgrouped([_qprob(), _qprob(k=(1 << 28) + 128)]), SHAPE),
    (lambda: _qgrouped([_qprob(), _qprob(w=None)]), NULL),
    (lambda: _qgrouped([_qprob(), _qprob(zr=None)]), NULL),
    (lambda: _qgrouped([_qprob(), _qprob(qw=A16 + 4)]), ALIGN),
    (lambda: _qgrouped([_qprob(), _qprob(w=A16 + 8)]), ALIGN),
    (lambda: _qgrouped([_qprob(), _qprob()], g=48), GROUP),
    (lambda: _qgrouped([_qprob(), _qprob()], wd=7), DTYPE),
])
def test_grouped_quantize_validation_rejects_before_launch(call, code):
    """Every matrix is checked before anything is enqueued; the first failure is returned."""
    assert call() == code
    assert q4.q4_last_kernel() == ""


def test_quantize_row_length_limit():
    lib = q4.lib()
    assert lib.q4_quantize_pack(A16, F32, 1, (1 << 28) + 128, 128, 0, A16, A16, A16, None) == SHAPE
    assert _qgrouped([_qprob(zr=None), _qprob(zr=None)], g=16, sym=1) == GROUP


@pytest.mark.parametrize("args,code", [
    ((None, BF16, 4, 128, 128, 0, A16, A16, A16, None), NULL),
    ((A16, BF16, 4, 100, 32, 0, A16, A16, A16, None), SHAPE),
    ((A16, BF16, 4, 128, 16, 0, A16, A16, A16, None), GROUP),
    ((A16, 9, 4, 128, 128, 0, A16, A16, A16, None), DTYPE),
    ((A16, BF16, 4, 128, 128, 0, A16, A16, None, None), NULL),
    ((A16 + 4, BF16, 4, 128, 128, 0, A16, A16, A16, None), ALIGN),
    ((A16, F32, 1, (1 << 28) + 128, 128, 1, A16, A16, None, None), SHAPE),
])
def test_quantize_mse_validation_rejects_before_launch(args, code):
    assert q4.lib().q4_quantize_pack_mse(*args) == code
    assert q4.q4_last_kernel() == ""


def _kvq(kv=A16, dt=BF16, t_new=1, heads=4, d=128, g=32, sym=0, t_cap=16, t0=0, qc=A16, sc=A16,
         zc=A16):
    return q4.lib().q4_kv_quantize(kv, dt, t_new, heads, d, g, sym, t_cap, t0, qc, sc, zc, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _kvq(g=16), GROUP), (lambda: _kvq(t_new=0), SHAPE), (lambda: _kvq(t0=-1), SHAPE),
    (lambda: _kvq(t0=15, t_new=2), SHAPE), (lambda: _kvq(t0=16), SHAPE),
    (lambda: _kvq(heads=0), SHAPE), (lambda: _kvq(d=96, g=64), SHAPE),
    (lambda: _kvq(d=1 << 17, g=128), SHAPE), (lambda: _kvq(heads=1 << 16, t_cap=1 << 15), SHAPE),
    (lambda: _kvq(t_cap=0), SHAPE), (lambda: _kvq(dt=7), DTYPE), (lambda: _kvq(kv=None), NULL),
    (lambda: _kvq(qc=None), NULL), (lambda: _kvq(sc=None), NULL), (lambda: _kvq(zc=None), NULL),
    (lambda: _kvq(kv=A16 + 8), ALIGN), (lambda: _kvq(qc=A16 + 4), ALIGN),
    (lambda: _kvq(zc=A16 + 2), ALIGN),
])
def test_kv_quantize_validation_rejects_before_launch(call, code):
    assert call() == code
    assert q4.q4_last_kernel() == ""


def test_kv_quantize_symmetric_accepts_null_zeros():
    assert _kvq(sym=1, zc=None, g=16) == GROUP
    assert _kvq(sym=1, zc=None, t_new=0) == SHAPE


def _kva(q=A16, qd=BF16, heads=4, d=128, n_tok=100, t_cap=128, kq=A16, ks=A16, kz=A16, vq=A16,
         vs=A16, vz=A16, g=32, sym=0, scale=0.088, out=A16, ws=A16, ws_bytes=1 << 30):
    return q4.lib().q4_kv_attention(q, qd, heads, d, n_tok, t_cap, kq, ks, kz, vq, vs, vz, g, sym,
                                    scale, out, ws, ws_bytes, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _kva(g=16), GROUP), (lambda: _kva(d=96), SHAPE), (lambda: _kva(d=512), SHAPE),
    (lambda: _kva(d=64, g=128), SHAPE), (lambda: _kva(n_tok=0), SHAPE),
    (lambda: _kva(n_tok=129), SHAPE), (lambda: _kva(heads=0), SHAPE),
    (lambda: _kva(heads=65537, t_cap=128), SHAPE),
    (lambda: _kva(n_tok=(1 << 24) + 1, t_cap=(1 << 24) + 1, heads=1), SHAPE),
    (lambda: _kva(heads=1 << 10, t_cap=1 << 21), SHAPE),
    (lambda: _kva(qd=F32), DTYPE), (lambda: _kva(q=None), NULL), (lambda: _kva(out=None), NULL),
    (lambda: _kva(ws=None), NULL), (lambda: _kva(kz=None), NULL), (lambda: _kva(vs=None), NULL),
    (lambda: _kva(vq=None), NULL), (lambda: _kva(q=A16 + 8), ALIGN),
    (lambda: _kva(ws=A16 + 4), ALIGN), (lambda: _kva(out=A16 + 2), ALIGN),
    (lambda: _kva(kq=A16 + 4), ALIGN), (lambda: _kva(vz=A16 + 2), ALIGN),
    (lambda: _kva(ws_bytes=16), SHAPE),
])
def test_kv_attention_validation_rejects_before_launch(call, code):
    assert call() == code
    assert q4.q4_last_kernel() == ""


def _kvn(q=A16, qd=BF16, heads=4, d=128, n_tok=100, t_cap=128, kq=A16, ks=A16, kz=A16, vq=A16,
         vs=A16, vz=A16, g=32, sym=0, scale=0.088, out=A16):
    return q4.lib().q4_kv_attention_noalloc(q, qd, heads, d, n_tok, t_cap, kq, ks, kz, vq, vs, vz, g,
                                            sym, scale, out, None)


SCRATCH = 7


@pytest.mark.parametrize("call,code", [
    (lambda: _kvn(g=16), GROUP), (lambda: _kvn(d=96), SHAPE), (lambda: _kvn(n_tok=129), SHAPE),
    (lambda: _kvn(heads=0), SHAPE), (lambda: _kvn(qd=F32), DTYPE), (lambda: _kvn(q=None), NULL),
    (lambda: _kvn(out=None), NULL), (lambda: _kvn(kz=None), NULL), (lambda: _kvn(q=A16 + 8), ALIGN),
    (lambda: _kvn(out=A16 + 2), ALIGN), (lambda: _kvn(vz=A16 + 2), ALIGN),
    # partials of 2048 heads x 32 chunks x 258 floats: beyond the 16 MiB scratch
    (lambda: _kvn(heads=2048, d=256, g=64, n_tok=8192, t_cap=8192), SCRATCH),
    (lambda: _kvn(heads=65536, d=64, g=64, n_tok=1, t_cap=1), SCRATCH),
])
def test_kv_attention_noalloc_validation_rejects_before_launch(call, code):
    assert call() == code
    assert q4.q4_last_kernel() == ""


def test_kv_attention_noalloc_scratch_size():
    lib = q4.lib()
    assert lib.q4_kv_attention_noalloc_max_bytes() == 16 << 20
    # the 7B decode step (32 heads of 128 over 4096 tokens) needs 32 x 64 x 130 x 4 bytes
    assert lib.q4_kv_attention_workspace(32, 128, 4096) <= lib.q4_kv_attention_noalloc_max_bytes()


def test_kv_attention_symmetric_accepts_null_zeros():
    assert _kva(sym=1, kz=None, vz=None, g=16) == GROUP


def test_kv_attention_workspace_size():
    # (head_dim + 2) floats for each of at most ceil(n_tok * head_dim / 8192) chunks per
    # head; never smaller for a larger n_tok
    lib = q4.lib()
    for heads, d, n in [(32, 128, 4096), (1, 128, 5000), (3, 64, 777), (64, 256, 1), (8, 128, 4113)]:
        assert lib.q4_kv_attention_workspace(heads, d, n) == 4 * heads * (d + 2) * -(-n * d // 8192)
    assert lib.q4_kv_attention_workspace(32, 128, 4096) == 32 * 64 * 130 * 4
    for heads, d in [(1, 256), (2, 128), (32, 128), (5, 64)]:
        sizes = [lib.q4_kv_attention_workspace(heads, d, n) for n in range(1, 20000, 7)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert lib.q4_kv_attention_workspace(32, 96, 4096) == -1
    assert lib.q4_kv_attention_workspace(0, 128, 4096) == -1
    assert lib.q4_kv_attention_workspace(4, 128, 0) == -1


def _gq(w=A16, wd=BF16, n=16, k=256, x=A16, xd=BF16, tokens=64, g=128, sym=0, damp=0.01, qw=A16, sc=A16,
        zr=A16, ws=A16, ws_bytes=1 << 40, act_order=False):
    entry = q4.lib().q4_gptq_quantize_act_order if act_order else q4.lib().q4_gptq_quantize
    return entry(w, wd, n, k, x, xd, tokens, g, sym, damp, qw, sc, zr, ws, ws_bytes, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _gq(g=16), GROUP), (lambda: _gq(k=200), SHAPE), (lambda: _gq(tokens=0), SHAPE),
    (lambda: _gq(k=32768 + 128), SHAPE), (lambda: _gq(damp=0.0), SHAPE), (lambda: _gq(damp=-1.0), SHAPE),
    (lambda: _gq(damp=float("nan")), SHAPE), (lambda: _gq(damp=2.0), SHAPE), (lambda: _gq(xd=F32), DTYPE),
    (lambda: _gq(wd=7), DTYPE), (lambda: _gq(x=None), NULL), (lambda: _gq(ws=None), NULL),
    (lambda: _gq(w=None), NULL), (lambda: _gq(zr=None), NULL), (lambda: _gq(x=A16 + 2), ALIGN),
    (lambda: _gq(ws=A16 + 4), ALIGN), (lambda: _gq(ws_bytes=1024), SHAPE),
])
def test_gptq_validation_rejects_before_launch(call, code):
    assert call() == code
    assert q4.q4_last_kernel() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(g=16), GROUP), (dict(k=200), SHAPE), (dict(tokens=0), SHAPE), (dict(damp=0.0), SHAPE),
    (dict(xd=F32), DTYPE), (dict(x=None), NULL), (dict(ws=A16 + 4), ALIGN),
    (dict(n=16, k=256, ws_bytes=4 * (256 * 256 + 16 * 256 + 256 * 16)), SHAPE),
])
def test_gptq_act_order_validation(kw, code):
    """The act-order entry point shares the rules, and needs its larger workspace: the
    natural-order size is refused."""
    assert _gq(act_order=True, **kw) == code
    assert q4.q4_last_kernel() == ""


def test_gptq_workspace_size():
    lib = q4.lib()
    assert lib.q4_gptq_workspace(11008, 4096, 128) == 4 * (4096 * 4096 + 11008 * 4096 + 256 * 11008)
    assert lib.q4_gptq_workspace(16, 200, 32) == -1
    assert lib.q4_gptq_workspace(16, 32768 + 128, 128) == -1
    n, k = 11008, 4096
    assert lib.q4_gptq_act_order_workspace(n, k, 128) == (lib.q4_gptq_workspace(n, k, 128)
                                                           + 4 * 3 * k + n * k)
    assert lib.q4_gptq_act_order_workspace(16, 200, 32) == -1


def _gws(x=A16, xd=BF16, m=128, qw=A16, sc=A16, zr=A16, n=4096, k=11008, g=128, sym=0, y=A16, yd=F32,
         ws=A16, ws_bytes=1 << 40):
    return q4.lib().q4_w4a16_gemm_ws(x, xd, m, qw, sc, zr, n, k, g, sym, y, yd, ws, ws_bytes, None)


def test_gemm_workspace_size_and_rules():
    """Split-K sizes (this host has no GPU: 256 CUs assumed): parts x m x n fp32 partials for
    a narrow mid-size product, 0 where the product does not split, -1 for rejected sizes;
    the workspace entry point refuses a short or misaligned workspace before launching."""
    lib = q4.lib()
    # 128 x 4096: 32 tiles of 128 x 128 -> 8 parts (172 stages, at least 8 per part)
    assert lib.q4_w4a16_gemm_workspace(128, 4096, 11008, 128) == 8 * 128 * 4096 * 4
    assert lib.q4_w4a16_gemm_workspace(16, 4096, 11008, 128) == 0     # the GEMV
    assert lib.q4_w4a16_gemm_workspace(64, 4096, 11008, 128) == 0     # chunked GEMV
    assert lib.q4_w4a16_gemm_workspace(2048, 28672, 8192, 128) == 0   # tiles fill the CUs
    assert lib.q4_w4a16_gemm_workspace(128, 4096, 96, 32) == 0        # too few stages
    assert lib.q4_w4a16_gemm_workspace(128, 4096, 100, 32) == -1
    need = lib.q4_w4a16_gemm_workspace(128, 4096, 11008, 128)
    assert _gws(ws_bytes=need - 1) == SHAPE
    assert _gws(ws=A16 + 4) == ALIGN
    assert _gws(g=48) == GROUP and _gws(x=None) == NULL
    assert q4.q4_last_kernel() == ""

