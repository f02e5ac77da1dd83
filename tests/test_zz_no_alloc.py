"""q4_kv_attention_noalloc (the attention entry point that allocates nothing, for callers
that cannot call hipMalloc) against q4_kv_attention, through the C ABI.

Both run the same kernels with the same chunking and summation order, so the outputs must
be identical bit for bit; the second call is smaller than the first, so it runs on a
scratch still holding the first call's partials.  Sizes whose partials exceed the fixed
scratch are refused on the host.  The regular entry point's output is itself checked
against the CPU oracle within the fp32 attention bound (test_gpu_kv.py); the smaller call
is also checked against the oracle here.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic
import w4a16_group_wise_q4_amd as q4
from gpu_util import DEV, SENTINEL_F32, guard_intact, guarded, host_input, note
from test_gpu_kv import assert_attention_close, build_caches, cache_to_device, tolerance

pytestmark = pytest.mark.gpu

Q4_ERR_SCRATCH = 7


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_raw(q, kc, vc, n_tok, scale, out):
    """The C entry point called directly through ctypes (no Python-side allocation)."""
    heads, d = q.shape
    code = q4.lib().q4_kv_attention_noalloc(
        _p(q), 2 if q.dtype == torch.bfloat16 else 1, heads, d, n_tok, kc.t_cap,
        _p(kc.qcache), _p(kc.scache), _p(kc.zcache), _p(vc.qcache), _p(vc.scache), _p(vc.zcache),
        kc.group_size, int(kc.symmetric), ctypes.c_float(scale), _p(out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return int(code)


# (heads, head_dim, group, sym, n_tok, t_cap, q dtype): the 7B decode shape, then a smaller one
CALLS = [(32, 128, 32, False, 4096, 4096, torch.bfloat16),
         (8, 64, 64, True, 333, 400, torch.float16)]


def test_noalloc_matches_workspace_entry_point():
    for i, (heads, d, g, sym, n_tok, t_cap, qdt) in enumerate(CALLS):
        note(f"kv_attention_noalloc call {i}: heads={heads} d={d} g={g} sym={sym} n_tok={n_tok}")
        _, _, kref, vref = build_caches(heads, d, g, sym, n_tok, t_cap, seed=900 + i)
        kc = cache_to_device(kref, heads, t_cap, d, g, sym)
        vc = cache_to_device(vref, heads, t_cap, d, g, sym)
        q = synthetic.query(heads, d, seed=910 + i, dtype=qdt).to(DEV)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        ws = torch.empty(q4.q4_kv_attention_workspace(heads, d, n_tok), dtype=torch.uint8, device=DEV)
        ref = q4.q4_kv_attention(q, kc, vc, n_tok, scale, out=torch.empty((heads, d), dtype=torch.float32,
                                                                           device=DEV), workspace=ws)
        ob, ov = guarded((heads, d), torch.float32, SENTINEL_F32)
        assert noalloc_raw(q, kc, vc, n_tok, scale, ov) == 0
        kname = q4.q4_last_kernel()
        torch.cuda.synchronize()
        assert guard_intact(ob), "store outside out"
        assert kname == ("q4_kv_attention_bf16" if qdt == torch.bfloat16 else "q4_kv_attention_f16")
        got, want = ov.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
            f"call {i}: {int((got != want).sum())} outputs differ from q4_kv_attention"
        if i == len(CALLS) - 1:
            o = oracle.default()
            qh = host_input(q.cpu())
            r64, _, vabs = o.kv_attention(qh, kref, vref, n_tok, g, sym, scale)
            tol = tolerance(qh, kref, vref, heads, t_cap, d, g, n_tok, scale, vabs)
            assert_attention_close(got.astype(np.float64), r64, tol, f"noalloc call {i}")


def test_noalloc_binding_and_limit():
    heads, d, g, n_tok = 4, 128, 32, 100
    _, _, kref, vref = build_caches(heads, d, g, False, n_tok, 128, seed=920)
    kc = cache_to_device(kref, heads, 128, d, g, False)
    vc = cache_to_device(vref, heads, 128, d, g, False)
    q = synthetic.query(heads, d, seed=921).to(DEV)
    out = torch.empty((heads, d), dtype=torch.float32, device=DEV)
    note("kv_attention_noalloc binding and scratch limit")
    q4.q4_kv_attention_noalloc(q, kc, vc, n_tok, 0.125, out)
    ref = q4.q4_kv_attention(q, kc, vc, n_tok, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert q4.lib().q4_kv_attention_noalloc_max_bytes() == 16 << 20
    # 2048 heads of 256 over 8192 tokens need 67 MB of partials: refused before any launch
    big = (2048, 256, 8192)
    qb = torch.empty((2048, 256), dtype=torch.bfloat16, device=DEV)
    kb = q4.KvCache(kc.qcache, kc.scache, kc.zcache, big[0], big[2], big[1], 64, False)
    code = noalloc_raw(qb, kb, kb, big[2], 0.0625, out)
    assert code == Q4_ERR_SCRATCH, code
    # through the binding the same call stops earlier: the cache tensors are far shorter
    # than 2048 heads x 8192 tokens
    with pytest.raises(ValueError):
        q4.q4_kv_attention_noalloc(qb, kb, kb, big[2], 0.0625,
                                   torch.empty((2048, 256), dtype=torch.float32, device=DEV))
