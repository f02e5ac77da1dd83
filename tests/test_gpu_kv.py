"""INT4 KV cache on the GPU vs the CPU oracle, through the C ABI (needs an MI355X).

Cache quantization (codes, fp16 scales, zero points, and every row the call must leave
alone) must match the oracle bit for bit.  Decode attention over the cache must satisfy,
elementwise, with u = 2^-24 and gamma(n) = n u / (1 - n u):

    |out - out_oracle| <= 2 (delta_h + gamma(L + 8)) max_t |V_hat[h][t][i]|
                          + gamma(L) 60 max_t S_V(h, t, i)
    delta_h = gamma(64) |scale| max_t sum_i |q[h][i]| 30 S_K(h, t, i)
    L = ceil(n_tok d / 8192) + 32   (the chunks of a head are at most ceil(n_tok d / 8192))

the fp32 rounding bound of the kernel's arithmetic.  A score is a sum of 32 products of a
16-bit query value and a 4-bit code (at most 15) per lane, minus the zero point (at most
15) times the lane's query sum, over at most 8 lanes, so its rounding error is relative to
|q| 30 S (delta_h).  A score error delta, and the relative errors of the exponentials and
of the sums of weights, move each softmax weight by a factor within e^(+-2 (...)).  The
weighted sum of S (u - z) has terms of size at most p S 30 and is added along chains of at
most L terms: at most 8 tokens per lane, 3 levels within a row of 16 lanes, the 16 rows
of the workgroup, then the chunks of the head.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import w4a16_group_wise_q4_amd as q4
from gpu_util import DEV, SENTINEL_F32, SENTINEL_I32, guard_intact, guarded, host_input, note

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
SQ = 0xDEADBEEF          # sentinel of code and zero-point words
SS = 0xFFFF              # sentinel of scales


def gamma(n):
    return n * U / (1 - n * U)


def gpu_cache(heads, t_cap, d, g, sym):
    """A sentinel-filled cache on the GPU, each array a view into a guarded buffer."""
    rows, G = heads * t_cap, d // g
    qb, qv = guarded((rows, d // 8), torch.int32, SENTINEL_I32)
    sb, sv = guarded((rows, G), torch.int16, -1)
    zb, zv = (None, None) if sym else guarded((rows, (G + 7) // 8), torch.int32, SENTINEL_I32)
    c = q4.KvCache(qv, sv.view(torch.float16), zv, heads, t_cap, d, g, sym)
    return c, (qb, sb, zb)


def oracle_cache(heads, t_cap, d, g):
    qc, sc, zc = oracle.default().kv_cache(heads, t_cap, d, g)
    qc[:], sc[:], zc[:] = SQ, SS, SQ
    return qc, sc, zc


def cache_to_host(c):
    qc = c.qcache.cpu().numpy().view(np.uint32)
    sc = c.scache.cpu().view(torch.int16).numpy().view(np.uint16)
    zc = None if c.zcache is None else c.zcache.cpu().numpy().view(np.uint32)
    return qc, sc, zc


def cache_to_device(host, heads, t_cap, d, g, sym):
    qc, sc, zc = host
    return q4.KvCache(torch.from_numpy(qc.view(np.int32)).to(DEV),
                      torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.float16),
                      None if sym else torch.from_numpy(zc.view(np.int32)).to(DEV),
                      heads, t_cap, d, g, sym)


def assert_cache_equal(gpu, ref, sym):
    qc, sc, zc = cache_to_host(gpu)
    assert np.array_equal(qc, ref[0]), f"codes differ in {np.count_nonzero(qc != ref[0])} words"
    assert np.array_equal(sc, ref[1]), f"scales differ in {np.count_nonzero(sc != ref[1])} entries"
    if not sym:
        assert np.array_equal(zc, ref[2]), f"zeros differ in {np.count_nonzero(zc != ref[2])} words"


def check_guards(bufs, sym):
    qb, sb, zb = bufs
    assert guard_intact(qb, sentinel=SENTINEL_I32), "store outside qcache"
    assert guard_intact(sb, sentinel=-1), "store outside scache"
    if not sym:
        assert guard_intact(zb, sentinel=SENTINEL_I32), "store outside zcache"


# --------------------------------------------------------------------------- quantize

# (heads, head_dim, group, t_cap, appends as (t0, t_new) in order)
QUANT_CASES = [
    (4, 128, 32, 10, [(3, 1)]),                   # one decode token
    (32, 128, 32, 64, [(0, 63), (63, 1)]),        # prefill, then the last slot
    (3, 64, 64, 17, [(5, 7), (12, 1), (0, 2)]),
    (2, 256, 128, 9, [(0, 9)]),
    (5, 128, 128, 33, [(32, 1)]),
    (7, 96, 32, 5, [(1, 3)]),                     # head_dim that attention does not take
    (5, 64, 32, 11, [(2, 3), (9, 2)]),            # two groups per row, a part-filled last task
    (3, 32, 32, 6, [(0, 5)]),                     # one group per row
    (2, 512, 32, 4, [(1, 3)]),                    # 16 groups per row: the row kernel
    (3, 512, 128, 5, [(0, 4)]),                   # a whole task per row
]


@pytest.mark.parametrize("heads,d,g,t_cap,appends", QUANT_CASES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sym", [False, True])
def test_kv_quantize(heads, d, g, t_cap, appends, dtype, sym):
    o = oracle.default()
    c, bufs = gpu_cache(heads, t_cap, d, g, sym)
    ref = oracle_cache(heads, t_cap, d, g)
    for i, (t0, t_new) in enumerate(appends):
        kv = synthetic.kv_tokens(t_new, heads, d, seed=300 + i, kind="k" if i % 2 == 0 else "v",
                                 dtype=dtype)
        note(f"kv_quantize heads={heads} d={d} g={g} t_cap={t_cap} t0={t0} t_new={t_new} "
             f"{dtype} sym={sym}")
        q4.q4_kv_quantize(kv.to(DEV), c, t0)
        o.kv_quantize(host_input(kv), g, sym, ref, t0)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel().startswith("q4_kv_quant_")
    check_guards(bufs, sym)
    assert_cache_equal(c, ref, sym)


def test_kv_quantize_7b_prefill_then_decode():
    cfg = synthetic.KV_7B
    H, D, g, T = cfg["heads"], cfg["head_dim"], cfg["group_size"], cfg["t_cap"]
    for kind, seed in (("k", cfg["k_seed"]), ("v", cfg["v_seed"])):
        kv = synthetic.kv_tokens(T, H, D, seed, kind)
        c, bufs = gpu_cache(H, T, D, g, False)
        note(f"kv_quantize 7B {kind}: prefill {T - 1} tokens, then one")
        q4.q4_kv_quantize(kv[:T - 1].contiguous().to(DEV), c, 0)
        q4.q4_kv_quantize(kv[T - 1:].contiguous().to(DEV), c, T - 1)
        torch.cuda.synchronize()
        check_guards(bufs, False)
        ref = oracle_cache(H, T, D, g)
        oracle.default().kv_quantize(host_input(kv), g, False, ref, 0)
        assert_cache_equal(c, ref, False)


# --------------------------------------------------------------------------- attention

def f16_values(u16):
    return u16.view(np.float16).astype(np.float64)


def chunking(heads, d, n_tok):
    """The most chunks per head the split can use: ceil(n_tok d / 8192)."""
    return -(-n_tok * d // 8192)


def tolerance(q_host, kref, vref, heads, t_cap, d, g, n_tok, scale, vabs):
    """The fp32 error bound stated in the module docstring, elementwise [heads, d]."""
    qf = np.asarray(q_host, dtype=np.float64) if not isinstance(q_host, tuple) else None
    if qf is None:
        bits, code = q_host
        qf = (torch.from_numpy(bits.view(np.int16)).view(
            torch.bfloat16 if code == oracle.BF16 else torch.float16).double().numpy())
    G = d // g
    sk = f16_values(kref[1]).reshape(heads, t_cap, G)[:, :n_tok]
    sv = f16_values(vref[1]).reshape(heads, t_cap, G)[:, :n_tok]
    qg = np.abs(qf).reshape(heads, G, g).sum(axis=2)                 # [heads, G]
    delta = gamma(64) * abs(scale) * 30.0 * (sk * qg[:, None, :]).sum(axis=2).max(axis=1)
    svmax = np.repeat(sv.max(axis=1), g, axis=1)                     # [heads, d]
    L = chunking(heads, d, n_tok) + 32
    return 2.0 * (delta[:, None] + gamma(L + 8)) * vabs + gamma(L) * 60.0 * svmax


def assert_attention_close(out, ref, tol, what):
    err = np.abs(out - ref)
    ratio = float((err / tol).max())
    note(f"{what}: max |err| {err.max():.3e}, worst err/tol {ratio:.4f}")
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {ratio:.3f}"


def build_caches(heads, d, g, sym, n_tok, t_cap, seed, dtype=torch.bfloat16):
    """Oracle caches holding n_tok tokens of the K and V recipes (rest sentinel)."""
    o = oracle.default()
    k = synthetic.kv_tokens(n_tok, heads, d, seed, "k", dtype)
    v = synthetic.kv_tokens(n_tok, heads, d, seed + 1, "v", dtype)
    kref, vref = oracle_cache(heads, t_cap, d, g), oracle_cache(heads, t_cap, d, g)
    o.kv_quantize(host_input(k), g, sym, kref, 0)
    o.kv_quantize(host_input(v), g, sym, vref, 0)
    return k, v, kref, vref


def run_attention(q, kc, vc, n_tok, scale):
    heads, d = q.shape
    need = q4.q4_kv_attention_workspace(heads, d, n_tok)
    assert need > 0
    wb, wv = guarded((need // 4,), torch.float32, SENTINEL_F32)
    ob, ov = guarded((heads, d), torch.float32, SENTINEL_F32)
    q4.q4_kv_attention(q.to(DEV), kc, vc, n_tok, scale, out=ov, workspace=wv)
    kname = q4.q4_last_kernel()
    torch.cuda.synchronize()
    assert guard_intact(wb), "store outside the workspace"
    assert guard_intact(ob), "store outside out"
    return ov.cpu().numpy().astype(np.float64), kname


# (heads, head_dim, group, sym, n_tok, t_cap)
ATTN_CASES = [
    (4, 128, 32, False, 1, 8),
    (4, 128, 32, False, 100, 128),
    (2, 64, 32, True, 333, 400),
    (3, 256, 64, False, 700, 700),
    (1, 128, 128, True, 5000, 5003),     # one head: many 64-token chunks, ragged tail
    (8, 128, 32, False, 4113, 4200),     # chunks of several hundred tokens, ragged tail
    (64, 64, 64, False, 64, 64),
    (40, 256, 128, True, 129, 130),
]


@pytest.mark.parametrize("heads,d,g,sym,n_tok,t_cap", ATTN_CASES)
@pytest.mark.parametrize("qdtype", [torch.bfloat16, torch.float16])
def test_kv_attention(heads, d, g, sym, n_tok, t_cap, qdtype):
    o = oracle.default()
    _, _, kref, vref = build_caches(heads, d, g, sym, n_tok, t_cap, seed=400 + heads)
    q = synthetic.query(heads, d, seed=500 + n_tok, dtype=qdtype)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kc = cache_to_device(kref, heads, t_cap, d, g, sym)
    vc = cache_to_device(vref, heads, t_cap, d, g, sym)
    note(f"kv_attention heads={heads} d={d} g={g} sym={sym} n_tok={n_tok} {qdtype}")
    out, kname = run_attention(q, kc, vc, n_tok, scale)
    assert kname == ("q4_kv_attention_bf16" if qdtype == torch.bfloat16 else "q4_kv_attention_f16")
    ref, _, vabs = o.kv_attention(host_input(q), kref, vref, n_tok, g, sym, scale)
    tol = tolerance(host_input(q), kref, vref, heads, t_cap, d, g, n_tok, scale, vabs)
    assert_attention_close(out, ref, tol, f"heads={heads} d={d} n_tok={n_tok}")


def test_kv_attention_7b_end_to_end():
    """The 7B decode-attention workload at full size: GPU quantize then GPU attention,
    against oracle quantize then oracle attention, every output."""
    cfg = synthetic.KV_7B
    H, D, g, T = cfg["heads"], cfg["head_dim"], cfg["group_size"], cfg["t"]
    k = synthetic.kv_tokens(T, H, D, cfg["k_seed"], "k")
    v = synthetic.kv_tokens(T, H, D, cfg["v_seed"], "v")
    q = synthetic.query(H, D, cfg["q_seed"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    kc = q4.empty_kv_cache(H, cfg["t_cap"], D, g, False, DEV)
    vc = q4.empty_kv_cache(H, cfg["t_cap"], D, g, False, DEV)
    note("kv 7B end to end: quantize K, V (4096 tokens), attention")
    q4.q4_kv_quantize(k.to(DEV), kc, 0)
    q4.q4_kv_quantize(v.to(DEV), vc, 0)
    out, _ = run_attention(q, kc, vc, T, scale)
    o = oracle.default()
    kref, vref = oracle_cache(H, T, D, g), oracle_cache(H, T, D, g)
    o.kv_quantize(host_input(k), g, False, kref, 0)
    o.kv_quantize(host_input(v), g, False, vref, 0)
    assert_cache_equal(kc, kref, False)
    assert_cache_equal(vc, vref, False)
    ref, _, vabs = o.kv_attention(host_input(q), kref, vref, T, g, False, scale)
    tol = tolerance(host_input(q), kref, vref, H, T, D, g, T, scale, vabs)
    assert_attention_close(out, ref, tol, "7B decode attention")
    # bit-identical on a second run (the chunk split and every summation order are fixed)
    out2, _ = run_attention(q, kc, vc, T, scale)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("heads,n_tok", [(32, 4096), (1, 5000), (3, 777)])
def test_kv_attention_every_position_reachable(heads, n_tok):
    """A token whose key is a large multiple of the query takes all the weight, so the
    output is that token's value: checked at chunk edges and the last token."""
    D, g = 128, 32
    o = oracle.default()
    q = synthetic.query(heads, D, seed=600)
    k = synthetic.kv_tokens(n_tok, heads, D, 601, "k")
    v = synthetic.kv_tokens(n_tok, heads, D, 602, "v")
    # chunks hold 64, 128, 256, ... tokens at head_dim 128: 63/64 and 255/256 are edges
    positions = sorted({0, 63, 64, 255, 256, n_tok // 2, n_tok - 2, n_tok - 1})
    scale = float(np.float32(1.0 / np.sqrt(D)))
    for p in positions:
        kk = k.clone()
        kk[p] = (q.float() * 4.0).to(kk.dtype)
        kref, vref = oracle_cache(heads, n_tok, D, g), oracle_cache(heads, n_tok, D, g)
        o.kv_quantize(host_input(kk), g, False, kref, 0)
        o.kv_quantize(host_input(v), g, False, vref, 0)
        kc = cache_to_device(kref, heads, n_tok, D, g, False)
        vc = cache_to_device(vref, heads, n_tok, D, g, False)
        note(f"kv_attention reachability heads={heads} n_tok={n_tok} p={p}")
        out, _ = run_attention(q, kc, vc, n_tok, scale)
        vhat = o.dequant(*vref, heads * n_tok, D, g, False).reshape(heads, n_tok, D)[:, p]
        assert np.allclose(out, vhat, rtol=1e-5, atol=1e-5 * np.abs(vhat).max())
