"""GPTQ on the GPU vs the fp64 oracle, through the C ABI (needs an MI355X).

The GPU decides each code in fp32, the oracle in fp64, and a code can differ where an
updated weight falls within rounding of a code boundary (after which the error it carries
differs too).  So the checks are:
  * scales and zero points: bit-exact (they are RTN's, fixed before the sweep);
  * the factor U (H = U U^T) the kernels leave in the workspace: against numpy's fp64
    Cholesky of the oracle's Hessian, relative to the largest entry of its column;
  * self-consistency at every weight: recomputing in fp64, from the GPU's own codes and the
    oracle's factor, the value each column is quantized at (w_j + sum_{i<j} d_i U_ij / U_jj),
    its rounding must give the GPU's code, except within ETA of a code boundary;
  * a layer-output error within 2% of the oracle's and below RTN's, and agreement with the
    oracle's codes on most weights (a flip near a boundary changes the error carried into
    every later column, so two valid sweeps drift apart as k grows: about 3% of the codes
    at k = 4096).
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.gptq as gq
import pins
import synthetic
import w4a16_group_wise_q4_amd as q4
from gpu_util import DEV, host_input, note

pytestmark = pytest.mark.gpu

ETA = 2e-3  # distance from a code boundary (in units of the scale) below which fp32 may decide otherwise


def calib(tokens, k, seed, dtype=torch.bfloat16, dead=()):
    """Correlated calibration activations: N(0, 1) plus 8 shared factors."""
    g = torch.Generator().manual_seed(seed)
    f = torch.randn((tokens, 8), generator=g)
    b = torch.randn((k, 8), generator=g) / 8 ** 0.5
    x = torch.randn((tokens, k), generator=g) + 1.5 * f @ b.T
    for c in dead:
        x[:, c] = 0
    return x.to(dtype)


def x_f64(x):
    return x.float().double().numpy()


def run_gpu(w, x, g, sym, act_order=False):
    n, k = w.shape
    need = (q4.q4_gptq_act_order_workspace if act_order else q4.q4_gptq_workspace)(n, k, g)
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    p = q4.q4_gptq_quantize(w.to(DEV), x.to(DEV), g, sym, workspace=ws, act_order=act_order)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel().startswith("q4_gptq_act_order_" if act_order else "q4_gptq_")
    names = q4.q4_last_kernels()
    assert names[0].startswith("q4_quant_pack_") and "q4_gptq_hessian" in names
    assert {"q4_gptq_chol_diag", "q4_gptq_fill_zero", "q4_gptq_sweep"} <= set(names)
    blocks = -(-k // 64)  # the quantizer, the Hessian, a diagonal factor per 64 columns, ...
    assert q4.q4_last_launch_count() >= 3 + blocks + 1 + blocks
    A = ws[:k * k].view(k, k).cpu().double().numpy()
    order = None
    if act_order:
        assert {"q4_gptq_energy", "q4_gptq_rank", "q4_gptq_order", "q4_gptq_pack_codes"} <= set(names)
        base = k * k + n * k + 256 * n  # the energies, ranks and order follow A, C and D
        key = ws[base:base + k].cpu().double().numpy()
        order = ws[base + 2 * k:base + 3 * k].view(torch.int32).cpu().numpy().astype(np.int64)
        check_order(order, key, x)
    qw = p.qweight.cpu().numpy().view(np.uint32)
    sc = p.scales.cpu().view(torch.int16).numpy().view(np.uint16)
    zr = None if sym else p.zeros.cpu().numpy().view(np.uint32)
    return qw, sc, zr, A, order


def check_order(order, key, x):
    """The GPU's act-order: a permutation, sorted by its own fp32 energies (descending,
    ties by index); those energies within fp32 summation rounding of the exact ones; and
    wherever it orders two columns against the exact energies, they are within that
    rounding of each other."""
    k = len(key)
    assert sorted(order.tolist()) == list(range(k)), "not a permutation"
    ks = key[order]
    assert np.all((ks[:-1] > ks[1:]) | ((ks[:-1] == ks[1:]) & (order[:-1] < order[1:])))
    xo = x_f64(x)
    e = np.sum(xo * xo, axis=0)
    tol = (x.shape[0] + 2) * 2.0 ** -24 * e
    assert np.all(np.abs(key - e) <= tol), float(np.max(np.abs(key - e) / np.maximum(e, 1e-300)))
    ref = gq.act_order(xo)
    es = e[order]
    inv = es[1:] > es[:-1] + tol[order][1:] + tol[order][:-1]
    assert not inv.any(), "an inversion beyond rounding"
    note(f"act-order: {int(np.sum(order != ref))} of {k} positions differ from the fp64 order")


def check(w, x, g, sym, rows=None, what="", act_order=False):
    n, k = w.shape
    qw, sc, zr, A, order = run_gpu(w, x, g, sym, act_order)
    wh = host_input(w)
    qr, sr, zrr = oracle.quantize_pack(wh, g, sym)
    assert np.array_equal(sc, sr), "scales differ from RTN's"
    if not sym:
        assert np.array_equal(zr, zrr), "zero points differ from RTN's"
    order = np.arange(k) if order is None else order
    H = gq.hessian(x_f64(x))[np.ix_(order, order)]                # in sweep order
    U = np.linalg.cholesky(H[::-1, ::-1])[::-1, ::-1]          # H = U U^T, U upper
    Ug = A[::-1, ::-1]                                          # the kernels' factor (upper part)
    err_u = np.abs(np.triu(Ug) - U).max(axis=0) / np.abs(U).max(axis=0)
    note(f"{what}: factor max column-relative error {err_u.max():.2e}")
    assert err_u.max() < 1e-3
    rows = np.arange(n) if rows is None else np.asarray(rows)
    if isinstance(wh, tuple):
        bits = np.asarray(wh[0], dtype=np.uint16)
        wf = ((bits.astype(np.uint32) << 16).view(np.float32) if wh[1] == oracle.BF16
              else bits.view(np.float16)).astype(np.float64)
    else:
        wf = np.asarray(wh, dtype=np.float64)
    wf = wf[rows]
    cg = pins.unpack_codes(qw[rows], k)
    s = pins.f16_values(sc[rows])
    z = np.full(s.shape, 8) if sym else pins.unpack_zeros(zr[rows], k // g)
    # self-consistency in fp64 from the GPU's own codes, in sweep order
    gi = np.arange(k) // g
    what_ = s[:, gi] * (cg - z[:, gi])
    gp = order // g
    d = (wf - what_)[:, order]
    wp = wf[:, order] + (d @ np.triu(U, 1)) / np.diag(U)[None, :]
    t = wp / s[:, gp]
    u = np.clip(np.rint(t) + z[:, gp], 0, 15)
    frac = np.abs(t - np.floor(t) - 0.5)                         # 0 at a rounding boundary
    cgp = cg[:, order]
    bad = (u != cgp) & ~(frac < ETA)
    note(f"{what}: self-consistency violations {int(bad.sum())} of {bad.size}, "
         f"near-boundary mismatches {int(((u != cgp) & (frac < ETA)).sum())}")
    assert not bad.any()
    # against the oracle (rows are independent given H), swept in the same order
    w_rows = (wh[0][rows], wh[1]) if isinstance(wh, tuple) else wh[rows]
    qo, so, zo = gq.gptq_quantize(w_rows, gq.hessian(x_f64(x)), g, sym,
                                  order=order if act_order else None)
    co = pins.unpack_codes(qo, k)
    agree = float(np.mean(co == cg))
    xo = x_f64(x)
    e_gpu = gq.layer_error(wf, what_, xo)
    zo_v = np.full(s.shape, 8) if sym else pins.unpack_zeros(zo, k // g)
    e_orc = gq.layer_error(wf, pins.f16_values(so)[:, gi] * (co - zo_v[:, gi]), xo)
    rr = pins.unpack_codes(qr[rows], k)
    zr_v = np.full(s.shape, 8) if sym else pins.unpack_zeros(zrr[rows], k // g)
    e_rtn = gq.layer_error(wf, s[:, gi] * (rr - zr_v[:, gi]), xo)
    note(f"{what}: codes agreeing with the oracle {agree:.5f}; layer error gpu/oracle "
         f"{e_gpu / e_orc:.4f}, gpu/rtn {e_gpu / e_rtn:.4f}")
    assert agree > 0.9
    assert e_gpu < 1.02 * e_orc and e_gpu < e_rtn


CASES = [(64, 256, 32, False, torch.bfloat16, 512), (100, 512, 128, True, torch.float16, 700),
         (37, 384, 64, False, torch.float32, 300), (20, 352, 32, True, torch.bfloat16, 200),
         (256, 1024, 128, False, torch.bfloat16, 1024)]


@pytest.mark.parametrize("n,k,g,sym,dtype,tokens", CASES)
def test_gptq_cases(n, k, g, sym, dtype, tokens):
    # the stress rows, kept within the fp16 range (non-finite weights are unspecified)
    w = torch.from_numpy(np.clip(pins.random_weights(n + k, max(n, 12), k)[:n], -6e4, 6e4)).to(dtype)
    x = calib(tokens, k, seed=n + k)
    note(f"gptq n={n} k={k} g={g} sym={sym} {dtype} tokens={tokens}")
    check(w, x, g, sym, what=f"gptq {n}x{k}")


def test_gptq_dead_features_and_fp16_x():
    n, k = 48, 256
    w = torch.from_numpy(pins.random_weights(7, n, k)).to(torch.bfloat16)
    x = calib(400, k, seed=8, dtype=torch.float16, dead=(0, 77, 255))
    note("gptq dead features")
    check(w, x, 64, False, what="gptq dead features")


def test_gptq_7b_up_sampled_rows():
    """The 7B-shaped up projection [11008 x 4096], 2048 calibration tokens, g128 sym (the
    pages' GPTQ setting); checked on a seeded sample of 192 rows (rows are independent
    given the Hessian)."""
    mat = synthetic.MLP_SWEEP["mats"][0]
    w = mat.make()
    x = calib(2048, mat.k, seed=300)
    rows = synthetic.sample_rows(mat.n, 192, 301).numpy()
    note("gptq 7B up 11008x4096, 2048 tokens")
    check(w, x, 128, True, rows=rows, what="gptq 7B up")


# ----------------------------------------------------------------------------- act-order

def spread(x, seed):
    """Calibration activations whose feature scales vary over 6x in a shuffled pattern, so
    the act-order sequence is far from the natural one and crosses every group."""
    k = x.shape[1]
    f = torch.linspace(0.4, 2.4, k)[torch.randperm(k, generator=torch.Generator().manual_seed(seed))]
    return (x.float() * f).to(x.dtype)


ACT_CASES = [(64, 256, 32, False, torch.bfloat16, 512), (100, 512, 128, True, torch.float16, 700),
             (37, 384, 64, False, torch.float32, 300), (256, 1024, 128, True, torch.bfloat16, 1024)]


@pytest.mark.parametrize("n,k,g,sym,dtype,tokens", ACT_CASES)
def test_gptq_act_order_cases(n, k, g, sym, dtype, tokens):
    w = torch.from_numpy(np.clip(pins.random_weights(n + k + 1, max(n, 12), k)[:n], -6e4, 6e4)).to(dtype)
    x = spread(calib(tokens, k, seed=n + k + 1), seed=k)
    note(f"gptq act-order n={n} k={k} g={g} sym={sym} {dtype} tokens={tokens}")
    check(w, x, g, sym, what=f"gptq act-order {n}x{k}", act_order=True)


def test_gptq_act_order_ties_and_dead_features():
    """Duplicated feature columns have equal energies (taken by the lower index), and
    never-active features come last."""
    n, k = 48, 256
    w = torch.from_numpy(pins.random_weights(9, n, k)).to(torch.bfloat16)
    x = spread(calib(400, k, seed=10, dtype=torch.float16, dead=(3, 100, 250)), seed=11)
    for a, b in [(5, 200), (17, 18), (64, 130)]:
        x[:, b] = x[:, a]
    note("gptq act-order ties and dead features")
    _, _, _, _, order = run_gpu(w, x, 64, False, act_order=True)
    assert order[-3:].tolist() == [3, 100, 250]
    pos = np.argsort(order)
    for a, b in [(5, 200), (17, 18), (64, 130)]:
        assert pos[b] == pos[a] + 1, (a, b)
    check(w, x, 64, False, what="gptq act-order ties", act_order=True)


def test_gptq_act_order_7b_up_sampled_rows():
    """The 7B-shaped up projection with act-order, g128 sym (the pages' GPTQ setting with
    act-order on), 2048 calibration tokens; a seeded sample of 192 rows."""
    mat = synthetic.MLP_SWEEP["mats"][0]
    w = mat.make()
    x = spread(calib(2048, mat.k, seed=302), seed=303)
    rows = synthetic.sample_rows(mat.n, 192, 304).numpy()
    note("gptq act-order 7B up 11008x4096, 2048 tokens")
    check(w, x, 128, True, rows=rows, what="gptq act-order 7B up", act_order=True)
