"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Packing (codes, fp16 scales, zero points) must match bit for bit; the W4A16 matmul must
satisfy |y - y_oracle| <= 1e-3 * (|x| . |x_hat|^T) + 1e-5 elementwise, with y_oracle the
fp64 product of x and the oracle's dequantized weights.  Every output buffer sits inside
a sentinel-filled guard region that must come back untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import scales as oscales
import pins
from clip_check import check_clip_choice
import synthetic
import w4a16_group_wise_q4_amd as q4
from gpu_util import (DEV, SENTINEL_F32, SENTINEL_I32, assert_linear_close, assert_pack_exact,
                      guard_intact, guarded, host_input, note, pack_guarded)

pytestmark = pytest.mark.gpu


def run_linear(x_cpu, p, guard=True, split=False):
    """One product through q4_w4a16_gemm into a guarded fp32 output; unsplit unless asked
    (the split-K path has tests of its own)."""
    m = x_cpu.shape[0]
    yb, yv = guarded((m, p.n), torch.float32, SENTINEL_F32)
    q4.q4_w4a16_gemm(x_cpu.to(DEV), p, out=yv, split=split)
    kname = q4.q4_last_kernel()
    torch.cuda.synchronize()
    assert guard_intact(yb), "store outside y"
    return yv.cpu().numpy(), kname


def check_guards(bufs, sym):
    qb, sb, zb = bufs
    assert guard_intact(qb, sentinel=SENTINEL_I32), "store outside qweight"
    assert guard_intact(sb, sentinel=-1), "store outside scales"
    if not sym:
        assert guard_intact(zb, sentinel=SENTINEL_I32), "store outside zeros"


# ----------------------------------------------------------------------------- packing

@pytest.mark.parametrize("sym", [False, True])
def test_quant_tiny_reference(sym):
    cfg = synthetic.TINY
    w = cfg["w"].make()
    note(f"quant tiny fp32 {tuple(w.shape)} g=128 sym={sym}")
    p, bufs = pack_guarded(w.to(DEV), 128, sym)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() == "q4_quant_pack_f32"
    check_guards(bufs, sym)
    assert_pack_exact(p, host_input(w), 128, sym)


@pytest.mark.parametrize("idx", [0, 1])
def test_quant_decode_7b(idx):
    mat = synthetic.DECODE_7B["mats"][idx]
    w = mat.make()
    note(f"quant {mat.name} bf16 g=128 asym")
    p, bufs = pack_guarded(w.to(DEV), 128, False)
    torch.cuda.synchronize()
    check_guards(bufs, False)
    assert_pack_exact(p, host_input(w), 128, False)


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("idx", [0, 1])
def test_quant_mlp_sweep(idx, g, sym):
    mat = synthetic.MLP_SWEEP["mats"][idx]
    w = mat.make()
    note(f"quant {mat.name} g={g} sym={sym}")
    p, bufs = pack_guarded(w.to(DEV), g, sym)
    torch.cuda.synchronize()
    check_guards(bufs, sym)
    assert_pack_exact(p, host_input(w), g, sym)


def test_quant_prefill_70b_full():
    mat = synthetic.PREFILL_70B["w"]
    w = mat.make()
    note(f"quant {mat.name} bf16 g=128 asym (full tensor)")
    p, bufs = pack_guarded(w.to(DEV), 128, False)
    torch.cuda.synchronize()
    check_guards(bufs, False)
    assert_pack_exact(p, host_input(w), 128, False)


@pytest.mark.parametrize("sym", [False, True])
def test_quant_checkpoint_sampled_rows(sym):
    """Two layers of the 32-layer checkpoint, generated on the device; seeded sample of
    rows (always including the first and last) compared against the oracle."""
    for mat in synthetic.checkpoint_7b(2):
        w_dev = mat.make(device="cuda")
        note(f"quant checkpoint {mat.name} sym={sym}")
        p, _ = pack_guarded(w_dev, 128, sym)
        torch.cuda.synchronize()
        rows = synthetic.sample_rows(mat.n, 48, mat.seed).numpy()
        w_rows = w_dev[torch.as_tensor(rows, device=DEV)].cpu()
        assert_pack_exact(p, host_input(w_rows), 128, sym, rows=rows)


EDGE_SHAPES = [(1, 32, 32), (3, 96, 32), (5, 64, 64), (7, 192, 64), (17, 384, 128),
               (33, 11008, 128), (2, 8 * 128 * 3 + 128, 128), (9, 4096 + 32, 32)]


@pytest.mark.parametrize("n,k,g", EDGE_SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sym", [False, True])
def test_quant_edge_cases(n, k, g, dtype, sym):
    """Odd shapes (one group, partial zero-point words, single rows) and the stress
    distribution: all-zero and constant rows, one-sided groups, outliers, scales in the
    fp16 subnormal range, scales that underflow to 0 or overflow to inf."""
    base = pins.random_weights(n * 1000 + k, max(n, 12), k)[:n] if n >= 1 else None
    w = torch.from_numpy(base).to(dtype)
    if dtype == torch.float16:
        w = torch.nan_to_num(w, posinf=60000.0, neginf=-60000.0)
    note(f"quant edge n={n} k={k} g={g} {dtype} sym={sym}")
    p, bufs = pack_guarded(w.to(DEV), g, sym)
    torch.cuda.synchronize()
    check_guards(bufs, sym)
    assert_pack_exact(p, host_input(w), g, sym)


def scale_tie_rows(dtype, count=64, g=32):
    """Rows of asymmetric groups whose fp32 scale (x_max - x_min) / 15 lies exactly halfway
    between two fp16 values, so the stored scale depends on rounding to fp32 first and then
    to fp16 with ties to even.  Each group holds x_max = a > 0 and x_min = -b <= 0 with
    a + b = 15 * m, m an fp16 midpoint; a and b are representable in the weight dtype."""
    rng = np.random.default_rng(21)
    rows = []
    while len(rows) < count:
        h = int(rng.integers(0x1400, 0x5800))            # fp16 bits: normal range
        lo = np.array([h], dtype=np.uint16).view(np.float16).astype(np.float64)[0]
        hi = np.array([h + 1], dtype=np.uint16).view(np.float16).astype(np.float64)[0]
        m = (lo + hi) / 2                                 # exact in fp64 and in fp32
        T = np.float32(15 * m)
        if float(T) != 15 * m:
            continue
        a = torch.tensor([float(T)], dtype=torch.float32).to(dtype).float().item()
        if a > float(T):
            a = float(np.nextafter(np.float32(a), np.float32(0)))
            a = torch.tensor([a], dtype=torch.float32).to(dtype).float().item()
        b = float(T) - a
        if b < 0 or torch.tensor([b]).to(dtype).float().item() != b or a <= 0:
            continue
        if float(np.float32(a) + np.float32(b)) != float(T):
            continue
        grp = np.zeros(g, dtype=np.float32)
        grp[0], grp[1] = a, -b
        grp[2:] = np.float32(a) * rng.uniform(0.0, 1.0, g - 2).astype(np.float32)  # inside [-b, a]
        rows.append(grp)
    return torch.from_numpy(np.stack(rows)).to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_quant_scale_ties(dtype):
    """Scales exactly on an fp16 rounding tie: the stored scale is the double rounding
    (fp32, then fp16 ties-to-even) of the definition, never a single rounding of the
    exact quotient."""
    w = scale_tie_rows(dtype)
    note(f"quant scale ties {dtype}")
    p, bufs = pack_guarded(w.to(DEV), 32, False)
    torch.cuda.synchronize()
    check_guards(bufs, False)
    assert_pack_exact(p, host_input(w), 32, False)


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sym", [False, True])
def test_quant_grouped(g, dtype, sym):
    """Several matrices of different shapes (one row, one group, partial zero-point words,
    the stress distribution) in one grouped launch: each bit-identical to the oracle, no
    store outside its buffers."""
    shapes = [(33, 8 * g * 3 + g), (1, g), (200, 1024), (7, 4096 + g), (64, 256 if g < 256 else g)]
    ws = []
    for i, (n, k) in enumerate(shapes):
        w = torch.from_numpy(pins.random_weights(300 + 7 * i + g, max(n, 12), k)[:n]).to(dtype)
        if dtype == torch.float16:
            w = torch.nan_to_num(w, posinf=60000.0, neginf=-60000.0)
        ws.append(w)
    note(f"quant grouped g={g} {dtype} sym={sym}")
    outs, bufs = [], []
    for w in ws:
        n, k = w.shape
        G = k // g
        qb, qv = guarded((n, k // 8), torch.int32, SENTINEL_I32)
        sb, sv = guarded((n, G), torch.int16, -1)
        zb, zv = (None, None) if sym else guarded((n, (G + 7) // 8), torch.int32, SENTINEL_I32)
        outs.append(q4.PackedWeight(qweight=qv, scales=sv.view(torch.float16), zeros=zv, n=n, k=k,
                                    group_size=g, symmetric=sym))
        bufs.append((qb, sb, zb))
    q4.q4_quantize_pack_grouped([w.to(DEV) for w in ws], g, sym, outs=outs)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() == {torch.float32: "q4_quant_pack_f32", torch.float16: "q4_quant_pack_f16",
                                   torch.bfloat16: "q4_quant_pack_bf16"}[dtype]
    for w, p, b in zip(ws, outs, bufs):
        check_guards(b, sym)
        assert_pack_exact(p, host_input(w), g, sym)


MSE_SHAPES = [(12, 256, 32), (12, 512, 64), (12, 1024, 128), (1, 32, 32), (5, 4096 + 64, 64),
              (33, 11008, 128)]


@pytest.mark.parametrize("n,k,g", MSE_SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sym", [False, True])
def test_quant_mse(n, k, g, dtype, sym):
    """Every group the GPU's clip search writes is the oracle's quantization at one clip
    ratio, whose error is the oracle's minimum up to the fp64 rounding of the sums (the
    two sides add the squares in different orders); the stress rows cover degenerate,
    one-sided, saturated and subnormal-scale groups."""
    w = torch.from_numpy(pins.random_weights(900 + n + k + g, max(n, 12), k)[:n]).to(dtype)
    if dtype == torch.float16:
        w = torch.nan_to_num(w, posinf=60000.0, neginf=-60000.0)
    note(f"quant mse n={n} k={k} g={g} {dtype} sym={sym}")
    G = k // g
    qb, qv = guarded((n, k // 8), torch.int32, SENTINEL_I32)
    sb, sv = guarded((n, G), torch.int16, -1)
    zb, zv = (None, None) if sym else guarded((n, (G + 7) // 8), torch.int32, SENTINEL_I32)
    p = q4.PackedWeight(qweight=qv, scales=sv.view(torch.float16), zeros=zv, n=n, k=k,
                        group_size=g, symmetric=sym)
    q4.q4_quantize_pack_mse(w.to(DEV), g, sym, out=p)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() == {torch.float32: "q4_quant_mse_f32", torch.float16: "q4_quant_mse_f16",
                                   torch.bfloat16: "q4_quant_mse_bf16"}[dtype]
    check_guards((qb, sb, zb), sym)
    same = check_clip_choice(oracle.default(), host_input(w), g, sym, p.qweight.cpu().numpy(),
                             p.scales.cpu().numpy(), None if sym else p.zeros.cpu().numpy())
    note(f"  ratio equal to the oracle's in {same:.4f} of the groups")


def test_quant_mse_decode_7b_sampled():
    """The 4096x4096 decode matrix at full size (bf16, g128 asym): a seeded sample of 64
    rows passes the clip-choice validity check against the oracle, and the whole matrix's
    squared error is below RTN's."""
    mat = synthetic.DECODE_7B["mats"][0]
    w = mat.make()
    note("quant mse decode 4096x4096 g128 asym")
    p = q4.q4_quantize_pack_mse(w.to(DEV), 128, False)
    r = q4.q4_quantize_pack(w.to(DEV), 128, False)
    torch.cuda.synchronize()
    rows_t = synthetic.sample_rows(mat.n, 64, seed=17)
    rows = rows_t.numpy()
    check_clip_choice(oracle.default(), host_input(w[rows_t].contiguous()), 128, False,
                      p.qweight.cpu().numpy()[rows], p.scales.cpu().numpy()[rows],
                      p.zeros.cpu().numpy()[rows])
    wf = w.float().to(DEV)
    e_mse = (q4.q4_dequant(p) - wf).double().pow(2).sum().item()
    e_rtn = (q4.q4_dequant(r) - wf).double().pow(2).sum().item()
    assert e_mse < e_rtn


# ----------------------------------------------------------------------------- dequant

@pytest.mark.parametrize("g,sym", [(32, False), (64, True), (128, False), (128, True)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_dequant(g, sym, out_dtype):
    w = torch.from_numpy(pins.random_weights(77, 40, 1024))
    note(f"dequant g={g} sym={sym} -> {out_dtype}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    ob, ov = guarded((40, 1024), out_dtype, 0)
    q4.q4_dequant(p, out=ov)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel().startswith("q4_dequant_")
    assert (ob[:256] == 0).all() and (ob[-256:] == 0).all(), "store outside w_out"
    qo, so, zo = assert_pack_exact(p, host_input(w), g, sym)
    ref = oracle.dequant(qo, so, zo, 40, 1024, g, sym)
    ref32 = torch.from_numpy(ref.astype(np.float32))
    assert np.array_equal(ref32.numpy().astype(np.float64), ref), "S*(u-z) exact in fp32"
    got = ov.cpu()
    want = ref32.to(out_dtype)  # one round-to-nearest-even of the exact value
    assert torch.equal(got.view(torch.int16) if out_dtype != torch.float32 else got,
                       want.view(torch.int16) if out_dtype != torch.float32 else want)


# ----------------------------------------------------------------------------- matmul

@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("m", [1, 40])
def test_linear_tiny_reference(sym, m):
    cfg = synthetic.TINY
    w = cfg["w"].make()
    x = synthetic.activations(m, w.shape[1], cfg["x_seed"])
    note(f"linear tiny m={m} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), 128, sym)
    y, kname = run_linear(x, p)
    assert kname in matmul_kernels(m, 256)
    packed = assert_pack_exact(p, host_input(w), 128, sym)
    assert_linear_close(y, host_input(x), packed, 256, 512, 128, sym, what=kname)


@pytest.mark.parametrize("idx", [0, 1])
def test_gemv_decode_7b_full(idx):
    cfg = synthetic.DECODE_7B
    mat = cfg["mats"][idx]
    w = mat.make()
    x = synthetic.activations(1, mat.k, cfg["x_seed"])
    note(f"gemv {mat.name} m=1 g=128 asym")
    p, _ = pack_guarded(w.to(DEV), 128, False)
    y, kname = run_linear(x, p)
    assert kname == "q4_gemv_tile_bf16"
    packed = assert_pack_exact(p, host_input(w), 128, False)
    assert_linear_close(y, host_input(x), packed, mat.n, mat.k, 128, False, what=kname)


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("idx", [0, 1])
def test_gemv_mlp_sweep(idx, g, sym):
    """All five batch sizes on one packed matrix; columns sampled (every 7th plus the
    first and last), all rows."""
    cfg = synthetic.MLP_SWEEP
    mat = cfg["mats"][idx]
    w = mat.make()
    p, _ = pack_guarded(w.to(DEV), g, sym)
    packed = assert_pack_exact(p, host_input(w), g, sym)
    x16 = synthetic.activations(16, mat.k, cfg["x_seed"])
    cols = np.unique(np.concatenate([np.arange(0, mat.n, 7), [mat.n - 1]]))
    for m in cfg["ms"]:
        note(f"gemv {mat.name} m={m} g={g} sym={sym}")
        x = x16[:m].contiguous()
        y, kname = run_linear(x, p)
        assert kname in gemv_kernels()
        assert_linear_close(y, host_input(x), packed, mat.n, mat.k, g, sym, cols=cols,
                            what=f"{kname} m={m}")


def gemv_kernels(xdtype=torch.bfloat16):
    """Names of the decode kernels for an activation dtype: the tile kernel (m <= 4), the
    wide tile kernel (4 < m <= 16), the resident kernel (8 < m <= 16 with many tiles) and
    the streaming kernel (shapes none of them takes)."""
    t = "f16" if xdtype == torch.float16 else "bf16"
    return {f"q4_gemv_tile_{t}", f"q4_gemv_wide_{t}", f"q4_gemv_resident_{t}", f"q4_gemv_mfma_{t}"}


# (m, n, k): every slice width of the tile kernel (2, 4, 8, 12 and 16 units per wave, two
# to fourteen waves, a short last slice), ragged tiles, m = 1..4
TILE_CASES = [(1, 1, 512), (2, 17, 512), (4, 33, 1024), (3, 100, 2048), (2, 300, 5120),
              (4, 48, 8192), (1, 130, 8192), (1, 16, 2560), (3, 15, 1536), (1, 40, 7168),
              (1, 70, 11008), (2, 50, 11008), (1, 20, 28672), (3, 9, 14336)]


def tile_fits(g, m, k, n, num_cus=256):
    """Whether the launcher picks the tile kernel: the same rule as its shape search
    (slices of 2..16 units, at most 16 waves at m = 1 and 8 otherwise, an even group count,
    activations and partial sums within 96 KiB of LDS)."""
    if m > 4 or k % 128 or (k // g) % 2:
        return False
    units, mq = k // 128, (1 if m <= 1 else 4)
    max_upw = {128: 16, 64: 12, 32: 8}[g]
    for u in (2, 4, 8, 12, 16):
        sw = -(-units // u)
        if u <= max_upw and sw <= (16 if mq == 1 else 8) and \
                m * sw * u * 256 + sw * 64 * mq * 4 <= 96 * 1024:
            return True
    return False


def tile_route(g, m, k, n, num_cus=256):
    """Whether the launcher runs the tile kernel: it fits (tile_fits), and either m = 1 or
    the launch has more than four tiles per CU (from m = 2 on, launches with fewer go to the
    wide kernel when it fits)."""
    if not tile_fits(g, m, k, n, num_cus):
        return False
    return m == 1 or -(-n // 16) > 4 * num_cus or not wide_fits(g, m, k)


def wide_fits(g, m, k):
    """Whether the wide tile kernel can take a product (m <= 16; the launcher uses it for
    m > 4 and for the m <= 4 shapes the tile kernel cannot take): slices of 4..16 units over
    at most eight waves, K a multiple of 128, an even group count."""
    if not 1 <= m <= 16 or k % 128 or (k // g) % 2:
        return False
    return any(-(-(k // 128) // u) <= 8 for u in (4, 8, 12, 16))


# (m, n, k): slice widths 4, 8, 12 and 16, one to eight waves, short last slices, ragged
# tiles, m = 5..16
WIDE_CASES = [(5, 17, 512), (8, 100, 1024), (16, 33, 4096), (12, 64, 5120), (9, 48, 11008),
              (16, 20, 16384), (6, 130, 2560), (16, 1, 1536)]


@pytest.mark.parametrize("m,n,k", WIDE_CASES)
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_wide_cases(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 7 * k + m + g, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m * 19 + k).to(xdtype)
    note(f"gemv wide m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert kname == (f"q4_gemv_wide_{t}" if wide_fits(g, m, k) else f"q4_gemv_mfma_{t}")
    packed = assert_pack_exact(p, host_input(w), g, sym)
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, what=kname)


# (m, n, k, g): wide products with at least 4 x 256 tiles, which the launcher serves with two
# 16-row tiles per workgroup (rows 16392: the last pair holds one tile of 8 rows); ring rows
# 4, 8 and 16
WIDE_PAIR_CASES = [(16, 16392, 512, 128), (5, 16392, 1024, 32), (8, 16400, 2048, 64),
                   (4, 16392, 14336, 128)]


@pytest.mark.parametrize("m,n,k,g", WIDE_PAIR_CASES)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_wide_pair_cases(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 11 * k + m + g, n, k))
    x = synthetic.activations(m, k, seed=m * 23 + k).to(xdtype)
    note(f"gemv wide pair m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    assert not tile_fits(g, m, k, n) and wide_fits(g, m, k)
    y, kname = run_linear(x, p)  # stores outside y are checked there
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert kname == f"q4_gemv_wide_{t}"
    packed = assert_pack_exact(p, host_input(w), g, sym)
    # every 5th column and the last tile's rows (the ragged pair)
    cols = np.unique(np.concatenate([np.arange(0, n, 5), np.arange(n - 24, n)]))
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=kname)


@pytest.mark.parametrize("m", [6, 16])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_gemm_grouped_wide_pair(m, xdtype):
    """Two problems with 1063 tiles in all (paired tiles, first workgroups recounted per
    problem), ragged last pairs; every output of both."""
    k, g, sym = 512, 64, False
    ns = [9000, 8000 - 8]
    ws = [torch.from_numpy(pins.random_weights(61 + i, n, k)) for i, n in enumerate(ns)]
    x = synthetic.activations(m, k, seed=77).to(xdtype)
    note(f"grouped wide pair m={m} {xdtype}")
    packs = [pack_guarded(w.to(DEV), g, sym)[0] for w in ws]
    guards = [guarded((m, n), torch.float32, SENTINEL_F32) for n in ns]
    q4.q4_w4a16_gemm_grouped(x.to(DEV), packs, outs=[v for _, v in guards])
    torch.cuda.synchronize()
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert q4.q4_last_kernel() == f"q4_gemv_wide_{t}"
    for w, p, (gb, gv) in zip(ws, packs, guards):
        assert guard_intact(gb), "store outside y"
        packed = assert_pack_exact(p, host_input(w), g, sym)
        assert_linear_close(gv.cpu().numpy(), host_input(x), packed, p.n, k, g, sym,
                            what="grouped pair")


def resident_fits(g, m, k, tiles, num_cus=256):
    """Whether the launcher picks the resident kernel: 8 < m <= 16, slices of 4 or 8 units
    over at most eight waves, an even group count, all activations (16 rows per 128-column
    unit) and two regions of partial sums within 160 KiB of LDS, and at least two tiles per
    workgroup the CUs hold at that LDS size."""
    if not 8 < m <= 16 or k % 128 or (k // g) % 2:
        return False
    units = k // 128
    shapes = [(-(-units // u), u) for u in (4, 8) if -(-units // u) <= 8]
    if not shapes:
        return False
    waves = max(sw for sw, _ in shapes)
    lds = units * 16 * 256 + 2 * waves * 64 * 16
    if lds > 160 * 1024:
        return False
    return tiles >= 2 * num_cus * (160 * 1024 // lds)


# (m, n, k, g): resident products -- ragged last tiles (8, 15, 6 rows), workgroups of three
# tiles (odd: the tile after the last pair), of two and three tiles in one launch, and of two
# (even: the pair loop's last prefetch reads nothing); slices of 4 units (8 and 4 waves) and
# of 8 units over 5 waves with a short last slice (k = 4608)
RESIDENT_CASES = [(16, 8200, 4096, 128), (12, 9999, 4096, 64), (9, 16390, 2048, 32),
                  (16, 8192, 4608, 128), (13, 8300, 4608, 32)]


@pytest.mark.parametrize("m,n,k,g", RESIDENT_CASES)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_resident_cases(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 13 * k + m + g, n, k))
    x = synthetic.activations(m, k, seed=m * 29 + k).to(xdtype)
    note(f"gemv resident m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    assert resident_fits(g, m, k, -(-n // 16))
    y, kname = run_linear(x, p)  # stores outside y are checked there
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert kname == f"q4_gemv_resident_{t}"
    packed = assert_pack_exact(p, host_input(w), g, sym)
    # every 5th column, the first tiles' and the last (ragged) tile's columns
    cols = np.unique(np.concatenate([np.arange(0, n, 5), np.arange(0, 48), np.arange(n - 24, n)]))
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=kname)


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_gemv_resident_output_dtype(out_dtype):
    """The resident kernel's 16-bit epilogue: y rounded once from the fp32 sums, equal to the
    fp32 result rounded to nearest even."""
    m, n, k, g = 16, 8200, 4096, 128
    w = torch.from_numpy(pins.random_weights(91, n, k))
    x = synthetic.activations(m, k, seed=92).to(DEV)
    note(f"gemv resident output {out_dtype}")
    p, _ = pack_guarded(w.to(DEV), g, False)
    y32 = q4.q4_w4a16_gemm(x, p)
    assert q4.q4_last_kernel() == "q4_gemv_resident_bf16"
    yb, yv = guarded((m, n), out_dtype, 0.0)
    q4.q4_w4a16_gemm(x, p, out=yv)
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() == "q4_gemv_resident_bf16"
    assert torch.equal(yv.cpu(), y32.cpu().to(out_dtype))


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("g,sym", [(128, False), (32, True)])
def test_gemm_grouped_resident(xdtype, g, sym):
    """Three problems sharing x (519 tiles: the launch's workgroups cross problems, ragged
    last tiles) through the resident kernel; the same problems with one x each take the wide
    kernel.  Every output of every problem, both ways."""
    m, k = 16, 4096
    ns = [4096, 4000 - 3, 200]
    ws = [torch.from_numpy(pins.random_weights(71 + i, n, k)) for i, n in enumerate(ns)]
    x = synthetic.activations(m, k, seed=73).to(xdtype)
    note(f"grouped resident g={g} sym={sym} {xdtype}")
    packs = [pack_guarded(w.to(DEV), g, sym)[0] for w in ws]
    packed = [assert_pack_exact(p, host_input(w), g, sym) for w, p in zip(ws, packs)]
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert resident_fits(g, m, k, sum(-(-n // 16) for n in ns))
    for xs, want in ((x.to(DEV), "resident"), ([x.clone().to(DEV) for _ in ns], "wide")):
        guards = [guarded((m, n), torch.float32, SENTINEL_F32) for n in ns]
        q4.q4_w4a16_gemm_grouped(xs, packs, outs=[v for _, v in guards])
        torch.cuda.synchronize()
        assert q4.q4_last_kernel() == f"q4_gemv_{want}_{t}"
        for p, pk, (gb, gv) in zip(packs, packed, guards):
            assert guard_intact(gb), "store outside y"
            assert_linear_close(gv.cpu().numpy(), host_input(x), pk, p.n, k, g, sym,
                                what=f"grouped {want}")


@pytest.mark.parametrize("m,n,k", TILE_CASES)
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_tile_cases(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 5 * k + m + g, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m * 17 + k).to(xdtype)
    note(f"gemv tile m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    t = "f16" if xdtype == torch.float16 else "bf16"
    want = "tile" if tile_route(g, m, k, n) else ("wide" if wide_fits(g, m, k) else "mfma")
    assert kname == f"q4_gemv_{want}_{t}"
    packed = assert_pack_exact(p, host_input(w), g, sym)
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, what=kname)


# (m, n, k): m = 2..4 with more than four tiles per CU, where the tile kernel runs (fewer
# tiles go to the wide kernel); ragged last tiles, slices of 2 to 8 units
TILE_MANY_CASES = [(2, 16400, 512), (3, 16401, 2048), (4, 16500, 4096)]


@pytest.mark.parametrize("m,n,k", TILE_MANY_CASES)
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_tile_many_tiles(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 7 * k + m + g, n, k))
    x = synthetic.activations(m, k, seed=m * 37 + k).to(xdtype)
    note(f"gemv tile many tiles m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    assert tile_route(g, m, k, n)
    y, kname = run_linear(x, p)
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert kname == f"q4_gemv_tile_{t}"
    packed = assert_pack_exact(p, host_input(w), g, sym)
    cols = np.unique(np.concatenate([np.arange(0, n, 5), np.arange(n - 24, n)]))
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=kname)


GEMV_EDGE = [(1, 16, 32, 32), (16, 1, 32, 32), (5, 37, 96, 32), (16, 33, 192, 64),
             (3, 300, 4096 + 64, 64), (2, 17, 4096 + 32, 32), (11, 129, 1280, 128),
             (16, 4096, 11008, 128), (8, 1000, 256, 128)]


@pytest.mark.parametrize("m,n,k,g", GEMV_EDGE)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_edge_cases(m, n, k, g, xdtype, sym):
    w = torch.from_numpy(pins.random_weights(n + 3 * k, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m * 31 + k).to(xdtype)
    note(f"gemv edge m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    assert kname in gemv_kernels(xdtype)
    packed = assert_pack_exact(p, host_input(w), g, sym)
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, what=kname)


def sparse_group_cases():
    """(m, k, g, kernel, n) for the sparse-group input: the tile kernel (m = 1, and m = 4
    over more than four tiles per CU), the wide kernel (m = 4 and 16), the resident kernel
    (m = 16 over many tiles), the streaming kernel (k not a multiple of 128, or an odd group
    count) and its column-chunked form (m = 16, activations beyond the LDS budget)."""
    out = []
    for g in (32, 64, 128):
        out += [(1, 2048, g, "tile", 40), (4, 2048, g, "tile", 16400), (4, 2048, g, "wide", 40),
                (16, 2048, g, "wide", 40), (16, 2048, g, "resident", 16400),
                (1, 2048 + g, g, "mfma", 40), (4, 2048 + g, g, "mfma", 40), (16, 4096 + g, g, "mfma", 40)]
    return out


@pytest.mark.parametrize("m,k,g,path,n", sparse_group_cases())
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemv_sparse_groups(m, k, g, path, n, xdtype, sym):
    """Groups whose codes all equal the zero point but one, with large activations on
    those columns: sum |x| per group is about 64 g while each row's result is small, so a
    kernel that formed x * (u - z) as a difference of two large biased sums would miss the
    bound by far.  Every GEMV kernel must stay within it (the operand is the exact u - z)."""
    w, x = synthetic.sparse_groups(n, k, g, m, xdtype)
    note(f"gemv sparse groups m={m} k={k} g={g} {path} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    t = "f16" if xdtype == torch.float16 else "bf16"
    assert kname == f"q4_gemv_{path}_{t}"
    packed = assert_pack_exact(p, host_input(w), g, sym)
    worst = assert_linear_close(y, host_input(x), packed, n, k, g, sym, what=kname)
    assert worst < 1e-4, f"{kname}: worst error / (|x||w|) = {worst:.3g}"


def ranged_activations(kind, m, k, seed):
    """bf16 activations whose exponent range picks the operand route of the decode kernels'
    bf16 path: 'narrow' N(0,1); 'huge' and 'tiny' the same times 2^100 and 2^-100 (narrow,
    far from 1); 'wide' with every 37th entry times 2^24 and every 41st times 2^-24 (more
    than 29 binades in every slice); 'subnormal' with every 53rd entry a bf16 subnormal;
    'split' wide in the first half of k and narrow in the second."""
    x = synthetic.activations(m, k, seed, dtype=torch.float32)
    kk = torch.arange(k)
    if kind == "huge":
        x = x * 2.0 ** 100
    elif kind == "tiny":
        x = x * 2.0 ** -100
    elif kind in ("wide", "split"):
        sel = kk < k // 2 if kind == "split" else torch.ones(k, dtype=torch.bool)
        x[:, (kk % 37 == 0) & sel] *= 2.0 ** 24
        x[:, (kk % 41 == 0) & sel] *= 2.0 ** -24
    elif kind == "subnormal":
        x[:, kk % 53 == 0] *= 2.0 ** -130
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("kind", ["narrow", "huge", "tiny", "wide", "subnormal", "split"])
@pytest.mark.parametrize("m,n,k,g", [(1, 70, 4096, 128), (3, 40, 2048, 32), (2, 33, 5120, 64),
                                     (8, 40, 2048, 128), (1, 40, 2048 + 64, 64),
                                     (16, 8200, 4096, 128), (3, 16400, 2048, 32)])
def test_gemv_activation_ranges(kind, m, n, k, g):
    """bf16 activations of every exponent range the decode kernels distinguish: the tile
    kernel (m = 1, and m = 3 over more than four tiles per CU) converts a slice to exact
    fp16 when its nonzero exponents span at most 29 binades and keeps the exact bf16
    operand otherwise; the other kernels (wide, resident, streaming) keep the bf16 operand.
    Each result must meet the bound whichever route a wave took."""
    w = torch.from_numpy(pins.random_weights(n + k + g, max(n, 12), k)[:n])
    x = ranged_activations(kind, m, k, seed=m * 29 + k)
    note(f"gemv activation range {kind} m={m} n={n} k={k} g={g}")
    for sym in (False, True):
        p, _ = pack_guarded(w.to(DEV), g, sym)
        y, kname = run_linear(x, p)
        assert kname in gemv_kernels()
        packed = assert_pack_exact(p, host_input(w), g, sym)
        assert np.isfinite(y).all()
        assert_linear_close(y, host_input(x), packed, n, k, g, sym, what=f"{kname} {kind}")


@pytest.mark.parametrize("m,g", [(1, 64), (5, 64), (16, 64), (17, 64), (64, 64), (1, 128),
                                 (3, 128)])
@pytest.mark.parametrize("sym", [False, True])
def test_linear_special_inputs(m, g, sym):
    """x = 0 gives exactly 0; one-hot x picks one dequantized column.  The decode GEMV
    reproduces it exactly (exact products, one scale multiply per group).  The prefill
    GEMM keeps its sums in units of the current group's scale and moves them to the next
    group's units with an fp32 ratio: a column in group j passes through two roundings
    (ratio, product) per later group and one final product, so its relative error is at
    most (2 * (G - 1 - j) + 1) * 2^-24 to first order."""
    n, k = 48, 512
    w = torch.from_numpy(pins.random_weights(5, n, k))
    p, _ = pack_guarded(w.to(DEV), g, sym)
    qo, so, zo = assert_pack_exact(p, host_input(w), g, sym)
    xhat = oracle.dequant(qo, so, zo, n, k, g, sym)
    note(f"linear zero x m={m} g={g} sym={sym}")
    y, _ = run_linear(torch.zeros(m, k, dtype=torch.bfloat16), p)
    assert np.all(y == 0)
    x = torch.zeros(m, k, dtype=torch.bfloat16)
    cols = [(7 * i + 3) % k for i in range(m)]
    for i, kk in enumerate(cols):
        x[i, kk] = 1.0
    note(f"linear one-hot x m={m} g={g} sym={sym}")
    y, _ = run_linear(x, p)
    for i, kk in enumerate(cols):
        if m <= 16:
            assert np.array_equal(y[i].astype(np.float64), xhat[:, kk]), (i, kk)
        else:
            later = k // g - 1 - kk // g
            bound = (2 * later + 1) * 2.0 ** -24 * (1 + 2.0 ** -20) * np.abs(xhat[:, kk])
            assert np.all(np.abs(y[i].astype(np.float64) - xhat[:, kk]) <= bound), (i, kk)


@pytest.mark.parametrize("m,g", [(1, 64), (16, 64), (17, 64), (300, 64), (1, 128), (4, 128), (300, 128),
                                 (300, 32)])
@pytest.mark.parametrize("sym", [False, True])
def test_linear_zero_scale_groups(m, g, sym):
    """Packed weights from elsewhere may hold S = 0 for a group (a group of zeros stored
    without the 1.0 substitute): such a group contributes exactly 0.  Zero scales sit at
    the first, last and consecutive groups of some rows and cover whole rows of others."""
    n, k = 200, 1024
    G = k // g
    w = torch.from_numpy(pins.random_weights(11, n, k))
    p, _ = pack_guarded(w.to(DEV), g, sym)
    qo, so, zo = assert_pack_exact(p, host_input(w), g, sym)
    so = so.copy()
    rng = np.random.default_rng(12)
    for r in range(0, n, 3):
        so[r, rng.choice(G, size=3, replace=False)] = 0
    so[1, 0] = so[2, G - 1] = 0
    so[4, 3:9] = 0
    so[5, :] = 0
    so[n - 1, :] = 0
    p.scales.copy_(torch.from_numpy(so.view(np.float16)).to(DEV))
    x = synthetic.activations(m, k, seed=13)
    note(f"linear zero-scale groups m={m} g={g} sym={sym}")
    y, kname = run_linear(x, p)
    assert np.all(y[:, 5] == 0) and np.all(y[:, n - 1] == 0)
    assert_linear_close(y, host_input(x), (qo, so, zo), n, k, g, sym, what=kname)


def test_gemm_grouped_decode_pair():
    """The two 7B-like decode projections in one grouped launch (shared x, m = 1): each
    output matches the oracle over all rows and columns."""
    cfg = synthetic.DECODE_7B
    mats = cfg["mats"]
    ws = [m_.make() for m_ in mats]
    x = synthetic.activations(1, mats[0].k, cfg["x_seed"])
    note("grouped decode pair m=1 g=128 asym")
    packs = [pack_guarded(w.to(DEV), 128, False)[0] for w in ws]
    guards = [guarded((1, p.n), torch.float32, SENTINEL_F32) for p in packs]
    q4.q4_w4a16_gemm_grouped(x.to(DEV), packs, outs=[v for _, v in guards])
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() == "q4_gemv_tile_bf16"
    for w, p, (gb, gv) in zip(ws, packs, guards):
        assert guard_intact(gb), "store outside y"
        packed = assert_pack_exact(p, host_input(w), 128, False)
        assert_linear_close(gv.cpu().numpy(), host_input(x), packed, p.n, p.k, 128, False,
                            what="grouped")


@pytest.mark.parametrize("m", [1, 5, 16])
@pytest.mark.parametrize("g,sym", [(32, False), (128, True), (64, False)])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_gemm_grouped_mixed(m, g, sym, xdtype):
    """Three problems of different n (ragged tiles), each with its own activations."""
    k = 1024
    ns = [48, 200, 1000]
    ws = [torch.from_numpy(pins.random_weights(31 + i, max(n, 12), k)[:n]) for i, n in enumerate(ns)]
    xs = [synthetic.activations(m, k, seed=40 + i).to(xdtype) for i in range(len(ns))]
    note(f"grouped mixed m={m} g={g} sym={sym} {xdtype}")
    packs = [pack_guarded(w.to(DEV), g, sym)[0] for w in ws]
    guards = [guarded((m, n), torch.float32, SENTINEL_F32) for n in ns]
    q4.q4_w4a16_gemm_grouped([x.to(DEV) for x in xs], packs, outs=[v for _, v in guards])
    torch.cuda.synchronize()
    assert q4.q4_last_kernel() in gemv_kernels(xdtype)
    for w, x, p, (gb, gv) in zip(ws, xs, packs, guards):
        assert guard_intact(gb), "store outside y"
        packed = assert_pack_exact(p, host_input(w), g, sym)
        assert_linear_close(gv.cpu().numpy(), host_input(x), packed, p.n, k, g, sym,
                            what="grouped")


@pytest.mark.parametrize("m,k,g", [(40, 512, 128), (16, 4160, 64), (16, 11008, 128)])
def test_gemm_grouped_one_by_one(m, k, g):
    """m > 16 (prefill GEMM per problem), a K no tile kernel takes with activations too
    large for the streaming kernel's LDS (decode kernel per problem), and the wide tile
    kernel over both problems in one launch: same results either way."""
    ns = [64, 130]
    ws = [torch.from_numpy(pins.random_weights(50 + i, max(n, 12), k)[:n]) for i, n in enumerate(ns)]
    x = synthetic.activations(m, k, seed=60)
    note(f"grouped one-by-one m={m} k={k} g={g}")
    packs = [pack_guarded(w.to(DEV), g, False)[0] for w in ws]
    ys = q4.q4_w4a16_gemm_grouped(x.to(DEV), packs)
    torch.cuda.synchronize()
    for w, p, y in zip(ws, packs, ys):
        packed = assert_pack_exact(p, host_input(w), g, False)
        assert_linear_close(y.cpu().numpy(), host_input(x), packed, p.n, k, g, False,
                            what="grouped")


def gemm_path(m, n, num_cus=256):
    """Mirror of the C ABI's choice for 16 < m: the GEMV on 16-row chunks (m <= 256) when
    the GEMM's grid (128 x 256 tiles) fits in one round and ceil(m/16) * n < 147456."""
    chunks = -(-m // 16)
    gemm_wgs = -(-m // 128) * -(-n // 256)
    chunked = m <= 256 and gemm_wgs <= 2 * num_cus and chunks * n < 144 * 1024
    return not chunked


def matmul_kernels(m, n, xdtype=torch.bfloat16):
    gemm = {"q4_gemm_mfma_f16" if xdtype == torch.float16 else "q4_gemm_mfma_bf16"}
    return gemm if m > 16 and gemm_path(m, n) else gemv_kernels(xdtype)


# the prefill GEMM itself, also at small m where the grid is wide (n large); k = 96 and 160
# end on a half stage (k % 64 == 32, g = 32)
# (the last three: m >= 512 with a tile per CU, the 256 x 128 tile: ragged m and n, k % 64 == 32)
GEMM_CASES = [(17, 73800, 256, 128), (130, 16400, 384, 64), (300, 129, 96, 32), (256, 9300, 1024, 128),
              (129, 16448, 4096 + 64, 64), (64, 36900, 512, 32), (257, 300, 512, 128), (128, 18500, 1024, 64),
              (40, 73800, 160, 32), (520, 16400, 512, 64), (600, 11000, 1024 + 32, 32), (1000, 8300, 1024, 128)]


@pytest.mark.parametrize("m,n,k,g", GEMM_CASES)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemm_cases(m, n, k, g, xdtype, sym):
    assert gemm_path(m, n)
    w = torch.from_numpy(pins.random_weights(m + n + k, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m + 7 * k).to(xdtype)
    note(f"gemm m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    assert kname == ("q4_gemm_mfma_f16" if xdtype == torch.float16 else "q4_gemm_mfma_bf16")
    packed = assert_pack_exact(p, host_input(w), g, sym)
    # wide shapes: every activation row against a seeded sample of 200 weight rows
    cols = None if m * n * k <= 1 << 28 else synthetic.sample_rows(n, 200, 3).numpy()
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=kname)


# 16 < m <= 256 on narrow grids: the GEMV on 16-row chunks (full chunks grouped by up to 8,
# the rest alone), including m = 17 (one full chunk and one row), multiples of 16, and
# m > 128 (two grouped launches)
MIDM_CASES = [(17, 64, 256, 128), (64, 48, 11008, 128), (40, 1000, 4096, 64), (128, 300, 1024, 32),
              (33, 4096, 11008, 128), (96, 11008, 4096, 128), (112, 5, 512, 64), (256, 300, 1024, 128),
              (200, 4096, 11008, 128), (145, 64, 256, 32), (32, 28672, 1024, 128),
              (64, 28672, 512, 64), (128, 11008, 512, 32)]


@pytest.mark.parametrize("m,n,k,g", MIDM_CASES)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_midm_chunked_cases(m, n, k, g, xdtype, sym):
    assert not gemm_path(m, n)
    w = torch.from_numpy(pins.random_weights(m + n + k, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m + 7 * k).to(xdtype)
    note(f"mid-m chunked m={m} n={n} k={k} g={g} {xdtype} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y, kname = run_linear(x, p)
    assert kname in gemv_kernels(xdtype)
    packed = assert_pack_exact(p, host_input(w), g, sym)
    # large shapes: every activation row against a seeded sample of 200 weight rows
    cols = None if n * k <= 1 << 24 else synthetic.sample_rows(n, 200, 5).numpy()
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=kname)


# mid-size batches on narrow weights: the GEMM with its K range split into a workspace
# (m > 64, or m > 32 from 2^27 weights on, where 128 x 128 tiles leave CUs idle), including
# ragged m, k % 64 == 32 (a short last stage in the last split) and every group size
SPLITK_CASES = [(128, 4096, 11008, 128), (256, 4096, 11008, 64), (100, 300, 4096, 32),
                (200, 11008, 4096, 128), (80, 28672, 2048, 128), (65, 1000, 8192, 64),
                (72, 500, 4096 + 32, 32)]


@pytest.mark.parametrize("m,n,k,g", SPLITK_CASES)
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sym", [False, True])
def test_gemm_splitk_cases(m, n, k, g, xdtype, sym):
    need = q4.q4_w4a16_gemm_workspace(m, n, k, g)
    assert need > 0 and need % (4 * m * n) == 0, need
    w = torch.from_numpy(pins.random_weights(m + 3 * n + k, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m + 11 * k).to(xdtype)
    note(f"gemm split-K m={m} n={n} k={k} g={g} {xdtype} sym={sym} parts={need // (4 * m * n)}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    wsb, wsv = guarded((need // 4,), torch.float32, SENTINEL_F32)
    yb, yv = guarded((m, n), torch.float32, SENTINEL_F32)
    q4.q4_w4a16_gemm(x.to(DEV), p, out=yv, workspace=wsv)
    torch.cuda.synchronize()
    gname = "q4_gemm_mfma_f16" if xdtype == torch.float16 else "q4_gemm_mfma_bf16"
    assert q4.q4_last_kernels() == [gname, "q4_gemm_splitk_reduce"], q4.q4_last_kernels()
    assert guard_intact(yb), "store outside y"
    assert guard_intact(wsb), "store outside the workspace"
    y = yv.cpu().numpy()
    packed = assert_pack_exact(p, host_input(w), g, sym)
    cols = None if m * n * k <= 1 << 28 else synthetic.sample_rows(n, 200, 9).numpy()
    assert_linear_close(y, host_input(x), packed, n, k, g, sym, cols=cols, what=f"{gname} split-K")
    # the parts add in a fixed order: a second call gives the same bits
    q4.q4_w4a16_gemm(x.to(DEV), p, out=yv, workspace=wsv)
    assert np.array_equal(yv.cpu().numpy(), y)
    # 16-bit output: the rounding of the same fp32 sums
    yh = q4.q4_w4a16_gemm(x.to(DEV), p, out_dtype=torch.bfloat16, workspace=wsv)
    assert torch.equal(yh.cpu(), torch.from_numpy(y).to(torch.bfloat16))


# corrupted scale detection: ragged n, k % 64 == 32, sym and asym, the 7B MLP shape
@pytest.mark.parametrize("n,k,g,sym", [(300, 1024, 128, False), (77, 4096 + 32, 32, True),
                                       (11008, 4096, 128, False), (5, 64, 64, True)])
def test_check_scales(n, k, g, sym):
    """A packed weight from the quantizer reports no corrupted scale; scales overwritten
    with infinities, NaNs and negative values (and -0, which stays legal) give the oracle's
    counts and first index, through the binding and through the C ABI into a guarded
    result."""
    w = torch.from_numpy(pins.random_weights(n + k, max(n, 12), k)[:n])
    note(f"check scales n={n} k={k} g={g} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    assert q4.q4_check_scales(p) == (0, 0, -1)
    assert q4.q4_last_kernels() == ["q4_check_scales_clear", "q4_check_scales", "q4_check_scales_finish"]
    so = p.scales.cpu().numpy().view(np.uint16).copy()
    G = k // g
    rng = np.random.default_rng(n + g)
    idx = rng.choice(n * G, size=min(40, n * G), replace=False)
    pats = np.array([0x7C00, 0xFC00, 0x7E00, 0xBC00, 0x8001, 0x8000, 0xFE01], dtype=np.uint16)
    flat = so.reshape(-1)
    flat[idx] = pats[np.arange(idx.size) % pats.size]
    p.scales.copy_(torch.from_numpy(so.view(np.float16)).to(DEV))
    exp = oscales.check_scales(so)
    assert exp[0] > 0 and exp[1] > 0
    rb, rv = guarded((3,), torch.int64, -7)
    assert q4.lib().q4_check_scales(p.scales.data_ptr(), n, k, g, rv.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert guard_intact(rb, sentinel=-7), "store outside the result"
    assert tuple(rv.cpu().tolist()) == exp
    assert q4.q4_check_scales(p) == exp


def test_gemm_splitk_workspace_rules():
    """The binding allocates the workspace when not given; a short one is refused by the
    C ABI; split=False and no workspace run the product unsplit."""
    m, n, k, g = 128, 4096, 11008, 128
    w = torch.from_numpy(pins.random_weights(5, n, k))
    p = q4.q4_quantize_pack(w.to(DEV), g, False)
    x = synthetic.activations(m, k, seed=6).to(DEV)
    y1 = q4.q4_w4a16_gemm(x, p)
    assert q4.q4_last_kernels()[-1] == "q4_gemm_splitk_reduce"
    y0 = q4.q4_w4a16_gemm(x, p, split=False)
    assert "q4_gemm_splitk_reduce" not in q4.q4_last_kernels()
    need = q4.q4_w4a16_gemm_workspace(m, n, k, g)
    short = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(q4.Q4Error):
        q4.q4_w4a16_gemm(x, p, workspace=short)
    torch.cuda.synchronize()
    rows = np.arange(0, m, 17)
    cols = synthetic.sample_rows(n, 64, 4).numpy()
    packed = (p.qweight.cpu().numpy().view(np.uint32), p.scales.cpu().view(torch.int16).numpy().view(np.uint16),
              p.zeros.cpu().numpy().view(np.uint32))
    for y in (y0, y1):
        assert_linear_close(y.cpu().numpy(), host_input(x.cpu()), packed, n, k, g, False, rows=rows,
                            cols=cols, what="split-K rules")


def test_launch_record_names_every_kernel():
    """q4_last_kernels / q4_last_launch_count report every launch of the last call: one
    for a decode product, the grouped chunk launch plus the remainder for a chunked mid-m
    product, partial and combine for attention."""
    n, k, g = 1000, 4096, 64
    w = torch.from_numpy(pins.random_weights(77, n, k))
    p, _ = pack_guarded(w.to(DEV), g, False)
    assert q4.q4_last_kernels() == ["q4_quant_pack_f32"] and q4.q4_last_launch_count() == 1
    x1 = synthetic.activations(1, k, seed=3).to(DEV)
    q4.q4_w4a16_gemm(x1, p)
    assert q4.q4_last_kernels() == ["q4_gemv_tile_bf16"] and q4.q4_last_launch_count() == 1
    x40 = synthetic.activations(40, k, seed=4).to(DEV)
    note("launch record: chunked m = 40")
    q4.q4_w4a16_gemm(x40, p)
    assert q4.q4_last_kernels() == ["q4_gemv_wide_bf16"], q4.q4_last_kernels()
    assert q4.q4_last_launch_count() == 2          # two 16-row chunks grouped, then 8 rows
    heads, d = 4, 128
    kc = q4.empty_kv_cache(heads, 64, d, 32, False, DEV)
    vc = q4.empty_kv_cache(heads, 64, d, 32, False, DEV)
    kv = synthetic.kv_tokens(64, heads, d, 5, "k").to(DEV)
    q4.q4_kv_quantize(kv, kc, 0)
    q4.q4_kv_quantize(kv, vc, 0)
    q4.q4_kv_attention(synthetic.query(heads, d, 6).to(DEV), kc, vc, 64, 0.1)
    assert q4.q4_last_kernel() == "q4_kv_attention_bf16"
    assert q4.q4_last_kernels() == ["q4_kv_partial_bf16", "q4_kv_combine"]
    assert q4.q4_last_launch_count() == 2
    torch.cuda.synchronize()


def test_gemm_prefill_70b_sampled():
    """The 70B-like prefill at full size, in the configuration the benchmark times;
    checked on a seeded sample of 40 activation rows x 320 weight rows (with edges)."""
    cfg = synthetic.PREFILL_70B
    mat = cfg["w"]
    w = mat.make()
    x = synthetic.activations(cfg["m"], mat.k, cfg["x_seed"], outlier_seed=mat.seed,
                              outlier_factor=cfg["x_outlier_factor"])
    note(f"gemm prefill {mat.name} m={cfg['m']}")
    p, _ = pack_guarded(w.to(DEV), 128, False)
    y, kname = run_linear(x, p)
    assert kname == "q4_gemm_mfma_bf16"
    assert np.isfinite(y).all()
    rows_w = synthetic.sample_rows(mat.n, 320, 11).numpy()
    rows_x = synthetic.sample_rows(cfg["m"], 40, 12).numpy()
    w_rows = w[torch.as_tensor(rows_w)]
    qo, so, zo = assert_pack_exact(p, host_input(w_rows), 128, False, rows=rows_w)
    yr, ya = oracle.linear(host_input(x), qo, so, zo, len(rows_w), mat.k, 128, False,
                           rows=rows_x)
    yg = y[np.ix_(rows_x, rows_w)]
    ok = oracle.within_tolerance(yg, yr, ya)
    assert ok.all(), f"{int((~ok).sum())} sampled outputs outside the bound"


# --------------------------------------------------------------------------- output epilogue
# (m, n, k, g, path): every product path with a 16-bit output: the tile kernel, the wide
# kernel (one tile and two tiles per workgroup), the streaming kernel (k not a multiple of
# 128), the chunked mid-M GEMV and the prefill GEMM (a ragged m, and k ending on a half stage)
EPILOGUE_CASES = [(1, 300, 1024, 128, "tile"), (3, 16500, 1024, 64, "tile"), (3, 130, 2048, 64, "wide"),
                  (8, 100, 1024, 32, "wide"),
                  (16, 16392, 512, 128, "wide"), (2, 300, 4096 + 64, 64, "mfma"), (40, 1000, 1024, 64, "midm"),
                  (300, 129, 96, 32, "gemm"), (257, 300, 512, 128, "gemm"), (520, 16400, 512, 128, "gemm")]
HALF_ULP = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def assert_epilogue(y16: torch.Tensor, y32: np.ndarray, ydt, x, packed, n, k, g, sym, what):
    """y16 is the round-to-nearest-even of the fp32 result of the same product (bit for
    bit), and within the matmul bound plus half an ulp of the 16-bit type of the oracle."""
    exp = torch.from_numpy(np.ascontiguousarray(y32)).to(ydt)
    got = y16.cpu()
    assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), f"{what}: not the rounding of the fp32 sums"
    qo, so, zo = packed
    yr, ya = oracle.linear(host_input(x), qo, so, zo, n, k, g, sym)
    base = 1e-3 * ya + 1e-5
    bound = base + HALF_ULP[ydt] * (np.abs(yr) + base) + (2.0 ** -25 if ydt == torch.float16 else 0.0)
    gv = got.float().numpy().astype(np.float64)
    # sums beyond the 16-bit range (fp16 above 65504: the seeded stress rows) are signed
    # infinities, as the rounding defines; the bound applies to the rest
    over = ~np.isfinite(gv)
    assert (np.sign(gv[over]) == np.sign(yr[over])).all() and (np.abs(yr[over]) > 65504 * 0.999).all(), \
        f"{what}: an infinity where the sum is in range"
    gv[over] = yr[over]
    err = np.abs(gv - yr)
    if not (err <= bound).all():
        bad = np.argwhere(err > bound)[:4]
        det = [(int(i), int(j), float(gv[i, j]), float(y32[i, j]), float(yr[i, j]), float(ya[i, j]),
                float(bound[i, j])) for i, j in bad]
        raise AssertionError(f"{what}: {int((err > bound).sum())} outside the bound; "
                             f"(row, col, y16, y32, oracle, |x||w|, bound): {det}")


@pytest.mark.parametrize("m,n,k,g,path", EPILOGUE_CASES)
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float16])
def test_output_epilogue(m, n, k, g, path, ydt, xdtype):
    sym = (m + g) % 2 == 1
    w = torch.from_numpy(pins.random_weights(n + 13 * k + m, max(n, 12), k)[:n])
    x = synthetic.activations(m, k, seed=m * 29 + k).to(xdtype)
    note(f"epilogue {path} m={m} n={n} k={k} g={g} {xdtype} -> {ydt} sym={sym}")
    p, _ = pack_guarded(w.to(DEV), g, sym)
    y32, k32 = run_linear(x, p)
    yb, yv = guarded((m, n), ydt, SENTINEL_F32)
    q4.q4_w4a16_gemm(x.to(DEV), p, out=yv, split=False)
    k16 = q4.q4_last_kernel()
    torch.cuda.synchronize()
    assert guard_intact(yb), "store outside y"
    assert k16 == k32, (k16, k32)  # the same path, only the store differs
    packed = assert_pack_exact(p, host_input(w), g, sym)
    assert_epilogue(yv, y32, ydt, x, packed, n, k, g, sym, f"{k16} -> {ydt}")


@pytest.mark.parametrize("m", [1, 5])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float16])
def test_output_epilogue_grouped(m, ydt):
    """Grouped products (one decode launch, shared and separate activations) with 16-bit
    outputs: each the rounding of the same call's fp32 outputs."""
    k, g, sym = 1024, 64, False
    ns = [48, 200, 1000]
    ws = [torch.from_numpy(pins.random_weights(71 + i, max(n, 12), k)[:n]) for i, n in enumerate(ns)]
    x = synthetic.activations(m, k, seed=81)
    note(f"epilogue grouped m={m} -> {ydt}")
    packs = [pack_guarded(w.to(DEV), g, sym)[0] for w in ws]
    y32 = q4.q4_w4a16_gemm_grouped(x.to(DEV), packs)
    guards = [guarded((m, n), ydt, SENTINEL_F32) for n in ns]
    q4.q4_w4a16_gemm_grouped(x.to(DEV), packs, outs=[v for _, v in guards])
    torch.cuda.synchronize()
    for w, p, y, (gb, gv) in zip(ws, packs, y32, guards):
        assert guard_intact(gb), "store outside y"
        packed = assert_pack_exact(p, host_input(w), g, sym)
        assert_epilogue(gv, y.cpu().numpy(), ydt, x, packed, p.n, k, g, sym, f"grouped -> {ydt}")
