"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` on a mismatch.
The same checks run against the real oracle (test_oracle_pins.py) and against copies of
its C source with a planted mistake (test_oracle_mutants.py), which must each fail at
least one check.

What pins what:
  * hand-worked groups (tests/golden/hand_worked_groups.txt): codes, scales, zero points
    and word layout, derived by hand from the affine quantizer of "LLM Quantization:
    GPTQ·AWQ·SmoothQuant·FP8·KV Cache (7/10)" §Affine Quantization;
  * numpy's float16 conversion (an independent implementation) pins fp32 <-> fp16;
  * closed-form properties: code ranges, zero exactly representable, |x - x_hat| <= s/2
    for unclipped weights, 15*S and 7*S against the data range, 2^4 levels;
  * brute force: each code is the nearest grid level (search over all 16 levels);
  * byte accounting from the pages' arithmetic (payload P*b/8, fp16 scale per 128 weights
    = 0.015625 B/weight, 32 four-bit codes + one fp16 scale = 4.5 bits/weight);
  * the fp64 matmul against numpy's float64 matmul of the dequantized weights, one-hot
    and zero activations, integer data with unit scales;
  * the KV cache ("Quantization Algorithms 단권화", KV-cache chapter, §INT4 group scheme):
    cache rows against the weight quantizer applied to each (token, head) row, appends in
    steps against one append, untouched rows; attention against the special cases
    softmax reduces to (one token: that token's value; zero query: the mean; two tokens:
    the logistic form; a huge scale: the top-scoring token's value), token-order
    invariance and a brute-force loop with Python's math.exp.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_worked_groups.txt")


# --------------------------------------------------------------------------- helpers

def load_golden():
    rows = []
    with open(GOLDEN, encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            f = [c.strip() for c in line.split("|")]
            rows.append(dict(
                name=f[0], sym=(f[1] == "sym"), g=int(f[2]),
                values=np.array([np.float32(v) for v in f[3].split()], dtype=np.float32),
                s16=int(f[4], 16), z=int(f[5]),
                codes=[int(c) for c in f[6].split()],
                words=[int(w, 16) for w in f[7].split()]))
    return rows


def unpack_codes(qweight: np.ndarray, k: int) -> np.ndarray:
    """Stored 4-bit codes [n, k] from packed words (little-endian nibbles)."""
    q = qweight.astype(np.uint64)
    shifts = (4 * np.arange(8, dtype=np.uint64))
    codes = (q[:, :, None] >> shifts[None, None, :]) & np.uint64(0xF)
    return codes.reshape(qweight.shape[0], k).astype(np.int64)


def unpack_zeros(zeros: np.ndarray, G: int) -> np.ndarray:
    z = zeros.astype(np.uint64)
    shifts = (4 * np.arange(8, dtype=np.uint64))
    nib = (z[:, :, None] >> shifts[None, None, :]) & np.uint64(0xF)
    return nib.reshape(zeros.shape[0], -1)[:, :G].astype(np.int64)


def f16_values(scales: np.ndarray) -> np.ndarray:
    return scales.view(np.float16).astype(np.float64)


def random_weights(seed: int, n: int, k: int) -> np.ndarray:
    """A mix of distributions that stresses every branch: normal, heavy outliers,
    one-sided groups, all-zero rows, constant rows, tiny values (subnormal fp16
    scales) and huge values (fp16 scale saturation)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    w[1] *= 50                                   # wide row
    w[2, ::37] *= 400                            # sparse outliers
    w[3] = np.abs(w[3]) + np.float32(0.5)        # all positive (one-sided)
    w[4] = -np.abs(w[4]) - np.float32(0.25)      # all negative (one-sided)
    w[5] = 0                                     # degenerate groups
    w[6] = np.float32(0.375)                     # constant row
    w[7] *= np.float32(1e-4)                     # scales in the fp16 subnormal range
    w[10] *= np.float32(1e-7)                    # scales that underflow fp16 to zero
    w[8] = rng.standard_normal(k).astype(np.float32) * np.float32(3e5)  # scale > 65504
    w[9] = np.round(rng.standard_normal(k) * 3).astype(np.float32)      # small integers
    return w


# --------------------------------------------------------------------------- checks

def check_golden_groups(o):
    for r in load_golden():
        v = r["values"].reshape(1, -1)
        q, s, z = o.quantize_pack(v, r["g"], r["sym"])
        k = v.shape[1]
        codes = unpack_codes(q, k)[0].tolist()
        assert codes == r["codes"], (r["name"], codes, r["codes"])
        assert [int(x) for x in q[0]] == r["words"], (r["name"], [hex(int(x)) for x in q[0]])
        assert int(s[0, 0]) == r["s16"], (r["name"], hex(int(s[0, 0])))
        if not r["sym"]:
            assert int(unpack_zeros(z, 1)[0, 0]) == r["z"], (r["name"], int(z[0, 0]))
        # dequantized value of each code: S * (u - z), z = 8 for symmetric
        xh = o.dequant(q, s, z, 1, k, r["g"], r["sym"])[0]
        S = float(np.uint16(r["s16"]).view(np.float16))
        zz = 8 if r["sym"] else r["z"]
        assert np.array_equal(xh, S * (np.array(r["codes"], dtype=np.float64) - zz)), r["name"]


def check_fp16_conversion(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    finite = np.isfinite(ref)
    # widening: every binary16 pattern
    for b, r in zip(bits.tolist(), ref.tolist()):
        got = o.f16_bits_to_f32(b)
        if np.isnan(r):
            assert np.isnan(got), hex(b)
        else:
            assert got == r and np.signbit(got) == np.signbit(r), (hex(b), got, r)
    # narrowing: exact values, midpoints (ties), and one fp32 ulp either side
    vals = ref[finite & (np.abs(ref) < np.float32(65504))]
    vals = np.sort(np.unique(vals[vals >= 0]))
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    rng = np.random.default_rng(0)
    rnd = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e9, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
                        2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11), 6.1e-5, 1e-45, -1e-45],
                       dtype=np.float32)
    pool = np.concatenate([vals, -vals, mids, -mids, up, dn, rnd, special]).astype(np.float32)
    for f in pool.tolist():
        f32 = np.float32(f)
        with np.errstate(over="ignore"):
            want = np.array([f32]).astype(np.float16).view(np.uint16)[0]
        got = o.f32_to_f16_bits(float(f32))
        if np.isnan(f32):
            assert (got & 0x7C00) == 0x7C00 and (got & 0x3FF), hex(got)
        else:
            assert got == int(want), (float(f32), hex(got), hex(int(want)))


def _quantize_many(o, w, g, sym):
    n, k = w.shape
    q, s, z = o.quantize_pack(w, g, sym)
    G = k // g
    codes = unpack_codes(q, k)
    S = f16_values(s)
    zz = np.full((n, G), 8, dtype=np.int64) if sym else unpack_zeros(z, G)
    return q, s, z, codes, S, zz


def check_invariants(o):
    for seed, (n, k, g) in enumerate([(12, 256, 32), (12, 512, 64), (12, 1024, 128),
                                      (12, 96, 32)]):
        w = random_weights(seed, n, k)
        for sym in (False, True):
            q, s, z, codes, S, zz = _quantize_many(o, w, g, sym)
            G = k // g
            assert codes.min() >= 0 and codes.max() <= 15
            normal_g = ((s & 0x7C00) != 0) & (s != 0x7BFF)   # normal, unsaturated scale
            if sym:
                # |x / S| <= 7 (1 + 2^-11) rounds to <= 7 when S is a normal fp16 value,
                # so symmetric codes never need q = -8
                assert (codes[np.repeat(normal_g, g, axis=1)] != 0).all()
            assert zz.min() >= 0 and zz.max() <= 15
            assert np.all(np.isfinite(S)) and np.all(S > 0)
            xh = o.dequant(q, s, z, n, k, g, sym)
            Sk = np.repeat(S, g, axis=1)
            zk = np.repeat(zz, g, axis=1)
            # x_hat is S * (u - z) with the stored z
            assert np.array_equal(xh, Sk * (codes - zk))
            wd = w.astype(np.float64)
            err = np.abs(wd - xh)
            bound = Sk / 2 * (1 + 2.0 ** -19)
            big = err > bound
            # zero is exactly representable: a zero weight lands on the zero point
            zero = wd == 0
            assert np.all(codes[zero] == zk[zero]) and np.all(xh[zero] == 0)
            if sym:
                # no clipping in symmetric mode while S is a normal fp16 value
                nz = np.repeat(normal_g, g, axis=1)
                assert not np.any(big & nz), np.argwhere(big & nz)[:4]
            else:
                sat = np.repeat(s == 0x7BFF, g, axis=1)
                clip = big & ~sat
                # clipping happens only from above, at the top code
                assert np.all((codes[clip] == 15) & (wd[clip] > xh[clip])), \
                    np.argwhere(clip & ((codes != 15) | (wd <= xh)))[:4]
                # with a normal fp16 scale it costs less than one level; a subnormal scale
                # can round far below s and clip more, but only when 15*S < the range
                normal = np.repeat((s & 0x7C00) != 0, g, axis=1)
                assert np.all(err[clip & normal] < Sk[clip & normal])
                wg_ = wd.reshape(n, G, g)
                span_ = np.maximum(wg_.max(axis=2), 0) - np.minimum(wg_.min(axis=2), 0)
                short = np.repeat(15 * S < span_, g, axis=1)
                assert np.all(short[clip])
            # the grid spans the data: 15 S (asym) or 7 S (sym) equals the range up to
            # the fp16 rounding of the scale
            wg = wd.reshape(n, G, g)
            if sym:
                span = np.abs(wg).max(axis=2)
                lev = 7.0
            else:
                span = np.maximum(wg.max(axis=2), 0) - np.minimum(wg.min(axis=2), 0)
                lev = 15.0
            ok = (span == 0) | (s == 0x7BFF) | (span < 2.0 ** -14 * lev)
            rel = np.abs(lev * S - span) / np.where(span > 0, span, 1)
            assert np.all(ok | (rel <= 2.0 ** -11 * 1.0001)), rel[~ok].max()


def check_brute_force_nearest(o):
    rng = np.random.default_rng(7)
    for trial in range(40):
        g = int(rng.choice([8, 16, 32]))
        n = 8
        w = (rng.standard_normal((n, 4 * g)) * rng.choice([0.02, 1.0, 30.0])).astype(np.float32)
        if trial % 5 == 0:
            w += np.float32(rng.standard_normal())
        for sym in (False, True):
            q, s, z, codes, S, zz = _quantize_many(o, w, g, sym)
            Sk = np.repeat(S, g, axis=1)
            zk = np.repeat(zz, g, axis=1)
            levels = np.arange(16, dtype=np.float64)
            grid = Sk[:, :, None] * (levels[None, None, :] - zk[:, :, None])
            d = np.abs(w.astype(np.float64)[:, :, None] - grid)
            if sym:
                d[:, :, 0] = np.inf  # q = -8 is outside what max|x|/7 can reach
            best = d.argmin(axis=2)
            srt = np.sort(d, axis=2)
            clear = (srt[:, :, 1] - srt[:, :, 0]) > 1e-6 * Sk  # not a near-tie
            assert np.all(codes[clear] == best[clear]), np.argwhere(codes != best)[:4]


def check_levels_and_bytes(o):
    # 4 bits -> 2^4 = 16 levels: the L16 golden group reaches all of them
    rows = {r["name"]: r for r in load_golden()}
    assert sorted(set(rows["L16"]["codes"])) == list(range(16))
    # payload = P * b / 8 bytes; 7e9 parameters at 4 bits = 3.5e9 bytes
    qw, sc, zw = o.sizes(4096, 4096, 128)
    assert qw * 4 == 4096 * 4096 * 4 // 8
    P = 7_000_000_000
    assert o.sizes(1, 8 * (P // 8), 8)[0] * 4 == P * 4 // 8 == 3_500_000_000
    # one fp16 scale per 128 weights = 2/128 = 0.015625 bytes per weight
    assert sc * 2 / (4096 * 4096) == 0.015625
    # zero points: 8 four-bit values per word, rows padded to whole words
    assert zw == 4096 * ((4096 // 128 + 7) // 8)
    assert o.sizes(11008, 11008, 128)[2] == 11008 * 11  # 86 groups -> 11 words per row
    # symmetric, group 32: 32 four-bit codes + one fp16 scale = 4.5 bits per weight
    qw, sc, _ = o.sizes(64, 4096, 32)
    assert (qw * 4 + sc * 2) * 8 / (64 * 4096) == 4.5


def check_dequant_closed_forms(o):
    # integer data with range [0, 15] (asym) or max |x| = 7 (sym) has S = 1 exactly and
    # dequantizes to itself
    rng = np.random.default_rng(3)
    a = rng.integers(0, 16, (6, 64)).astype(np.float32)
    a[:, 0], a[:, 1], a[:, 32], a[:, 63] = 0, 15, 0, 15
    q, s, z = o.quantize_pack(a, 32, False)
    assert np.all(s == 0x3C00)
    assert np.array_equal(o.dequant(q, s, z, 6, 64, 32, False), a.astype(np.float64))
    b = rng.integers(-7, 8, (6, 64)).astype(np.float32)
    b[:, 0], b[:, 33] = 7, -7
    q, s, z = o.quantize_pack(b, 32, True)
    assert np.all(s == 0x3C00)
    assert np.array_equal(o.dequant(q, s, z, 6, 64, 32, True), b.astype(np.float64))
    # symmetric storage is asymmetric storage with every zero point equal to 8
    w = random_weights(11, 12, 256)
    q, s, _ = o.quantize_pack(w, 64, True)
    eights = np.full((12, 1), 0x88888888, dtype=np.uint32)
    assert np.array_equal(o.dequant(q, s, eights, 12, 256, 64, False),
                          o.dequant(q, s, eights, 12, 256, 64, True))


def check_linear(o):
    rng = np.random.default_rng(5)
    n, k, g, m = 24, 384, 64, 3
    w = random_weights(21, n, k)
    for sym in (False, True):
        q, s, z = o.quantize_pack(w, g, sym)
        xh = o.dequant(q, s, z, n, k, g, sym)
        x = rng.standard_normal((m, k)).astype(np.float32)
        y, yabs = o.linear(x, q, s, z, n, k, g, sym)
        ref = x.astype(np.float64) @ xh.T
        refabs = np.abs(x.astype(np.float64)) @ np.abs(xh).T
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * refabs.max())
        assert np.allclose(yabs, refabs, rtol=1e-12)
        # sampled (m, n) pairs equal the full result
        rows, cols = np.array([2, 0]), np.array([23, 5, 0, 7])
        ys, _ = o.linear(x, q, s, z, n, k, g, sym, rows=rows, cols=cols)
        assert np.array_equal(ys, y[np.ix_(rows, cols)])
        # one-hot activation picks one dequantized column exactly; zero gives zero
        for kk in (0, 1, 63, 64, k - 1):
            e = np.zeros((1, k), dtype=np.float32)
            e[0, kk] = 1
            ye, _ = o.linear(e, q, s, z, n, k, g, sym)
            assert np.array_equal(ye[0], xh[:, kk])
        y0, _ = o.linear(np.zeros((2, k), dtype=np.float32), q, s, z, n, k, g, sym)
        assert np.all(y0 == 0)
        # bf16 and fp16 activations are read exactly
        xb = x.astype(np.float16)
        yb, _ = o.linear(xb, q, s, z, n, k, g, sym)
        assert np.allclose(yb, xb.astype(np.float64) @ xh.T, rtol=1e-12,
                           atol=1e-12 * refabs.max())
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16
        xbf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        yb2, _ = o.linear((bits, 2), q, s, z, n, k, g, sym)
        assert np.allclose(yb2, xbf @ xh.T, rtol=1e-12, atol=1e-12 * refabs.max())
    # integer weights with unit scales and integer activations give exact integers
    a = rng.integers(0, 16, (8, 128)).astype(np.float32)
    a[:, 0], a[:, 1] = 0, 15
    q, s, z = o.quantize_pack(a, 128, False)
    xi = rng.integers(-4, 5, (2, 128)).astype(np.float32)
    y, _ = o.linear(xi, q, s, z, 8, 128, 128, False)
    assert np.array_equal(y, xi.astype(np.float64) @ a.astype(np.float64).T)


def check_argument_rejection(o):
    w = np.zeros((2, 96), dtype=np.float32)
    for g in (64, 7, 12):          # 96 is not a multiple of 64 or 7; 12 leaves k % 8 == 0
        try:
            o.quantize_pack(w, g, False)
        except ValueError:
            assert g != 12, "k=96, g=12 is a valid layout"
            continue
        assert g == 12, f"group {g} should be rejected for k=96"
    assert o.lib.orc_quantize_pack(None, 0, 2, 96, 0, 0, None, None, None, None) == -1
    assert o.lib.orc_quantize_pack(None, 0, 2, 20, 4, 0, None, None, None, None) == -1


# --------------------------------------------------------------------------- MSE clip search

MSE_CANDIDATES = 11


def _fp16_scale(s32):
    """Stored fp16 scale bits of an fp32 scale, degenerate values replaced (numpy's own
    float16 conversion, round-to-nearest-even)."""
    with np.errstate(over="ignore"):         # scales past fp16's range become inf, then 65504
        b = int(np.array([s32], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
    if b & 0x7FFF == 0:
        b = 0x3C00
    if b == 0x7C00:
        b = 0x7BFF
    return b


def mse_candidates_numpy(v, sym):
    """Every clip ratio alpha = (20 - i) / 20 of one group v (float32), quantized the way
    the affine RTN quantizer does with the range scaled by alpha, written again in numpy:
    a list of (error in float64, s16 bits, z, codes) per candidate."""
    f32 = np.float32
    out = []
    for i in range(MSE_CANDIDATES):
        alpha = f32(20 - i) / f32(20)
        if sym:
            s = (alpha * np.max(np.abs(v))) / f32(7)
            lo = f32(0)
        else:
            mn = min(f32(0), v.min())
            mx = max(f32(0), v.max())
            lo = alpha * mn
            s = (alpha * mx - lo) / f32(15)
        s16 = _fp16_scale(s)
        S = np.array([s16], dtype=np.uint16).view(np.float16).astype(np.float32)[0]
        qmin, qmax = (f32(-8), f32(7)) if sym else (f32(0), f32(15))
        z = 0 if sym else int(np.clip(np.rint(-lo / S), qmin, qmax))
        q = np.clip(np.rint(v / S) + f32(z), qmin, qmax).astype(np.int64)
        xhat = np.float64(S) * (q - z).astype(np.float64)
        err = float(np.sum((v.astype(np.float64) - xhat) ** 2))
        out.append((err, s16, z, q))
    return out


def check_mse_brute_force(o):
    """Each group's pick is a minimal-error candidate of an independent numpy search (up
    to the order of the fp64 sum), no earlier candidate quantizes the group identically
    (equal errors keep the earlier ratio), and the stored bits are that candidate's."""
    for seed, n, k, g, sym in [(41, 12, 256, 32, False), (42, 12, 256, 128, True),
                               (43, 12, 512, 64, False), (44, 12, 128, 32, True)]:
        w = random_weights(seed, n, k)
        w[11, :g] = np.linspace(-1, 1, g, dtype=np.float32)
        w[11, g - 1] = np.float32(20)              # one far outlier
        q, s, z, ch = o.quantize_pack_mse(w, g, sym, with_choice=True)
        G = k // g
        codes = unpack_codes(q, k)
        zz = unpack_zeros(z, G) if not sym else None
        picked_clip = 0
        for row in range(n):
            for j in range(G):
                v = w[row, j * g:(j + 1) * g]
                cands = mse_candidates_numpy(v, sym)
                i = int(ch[row, j])
                assert 0 <= i < MSE_CANDIDATES
                err, s16, zc, qc = cands[i]
                emin = min(c[0] for c in cands)
                assert err <= emin * (1 + 1e-12), (seed, row, j, i, err, emin)
                for i2 in range(i):
                    c2 = cands[i2]
                    assert not (c2[1] == s16 and c2[2] == zc and np.array_equal(c2[3], qc)), \
                        (seed, row, j, i, i2)
                    assert c2[0] >= err * (1 - 1e-12), (seed, row, j, i, i2)
                assert int(s[row, j]) == s16, (seed, row, j)
                u = codes[row, j * g:(j + 1) * g]
                assert np.array_equal(u, qc + 8 if sym else qc), (seed, row, j)
                if not sym:
                    assert int(zz[row, j]) == zc, (seed, row, j)
                picked_clip += i > 0
        assert picked_clip > 0, "no group chose a clipped range"
    # a Gaussian group: a clipped range strictly lowers the error below plain RTN's
    w = np.random.default_rng(45).standard_normal((1, 128)).astype(np.float32)
    _, _, _, ch = o.quantize_pack_mse(w, 128, False, with_choice=True)
    c = mse_candidates_numpy(w[0], False)
    assert int(ch[0, 0]) > 0 and c[int(ch[0, 0])][0] < c[0][0] * (1 - 1e-6)


def check_mse_errors_exact(o):
    """Every candidate's error, as the oracle sums it, is the exact sum of squares of that
    candidate's reconstruction (rational arithmetic on the independent numpy candidates)
    to within the rounding of g fp64 squares and g - 1 fp64 additions: relative error at
    most (g + 2) * 2^-53."""
    from fractions import Fraction
    u = 2.0 ** -53
    rows = [0, 2, 3, 7, 8, 10]  # normal, outliers, one-sided, fp16-subnormal, saturated, underflow
    for seed, k, g, sym in [(46, 256, 128, False), (47, 128, 32, True), (48, 256, 64, False)]:
        w = np.ascontiguousarray(random_weights(seed, 12, k)[rows])
        w[0, :g] *= np.float32(1e-3)                  # small errors next to large ones
        w[0, g - 1] = np.float32(30)                  # an outlier: clipping matters
        n = len(rows)
        errs = o.mse_errors(w, g, sym)
        assert errs.shape == (n, k // g, MSE_CANDIDATES)
        for row in range(n):
            for j in range(k // g):
                v = w[row, j * g:(j + 1) * g]
                for i, (_, s16, z, q) in enumerate(mse_candidates_numpy(v, sym)):
                    S = Fraction(float(np.array([s16], np.uint16).view(np.float16)[0]))
                    exact = sum((Fraction(float(x)) - S * int(c - z)) ** 2 for x, c in zip(v, q))
                    got = Fraction(float(errs[row, j, i]))
                    assert abs(got - exact) <= (g + 2) * Fraction(u) * exact, (seed, row, j, i)


def check_mse_pack_at_ratio(o):
    """Quantizing at a given clip ratio reproduces that candidate of the independent numpy
    search bit for bit; ratio index 0 (alpha = 1) is the RTN quantizer; the search's
    result is the pack at its chosen ratio, and that ratio is the first smallest error."""
    for seed, n, k, g, sym in [(49, 12, 256, 64, False), (50, 12, 256, 128, True)]:
        w = random_weights(seed, n, k)
        w[2, 5] = np.float32(-25)
        G = k // g
        errs = o.mse_errors(w, g, sym)
        qm, sm, zm, ch = o.quantize_pack_mse(w, g, sym, with_choice=True)
        for row in range(n):
            for j in range(G):
                e = errs[row, j]
                assert int(ch[row, j]) == int(np.flatnonzero(e == e.min())[0]), (seed, row, j)
        qc, sc, zc = o.quantize_pack_clip(w, g, sym, ch)
        assert np.array_equal(qc, qm) and np.array_equal(sc, sm) and np.array_equal(zc, zm)
        qr, sr, zr = o.quantize_pack(w, g, sym)
        q0, s0, z0 = o.quantize_pack_clip(w, g, sym, 0)
        assert np.array_equal(q0, qr) and np.array_equal(s0, sr) and np.array_equal(z0, zr)
        for i in (3, MSE_CANDIDATES - 1):
            qi, si, zi = o.quantize_pack_clip(w, g, sym, i)
            codes, zz = unpack_codes(qi, k), (None if sym else unpack_zeros(zi, G))
            for row in range(n):
                for j in range(G):
                    _, s16, z, q = mse_candidates_numpy(w[row, j * g:(j + 1) * g], sym)[i]
                    assert int(si[row, j]) == s16, (seed, i, row, j)
                    assert np.array_equal(codes[row, j * g:(j + 1) * g], q + 8 if sym else q)
                    if not sym:
                        assert int(zz[row, j]) == z, (seed, i, row, j)
    try:
        o.quantize_pack_clip(np.zeros((1, 32), np.float32), 32, False, MSE_CANDIDATES)
    except ValueError:
        pass
    else:
        raise AssertionError("a ratio index past the grid was accepted")


def check_mse_rtn_limit(o):
    """alpha = 1 is plain RTN: wherever the search keeps it, the bits equal the RTN
    quantizer's (itself pinned by the hand-worked groups)."""
    for g, sym in [(32, False), (128, True), (64, False)]:
        w = random_weights(50 + g, 12, 512)
        qm, sm, zm, ch = o.quantize_pack_mse(w, g, sym, with_choice=True)
        qr, sr, zr = o.quantize_pack(w, g, sym)
        G = 512 // g
        keep = ch == 0
        assert keep.any()
        assert np.array_equal(sm[keep], sr[keep])
        cm, cr = unpack_codes(qm, 512), unpack_codes(qr, 512)
        for row, j in zip(*np.nonzero(keep)):
            assert np.array_equal(cm[row, j * g:(j + 1) * g], cr[row, j * g:(j + 1) * g])
        if not sym:
            assert np.array_equal(unpack_zeros(zm, G)[keep], unpack_zeros(zr, G)[keep])


# --------------------------------------------------------------------------- KV cache

def _kv_fill(o, seed, heads, t_cap, d, g, sym, n_tok):
    """Random K and V for n_tok tokens quantized into fresh head-major caches."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_tok, heads, d)).astype(np.float32)
    v = (rng.standard_normal((n_tok, heads, d)) * 0.5 + 0.25).astype(np.float32)
    kc, vc = o.kv_cache(heads, t_cap, d, g), o.kv_cache(heads, t_cap, d, g)
    o.kv_quantize(k, g, sym, kc, 0)
    o.kv_quantize(v, g, sym, vc, 0)
    return k, v, kc, vc


def _kv_hat(o, cache, heads, d, g, sym):
    qc, sc, zc = cache
    rows = qc.shape[0]
    return o.dequant(qc, sc, zc, rows, d, g, sym).reshape(heads, rows // heads, d)


def check_kv_cache_placement(o):
    heads, t_cap, d, g = 3, 10, 128, 32
    kv = random_weights(31, 7 * heads, d).reshape(7, heads, d)
    for sym in (False, True):
        cache = o.kv_cache(heads, t_cap, d, g)
        cache[0][:], cache[1][:], cache[2][:] = 0xDEADBEEF, 0x1234, 0xCAFEF00D
        o.kv_quantize(kv[:5], g, sym, cache, 2)      # a prefill of 5 tokens at positions 2..6
        o.kv_quantize(kv[5:6], g, sym, cache, 7)     # then one decode token at position 7
        rq, rs, rz = o.quantize_pack(kv[:6].reshape(6 * heads, d), g, sym)
        qc, sc, zc = cache
        for t in range(6):
            for h in range(heads):
                r, src = h * t_cap + 2 + t, t * heads + h
                assert np.array_equal(qc[r], rq[src]) and np.array_equal(sc[r], rs[src])
                if not sym:
                    assert np.array_equal(zc[r], rz[src])
        for h in range(heads):
            for t in (0, 1, 8, 9):                   # rows never written
                r = h * t_cap + t
                assert np.all(qc[r] == 0xDEADBEEF) and np.all(sc[r] == 0x1234)
        if sym:
            assert np.all(zc == 0xCAFEF00D)          # symmetric caches have no zero points
        # writing past the cache's capacity is refused
        try:
            o.kv_quantize(kv[:4], g, sym, cache, 7)
        except ValueError:
            pass
        else:
            raise AssertionError("t0 + t_new > t_cap accepted")


def check_kv_attention(o):
    import math
    heads, t_cap, d, g = 4, 24, 64, 32
    rng = np.random.default_rng(41)
    for sym in (False, True):
        _, _, kc, vc = _kv_fill(o, 43 + sym, heads, t_cap, d, g, sym, t_cap)
        kh, vh = _kv_hat(o, kc, heads, d, g, sym), _kv_hat(o, vc, heads, d, g, sym)
        q = rng.standard_normal((heads, d)).astype(np.float32)
        q64 = q.astype(np.float64)
        scores = (kh @ q64[:, :, None])[..., 0]      # [heads, t_cap], unscaled
        # one token: its softmax weight is exactly 1
        out, _, _ = o.kv_attention(q, kc, vc, 1, g, sym, 0.125)
        assert np.array_equal(out, vh[:, 0])
        # zero query: equal weights, the mean of the cached values
        out, _, _ = o.kv_attention(np.zeros_like(q), kc, vc, 17, g, sym, 0.125)
        assert np.allclose(out, vh[:, :17].mean(axis=1), rtol=1e-13, atol=1e-15)
        # two tokens: o = v1 + (v0 - v1) / (1 + e^(s1 - s0))
        out, _, _ = o.kv_attention(q, kc, vc, 2, g, sym, 0.125)
        s = 0.125 * scores[:, :2]
        ref = vh[:, 1] + (vh[:, 0] - vh[:, 1]) / (1.0 + np.exp(s[:, 1] - s[:, 0]))[:, None]
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
        # a huge scale leaves the top-scoring token alone (every other weight underflows)
        n = 20
        srt = np.sort(scores[:, :n], axis=1)
        gap = float((srt[:, -1] - srt[:, -2]).min())
        big = 1000.0 / gap
        out, _, _ = o.kv_attention(q, kc, vc, n, g, sym, big)
        top = scores[:, :n].argmax(axis=1)
        assert np.array_equal(out, vh[np.arange(heads), top])
        # tolerance references
        out, sabs, vabs = o.kv_attention(q, kc, vc, n, g, sym, 0.125)
        assert np.allclose(sabs, 0.125 * (np.abs(kh[:, :n]) @ np.abs(q64)[:, :, None])[..., 0]
                           .max(axis=1), rtol=1e-13)
        assert np.array_equal(vabs, np.abs(vh[:, :n]).max(axis=1))
        # the order of the cached tokens does not matter
        k, v, _, _ = _kv_fill(o, 43 + sym, heads, t_cap, d, g, sym, t_cap)
        perm = rng.permutation(n)
        kc2, vc2 = o.kv_cache(heads, t_cap, d, g), o.kv_cache(heads, t_cap, d, g)
        o.kv_quantize(np.ascontiguousarray(k[:n][perm]), g, sym, kc2, 0)
        o.kv_quantize(np.ascontiguousarray(v[:n][perm]), g, sym, vc2, 0)
        out2, _, _ = o.kv_attention(q, kc2, vc2, n, g, sym, 0.125)
        assert np.allclose(out2, out, rtol=1e-12, atol=1e-14)
        # brute force with Python floats on a small slice: heads 0..1, 5 tokens
        out5, _, _ = o.kv_attention(q, kc, vc, 5, g, sym, 0.125)
        for h in range(2):
            sc = [0.125 * sum(float(q[h, i]) * float(kh[h, t, i]) for i in range(d)) for t in range(5)]
            w = [math.exp(x - max(sc)) for x in sc]
            for i in (0, 7, 31, 32, 63):
                val = sum(w[t] * float(vh[h, t, i]) for t in range(5)) / sum(w)
                assert abs(out5[h, i] - val) <= 1e-12 * max(1.0, abs(val))


ALL_CHECKS = [check_golden_groups, check_fp16_conversion, check_invariants,
              check_brute_force_nearest, check_levels_and_bytes, check_dequant_closed_forms,
              check_linear, check_argument_rejection, check_mse_brute_force,
              check_mse_rtn_limit, check_mse_errors_exact, check_mse_pack_at_ratio,
              check_kv_cache_placement, check_kv_attention]


# --------------------------------------------------------------------------- GPTQ

def _gptq_x(seed, t, k, rank=8):
    """Correlated calibration tokens: N(0,1) plus a few shared factors."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((t, rank))
    b = rng.standard_normal((k, rank)) / np.sqrt(rank)
    return (rng.standard_normal((t, k)) + 1.5 * f @ b.T).astype(np.float32)


def check_gptq_hessian(gq, o):
    """H = 2 X^T X (numpy's fp64 matmul), the diagonal scaled by 1 + 0.01, a dead feature's
    diagonal 1 + 0.01 and its row and column zero."""
    x = _gptq_x(60, 50, 32)
    x[:, 5] = 0
    h = gq.hessian(x)
    ref = 2.0 * x.astype(np.float64).T @ x.astype(np.float64)
    off = ~np.eye(32, dtype=bool)
    assert np.allclose(h[off], ref[off], rtol=1e-13, atol=1e-12)
    d = np.diag(ref).copy()
    d[5] = 1.0
    assert np.allclose(np.diag(h), d * 1.01, rtol=1e-13)
    assert np.all(h[5, off[5]] == 0) and np.all(h[off[:, 5], 5] == 0)


def check_gptq_identity_is_rtn(gq, o):
    """With H a multiple of the identity nothing propagates: GPTQ is RTN, bit for bit."""
    for g, sym in [(32, False), (128, True), (64, False)]:
        w = random_weights(61 + g, 12, 256)
        qg, sg, zg = gq.gptq_quantize(w, 3.7 * np.eye(256), g, sym, oracle=o)
        qr, sr, zr = o.quantize_pack(w, g, sym)
        assert np.array_equal(qg, qr) and np.array_equal(sg, sr)
        if not sym:
            assert np.array_equal(zg, zr)


def check_gptq_pair_closed_form(gq, o):
    """Only features 0 and 1 coupled, H = [[a, b], [b, c]] (+ identity elsewhere): column
    1 is quantized at w_1 + (w_0 - w_hat_0) b / c (the one-step optimal update), every
    other column as RTN."""
    n, k, g = 48, 64, 32
    w = random_weights(62, n, k)
    a, b, c = 2.0, 1.2, 1.3
    h = np.eye(k)
    h[0, 0], h[0, 1], h[1, 0], h[1, 1] = a, b, b, c
    for sym in (False, True):
        qg, sg, zg = gq.gptq_quantize(w, h, g, sym, oracle=o)
        qr, _, zr = o.quantize_pack(w, g, sym)
        cg, cr = unpack_codes(qg, k), unpack_codes(qr, k)
        assert np.array_equal(cg[:, 2:], cr[:, 2:]) and np.array_equal(cg[:, 0], cr[:, 0])
        s0 = f16_values(sg)[:, 0]
        z0 = np.full(n, 8) if sym else unpack_zeros(zr, k // g)[:, 0]
        w64 = w.astype(np.float64)
        w_hat0 = s0 * (cr[:, 0] - z0)
        w1 = w64[:, 1] + (w64[:, 0] - w_hat0) * b / c
        u1 = np.clip(np.rint(w1 / s0) + z0, 0, 15)
        assert np.array_equal(cg[:, 1], u1), (sym, cg[:, 1], u1)
        assert not np.array_equal(cg[:, 1], cr[:, 1]), "the pair should change a code"


def check_gptq_block_and_scale_invariance(gq, o):
    """Blocks of 128 with the lazy update give the same codes as one block; scaling H by
    a constant changes nothing."""
    k = 384
    x = _gptq_x(63, 600, k)
    h = gq.hessian(x)
    w = random_weights(64, 12, k)
    q1, _, _ = gq.gptq_quantize(w, h, 64, False, oracle=o)
    q2, _, _ = gq.gptq_quantize(w, h, 64, False, block=k, oracle=o)
    q3, _, _ = gq.gptq_quantize(w, 7.25 * h, 64, False, oracle=o)
    assert np.array_equal(q1, q2)
    assert np.array_equal(q1, q3)


def check_gptq_upper_factor_form(gq, o):
    """An independent formulation: with H = U U^T (U upper, the Cholesky factor of H in
    reversed order), column j is quantized at w_j + sum_{i<j} (w_i - w_hat_i) U_ij / U_jj.
    No inverse is taken; the codes must equal the oracle's."""
    n, k, g = 12, 128, 32
    x = _gptq_x(65, 400, k)
    h = gq.hessian(x)
    w = random_weights(66, n, k)
    qg, sg, zg = gq.gptq_quantize(w, h, g, False, oracle=o)
    rev = np.linalg.cholesky(h[::-1, ::-1])          # J H J = R R^T, R lower
    U = rev[::-1, ::-1]                               # H = U U^T, U upper
    s = f16_values(sg)
    z = unpack_zeros(zg, k // g)
    w64 = w.astype(np.float64)
    codes = np.zeros((n, k), dtype=np.int64)
    d = np.zeros((n, k))
    for j in range(k):
        wj = w64[:, j] + (d[:, :j] @ U[:j, j]) / U[j, j]
        u = np.clip(np.rint(wj / s[:, j // g]) + z[:, j // g], 0, 15)
        codes[:, j] = u
        d[:, j] = w64[:, j] - s[:, j // g] * (u - z[:, j // g])
    assert np.array_equal(unpack_codes(qg, k), codes)


def check_gptq_lowers_layer_error(gq, o):
    """On correlated calibration data GPTQ's layer-output error is below RTN's."""
    k, g = 256, 64
    x = _gptq_x(67, 1000, k)
    h = gq.hessian(x)
    w = random_weights(68, 24, k)[12:]   # the Gaussian-like rows
    for sym in (False, True):
        qg, sg, zg = gq.gptq_quantize(w, h, g, sym, oracle=o)
        qr, sr, zr = o.quantize_pack(w, g, sym)
        eg = gq.layer_error(w, o.dequant(qg, sg, zg, 12, k, g, sym), x)
        er = gq.layer_error(w, o.dequant(qr, sr, zr, 12, k, g, sym), x)
        assert eg < 0.9 * er, (sym, eg, er)


def check_gptq_act_order_hand_worked(gq, o):
    """Act-order by hand: column energies sum_t x_ti^2 = [4, 2, 0, 4, 2, 9] sort to the
    order [5, 0, 3, 1, 4, 2] (largest first, equal energies by the lower index, the
    never-active column last); energies all equal give the natural order."""
    x = np.array([[2, 1, 0, 2, 1, 3], [0, 1, 0, 0, 1, 0]], dtype=np.float32)
    assert gq.act_order(x).tolist() == [5, 0, 3, 1, 4, 2]
    signs = np.where(np.random.default_rng(70).random((16, 40)) < 0.5, -1.0, 1.0)
    assert gq.act_order(signs.astype(np.float32)).tolist() == list(range(40))


def _upper_factor_sweep(w64, h, s, z, g, order):
    """The sweep in the upper-factor form (no inverse) over the columns in ``order``:
    with Hp = h[order][:, order] = U U^T (U upper), the column at position p is quantized
    at w_p + sum_{i<p} d_i U_ip / U_pp with its own group's quantizer; codes are returned in
    column order."""
    n, k = w64.shape
    hp = h[np.ix_(order, order)]
    U = np.linalg.cholesky(hp[::-1, ::-1])[::-1, ::-1]
    wp = w64[:, order]
    codes = np.zeros((n, k), dtype=np.int64)
    d = np.zeros((n, k))
    for p in range(k):
        gi = order[p] // g
        v = wp[:, p] + (d[:, :p] @ U[:p, p]) / U[p, p]
        u = np.clip(np.rint(v / s[:, gi]) + z[:, gi], 0, 15)
        codes[:, order[p]] = u
        d[:, p] = wp[:, p] - s[:, gi] * (u - z[:, gi])
    return codes


def check_gptq_act_order_upper_factor(gq, o):
    """Act-order against the independent upper-factor formulation run in the act-order
    sequence: the codes must be equal; the sequence crosses groups, and the result differs
    from the natural-order sweep."""
    n, k, g = 12, 128, 32
    x = _gptq_x(71, 400, k)
    x *= np.linspace(0.3, 3.0, k, dtype=np.float32)[::-1][np.random.default_rng(72).permutation(k)]
    h = gq.hessian(x)
    order = gq.act_order(x)
    assert (np.asarray(order) // g != np.arange(k) // g).any()
    w = random_weights(73, n, k)
    qa, sa, za = gq.gptq_quantize(w, h, g, False, oracle=o, order=order)
    qn, _, _ = gq.gptq_quantize(w, h, g, False, oracle=o)
    codes = _upper_factor_sweep(w.astype(np.float64), h, f16_values(sa), unpack_zeros(za, k // g),
                                g, np.asarray(order))
    assert np.array_equal(unpack_codes(qa, k), codes)
    assert not np.array_equal(qa, qn)


def check_gptq_act_order_permutation_invariance(gq, o):
    """Permuting the input features within their groups (W's columns, X's columns, H's
    rows and columns) permutes act-order's codes the same way, bit for bit: the sweep
    order follows the energies, not the positions.  (The natural order has no such
    property.)"""
    n, k, g = 12, 256, 64
    x = _gptq_x(74, 500, k)
    w = random_weights(75, n, k)
    rng = np.random.default_rng(76)
    pi = np.concatenate([j * g + rng.permutation(g) for j in range(k // g)])
    h = gq.hessian(x)
    e = np.sum(x.astype(np.float64) ** 2, axis=0)
    assert len(np.unique(e)) == k
    for sym in (False, True):
        q1, s1, z1 = gq.gptq_quantize(w, h, g, sym, oracle=o, order=gq.act_order(x))
        q2, s2, z2 = gq.gptq_quantize(np.ascontiguousarray(w[:, pi]), h[np.ix_(pi, pi)], g, sym,
                                      oracle=o, order=gq.act_order(x[:, pi]))
        assert np.array_equal(unpack_codes(q1, k)[:, pi], unpack_codes(q2, k)), sym
        assert np.array_equal(s1, s2)


def check_gptq_act_order_lowers_layer_error(gq, o):
    """With act-order the layer-output error is still below RTN's."""
    k, g = 256, 64
    x = _gptq_x(77, 1000, k) * np.geomspace(0.1, 10, 256, dtype=np.float32)
    h = gq.hessian(x)
    w = random_weights(78, 24, k)[12:]
    qa, sa, za = gq.gptq_quantize(w, h, g, True, oracle=o, order=gq.act_order(x))
    qr, sr, zr = o.quantize_pack(w, g, True)
    ea = gq.layer_error(w, o.dequant(qa, sa, za, 12, k, g, True), x)
    er = gq.layer_error(w, o.dequant(qr, sr, zr, 12, k, g, True), x)
    assert ea < 0.9 * er, (ea, er)


GPTQ_CHECKS = [check_gptq_hessian, check_gptq_identity_is_rtn, check_gptq_pair_closed_form,
               check_gptq_block_and_scale_invariance, check_gptq_upper_factor_form,
               check_gptq_lowers_layer_error, check_gptq_act_order_hand_worked,
               check_gptq_act_order_upper_factor, check_gptq_act_order_permutation_invariance,
               check_gptq_act_order_lowers_layer_error]
