"""The sparse-group decode input has the power to catch a biased-operand GEMV.

A decode kernel may be tempted to multiply the activations by a biased code 128 + u (exact
in bf16) and remove the bias with a second sum over 128 + z.  Both sums are then about
128 sum |x| while their difference, the group's dot product, can be tiny; the fp32
rounding of the two sums is relative to the large values and escapes the bound
1e-3 * sum |x| |w_hat| + 1e-5.  This CPU test plants that formulation (fp32 sums in
numpy, sequential order) and checks that the input of ``synthetic.sparse_groups`` drives
it outside the bound, while the exact-operand formulation (products x * (u - z), then fp32
sums) stays inside.  The GPU parity test on the same input therefore fails a kernel that
computes the biased form.
"""
import numpy as np

import oracle
import synthetic


def _codes(q, so, zo, n, k, g, sym):
    """Unpacked codes u [n, k], zero points z [n, G] and scales S [n, G] (fp32)."""
    u = np.zeros((n, k), dtype=np.int64)
    for i in range(8):
        u[:, i::8] = (q >> (4 * i)) & 0xF
    G = k // g
    if sym:
        z = np.full((n, G), 8, dtype=np.int64)
    else:
        z = np.zeros((n, G), dtype=np.int64)
        for j in range(G):
            z[:, j] = (zo[:, j // 8] >> (4 * (j % 8))) & 0xF
    s = so.view(np.float16).astype(np.float32)
    return u, z, s


def _fp32_dot(a):
    acc = np.float32(0.0)
    for v in a:
        acc = np.float32(acc + v)
    return acc


def _gemv(x, u, z, s, g, biased):
    """y [m, n] with fp32 products and sequential fp32 sums per group, then acc += S * part."""
    m, k = x.shape
    n = u.shape[0]
    y = np.zeros((m, n), dtype=np.float32)
    for i in range(m):
        for r in range(n):
            acc = np.float32(0.0)
            for j in range(k // g):
                xs = x[i, j * g:(j + 1) * g]
                uu = u[r, j * g:(j + 1) * g]
                if biased:
                    d = _fp32_dot(xs * (np.float32(128) + uu.astype(np.float32)))
                    c = _fp32_dot(xs * np.float32(128 + z[r, j]))
                    part = np.float32(d - c)
                else:
                    part = _fp32_dot(xs * (uu - z[r, j]).astype(np.float32))
                acc = np.float32(acc + s[r, j] * part)
            y[i, r] = acc
    return y


def test_sparse_groups_defeat_biased_sums():
    n, k, g, m = 6, 512, 128, 2
    w, x = synthetic.sparse_groups(n, k, g, m)
    xb = synthetic.as_u16(x)
    xf = x.float().numpy()
    for sym in (False, True):
        q, so, zo = oracle.quantize_pack(w.numpy(), g, sym)
        yr, ya = oracle.linear((xb, oracle.BF16), q, so, zo, n, k, g, sym)
        u, z, s = _codes(q, so, zo, n, k, g, sym)
        exact = _gemv(xf, u, z, s, g, biased=False)
        biased = _gemv(xf, u, z, s, g, biased=True)
        assert oracle.within_tolerance(exact, yr, ya).all()
        bad = ~oracle.within_tolerance(biased, yr, ya)
        assert bad.sum() >= n, f"sym={sym}: the biased sums stayed inside the bound"
        worst = float((np.abs(biased - yr) / (1e-3 * ya + 1e-5)).max())
        assert worst > 10, worst
