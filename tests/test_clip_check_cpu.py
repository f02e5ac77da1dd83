"""The clip-choice validity check accepts the oracle's own search and rejects planted
mistakes made with the oracle on the CPU: a group packed at its second-best ratio, a
flipped code, a scale off by one ulp."""
import numpy as np
import pytest
import torch

import oracle
import pins
import synthetic
from clip_check import check_clip_choice, clip_choice_report


def _case(sym):
    w = pins.random_weights(61 if sym else 62, 12, 512)
    w[0, 3] = np.float32(9.0)   # outliers, so clipping wins in some groups
    w[1, 200] = np.float32(-40.0)
    return w


@pytest.mark.parametrize("sym", [False, True])
def test_accepts_the_oracle(sym):
    w = _case(sym)
    q, s, z = oracle.quantize_pack_mse(w, 64, sym)
    assert check_clip_choice(oracle.default(), w, 64, sym, q, s, z) == 1.0


@pytest.mark.parametrize("sym", [False, True])
def test_accepts_the_oracle_bf16_bits(sym):
    w = torch.from_numpy(_case(sym)).to(torch.bfloat16)
    host = (synthetic.as_u16(w), oracle.BF16)
    q, s, z = oracle.quantize_pack_mse(host, 64, sym)
    assert check_clip_choice(oracle.default(), host, 64, sym, q, s, z) == 1.0


@pytest.mark.parametrize("sym", [False, True])
def test_rejects_second_best_ratio(sym):
    w = _case(sym)
    o = oracle.default()
    errs = o.mse_errors(w, 64, sym)
    _, _, _, ch = o.quantize_pack_mse(w, 64, sym, with_choice=True)
    # a group whose second-best error is clearly above its best
    order = np.sort(errs, axis=2)
    gap = order[..., 1] > order[..., 0] * (1 + 1e-9)
    row, j = map(int, np.argwhere(gap & (ch > 0))[0])
    alt = ch.copy()
    e = errs[row, j].copy()
    e[ch[row, j]] = np.inf
    alt[row, j] = int(np.argmin(e))
    q, s, z = o.quantize_pack_clip(w, 64, sym, alt)
    ratio, err_at, _, bound = clip_choice_report(o, w, 64, sym, q, s, z)
    assert ratio[row, j] >= 0 and err_at[row, j] > bound[row, j]
    with pytest.raises(AssertionError, match="above the bound"):
        check_clip_choice(o, w, 64, sym, q, s, z)


def test_rejects_flipped_code_and_scale():
    w = _case(False)
    o = oracle.default()
    q, s, z = o.quantize_pack_mse(w, 64, False)
    q2 = q.copy()
    q2[3, 5] ^= np.uint32(1 << 8)
    with pytest.raises(AssertionError, match="no clip ratio"):
        check_clip_choice(o, w, 64, False, q2, s, z)
    s2 = s.copy()
    s2[4, 1] += np.uint16(1)
    with pytest.raises(AssertionError, match="no clip ratio"):
        check_clip_choice(o, w, 64, False, q, s2, z)
