"""The GPTQ oracle against its pins, and planted mistakes in a copy of it (CPU only)."""
import importlib.util
import os

import pytest

import oracle
import oracle.gptq as gq
import pins


@pytest.mark.parametrize("check", pins.GPTQ_CHECKS, ids=lambda c: c.__name__)
def test_gptq_pin(orc, check):
    check(gq, orc)


MUTANTS = [
    ("lower_factor", "    L = lo.T\n", "    L = lo\n"),
    ("err_not_normalized", "err = (W[:, j] - w_hat) / L[j, j]", "err = (W[:, j] - w_hat)"),
    ("update_sign", "W[:, j + 1:b1] -= np.outer(err, L[j, j + 1:b1])",
     "W[:, j + 1:b1] += np.outer(err, L[j, j + 1:b1])"),
    ("no_lazy_update", "        W[:, b1:] -= err_block @ L[b0:b1, b1:]\n", "        pass\n"),
    ("damp_everything", "h[np.diag_indices_from(h)] = d + damp * d  # G3", "h = h + damp * h  # G3"),
    ("dead_feature_kept", "    d[d == 0.0] = 1.0                      # G4\n", ""),
    ("floor_rounding", "np.rint(W[:, j] / s[:, gj])", "np.floor(W[:, j] / s[:, gj])"),
    ("hessian_not_doubled", "h = 2.0 * (x64.T @ x64)", "h = x64.T @ x64"),
    ("update_from_quantized", "err = (W[:, j] - w_hat) / L[j, j]", "err = (wf[:, j] - w_hat) / L[j, j]"),
    ("act_order_ascending", 'np.argsort(-energy, kind="stable")', 'np.argsort(energy, kind="stable")'),
    ("act_order_ties_by_higher_index", 'np.argsort(-energy, kind="stable")',
     'np.lexsort((-np.arange(energy.size), -energy))'),
    ("act_order_group_of_position", "gj = order[j] // g", "gj = j // g"),
    ("act_order_codes_not_placed", "placed[:, order] = codes", "placed[:, :] = codes"),
    ("act_order_hessian_not_permuted", "h = np.asarray(h, dtype=np.float64)[np.ix_(order, order)]",
     "h = np.asarray(h, dtype=np.float64)"),
    ("act_order_energy_abs", "energy = np.sum(x64 * x64, axis=0)", "energy = np.sum(np.abs(x64), axis=0)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_gptq_pins_catch_mutant(tmp_path, orc, name, old, new):
    src = open(gq.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / "gptq_mutant.py"
    path.write_text(src.replace(old, new).replace("from . import default as _default",
                                                  "from oracle import default as _default"),
                    encoding="utf-8")
    spec = importlib.util.spec_from_file_location("gptq_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for check in pins.GPTQ_CHECKS:
        try:
            check(mod, orc)
        except Exception as exc:
            caught.append(f"{check.__name__}: {type(exc).__name__}")
    assert caught, f"mutant {name} passed every GPTQ pin"
