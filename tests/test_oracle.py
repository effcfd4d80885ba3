"""CPU tests: the fp64 oracle against its pins, and planted mistakes that the pins must catch."""

import os
import sys
import types

import pytest

import oracle
from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


# Plausible mistakes, each planted in a copy of the oracle's source on the CPU. Every one of them
# must make at least one pin fail; otherwise the pins would not be able to tell a wrong oracle.
MUTANTS = {
    "causal_strict": ("return j <= i", "return j < i"),
    "causal_flipped": ("return j <= i", "return j >= i"),
    "scale_dropped": ("s = scale * (q[b, h] @ k[b, g].T)", "s = (q[b, h] @ k[b, g].T)"),
    "gqa_modulo": ("return h // (heads_q // heads_kv)", "return h % heads_kv"),
    "padding_keys_only": ("return (i < n) & (j < n)", "return (j < n)"),
    "lse_without_max": ("lse = np.where(nonempty, m + np.log(", "lse = np.where(nonempty, 0 * m + np.log("),
    "softmax_unnormalised": ("e / np.where(nonempty, denom, 1.0)[:, None]", "e"),
    "dv_untransposed": ("dv[b, g] += p.T @ do[b, h]", "dv[b, g] += p @ do[b, h]"),
    "ds_missing_rowdot": ("ds = p * (dp - rowdot[:, None])", "ds = p * dp"),
    "ds_rowdot_sign": ("ds = p * (dp - rowdot[:, None])", "ds = p * (dp + rowdot[:, None])"),
    "dq_scale_dropped": ("dq[b, h] = scale * (ds @ k[b, g])", "dq[b, h] = (ds @ k[b, g])"),
    "dk_transposed": ("dk[b, g] += scale * (ds.T @ q[b, h])", "dk[b, g] += scale * (ds @ q[b, h])"),
    "dk_overwrite_group": ("dk[b, g] += scale", "dk[b, g] = scale"),
    "block_rows_cols_swapped": ("return keep[rows[:, None], cols[None, :]]", "return keep.T[rows[:, None], cols[None, :]]"),
}


def _load_mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found in the oracle: {old!r}"
    name = "oracle_mutant_%d" % abs(hash((old, new)))
    mod = types.ModuleType(name)
    sys.modules[name] = mod  # dataclasses resolve annotations through sys.modules
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    except Exception:
        del sys.modules[name]
        raise
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake {name}"
