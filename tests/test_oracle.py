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
    "block_rows_cols_swapped": ("return keep[brows[:, None], bcols[None, :]]",
                                "return keep.T[brows[:, None], bcols[None, :]]"),
    "dense_transposed": ("return arr[:sq, :sk][qi] != 0", "return arr.T[:sq, :sk][qi] != 0"),
    "dense_inverted": ("return arr[:sq, :sk][qi] != 0", "return arr[:sq, :sk][qi] == 0"),
    "dense_head_ignored": ("        arr = arr[b, h]\n        return arr[:sq, :sk][qi] != 0",
                           "        arr = arr[0, 0]\n        return arr[:sq, :sk][qi] != 0"),
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


def test_row_subset_matches_full_oracle():
    """attention_rows evaluates the same definition on a subset of rows."""
    import numpy as np

    r = np.random.default_rng(3)
    q, k, v = r.standard_normal((2, 4, 70, 8)), r.standard_normal((2, 2, 70, 8)), r.standard_normal((2, 2, 70, 8))
    lay = (r.random((2, 2)) < 0.5).astype(np.uint8)
    dense = (r.random((70, 70)) < 0.4).astype(np.uint8)
    dense[5] = 0                                   # a row that sees nothing
    dense4 = (r.random((2, 4, 70, 70)) < 0.4).astype(np.uint8)
    specs = [oracle.MaskSpec("none"), oracle.MaskSpec("causal"),
             oracle.MaskSpec("padding", lengths=np.array([30, 70], np.int32)),
             oracle.MaskSpec("block", layout=lay), oracle.MaskSpec("dense", dense=dense),
             oracle.MaskSpec("dense", dense=dense4)]
    rows = np.array([0, 5, 31, 63, 64, 69])
    for spec in specs:
        o, lse = oracle.attention_fwd(q, k, v, spec, 0.3)
        for b in range(2):
            for h in range(4):
                o_r, lse_r = oracle.attention_rows(q, k, v, spec, 0.3, b, h, rows)
                np.testing.assert_allclose(o_r, o[b, h, rows], rtol=0, atol=1e-14)
                np.testing.assert_array_equal(np.isneginf(lse_r), np.isneginf(lse[b, h, rows]))
                fin = np.isfinite(lse_r)
                np.testing.assert_allclose(lse_r[fin], lse[b, h, rows][fin], rtol=0, atol=1e-14)


def test_bwd_head_matches_full_oracle():
    """attention_bwd_head is the per-(b, h) share of attention_bwd."""
    import numpy as np

    r = np.random.default_rng(4)
    q, k, v = r.standard_normal((2, 4, 40, 8)), r.standard_normal((2, 2, 40, 8)), r.standard_normal((2, 2, 40, 8))
    do = r.standard_normal(q.shape)
    lay4 = (r.random((2, 4, 1, 1)) < 2).astype(np.uint8)
    dense = (r.random((40, 40)) < 0.4).astype(np.uint8)
    dense4 = (r.random((2, 4, 40, 40)) < 0.4).astype(np.uint8)
    dense4[1, 2, 7] = 0                            # a row that sees nothing
    for spec in (oracle.MaskSpec("none"), oracle.MaskSpec("causal"),
                 oracle.MaskSpec("padding", lengths=np.array([13, 40], np.int32)),
                 oracle.MaskSpec("block", layout=lay4), oracle.MaskSpec("dense", dense=dense),
                 oracle.MaskSpec("dense", dense=dense4)):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, spec, 0.5)
        dk_sum, dv_sum = np.zeros_like(dk), np.zeros_like(dv)
        for b in range(2):
            for h in range(4):
                dq_h, dk_h, dv_h = oracle.attention_bwd_head(q, k, v, do, spec, 0.5, b, h)
                np.testing.assert_allclose(dq_h, dq[b, h], rtol=0, atol=1e-13)
                dk_sum[b, h // 2] += dk_h
                dv_sum[b, h // 2] += dv_h
        np.testing.assert_allclose(dk_sum, dk, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv_sum, dv, rtol=0, atol=1e-13)


def test_dq_rows_match_full_oracle():
    """attention_dq_rows is attention_bwd's dQ restricted to a subset of rows."""
    import numpy as np

    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((2, 4, 70, 8)), r.standard_normal((2, 2, 70, 8)), r.standard_normal((2, 2, 70, 8))
    do = r.standard_normal(q.shape)
    lay = (r.random((2, 2)) < 0.5).astype(np.uint8)
    dense = (r.random((70, 70)) < 0.4).astype(np.uint8)
    specs = [oracle.MaskSpec("none"), oracle.MaskSpec("causal"),
             oracle.MaskSpec("padding", lengths=np.array([30, 70], np.int32)),
             oracle.MaskSpec("block", layout=lay), oracle.MaskSpec("dense", dense=dense)]
    rows = np.array([0, 5, 31, 63, 64, 69])
    for spec in specs:
        dq, _, _ = oracle.attention_bwd(q, k, v, do, spec, 0.3)
        for b in range(2):
            for h in range(4):
                got = oracle.attention_dq_rows(q, k, v, do, spec, 0.3, b, h, rows)
                np.testing.assert_allclose(got, dq[b, h, rows], rtol=0, atol=1e-13)
