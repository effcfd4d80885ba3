"""Forward and backward parity on seeded random shapes, against the fp64 oracle, through the C ABI.

Each case draws a mask kind (none, causal, padding, block layouts shared or per head, dense), a
head_dim, batch, key/value heads and group size, and query and key lengths from 1 to 1400 (equal
for causal), so ragged tails, single rows, rectangular problems and grouped-query attention mix in
ways the hand-picked shapes do not. Outputs are written into NaN-filled buffers. The bf16 cases run
forward and backward at the bf16 tolerances; the fp8 (e4m3) forward cases, with a random split-KV
count, are held to the bound derived from rounding the probabilities to e4m3; the fp32 forward
cases to the fp32 tolerance.
"""

import random

import pytest

import oracle
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import (TOL_BF16_FWD, TOL_F32, bwd_into_nan, check_grads, compare_fwd, fwd_into_nan,
                               oracle_mask, say, to_np64)
from tests.test_fp8_gpu import _check as check_fp8

pytestmark = pytest.mark.gpu


def _cases(seed=2024, n=24, smax=1400):
    """(index, mask, head_dim, batch, heads_q, heads_kv, seq_q, seq_k, per-head layout, keep probability)"""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        mask = rng.choice(["none", "causal", "padding", "block", "block", "dense"])
        d = rng.choice([64, 128])
        hkv, g, b = rng.choice([1, 2, 3]), rng.choice([1, 2, 4]), rng.choice([1, 2, 3])
        sq = rng.randint(1, smax)
        sk = sq if mask == "causal" else rng.randint(1, smax)
        per_head = mask in ("block", "dense") and rng.random() < 0.3
        keep = rng.choice([0.1, 0.3, 0.6])
        out.append((i, mask, d, b, hkv * g, hkv, sq, sk, per_head, keep))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(map(str, c)))
def test_random_shape_fwd_bwd(gpu_available, case):
    i, mask, d, b, hq, hkv, sq, sk, per_head, keep = case
    w = Workload(f"rand{i}", "bf16", b, hq, hkv, sq, sk, d, mask, backward=True,
                 len_range=(max(1, min(sq, sk) // 4), min(sq, sk)), keep_prob=keep, layout_per_head=per_head)
    say(f"random shape {case}")
    inp = make_inputs(w, 6000 + i)
    o, lse = fwd_into_nan(w, inp)
    q, k, v = to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"])
    om = oracle_mask(w, inp)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, om, inp["scale"])
    compare_fwd(to_np64(o), to_np64(lse), o_ref, lse_ref, TOL_BF16_FWD, str(case))
    grads = bwd_into_nan(w, inp, o, lse)
    ref = oracle.attention_bwd(q, k, v, to_np64(inp["do"]), om, inp["scale"])
    check_grads(tuple(to_np64(x) for x in grads), ref, str(case))


@pytest.mark.parametrize("case", _cases(seed=77, n=12, smax=900), ids=lambda c: "-".join(map(str, c)))
def test_random_shape_fp8_fwd(gpu_available, case):
    i, mask, d, b, hq, hkv, sq, sk, per_head, keep = case
    splits = random.Random(i).choice([0, 1, 3])
    w = Workload(f"rand8_{i}", "fp8", b, hq, hkv, sq, sk, d, mask,
                 len_range=(max(1, min(sq, sk) // 4), min(sq, sk)), keep_prob=keep, layout_per_head=per_head)
    say(f"random fp8 shape {case} kv_splits {splits}")
    inp = make_inputs(w, 7000 + i)
    o, lse = fwd_into_nan(w, inp, kv_splits=splits)
    check_fp8(w, inp, o, lse, f"{case} splits {splits}")


@pytest.mark.parametrize("case", _cases(seed=99, n=12, smax=1400), ids=lambda c: "-".join(map(str, c)))
def test_random_shape_f32_fwd(gpu_available, case):
    i, mask, d, b, hq, hkv, sq, sk, per_head, keep = case
    w = Workload(f"rand32_{i}", "f32", b, hq, hkv, sq, sk, d, mask,
                 len_range=(max(1, min(sq, sk) // 4), min(sq, sk)), keep_prob=keep, layout_per_head=per_head)
    say(f"random fp32 shape {case}")
    inp = make_inputs(w, 8000 + i)
    o, lse = fwd_into_nan(w, inp)
    q, k, v = to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"])
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, oracle_mask(w, inp), inp["scale"])
    compare_fwd(to_np64(o), to_np64(lse), o_ref, lse_ref, TOL_F32, str(case))
