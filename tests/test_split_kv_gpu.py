"""GPU parity of the split-KV forward (attn_fwd_ex) against the fp64 oracle, through the C ABI.

The key range of every (batch, head, query tile) item is shared by several workgroups whose
partial results a merge kernel combines; the result must match the oracle to the same tolerance
as the unsplit forward, for every mask kind, ragged tails, splits that see no key at all (early
causal tiles, padded rows), more splits than key tiles, and the automatic choice on shapes with
few items (few heads and long keys, and decode-like short query blocks).
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_09_amd import binding as libattn
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import TOL_BF16_FWD, compare_fwd, device_inputs, lib_mask, oracle_mask, say, to_np64

pytestmark = pytest.mark.gpu

CASES = []
for d in (64, 128):
    for mask in ("none", "causal", "padding", "block"):
        for (b, hq, hkv, s) in ((1, 2, 1, 600), (2, 2, 2, 1030)):
            for splits in (2, 3, 32):
                CASES.append((d, mask, b, hq, hkv, s, splits))


def _workload(d, mask, b, hq, hkv, sq, sk=None, scale=None):
    sk = sq if sk is None else sk
    return Workload(f"split_{d}_{mask}_{b}_{hq}_{hkv}_{sq}_{sk}", "bf16", b, hq, hkv, sq, sk, d, mask,
                    len_range=(max(1, sq // 4), sq), keep_prob=0.3, scale=scale)


def _run(w, seed, kv_splits, lengths=None):
    inp = make_inputs(w, seed)
    if lengths is not None:
        inp["lengths"] = torch.tensor(lengths, dtype=torch.int32)
    dev = device_inputs(inp)
    o, lse = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=lib_mask(w, dev), scale=inp["scale"],
                              kv_splits=kv_splits)
    torch.cuda.synchronize()
    return inp, dev, o, lse


def _check_full(w, inp, o, lse, label):
    o_ref, lse_ref = oracle.attention_fwd(to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"]),
                                          oracle_mask(w, inp), inp["scale"])
    compare_fwd(to_np64(o), to_np64(lse), o_ref, lse_ref, TOL_BF16_FWD, label)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_split_forced_parity(gpu_available, case):
    d, mask, b, hq, hkv, s, splits = case
    w = _workload(d, mask, b, hq, hkv, s)
    say(f"split-kv forced {case}")
    inp, dev, o, lse = _run(w, 300 + s + d + splits, splits)
    used = libattn.attn_fwd_kv_splits(dev["q"], dev["k"], lib_mask(w, dev), splits)
    assert used == min(splits, (s + 63) // 64)
    _check_full(w, inp, o, lse, str(case))


@pytest.mark.parametrize("d", (64, 128))
def test_split_matches_unsplit(gpu_available, d):
    """Split and unsplit forwards of the same inputs agree to bf16 rounding of O."""
    w = _workload(d, "causal", 1, 4, 2, 1500)
    _, dev, o1, l1 = _run(w, 41, 1)
    _, _, o8, l8 = _run(w, 41, 8)
    # both are one round-to-nearest of nearly equal fp32 values: at most one bf16 ulp apart
    diff = (o1.float() - o8.float()).abs()
    assert torch.all(diff <= 2 ** -7 * o1.float().abs().clamp(min=1.0))
    # the denominators sum bf16-rounded probabilities (each within 2^-9 relative of exact, so each
    # log-denominator is within 2^-9 of exact) against different reference maxima
    assert torch.allclose(l1, l8, atol=2 ** -8 + 1e-5, rtol=0)


def test_split_padding_empty_rows(gpu_available):
    """Lengths 0 and 1 with splits: rows no split sees give O = 0 exactly and LSE = -inf."""
    w = _workload(128, "padding", 3, 2, 2, 700)
    inp, _, o, lse = _run(w, 7, 4, lengths=[0, 1, 700])
    _check_full(w, inp, o, lse, "split padding 0/1")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_split_auto_few_heads_long_keys(gpu_available):
    """B1 H2 S8192 D128, no mask: 128 items, so the automatic choice splits; sampled rows."""
    w = _workload(128, "none", 1, 2, 2, 8192)
    inp, dev, o, lse = _run(w, 11, 0)
    used = libattn.attn_fwd_kv_splits(dev["q"], dev["k"], lib_mask(w, dev), 0)
    say(f"split-kv auto: {used} splits")
    assert used > 1
    q64, k64, v64 = to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"])
    rng = np.random.default_rng(3)
    for h in range(2):
        rows = np.unique(np.concatenate([np.arange(32), rng.integers(0, 8192, 96), np.arange(8192 - 32, 8192)]))
        o_ref, lse_ref = oracle.attention_rows(q64, k64, v64, oracle_mask(w, inp), inp["scale"], 0, h, rows)
        idx = torch.from_numpy(rows).to(o.device)
        compare_fwd(to_np64(o[0, h, idx]), to_np64(lse[0, h, idx]), o_ref, lse_ref, TOL_BF16_FWD, f"auto h{h}")


def test_split_auto_decode_like(gpu_available):
    """64 queries against 8192 keys (B2 Hq8 Hkv2 D128): 16 items; the automatic choice splits."""
    w = _workload(128, "none", 2, 8, 2, 64, sk=8192)
    inp, dev, o, lse = _run(w, 13, 0)
    used = libattn.attn_fwd_kv_splits(dev["q"], dev["k"], lib_mask(w, dev), 0)
    say(f"split-kv decode-like: {used} splits")
    assert used > 1
    _check_full(w, inp, o, lse, "decode-like")


def test_split_deterministic(gpu_available):
    w = _workload(128, "block", 1, 2, 1, 1030)
    _, _, o1, l1 = _run(w, 21, 5)
    _, _, o2, l2 = _run(w, 21, 5)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
