"""GPU parity of the single-pass backward (attn_bwd_ex with ATTN_BWD_ATOMIC_DQ) through the C ABI.

The dK/dV pass also adds every block's dQ contribution into an fp32 accumulator with hardware
atomics. Checked here: dQ, dK, dV against the fp64 oracle (max|g - g_ref| / max|g_ref| <= 5e-2)
for every mask kind, both head dims, GQA, ragged tails and empty rows; dQ, dK and dV within a few
bf16 units of the two-pass backward's. The two modes run different dK/dV kernels (the single pass
keeps one wave per 32 keys and all four products in it; the two-pass mode splits them over a pair
of waves that pass P to each other in bf16), so their sums differ in order and rounding.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_09_amd.inputs import WORKLOADS, Workload, make_inputs, workload_inputs
from tests.gpu_helpers import TOL_BF16_BWD_REL, device_inputs, lib_mask, libattn, oracle_mask, say, to_np64

pytestmark = pytest.mark.gpu


def _both(w: Workload, inp: dict):
    d = device_inputs(inp)
    m = lib_mask(w, d)
    o, lse = libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=inp["scale"])
    two = libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=inp["scale"])
    one = libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=inp["scale"],
                           flags=libattn.ATTN_BWD_ATOMIC_DQ)
    torch.cuda.synchronize()
    return two, one


def _rel_err(got, ref):
    denom = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / denom if denom > 0 else num


CASES = []
for d in (64, 128):
    for mask in ("none", "causal", "padding", "block"):
        for (b, hq, hkv, s) in ((2, 2, 1, 17), (1, 4, 2, 130), (2, 2, 2, 520)):
            CASES.append((d, mask, b, hq, hkv, s))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_atomic_bwd_parity(gpu_available, case):
    d, mask, b, hq, hkv, s = case
    w = Workload(f"bwd1_{case}", "bf16", b, hq, hkv, s, s, d, mask, backward=True,
                 len_range=(max(1, s // 4), s), keep_prob=0.3)
    seed = 51 + s + d
    say(f"single-pass bwd {case} seed {seed}")
    inp = make_inputs(w, seed)
    (dq2, dk2, dv2), (dq1, dk1, dv1) = _both(w, inp)
    ref = oracle.attention_bwd(to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"]), to_np64(inp["do"]),
                               oracle_mask(w, inp), inp["scale"])
    for name, got, r in zip(("dq", "dk", "dv"), (dq1, dk1, dv1), ref):
        g = to_np64(got)
        assert np.all(np.isfinite(g)), f"{case} {name}: non-finite"
        e = _rel_err(g, r)
        say(f"  {name}: rel max err {e:.3e}")
        assert e <= TOL_BF16_BWD_REL, f"{case} {name}: {e}"
    # same products, fp32 sums in another order, one bf16 rounding of each result: the two modes
    # agree to 1e-2 of the gradient's largest magnitude (each is within a few 1e-3 of the oracle)
    for name, a, b2 in (("dq", dq1, dq2), ("dk", dk1, dk2), ("dv", dv1, dv2)):
        e = float((a.float() - b2.float()).abs().max() / b2.float().abs().max().clamp_min(1e-30))
        assert e <= 1e-2, f"{case}: {name} differs from the two-pass backward by {e:.3e} of its max"


def test_atomic_bwd_empty_rows(gpu_available):
    w = Workload("bwd1_pad0", "bf16", 3, 2, 2, 150, 150, 64, "padding", backward=True)
    inp = make_inputs(w, 4)
    inp["lengths"] = torch.tensor([0, 1, 100], dtype=torch.int32)
    (_, _, _), (dq, dk, dv) = _both(w, inp)
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    assert torch.all(dq[2, :, 100:] == 0)


def test_atomic_bwd_workload_sampled_heads(gpu_available):
    """The block-sparse workload at full size: two (batch, head) pairs against the oracle."""
    cfg = 5
    w = WORKLOADS[cfg]
    inp = workload_inputs(cfg, with_do=True)
    (dq2, dk2, dv2), (dq1, dk1, dv1) = _both(w, inp)
    spec = oracle_mask(w, inp)
    q64, k64, v64, do64 = (to_np64(inp[x]) for x in ("q", "k", "v", "do"))
    for (b, h) in ((0, 0), (w.batch - 1, w.heads_q - 1)):
        ref = oracle.attention_bwd_head(q64, k64, v64, do64, spec, inp["scale"], b, h)
        for name, got, r in zip(("dq", "dk", "dv"), (dq1[b, h], dk1[b, h], dv1[b, h]), ref):
            e = _rel_err(to_np64(got), r)
            say(f"  cfg5 b{b} h{h} {name}: rel max err {e:.3e}")
            assert e <= TOL_BF16_BWD_REL
