"""GPU parity of the dense element mask (mask[i][j], 0 = hidden) through the C ABI.

Forward (bf16 and fp32, with and without split-KV) and backward (two-pass and single-pass) are
compared with the fp64 oracle on masks that hide single pairs, whole 64x64 blocks and whole
rows, shared by every (batch, head) or one per (batch, head), on square and rectangular shapes
with ragged tails. A dense mask holding the causal pattern must reproduce the causal forward bit
for bit (same tiles, same order, same arithmetic) and its gradients up to summation order.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_fwd_09_amd import binding as libattn
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import (TOL_BF16_BWD_REL, TOL_BF16_FWD, TOL_F32, compare_fwd, device_inputs, lib_mask,
                               oracle_mask, say, to_np64)

pytestmark = pytest.mark.gpu


def _w(dtype, d, b, hq, hkv, sq, sk, per_head, keep=0.5):
    return Workload(f"dense_{dtype}_{d}_{b}_{hq}_{hkv}_{sq}_{sk}_{int(per_head)}", dtype, b, hq, hkv, sq, sk, d,
                    "dense", backward=True, keep_prob=keep, layout_per_head=per_head)


FWD = []
for dtype in ("bf16", "f32"):
    for d in (64, 128):
        for (b, hq, hkv, sq, sk, per_head) in ((1, 2, 1, 130, 130, False), (2, 2, 2, 300, 77, True),
                                               (1, 4, 2, 520, 1030, False)):
            FWD.append((dtype, d, b, hq, hkv, sq, sk, per_head))


def _inputs(w, seed, empty_row=True):
    inp = make_inputs(w, seed)
    if empty_row:
        # one query row that sees nothing, in every (b, h)
        inp["dense"][..., w.seq_q // 2, :] = 0
    return inp


@pytest.mark.parametrize("case", FWD, ids=lambda c: "-".join(map(str, c)))
def test_dense_fwd_parity(gpu_available, case):
    w = _w(*case)
    say(f"dense fwd {case}")
    inp = _inputs(w, 600 + case[4] + case[1])
    dev = device_inputs(inp)
    o, lse = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=lib_mask(w, dev), scale=inp["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"]),
                                          oracle_mask(w, inp), inp["scale"])
    compare_fwd(to_np64(o), to_np64(lse), o_ref, lse_ref, TOL_F32 if w.dtype == "f32" else TOL_BF16_FWD, str(case))


@pytest.mark.parametrize("splits", (2, 5))
def test_dense_fwd_split_kv(gpu_available, splits):
    w = _w("bf16", 128, 1, 2, 1, 300, 1100, True)
    inp = _inputs(w, 77)
    dev = device_inputs(inp)
    o, lse = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=lib_mask(w, dev), scale=inp["scale"],
                              kv_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"]),
                                          oracle_mask(w, inp), inp["scale"])
    compare_fwd(to_np64(o), to_np64(lse), o_ref, lse_ref, TOL_BF16_FWD, f"dense split {splits}")


BWD = []
for d in (64, 128):
    for (b, hq, hkv, s, per_head) in ((1, 2, 1, 130, False), (2, 2, 2, 257, True), (1, 4, 2, 520, False)):
        for flags in (0, libattn.ATTN_BWD_ATOMIC_DQ):
            BWD.append((d, b, hq, hkv, s, per_head, flags))


def _rel(got, ref):
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 0 else num


@pytest.mark.parametrize("case", BWD, ids=lambda c: "-".join(map(str, c)))
def test_dense_bwd_parity(gpu_available, case):
    d, b, hq, hkv, s, per_head, flags = case
    w = _w("bf16", d, b, hq, hkv, s, s, per_head)
    say(f"dense bwd {case}")
    inp = _inputs(w, 700 + s + d)
    dev = device_inputs(inp)
    m = lib_mask(w, dev)
    o, lse = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=m, scale=inp["scale"])
    dq, dk, dv = libattn.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, mask=m, scale=inp["scale"],
                                  flags=flags)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(to_np64(inp["q"]), to_np64(inp["k"]), to_np64(inp["v"]), to_np64(inp["do"]),
                               oracle_mask(w, inp), inp["scale"])
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = _rel(to_np64(got), r)
        say(f"  {name}: rel max err {e:.3e}")
        assert np.all(np.isfinite(to_np64(got))) and e <= TOL_BF16_BWD_REL, f"{case} {name}: {e}"
    # the row that sees nothing has zero dQ
    assert torch.all(dq[:, :, s // 2] == 0)


@pytest.mark.parametrize("d", (64, 128))
def test_dense_causal_pattern_matches_causal_kernels(gpu_available, d):
    s = 600
    wc = Workload("c", "bf16", 2, 4, 2, s, s, d, "causal", backward=True)
    inp = make_inputs(wc, 91)
    dev = device_inputs(inp)
    tri = torch.tril(torch.ones(s, s, dtype=torch.uint8)).cuda()
    mc = libattn.Mask(kind="causal")
    md = libattn.Mask(kind="dense", dense=tri)
    oc, lc = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=mc, scale=inp["scale"])
    od, ld = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=md, scale=inp["scale"])
    gc = libattn.attn_bwd(dev["q"], dev["k"], dev["v"], oc, dev["do"], lc, mask=mc, scale=inp["scale"])
    gd = libattn.attn_bwd(dev["q"], dev["k"], dev["v"], oc, dev["do"], lc, mask=md, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(oc, od) and torch.equal(lc, ld)
    # the backward passes visit the same blocks but in another order (the causal dK/dV pass runs
    # 128-key workgroups and its mask-free query tiles first): equal up to fp32 summation order
    for a, bb in zip(gc, gd):
        a, bb = a.float(), bb.float()
        assert torch.all((a - bb).abs() <= 2 ** -6 * a.abs() + 1e-3 * a.abs().max())


def test_dense_all_hidden(gpu_available):
    """A mask that hides everything: O = 0, LSE = -inf, zero gradients."""
    w = _w("bf16", 128, 1, 2, 2, 200, 200, False)
    inp = make_inputs(w, 5)
    inp["dense"].zero_()
    dev = device_inputs(inp)
    m = lib_mask(w, dev)
    o, lse = libattn.attn_fwd(dev["q"], dev["k"], dev["v"], mask=m, scale=inp["scale"])
    dq, dk, dv = libattn.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, mask=m, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)
