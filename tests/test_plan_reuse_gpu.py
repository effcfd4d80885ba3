"""GPU tests of planning the backward in the forward's planner launch (attn_fwd_with_bwd_plan,
then attn_bwd_ex with ATTN_BWD_PLANNED), through the C ABI.

The planned pair must give bit for bit the outputs of the plain pair: the forward's O and LSE, and
the backward's dQ, dK and dV. The lists are the same lists (the same planner on the same layout),
so any difference would mean a list was not written, written for another problem, or read from
the wrong place. Covered: every mask kind (for no mask and causal the forward has no list of its
own, so the backward's two lists get a launch of their own inside the forward call), a layout per
(batch, head), a dense mask (the forward plans on the block layout it derives from it), GQA, shapes
whose units spread over the XCDs, ragged tails, and two planned pairs in a row on one workspace.
"""

import pytest
import torch

from attention_attn_fwd_09_amd import binding as libattn
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import device_inputs, lib_mask, say

pytestmark = pytest.mark.gpu

SHAPES = ((2, 8, 4, 200, 128), (1, 16, 8, 333, 64), (2, 4, 2, 130, 64), (1, 2, 1, 70, 128))
CASES = [(mask, per_head, *shape) for mask in ("none", "causal", "padding", "block", "dense")
         for per_head in ((False, True) if mask in ("block", "dense") else (False,)) for shape in SHAPES]


def _pair(w, d, planned):
    m = lib_mask(w, d)
    ws = torch.empty(max(1, libattn.attn_bwd_workspace_bytes(d["q"], d["k"], m)), dtype=torch.uint8, device="cuda")
    if planned:
        o, lse = libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=d["scale"], bwd_plan=ws)
    else:
        o, lse = libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=d["scale"])
    grads = libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=d["scale"], workspace=ws,
                             planned=planned)
    torch.cuda.synchronize()
    return (o, lse, *grads)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_planned_pair_equals_plain_pair(gpu_available, case):
    mask, per_head, b, hq, hkv, s, dim = case
    w = Workload(f"plan_{case}", "bf16", b, hq, hkv, s, s, dim, mask, backward=True, len_range=(max(1, s // 4), s),
                 keep_prob=0.3, layout_per_head=per_head)
    seed = 1300 + s + dim
    say(f"planned pair {case} seed {seed}")
    d = device_inputs(make_inputs(w, seed))
    plain = _pair(w, d, planned=False)
    planned = _pair(w, d, planned=True)
    for name, a, p in zip(("o", "lse", "dq", "dk", "dv"), plain, planned):
        assert torch.equal(a, p), f"{case}: {name} differs between the planned and the plain pair"


def test_planned_pairs_in_a_row(gpu_available):
    """Two planned pairs of different problems on one workspace: each backward uses its own forward's lists."""
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    for i, (b, hq, hkv, s, dim, mask) in enumerate(((2, 8, 4, 300, 128, "block"), (1, 4, 2, 150, 64, "padding"))):
        w = Workload(f"plan_row_{i}", "bf16", b, hq, hkv, s, s, dim, mask, backward=True,
                     len_range=(max(1, s // 4), s), keep_prob=0.3)
        d = device_inputs(make_inputs(w, 1400 + i))
        say(f"planned pair in a row {i}: {w.name}")
        m = lib_mask(w, d)
        assert libattn.attn_bwd_workspace_bytes(d["q"], d["k"], m) <= ws.numel()
        plain = _pair(w, d, planned=False)
        o, lse = libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=d["scale"], bwd_plan=ws)
        grads = libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=d["scale"], workspace=ws,
                                 planned=True)
        torch.cuda.synchronize()
        for name, a, p in zip(("o", "lse", "dq", "dk", "dv"), plain, (o, lse, *grads)):
            assert torch.equal(a, p), f"pair {i}: {name} differs"
