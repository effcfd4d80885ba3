"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph on ROCm).

Every call launches its kernels on the caller's stream and, given its buffers, allocates nothing
and issues no memset or synchronisation, so a forward/backward pair can be captured once and
replayed. Each graph is replayed several times with eager work (the outputs refilled with NaN) and
a synchronisation between replays, and every replay must equal the eager result bit for bit.
"""

import pytest
import torch

from attention_attn_fwd_09_amd import binding as libattn
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import device_inputs, lib_mask, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _buffers(d):
    q, k, v = d["q"], d["k"], d["v"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return o, lse, torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)


def _capture_and_replay(run, outs, label):
    run()   # eager: the reference (and the first call's one-time set-up)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for i in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, want), f"{label}: replay {i} differs from the eager call in {name}"
    say(f"  {label}: {REPLAYS} replays equal the eager result bit for bit")


def test_graph_forward_and_noalloc_backward(gpu_available):
    """attn_fwd with a caller workspace, then attn_bwd_noalloc (its scratch is the library's
    fixed array): the callers the allocation-free entry point is for."""
    w = Workload("graph_noalloc", "bf16", 2, 4, 2, 600, 600, 128, "block", backward=True, keep_prob=0.3)
    inp = make_inputs(w, 81)
    d = device_inputs(inp)
    m = lib_mask(w, d)
    o, lse, dq, dk, dv = _buffers(d)
    ws = torch.empty(max(1, libattn.attn_fwd_workspace_bytes(d["q"], d["k"], m)), dtype=torch.uint8, device="cuda")

    def run():
        libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=inp["scale"], out=o, lse=lse, workspace=ws)
        libattn.attn_bwd_noalloc(d["q"], d["k"], d["v"], o, d["do"], lse, dq, dk, dv, mask=m, scale=inp["scale"])

    _capture_and_replay(run, (o, lse, dq, dk, dv), "fwd + bwd_noalloc")


@pytest.mark.parametrize("mask", ("block", "causal"))
def test_graph_planned_pair(gpu_available, mask):
    """The benchmark's step: attn_fwd whose planner launch also plans the backward, then
    attn_bwd on that workspace with ATTN_BWD_PLANNED."""
    w = Workload(f"graph_pair_{mask}", "bf16", 1, 4, 2, 1000, 1000, 64, mask, backward=True, keep_prob=0.3)
    inp = make_inputs(w, 82)
    d = device_inputs(inp)
    m = lib_mask(w, d)
    o, lse, dq, dk, dv = _buffers(d)
    ws_f = torch.empty(max(1, libattn.attn_fwd_workspace_bytes(d["q"], d["k"], m)), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(1, libattn.attn_bwd_workspace_bytes(d["q"], d["k"], m)), dtype=torch.uint8, device="cuda")

    def run():
        libattn.attn_fwd(d["q"], d["k"], d["v"], mask=m, scale=inp["scale"], out=o, lse=lse, workspace=ws_f,
                         bwd_plan=ws_b)
        libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=inp["scale"], dq=dq, dk=dk, dv=dv,
                         workspace=ws_b, planned=True)

    _capture_and_replay(run, (o, lse, dq, dk, dv), f"planned pair ({mask})")
