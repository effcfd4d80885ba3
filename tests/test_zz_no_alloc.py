"""attn_bwd_noalloc: the backward that allocates nothing (its workspace is a fixed device array).

It runs the same kernels as attn_bwd, so its gradients must equal attn_bwd's bit for bit. Two
calls in a row, the second on a smaller problem, check that the array's leftover contents from
the first call do not leak into the second. A problem too large for the array is rejected on the
host with ATTN_ERR_TOO_LARGE (CPU test).
"""

import ctypes

import pytest
import torch

from attention_attn_fwd_09_amd import binding as libattn
from attention_attn_fwd_09_amd.inputs import Workload, make_inputs
from tests.gpu_helpers import device_inputs, fwd_into_nan, lib_mask, nan_filled, say


def _compare(w: Workload, seed: int):
    inp = make_inputs(w, seed)
    d = device_inputs(inp)
    m = lib_mask(w, d)
    o, lse = fwd_into_nan(w, inp)
    ref = libattn.attn_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, mask=m, scale=inp["scale"])
    got = tuple(nan_filled(t.shape, t.dtype) for t in (d["q"], d["k"], d["v"]))
    libattn.attn_bwd_noalloc(d["q"], d["k"], d["v"], o, d["do"], lse, *got, mask=m, scale=inp["scale"])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{w.name} {name}: attn_bwd_noalloc differs from attn_bwd"
    say(f"  {w.name}: attn_bwd_noalloc equals attn_bwd bit for bit")


@pytest.mark.gpu
def test_noalloc_backward_equals_attn_bwd_twice(gpu_available):
    """A large call, then a smaller one with another mask kind, on the same device array."""
    big = Workload("noalloc_big", "bf16", 2, 8, 4, 1500, 1500, 128, "block", backward=True, keep_prob=0.3)
    small = Workload("noalloc_small", "bf16", 1, 2, 2, 300, 300, 64, "padding", backward=True,
                     len_range=(100, 300))
    _compare(big, 61)
    _compare(small, 62)


@pytest.mark.gpu
def test_noalloc_backward_dense_and_causal(gpu_available):
    """The dense mask packs its bits into the array too; causal has no mask data at all."""
    _compare(Workload("noalloc_dense", "bf16", 1, 4, 2, 700, 700, 128, "dense", backward=True, keep_prob=0.5), 63)
    _compare(Workload("noalloc_causal", "bf16", 2, 4, 4, 257, 257, 64, "causal", backward=True), 64)


def test_noalloc_rejects_problems_beyond_the_array():
    """64 x 64 query heads of 2048 rows need 64 MiB of row statistics: more than the 32 MiB array.
    Rejected on the host (the pointers are never dereferenced)."""
    lib = libattn.load_library()
    assert lib.attn_bwd_noalloc_scratch_bytes() == 32 << 20
    p = libattn.AttnProblem()
    p.batch, p.heads_q, p.heads_kv, p.seq_q, p.seq_k, p.head_dim, p.dtype = 64, 64, 64, 2048, 2048, 128, 1
    assert lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), None, 0) > lib.attn_bwd_noalloc_scratch_bytes()
    m = libattn.Mask().to_c()
    ptrs = [(1 << 44) + i * (1 << 36) for i in range(10)]   # distinct, aligned, far apart
    st = lib.attn_bwd_noalloc(ctypes.byref(p), *ptrs[:6], ctypes.byref(m), 0.1, *ptrs[6:9], None)
    assert st == libattn.ATTN_ERR_TOO_LARGE
    assert "scratch" in libattn.attn_status_string(st)
    # a smaller problem passes every host check before the array is needed: a null pointer is still
    # reported first
    p.batch = 1
    st = lib.attn_bwd_noalloc(ctypes.byref(p), None, *ptrs[1:6], ctypes.byref(m), 0.1, *ptrs[6:9], None)
    assert st == libattn.ATTN_ERR_NULL
