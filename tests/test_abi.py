"""CPU tests of the C ABI: the library loads, exports every function include/attn.h declares, and
rejects invalid calls on the host before any GPU call.

No call here passes validation: the pointers are fake (never dereferenced), so a call that got as
far as a launch would be a bug in the checks. Every call is expected to return an error status.
"""

import ctypes
import os
import re

import pytest

from attention_attn_fwd_09_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _lib():
    if not os.path.exists(B._LIB_PATH):
        pytest.skip("libattn.so not built (run __graft_entry__.build())")
    lib = B.load_library()
    lib.attn_set_timing_events.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_int32)]
    lib.attn_set_timing_events.restype = ctypes.c_int
    return lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("attn_fwd", "attn_bwd", "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes", "attn_status_string",
              "attn_version", "attn_set_timing_events", "attn_fwd_ex", "attn_fwd_ex_workspace_bytes",
              "attn_fwd_kv_splits"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), f"libattn.so does not export {name}"
    # the exported dynamic symbols carry C linkage (no C++ mangling)
    out = os.popen(f"nm -D --defined-only {B._LIB_PATH}").read()
    for name in _declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), f"{name} is not an exported C symbol"


def test_status_strings():
    lib = _lib()
    for code in range(11):
        s = lib.attn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.attn_status_string(99).decode() == "unknown status"
    assert lib.attn_version() >= 100


def _problem(b=1, hq=2, hkv=2, sq=64, sk=64, d=64, dtype=B.ATTN_BF16):
    p = B.AttnProblem()
    p.batch, p.heads_q, p.heads_kv, p.seq_q, p.seq_k, p.head_dim, p.dtype = b, hq, hkv, sq, sk, d, dtype
    return p


def _mask(kind=0, lengths=None, layout=None, bq=64, bk=64, sb=0, sh=0):
    m = B.AttnMask()
    m.kind, m.lengths, m.block_layout, m.block_q, m.block_k = kind, lengths, layout, bq, bk
    m.layout_stride_b, m.layout_stride_h = sb, sh
    return m


def _fwd(lib, p, m, scale=0.125, q=FAKE, k=FAKE * 2, v=FAKE * 3, o=FAKE * 4, lse=FAKE * 5, ws=None, ws_bytes=0):
    return lib.attn_fwd(ctypes.byref(p), q, k, v, ctypes.byref(m) if m is not None else None, scale, o, lse, ws,
                        ws_bytes, None)


def _spaced(n):
    """n distinct fake pointers far enough apart that no ranges overlap (1 TiB spacing)."""
    return [FAKE + (i + 1) * (1 << 40) for i in range(n)]


def _fwd_ok_ptrs():
    q, k, v, o, lse, ws = _spaced(6)
    return dict(q=q, k=k, v=v, o=o, lse=lse, ws=ws)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, B.ATTN_ERR_SHAPE), ("heads_q", 0, B.ATTN_ERR_SHAPE), ("heads_kv", 0, B.ATTN_ERR_SHAPE),
    ("seq_q", 0, B.ATTN_ERR_SHAPE), ("seq_k", -1, B.ATTN_ERR_SHAPE), ("heads_kv", 3, B.ATTN_ERR_SHAPE),
    ("dtype", 7, B.ATTN_ERR_DTYPE), ("dtype", 3, B.ATTN_ERR_DTYPE), ("head_dim", 96, B.ATTN_ERR_UNSUPPORTED), ("head_dim", 256, B.ATTN_ERR_UNSUPPORTED),
    ("seq_q", 1 << 24, B.ATTN_ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_problem(field, value, status):
    lib = _lib()
    p = _problem()
    setattr(p, field, value)
    ptr = _fwd_ok_ptrs()
    assert _fwd(lib, p, _mask(), q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"]) == status


def test_fwd_rejects_null_pointers():
    lib = _lib()
    p, m = _problem(), _mask()
    ptr = _fwd_ok_ptrs()
    for name in ("q", "k", "v", "o", "lse"):
        args = dict(q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"])
        args[name] = None
        assert _fwd(lib, p, m, **args) == B.ATTN_ERR_NULL
    assert lib.attn_fwd(None, ptr["q"], ptr["k"], ptr["v"], None, 0.1, ptr["o"], ptr["lse"], None, 0, None) == B.ATTN_ERR_NULL


def test_fwd_rejects_bad_scale_and_masks():
    lib = _lib()
    ptr = _fwd_ok_ptrs()
    kw = dict(q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"])
    assert _fwd(lib, _problem(), _mask(), scale=float("nan"), **kw) == B.ATTN_ERR_SHAPE
    assert _fwd(lib, _problem(), _mask(), scale=-1.0, **kw) == B.ATTN_ERR_SHAPE
    assert _fwd(lib, _problem(), _mask(), scale=float("inf"), **kw) == B.ATTN_ERR_SHAPE
    assert _fwd(lib, _problem(), _mask(kind=9), **kw) == B.ATTN_ERR_MASK
    assert _fwd(lib, _problem(sq=64, sk=65), _mask(kind=1), **kw) == B.ATTN_ERR_SHAPE   # causal needs square
    assert _fwd(lib, _problem(), _mask(kind=2), **kw) == B.ATTN_ERR_MASK               # padding without lengths
    assert _fwd(lib, _problem(), _mask(kind=3), **kw) == B.ATTN_ERR_MASK               # block without layout
    assert _fwd(lib, _problem(), _mask(kind=3, layout=FAKE, bq=32), **kw) == B.ATTN_ERR_MASK
    assert _fwd(lib, _problem(), _mask(kind=3, layout=FAKE, sb=-1), **kw) == B.ATTN_ERR_MASK
    assert _fwd(lib, _problem(sq=70000, sk=70000), _mask(kind=3, layout=FAKE), **kw) == B.ATTN_ERR_UNSUPPORTED


def test_fwd_rejects_misaligned_and_missing_workspace():
    lib = _lib()
    ptr = _fwd_ok_ptrs()
    kw = dict(q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"])
    bad = dict(kw, q=ptr["q"] + 2)
    assert _fwd(lib, _problem(), _mask(), **bad) == B.ATTN_ERR_ALIGN
    # padding forward needs the planner's workspace
    p, m = _problem(), _mask(kind=2, lengths=FAKE)
    need = lib.attn_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
    assert need > 0
    assert _fwd(lib, p, m, **kw) == B.ATTN_ERR_WORKSPACE
    assert _fwd(lib, p, m, ws=ptr["ws"], ws_bytes=need - 1, **kw) == B.ATTN_ERR_WORKSPACE
    assert _fwd(lib, p, m, ws=ptr["ws"] + 4, ws_bytes=need, **kw) == B.ATTN_ERR_ALIGN
    # no-mask and causal bf16 forwards and every fp32 forward need none
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(_problem()), ctypes.byref(_mask())) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(_problem()), ctypes.byref(_mask(kind=1))) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(_problem(dtype=B.ATTN_F32)), ctypes.byref(m)) == 0
    # an invalid problem has no workspace size
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(_problem(b=0)), ctypes.byref(_mask())) == 0


def test_fwd_rejects_aliasing_outputs():
    lib = _lib()
    p = _problem(b=1, hq=2, sq=64, d=64)
    nbytes = 1 * 2 * 64 * 64 * 2
    q, k, v = _spaced(3)
    assert _fwd(lib, p, _mask(), q=q, k=k, v=v, o=q + 16, lse=_spaced(5)[4]) == B.ATTN_ERR_ALIAS
    assert _fwd(lib, p, _mask(), q=q, k=k, v=v, o=_spaced(4)[3], lse=v + nbytes - 16) == B.ATTN_ERR_ALIAS
    o = _spaced(4)[3]
    assert _fwd(lib, p, _mask(), q=q, k=k, v=v, o=o, lse=o + 64) == B.ATTN_ERR_ALIAS


def test_bwd_rejections():
    lib = _lib()
    q, k, v, o, do, lse, dq, dk, dv, ws = _spaced(10)
    p, m = _problem(), _mask()

    def call(pp=p, mm=m, scale=0.1, **over):
        a = dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws, wsb=1 << 30)
        a.update(over)
        return lib.attn_bwd(ctypes.byref(pp), a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], ctypes.byref(mm),
                            scale, a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)

    assert call(do=None) == B.ATTN_ERR_NULL
    assert call(pp=_problem(dtype=B.ATTN_F32)) == B.ATTN_ERR_UNSUPPORTED
    assert call(dk=dk + 8) == B.ATTN_ERR_ALIGN
    assert call(ws=None) == B.ATTN_ERR_WORKSPACE
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
    assert need > 0
    assert call(wsb=need - 1) == B.ATTN_ERR_WORKSPACE
    assert call(dq=q) == B.ATTN_ERR_ALIAS
    assert call(dv=dk) == B.ATTN_ERR_ALIAS
    assert call(ws=dq) == B.ATTN_ERR_ALIAS
    assert call(scale=-0.5) == B.ATTN_ERR_SHAPE
    big = _problem(hq=128, hkv=1, sq=8192, sk=8192, d=128)
    assert call(pp=big, mm=_mask(kind=3, layout=FAKE)) == B.ATTN_ERR_UNSUPPORTED   # group too large for the step list


def test_timing_hook_argument_checks():
    lib = _lib()
    assert lib.attn_set_timing_events(-1, None, None, 0, None) == B.ATTN_ERR_SHAPE
    n_classes = int(re.search(r"ATTN_KERNEL_CLASSES\s*=\s*(\d+)", open(HEADER).read()).group(1))
    assert lib.attn_set_timing_events(n_classes, None, None, 0, None) == B.ATTN_ERR_SHAPE
    assert lib.attn_set_timing_events(n_classes - 1, None, None, 0, None) == B.ATTN_OK
    arr = (ctypes.c_void_p * 1)()
    assert lib.attn_set_timing_events(1, arr, arr, 1, None) == B.ATTN_ERR_NULL
    assert lib.attn_set_timing_events(1, None, None, 0, None) == B.ATTN_OK


def test_python_binding_rejects_noncontiguous_and_mixed_dtypes():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.attn_fwd(q.transpose(1, 2), q, q)
    with pytest.raises(TypeError):
        B.attn_fwd(q.to(torch.float16), q, q)


def test_split_kv_arguments_and_choice():
    lib = _lib()
    ptr = _fwd_ok_ptrs()

    def fwd_ex(p, m, splits, ws=None, wsb=0):
        return lib.attn_fwd_ex(ctypes.byref(p), ptr["q"], ptr["k"], ptr["v"], ctypes.byref(m), 0.1, ptr["o"],
                               ptr["lse"], ws, wsb, splits, None)

    small = _problem(b=1, hq=2, hkv=1, sq=8192, sk=8192, d=128)
    m = _mask()
    assert fwd_ex(small, m, -1) == B.ATTN_ERR_SHAPE
    assert fwd_ex(small, m, 33) == B.ATTN_ERR_SHAPE
    assert fwd_ex(_problem(dtype=B.ATTN_F32), m, 2) == B.ATTN_ERR_UNSUPPORTED
    # 128 items of 128 queries leave most workgroup slots idle: split, 8+ key tiles each
    auto = lib.attn_fwd_kv_splits(ctypes.byref(small), ctypes.byref(m), 0)
    assert 2 <= auto <= 32 and 128 // auto >= 8
    assert lib.attn_fwd_kv_splits(ctypes.byref(small), ctypes.byref(m), 1) == 1
    assert lib.attn_fwd_kv_splits(ctypes.byref(small), ctypes.byref(m), 7) == 7
    # forced splits are capped at one per 64-key tile
    short = _problem(b=1, hq=2, hkv=1, sq=150, sk=150, d=64)
    assert lib.attn_fwd_kv_splits(ctypes.byref(short), ctypes.byref(m), 32) == 3
    # many items: no split; fp32 never splits
    big = _problem(b=4, hq=32, hkv=32, sq=4096, sk=4096, d=128)
    assert lib.attn_fwd_kv_splits(ctypes.byref(big), ctypes.byref(m), 0) == 1
    assert lib.attn_fwd_kv_splits(ctypes.byref(_problem(dtype=B.ATTN_F32)), ctypes.byref(m), 0) == 1
    # the partial results live in the workspace: rows * (D + 1) fp32 per split
    rows = 1 * 2 * 8192
    need = lib.attn_fwd_ex_workspace_bytes(ctypes.byref(small), ctypes.byref(m), 4)
    assert need >= 4 * rows * (128 + 1) * 4
    assert lib.attn_fwd_ex_workspace_bytes(ctypes.byref(small), ctypes.byref(m), 1) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(small), ctypes.byref(m)) == \
        lib.attn_fwd_ex_workspace_bytes(ctypes.byref(small), ctypes.byref(m), 0)
    assert fwd_ex(small, m, 4) == B.ATTN_ERR_WORKSPACE
    assert fwd_ex(small, m, 4, ws=ptr["ws"], wsb=need - 1) == B.ATTN_ERR_WORKSPACE


def test_single_pass_backward_arguments():
    lib = _lib()
    q, k, v, o, do, lse, dq, dk, dv, ws = _spaced(10)
    p, m = _problem(b=2, hq=4, hkv=2, sq=300, sk=300, d=128), _mask()
    two = lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), ctypes.byref(m), 0)
    one = lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), ctypes.byref(m), B.ATTN_BWD_ATOMIC_DQ)
    assert two == lib.attn_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
    # the single pass keeps an fp32 [B, Hq, Sq, D] dQ accumulator instead of the dQ item list
    assert one >= 2 * 4 * 300 * 128 * 4
    assert lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), ctypes.byref(m), 4) == 0
    # the planned backward uses the two-pass layout; it does not combine with the single pass
    assert lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), ctypes.byref(m), B.ATTN_BWD_PLANNED) == two
    assert lib.attn_bwd_ex_workspace_bytes(ctypes.byref(p), ctypes.byref(m),
                                           B.ATTN_BWD_PLANNED | B.ATTN_BWD_ATOMIC_DQ) == 0

    def call(flags, wsb):
        return lib.attn_bwd_ex(ctypes.byref(p), q, k, v, o, do, lse, ctypes.byref(m), 0.1, dq, dk, dv, ws, wsb,
                               flags, None)

    assert call(4, 1 << 40) == B.ATTN_ERR_SHAPE
    assert call(-1, 1 << 40) == B.ATTN_ERR_SHAPE
    assert call(B.ATTN_BWD_ATOMIC_DQ, one - 1) == B.ATTN_ERR_WORKSPACE
    assert call(B.ATTN_BWD_ATOMIC_DQ, two) == B.ATTN_ERR_WORKSPACE
    assert call(B.ATTN_BWD_PLANNED | B.ATTN_BWD_ATOMIC_DQ, 1 << 40) == B.ATTN_ERR_UNSUPPORTED
    assert call(B.ATTN_BWD_PLANNED, two - 1) == B.ATTN_ERR_WORKSPACE


def test_row_pairing_workspace():
    """A block layout shared by every (batch, head), of at most 64 rows and 64 key tiles, gets a
    row-pairs region (4 bytes per 128-row query tile, 256-byte aligned) in the bf16 forward's and
    the two-pass backward's workspaces; per-head layouts, more rows or other dtypes do not."""
    lib = _lib()
    layout = _spaced(1)[0]

    def sizes(sq, sk, dtype=B.ATTN_BF16, per_head=False):
        p = _problem(b=2, hq=4, hkv=2, sq=sq, sk=sk, d=128, dtype=dtype)
        nbq, nbk = -(-sq // 64), -(-sk // 64)
        m = _mask(kind=3, layout=layout, sb=4 * nbq * nbk if per_head else 0, sh=nbq * nbk if per_head else 0)
        fwd = lib.attn_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
        bwd = lib.attn_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m)) if dtype == B.ATTN_BF16 else 0
        return fwd, bwd

    for sq, sk in ((4096, 4096), (4022, 4022), (150, 4096), (4096, 300)):
        shared, per_head = sizes(sq, sk), sizes(sq, sk, per_head=True)
        assert shared[0] - per_head[0] == 256 and shared[1] - per_head[1] == 256, (sq, sk)
    for sq, sk in ((4100, 4096), (4096, 4160)):   # 65 rows; 65 key tiles per row
        assert sizes(sq, sk) == sizes(sq, sk, per_head=True), (sq, sk)
    for dtype in (B.ATTN_F32, B.ATTN_FP8_E4M3):
        assert sizes(4096, 4096, dtype)[0] == sizes(4096, 4096, dtype, per_head=True)[0]


def _fwd_plan(lib, p, m, bws, bws_bytes, ptrs=None):
    ptrs = ptrs or _fwd_ok_ptrs()
    return lib.attn_fwd_with_bwd_plan(ctypes.byref(p), ptrs["q"], ptrs["k"], ptrs["v"], ctypes.byref(m), 0.125,
                                      ptrs["o"], ptrs["lse"], ptrs["ws"], 1 << 40, bws, bws_bytes, None)


def test_forward_with_backward_plan_arguments():
    """Host-side rejections of attn_fwd_with_bwd_plan (nothing is launched)."""
    lib = _lib()
    p, m = _problem(b=2, hq=4, hkv=2, sq=300, sk=300, d=128), _mask()
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
    bws = _spaced(8)[7]
    assert _fwd_plan(lib, p, m, None, need) == B.ATTN_ERR_NULL
    assert _fwd_plan(lib, p, m, bws, need - 1) == B.ATTN_ERR_WORKSPACE
    assert _fwd_plan(lib, p, m, bws + 8, need) == B.ATTN_ERR_ALIGN
    ptrs = _fwd_ok_ptrs()
    assert _fwd_plan(lib, p, m, ptrs["q"] + 256, need, ptrs) == B.ATTN_ERR_ALIAS      # inside Q
    # a block mask: the forward has a workspace (its own list) and the layout is mask data
    layout = _spaced(9)[8]
    mb = _mask(kind=3, layout=layout)
    need_b = lib.attn_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(mb))
    assert _fwd_plan(lib, p, mb, ptrs["ws"], need_b, ptrs) == B.ATTN_ERR_ALIAS       # the forward's workspace
    assert _fwd_plan(lib, p, mb, layout, need_b, ptrs) == B.ATTN_ERR_ALIAS           # the layout
    # problems the backward does not support: F32 and FP8 inputs
    for dtype in (B.ATTN_F32, B.ATTN_FP8_E4M3):
        pf = _problem(b=2, hq=4, hkv=2, sq=300, sk=300, d=128, dtype=dtype)
        assert _fwd_plan(lib, pf, m, bws, 1 << 40) == B.ATTN_ERR_UNSUPPORTED
    # the forward's own checks still come first
    assert _fwd_plan(lib, _problem(hkv=3), m, bws, 1 << 40) == B.ATTN_ERR_SHAPE


def test_dense_mask_arguments():
    lib = _lib()
    ptr = _fwd_ok_ptrs()
    kw = dict(q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"])
    m = _mask(kind=4)
    assert _fwd(lib, _problem(), m, **kw) == B.ATTN_ERR_MASK                 # no dense pointer
    m.dense = _spaced(7)[6]
    m.dense_stride_b = -1
    assert _fwd(lib, _problem(), m, **kw) == B.ATTN_ERR_MASK                 # negative stride
    m.dense_stride_b = 0
    # rectangular problems are fine for a dense mask; the bf16 forward packs it in the workspace
    p = _problem(sq=100, sk=300)
    need = lib.attn_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(m))
    assert need >= 100 * ((300 + 31) // 32) * 4 + 2 * 5
    assert _fwd(lib, p, m, **kw) == B.ATTN_ERR_WORKSPACE
    # the fp32 forward reads the bytes directly and needs no workspace
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(_problem(dtype=B.ATTN_F32)), ctypes.byref(m)) == 0
    # the mask is an input: an output overlapping it is rejected
    m.dense = ptr["o"] + 64
    assert _fwd(lib, p, m, ws=ptr["ws"], ws_bytes=need, **kw) == B.ATTN_ERR_ALIAS


def test_fp8_inputs_arguments():
    lib = _lib()
    ptr = _fwd_ok_ptrs()
    kw = dict(q=ptr["q"], k=ptr["k"], v=ptr["v"], o=ptr["o"], lse=ptr["lse"])
    p8 = _problem(dtype=B.ATTN_FP8_E4M3, sq=64, sk=64, d=128)
    # accepted by the forward (workspace only for masks that plan); the output is bf16-sized
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(p8), ctypes.byref(_mask())) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(p8), ctypes.byref(_mask(kind=3, layout=FAKE))) > 0
    # O of 2 x 64 x 128 bf16 = 32 KiB: an O placed 16 KiB below Q overlaps it, although an fp8-sized O would not
    q = ptr["q"]
    assert _fwd(lib, p8, _mask(), q=q, k=kw["k"], v=kw["v"], o=q - 16384, lse=kw["lse"]) == B.ATTN_ERR_ALIAS
    # split-KV accepts fp8; the backward does not
    assert lib.attn_fwd_kv_splits(ctypes.byref(p8), ctypes.byref(_mask()), 2) == 1   # one 64-key tile
    p8_long = _problem(dtype=B.ATTN_FP8_E4M3, sq=64, sk=4096, d=128)
    assert lib.attn_fwd_kv_splits(ctypes.byref(p8_long), ctypes.byref(_mask()), 4) == 4
    qq, k, v, o, do, lse, dq, dk, dv, ws = _spaced(10)
    assert lib.attn_bwd(ctypes.byref(p8), qq, k, v, o, do, lse, ctypes.byref(_mask()), 0.1, dq, dk, dv, ws, 1 << 30,
                        None) == B.ATTN_ERR_UNSUPPORTED
    assert _fwd(lib, _problem(dtype=3), _mask(), **kw) == B.ATTN_ERR_DTYPE
