"""Checks that pin the fp64 oracle to facts outside itself.

Each check takes a module exposing ``MaskSpec``, ``attention_fwd`` and
``attention_bwd`` (the oracle, or a deliberately broken copy of it) and raises
AssertionError when the module disagrees with:

* a library routine: torch's scaled_dot_product_attention and autograd, run on
  the CPU in float64 (an independent implementation of the same definition);
* closed forms of the definition (page 2, zwxr.cn, section 3.1): Q = 0, one
  key, constant V, the first causal row, a shift of every key;
* invariants: probabilities that sum to one, joint permutation of keys and
  values, sum over keys of dK is zero, sum of dV equals the sum of dO;
* reductions to simpler problems: padding equals truncation, grouped-query
  equals repeated heads, an all-ones block layout equals no mask, an identity
  block layout equals independent attention on every block;
* central finite differences of L = sum(dO * O) on tiny shapes;
* the hand-derived fixture tests/golden/two_keys.json.

The masks used for comparison are rebuilt here with torch ops, independently
of the oracle's own mask builder.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, b, hq, hkv, sq, sk, d, dv=None):
    r = _rng(seed)
    dv = d if dv is None else dv
    return (r.standard_normal((b, hq, sq, d)), r.standard_normal((b, hkv, sk, d)),
            r.standard_normal((b, hkv, sk, dv)))


def _torch_mask(kind, b, hq, sq, sk, lengths=None, layout=None, bq=64, bk=64, dense=None):
    """[b, hq, sq, sk] bool (True = attend), built with torch ops."""
    if kind == "none":
        return torch.ones(b, hq, sq, sk, dtype=torch.bool)
    if kind == "causal":
        return torch.tril(torch.ones(sq, sk, dtype=torch.bool)).expand(b, hq, sq, sk)
    if kind == "padding":
        ar_q = torch.arange(sq)
        ar_k = torch.arange(sk)
        n = torch.as_tensor(lengths).view(b, 1, 1, 1)
        return ((ar_q.view(1, 1, sq, 1) < n) & (ar_k.view(1, 1, 1, sk) < n)).expand(b, hq, sq, sk)
    if kind == "block":
        lay = torch.as_tensor(np.asarray(layout)).bool()
        dense = lay.repeat_interleave(bq, dim=-2).repeat_interleave(bk, dim=-1)[..., :sq, :sk]
        if dense.dim() == 2:
            dense = dense.expand(b, hq, sq, sk)
        return dense
    if kind == "dense":
        m = torch.as_tensor(np.asarray(dense)) != 0
        return m.expand(b, hq, sq, sk) if m.dim() == 2 else m
    raise ValueError(kind)


def _spec(mod, kind, lengths=None, layout=None, bq=64, bk=64, dense=None):
    spec = mod.MaskSpec(kind=kind, lengths=lengths, layout=layout, block_q=bq, block_k=bk)
    if dense is not None:
        spec.dense = dense
    return spec


def _sdpa(q, k, v, tmask, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=tmask, scale=scale,
                                          enable_gqa=qt.shape[1] != kt.shape[1])


def _torch_lse(q, k, tmask, scale):
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    s = s.masked_fill(~tmask, float("-inf"))
    return torch.logsumexp(s, dim=-1)


def _mask_cases(mod):
    """(name, b, hq, hkv, sq, sk, d, spec, tmask) covering every mask kind, GQA and ragged tails."""
    r = _rng(7)
    cases = []
    b, hq, hkv, s, d = 2, 4, 2, 37, 16
    cases.append(("none_gqa", b, hq, hkv, s, s, d, _spec(mod, "none"), _torch_mask("none", b, hq, s, s)))
    cases.append(("causal_gqa", b, hq, hkv, s, s, d, _spec(mod, "causal"), _torch_mask("causal", b, hq, s, s)))
    lengths = np.array([29, 11], dtype=np.int32)
    cases.append(("padding", b, hq, hq, s, s, d, _spec(mod, "padding", lengths=lengths),
                  _torch_mask("padding", b, hq, s, s, lengths=lengths)))
    nb = -(-s // 8)
    lay = (r.random((nb, nb)) < 0.3).astype(np.uint8)
    lay[np.arange(nb), np.arange(nb)] = 1
    cases.append(("block_shared", b, hq, hkv, s, s, d, _spec(mod, "block", layout=lay, bq=8, bk=8),
                  _torch_mask("block", b, hq, s, s, layout=lay, bq=8, bk=8)))
    lay4 = (r.random((b, hq, nb, nb)) < 0.3).astype(np.uint8)
    lay4[0, 1, 2, :] = 0  # one fully masked block row -> empty query rows
    cases.append(("block_per_head", b, hq, hq, s, s, d, _spec(mod, "block", layout=lay4, bq=8, bk=8),
                  _torch_mask("block", b, hq, s, s, layout=lay4, bq=8, bk=8)))
    # non-square, no mask, key count not a multiple of anything
    cases.append(("none_rect", 1, 2, 1, 5, 23, 8, _spec(mod, "none"), _torch_mask("none", 1, 2, 5, 23)))
    # the generic element mask: shared by every (b, h), with one fully masked query row ...
    dense = (r.random((s, s)) < 0.5).astype(np.uint8)
    dense[5, :] = 0
    cases.append(("dense_shared", b, hq, hkv, s, s, d, _spec(mod, "dense", dense=dense),
                  _torch_mask("dense", b, hq, s, s, dense=dense)))
    # ... and one per (b, h), non-square, every row keeping at least one key
    dense4 = (r.random((b, hq, 9, s)) < 0.4).astype(np.uint8)
    dense4[..., 0] = 1
    cases.append(("dense_per_head", b, hq, hkv, 9, s, d, _spec(mod, "dense", dense=dense4),
                  _torch_mask("dense", b, hq, 9, s, dense=dense4)))
    return cases


# ----------------------------------------------------------------------------------------------
def check_sdpa_forward(mod):
    for i, (name, b, hq, hkv, sq, sk, d, spec, tmask) in enumerate(_mask_cases(mod)):
        q, k, v = _qkv(100 + i, b, hq, hkv, sq, sk, d)
        scale = 1.0 / math.sqrt(d)
        o, lse = mod.attention_fwd(q, k, v, spec, scale)
        nonempty = tmask.any(-1).numpy()
        ref_o = _sdpa(q, k, v, tmask, scale).numpy()
        ref_lse = _torch_lse(q, k, tmask, scale).numpy()
        assert o.shape == ref_o.shape and lse.shape == ref_lse.shape, name
        np.testing.assert_allclose(o[nonempty], ref_o[nonempty], rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(lse[nonempty], ref_lse[nonempty], rtol=0, atol=1e-12, err_msg=name)
        assert np.all(o[~nonempty] == 0.0), name
        assert np.all(np.isneginf(lse[~nonempty])), name


def check_autograd_backward(mod):
    for i, (name, b, hq, hkv, sq, sk, d, spec, tmask) in enumerate(_mask_cases(mod)):
        if not bool(tmask.any(-1).all()):
            continue  # SDPA yields NaN on empty rows; those are pinned by the padding reduction
        q, k, v = _qkv(200 + i, b, hq, hkv, sq, sk, d)
        do = _rng(300 + i).standard_normal((b, hq, sq, d))
        scale = 0.7 / math.sqrt(d)
        qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=tmask, scale=scale, enable_gqa=hq != hkv)
        out.backward(torch.from_numpy(do))
        dq, dk, dv = mod.attention_bwd(q, k, v, do, spec, scale)
        for got, ref, nm in ((dq, qt.grad, "dq"), (dk, kt.grad, "dk"), (dv, vt.grad, "dv")):
            np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11, err_msg=f"{name} {nm}")


def check_finite_differences(mod):
    r = _rng(11)
    cases = [("none", 1, 2, 2, 5, 7, 4, _spec(mod, "none")),
             ("causal_gqa", 1, 2, 1, 6, 6, 3, _spec(mod, "causal")),
             ("padding", 2, 1, 1, 9, 9, 4, _spec(mod, "padding", lengths=np.array([4, 9], np.int32))),
             ("block", 1, 1, 1, 12, 12, 2,
              _spec(mod, "block", layout=np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8), bq=4, bk=4))]
    h = 1e-6
    for name, b, hq, hkv, sq, sk, d, spec in cases:
        q, k, v = (x * 0.8 for x in _qkv(400, b, hq, hkv, sq, sk, d))
        do = r.standard_normal((b, hq, sq, d))
        scale = 0.9
        grads = mod.attention_bwd(q, k, v, do, spec, scale)

        def loss(qq, kk, vv):
            o, _ = mod.attention_fwd(qq, kk, vv, spec, scale)
            return float((o * do).sum())

        for which, arr in enumerate((q, k, v)):
            flat_idx = r.choice(arr.size, size=min(6, arr.size), replace=False)
            for fi in flat_idx:
                idx = np.unravel_index(fi, arr.shape)
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                an = grads[which][idx]
                assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, which, idx, fd, an)


def check_closed_forms(mod):
    b, h, s, d = 2, 3, 19, 8
    q, k, v = _qkv(500, b, h, h, s, s, d)
    scale = 0.5
    # Q = 0: uniform weights over the kept keys
    for kind, spec, tm in (("none", _spec(mod, "none"), _torch_mask("none", b, h, s, s)),
                           ("causal", _spec(mod, "causal"), _torch_mask("causal", b, h, s, s))):
        o, lse = mod.attention_fwd(np.zeros_like(q), k, v, spec, scale)
        m = tm.numpy().astype(np.float64)
        cnt = m.sum(-1)
        ref = np.einsum("bhij,bhjd->bhid", m, v) / cnt[..., None]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12, err_msg=kind)
        np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-12, err_msg=kind)
    # a single key: O = V, LSE = scale * q . k
    o, lse = mod.attention_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], _spec(mod, "none"), scale)
    np.testing.assert_allclose(o, v[:, :, :1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[..., 0], scale * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=0, atol=1e-12)
    # first causal row: O_0 = V_0, LSE_0 = scale * q_0 . k_0
    o, lse = mod.attention_fwd(q, k, v, _spec(mod, "causal"), scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], scale * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=0, atol=1e-12)
    # constant V rows give that constant
    c = _rng(3).standard_normal(d)
    vc = np.broadcast_to(c, v.shape).copy()
    o, _ = mod.attention_fwd(q, k, vc, _spec(mod, "causal"), scale)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)
    # adding c to every key leaves O unchanged and shifts LSE by scale * q . c
    o0, lse0 = mod.attention_fwd(q, k, v, _spec(mod, "none"), scale)
    o1, lse1 = mod.attention_fwd(q, k + c, v, _spec(mod, "none"), scale)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1 - lse0, scale * np.einsum("bhid,d->bhi", q, c), rtol=0, atol=1e-12)


def check_invariants(mod):
    b, hq, hkv, s, d = 1, 4, 2, 40, 8
    q, k, v = _qkv(600, b, hq, hkv, s, s, d)
    scale = 1.0 / math.sqrt(d)
    r = _rng(5)
    nb = 5
    lay = (r.random((nb, nb)) < 0.4).astype(np.uint8)
    lay[np.arange(nb), np.arange(nb)] = 1
    spec = _spec(mod, "block", layout=lay, bq=8, bk=8)
    tmask = _torch_mask("block", b, hq, s, s, layout=lay, bq=8, bk=8)
    o, lse = mod.attention_fwd(q, k, v, spec, scale)
    # probabilities computed here from the definition with the oracle's LSE sum to one
    kr = np.repeat(k, hq // hkv, axis=1)
    sc = scale * np.einsum("bhid,bhjd->bhij", q, kr)
    p = np.where(tmask.numpy(), np.exp(sc - lse[..., None]), 0.0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    # jointly permuting whole key blocks and the layout columns leaves O and LSE unchanged
    perm_blocks = r.permutation(nb)
    perm = np.concatenate([np.arange(pb * 8, pb * 8 + 8) for pb in perm_blocks])
    spec_p = _spec(mod, "block", layout=lay[:, perm_blocks], bq=8, bk=8)
    o_p, lse_p = mod.attention_fwd(q, k[:, :, perm], v[:, :, perm], spec_p, scale)
    np.testing.assert_allclose(o_p, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-12)
    # backward identities
    do = r.standard_normal(q.shape)
    dq, dk, dv = mod.attention_bwd(q, k, v, do, spec, scale)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-11)
    g = hq // hkv
    ref_dv_sum = do.reshape(b, hkv, g, s, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), ref_dv_sum, rtol=0, atol=1e-11)


def check_reductions(mod):
    b, h, s, d = 2, 2, 33, 8
    q, k, v = _qkv(700, b, h, h, s, s, d)
    do = _rng(701).standard_normal(q.shape)
    scale = 0.4
    # padding on batch element i equals no mask on the first L_i rows and keys
    lengths = np.array([20, 33], dtype=np.int32)
    o, lse = mod.attention_fwd(q, k, v, _spec(mod, "padding", lengths=lengths), scale)
    dq, dk, dv = mod.attention_bwd(q, k, v, do, _spec(mod, "padding", lengths=lengths), scale)
    for bi, n in enumerate(lengths):
        sl = (slice(bi, bi + 1), slice(None), slice(0, n))
        o_t, lse_t = mod.attention_fwd(q[sl], k[sl], v[sl], _spec(mod, "none"), scale)
        g_t = mod.attention_bwd(q[sl], k[sl], v[sl], do[sl], _spec(mod, "none"), scale)
        np.testing.assert_allclose(o[sl], o_t, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[sl], lse_t, rtol=0, atol=1e-12)
        for got, ref in zip((dq, dk, dv), g_t):
            np.testing.assert_allclose(got[sl], ref, rtol=0, atol=1e-12)
        tail = (bi, slice(None), slice(n, None))
        assert np.all(o[tail] == 0) and np.all(np.isneginf(lse[tail]))
        assert np.all(dq[tail] == 0) and np.all(dk[tail] == 0) and np.all(dv[tail] == 0)
    # grouped-query equals multi-head with repeated key/value heads (dK, dV summed per group)
    hq, hkv = 6, 2
    q6, k2, v2 = _qkv(702, 1, hq, hkv, s, s, d)
    do6 = _rng(703).standard_normal(q6.shape)
    o_g, lse_g = mod.attention_fwd(q6, k2, v2, _spec(mod, "causal"), scale)
    k6, v6 = np.repeat(k2, 3, axis=1), np.repeat(v2, 3, axis=1)
    o_m, lse_m = mod.attention_fwd(q6, k6, v6, _spec(mod, "causal"), scale)
    np.testing.assert_allclose(o_g, o_m, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_g, lse_m, rtol=0, atol=1e-13)
    dq_g, dk_g, dv_g = mod.attention_bwd(q6, k2, v2, do6, _spec(mod, "causal"), scale)
    dq_m, dk_m, dv_m = mod.attention_bwd(q6, k6, v6, do6, _spec(mod, "causal"), scale)
    np.testing.assert_allclose(dq_g, dq_m, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_g, dk_m.reshape(1, hkv, 3, s, d).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_g, dv_m.reshape(1, hkv, 3, s, d).sum(2), rtol=0, atol=1e-12)
    # an all-ones block layout equals no mask
    nb = -(-s // 8)
    ones = np.ones((nb, nb), np.uint8)
    o_b, lse_b = mod.attention_fwd(q, k, v, _spec(mod, "block", layout=ones, bq=8, bk=8), scale)
    o_n, lse_n = mod.attention_fwd(q, k, v, _spec(mod, "none"), scale)
    np.testing.assert_allclose(o_b, o_n, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_b, lse_n, rtol=0, atol=1e-13)
    # an identity block layout equals independent attention on each diagonal block
    eye = np.eye(nb, dtype=np.uint8)
    o_i, lse_i = mod.attention_fwd(q, k, v, _spec(mod, "block", layout=eye, bq=8, bk=8), scale)
    for blk in range(nb):
        sl = (slice(None), slice(None), slice(blk * 8, min(s, blk * 8 + 8)))
        o_t, lse_t = mod.attention_fwd(q[sl], k[sl], v[sl], _spec(mod, "none"), scale)
        np.testing.assert_allclose(o_i[sl], o_t, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse_i[sl], lse_t, rtol=0, atol=1e-13)


def check_golden_two_keys(mod):
    with open(os.path.join(GOLDEN, "two_keys.json")) as f:
        g = json.load(f)
    q = np.array(g["q"]).reshape(1, 1, 2, 1)
    k = np.array(g["k"]).reshape(1, 1, 2, 1)
    v = np.array(g["v"]).reshape(1, 1, 2, 1)
    do = np.array(g["do"]).reshape(1, 1, 2, 1)
    for kind in ("none", "causal"):
        o, lse = mod.attention_fwd(q, k, v, _spec(mod, kind), g["scale"])
        np.testing.assert_allclose(o.ravel(), g[kind]["o"], rtol=0, atol=1e-14, err_msg=kind)
        np.testing.assert_allclose(lse.ravel(), g[kind]["lse"], rtol=0, atol=1e-14, err_msg=kind)
    dq, dk, dv = mod.attention_bwd(q, k, v, do, _spec(mod, "none"), g["scale"])
    np.testing.assert_allclose(dq.ravel(), g["none"]["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), g["none"]["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), g["none"]["dv"], rtol=0, atol=1e-14)


ALL_CHECKS = [
    check_sdpa_forward,
    check_autograd_backward,
    check_finite_differences,
    check_closed_forms,
    check_invariants,
    check_reductions,
    check_golden_two_keys,
]
