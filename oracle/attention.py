"""fp64 CPU oracle for multi-head attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

What it computes is the plain definition of attention, written out with the
full score matrix materialised, one (batch, head) pair at a time:

* page 2 (zwxr.cn, "fused multi-head attention operator"), section 3.1: inputs
  Q, K, V of shape [batch, head, seq_len, head_dim] plus an optional mask; for
  every query, dot products with all keys, multiplied by the scale, a softmax
  over keys, then the V rows weighted by those probabilities;
* page 2, section 1.2 and page 1 (smzdm.com), section 03: the unfused form
  materialises the [seq_len, seq_len] score matrix; this oracle does exactly
  that, in float64;
* page 2, section 3.3: a mask entry of 0 sends the score to minus infinity
  (the generic element mask mask[i][j]; the structured kinds below are
  special cases of it).
* page 1, section 03: the backward produces the three gradients dQ, dK, dV.
  They are written in closed form below from the chain rule through the
  softmax (the pages name the gradients but print no formula).

Readings taken where the pages are silent:

* a row whose every key is masked has O = 0 and LSE = -inf (the plain formula
  gives 0/0); its gradient rows are 0;
* LSE is the natural log of the softmax denominator of the scaled, masked
  scores;
* grouped-query attention maps query head h to key/value head h // G, with
  G = heads_q / heads_kv (contiguous groups); dK and dV of a key/value head sum
  over its G query heads;
* causal masks key j for query i when j > i (top-left aligned, square only);
  padding keeps (i, j) when i < L_b and j < L_b; a block layout keeps the
  whole block_q x block_k tile where the layout byte is non-zero; a dense mask
  keeps (i, j) where its byte is non-zero.

Nothing here is blocked, fused or reordered beyond the definition: a numpy
matmul is the only library primitive used.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "MaskSpec",
    "mask_matrix",
    "attention_fwd",
    "attention_probs",
    "attention_rows",
    "attention_bwd",
    "attention_bwd_head",
    "attention_dq_rows",
]


@dataclass
class MaskSpec:
    """Description of a structured mask, in the oracle's own terms.

    kind: "none", "causal", "padding", "block" or "dense".
    lengths: padding only; int array [batch], the valid length of both the
        queries and the keys of each batch element.
    layout: block only; uint8/bool array, either [nb_q, nb_k] (shared by every
        batch element and head) or [batch, heads_q, nb_q, nb_k]. Non-zero means
        the tile is kept.
    block_q, block_k: block only; tile sizes in query rows and key columns.
    dense: dense only; uint8/bool array, either [sq, sk] (shared by every batch
        element and head) or [batch, heads_q, sq, sk]. Non-zero means query i
        attends to key j.
    """

    kind: str = "none"
    lengths: Optional[np.ndarray] = None
    layout: Optional[np.ndarray] = None
    block_q: int = 64
    block_k: int = 64
    dense: Optional[np.ndarray] = None


def mask_matrix(spec: MaskSpec, b: int, h: int, sq: int, sk: int, rows=None) -> np.ndarray:
    """Dense boolean [sq, sk] matrix for batch element b and query head h (only the query rows
    ``rows`` of it, in that order, when given).

    True means query i attends to key j; False means the score is replaced by
    minus infinity (page 2, section 3.3: mask value 0 -> -inf).
    """
    qi = np.arange(sq) if rows is None else np.asarray(rows)
    i = qi[:, None]
    j = np.arange(sk)[None, :]
    if spec.kind == "none":
        return np.ones((len(qi), sk), dtype=bool)
    if spec.kind == "causal":
        return j <= i
    if spec.kind == "padding":
        n = int(spec.lengths[b])
        return (i < n) & (j < n)
    if spec.kind == "block":
        lay = np.asarray(spec.layout)
        if lay.ndim == 4:
            lay = lay[b, h]
        keep = lay != 0
        brows = np.minimum(qi // spec.block_q, keep.shape[0] - 1)
        bcols = np.minimum(np.arange(sk) // spec.block_k, keep.shape[1] - 1)
        return keep[brows[:, None], bcols[None, :]]
    if spec.kind == "dense":
        arr = np.asarray(spec.dense)
        if arr.ndim == 4:
            arr = arr[b, h]
        return arr[:sq, :sk][qi] != 0
    raise ValueError(f"unknown mask kind {spec.kind!r}")


def _kv_head(h: int, heads_q: int, heads_kv: int) -> int:
    """Key/value head used by query head h (contiguous groups of G = Hq/Hkv)."""
    return h // (heads_q // heads_kv)


def attention_probs(q, k, mask: MaskSpec, scale: float, b: int, h: int):
    """Score matrix, probabilities and LSE of one (b, h) pair, in float64.

    Returns (P, lse, keep): P is [sq, sk] with rows summing to 1 (rows with no
    kept key are all zero), lse is [sq] (natural log; -inf for empty rows),
    keep is the boolean mask used.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    g = _kv_head(h, hq, hkv)
    sq, sk = q.shape[2], k.shape[2]
    keep = mask_matrix(mask, b, h, sq, sk)
    s = scale * (q[b, h] @ k[b, g].T)
    s = np.where(keep, s, -np.inf)
    nonempty = keep.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    denom = e.sum(axis=1)
    p = np.where(nonempty[:, None], e / np.where(nonempty, denom, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(nonempty, m + np.log(np.where(nonempty, denom, 1.0)), -np.inf)
    return p, lse, keep


def attention_fwd(q, k, v, mask: MaskSpec, scale: float):
    """O = softmax(scale * Q K^T + mask) V and the per-row LSE, in float64.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]. Returns (o [B, Hq, Sq, D],
    lse [B, Hq, Sq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, hq, sq, d = q.shape
    hkv = k.shape[1]
    o = np.zeros((bsz, hq, sq, v.shape[3]), dtype=np.float64)
    lse = np.zeros((bsz, hq, sq), dtype=np.float64)
    for b in range(bsz):
        for h in range(hq):
            p, l, _ = attention_probs(q, k, mask, scale, b, h)
            o[b, h] = p @ v[b, _kv_head(h, hq, hkv)]
            lse[b, h] = l
    return o, lse


def attention_rows(q, k, v, mask: MaskSpec, scale: float, b: int, h: int, rows):
    """O and LSE of selected query rows of one (b, h) pair: the same definition as
    attention_fwd, evaluated only for ``rows`` (used to sample very long sequences)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    rows = np.asarray(rows)
    hq, hkv = q.shape[1], k.shape[1]
    g = _kv_head(h, hq, hkv)
    sq, sk = q.shape[2], k.shape[2]
    keep = mask_matrix(mask, b, h, sq, sk, rows)
    qr = np.asarray(q[b, h, rows], dtype=np.float64)
    kg = np.asarray(k[b, g], dtype=np.float64)
    vg = np.asarray(v[b, g], dtype=np.float64)
    s = np.where(keep, scale * (qr @ kg.T), -np.inf)
    nonempty = keep.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    denom = e.sum(axis=1)
    safe = np.where(nonempty, denom, 1.0)
    o = np.where(nonempty[:, None], (e / safe[:, None]) @ vg, 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(nonempty, m + np.log(safe), -np.inf)
    return o, lse


def attention_dq_rows(q, k, v, do, mask: MaskSpec, scale: float, b: int, h: int, rows):
    """dQ of selected query rows of one (b, h) pair: the chain rule of attention_bwd restricted to
    those rows (row i of dQ needs only row i of P, dP and dS), for sampling very long sequences."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    rows = np.asarray(rows)
    hq, hkv = q.shape[1], k.shape[1]
    g = _kv_head(h, hq, hkv)
    sq, sk = q.shape[2], k.shape[2]
    keep = mask_matrix(mask, b, h, sq, sk, rows)
    qr = np.asarray(q[b, h, rows], dtype=np.float64)
    dor = np.asarray(do[b, h, rows], dtype=np.float64)
    kg = np.asarray(k[b, g], dtype=np.float64)
    vg = np.asarray(v[b, g], dtype=np.float64)
    s = np.where(keep, scale * (qr @ kg.T), -np.inf)
    nonempty = keep.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    p = e / np.where(nonempty, e.sum(axis=1), 1.0)[:, None]
    dp = dor @ vg.T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    return scale * (ds @ kg)


def attention_bwd(q, k, v, do, mask: MaskSpec, scale: float):
    """Gradients of L = sum(dO * O) with respect to Q, K and V, in float64.

    Chain rule through O = P V and P = softmax(S), S = scale * Q K^T:
      dV = P^T dO
      dP = dO V^T
      dS = P * (dP - rowsum(P * dP))
      dQ = scale * dS K
      dK = scale * dS^T Q
    Masked entries have P = 0 and hence dS = 0. For grouped-query attention
    dK and dV of a key/value head sum over the query heads that use it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bsz, hq, sq, d = q.shape
    hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            p, _, _ = attention_probs(q, k, mask, scale, b, h)
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            rowdot = (p * dp).sum(axis=1)
            ds = p * (dp - rowdot[:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_bwd_head(q, k, v, do, mask: MaskSpec, scale: float, b: int, h: int):
    """The contribution of one (b, h) pair to the gradients: dQ[b, h] and the parts of dK[b, g],
    dV[b, g] that query head h adds (g = h // G); the same chain rule as attention_bwd,
    evaluated for one pair only (used to sample long sequences)."""
    hq, hkv = np.asarray(q).shape[1], np.asarray(k).shape[1]
    g = _kv_head(h, hq, hkv)
    q64 = np.asarray(q[b:b + 1, h:h + 1], dtype=np.float64)
    k64 = np.asarray(k[b:b + 1, g:g + 1], dtype=np.float64)
    v64 = np.asarray(v[b:b + 1, g:g + 1], dtype=np.float64)
    do64 = np.asarray(do[b:b + 1, h:h + 1], dtype=np.float64)
    sub = MaskSpec(kind=mask.kind, block_q=mask.block_q, block_k=mask.block_k)
    if mask.kind == "padding":
        sub.lengths = np.asarray(mask.lengths)[b:b + 1]
    if mask.kind == "block":
        lay = np.asarray(mask.layout)
        sub.layout = lay[b:b + 1, h:h + 1] if lay.ndim == 4 else lay
    if mask.kind == "dense":
        arr = np.asarray(mask.dense)
        sub.dense = arr[b:b + 1, h:h + 1] if arr.ndim == 4 else arr
    dq, dk, dv = attention_bwd(q64, k64, v64, do64, sub, scale)
    return dq[0, 0], dk[0, 0], dv[0, 0]
