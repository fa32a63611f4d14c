"""Oracle: tree-masked GQA attention with RoPE at semantic positions, readout.

Sources:
  * [SpecOPD paper page, Figure 3]: packed queries share the trunk K/V and
    each row attends to itself and its ancestors only.
  * [SpecOPD notes page, "Equations"]: semantic positions a_b + i differ from
    packed offsets; the anchor row predicts y_{b,1}, the row of y_{b,i-1}
    predicts y_{b,i}; a token's own row is never read out.
  * [SpecOPD notes page, "Checks, negative controls, and limits"]: packed
    scoring must equal each branch's independent causal scoring.

Readings (the pages give positions only): rotate-half RoPE pairing dimension
j with j + D/2 at angle pos * base^(-2j/D), applied to Q and K; softmax scale
1/sqrt(D); query head h uses KV head floor(h / (Hq/Hkv)). Everything is float64
on the exact input values (bf16 widens to float32 exactly).
"""
from __future__ import annotations

import numpy as np


def rope_ref(x, pos, base):
    """Rotate the last axis of ``x`` (size D) at integer positions ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``. Pair (j, j + D/2) turns by the
    angle pos * base^(-2j/D), computed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv_freq = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _softmax_attend(qr, kr, v, scale):
    """One query row against its visible keys, all heads.

    qr [Hq, D] (rotated), kr [n, Hkv, D] (rotated), v [n, Hkv, D] -> [Hq, D].
    """
    hq, D = qr.shape
    hkv = kr.shape[1]
    g = hq // hkv
    qg = qr.reshape(hkv, g, D)
    s = np.einsum("chd,hgd->hgc", kr, qg) * scale          # [Hkv, G, n]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    o = np.einsum("hgc,chd->hgd", p, v)                     # [Hkv, G, D]
    return o.reshape(hq, D)


def tree_attn_ref(layout, q, k, v, rope_base, scale=None, rows=None):
    """Packed tree attention for the given rows (default: all), float64.

    q [N,Hq,D], k and v [N,Hkv,D] as float arrays; returns [len(rows), Hq, D].
    Row r attends to the trunk prefix [tree_off, row_trunk_hi[r]] and to its own
    branch rows [row_branch_lo[r], r]; RoPE uses row_pos (semantic positions).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = layout["row_pos"].astype(np.int64)
    kr = rope_ref(k, pos[:, None], rope_base)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), hq, D), dtype=np.float64)
    tree_off, trunk_hi, branch_lo = layout["tree_off"], layout["row_trunk_hi"], layout["row_branch_lo"]
    row_tree = layout["row_tree"]
    for i, r in enumerate(rows):
        lo = int(tree_off[row_tree[r]])
        vis = np.concatenate([np.arange(lo, int(trunk_hi[r]) + 1),
                              np.arange(int(branch_lo[r]), int(r) + 1)])
        qr = rope_ref(q[r], pos[r], rope_base)
        out[i] = _softmax_attend(qr, kr[vis], v[vis], scale)
    return out


def causal_attn_ref(q, k, v, rope_base, scale=None):
    """Plain causal GQA attention over one unpacked sequence, float64.

    q [L,Hq,D], k and v [L,Hkv,D]; position of token i is i; token i attends to
    tokens 0..i. Returns [L, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, hq, D = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = np.arange(L)
    qr = rope_ref(q, pos[:, None], rope_base).reshape(L, hkv, g, D)
    kr = rope_ref(k, pos[:, None], rope_base)
    s = np.einsum("ihgd,jhd->hgij", qr, kr) * scale         # [Hkv, G, L, L]
    future = np.triu(np.ones((L, L), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    o = np.einsum("hgij,jhd->ihgd", p, v)
    return o.reshape(L, hq, D)


def brute_force_branch_ref(layout, q, k, v, b, rope_base, scale=None):
    """Independent causal scoring of branch b as its own unpacked sequence.

    The sequence is the trunk tokens 0..a_b of b's tree followed by
    y_{b,1..W_b-1}; positions are plain sequence indices. Returns
    (packed_rows, outputs): the packed row each sequence token came from and
    its causal attention output, so the packed result can be compared row by
    row ([SpecOPD notes page, "Checks, negative controls, and limits"]).
    """
    t = int(layout["branch_tree"][b])
    a = int(layout["branch_anchor"][b])
    w = int(layout["branch_len"][b])
    lo = int(layout["tree_off"][t])
    bo = int(layout["branch_off"][b])
    packed_rows = np.concatenate([np.arange(lo, lo + a + 1), np.arange(bo, bo + w - 1)])
    out = causal_attn_ref(np.asarray(q)[packed_rows], np.asarray(k)[packed_rows],
                          np.asarray(v)[packed_rows], rope_base, scale)
    return packed_rows, out


def readout_ref(layout, o):
    """Predecessor-row readout: readout[s] = o[step_pred_row[s]]."""
    return np.asarray(o)[layout["step_pred_row"].astype(np.int64)]
