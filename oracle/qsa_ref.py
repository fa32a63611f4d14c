"""Oracle: sparse attention with branch-consistent indexer groups (test infrastructure only).

Source: [SpecOPD paper page, Figure 4] (branch-parallel scoring with sparse
attention). What the caption fixes:
  * keys are grouped a fixed number of tokens at a time, and every complete
    group carries one indexer group key;
  * a row reuses the complete groups of the shared trunk; a group that is not
    yet complete at the row stays in the row's causal tail;
  * in the figure's example (groups of 4) the anchor row at "evening" reads
    [a, quiet, evening] as a 3/4 causal tail, and the row of the branch token
    "with" completes [a, quiet, evening, with] (4/4), a group whose key must be
    built from that branch's own tokens (a branch-specific group key);
  * indexer queries pick the eligible complete groups by top-k; attention reads
    the keys of the picked groups plus the causal tail, which bypasses top-k.

Readings (the caption leaves these open; the plainest choice is taken):
  * groups cover semantic positions [jG, (j+1)G) of a row's history (the trunk
    through the anchor, then the branch's own tokens); at a row of position t
    the complete groups are j < floor((t+1)/G), the group the row itself
    completes included, and the causal tail is positions floor((t+1)/G)*G .. t;
  * a group key is the mean of the group's per-token indexer keys; the score of
    group j for a row is the dot product of the row's indexer query with it;
  * top-k keeps the k highest scores (ties: the lower group index first), or all
    complete groups when there are at most k;
  * one indexer query and key per token and KV head: the pick is shared by the
    query heads of a GQA group;
  * attention over the picked keys plus the tail is the full-attention rule of
    tree_attn_ref restricted to that set (rotate-half RoPE at semantic
    positions, scale 1/sqrt(D), float64).

Two independent statements follow. ``qsa_attn_ref`` walks each packed row's
history through the tree's parent chain (no sharing of any kind).
``qsa_causal_ref`` is sparse attention over one plain unpacked sequence (groups
by sequence index, no layout at all); ``qsa_brute_force_branch_ref`` runs it on
each branch's own sequence, the "independent causal scoring" the packed result
must equal.
"""
from __future__ import annotations

import numpy as np

from .attn_ref import rope_ref
from .pack_ref import parents_ref


def qsa_row_structure(t, G):
    """(number of complete groups, causal tail positions) of a row at position t."""
    n_c = (int(t) + 1) // int(G)
    return n_c, np.arange(n_c * G, int(t) + 1, dtype=np.int64)


def qsa_group_keys(ki_hist, G):
    """Mean indexer key of every complete group of a history.

    ki_hist [L, Hkv, DI] (position order) -> [floor(L/G), Hkv, DI].
    """
    ki_hist = np.asarray(ki_hist, dtype=np.float64)
    n = ki_hist.shape[0] // G
    return ki_hist[:n * G].reshape(n, G, *ki_hist.shape[1:]).mean(axis=1)


def qsa_pick(scores, top_k):
    """Indices of the top_k largest scores (ties: lower index), ascending; all if fewer."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if n <= top_k:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))   # score descending, then index ascending
    return np.sort(order[:top_k])


def _attend(q_row, k_keys, v_keys, pos_row, pos_keys, rope_base, scale):
    """q_row [Hq, D] against keys [n, Hkv, D] at the given semantic positions -> [Hq, D]."""
    hq, D = q_row.shape
    hkv = k_keys.shape[1]
    grp = hq // hkv
    qr = rope_ref(q_row, np.full(hq, pos_row), rope_base).reshape(hkv, grp, D)
    kr = rope_ref(k_keys, np.asarray(pos_keys)[:, None], rope_base)
    s = np.einsum("chd,hgd->hgc", kr, qr) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hgc,chd->hgd", p, np.asarray(v_keys, dtype=np.float64)).reshape(hq, D)


def _sparse_row(q_row, k_hist, v_hist, qi_row, ki_hist, t, G, top_k, rope_base, scale):
    """One row of position t over its history (position order): output [Hq, D] and the
    picked groups [Hkv, top_k] (ascending, -1 padded). Each KV head picks on its own and
    its query heads attend over the picked groups' keys plus the causal tail."""
    hq, D = q_row.shape
    hkv = k_hist.shape[1]
    grp = hq // hkv
    n_c, tail = qsa_row_structure(t, G)
    keys = qsa_group_keys(ki_hist[:n_c * G], G)                    # [n_c, Hkv, DI]
    out = np.empty((hq, D))
    picked = np.full((hkv, top_k), -1, dtype=np.int64)
    for g in range(hkv):
        sel = qsa_pick(keys[:, g] @ np.asarray(qi_row[g], dtype=np.float64), top_k) if n_c else \
            np.zeros(0, dtype=np.int64)
        picked[g, :len(sel)] = sel
        pos = np.concatenate([(G * sel[:, None] + np.arange(G)).ravel(), tail]).astype(np.int64)
        out[g * grp:(g + 1) * grp] = _attend(q_row[g * grp:(g + 1) * grp], k_hist[pos][:, g:g + 1],
                                             v_hist[pos][:, g:g + 1], t, pos, rope_base, scale)
    return out, picked


def qsa_history_ref(layout, r, parents=None):
    """Packed rows of row r's history in position order (root first, r last), by the
    parent chain ([SpecOPD notes page, "Equations"]: h_{b,i} = (x_{<=a_b}, y_{b,<i}))."""
    par = parents_ref(layout) if parents is None else parents
    chain = []
    c = int(r)
    while c >= 0:
        chain.append(c)
        c = int(par[c])
    return np.asarray(chain[::-1], dtype=np.int64)


def qsa_attn_ref(layout, q, k, v, qi, ki, G, top_k, rope_base, scale=None, rows=None):
    """Sparse attention of packed rows (default all): outputs [n, Hq, D] and picks
    [n, Hkv, top_k]. Each row's groups, keys and tail come from its own history."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    qi, ki = np.asarray(qi, dtype=np.float64), np.asarray(ki, dtype=np.float64)
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.arange(layout["n_rows"]) if rows is None else np.asarray(rows, dtype=np.int64)
    par = parents_ref(layout)
    out = np.empty((len(rows), q.shape[1], D))
    picks = np.empty((len(rows), k.shape[1], top_k), dtype=np.int64)
    for i, r in enumerate(rows):
        hist = qsa_history_ref(layout, r, par)
        t = len(hist) - 1
        assert t == int(layout["row_pos"][r])
        out[i], picks[i] = _sparse_row(q[r], k[hist], v[hist], qi[r], ki[hist], t, G, top_k,
                                       rope_base, scale)
    return out, picks


def qsa_causal_ref(q, k, v, qi, ki, G, top_k, rope_base, scale=None):
    """Sparse attention over one unpacked sequence, positions 0..L-1: [L, Hq, D], picks."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    qi, ki = np.asarray(qi, dtype=np.float64), np.asarray(ki, dtype=np.float64)
    L, hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    keys_all = qsa_group_keys(ki, G)                      # every complete group of the sequence
    out = np.empty((L, hq, D))
    picks = np.full((L, k.shape[1], top_k), -1, dtype=np.int64)
    hkv = k.shape[1]
    grp = hq // hkv
    for t in range(L):
        n_c = (t + 1) // G
        tail = np.arange(n_c * G, t + 1)
        for g in range(hkv):
            sc = keys_all[:n_c, g] @ qi[t, g]
            sel = qsa_pick(sc, top_k)
            picks[t, g, :len(sel)] = sel
            pos = np.concatenate([(G * sel[:, None] + np.arange(G)).ravel(), tail]).astype(np.int64)
            out[t, g * grp:(g + 1) * grp] = _attend(q[t, g * grp:(g + 1) * grp], k[pos, g:g + 1],
                                                    v[pos, g:g + 1], t, pos, rope_base, scale)
    return out, picks


def qsa_brute_force_branch_ref(layout, q, k, v, qi, ki, b, G, top_k, rope_base, scale=None):
    """Branch b scored as its own sequence: trunk tokens 0..a_b of its tree, then
    y_{b,1..W_b-1}. Returns (packed rows of the sequence's tokens, outputs, picks)."""
    t = int(layout["branch_tree"][b])
    a = int(layout["branch_anchor"][b])
    w = int(layout["branch_len"][b])
    lo = int(layout["tree_off"][t])
    bo = int(layout["branch_off"][b])
    rows = np.concatenate([np.arange(lo, lo + a + 1), np.arange(bo, bo + w - 1)]).astype(np.int64)
    out, picks = qsa_causal_ref(np.asarray(q)[rows], np.asarray(k)[rows], np.asarray(v)[rows],
                                np.asarray(qi)[rows], np.asarray(ki)[rows], G, top_k, rope_base, scale)
    return rows, out, picks
