"""Oracle: indexed GDN state replay for branch-parallel scoring, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * [SpecOPD paper page, Figure 5]: GDN scoring of branches. One pass over the
    trunk stores the FP32 state every C = 64 tokens; a branch loads the last
    stored state at or before its anchor, runs the trunk tokens from there to
    the anchor, then runs its own tokens and reads the state with each token's
    query for its output. Stored states are never overwritten, and each
    token's convolution window runs over its ancestors.
  * [SpecOPD paper page, Figure 13]: GDN work counts include that replay.
    The trunk pass here also gives every trunk token's output, which is what
    scoring the trunk needs.
  * [SpecOPD notes page, "Checks, negative controls, and limits"]: packed
    scoring must equal each branch's independent causal scoring.

Readings (the pages name GDN but do not write its recurrence out):
  1. Gated delta rule per head, state S in R^{dv x dk}:
        S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
        o_t = S_t q_t.
  2. Checkpoint c of a tree holds S after trunk tokens 0 .. cC-1 (checkpoint
     0 is the zero state). A branch anchored at trunk token a starts from
     checkpoint floor((a + 1) / C) and replays trunk tokens cC .. a, at most
     C - 1 of them.
  3. Features: a depthwise causal convolution of width K along the ancestry
     path (tap j multiplies the j-th ancestor, j = 0 the token itself; zero
     before the tree's first token), then SiLU, on the q, k and v channels;
     q and k are then L2-normalised per head and q is scaled by 1/sqrt(dk).
  4. The decay alpha in (0, 1] and the write strength beta in (0, 1) are
     inputs per token and head (their projections are not on this path).
  5. One key/value head per head and dk = dv = D.
"""
from __future__ import annotations

import numpy as np

from .pack_ref import parents_ref


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def ancestors_ref(layout, K):
    """[N, K] packed rows of each row's K nearest path members: itself, its
    parent, its grandparent, ...; -1 past the tree's first trunk token."""
    par = parents_ref(layout)
    N = layout["n_rows"]
    anc = np.full((N, K), -1, dtype=np.int64)
    for r in range(N):
        a = r
        for j in range(K):
            anc[r, j] = a
            a = par[a] if a >= 0 else -1
    return anc


def conv_ancestry_ref(layout, x, w):
    """SiLU of the depthwise convolution along ancestry (reading 3).

    x [N, H, D] (any float), w [H, D, K] with tap j on the j-th ancestor."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[-1]
    anc = ancestors_ref(layout, K)
    acc = np.zeros_like(x)
    for j in range(K):
        rows = anc[:, j]
        ok = rows >= 0
        acc[ok] += w[None, :, :, j] * x[rows[ok]]
    return silu(acc)


def _l2norm(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def gdn_features_ref(layout, xq, xk, xv, wq, wk, wv):
    """(q~, k~, v~) for every packed row (reading 3): convolved along ancestry,
    SiLU, q and k L2-normalised per head, q scaled by 1/sqrt(D)."""
    D = np.asarray(xq).shape[-1]
    q = _l2norm(conv_ancestry_ref(layout, xq, wq)) / np.sqrt(D)
    k = _l2norm(conv_ancestry_ref(layout, xk, wk))
    v = conv_ancestry_ref(layout, xv, wv)
    return q, k, v


def gdn_step_ref(S, q, k, v, alpha, beta):
    """One gated delta-rule token for every head (reading 1).

    S [H, dv, dk]; q, k [H, dk]; v [H, dv]; alpha, beta [H]. Returns (S', o)."""
    a = np.asarray(alpha, dtype=np.float64)[:, None, None]
    b = np.asarray(beta, dtype=np.float64)[:, None, None]
    Sk = np.einsum("hvk,hk->hv", S, k)
    S = a * S + b * (v - a[:, :, 0] * Sk)[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def trunk_len_ref(layout):
    """Trunk length of every tree (rows whose branch is -1)."""
    T = np.zeros(layout["n_trees"], dtype=np.int64)
    for r in range(layout["n_rows"]):
        if layout["row_branch"][r] < 0:
            T[layout["row_tree"][r]] += 1
    return T


def gdn_trunk_ref(layout, q, k, v, alpha, beta, C):
    """The shared trunk pass: (checkpoints, outputs).

    Runs each tree's trunk from the zero state. Checkpoints [n_trees, max_T // C
    + 1, H, dv, dk]: slot c of tree t holds S after trunk tokens 0 .. cC-1
    (reading 2); slots a shorter tree never reaches stay zero. Outputs [N, H, D]:
    o_j of every trunk row, branch rows zero."""
    T = trunk_len_ref(layout)
    N, H, D = q.shape
    n_ckpt = int(T.max()) // C + 1 if len(T) else 1
    ck = np.zeros((layout["n_trees"], n_ckpt, H, D, D))
    out = np.zeros((N, H, D))
    for t in range(layout["n_trees"]):
        off = int(layout["tree_off"][t])
        S = np.zeros((H, D, D))
        for j in range(int(T[t])):
            r = off + j
            S, out[r] = gdn_step_ref(S, q[r], k[r], v[r], alpha[r], beta[r])
            if (j + 1) % C == 0:
                ck[t, (j + 1) // C] = S
    return ck, out


def gdn_checkpoints_ref(layout, q, k, v, alpha, beta, C):
    """The trunk pass's checkpoints alone (see gdn_trunk_ref)."""
    return gdn_trunk_ref(layout, q, k, v, alpha, beta, C)[0]


def gdn_replay_ref(layout, q, k, v, alpha, beta, ckpt, C, branches=None):
    """GDN outputs of every branch row by indexed replay, [N, H, D].

    Branch b copies checkpoint floor((a_b + 1) / C) of its tree, replays trunk
    tokens cC .. a_b, then steps through y_{b,1} .. y_{b,W_b-1} and reads each
    one's output (reading 2). Trunk rows are left at zero (the trunk pass owns
    them), and so are the rows of branches not in ``branches`` (default: all)."""
    N, H, D = q.shape
    out = np.zeros((N, H, D))
    for b in (range(layout["n_branches"]) if branches is None else branches):
        t, a = int(layout["branch_tree"][b]), int(layout["branch_anchor"][b])
        off = int(layout["tree_off"][t])
        c = (a + 1) // C
        S = np.array(ckpt[t, c], dtype=np.float64)       # a copy: the checkpoint stays as it is
        for j in range(c * C, a + 1):
            r = off + j
            S, _ = gdn_step_ref(S, q[r], k[r], v[r], alpha[r], beta[r])
        r0 = int(layout["branch_off"][b])
        for i in range(1, int(layout["branch_len"][b])):
            r = r0 + i - 1
            S, out[r] = gdn_step_ref(S, q[r], k[r], v[r], alpha[r], beta[r])
    return out


def gdn_branch_brute_ref(layout, xq, xk, xv, wq, wk, wv, alpha, beta, b):
    """Branch b scored as its own sequence: trunk tokens 0 .. a_b, then
    y_{b,1} .. y_{b,W_b-1}, with a plain causal convolution over sequence
    positions and the recurrence from the zero state. Returns [W_b-1, H, D].

    Uses neither the parent array nor checkpoints."""
    t, a = int(layout["branch_tree"][b]), int(layout["branch_anchor"][b])
    off, r0 = int(layout["tree_off"][t]), int(layout["branch_off"][b])
    W = int(layout["branch_len"][b])
    seq = list(range(off, off + a + 1)) + list(range(r0, r0 + W - 1))
    L = len(seq)

    def conv(x, w):
        x = np.asarray(x, dtype=np.float64)[seq]           # [L, H, D]
        w = np.asarray(w, dtype=np.float64)
        y = np.zeros_like(x)
        for p in range(L):
            for j in range(w.shape[-1]):
                if p - j >= 0:
                    y[p] += w[:, :, j] * x[p - j]
        return silu(y)

    D = np.asarray(xq).shape[-1]
    qs = _l2norm(conv(xq, wq)) / np.sqrt(D)
    ks = _l2norm(conv(xk, wk))
    vs = conv(xv, wv)
    al, be = np.asarray(alpha, dtype=np.float64)[seq], np.asarray(beta, dtype=np.float64)[seq]
    H = qs.shape[1]
    S = np.zeros((H, D, D))
    outs = []
    for p in range(L):
        S_new = np.empty_like(S)
        o = np.empty((H, D))
        for h in range(H):                                 # head by head, the update written out
            Sk = S[h] @ ks[p, h]
            S_new[h] = al[p, h] * S[h] + be[p, h] * np.outer(vs[p, h] - al[p, h] * Sk, ks[p, h])
            o[h] = S_new[h] @ qs[p, h]
        S = S_new
        if p > a:
            outs.append(o)
    return np.array(outs).reshape(W - 1, H, D)
