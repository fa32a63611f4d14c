"""Oracle: proposal-tree packing and tree visibility (test infrastructure only).

What a packed proposal tree is:
  * [SpecOPD paper page, Figure 2]: sampled continuations are attached to
    their anchors, giving a shared reference trunk and private draft branches.
  * [SpecOPD paper page, Figure 3]: rows and columns follow one packed token
    order; each row sees itself and its ancestors; terminal samples are read
    out from their predecessor and need no query row.
  * [SpecOPD notes page, "Equations"]: branch b's i-th sample is drawn from the
    history (x_{<=a_b}, y_{b,<i}); the anchor row predicts the first sample,
    the predecessor row predicts later ones, a token's own row is never used;
    the semantic position of y_{b,i} is a_b + i.
  * [SpecOPD notes page, "Inputs and code mapping"]: anchors are zero-based
    and the tree is built from trunk length, anchors and branch width only.

Readings taken where the pages leave a step open:
  * The terminal sample y_{b,W_b} gets no packed row, so branch b contributes
    W_b - 1 rows and W_b supervised steps (a one-token branch has no row).
  * Packed order: tree by tree; inside a tree the trunk rows 0..T-1 first,
    then its branches in ascending anchor order (ties by caller index), each
    branch in depth order. Supervised steps stay in caller branch order.
  * A one-token branch's ``branch_off`` is the packed row where its first row
    would have been placed (the next row in packed order).
"""
from __future__ import annotations

import numpy as np


def pack_ref(trunk_len, n_branches, anchors, branch_len):
    """Pack a batch of proposal trees with plain Python integers.

    Args: per tree ``trunk_len[t]`` (T_t >= 1) and ``n_branches[t]``; per branch,
    in caller order with tree t's branches consecutive, the local zero-based
    anchor ``anchors[b]`` (0 <= a_b < T_t) and width ``branch_len[b]`` (>= 1).

    Returns a dict of int32 arrays (names follow the packed layout):
      per tree  : tree_off [n_trees+1]
      per row   : row_tree, row_branch (-1 trunk), row_anchor (-1 trunk),
                  row_pos, row_depth, row_trunk_hi, row_branch_lo        [N]
      per branch: branch_tree, branch_anchor, branch_len, branch_off     [B]
                  step_off [B+1], branch_order [B] (branches in packed order)
      per step  : step_branch, step_pred_row, step_sample_row (-1 terminal) [R]
    and the scalars n_rows, n_steps, max_branch_len, max_pos.
    """
    trunk_len = [int(x) for x in trunk_len]
    n_branches = [int(x) for x in n_branches]
    anchors = [int(x) for x in anchors]
    branch_len = [int(x) for x in branch_len]
    n_trees = len(trunk_len)
    if len(n_branches) != n_trees:
        raise ValueError("trunk_len and n_branches differ in length")
    B = sum(n_branches)
    if len(anchors) != B or len(branch_len) != B:
        raise ValueError("anchors/branch_len must have sum(n_branches) entries")

    branch_tree = []
    for t in range(n_trees):
        if trunk_len[t] < 1 or n_branches[t] < 0:
            raise ValueError("tree %d: need T >= 1 and n_branches >= 0" % t)
        branch_tree += [t] * n_branches[t]
    for b in range(B):
        if not (0 <= anchors[b] < trunk_len[branch_tree[b]]):
            raise ValueError("branch %d: anchor %d outside [0, T)" % (b, anchors[b]))
        if branch_len[b] < 1:
            raise ValueError("branch %d: width must be >= 1" % b)

    rows = []          # (tree, branch, anchor, pos, depth)
    tree_off = []
    branch_off = [0] * B
    branch_order = []
    first = 0
    for t in range(n_trees):
        tree_off.append(len(rows))
        for j in range(trunk_len[t]):                      # the shared reference trunk
            rows.append((t, -1, -1, j, 0))
        mine = list(range(first, first + n_branches[t]))
        first += n_branches[t]
        mine.sort(key=lambda b: anchors[b])                 # stable: ties keep caller order
        for b in mine:
            branch_order.append(b)
            branch_off[b] = len(rows)
            for i in range(1, branch_len[b]):               # y_{b,1} .. y_{b,W-1}; y_{b,W} unpacked
                rows.append((t, b, anchors[b], anchors[b] + i, i))
    tree_off.append(len(rows))
    N = len(rows)

    row_trunk_hi, row_branch_lo = [], []
    for r, (t, b, a, pos, depth) in enumerate(rows):
        if b < 0:
            row_trunk_hi.append(r)                          # trunk: itself and everything before
            row_branch_lo.append(r + 1)                     # no own-branch rows
        else:
            row_trunk_hi.append(tree_off[t] + a)            # trunk through the anchor
            row_branch_lo.append(branch_off[b])             # own branch from y_{b,1}

    step_off = [0]
    for b in range(B):
        step_off.append(step_off[-1] + branch_len[b])
    R = step_off[-1]
    step_branch, step_pred, step_sample = [], [], []
    for b in range(B):
        t = branch_tree[b]
        for i in range(1, branch_len[b] + 1):
            step_branch.append(b)
            if i == 1:
                step_pred.append(tree_off[t] + anchors[b])  # the anchor row predicts y_{b,1}
            else:
                step_pred.append(branch_off[b] + i - 2)     # the row of y_{b,i-1} predicts y_{b,i}
            step_sample.append(branch_off[b] + i - 1 if i < branch_len[b] else -1)

    i32 = lambda x: np.asarray(x, dtype=np.int32)
    col = lambda k: i32([r[k] for r in rows])
    return dict(
        n_trees=n_trees, n_branches=B, n_rows=N, n_steps=R,
        max_branch_len=max(branch_len) if B else 0,
        max_pos=max((r[3] for r in rows), default=-1),
        tree_off=i32(tree_off),
        row_tree=col(0), row_branch=col(1), row_anchor=col(2), row_pos=col(3), row_depth=col(4),
        row_trunk_hi=i32(row_trunk_hi), row_branch_lo=i32(row_branch_lo),
        branch_tree=i32(branch_tree), branch_anchor=i32(anchors), branch_len=i32(branch_len),
        branch_off=i32(branch_off), step_off=i32(step_off), branch_order=i32(branch_order),
        step_branch=i32(step_branch), step_pred_row=i32(step_pred), step_sample_row=i32(step_sample),
    )


def parents_ref(layout):
    """Parent of every packed row from the tree's semantics, -1 for a trunk root.

    Trunk token j's parent is token j-1; y_{b,1}'s parent is its anchor; y_{b,i}'s
    parent is y_{b,i-1} ([SpecOPD notes page, "Equations"], histories h_{b,i}).
    Rows are located by (branch, depth) lookup, not by offset arithmetic.
    """
    N = layout["n_rows"]
    tree_off = layout["tree_off"]
    where = {}
    for r in range(N):
        if layout["row_branch"][r] >= 0:
            where[(int(layout["row_branch"][r]), int(layout["row_depth"][r]))] = r
    par = np.full(N, -1, dtype=np.int64)
    for r in range(N):
        t, b, d = int(layout["row_tree"][r]), int(layout["row_branch"][r]), int(layout["row_depth"][r])
        if b < 0:
            par[r] = r - 1 if r > tree_off[t] else -1
        elif d == 1:
            par[r] = int(tree_off[t]) + int(layout["row_anchor"][r])
        else:
            par[r] = where[(b, d - 1)]
    return par


def visible_ref(layout):
    """Dense visibility mask [N, N]: row r sees itself and its ancestors.

    [SpecOPD paper page, Figure 3]: the tree mask restricts each row to itself
    and its ancestors. Built by walking the parent chain; meant for N <= ~8k.
    """
    par = parents_ref(layout)
    N = len(par)
    mask = np.zeros((N, N), dtype=bool)
    for r in range(N):
        c = r
        while c >= 0:
            mask[r, c] = True
            c = par[c]
    return mask


def visible_intervals_ref(layout, r):
    """Visible packed rows of row r as the union of two index ranges.

    The trunk prefix [tree_off, row_trunk_hi] and the own-branch run
    [row_branch_lo, r]. Pinned against ``visible_ref`` by the oracle tests.
    """
    t = int(layout["row_tree"][r])
    lo = int(layout["tree_off"][t])
    hi = int(layout["row_trunk_hi"][r])
    blo = int(layout["row_branch_lo"][r])
    return np.concatenate([np.arange(lo, hi + 1), np.arange(blo, r + 1)]).astype(np.int64)
