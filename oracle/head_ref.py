"""Oracle: E2E-TV with the teacher logits read through an output head (test infrastructure only).

Sources:
  * [SpecOPD notes page, "Inputs and code mapping"]: the prediction logits are
    formed from hidden states and a head that the caller supplies, and the
    E2E-TV objective consumes logits aligned by history.
  * [SpecOPD paper page, Figure 3] and [SpecOPD notes page, "Equations"]: the
    logits of step (b,i) come from the row of its predecessor (the anchor row
    for i = 1), never from the sample's own row.

Reading: the teacher logits of step s are the dot products of the predecessor
row's hidden state with every row of the head,
    y[s, v] = sum_k hidden[step_pred_row[s], k] * head[v, k],
and then enter E2E-TV exactly as supplied teacher logits do (full-vocabulary
softmax, teacher mass kept, draft logits supplied by the caller).
"""
from __future__ import annotations

import numpy as np

from .e2etv_ref import e2etv_ref


def head_logits_ref(layout, hidden, head, steps=None):
    """Teacher logits [R, V] (or only the rows ``steps``) in float64."""
    pred = np.asarray(layout["step_pred_row"], dtype=np.int64)
    if steps is not None:
        pred = pred[np.asarray(steps, dtype=np.int64)]
    h = np.asarray(hidden, dtype=np.float64)[pred]
    return h @ np.asarray(head, dtype=np.float64).T


def e2etv_head_ref(layout, hidden, head, draft, inv_norm=None, want_grad=True):
    """(alpha [R], L, grad [R, V] or None, S [R]) of E2E-TV on head-formed teacher logits."""
    y = head_logits_ref(layout, hidden, head)
    return e2etv_ref(draft, y, layout["step_off"], inv_norm, want_grad)
