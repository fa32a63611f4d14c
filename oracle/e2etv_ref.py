"""Oracle: the E2E-TV surrogate, its loss and its gradient (test infrastructure only).

Sources:
  * [SpecOPD notes page, "Equations"]: alpha_{b,i} = sum_v min(q(v|h), p(v|h))
    over the full vocabulary and L = 1 - (1/(BW)) sum_b sum_{j=1..W}
    prod_{i<=j} alpha_{b,i}; samples and teacher distributions are held fixed
    when differentiating; teacher mass outside the draft support is kept,
    never renormalised away.
  * [SpecOPD notes page, "Inputs and code mapping"]: logits are aligned by
    history; low-precision inputs are promoted; inactive draft support may be
    NaN padding; the teacher must be finite everywhere.
  * [SpecOPD notes page, "Checks, negative controls, and limits"]: the teaching
    pair q = [.5, .5, 0] against p = [.4, .4, .2] gives loss 0.2.

Readings: a NaN or -inf draft logit means q = 0 there; with variable branch
widths or several trees the normaliser 1/(BW) becomes 1/sum_b W_b unless the
caller passes another; at an exact tie q_v = p_v the one-sided derivative with
the strict test q_v < p_v is taken.

Derivative used (samples and teacher fixed): for a row with draft softmax q
and M = {v : q_v < p_v}, d alpha / d z_u = q_u * (1[u in M] - S) with
S = sum_{v in M} q_v; dL/d z = (dL/d alpha) * d alpha / d z.
"""
from __future__ import annotations

import numpy as np


def _lse(x):
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def e2etv_row_stats_ref(draft, teacher):
    """Per-row statistics in float64.

    Returns (alpha, S, lse_q, lse_p, q, p) for rows of draft logits z and
    teacher logits y ([k, V] each). q = softmax(z) with NaN/-inf entries as 0,
    p = softmax(y) over the full vocabulary (no renormalisation).
    """
    z = np.array(draft, dtype=np.float64, copy=True)
    z[np.isnan(z)] = -np.inf
    y = np.asarray(teacher, dtype=np.float64)
    lq = _lse(z)
    lp = _lse(y)
    q = np.exp(z - lq[:, None])
    p = np.exp(y - lp[:, None])
    alpha = np.minimum(q, p).sum(axis=-1)
    S = np.where(q < p, q, 0.0).sum(axis=-1)
    return alpha, S, lq, lp, q, p


def _norm(step_off, inv_norm):
    R = int(step_off[-1])
    return 1.0 / R if (inv_norm is None or inv_norm <= 0) else float(inv_norm)


def e2etv_loss_ref(alpha, step_off, inv_norm=None):
    """L = 1 - inv_norm * sum_b sum_j prod_{i<=j} alpha_{b,i}, by the direct double loop."""
    alpha = np.asarray(alpha, dtype=np.float64)
    total = 0.0
    for b in range(len(step_off) - 1):
        s0, s1 = int(step_off[b]), int(step_off[b + 1])
        for j in range(s0, s1):
            total += float(np.prod(alpha[s0:j + 1]))
    return 1.0 - _norm(step_off, inv_norm) * total


def e2etv_coef_ref(alpha, step_off, inv_norm=None):
    """c_s = dL/d alpha_s for every step, by prefix products A and suffix sums G.

    With A_0 = 1, A_i = A_{i-1} alpha_i and G_W = 1, G_i = 1 + alpha_{i+1} G_{i+1}
    (per branch), dL/d alpha_i = -inv_norm * A_{i-1} * G_i; no division, so
    alpha = 0 is exact.
    """
    alpha = np.asarray(alpha, dtype=np.float64)
    c = np.zeros_like(alpha)
    w = _norm(step_off, inv_norm)
    for b in range(len(step_off) - 1):
        s0, s1 = int(step_off[b]), int(step_off[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        A = np.ones(n + 1)
        for i in range(1, n + 1):
            A[i] = A[i - 1] * alpha[s0 + i - 1]
        G = np.ones(n + 1)
        for i in range(n - 1, 0, -1):
            G[i] = 1.0 + alpha[s0 + i] * G[i + 1]
        for i in range(1, n + 1):
            c[s0 + i - 1] = -w * A[i - 1] * G[i]
    return c


def e2etv_grad_ref(q, p, S, c):
    """Gradient rows dL/dz = c_s * q * (1[q < p] - S_s)."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    return np.asarray(c)[:, None] * q * ((q < p).astype(np.float64) - np.asarray(S)[:, None])


def e2etv_ref(draft, teacher, step_off, inv_norm=None, want_grad=True):
    """Whole surrogate for small inputs: (alpha [R], L, grad [R,V] or None, S [R])."""
    alpha, S, _, _, q, p = e2etv_row_stats_ref(draft, teacher)
    L = e2etv_loss_ref(alpha, step_off, inv_norm)
    grad = None
    if want_grad:
        c = e2etv_coef_ref(alpha, step_off, inv_norm)
        grad = e2etv_grad_ref(q, p, S, c)
    return alpha, L, grad, S
