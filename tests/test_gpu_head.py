"""GPU parity: spec_e2etv_head_fwd_bwd (teacher logits through an output head) against the
float64 oracle."""
import numpy as np
import pytest

from _util import (ALPHA_RTOL, LOSS_ATOL, LOSS_RTOL, Case, check_grad_rows, from_device, say,
                   to_device, widen)
from oracle import e2etv_coef_ref, e2etv_grad_ref, e2etv_loss_ref, e2etv_row_stats_ref, head_logits_ref
from specgen import CONFIGS, gen_head, gen_head_draft_rows, small_config

pytestmark = pytest.mark.gpu


def _pack(s):
    import tree_attention_spec_amd as tas
    return tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])


def _inputs(case, d, V, draft_f32=False, nan_frac=0.0, seed=0, logit_std=3.0):
    inp = gen_head(seed, case.N, d, V, case.R, logit_std)
    draft = inp["draft"]
    if draft_f32 or nan_frac:
        draft = widen(draft).astype(np.float32)
        if nan_frac:
            rng = np.random.default_rng(seed + 7)
            draft[rng.random(draft.shape) < nan_frac] = np.nan
    return draft, inp["hidden"], inp["head"]


def _compare(case, d, V, **kw):
    import torch
    import tree_attention_spec_amd as tas
    draft, hidden, head = _inputs(case, d, V, **kw)
    tree = _pack(case.s)
    a, l, g = tas.spec_e2etv_head_fwd_bwd(tree, to_device(draft), to_device(hidden), to_device(head))
    torch.cuda.synchronize()
    y = head_logits_ref(case.lay, widen(hidden), widen(head))
    alpha, S, _, _, q, p = e2etv_row_stats_ref(widen(draft), y)
    L = e2etv_loss_ref(alpha, case.lay["step_off"])
    c = e2etv_coef_ref(alpha, case.lay["step_off"])
    gref = e2etv_grad_ref(q, p, S, c)
    ga, gl, gg = from_device(a), float(l.item()), from_device(g)
    arel = np.max(np.abs(ga - alpha) / np.maximum(alpha, 1e-30))
    gw, nt = check_grad_rows(gg, gref, q, p, c)
    say("  R %d V %d d %d: alpha rel %.2e, L %.8f vs %.8f, grad rel %.2e (%d near-ties)"
        % (case.R, V, d, arel, gl, L, gw, nt))
    assert arel <= ALPHA_RTOL
    assert abs(gl - L) <= max(LOSS_RTOL * abs(L), LOSS_ATOL)
    assert gw <= 1e-4
    return a, l, g


def test_head_tiny():
    say("e2etv head parity: tiny tree, V 512, d 64")
    _compare(Case(CONFIGS["tiny"]), 64, 512)


def test_head_ragged_tiles_f32_draft_with_nan():
    """Steps, vocabulary and hidden size all off the tile grid; fp32 draft with NaN padding."""
    say("e2etv head parity: ragged tiles, fp32 draft with NaN padding")
    case = Case(small_config("stress", trunk=500, branches=40, width=16, vocab=1000))
    assert case.R % 128 and 1000 % 128
    _compare(case, 192, 1000, draft_f32=True, nan_frac=0.02)


def test_head_several_tiles_bf16():
    say("e2etv head parity: several tile groups, bf16 draft")
    case = Case(small_config("gqa8b", trunk=700, branches=45, width=16, vocab=4104))
    assert case.R > 8 * 64
    _compare(case, 256, 4104)


def test_head_long_branches():
    """Branches of up to 40 steps. Logits of spread 0.5 keep alpha near 0.8: with independent
    logits of spread 3 (alpha ~ 0.03) the prefix products of late steps fall below float32's
    range, where dL/d alpha (a float32 output) is zero while the float64 oracle is not."""
    say("e2etv head parity: branches up to 40 steps")
    case = Case(small_config("stress", trunk=400, branches=6, width=40, vocab=2048))
    assert case.lay["max_branch_len"] > 16
    _compare(case, 128, 2048, logit_std=0.5)


def test_head_forward_only_and_determinism():
    import torch
    import tree_attention_spec_amd as tas
    say("e2etv head: forward only matches, repeated calls are bitwise equal")
    case = Case(small_config("gqa8b", trunk=300, branches=20, width=8, vocab=2048))
    draft, hidden, head = (to_device(x) for x in _inputs(case, 128, 2048))
    tree = _pack(case.s)
    a1, l1, g1 = tas.spec_e2etv_head_fwd_bwd(tree, draft, hidden, head)
    a2, l2, _ = tas.spec_e2etv_head_fwd_bwd(tree, draft, hidden, head, grad=False)
    a3, l3, g3 = tas.spec_e2etv_head_fwd_bwd(tree, draft, hidden, head)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(l1, l2)
    assert torch.equal(a1, a3) and torch.equal(l1, l3) and torch.equal(g1, g3)
    # each gradient row sums to zero (the same set {q < p} defines S and the indicator)
    assert g1.double().sum(dim=1).abs().max().item() < 1e-9


def test_head_matches_supplied_logit_path():
    """The same teacher logits, handed over as a tensor, through spec_e2etv_fwd_bwd."""
    import torch
    import tree_attention_spec_amd as tas
    say("e2etv head vs supplied float32 teacher logits")
    case = Case(small_config("gqa8b", trunk=300, branches=20, width=8, vocab=2048))
    draft, hidden, head = _inputs(case, 128, 2048, draft_f32=True)
    y = head_logits_ref(case.lay, widen(hidden), widen(head)).astype(np.float32)
    tree = _pack(case.s)
    a, l, _ = tas.spec_e2etv_head_fwd_bwd(tree, to_device(draft), to_device(hidden), to_device(head))
    a2, l2, _ = tas.spec_e2etv_fwd_bwd(tree, to_device(draft), to_device(y))
    torch.cuda.synchronize()
    assert np.max(np.abs(from_device(a) - from_device(a2)) / from_device(a2)) <= 2 * ALPHA_RTOL


def test_head_many_step_tiles():
    """R >= 256 steps (three 128-step tiles) at vocabulary 151936: every alpha, the oracle's
    own L and every gradient row against the oracle."""
    say("e2etv head parity: R >= 256 steps, vocabulary 151936")
    case = Case(small_config("gqa8b", trunk=2000, branches=20, width=16, vocab=151936))
    assert case.R >= 256
    _compare(case, 128, 151936)


@pytest.mark.slow
def test_head_gqa8b_full():
    """Full size (4096 steps, vocabulary 151936, hidden 4096): every step's alpha against the
    oracle (head product in float64, row blocks), the oracle's own L, and sampled gradient
    rows with the oracle's coefficients."""
    import torch
    import tree_attention_spec_amd as tas
    say("e2etv head parity: gqa8b full size, every alpha")
    cfg = CONFIGS["gqa8b"]
    case = Case(cfg)
    d, V = cfg.hq * cfg.head_dim, cfg.vocab
    inp = gen_head(0, case.N, d, V, case.R)
    tree = _pack(case.s)
    a, l, g = tas.spec_e2etv_head_fwd_bwd(tree, to_device(inp["draft"]), to_device(inp["hidden"]),
                                          to_device(inp["head"]))
    torch.cuda.synchronize()
    R = case.R
    hidden = widen(inp["hidden"])
    head = widen(inp["head"])
    alpha = np.empty(R)
    for r0 in range(0, R, 256):
        steps = np.arange(r0, min(R, r0 + 256))
        y = head_logits_ref(case.lay, hidden, head, steps=steps)
        alpha[steps] = e2etv_row_stats_ref(widen(inp["draft"][steps]), y)[0]
    ga = from_device(a)
    arel = np.max(np.abs(ga - alpha) / alpha)
    L = e2etv_loss_ref(alpha, case.lay["step_off"])
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, R - 1, 127, 128], rng.choice(R, size=12, replace=False)]))
    y = head_logits_ref(case.lay, hidden, head, steps=rows)
    z = widen(gen_head_draft_rows(0, R, V, rows))
    _, S, _, _, q, p = e2etv_row_stats_ref(z, y)
    c = e2etv_coef_ref(alpha, case.lay["step_off"])[rows]
    gref = e2etv_grad_ref(q, p, S, c)
    gw, nt = check_grad_rows(from_device(g[torch.from_numpy(rows).cuda()]), gref, q, p, c)
    say("  %d alphas: max rel %.2e; L %.7f vs oracle %.7f; %d grad rows rel %.2e (%d near-ties)"
        % (R, arel, l.item(), L, len(rows), gw, nt))
    assert arel <= ALPHA_RTOL
    assert abs(l.item() - L) <= max(LOSS_RTOL * abs(L), LOSS_ATOL)
    assert gw <= 1e-4
    assert torch.isfinite(g).all()
