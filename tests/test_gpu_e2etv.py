"""GPU parity: spec_e2etv_fwd_bwd against the float64 oracle."""
import numpy as np
import pytest

from _util import (ALPHA_RTOL, LOSS_ATOL, LOSS_RTOL, Case, check_grad_rows, from_device, say,
                   to_device, widen)
from oracle import e2etv_coef_ref, e2etv_grad_ref, e2etv_loss_ref, e2etv_ref, e2etv_row_stats_ref
from specgen import CONFIGS, gen_logit_rows, small_config

pytestmark = pytest.mark.gpu


def _pack(s):
    import tree_attention_spec_amd as tas
    return tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])


def _run(tree, z, y, inv_norm=0.0, grad=True):
    import torch
    import tree_attention_spec_amd as tas
    a, l, g = tas.spec_e2etv_fwd_bwd(tree, z, y, inv_norm=inv_norm, grad=grad)
    torch.cuda.synchronize()
    return a, l, g


def _full_compare(case, z, y, inv_norm=None):
    tree = _pack(case.s)
    a, l, g = _run(tree, to_device(z), to_device(y), inv_norm or 0.0)
    zz, yy = widen(z), widen(y)
    alpha, S, _, _, q, p = e2etv_row_stats_ref(zz, yy)
    L = e2etv_loss_ref(alpha, case.lay["step_off"], inv_norm)
    c = e2etv_coef_ref(alpha, case.lay["step_off"], inv_norm)
    gref = e2etv_grad_ref(q, p, S, c)
    ga, gl, gg = from_device(a), float(l.item()), from_device(g)
    arel = np.max(np.abs(ga - alpha) / np.maximum(alpha, 1e-30))
    lerr = abs(gl - L)
    gw, nt = check_grad_rows(gg, gref, q, p, c)
    say("  alpha rel %.2e, L %.8f vs %.8f, grad rel %.2e (%d near-ties skipped)" % (arel, gl, L, gw, nt))
    assert arel <= ALPHA_RTOL
    assert lerr <= max(LOSS_RTOL * abs(L), LOSS_ATOL)
    assert gw <= 1e-4
    return ga, gl, gg


def test_e2etv_teaching_example(golden):
    """The pages' teaching pair, through the GPU (vocab 3, -inf draft entry)."""
    say("e2etv parity: teaching example")
    gt = golden("teaching_example.json")
    with np.errstate(divide="ignore"):
        z = np.log(np.array([gt["draft_probs"]], np.float64)).astype(np.float32)
        y = np.log(np.array([gt["teacher_probs"]], np.float64)).astype(np.float32)
    tree = _pack(dict(trunk_len=np.array([4]), n_branches=np.array([1]), anchors=np.array([2], np.int32),
                      branch_len=np.array([1], np.int32)))
    a, l, g = _run(tree, to_device(z), to_device(y))
    assert abs(float(l.item()) - gt["loss"]) < 1e-6
    assert abs(float(a.item()) - gt["alpha"][0]) < 1e-6
    assert float(g[0, 2].item()) == 0.0


def test_e2etv_tiny_f32():
    say("e2etv parity: tiny fp32")
    case = Case(CONFIGS["tiny"])
    z, y = case.logits()
    _full_compare(case, z, y)


def test_e2etv_equal_and_nan():
    import torch
    say("e2etv: q == p and NaN padding")
    case = Case(small_config("tiny", branches=3, width=5, vocab=1000))
    z, y = case.logits()
    tree = _pack(case.s)
    zt = to_device(z)
    a, l, g = _run(tree, zt, zt.clone())
    assert torch.allclose(a, torch.ones_like(a), atol=2e-6, rtol=0)
    assert abs(float(l.item())) < 2e-6
    assert torch.count_nonzero(g).item() == 0
    zn = z.copy()
    zn[:, 900:] = np.nan
    zi = z.copy()
    zi[:, 900:] = -np.inf
    a1, l1, g1 = _run(tree, to_device(zn), to_device(y))
    a2, l2, g2 = _run(tree, to_device(zi), to_device(y))
    assert torch.equal(a1, a2) and torch.equal(l1, l2) and torch.equal(g1, g2)
    assert torch.count_nonzero(g1[:, 900:]).item() == 0
    _full_compare(case, zn, y)


@pytest.mark.parametrize("vocab", [151936, 50000, 4097])
def test_e2etv_bf16_rows(vocab):
    """Variable widths, full vocabulary rows, vector and scalar tails."""
    say("e2etv parity: bf16 vocab %d" % vocab)
    cfg = small_config("stress", trunk=500, branches=9, width=16, vocab=vocab)
    case = Case(cfg)
    z, y = case.logits()
    _full_compare(case, z, y)
    _full_compare(case, z, y, inv_norm=0.01)


def test_e2etv_bf16_nan_draft():
    """bf16 rows with NaN draft entries (scattered and whole blocks, quiet, signalling
    and negative NaN patterns) give the results of -inf entries."""
    import torch
    say("e2etv parity: bf16 NaN draft entries, vocab 151936")
    case = Case(small_config("gqa8b", trunk=300, branches=3, width=5, vocab=151936))
    z, y = case.logits()
    assert z.dtype == np.uint16
    rng = np.random.default_rng(5)
    zn = z.copy()
    pats = np.array([0x7FC0, 0x7F81, 0xFFC0, 0xFFFF], np.uint16)
    idx = rng.choice(zn.shape[1], 1000, replace=False)
    zn[0, idx] = pats[np.arange(idx.size) % 4]   # scattered
    zn[1, 100000:] = 0x7FC0                     # a tail block (whole slices)
    zn[2, :60000] = 0xFFC0                      # a head block
    isnan = (zn & 0x7FFF) > 0x7F80
    zi = np.where(isnan, np.uint16(0xFF80), zn).astype(np.uint16)
    tree = _pack(case.s)
    a1, l1, g1 = _run(tree, to_device(zn), to_device(y))
    a2, l2, g2 = _run(tree, to_device(zi), to_device(y))
    assert torch.equal(a1, a2) and torch.equal(l1, l2) and torch.equal(g1, g2)
    assert torch.count_nonzero(g1[1, 100000:]).item() == 0
    _full_compare(case, zi, y)


@pytest.mark.parametrize("width", [1, 2, 4])
def test_e2etv_bf16_few_rows(width):
    """A handful of rows: teams with one or two rows (pipeline prologue and tail)."""
    say("e2etv parity: bf16 vocab 151936, %d rows" % width)
    case = Case(small_config("gqa8b", trunk=64, branches=1, width=width, vocab=151936))
    z, y = case.logits()
    _full_compare(case, z, y)


def test_e2etv_status_word_after_calls():
    """The status word the fused kernel raises on a timed-out wait reads 0 after normal calls."""
    import torch
    import tree_attention_spec_amd as tas
    case = Case(small_config("gqa8b", trunk=300, branches=5, width=16, vocab=151936))
    z, y = case.logits()
    tree = _pack(case.s)
    work = torch.empty(tas.e2etv_work_bytes(tree, 151936, torch.bfloat16), dtype=torch.uint8, device="cuda")
    zt, yt = to_device(z), to_device(y)
    tas.spec_e2etv_fwd_bwd(tree, zt, yt, work=work)
    assert tas.spec_e2etv_status(tree, 151936, work) == 0


def test_e2etv_forward_only_and_determinism():
    import torch
    case = Case(small_config("gqa8b", trunk=300, branches=5, width=16, vocab=151936))
    z, y = case.logits()
    tree = _pack(case.s)
    zt, yt = to_device(z), to_device(y)
    a1, l1, g1 = _run(tree, zt, yt)
    a2, l2, g2 = _run(tree, zt, yt)
    a3, l3, g3 = _run(tree, zt, yt, grad=False)
    assert g3 is None
    assert torch.equal(a1, a2) and torch.equal(l1, l2) and torch.equal(g1, g2)
    assert torch.equal(a1, a3) and torch.equal(l1, l3)


def _oracle_stats_all(z, y, chunk=32):
    """Oracle alpha and S of every row, row chunks spread over the host's threads
    (NumPy releases the interpreter lock inside its array operations)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    R = z.shape[0]
    alpha, S = np.empty(R), np.empty(R)

    def run(r0):
        a, s_, _, _, _, _ = e2etv_row_stats_ref(widen(z[r0:r0 + chunk]), widen(y[r0:r0 + chunk]))
        alpha[r0:r0 + chunk], S[r0:r0 + chunk] = a, s_

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(run, range(0, R, chunk)))
    return alpha, S


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gqa8b", "long", "batched", "stress"])
def test_e2etv_workload_full(name):
    """Full-size workloads in the benchmarked launch: every step's alpha against the oracle,
    the oracle's own L (from its alphas) against the GPU's, and sampled gradient rows with
    the oracle's coefficients."""
    import torch
    say("e2etv parity: %s full size, every alpha" % name)
    case = Case(CONFIGS[name])
    tree = _pack(case.s)
    z, y = case.logits()
    zt, yt = to_device(z), to_device(y)
    a, l, g = _run(tree, zt, yt)
    del zt, yt
    R = case.R
    ga = from_device(a)
    alpha, _ = _oracle_stats_all(z, y)
    case.drop_logits()
    del z, y
    arel = np.max(np.abs(ga - alpha) / alpha)
    L = e2etv_loss_ref(alpha, case.lay["step_off"])
    c_all = e2etv_coef_ref(alpha, case.lay["step_off"])
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, R - 1], rng.choice(R, size=30, replace=False)]))
    zs, ys = gen_logit_rows(case.cfg, R, rows)
    _, S, _, _, q, p = e2etv_row_stats_ref(zs.astype(np.float64), ys.astype(np.float64))
    gref = e2etv_grad_ref(q, p, S, c_all[rows])
    gg = from_device(g[torch.from_numpy(rows).cuda()])
    gw, nt = check_grad_rows(gg, gref, q, p, c_all[rows])
    say("  %d alphas: max rel %.2e; L %.7f vs oracle %.7f; %d grad rows rel %.2e (%d near-ties)"
        % (R, arel, l.item(), L, len(rows), gw, nt))
    assert arel <= ALPHA_RTOL
    assert abs(l.item() - L) <= max(LOSS_RTOL * abs(L), LOSS_ATOL)
    assert gw <= 1e-4
    assert torch.isfinite(g).all()


@pytest.mark.parametrize("recipe", ["stress", "gqa8b"])
def test_e2etv_fused_pipeline_depth(recipe):
    """Enough steps (R >= 256 over the fused kernel's 25 teams at vocabulary 151936) that
    every team runs its pipeline at full depth for many rows, with branches that cross from
    the last team to the first: every alpha, the oracle's own L and every gradient row
    against the oracle."""
    import tree_attention_spec_amd as tas
    say("e2etv parity: fused pipeline depth, %s recipe" % recipe)
    if recipe == "stress":
        cfg = small_config("stress", trunk=3000, branches=72, width=16, vocab=151936)
    else:
        cfg = small_config("gqa8b", trunk=2000, branches=40, width=16, vocab=151936)
    case = Case(cfg)
    assert case.R >= 256, case.R
    z, y = case.logits()
    tm = tas.KernelTimer(capacity=16)
    with tm:
        _full_compare(case, z, y)
    names = [n for n, _ in tm.durations()]
    assert "e2etv_fused" in names, names


def test_e2etv_long_branches_multipass():
    """Long branches (40 steps) through the same kernels; same contract."""
    say("e2etv parity: bf16, branches up to 40 steps")
    cfg = small_config("stress", trunk=400, branches=6, width=40, vocab=151936)
    case = Case(cfg)
    assert case.lay["max_branch_len"] > 16
    z, y = case.logits()
    _full_compare(case, z, y)


def test_e2etv_branch_lengths_at_path_limits():
    """Branches of 1, 26, 27 and 64 steps (the ABI maximum) in one tree, V = 151,936 bf16:
    the fused cooperative path takes a branch of at most one step more than its team
    count (25 on MI355X at this vocabulary), the three-kernel path the rest; every row
    matches the oracle either way."""
    import numpy as np
    say("e2etv parity: branch lengths 1, 26, 27, 64")
    s = dict(trunk_len=np.array([300], np.int32), n_branches=np.array([4], np.int32),
             anchors=np.array([20, 150, 151, 299], np.int32), branch_len=np.array([1, 26, 27, 64], np.int32))
    case = Case(small_config("gqa8b", vocab=151936), structure=s)
    assert case.lay["max_branch_len"] == 64
    z, y = case.logits()
    _full_compare(case, z, y)
    for w in (26, 27):
        s1 = dict(trunk_len=np.array([300], np.int32), n_branches=np.array([2], np.int32),
                  anchors=np.array([40, 200], np.int32), branch_len=np.array([w, 3], np.int32))
        c1 = Case(small_config("gqa8b", vocab=151936), structure=s1)
        z1, y1 = c1.logits()
        _full_compare(c1, z1, y1)
