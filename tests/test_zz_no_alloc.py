"""GPU check of spec_e2etv_fwd_bwd_noalloc: the no-allocation entry point gives the
results of spec_e2etv_fwd_bwd (same kernels) on consecutive calls, the second smaller
than the first, so the shared library-owned array holds the first call's contents when
the second starts."""
import numpy as np
import pytest

from _util import ALPHA_RTOL, LOSS_ATOL, LOSS_RTOL, Case, from_device, say, to_device
from specgen import small_config

pytestmark = pytest.mark.gpu


def _both(case, z, y, inv_norm=0.0):
    import torch
    import tree_attention_spec_amd as tas
    s = case.s
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    zt, yt = to_device(z), to_device(y)
    R, V = zt.shape
    a0, l0, g0 = tas.spec_e2etv_fwd_bwd(tree, zt, yt, inv_norm=inv_norm)
    a1 = torch.full((R,), float("nan"), dtype=torch.float32, device=zt.device)
    l1 = torch.full((1,), float("nan"), dtype=torch.float32, device=zt.device)
    g1 = torch.full((R, V), float("nan"), dtype=torch.float32, device=zt.device)
    torch.cuda.synchronize()
    tas.spec_e2etv_fwd_bwd_noalloc(tree, zt, yt, inv_norm=inv_norm, alpha_out=a1, loss_out=l1, grad_out=g1)
    torch.cuda.synchronize()
    return (a0, l0, g0), (a1, l1, g1)


def _check(ref, got):
    import torch
    (a0, l0, g0), (a1, l1, g1) = ref, got
    ga0, ga1 = from_device(a0), from_device(a1)
    arel = np.max(np.abs(ga1 - ga0) / np.maximum(ga0, 1e-30))
    lerr = abs(float(l1.item()) - float(l0.item()))
    gg0, gg1 = from_device(g0), from_device(g1)
    scale = np.maximum(np.abs(gg0).max(axis=1), 1e-300)
    grel = float(np.max(np.abs(gg1 - gg0).max(axis=1) / scale))
    same = torch.equal(a0, a1) and torch.equal(l0, l1) and torch.equal(g0, g1)
    say("  alpha rel %.2e, L diff %.2e, grad rel %.2e, bitwise equal %s" % (arel, lerr, grel, same))
    assert arel <= ALPHA_RTOL
    assert lerr <= max(LOSS_RTOL * abs(float(l0.item())), LOSS_ATOL)
    assert grel <= 1e-4


def test_noalloc_matches_workspace_call_twice():
    say("e2etv no-allocation entry: two calls in a row, the second smaller")
    # first call: 151936-entry bf16 rows on the fused pipeline, several hundred steps
    big = Case(small_config("stress", trunk=3000, branches=40, width=16, vocab=151936))
    z, y = big.logits()
    _check(*_both(big, z, y))
    # second call: fewer steps and a shorter vocabulary, with a caller normaliser
    small = Case(small_config("gqa8b", trunk=300, branches=5, width=6, vocab=50000))
    z, y = small.logits()
    assert small.R < big.R
    _check(*_both(small, z, y, inv_norm=0.01))


def test_noalloc_fallback_path_with_bitmask():
    """float32 logits take the statistics/scan/gradient kernels, which keep the {q < p}
    bitmask in the library's array."""
    say("e2etv no-allocation entry: float32 rows (bitmask path)")
    case = Case(small_config("tiny", branches=6, width=5, vocab=3000))
    z, y = case.logits()
    assert z.dtype == np.float32
    _check(*_both(case, z, y))
