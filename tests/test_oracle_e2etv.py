"""Pins for the E2E-TV oracle: the pages' teaching example, closed forms,
invariants and central finite differences."""
import numpy as np
import pytest

from oracle import e2etv_coef_ref, e2etv_grad_ref, e2etv_loss_ref, e2etv_ref, e2etv_row_stats_ref
from specgen import bf16_bits_to_f32, f32_to_bf16_bits, gen_logits, get_config


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def test_teaching_example(golden):
    g = golden("teaching_example.json")
    z = _log(g["draft_probs"])[None]           # the zero-probability entry is a -inf logit
    y = _log(g["teacher_probs"])[None]
    step_off = np.concatenate([[0], np.cumsum(g["branch_widths"])])
    alpha, L, grad, _ = e2etv_ref(z, y, step_off)
    assert alpha.tolist() == pytest.approx(g["alpha"], abs=1e-15)
    assert L == pytest.approx(g["loss"], abs=1e-15)
    # negative control: renormalising the teacher onto the draft support loses its outside mass
    p = np.asarray(g["teacher_probs"])
    support = np.asarray(g["draft_probs"]) > 0
    y_renorm = _log(np.where(support, p / p[support].sum(), 0.0))[None]
    _, L_bad, _, _ = e2etv_ref(z, y_renorm, step_off)
    assert L_bad == pytest.approx(g["loss_if_teacher_renormalised"], abs=1e-15)
    assert grad[0, 2] == 0.0                   # no gradient on inactive support


def test_hand_worked_two_step_branch():
    # q = softmax([0, ln 2]) = [1/3, 2/3], p = [1/2, 1/2] -> alpha = 1/3 + 1/2 = 5/6, S = 1/3
    z = np.array([[0.0, np.log(2.0)], [0.0, 0.0]])
    y = np.array([[0.0, 0.0], [0.0, 0.0]])
    alpha, L, grad, S = e2etv_ref(z, y, [0, 2])
    assert alpha == pytest.approx([5 / 6, 1.0], abs=1e-15)
    assert S[0] == pytest.approx(1 / 3, abs=1e-15)
    assert L == pytest.approx(1 - (5 / 6 + 5 / 6) / 2, abs=1e-15)
    # dL/dalpha_1 = -(1/2)(1 + alpha_2) = -1; d alpha_1/dz = q * (1[q<p] - S) = [1/3*(2/3), 2/3*(-1/3)]
    assert grad[0] == pytest.approx([-(1 / 3) * (2 / 3), (2 / 3) * (1 / 3)], abs=1e-15)


def test_equal_distributions():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((6, 50)) * 2
    # identical logits: q == p exactly, the strict set {q < p} is empty, the gradient is exactly 0
    alpha, L, grad, S = e2etv_ref(z, z.copy(), [0, 2, 6])
    np.testing.assert_allclose(alpha, 1.0, atol=1e-14)
    assert abs(L) < 1e-14
    assert np.all(S == 0.0) and np.all(grad == 0.0)
    # a constant shift gives the same distribution up to rounding: alpha = 1 and L = 0 still hold
    # (the gradient is then a subgradient picked by rounding noise, so it is not checked here)
    alpha, L, _, _ = e2etv_ref(z, z + 7.0, [0, 2, 6])
    np.testing.assert_allclose(alpha, 1.0, atol=1e-14)
    assert abs(L) < 1e-14


def test_ranges_and_row_sums():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((12, 64)) * 3
    y = rng.standard_normal((12, 64)) * 3
    alpha, L, grad, S = e2etv_ref(z, y, [0, 4, 5, 12])
    assert np.all((alpha >= 0) & (alpha <= 1)) and 0 <= L <= 1
    assert np.all((S >= 0) & (S <= alpha + 1e-15))
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-16)


@pytest.mark.parametrize("W,k,x", [(5, 1, 0.3), (5, 3, 0.3), (5, 5, 0.3), (8, 2, 0.0)])
def test_early_mismatch_costs_more(W, k, x):
    alpha = np.ones(W)
    alpha[k - 1] = x
    L = e2etv_loss_ref(alpha, [0, W])
    assert L == pytest.approx((1 - x) * (W - k + 1) / W, abs=1e-15)


def test_early_mismatch_is_monotone():
    W = 6
    Ls = []
    for k in range(1, W + 1):
        alpha = np.ones(W)
        alpha[k - 1] = 0.5
        Ls.append(e2etv_loss_ref(alpha, [0, W]))
    assert all(a > b for a, b in zip(Ls, Ls[1:]))


def test_coefficients_match_direct_derivative():
    rng = np.random.default_rng(2)
    alpha = rng.uniform(0, 1, size=11)
    alpha[3] = 0.0                             # an exact zero must not break anything
    step_off = [0, 4, 5, 11]
    c = e2etv_coef_ref(alpha, step_off)
    R = step_off[-1]
    for b in range(len(step_off) - 1):
        s0, s1 = step_off[b], step_off[b + 1]
        for i in range(s0, s1):
            d = sum(np.prod([alpha[m] for m in range(s0, j + 1) if m != i]) for j in range(i, s1))
            assert c[i] == pytest.approx(-d / R, abs=1e-15)
    # and against finite differences of the loss in alpha
    h = 1e-7
    for i in range(R):
        ap, am = alpha.copy(), alpha.copy()
        ap[i] += h
        am[i] -= h
        fd = (e2etv_loss_ref(ap, step_off) - e2etv_loss_ref(am, step_off)) / (2 * h)
        assert c[i] == pytest.approx(fd, abs=1e-8)


def test_single_step_closed_form():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((3, 40))
    y = rng.standard_normal((3, 40))
    alpha, L, grad, S = e2etv_ref(z, y, [0, 1, 2, 3], inv_norm=0.25)
    q = np.exp(z - z.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    p = np.exp(y - y.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = -0.25 * q * ((q < p) - S[:, None])
    np.testing.assert_allclose(grad, want, atol=1e-16)
    assert L == pytest.approx(1 - 0.25 * alpha.sum(), abs=1e-15)


def test_finite_difference_gradcheck():
    rng = np.random.default_rng(4)
    V = 12
    z = rng.standard_normal((7, V)) * 1.5
    y = rng.standard_normal((7, V)) * 1.5
    step_off = [0, 3, 4, 7]
    _, _, grad, _ = e2etv_ref(z, y, step_off)
    h = 1e-6
    fd = np.zeros_like(z)
    for r in range(z.shape[0]):
        for u in range(V):
            zp, zm = z.copy(), z.copy()
            zp[r, u] += h
            zm[r, u] -= h
            fd[r, u] = (e2etv_ref(zp, y, step_off, want_grad=False)[1]
                        - e2etv_ref(zm, y, step_off, want_grad=False)[1]) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-10)


def test_teacher_is_held_fixed():
    """Moving the teacher changes alpha but the gradient formula only ever differentiates the draft."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal((2, 9))
    y = rng.standard_normal((2, 9))
    step_off = [0, 2]
    _, _, g1, _ = e2etv_ref(z, y, step_off)
    h = 1e-6
    zp = z + h * g1 / np.linalg.norm(g1)
    # a step along the gradient raises the loss by ~h*|g| (first order), teacher untouched
    d = e2etv_ref(zp, y, step_off, want_grad=False)[1] - e2etv_ref(z, y, step_off, want_grad=False)[1]
    assert d == pytest.approx(h * np.linalg.norm(g1), rel=1e-4)


def test_nan_padding_is_inactive_support():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((2, 10))
    y = rng.standard_normal((2, 10))
    z_nan, z_inf = z.copy(), z.copy()
    z_nan[:, 7:] = np.nan
    z_inf[:, 7:] = -np.inf
    a1, L1, g1, _ = e2etv_ref(z_nan, y, [0, 2])
    a2, L2, g2, _ = e2etv_ref(z_inf, y, [0, 2])
    assert np.array_equal(a1, a2) and L1 == L2 and np.array_equal(g1, g2)
    assert np.all(g1[:, 7:] == 0.0)
    # the teacher mass on the padded entries is not renormalised away
    _, _, _, _, q, p = e2etv_row_stats_ref(z_nan, y)
    assert np.all(a1 <= 1 - p[:, 7:].sum(axis=1) + 1e-15)


def test_low_precision_inputs_are_promoted():
    """bf16 logits widen exactly; the float64 statistics of the widened values differ
    from a float32 evaluation by no more than float32 rounding."""
    cfg = get_config("tiny")
    z, y = gen_logits(cfg, 4)
    zb = bf16_bits_to_f32(f32_to_bf16_bits(z)).astype(np.float64)
    yb = bf16_bits_to_f32(f32_to_bf16_bits(y)).astype(np.float64)
    a64, _, _, _, _, _ = e2etv_row_stats_ref(zb, yb)
    z32, y32 = zb.astype(np.float32), yb.astype(np.float32)
    q32 = np.exp(z32 - z32.max(1, keepdims=True))
    q32 /= q32.sum(1, keepdims=True, dtype=np.float32)
    p32 = np.exp(y32 - y32.max(1, keepdims=True))
    p32 /= p32.sum(1, keepdims=True, dtype=np.float32)
    a32 = np.minimum(q32, p32).sum(1, dtype=np.float32)
    np.testing.assert_allclose(a32, a64, rtol=1e-5)


def test_gradient_check_bound():
    """The GPU tests' gradient check (test infrastructure): a few float32 ulps of error in
    the S a row is formed from pass only through the |c| max q floor, which a real error
    (a wrong coefficient, a flipped indicator) does not reach."""
    from _util import check_grad_rows
    q = np.array([[1 - 2e-5, 1.5e-5, 5e-6]])          # draft almost certain of token 0
    p = np.array([[1 - 1e-6, 5e-7, 5e-7]])            # teacher more so: only token 0 has q < p
    S = np.array([q[0, 0]])
    c = np.array([-0.3])
    g = e2etv_grad_ref(q, p, S, c)
    assert np.abs(g).max() < 1e-4 * abs(c[0])          # a row of size |c| (1 - S)
    g_ulps = e2etv_grad_ref(q, p, S + 4 * 2.0 ** -24, c)   # S off by four float32 ulps of 1
    assert check_grad_rows(g_ulps, g, q, p)[0] > 1e-4      # fails the plain normwise bound
    assert check_grad_rows(g_ulps, g, q, p, c)[0] <= 1e-4  # within the floor
    g_off = e2etv_grad_ref(q, p, S + 1e-5, c)              # S off by ~80 ulps
    assert check_grad_rows(g_off, g, q, p, c)[0] > 1e-4
    flip = g.copy()
    flip[0, 1] = -flip[0, 1] + c[0] * q[0, 1]               # token 1 taken as inside {q < p}
    assert check_grad_rows(flip, g, q, p, c)[0] > 1e-4
    q2 = np.array([[0.5, 0.3, 0.2]])
    p2 = np.array([[0.2, 0.5, 0.3]])
    S2 = np.array([0.5])
    g2 = e2etv_grad_ref(q2, p2, S2, c)
    assert check_grad_rows(e2etv_grad_ref(q2, p2, S2 + 1e-3, c), g2, q2, p2, c)[0] > 1e-4
    assert check_grad_rows(e2etv_grad_ref(q2, p2, S2, 1.01 * c), g2, q2, p2, c)[0] > 1e-4  # 1% in c
    assert check_grad_rows(e2etv_grad_ref(q2, p2, S2 + 4 * 2.0 ** -24, c), g2, q2, p2, c)[0] <= 1e-4
