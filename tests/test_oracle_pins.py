"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compares the oracle with itself: each checks it against a
closed form (spectral action of the quintic on singular values, exact
rational evaluation of f^5), an algebraic invariant, or hand arithmetic.
Sources: "Infra Optimizers" Background eq. (1)-(2) and "Scaling Up Muon"
eq. (3)-(4), Lemma 1; "Scaling Muon for Diffusion Transformers" 2.1 and 3.1;
"DMuon" 2.2 (Gram-space recursion)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon_oracle as O

HP = O.Hyper()
A_, B_, C_ = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ns5_scalar_values.txt")


def f5_exact(x: Fraction) -> Fraction:
    for _ in range(5):
        x = A_ * x + B_ * x ** 3 + C_ * x ** 5
    return x


def f5_float(x: float) -> float:
    return float(f5_exact(Fraction(x)))


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b))


def test_golden_scalar_values():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for x, v in rows:
        assert f5_float(float(Fraction(x))) == pytest.approx(float(v), rel=0, abs=1e-15)


@pytest.mark.parametrize("shape", [(4, 7), (7, 4), (8, 20), (16, 16), (3, 40)])
def test_ns5_matches_svd_closed_form(shape):
    # NS acts on each singular value by f five times: O = U diag(f^5(s/|M|_F)) V^T.
    rng = np.random.default_rng(100 + shape[0] * 31 + shape[1])
    M = rng.standard_normal(shape)
    X, tr = O.orient(M)
    out = O.unorient(O.ns5_direct(X), tr)
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    s = s / np.linalg.norm(M)
    expect = U @ np.diag([f5_float(v) for v in s]) @ Vt
    assert rel(out, expect) < 1e-12


@pytest.mark.parametrize("steps,coef", [(1, (3.4445, -4.7750, 2.0315)), (8, (3.4445, -4.7750, 2.0315)),
                                        (5, (2.0, -1.5, 0.5)), (10, (3.0, -3.2, 1.2))])
def test_other_iteration_counts_and_coefficients_follow_the_svd_closed_form(steps, coef):
    # Any count N and any odd quintic f(s) = a s + b s^3 + c s^5: both the
    # direct and the Gram routines act on each singular value by f, N times.
    a, b, c = coef
    hp = O.Hyper(ns_steps=steps, a=a, b=b, c=c)
    rng = np.random.default_rng(300 + steps)
    M = rng.standard_normal((6, 17))
    U, sv, Vt = np.linalg.svd(M, full_matrices=False)
    fs = []
    for v in sv / np.linalg.norm(M):
        for _ in range(steps):
            v = a * v + b * v ** 3 + c * v ** 5
        fs.append(v)
    expect = U @ np.diag(fs) @ Vt
    assert rel(O.ns5_direct(M, hp), expect) < 1e-12
    assert rel(O.ns5_gram(M, hp), expect) < 1e-10


def test_ns5_rank_one_gives_f5_of_one():
    rng = np.random.default_rng(1)
    u, v = rng.standard_normal(9), rng.standard_normal(23)
    M = np.outer(u, v)
    X0 = M / np.linalg.norm(M)
    out = O.ns5_direct(M)
    assert rel(out, 0.6964364094697528 * X0) < 1e-13


@pytest.mark.parametrize("r", [4, 16])
def test_ns5_scaled_orthogonal(r):
    rng = np.random.default_rng(r)
    Qm, _ = np.linalg.qr(rng.standard_normal((r, r)))
    out = O.ns5_direct(5.0 * Qm)  # normalised singular values are 1/sqrt(r)
    expect = f5_float(1.0 / math.sqrt(r)) * Qm
    assert rel(out, expect) < 1e-13
    golden = {4: 0.7654385304543384, 16: 0.7145262613330345}[r]
    assert f5_float(1.0 / math.sqrt(r)) == pytest.approx(golden, abs=1e-15)


def test_ns5_diagonal_is_elementwise_and_odd():
    d = np.array([3.0, -1.0, 0.5, -0.25, 2.0])
    out = O.ns5_direct(np.diag(d))
    dn = d / np.linalg.norm(d)
    expect = np.diag([math.copysign(f5_float(abs(x)), x) for x in dn])
    assert rel(out, expect) < 1e-13


def test_ns5_zero_input_is_zero():
    assert np.all(O.ns5_direct(np.zeros((3, 5))) == 0.0)


@pytest.mark.parametrize("shape", [(5, 9), (12, 40), (16, 16), (30, 31)])
def test_gram_and_direct_agree(shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    X = rng.standard_normal(shape)
    assert rel(O.ns5_gram(X), O.ns5_direct(X)) < 1e-12


def test_orientation_round_trip_tall():
    # NS of a tall U computed directly (m x m Gram, no transpose) equals the
    # transposed route through the short side.
    rng = np.random.default_rng(3)
    U = rng.standard_normal((40, 9))
    direct_tall = O.ns5_direct(U)  # iterates with the 40 x 40 A = U U^T
    X, tr = O.orient(U)
    assert tr and X.shape == (9, 40)
    assert rel(O.unorient(O.ns5_direct(X), tr), direct_tall) < 1e-12


def test_orient_keeps_square_and_wide():
    for shape in [(6, 6), (3, 8)]:
        X, tr = O.orient(np.ones(shape))
        assert not tr and X.shape == shape


def test_momentum_and_nesterov_scalars():
    M = np.full((2, 3), 1.0)
    G = np.full((2, 3), 2.0)
    Mn = O.momentum_update(M, G, 0.95)
    assert np.all(Mn == 0.95 * 1.0 + 2.0)
    U = O.nesterov_input(Mn, G, 0.95)
    assert np.allclose(U, 0.95 * 2.95 + 2.0, rtol=0, atol=1e-15)
    assert np.all(O.nesterov_input(Mn, G, 0.95, nesterov=False) == Mn)


def test_momentum_constant_gradient_closed_form():
    mu = 0.95
    G = np.random.default_rng(5).standard_normal((3, 4))
    M = np.zeros_like(G)
    for k in range(1, 8):
        M = O.momentum_update(M, G, mu)
        assert np.allclose(M, G * (1 - mu ** k) / (1 - mu), rtol=1e-14, atol=0)


def test_first_step_from_zero_momentum():
    # M_0 = 0: M_1 = G and U = (1 + mu) G, so X0 = G / |G|_F for any mu.
    rng = np.random.default_rng(6)
    W = rng.standard_normal((6, 10)) * 0.02
    G = rng.standard_normal((6, 10)) * 1e-3
    for mu in (0.5, 0.95):
        hp = O.Hyper(momentum=mu)
        W1, M1, O1 = O.muon_step(W, np.zeros_like(W), G, 0.02, 0.1, hp)
        assert np.array_equal(M1, G)
        assert rel(O1, O.ns5_direct(G)) < 1e-13


def test_second_step_uses_updated_momentum():
    # With M_0 = 0, two steps give U_2 = mu^2 G1 + (1 + mu) G2.  Choose G1, G2
    # with orthogonal row spaces so the NS output separates them: each block
    # keeps its own singular values, which fixes the relative weights.
    mu = 0.95
    G1 = np.zeros((2, 4)); G1[0, 0] = 1.0
    G2 = np.zeros((2, 4)); G2[1, 1] = 1.0
    _, M1, _ = O.muon_step(np.zeros((2, 4)), np.zeros((2, 4)), G1, 0.0, 0.0)
    _, M2, O2 = O.muon_step(np.zeros((2, 4)), M1, G2, 0.0, 0.0)
    assert np.allclose(M2, mu * G1 + G2, atol=1e-15)
    u = np.array([mu * mu, 1 + mu])
    s = u / np.linalg.norm(u)
    assert O2[0, 0] == pytest.approx(f5_float(s[0]), abs=1e-13)
    assert O2[1, 1] == pytest.approx(f5_float(s[1]), abs=1e-13)


def test_zero_gradient_and_momentum_pure_decay():
    W = np.random.default_rng(7).standard_normal((5, 8))
    Z = np.zeros_like(W)
    W1, M1, O1 = O.muon_step(W, Z, Z, 0.02, 0.1)
    assert np.all(O1 == 0) and np.all(M1 == 0)
    assert np.allclose(W1, 0.998 * W, rtol=1e-15, atol=0)
    W2, _, R2 = O.rownorm_step(W, Z, Z, 0.02, 0.1)
    assert np.all(R2 == 0)
    assert np.allclose(W2, 0.998 * W, rtol=1e-15, atol=0)


@pytest.mark.parametrize("m,n,expect", [(256, 1024, 6.4), (3584, 3584, 11.973304), (256, 256, 3.2),
                                         (18944, 3584, 27.527441), (4096, 4096, 12.8),
                                         (4096, 16384, 25.6)])
def test_update_scale(m, n, expect):
    assert O.update_scale(m, n) == pytest.approx(expect, abs=1e-6)


def test_full_step_rank_one_closed_form():
    # First step, rank-1 gradient: O = f^5(1) G/|G|_F, and
    # W' = (1 - lr wd) W - lr 0.2 sqrt(max(m,n)) O  (eq. (4) / DiT 2.1).
    rng = np.random.default_rng(8)
    m, n = 12, 5  # tall: exercises the transposed orientation too
    G = np.outer(rng.standard_normal(m), rng.standard_normal(n)) * 1e-3
    W = rng.standard_normal((m, n)) * 0.02
    lr, wd = 0.02, 0.1
    W1, _, O1 = O.muon_step(W, np.zeros_like(W), G, lr, wd)
    X0 = G / np.linalg.norm(G)
    expect_O = 0.6964364094697528 * X0
    assert rel(O1, expect_O) < 1e-13
    expect_W = (1 - lr * wd) * W - lr * 0.2 * math.sqrt(m) * expect_O
    assert rel(W1, expect_W) < 1e-14


def test_lemma1_polar_rms():
    # Lemma 1: a full-rank orthogonalised update U V^T has RMS 1/sqrt(max(A,B)).
    rng = np.random.default_rng(9)
    for shape in [(8, 30), (30, 8), (16, 16)]:
        U, _, Vt = np.linalg.svd(rng.standard_normal(shape), full_matrices=False)
        P = U @ Vt
        assert math.sqrt(np.mean(P ** 2)) == pytest.approx(1 / math.sqrt(max(shape)), rel=1e-12)


def test_rownorm_invariants():
    rng = np.random.default_rng(10)
    X = rng.standard_normal((6, 9))
    eps = 1e-8
    X[2] *= 1e-12          # ||row|| ~ 3e-12 < eps: divided by eps
    X[4] = 0.0             # zero row stays zero
    R = O.rownorm(X, eps)
    for i in (0, 1, 3, 5):
        assert np.linalg.norm(R[i]) == pytest.approx(1.0, abs=1e-14)
        assert np.allclose(R[i] * np.linalg.norm(X[i]), X[i], rtol=1e-13, atol=0)
    assert np.allclose(R[2], X[2] / eps, rtol=1e-15, atol=0)
    assert np.linalg.norm(R[2]) < 1.0
    assert np.all(R[4] == 0.0)
    # idempotent on rows that were normalised or zero (an eps-branch row
    # X/eps has norm above eps once scaled, so it is normalised again)
    R2 = O.rownorm(R, eps)
    keep = [0, 1, 3, 4, 5]
    assert np.allclose(R2[keep], R[keep], rtol=1e-14, atol=0)


def test_rownorm_rms_is_lemma1():
    rng = np.random.default_rng(11)
    for shape in [(8, 30), (30, 8)]:
        X, tr = O.orient(rng.standard_normal(shape))
        R = O.unorient(O.rownorm(X, 1e-8), tr)
        assert math.sqrt(np.mean(R ** 2)) == pytest.approx(1 / math.sqrt(max(shape)), rel=1e-13)


def test_rownorm_step_normalises_columns_when_tall():
    rng = np.random.default_rng(12)
    m, n = 20, 6
    W = rng.standard_normal((m, n)) * 0.02
    M = rng.standard_normal((m, n)) * 1e-3
    G = rng.standard_normal((m, n)) * 1e-3
    lr, wd = 0.02, 0.1
    W1, M1, R = O.rownorm_step(W, M, G, lr, wd)
    Mn = 0.95 * M + G
    U = 0.95 * Mn + G
    assert np.allclose(M1, Mn, rtol=1e-15, atol=0)
    col = np.linalg.norm(U, axis=0)
    assert np.allclose(R, U / col[None, :], rtol=1e-13, atol=0)
    assert np.allclose(np.linalg.norm(R, axis=0), 1.0, atol=1e-14)
    assert np.allclose(W1, (1 - lr * wd) * W - lr * 0.2 * math.sqrt(m) * R, rtol=1e-14, atol=1e-18)


def test_rownorm_step_square_normalises_rows():
    rng = np.random.default_rng(13)
    U = rng.standard_normal((7, 7))
    R = O.rownorm_step(np.zeros((7, 7)), np.zeros((7, 7)), U, 0.0, 0.0)[2]
    # first step: U_nesterov = (1 + mu) G, rows normalised
    assert np.allclose(np.linalg.norm(R, axis=1), 1.0, atol=1e-14)


def test_ns5_is_not_polar():
    # Five iterations do not reach the polar factor (DiT 2.1 remark): the
    # output singular values are f^5(s), not 1.
    rng = np.random.default_rng(14)
    M = rng.standard_normal((16, 48))
    s = np.linalg.svd(O.ns5_direct(M), compute_uv=False)
    assert np.max(np.abs(s - 1.0)) > 0.05
    assert np.max(s) <= 1.2025


def test_non_finite_inputs_reach_the_whole_direction():
    # The pages' formulas on a gradient holding a NaN or an Inf: ||U||_F is
    # NaN or Inf, so X0 = U / ||U||_F holds a NaN (NaN / x, Inf / Inf) and
    # eq. (2) spreads it through X X^T to every entry: the matrix's direction
    # and weights are all NaN.  The momentum keeps NaN / Inf only where the
    # gradient had it.  R_eps works row by row: only the affected oriented row
    # changes (NaN row for a NaN; for an Inf, NaN at the Inf and 0 elsewhere,
    # as x / Inf = 0).
    rng = np.random.default_rng(21)
    W = rng.standard_normal((6, 9)) * 0.02
    with np.errstate(invalid="ignore"):
        _non_finite_cases(rng, W)


def _non_finite_cases(rng, W):
    for bad in (np.nan, np.inf, -np.inf):
        G = rng.standard_normal((6, 9)) * 1e-3
        G[2, 3] = bad
        Wn, Mn, D = O.muon_step(W, np.zeros_like(W), G, 0.02, 0.1)
        assert np.isnan(D).all() and np.isnan(Wn).all()
        assert np.isfinite(np.delete(Mn.ravel(), 2 * 9 + 3)).all()
        assert Mn[2, 3] == bad or (np.isnan(bad) and np.isnan(Mn[2, 3]))
        Wr, Mr, R = O.rownorm_step(W, np.zeros_like(W), G, 0.02, 0.1)
        others = [i for i in range(6) if i != 2]
        assert np.isfinite(R[others]).all() and np.isfinite(Wr[others]).all()
        if np.isnan(bad):
            assert np.isnan(R[2]).all()
        else:
            assert np.isnan(R[2, 3]) and (np.delete(R[2], 3) == 0).all()
        # tall: the oriented rows are columns of U
        Wt, Mt, Rt = O.rownorm_step(W.T, np.zeros_like(W.T), G.T, 0.02, 0.1)
        assert np.array_equal(np.isnan(Rt), np.isnan(R.T))


@pytest.mark.slow
@pytest.mark.parametrize("shape", [(3584, 3584), (3584, 18944), (4096, 16384)])
def test_gram_and_direct_agree_at_full_size(shape):
    # The Gram-space routine stands in for the direct definition at the
    # workloads' full sizes (it needs a quarter of the flops on wide
    # matrices); pin the two together there in float64.
    rng = np.random.default_rng(shape[1])
    X = rng.standard_normal(shape)
    assert rel(O.ns5_gram(X), O.ns5_direct(X)) < 1e-10
