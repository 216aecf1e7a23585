"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these tests retypes an oracle formula: each compares the oracle with
an independent route (SVD, eigendecomposition, scipy's polar decomposition,
the r/q recursion of Theorem 1, printed constants, closed forms on special
inputs) chosen so that a dropped term, a wrong sign or index or a transposed
operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tables():
    with open(os.path.join(GOLDEN, "coefficient_tables.json")) as f:
        raw = json.load(f)
    out = {}
    for k, v in raw.items():
        if k.startswith("_"):
            continue
        rows = np.asarray(v["rows"], dtype=np.float64) / float(v.get("denominator", 1))
        if rows.shape[0] == 1 and v["steps"] > 1:
            rows = np.repeat(rows, v["steps"], axis=0)
        out[k] = (rows, v["steps"])
    return out


TABLES = _tables()


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --- constants -------------------------------------------------------------

def test_keller_constants_match_page():
    rows, steps = TABLES["keller"]
    assert steps == O.DEFAULT_STEPS == 5
    assert tuple(rows[0]) == O.KELLER_ABC


def test_schedule_expands_and_checks_tables():
    assert O.coefficient_schedule(None, 3) == [O.KELLER_ABC] * 3
    yj, t = TABLES["youjiacheng_t6"]
    sched = O.coefficient_schedule(yj, t)
    assert len(sched) == 6 and sched[0] == (3955 / 1024, -8306 / 1024, 5008 / 1024)
    with pytest.raises(ValueError):
        O.coefficient_schedule(yj, 5)
    with pytest.raises(ValueError):
        O.coefficient_schedule(None, 0)


# --- scalar map --------------------------------------------------------------

def test_phi_one_step_at_one_is_coefficient_sum():
    # p(1) = a + b + c: the value an orthonormal input keeps after one
    # unnormalised step (0.701 for the Keller triple)
    assert O.phi(1.0, steps=1) == pytest.approx(0.701, abs=1e-12)


def test_phi_derivative_at_zero_is_a_to_the_T():
    # nil9.net, fixed-point coefficient design: phi'(0) = a^5 for five steps
    h = 1e-9
    for name in ("keller", "dion_t5", "ours_x3_t5"):
        rows, t = TABLES[name]
        d = (O.phi(h, rows, t) - O.phi(-h, rows, t)) / (2 * h)
        assert d == pytest.approx(float(np.prod(rows[:, 0])), rel=1e-6)


def test_phi_odd_and_superattracting_fixed_point():
    # Proposition 2's example h = 15/8 - 10/8 x + 3/8 x^2 gives
    # p(x) = (15x - 10x^3 + 3x^5)/8 with p(1) = 1 and p'(1) = 0
    rows, _ = TABLES["prop2_example_h"]
    x = np.linspace(0.05, 1.0, 40)
    assert np.allclose(O.phi(x, rows[0], 30), 1.0, atol=1e-12)
    assert O.phi(1.0, rows[0], 7) == 1.0
    assert np.allclose(O.phi(-x, None, 5), -O.phi(x, None, 5), atol=0)


def test_theorem1_matches_composition():
    # Gram Newton-Schulz §2.2 Theorem 1: x q_T(x^2) = (p_T o ... o p_1)(x)
    x = np.linspace(-1.0, 1.0, 2001)
    for name, (rows, t) in TABLES.items():
        assert np.allclose(O.theorem1_xq(x, rows, t), O.phi(x, rows, t), rtol=1e-13, atol=1e-13), name


# --- exact msign ---------------------------------------------------------------

@pytest.mark.parametrize("shape", [(7, 7), (5, 9), (9, 5), (1, 6), (6, 1)])
def test_svd_msign_equals_scipy_polar_factor(shape):
    m = _rand(shape, 11)
    side = "right" if shape[0] >= shape[1] else "left"
    u, _ = scipy.linalg.polar(m, side=side)
    assert np.allclose(O.svd_msign(m), u, atol=1e-10)


def test_svd_msign_equals_inverse_sqrt_form_and_is_orthogonal():
    m = _rand((12, 12), 3)
    y = O.svd_msign(m)
    assert np.allclose(y, O.inverse_sqrt_msign(m), atol=1e-10)
    assert np.allclose(y.T @ y, np.eye(12), atol=1e-10)
    w = _rand((6, 10), 4)
    assert np.allclose(O.svd_msign(w), O.inverse_sqrt_msign(w), atol=1e-10)
    assert np.allclose(O.svd_msign(w) @ O.svd_msign(w).T, np.eye(6), atol=1e-10)


def test_svd_msign_is_best_orthogonal_approximation():
    # kexue.fm 10922 §写在前面: for square full-rank M, msign(M) minimises
    # ||M - O||_F over orthogonal O
    m = _rand((8, 8), 5)
    best = np.linalg.norm(m - O.svd_msign(m))
    rng = np.random.default_rng(6)
    for _ in range(200):
        q, _ = np.linalg.qr(rng.standard_normal((8, 8)))
        assert np.linalg.norm(m - q) >= best - 1e-12


def test_svd_msign_symmetric_is_matrix_sign_and_spd_is_identity():
    s = _rand((9, 9), 7)
    s = s + s.T
    w, v = np.linalg.eigh(s)
    assert np.allclose(O.svd_msign(s), (v * np.sign(w)) @ v.T, atol=1e-10)
    spd = s @ s.T + 0.1 * np.eye(9)
    assert np.allclose(O.svd_msign(spd), np.eye(9), atol=1e-10)


def test_svd_msign_rank_deficient_and_zero():
    rng = np.random.default_rng(8)
    m = rng.standard_normal((6, 2)) @ rng.standard_normal((2, 10))
    y = O.svd_msign(m)
    sv = np.linalg.svd(y, compute_uv=False)
    assert np.allclose(sv[:2], 1.0, atol=1e-10) and np.allclose(sv[2:], 0.0, atol=1e-10)
    assert np.array_equal(O.svd_msign(np.zeros((3, 4))), np.zeros((3, 4)))


# --- Newton-Schulz iteration -------------------------------------------------

@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (24, 24), (3, 50)])
@pytest.mark.parametrize("table", ["keller", "youjiacheng_t6", "dion_t5", "bernstein_cubic", "nil9_cubic"])
def test_ns_equals_per_singular_value_composition(shape, table):
    # kexue.fm 10922 §原理分析 / Gram NS Proposition 1
    rows, t = TABLES[table]
    m = _rand(shape, 21, 3.0)
    assert np.allclose(O.ns_single(m, rows, t), O.spectral_ns_single(m, rows, t), atol=1e-12)


@pytest.mark.parametrize("where", ["first", "every"])
def test_safety_factor_as_scaled_coefficients(where):
    # "Gram Newton-Schulz" §3.3 asks for a safety factor so that singular
    # values up to 1.05 still converge; its formula is lost in the text.
    # Both plain readings are per-step tables: dividing X_0 by s is the first
    # step's polynomial taken at x / s, i.e. (a / s, b / s^3, c / s^5); taking
    # every step's polynomial at x / s scales every row.  Checked against the
    # SVD route, where the singular values are divided by s directly.
    s = 1.05
    a, b, c = O.KELLER_ABC
    scaled = (a / s, b / s ** 3, c / s ** 5)
    table = [scaled] + [(a, b, c)] * 4 if where == "first" else [scaled] * 5
    m = _rand((12, 40), 77, 2.0)
    u, sv, vt = np.linalg.svd(m, full_matrices=False)
    y = sv / math.sqrt(float(np.sum(sv * sv)) + O.DEFAULT_EPS)
    for t in range(5):
        z = y / s if (t == 0 or where == "every") else y
        y = a * z + b * z ** 3 + c * z ** 5
    expect = (u * y) @ vt
    assert np.allclose(O.ns_single(m, table, 5), expect, atol=1e-12)
    assert np.allclose(O.gram_ns_single(m, table, 5, restart_after=(2,)), expect, atol=1e-12)
    # a singular value pushed to 1.05 by an error of the normalisation is
    # mapped as 1.0 is without the factor (first-step reading)
    if where == "first":
        def comp(x, rows):
            for ra, rb, rc in rows:
                x = ra * x + rb * x ** 3 + rc * x ** 5
            return x
        assert comp(1.05, table) == pytest.approx(comp(1.0, [(a, b, c)] * 5), abs=1e-14)


@pytest.mark.parametrize("table", ["bernstein_cubic", "nil9_cubic"])
def test_cubic_tables_fix_one(table):
    # nil9.net, third-order iteration: f(1) = a + b = 1 and |f'(1)| = |a + 3b| < 1
    rows, _ = TABLES[table]
    a, b, c = rows[0]
    assert c == 0.0 and abs(a + b - 1.0) < 1e-15 and abs(a + 3 * b) < 1.0


def test_cubic_iteration_converges_to_polar_factor():
    # The classical cubic Newton-Schulz step x -> (3x - x^3) / 2 maps (0, 1]
    # into itself and converges to 1 (quadratically near 1), so enough steps
    # from the Frobenius-normalised start give U V^T of a full-rank matrix.
    rows, _ = TABLES["bernstein_cubic"]
    m = _rand((20, 50), 31)
    y = O.ns_single(m, tuple(rows[0]), 40)
    assert np.allclose(y, O.svd_msign(m), atol=1e-10)
    # and of the transposed (tall) input
    assert np.allclose(O.ns_single(m.T, tuple(rows[0]), 40), O.svd_msign(m).T, atol=1e-10)


def test_ns_on_spd_matches_eigendecomposition():
    s = _rand((10, 10), 9)
    spd = s @ s.T + np.eye(10)
    w, v = np.linalg.eigh(spd)
    fro = math.sqrt(float(np.sum(w * w)) + O.DEFAULT_EPS)
    expect = (v * O.phi(w / fro)) @ v.T
    y = O.ns_single(spd)
    assert np.allclose(y, expect, atol=1e-12)
    assert np.allclose(y, y.T, atol=1e-14)


@pytest.mark.parametrize("n,m", [(4, 4), (8, 32), (128, 256)])
def test_ns_on_orthonormal_rows(n, m):
    # Frobenius normalisation maps sigma = 1 to 1/sqrt(n); the output is
    # phi(1/sqrt(n)) Q, the input itself up to the polynomial's value
    q, _ = np.linalg.qr(_rand((m, n), 10))
    q = q.T
    assert np.allclose(O.svd_msign(q), q, atol=1e-12)
    assert np.allclose(O.ns_single(q), O.phi(1 / math.sqrt(n)) * q, atol=1e-12)
    if n == 128:
        assert O.phi(1 / math.sqrt(128)) == pytest.approx(0.722762, abs=5e-7)


def test_ns_on_a_vector():
    v = _rand((1, 17), 12)
    unit = v / np.linalg.norm(v)
    assert np.allclose(O.svd_msign(v), unit, atol=1e-14)
    assert np.allclose(O.ns_single(v), O.phi(1.0) * unit, atol=1e-14)
    assert O.phi(1.0) == pytest.approx(0.696436, abs=5e-7)
    assert np.allclose(O.ns_single(v.T), O.phi(1.0) * unit.T, atol=1e-14)


def test_ns_tiny_diagonal_brute_force():
    m = np.diag([3.0, -4.0])
    y = O.ns_single(m)
    assert y[0, 1] == 0.0 and y[1, 0] == 0.0
    assert y[0, 0] == pytest.approx(O.phi(0.6), abs=1e-14)
    assert y[1, 1] == pytest.approx(-O.phi(0.8), abs=1e-14)
    one = O.ns_single(np.array([[-2.5]]))
    assert one[0, 0] == pytest.approx(-O.phi(1.0), abs=1e-14)


def test_ns_transpose_and_scale_invariance():
    m = _rand((12, 30), 13)
    assert np.allclose(O.ns_single(m.T), O.ns_single(m).T, atol=1e-13)
    assert np.allclose(O.ns_single(1e3 * m), O.ns_single(m), atol=1e-12)
    assert np.allclose(O.ns_single(1e-3 * m), O.ns_single(m), atol=1e-12)


def test_ns_rank_deficient_keeps_null_space():
    rng = np.random.default_rng(14)
    u, _ = np.linalg.qr(rng.standard_normal((10, 3)))
    v, _ = np.linalg.qr(rng.standard_normal((20, 3)))
    s = np.array([5.0, 2.0, 0.5])
    m = (u * s) @ v.T
    y = O.ns_single(m)
    expect = (u * O.phi(s / np.linalg.norm(s))) @ v.T
    assert np.allclose(y, expect, atol=1e-12)
    assert np.linalg.matrix_rank(y, tol=1e-9) == 3


def test_ns_error_bound_against_exact():
    m = _rand((20, 50), 15)
    s = np.linalg.svd(m, compute_uv=False)
    bound = float(np.max(np.abs(O.phi(s / np.linalg.norm(s)) - 1.0)))
    err = O.max_rel_fro_error(O.ns_single(m), O.svd_msign(m))
    assert err <= bound + 1e-12
    assert err > 0.0


def test_ns_zero_and_batched():
    assert np.array_equal(O.ns_single(np.zeros((4, 6))), np.zeros((4, 6)))
    b = _rand((3, 5, 8), 16)
    y = O.ns(b)
    for i in range(3):
        assert np.array_equal(y[i], O.ns_single(b[i]))
    assert O.ns(np.zeros((0, 4, 6))).shape == (0, 4, 6)


# --- Gram Newton-Schulz -------------------------------------------------------

@pytest.mark.parametrize("restarts", [(), (2,), (1, 2, 3, 4)])
@pytest.mark.parametrize("shape", [(12, 48), (48, 12), (16, 16)])
def test_gram_equals_standard_ns(restarts, shape):
    # Gram NS §2 and §3.4: same output in exact arithmetic, any restarts
    m = _rand(shape, 17, 0.1)
    assert np.allclose(O.gram_ns_single(m, restart_after=restarts), O.ns_single(m), atol=1e-12)


def test_gram_with_per_step_table():
    rows, t = TABLES["youjiacheng_t6"]
    m = _rand((10, 30), 18)
    assert np.allclose(O.gram_ns_single(m, rows, t, restart_after=(3,)),
                       O.spectral_ns_single(m, rows, t), atol=1e-12)


def test_gram_restart_list_outside_range_is_inert():
    m = _rand((8, 20), 19)
    assert np.allclose(O.gram_ns_single(m, restart_after=(5, 9)),
                       O.gram_ns_single(m, restart_after=()), atol=1e-15)


# --- improved initial normalisation -------------------------------------------

def test_improved_init_closed_form():
    # kexue.fm 10922 §改良初值: the extra factor is the 4th root of
    # ||(X X^T)^2||_F, i.e. (sum sigma^8)^(1/8) of the normalised X
    m = _rand((15, 40), 20)
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    shat = s / np.linalg.norm(s)
    scale = float(np.sum(shat ** 8)) ** 0.125
    expect = (u * O.phi(shat / scale)) @ vt
    assert np.allclose(O.ns_improved_init_single(m), expect, atol=1e-12)
    # the norm chain sigma_1 <= (sum s^8)^(1/8) <= (sum s^4)^(1/4) <= ||s||_2
    s8, s4 = float(np.sum(s ** 8)) ** 0.125, float(np.sum(s ** 4)) ** 0.25
    assert s[0] <= s8 <= s4 <= np.linalg.norm(s)


def test_improved_init_raises_smallest_singular_value():
    # kexue.fm 10922 §改良初值: on 100x100 Gaussian matrices the smallest
    # output singular value is mostly more than twice the plain one
    wins = 0
    for seed in range(12):
        m = _rand((100, 100), 100 + seed)
        a = np.linalg.svd(O.ns_single(m), compute_uv=False)[-1]
        b = np.linalg.svd(O.ns_improved_init_single(m), compute_uv=False)[-1]
        wins += b > 2 * a
    assert wins > 6


# --- error measure and FLOP models -----------------------------------------------

def test_max_rel_fro_error():
    o = _rand((2, 3, 4), 22)
    assert O.max_rel_fro_error(o * 1.01, o) == pytest.approx(0.01, rel=1e-12)
    assert O.max_rel_fro_error(np.ones((1, 2, 2)), np.zeros((1, 2, 2))) == pytest.approx(2.0)


def test_flop_models_reproduce_printed_reductions():
    with open(os.path.join(GOLDEN, "flop_reductions.json")) as f:
        g = json.load(f)
    n = 1024
    models = {"dense_ns": O.dense_ns_flops, "symmetric_ns": O.symmetric_ns_flops,
              "naive_gram": O.naive_gram_flops, "restart_gram": O.restart_gram_flops}
    for case in g["cases"]:
        m = case["alpha"] * n
        new = models[case["new"]](n, m, case["steps"])
        old = models[case["old"]](n, m, case["steps"])
        assert round(100 * (1 - new / old)) == case["percent"], case
    assert O.dense_ns_flops(n, 3 * n) == (20 * 3 + 10) * n ** 3
    assert O.naive_gram_flops(n, 2 * n) == (17 + 3 * 2) * n ** 3
    assert O.symmetric_ns_flops(n, 4 * n, 1) == (3 * 4 + 1) * n ** 3
    assert O.restart_gram_flops(n, 8 * n) == (14 + 6 * 8) * n ** 3


# --- Muon step around msign --------------------------------------------------------

def _orthogonal(n, seed):
    q, r = np.linalg.qr(_rand((n, n), seed))
    return q * np.sign(np.diag(r))


def test_muon_two_steps_closed_form():
    """With exact msign and M_0 = 0: G_1 = Q_1 (orthogonal) and
    G_2 = P Q_2 - mu Q_1 (P symmetric positive definite) give M_1 = Q_1,
    M_2 = P Q_2, whose polar factor is Q_2, so W_2 = W_0 - eta (Q_1 + Q_2).
    Any other momentum rule (M + mu G, mu (M + G), (1 - mu) M + G ...) or a
    sign slip in the update moves W_2 off this value."""
    n, mu, lr = 24, 0.9, 0.05
    q1, q2 = _orthogonal(n, 501), _orthogonal(n, 502)
    b = _rand((n, n), 503)
    p = b @ b.T + n * np.eye(n)
    w0 = _rand((n, n), 504)
    w1, m1 = O.muon_step(w0, q1, np.zeros((n, n)), mu, lr, msign=O.exact_msign)
    assert np.allclose(m1, q1, atol=1e-14)
    w2, m2 = O.muon_step(w1, p @ q2 - mu * q1, m1, mu, lr, msign=O.exact_msign)
    assert np.allclose(m2, p @ q2, atol=1e-12)
    assert np.allclose(w2, w0 - lr * (q1 + q2), atol=1e-12)


def test_muon_constant_gradient_and_rectangular_shapes():
    """A constant gradient G makes M_k = (1 + mu + ... + mu^(k-1)) G, a positive
    multiple of G, so every step moves W by -eta msign(G) (scale invariance of
    msign); holds for wide and tall batches with the NS map as well."""
    mu, lr = 0.95, 0.02
    for shape in ((2, 16, 40), (2, 40, 16)):
        g = _rand(shape, 510 + shape[1])
        w = _rand(shape, 520 + shape[1])
        m = np.zeros(shape)
        d_exact = O.exact_msign(g)
        d_ns = O.ns(g)
        for k in range(1, 4):
            w_next, m = O.muon_step(w, g, m, mu, lr)
            assert np.allclose(m, sum(mu ** j for j in range(k)) * g, atol=1e-12)
            assert np.allclose(w - w_next, lr * d_ns, atol=1e-10)
            w = w_next
        # the NS direction is the exact one up to NS's own error bound
        assert O.max_rel_fro_error(d_ns, d_exact) < 0.35


def test_muon_zero_momentum_coefficient_is_plain_msign_descent():
    """mu = 0: the momentum is the gradient, and the step is [MS]'s
    -eta msign(G) with eta = 1."""
    g = _rand((3, 12, 20), 530)
    w = _rand((3, 12, 20), 531)
    w1, m1 = O.muon_step(w, g, _rand((3, 12, 20), 532), 0.0, 1.0, msign=O.exact_msign)
    assert np.array_equal(m1, g)
    assert np.allclose(w1, w - O.exact_msign(g), atol=1e-13)
