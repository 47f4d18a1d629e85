"""Pins for the CPU oracle: checks against what the mathematics fixes.

None of these tests re-types the oracle's iteration.  They check it against
(a) LAPACK's SVD and the scalar map the iteration induces on singular values,
(b) exact rational arithmetic on diagonal and rank-1 inputs,
(c) the polar factor (the textbook limit of the cubic iteration),
(d) invariances (batch slices, transposition, scaling, orthogonal factors),
(e) the geometric-series closed form of the momentum, and
(f) planted mistakes, each of which must trip at least one pin.

Why the scalar map: write X = U S V^T.  Then A = X X^T = U S^2 U^T,
b A + c A^2 = U (b S^2 + c S^4) U^T and so one round sends X to
U (a S + b S^3 + c S^5) V^T: singular vectors stay, each singular value goes
through p(s) = a s + b s^3 + c s^5.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import muon_ref
from workloads import CUBIC, QUINTIC

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def p_scalar(s, coeffs, steps):
    a, b, c = (float(np.float32(v)) for v in coeffs)
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def p_exact(s: Fraction, coeffs, steps) -> Fraction:
    a, b, c = (Fraction(float(np.float32(v))) for v in coeffs)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def random_orthogonal(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


# ---------------------------------------------------------------- pin helpers
# Each helper takes the function under test so that the planted-mistake test
# below can run the same checks against deliberately broken copies.

def svd_invariant_error(ortho, shape, coeffs, steps, seed=0):
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(shape).astype(np.float32)
    o = ortho(m, steps, *coeffs)
    u, s, vt = np.linalg.svd(m.astype(np.float64), full_matrices=False)
    s0 = s / (np.sqrt(np.sum(s ** 2)) + oracle.DEFAULT_EPS)
    expect = (u * p_scalar(s0, coeffs, steps)) @ vt
    return np.linalg.norm(o - expect) / np.linalg.norm(expect)


def diag_exact_error(ortho, coeffs, steps):
    # G = [[3,0,0],[0,4,0]]: ||G||_F = 5, singular values 3/5 and 4/5.
    g = np.array([[3.0, 0.0, 0.0], [0.0, 4.0, 0.0]], dtype=np.float32)
    o = ortho(g, steps, *coeffs, eps=0.0)
    e0 = float(p_exact(Fraction(3, 5), coeffs, steps))
    e1 = float(p_exact(Fraction(4, 5), coeffs, steps))
    expect = np.array([[e0, 0, 0], [0, e1, 0]])
    return np.max(np.abs(o - expect))


def rank1_exact_error(ortho, coeffs, steps, shape=(5, 7), seed=3):
    # Small integers keep u v^T exactly rank one after the float32 store.
    rng = np.random.default_rng(seed)
    u = rng.integers(-8, 9, shape[0]).astype(np.float64)
    v = rng.integers(-8, 9, shape[1]).astype(np.float64)
    u[0], v[0] = 3.0, -5.0
    g = np.outer(u, v).astype(np.float32)
    o = ortho(g, steps, *coeffs, eps=0.0)
    g64 = g.astype(np.float64)
    direction = g64 / np.linalg.norm(g64)           # the unit singular triple u v^T
    expect = float(p_exact(Fraction(1), coeffs, steps)) * direction
    return np.max(np.abs(o - expect))


# ------------------------------------------------------------------ the pins

@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8), (1, 9), (24, 200)])
@pytest.mark.parametrize("coeffs", [QUINTIC, CUBIC])
def test_svd_invariant(shape, coeffs):
    assert svd_invariant_error(oracle.orthogonalize, shape, coeffs, 5) < 1e-12


@pytest.mark.parametrize("coeffs", [QUINTIC, CUBIC])
@pytest.mark.parametrize("steps", [0, 1, 5, 7])
def test_diagonal_exact(coeffs, steps):
    assert diag_exact_error(oracle.orthogonalize, coeffs, steps) < 1e-13


def test_cubic_diagonal_values():
    # The cubic keeps 1 fixed and pulls 0.6 and 0.8 towards it.
    v = [float(p_exact(Fraction(3, 5), CUBIC, 5)), float(p_exact(Fraction(4, 5), CUBIC, 5))]
    assert abs(v[0] - 1.0) < 1e-8 and abs(v[1] - 1.0) < 1e-12


@pytest.mark.parametrize("coeffs", [QUINTIC, CUBIC])
def test_rank1_exact(coeffs):
    assert rank1_exact_error(oracle.orthogonalize, coeffs, 5) < 1e-13


def test_quintic_fixed_values():
    # With the quintic coefficients 1 is not a fixed point; five rounds from 1
    # land near 0.6964 and every start in [0.01, 1] ends inside [0.68, 1.14].
    # Exact decimal coefficients give 0.696436409470; their float32 roundings
    # (what the step uses) move the value by about 3e-8.
    dec = tuple(Fraction(v) for v in ("3.4445", "-4.7750", "2.0315"))
    s_dec = Fraction(1)
    for _ in range(5):
        s_dec = dec[0] * s_dec + dec[1] * s_dec ** 3 + dec[2] * s_dec ** 5
    assert abs(float(s_dec) - 0.696436409470) < 1e-12
    assert abs(float(p_exact(Fraction(1), QUINTIC, 5)) - float(s_dec)) < 1e-7
    s = np.linspace(0.01, 1.0, 2000)
    out = p_scalar(s, QUINTIC, 5)
    assert out.min() > 0.68 and out.max() < 1.14


def test_equal_singular_values():
    rng = np.random.default_rng(5)
    n = 16
    q = random_orthogonal(rng, n).astype(np.float32)
    o = oracle.orthogonalize(q, 5, *QUINTIC, eps=0.0)
    q64 = q.astype(np.float64)
    s = np.linalg.svd(q64, compute_uv=False)
    # float32 rounding leaves the singular values within ~1e-7 of 1.
    assert np.max(np.abs(s - 1)) < 1e-6
    u, s, vt = np.linalg.svd(q64)
    expect = (u * p_scalar(s / np.linalg.norm(s), QUINTIC, 5)) @ vt
    assert np.max(np.abs(o - expect)) < 1e-12
    assert abs(p_scalar(1 / np.sqrt(n), QUINTIC, 5) - np.linalg.svd(o, compute_uv=False)[0]) < 1e-6


def test_cubic_limit_is_polar_factor():
    rng = np.random.default_rng(7)
    u = random_orthogonal(rng, 6)
    v = random_orthogonal(rng, 9)[:, :6]
    s = np.array([1.0, 0.9, 0.8, 0.7, 0.6, 0.5])
    g = ((u * s) @ v.T).astype(np.float32)
    o = oracle.orthogonalize(g, 60, *CUBIC)
    uu, _, vvt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    assert np.max(np.abs(o - uu @ vvt)) < 1e-10


def test_orientation_rule():
    x = np.zeros((5, 3))
    assert oracle.orient(x)[1] is True
    assert oracle.orient(x.T)[1] is False
    assert oracle.orient(np.zeros((4, 4)))[1] is False


def test_transpose_equivariance():
    rng = np.random.default_rng(11)
    g = rng.standard_normal((12, 30)).astype(np.float32)
    o = oracle.orthogonalize(g, 5, *QUINTIC)
    ot = oracle.orthogonalize(np.ascontiguousarray(g.T), 5, *QUINTIC)
    assert np.max(np.abs(o.T - ot)) < 1e-13


def test_scale_invariance():
    rng = np.random.default_rng(12)
    g = rng.standard_normal((9, 14)).astype(np.float32)
    o1 = oracle.orthogonalize(g, 5, *QUINTIC)
    o2 = oracle.orthogonalize(g * np.float32(1024.0), 5, *QUINTIC)
    assert np.max(np.abs(o1 - o2)) < 1e-6    # only eps breaks exact invariance


def test_orthogonal_invariance():
    rng = np.random.default_rng(13)
    g = rng.standard_normal((7, 11))
    q = random_orthogonal(rng, 7)
    z = random_orthogonal(rng, 11)
    o = oracle.orthogonalize(g, 5, *QUINTIC)
    o_rot = oracle.orthogonalize(q @ g @ z, 5, *QUINTIC)
    assert np.max(np.abs(o_rot - q @ o @ z)) < 1e-12


def test_batch_slices_are_independent():
    rng = np.random.default_rng(14)
    g = rng.standard_normal((3, 6, 10)).astype(np.float32)
    g[1] *= 100.0                                   # a slice of very different scale
    w = np.zeros_like(g)
    m = np.zeros_like(g)
    _, _, (o3,) = oracle.muon_step([w], [g], [m], lr=0.1, beta=0.9, ns_steps=5, a=QUINTIC[0],
                                   b=QUINTIC[1], c=QUINTIC[2])
    for e in range(3):
        o2 = oracle.orthogonalize(g[e], 5, *QUINTIC)
        assert np.array_equal(o3[e], o2)


def test_momentum_geometric_series():
    rng = np.random.default_rng(15)
    g = rng.standard_normal((4, 5)).astype(np.float32)
    beta = 0.95
    m = np.zeros_like(g)
    for t in range(1, 9):
        m = oracle.momentum_update(m, g, beta)
        b32 = float(np.float32(beta))
        expect = g.astype(np.float64) * (1 - b32 ** t) / (1 - b32)
        assert np.max(np.abs(m - expect) / np.abs(expect)) < 1e-6


def test_first_step_momentum_is_gradient():
    rng = np.random.default_rng(16)
    g = rng.standard_normal((4, 5)).astype(np.float32)
    m = oracle.momentum_update(np.zeros_like(g), g, 0.95)
    assert np.array_equal(m, g)


def test_ema_momentum_gives_same_direction():
    rng = np.random.default_rng(17)
    g = rng.standard_normal((6, 9)).astype(np.float32)
    m0 = rng.standard_normal((6, 9)).astype(np.float32)
    beta = 0.9
    s = np.float32(1 - beta)
    _, (mh,), (oh,) = oracle.muon_step([np.zeros_like(g)], [g], [m0], lr=1, beta=beta, ns_steps=5,
                                       a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2])
    _, (me,), (oe,) = oracle.muon_step([np.zeros_like(g)], [g * s], [m0 * s], lr=1, beta=beta,
                                       ns_steps=5, a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2])
    assert np.max(np.abs(oh - oe)) < 1e-5
    assert np.max(np.abs(me - mh * s)) < 1e-6 * np.max(np.abs(mh))


def test_zero_steps_is_normalised_momentum():
    rng = np.random.default_rng(18)
    g = rng.standard_normal((8, 3)).astype(np.float32)
    o = oracle.orthogonalize(g, 0, *QUINTIC)
    norm = np.linalg.norm(g.astype(np.float64))
    assert abs(np.linalg.norm(o) - norm / (norm + oracle.DEFAULT_EPS)) < 1e-15
    assert np.max(np.abs(o - g / norm)) < 1e-7


def test_zero_gradient_gives_zero_update():
    w = np.full((4, 6), 0.5, dtype=np.float32)
    z = np.zeros((4, 6), dtype=np.float32)
    (wn,), (mn,), (o,) = oracle.muon_step([w], [z], [z], lr=0.02, beta=0.95, ns_steps=5,
                                          a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2])
    assert not np.any(o) and np.array_equal(wn, w.astype(np.float64)) and not np.any(mn)


def test_update_rule_rank1():
    rng = np.random.default_rng(19)
    u = np.array([1.0, -2.0, 3.0, 0.5, 4.0])
    v = np.array([2.0, 1.0, -1.0, 0.25, 3.0, -6.0, 1.5, 2.0])
    g = np.outer(u, v).astype(np.float32)
    w = rng.standard_normal((5, 8)).astype(np.float32)
    lr = 0.25
    (wn,), _, _ = oracle.muon_step([w], [g], [np.zeros_like(g)], lr=lr, beta=0.95, ns_steps=5,
                                   a=CUBIC[0], b=CUBIC[1], c=CUBIC[2], eps=0.0)
    g64 = g.astype(np.float64)
    direction = g64 / np.linalg.norm(g64)
    expect = w.astype(np.float64) - lr * float(p_exact(Fraction(1), CUBIC, 5)) * direction
    assert np.max(np.abs(wn - expect)) < 1e-13


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = oracle.decode(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 1.0 + 2.0 ** -7
    assert vals[3] == 0.0 and np.signbit(vals[4])
    assert vals[5] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert vals[6] == 2.0 ** -133                   # smallest bf16 subnormal


def test_bf16_gradient_matches_float32_path():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(20)
    g32 = rng.standard_normal((6, 10)).astype(np.float32)
    bits = f32_to_bf16_bits(g32)
    g_rounded = oracle.decode(bits).astype(np.float32)
    o_bits = oracle.orthogonalize(oracle.momentum_update(np.zeros_like(g32), bits, 0.9), 5, *QUINTIC)
    o_f32 = oracle.orthogonalize(g_rounded, 5, *QUINTIC)
    assert np.array_equal(o_bits, o_f32)


def test_brute_force_tiny():
    """Pure-Python loops on a 2 x 3 input, written from the definition of the
    matrix products, against the numpy oracle."""
    g = [[0.5, -1.0, 2.0], [1.5, 0.25, -0.75]]
    a, b, c = (float(np.float32(v)) for v in QUINTIC)
    x = [row[:] for row in g]
    nrm = sum(v * v for row in x for v in row) ** 0.5 + oracle.DEFAULT_EPS
    x = [[v / nrm for v in row] for row in x]
    for _ in range(5):
        A = [[sum(x[i][k] * x[j][k] for k in range(3)) for j in range(2)] for i in range(2)]
        A2 = [[sum(A[i][k] * A[k][j] for k in range(2)) for j in range(2)] for i in range(2)]
        B = [[b * A[i][j] + c * A2[i][j] for j in range(2)] for i in range(2)]
        x = [[a * x[i][j] + sum(B[i][k] * x[k][j] for k in range(2)) for j in range(3)]
             for i in range(2)]
    o = oracle.orthogonalize(np.array(g, dtype=np.float32), 5, *QUINTIC)
    assert np.max(np.abs(o - np.array(x))) < 1e-14


def test_rejects_4d():
    z = np.zeros((2, 2, 2, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.muon_step([z], [z], [z], lr=1, beta=0.9, ns_steps=1, a=1, b=0, c=0)


# ------------------------------------------------------- planted mistakes

def _mutant_ns(kind):
    def ns(x, steps, a, b, c):
        a, b, c = oracle.f32(a), oracle.f32(b), oracle.f32(c)
        if kind == "off_by_one":
            steps = steps + 1
        for _ in range(steps):
            gram = x @ x.T
            if kind == "gram_transposed":
                gram = x.T @ x if x.shape[0] == x.shape[1] else x @ x.T * 1.0001
            if kind == "drop_c":
                poly = b * gram
            elif kind == "sign_b":
                poly = -b * gram + c * (gram @ gram)
            else:
                poly = b * gram + c * (gram @ gram)
            if kind == "right_multiply" and x.shape[0] == x.shape[1]:
                x = a * x + x @ poly
            elif kind == "right_multiply":
                x = a * x + 1.0001 * poly @ x
            else:
                x = a * x + poly @ x
        return x
    return ns


def _mutant_norm(x, eps=oracle.DEFAULT_EPS):
    return x / (np.max(np.abs(x)) + eps)


@pytest.mark.parametrize("kind", ["drop_c", "sign_b", "gram_transposed", "right_multiply",
                                  "off_by_one", "bad_norm"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    if kind == "bad_norm":
        monkeypatch.setattr(muon_ref, "frobenius_normalize", _mutant_norm)
    else:
        monkeypatch.setattr(muon_ref, "newton_schulz", _mutant_ns(kind))
    errs = [
        svd_invariant_error(muon_ref.orthogonalize, (8, 8), QUINTIC, 5),
        svd_invariant_error(muon_ref.orthogonalize, (6, 10), QUINTIC, 5),
        diag_exact_error(muon_ref.orthogonalize, QUINTIC, 5),
        rank1_exact_error(muon_ref.orthogonalize, QUINTIC, 5),
    ]
    # NaN (a diverged iteration) counts as caught.
    assert any(not (e <= 1e-6) for e in errs), f"mutation {kind} slipped past every pin: {errs}"


def test_planted_momentum_mistake_is_caught(monkeypatch):
    def ema(m, g, beta):
        return ((1 - oracle.f32(beta)) * oracle.decode(g) + oracle.f32(beta) * oracle.decode(m)).astype(np.float32)
    monkeypatch.setattr(muon_ref, "momentum_update", ema)
    g = np.ones((2, 2), dtype=np.float32)
    m = muon_ref.momentum_update(np.zeros_like(g), g, 0.95)
    assert not np.array_equal(m, g)       # the first-step pin would fail


def test_planted_slice_mistake_is_caught(monkeypatch):
    def whole_tensor_slices(shape):
        yield (Ellipsis,)
    monkeypatch.setattr(muon_ref, "_slices", whole_tensor_slices)
    rng = np.random.default_rng(14)
    g = rng.standard_normal((3, 6, 10)).astype(np.float32)
    with pytest.raises(ValueError):
        # a whole 3-D tensor cannot be oriented as one matrix
        muon_ref.muon_step([np.zeros_like(g)], [g], [np.zeros_like(g)], lr=0.1, beta=0.9,
                           ns_steps=5, a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2])


# --------------------------------------------------- opt-in update variants
# (Nesterov momentum, decoupled weight decay, shape factor; off by default.)

def _orthonormal_pair(shape, seed):
    """Two rank-one matrices u1 v1^T and u2 v2^T with u1 _|_ u2, v1 _|_ v2, unit norms."""
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((shape[0], 2)))
    v, _ = np.linalg.qr(rng.standard_normal((shape[1], 2)))
    return u[:, 0], v[:, 0], u[:, 1], v[:, 1]


def nesterov_pair_error(step, nesterov, beta=0.9, shape=(6, 9)):
    """Two steps from M = 0 with G1 = u1 v1^T then G2 = u2 v2^T.  Heavy ball
    gives M2 = beta G1 + G2 (singular values beta and 1); with Nesterov the
    orthogonalised matrix is G2 + beta M2 = beta^2 G1 + (1 + beta) G2.  O then
    has singular values p^5 of those values over their 2-norm, on the same
    singular vectors."""
    u1, v1, u2, v2 = _orthonormal_pair(shape, 5)
    g1 = np.outer(u1, v1).astype(np.float32)
    g2 = np.outer(u2, v2).astype(np.float32)
    b = float(np.float32(beta))
    zero = np.zeros(shape, np.float32)
    _, m1, _ = step([zero], [g1], [zero], lr=1.0, beta=beta, ns_steps=5, a=QUINTIC[0], b=QUINTIC[1],
                    c=QUINTIC[2], nesterov=nesterov)
    _, _, o = step([zero], [g2], m1, lr=1.0, beta=beta, ns_steps=5, a=QUINTIC[0], b=QUINTIC[1],
                   c=QUINTIC[2], nesterov=nesterov)
    # The exact singular values of the float32-stored G1 and G2 differ from 1
    # by float32 rounding only; the pin tolerance allows for that.
    s = np.array([b * b, 1.0 + b]) if nesterov else np.array([b, 1.0])
    s = s / np.linalg.norm(s)
    ps = p_scalar(s, QUINTIC, 5)
    expect = ps[0] * np.outer(u1, v1) + ps[1] * np.outer(u2, v2)
    return np.max(np.abs(o[0] - expect))


@pytest.mark.parametrize("nesterov", [False, True])
def test_nesterov_closed_form(nesterov):
    assert nesterov_pair_error(oracle.muon_step, nesterov) < 3e-5


def test_nesterov_changes_the_direction():
    """The two closed forms differ, so the pin can tell the variants apart."""
    b = 0.9
    r_plain = b / 1.0
    r_nest = b * b / (1.0 + b)
    assert abs(r_plain - r_nest) > 0.4


def test_weight_decay_with_zero_gradient_only_shrinks():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((5, 8)).astype(np.float32)
    zero = np.zeros_like(w)
    lr, wd = 0.02, 0.1
    w_new, _, o = oracle.muon_step([w], [zero], [zero], lr=lr, beta=0.95, ns_steps=5, a=QUINTIC[0],
                                   b=QUINTIC[1], c=QUINTIC[2], weight_decay=wd)
    assert not o[0].any()
    lr32, wd32 = float(np.float32(lr)), float(np.float32(wd))
    np.testing.assert_allclose(w_new[0], w.astype(np.float64) * (1.0 - lr32 * wd32), rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode,shape,factor", [
    ("none", (12, 5), 1.0),
    ("aspect", (12, 5), np.sqrt(12 / 5)),
    ("aspect", (5, 12), 1.0),
    ("rms", (12, 5), 0.2 * np.sqrt(12)),
    ("rms", (5, 12), 0.2 * np.sqrt(12)),
])
def test_update_scale_and_decay_rank1(mode, shape, factor):
    """Rank one G (integers, exact in float32): O = p^5(1) u v^T / (|u||v|),
    and W1 = (1 - lr wd) W0 - lr f O with the factor f of the stored shape."""
    rng = np.random.default_rng(4)
    u = rng.integers(-6, 7, shape[0]).astype(np.float64)
    v = rng.integers(-6, 7, shape[1]).astype(np.float64)
    u[0], v[0] = 2.0, -3.0
    g = np.outer(u, v).astype(np.float32)
    w = rng.standard_normal(shape).astype(np.float32)
    zero = np.zeros(shape, np.float32)
    lr, wd = 0.05, 0.2
    w_new, _, _ = oracle.muon_step([w], [g], [zero], lr=lr, beta=0.9, ns_steps=5, a=QUINTIC[0],
                                   b=QUINTIC[1], c=QUINTIC[2], eps=0.0, weight_decay=wd,
                                   update_scale_mode=mode)
    lr32, wd32 = float(np.float32(lr)), float(np.float32(wd))
    o = float(p_exact(Fraction(1), QUINTIC, 5)) * np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v))
    expect = (1.0 - lr32 * wd32) * w.astype(np.float64) - lr32 * factor * o
    np.testing.assert_allclose(w_new[0], expect, rtol=0, atol=1e-12)


def test_planted_nesterov_mistakes_are_caught(monkeypatch):
    """Broken directions: Nesterov ignored, or (1 + beta) M instead of G + beta M."""
    real = muon_ref.update_direction
    monkeypatch.setattr(muon_ref, "update_direction", lambda m, g, beta, nest: real(m, g, beta, False))
    assert nesterov_pair_error(muon_ref.muon_step, True) > 1e-3
    monkeypatch.setattr(muon_ref, "update_direction",
                        lambda m, g, beta, nest: (1.0 + float(np.float32(beta))) * real(m, g, beta, False))
    assert nesterov_pair_error(muon_ref.muon_step, True) > 1e-3


def test_float32_storage_option_is_only_a_timing_variant():
    """The float32 storage option (used only to time the CPU baseline in the
    GPU path's precision class) runs the same steps: it agrees with the
    float64 default to float32 accuracy and does not change the default."""
    rng = np.random.default_rng(5)
    g = rng.standard_normal((40, 300)).astype(np.float32)
    o64 = oracle.orthogonalize(g, 5, *QUINTIC)
    o32 = oracle.orthogonalize(g, 5, *QUINTIC, dtype=np.float32)
    assert o64.dtype == np.float64 and o32.dtype == np.float32
    assert np.linalg.norm(o32 - o64) / np.linalg.norm(o64) < 1e-5
    assert np.array_equal(o64, oracle.orthogonalize(g, 5, *QUINTIC, dtype=np.float64))
