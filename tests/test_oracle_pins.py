"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these re-types an oracle formula: each compares the oracle with a
worked example from the pages, a closed form, a library routine, an
invariant, or brute force on tiny inputs.
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle as O
import workloads as W
from golden_io import load


# ---------------------------------------------------------------- Hadamard
def test_hadamard_worked_example():
    g = load("hadamard4_example.txt")
    H = g["H_times_2"] / 2.0
    np.testing.assert_array_equal(O.hadamard(4), H)
    np.testing.assert_array_equal(H.T @ H, np.eye(4))
    out = O.fwht(g["x"])
    np.testing.assert_array_equal(out, g["Htx"])           # exact
    # fp32 gives the same exactly
    np.testing.assert_array_equal(out.astype(np.float32), g["Htx"].astype(np.float32))
    np.testing.assert_array_equal(O.fwht(g["inverse_in"]), g["inverse_out"])
    # infinity norm drops 20 -> 10, L2 norm kept
    assert np.abs(out).max() == 10 and np.abs(g["x"]).max() == 20
    assert np.linalg.norm(out) == pytest.approx(np.linalg.norm(g["x"]), rel=0, abs=1e-12)


# ---------------------------------------------------------------- structured Hadamard
def test_quadratic_character_textbook_residues():
    # nonzero squares mod 11 are {1, 3, 4, 5, 9}; mod 13 {1, 3, 4, 9, 10, 12};
    # mod 19 {1, 4, 5, 6, 7, 9, 11, 16, 17}
    for q, res in ((11, {1, 3, 4, 5, 9}), (13, {1, 3, 4, 9, 10, 12}),
                   (19, {1, 4, 5, 6, 7, 9, 11, 16, 17})):
        chi = O.quadratic_character(q)
        assert chi[0] == 0
        assert {a for a in range(1, q) if chi[a] == 1} == res
        # Euler's criterion: chi(a) = a^((q-1)/2) mod q
        for a in range(1, q):
            e = pow(a, (q - 1) // 2, q)
            assert chi[a] == (1 if e == 1 else -1)


@pytest.mark.parametrize("m", [12, 20, 28, 36, 44, 60, 108])
def test_paley_hadamard_is_hadamard(m):
    H = O.paley_hadamard(m)
    assert H.shape == (m, m) and set(np.unique(H)) == {-1, 1}
    np.testing.assert_array_equal(H @ H.T, m * np.eye(m, dtype=np.int64))
    np.testing.assert_array_equal(H.T @ H, m * np.eye(m, dtype=np.int64))


def test_paley_structure():
    # Paley I (q = 11): H - I is skew-symmetric (a skew Hadamard matrix)
    H = O.paley_hadamard(12)
    S = H - np.eye(12, dtype=np.int64)
    np.testing.assert_array_equal(S, -S.T)
    # Paley II (q = 13): the 2x2 blocks are +-[[1, 1], [1, -1]] off the diagonal
    # and [[1, -1], [-1, -1]] on it; H is symmetric
    H = O.paley_hadamard(28)
    np.testing.assert_array_equal(H, H.T)
    for b in range(14):
        np.testing.assert_array_equal(H[2 * b:2 * b + 2, 2 * b:2 * b + 2], [[1, -1], [-1, -1]])
    # Jacobsthal properties: J J^T = q I - ones, rows sum to zero
    for q in (11, 13, 19):
        J = O.jacobsthal(q)
        np.testing.assert_array_equal(J @ J.T, q * np.eye(q, dtype=np.int64) - 1)
        np.testing.assert_array_equal(J.sum(axis=1), 0)
    with pytest.raises(ValueError):
        O.paley_hadamard(52)          # q = 51 and q = 25 are not primes


@pytest.mark.parametrize("n,m", [(3, 12), (2, 20), (4, 28), (0, 12)])
def test_hadamard_kron_against_numpy_kron(n, m):
    rng = np.random.default_rng(n * 100 + m)
    A = 1 << n
    D = A * m
    x = rng.standard_normal((3, D))
    s = rng.choice([-1.0, 1.0], D)
    HA = scipy.linalg.hadamard(A).astype(np.float64)                 # library routine
    Hd = np.kron(HA, O.paley_hadamard(m).astype(np.float64)) / np.sqrt(D)
    np.testing.assert_allclose(O.hadamard_kron(x, m, s), (x * s) @ Hd.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.hadamard_kron(x, m), x @ Hd.T, rtol=0, atol=1e-12)
    # orthogonal: H_d^T undoes it (norm kept)
    y = O.hadamard_kron(x, m, s)
    np.testing.assert_allclose((y @ Hd) * s, x, rtol=0, atol=1e-12)


def test_hadamard_kron_power_of_two_is_the_wht():
    x = np.random.default_rng(5).standard_normal((4, 512))
    np.testing.assert_allclose(O.hadamard_kron(x, 1), O.fwht(x), rtol=0, atol=1e-13)
    ones = np.ones(512)
    np.testing.assert_allclose(O.hadamard_kron(x, 1, ones), O.fwht(x), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_h,D", [(32, 4096), (8, 256), (1, 64), (64, 64), (4, 24)])
def test_head_hadamard_cases(n_h, D):
    x = np.random.default_rng(n_h + D).standard_normal((3, D))
    d_h = D // n_h
    ref = x @ np.kron(scipy.linalg.hadamard(n_h), np.eye(d_h)).T / np.sqrt(n_h)
    np.testing.assert_allclose(O.head_hadamard(x, n_h), ref, rtol=0, atol=1e-12)
    if n_h == 1:
        np.testing.assert_array_equal(O.head_hadamard(x, 1), x)
    if d_h == 1:
        np.testing.assert_allclose(O.head_hadamard(x, n_h), O.fwht(x), rtol=0, atol=1e-13)


def test_head_hadamard_completes_the_full_transform():
    # with n_h and d_h powers of two, (H_{n_h} (x) I)(I (x) H_{d_h}) = H_D: the
    # per-head transform folded into the value/output weights plus the online
    # transform across heads give the whole Walsh-Hadamard transform
    n_h, d_h = 32, 128
    x = np.random.default_rng(9).standard_normal((5, n_h * d_h))
    within = O.fwht(x.reshape(5, n_h, d_h)).reshape(5, -1)
    np.testing.assert_allclose(O.head_hadamard(within, n_h), O.fwht(x), rtol=0, atol=1e-12)


def test_prequant_structured_transforms():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 28 * 16))
    fl = O.FLAG_FWHT | (28 << O.FLAG_KRON_SHIFT)
    Hd = np.kron(scipy.linalg.hadamard(16), O.paley_hadamard(28)) / np.sqrt(28 * 16)
    np.testing.assert_allclose(O.prequant(x, fl), x @ Hd.T, rtol=0, atol=1e-12)
    y = rng.standard_normal((3, 256))
    fl = 3 << O.FLAG_HEADS_SHIFT
    Hh = np.kron(scipy.linalg.hadamard(8), np.eye(32)) / np.sqrt(8)
    np.testing.assert_allclose(O.prequant(y, fl), y @ Hh.T, rtol=0, atol=1e-12)
    # weight preparation folds the same transform into the rows: W' x' = W x
    W = rng.standard_normal((5, 28 * 16))
    s = rng.choice([-1.0, 1.0], 28 * 16)
    _, _, Wr = O.prep_weight(W, True, 4, 28, s)
    xs = O.hadamard_kron(x, 28, s)
    np.testing.assert_allclose(xs @ Wr.astype(np.float64).T, x @ W.T, rtol=0, atol=1e-5)


@pytest.mark.parametrize("D", [2, 4, 8, 64, 256, 1024])
def test_fwht_matches_scipy_sylvester(D):
    Hs = scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D)   # library routine
    np.testing.assert_array_equal(O.hadamard(D), Hs)
    x = np.random.default_rng(D).standard_normal((5, D))
    np.testing.assert_allclose(O.fwht(x), x @ Hs.T, rtol=0, atol=1e-12 * np.sqrt(D))


@pytest.mark.parametrize("D", [16, 4096])
def test_fwht_involution_and_norm(D):
    x = np.random.default_rng(7).standard_normal((3, D))
    y = O.fwht(x)
    np.testing.assert_allclose(O.fwht(y), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_fwht_closed_forms():
    D = 512
    c = 3.0
    out = O.fwht(np.full((1, D), c))
    expect = np.zeros((1, D))
    expect[0, 0] = c * np.sqrt(D)
    np.testing.assert_allclose(out, expect, atol=1e-12)
    # unit vector e_k -> column k of H: (-1)^popcount(i & k) / sqrt(D)
    k = 0b101101011
    e = np.zeros((1, D))
    e[0, k] = 1.0
    idx = np.arange(D)
    sign = np.array([(-1.0) ** bin(i & k).count("1") for i in idx])
    np.testing.assert_allclose(O.fwht(e)[0], sign / np.sqrt(D), atol=1e-15)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.fwht(np.zeros((1, 12)))


# ---------------------------------------------------------------- alignment
def _basis(D, r, key=5, skew=0.02):
    return W.gen_basis(key, D, r, skew_std=skew)


def test_t_hat_is_special_orthogonal():
    Q, M = _basis(64, 8, skew=0.3)
    T = O.t_hat(Q, M)
    # Q, M are fp32 arrays: orthogonality holds to fp32 input accuracy
    np.testing.assert_allclose(T.T @ T, np.eye(64), atol=2e-6)
    assert np.linalg.det(T) == pytest.approx(1.0, abs=1e-5)
    # with exactly orthonormal float64 inputs it holds to 1e-12
    Qd, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((64, 8)))
    A = np.triu(np.random.default_rng(2).normal(0, 0.3, (8, 8)), 1)
    A = A - A.T
    Md = np.linalg.solve(np.eye(8) - A, np.eye(8) + A)
    Td = O.t_hat(Qd, Md)
    np.testing.assert_allclose(Td.T @ Td, np.eye(64), atol=1e-12)
    assert np.linalg.det(Td) == pytest.approx(1.0, abs=1e-12)


# ---------------------------------------------------------------- offline construction
def _rand_orth(rng, D):
    Qm, R = np.linalg.qr(rng.standard_normal((D, D)))
    Qm = Qm * np.sign(np.diag(R))
    if np.linalg.det(Qm) < 0:
        Qm[:, 0] = -Qm[:, 0]
    return Qm


def test_construct_recovers_an_exact_rank_r_transition():
    # T = I + Q0 (M0 - I) Q0^T: Delta T has rank r, its top-r left singular
    # vectors span col(Q0), T_sub = O^T M0 O is orthogonal already, so T_hat = T
    Q0, M0 = W.gen_basis(31, 96, 12, skew_std=0.3)
    Q0, M0 = Q0.astype(np.float64), M0.astype(np.float64)
    Q0, _ = np.linalg.qr(Q0)
    U, _, Vt = np.linalg.svd(M0)
    M0 = U @ Vt                                           # exactly orthogonal in fp64
    T = np.eye(96) + Q0 @ (M0 - np.eye(12)) @ Q0.T
    Q, R, S = O.construct_basis(T, 12)
    np.testing.assert_allclose(O.t_hat(Q, R), T, rtol=0, atol=1e-12)
    assert S[12] < 1e-12 and S[11] > 1e-3
    # the projector onto span(Q) is that of Q0
    np.testing.assert_allclose(Q @ Q.T, Q0 @ Q0.T, rtol=0, atol=1e-12)


def test_construct_full_rank_returns_the_transition():
    T = _rand_orth(np.random.default_rng(3), 24)
    Q, R, _ = O.construct_basis(T, 24)
    np.testing.assert_allclose(O.t_hat(Q, R), T, rtol=0, atol=1e-12)


def test_construct_polar_step():
    T = W.gen_hadamard_transition(5, 64, 6).astype(np.float64)
    Q, R, _ = O.construct_basis(T, 12)
    Tsub = Q.T @ T @ Q
    Rp, Pp = scipy.linalg.polar(Tsub)                         # library routine
    np.testing.assert_allclose(R, Rp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(R.T @ R, np.eye(12), rtol=0, atol=1e-12)
    # nearest orthogonal matrix in the Frobenius norm
    rng = np.random.default_rng(8)
    best = np.linalg.norm(Tsub - R)
    for _ in range(200):
        assert best <= np.linalg.norm(Tsub - _rand_orth(rng, 12)) + 1e-12


def test_construct_tiny_closed_form():
    # T = rot(0.9) (+) rot(0.2) on planes (e0, e1) and (e2, e3); with r = 2 the
    # larger plane is kept: T_hat = rot(0.9) (+) I
    def rot(a):
        return np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
    T = scipy.linalg.block_diag(rot(0.9), rot(0.2))
    Q, R, S = O.construct_basis(T, 2)
    np.testing.assert_allclose(S, [2 * np.sin(0.45)] * 2 + [2 * np.sin(0.1)] * 2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.t_hat(Q, R), scipy.linalg.block_diag(rot(0.9), np.eye(2)),
                               rtol=0, atol=1e-12)


def test_construct_eckart_young_and_special_orthogonal():
    T = W.gen_hadamard_transition(9, 256, 16).astype(np.float64)
    r = 32
    Q, R, S = O.construct_basis(T, r)
    np.testing.assert_allclose(Q.T @ Q, np.eye(r), rtol=0, atol=1e-12)
    dT = T - np.eye(256)
    # the residual of Delta T off span(Q) has 2-norm sigma_{r+1}
    assert np.linalg.norm(dT - Q @ (Q.T @ dT), 2) == pytest.approx(S[r], rel=1e-9)
    Th = O.t_hat(Q, R)
    np.testing.assert_allclose(Th @ Th.T, np.eye(256), rtol=0, atol=1e-12)
    assert np.linalg.det(Th) == pytest.approx(1.0, abs=1e-9)
    # the pages' claim: the approximation keeps most of Delta T
    assert np.linalg.norm(Th - T) < 0.05 * np.linalg.norm(dT)


def test_align_identity_cases():
    x = W.bf16_bits_to_f32(W.gen_x(3, 7, 64, 2, 50.0)).astype(np.float64)
    Q, _ = _basis(64, 8)
    np.testing.assert_array_equal(O.align(x, Q, np.eye(8, dtype=np.float32)), x)   # M = I
    np.testing.assert_array_equal(O.align(x, np.zeros((64, 0)), np.zeros((0, 0))), x)  # r = 0


def test_align_equals_dense_brute_force():
    Q, M = _basis(64, 8, skew=0.2)
    x = np.random.default_rng(11).standard_normal((9, 64))
    np.testing.assert_allclose(O.align(x, Q, M), O.align_dense(x, Q, M), atol=1e-12)
    # and T_hat via an explicit loop over matrix entries
    D, r = Q.shape
    Qd, Md = Q.astype(np.float64), M.astype(np.float64)
    T = np.zeros((D, D))
    for i in range(D):
        for j in range(D):
            s = 1.0 if i == j else 0.0
            for a in range(r):
                for b in range(r):
                    s += Qd[i, a] * (Md[a, b] - (1.0 if a == b else 0.0)) * Qd[j, b]
            T[i, j] = s
    np.testing.assert_allclose(O.t_hat(Q, M), T, atol=1e-13)


def test_align_subspace_cases():
    rng = np.random.default_rng(4)
    Qd, _ = np.linalg.qr(rng.standard_normal((64, 8)))          # exactly orthonormal (f64)
    A0 = np.triu(rng.normal(0, 0.3, (8, 8)), 1)
    Md = np.linalg.solve(np.eye(8) - (A0 - A0.T), np.eye(8) + (A0 - A0.T))
    Q, M = Qd, Md
    # x orthogonal to span(Q): unchanged
    v = rng.standard_normal((3, 64))
    v_perp = v - (v @ Qd) @ Qd.T
    np.testing.assert_allclose(O.align(v_perp, Q, M), v_perp, atol=1e-12)
    # x = Q c inside the subspace: rotated by M inside it (Q M c)
    c = rng.standard_normal((3, 8))
    x_in = c @ Qd.T
    np.testing.assert_allclose(O.align(x_in, Q, M), (Md @ c.T).T @ Qd.T, atol=1e-12)
    # norm kept
    x = rng.standard_normal((4, 64))
    Qo, _ = np.linalg.qr(rng.standard_normal((64, 8)))
    A = np.triu(rng.normal(0, 0.3, (8, 8)), 1)
    A = A - A.T
    Mo = np.linalg.solve(np.eye(8) - A, np.eye(8) + A)
    np.testing.assert_allclose(np.linalg.norm(O.align(x, Qo, Mo), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-12)


def test_align_full_rank_is_conjugated_rotation():
    # r = D: I + Q(M - I)Q^T = Q M Q^T for square orthogonal Q (full-rank reference case)
    rng = np.random.default_rng(9)
    Qo, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    A = np.triu(rng.normal(0, 0.3, (16, 16)), 1)
    A = A - A.T
    Mo = np.linalg.solve(np.eye(16) - A, np.eye(16) + A)
    x = rng.standard_normal((5, 16))
    np.testing.assert_allclose(O.align(x, Qo, Mo), x @ (Qo @ Mo @ Qo.T).T, atol=1e-12)


# ---------------------------------------------------------------- residual add
def test_residual_against_dense_transition():
    """bf16(T_hat x + addend): brute force through the dense T_hat (float64),
    one rounding (f64_to_bf16 is pinned against torch below); the addend joins
    after the alignment, not before it."""
    Q, M = _basis(64, 8, skew=0.3)
    rng = np.random.default_rng(21)
    xb = W.gen_x(21, 6, 64, 2, 30.0)
    ab = W.f32_to_bf16_bits(rng.standard_normal((6, 64)).astype(np.float32))
    x, a = O.bf16_to_f64(xb), O.bf16_to_f64(ab)
    got = O.residual(xb, Q, M, ab)
    np.testing.assert_array_equal(got, O.f64_to_bf16(x @ O.t_hat(Q, M).T + a))
    assert not np.array_equal(got, O.f64_to_bf16((x + a) @ O.t_hat(Q, M).T))
    # M = I: the skip passes unchanged and the sum is the exact bf16 add
    np.testing.assert_array_equal(O.residual(xb, Q, np.eye(8), ab), O.f64_to_bf16(x + a))


def test_residual_rounds_once():
    """D = r = 2, Q = I, M a rotation by theta: the aligned value of x = (c, 0)
    is c cos(theta) = 1 + 2^-8 - 2^-16, just under the midpoint of the bf16
    neighbours 1 and 1 + 2^-7. With the addend 2^-9 the exact sum lies above
    that midpoint, so one rounding gives 1 + 2^-7 (bits 0x3F81); rounding the
    alignment to bf16 first (1) and then the sum 1 + 2^-9 gives 1 (0x3F80)."""
    c = 1.0 + 2.0 ** -7
    cos = (1.0 + 2.0 ** -8 - 2.0 ** -16) / c
    sin = np.sqrt(1.0 - cos * cos)
    M = np.array([[cos, -sin], [sin, cos]])
    xb = O.f64_to_bf16(np.array([[c, 0.0]]))
    ab = O.f64_to_bf16(np.array([[2.0 ** -9, 0.0]]))
    assert O.bf16_to_f64(xb)[0, 0] == c and O.bf16_to_f64(ab)[0, 0] == 2.0 ** -9
    got = O.residual(xb, np.eye(2), M, ab)
    assert got[0, 0] == 0x3F81
    twice = O.f64_to_bf16(O.bf16_to_f64(O.f64_to_bf16(O.align(O.bf16_to_f64(xb), np.eye(2), M)))
                          + O.bf16_to_f64(ab))
    assert twice[0, 0] == 0x3F80


# ---------------------------------------------------------------- quantizer
def test_quant_worked_example():
    g = load("quant_example.txt")
    q, s = O.quant_int4(g["rows"].astype(np.float32))
    np.testing.assert_array_equal(q, g["codes"])
    nd = g["step_num_den"]
    np.testing.assert_array_equal(s, (nd[:, 0].astype(np.float32) / np.float32(7)))
    # dequantized values are exact: both vectors lie on their own grids
    np.testing.assert_array_equal(q * s[:, None], g["rows"].astype(np.float32))


def test_quant_ties_half_even():
    g = load("quant_ties.txt")
    q, s = O.quant_int4(g["rows"].astype(np.float32))
    np.testing.assert_array_equal(s, np.ones(2, np.float32))
    np.testing.assert_array_equal(q, g["codes"])


def _nearest_grid_brute(qf: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Nearest integer of [lo, hi] to each value, ties to the even one, by search."""
    out = np.empty(qf.shape, np.int64)
    for idx, v in np.ndenumerate(qf):
        best, bd = None, None
        for c in range(lo, hi + 1):
            d = abs(float(v) - c)
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        out[idx] = best
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quant_brute_force_and_bounds(bits):
    rng = np.random.default_rng(21 + bits)
    v = (rng.standard_normal((6, 48)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    v[2, 5] = 0.0
    q, s = O.quant_sym(v, bits) if bits != 4 else O.quant_int4(v)
    qmax, qmin = 2 ** (bits - 1) - 1, -2 ** (bits - 1)
    # brute-force step and nearest grid point, in the same fp32 precision
    for t in range(6):
        a = np.float32(max(abs(float(e)) for e in v[t]))
        st = np.float32(a / np.float32(qmax))
        assert s[t] == st
        qf = np.array([np.float32(e / st) for e in v[t]], np.float32)
        np.testing.assert_array_equal(q[t], _nearest_grid_brute(qf, qmin, qmax))
        # RTN bound |v - s q| <= s/2 (+ fp32 rounding of the quotient), max |q| = qmax
        err = np.abs(v[t].astype(np.float64) - float(st) * q[t])
        assert np.all(err <= float(st) * (0.5 + 8 * 2.0 ** -24))
        assert np.abs(q[t]).max() == qmax
    assert q.min() >= qmin and q.max() <= qmax


def test_quant_low_bit_closed_forms():
    # the page's outlier vector on the 3-bit grid: step 20/3, codes [3, 0, 0, 0];
    # after the rotation the flat [10, 10, 10, 10] maps to [3, 3, 3, 3]
    q, s = O.quant_sym(np.array([[20.0, 0, 0, 0], [10.0, 10, 10, 10]], np.float32), 3)
    assert s[0] == np.float32(20.0) / np.float32(3) and s[1] == np.float32(10.0) / np.float32(3)
    np.testing.assert_array_equal(q, [[3, 0, 0, 0], [3, 3, 3, 3]])
    # 2-bit grid: step = absmax, codes in {-1, 0, 1}; 0.5 ties to 0
    q, s = O.quant_sym(np.array([[4.0, 1.9, 2.0, 2.1, -3.0, -2.0]], np.float32), 2)
    assert s[0] == 4.0
    np.testing.assert_array_equal(q[0], [1, 0, 0, 1, -1, 0])


def test_quant_zero_row_and_bits():
    q, s = O.quant_int4(np.zeros((2, 8), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    # 3-bit grid: step absmax/3, codes in [-4, 3]
    v = np.array([[3.0, 1.5, -1.5, 0.4, -3.0, 2.5, 0.0, 0.5]], np.float32)
    q3, s3 = O.quant_sym(v, 3)
    assert s3[0] == np.float32(1.0)
    np.testing.assert_array_equal(q3[0], [3, 2, -2, 0, -3, 2, 0, 0])


def test_pack_example_and_roundtrip():
    g = load("pack_example.txt")
    p = O.pack_int4(g["codes"].astype(np.int8))
    np.testing.assert_array_equal(p, g["bytes"].astype(np.uint8))
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    np.testing.assert_array_equal(O.unpack_int4(O.pack_int4(q)), q)


# ---------------------------------------------------------------- GEMM
def test_gemm_int_against_loop_and_library():
    rng = np.random.default_rng(8)
    qa = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    qw = rng.integers(-8, 8, (7, 64)).astype(np.int8)
    acc = O.gemm_int(qa, qw)
    np.testing.assert_array_equal(acc, O.gemm_int_loop(qa, qw))
    np.testing.assert_array_equal(acc, np.dot(qa.astype(np.int64), qw.astype(np.int64).T))
    # extreme magnitude: all -8 at K = 16384 gives 64 K exactly
    K = 16384
    big = O.gemm_int(np.full((1, K), -8, np.int8), np.full((2, K), -8, np.int8))
    assert big.dtype == np.int32 and np.all(big == 64 * K)


def test_epilogue_example():
    g = load("epilogue_example.txt")
    y = O.epilogue(g["acc"].astype(np.int32), g["s_a"][:, 0].astype(np.float32),
                   g["s_w"][0].astype(np.float32))
    np.testing.assert_array_equal(y, g["y_bits"].astype(np.uint16))


def test_bf16_rounding_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-30, 30, 4096),
                        [0.0, 1.0, -2.5, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 2 ** -130, 3e38]])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f64_to_bf16(v32.astype(np.float64)), ref)
    # and the generator's independent conversion agrees
    np.testing.assert_array_equal(W.f32_to_bf16_bits(v32), ref)
    # f64 input is rounded once (no double rounding through fp32):
    # 1 + 2^-8 + 2^-30 is just above a bf16 tie, so it must round up
    assert O.f64_to_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 0x3F81
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_to_f64(ref), back)


# ---------------------------------------------------------------- invariance and chains
def test_computational_invariance():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((6, 128))
    Wt = rng.standard_normal((10, 128))
    Y = X @ Wt.T
    # R = normalized Hadamard: Y = (X H)(H^T W^T); the row-wise transform applies H
    np.testing.assert_allclose(O.fwht(X) @ O.fwht(Wt).T, Y, rtol=1e-10, atol=1e-10)
    # R = T_hat (orthogonal): W X = (W R)(R^T X)
    Qo, _ = np.linalg.qr(rng.standard_normal((128, 8)))
    A = np.triu(rng.normal(0, 0.3, (8, 8)), 1)
    A = A - A.T
    Mo = np.linalg.solve(np.eye(8) - A, np.eye(8) + A)
    np.testing.assert_allclose(O.align(X, Qo, Mo) @ O.align(Wt, Qo, Mo).T, Y,
                               rtol=1e-10, atol=1e-10)


def test_prequant_order_brute_force():
    Q, M = _basis(64, 8, skew=0.3)
    x = np.random.default_rng(14).standard_normal((4, 64))
    got = O.prequant(x, O.FLAG_ALIGN | O.FLAG_FWHT, Q, M)
    dense = x @ (O.hadamard(64) @ O.t_hat(Q, M)).T        # H T_hat x per token
    np.testing.assert_allclose(got, dense, atol=1e-12)


def test_silu_gate_closed_forms():
    rng = np.random.default_rng(15)
    g = rng.standard_normal((3, 32)) * 4
    u = rng.standard_normal((3, 32))
    h = O.silu_gate(np.concatenate([g, u], axis=1))
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-14, atol=1e-300)
    ones = np.ones_like(g)
    s_pos = O.silu_gate(np.concatenate([g, ones], axis=1))
    s_neg = O.silu_gate(np.concatenate([-g, ones], axis=1))
    np.testing.assert_allclose(s_pos - s_neg, g, atol=1e-13)       # SiLU(g) - SiLU(-g) = g
    z = O.silu_gate(np.concatenate([np.zeros_like(g), u], axis=1))
    assert np.all(z == 0)


def test_rotated_linear_quantization_error_bound():
    """End-to-end float bound: the chain's output differs from the exact
    (H T_hat x)(H w) = (T_hat x) w only by the INT4 rounding of both operands."""
    D, T, N = 256, 16, 24
    Q, M = _basis(D, 8, skew=0.3)
    xb = W.gen_x(31, T, D, 2, 50.0)
    Wf = W.gen_weight(31, N, D, 0.02)
    qw, s_w, wr = O.prep_weight(Wf, rotate=True)
    res = O.rotated_linear(xb, O.FLAG_ALIGN | O.FLAG_FWHT, qw, s_w, Q, M)
    x = O.bf16_to_f64(xb)
    exact = (x @ O.t_hat(Q, M).T) @ Wf.astype(np.float64).T
    y = O.bf16_to_f64(res["y"])
    a = res["prequant32"].astype(np.float64)
    sa = res["s_a"].astype(np.float64)
    sw = s_w.astype(np.float64)
    slack = 0.5 + 8 * 2.0 ** -24
    # |a.w - sa sw qa.qw| <= sa*slack*sum|sw qw| + sw*slack*sum|sa qa| + K sa sw slack^2
    bound = (sa[:, None] * slack * (np.abs(qw) * sw[:, None]).sum(1)[None, :]
             + sw[None, :] * slack * (np.abs(res["codes"]) * sa[:, None]).sum(1)[:, None]
             + D * sa[:, None] * sw[None, :] * slack ** 2)
    # plus: fp32 rounding of the pre-quant values and weights, and the bf16 output rounding
    bound = bound + 1e-5 * np.abs(a) @ np.abs(wr.astype(np.float64)).T + 2.0 ** -8 * np.abs(y)
    assert np.all(np.abs(y - exact) <= bound)
    # The worst-case bound is loose for INT4; a statistical check separates the
    # right chain from plausible wrong ones on this fixed seed: measured 0.167
    # here, 0.28 with the alignment left out, 1.38 with unrotated weights.
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel < 0.2
