"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test ties a step of the oracle to something other than the oracle's own
formula: a brute-force inverse, a hand-worked example, a closed form, a special
case that reduces to a textbook recurrence, or an invariant that only the right
update satisfies.  Source: "Variational Linear Attention" (arXiv 2605.11196),
sections 3.2-3.5 and 4 (Eqs. 9-14, Propositions 1-3); the delta rule from the
kexue.fm article on linearising attention ("linear version" section); the
cumulative-sum linear attention from the "Linear Attention" wiki article
("recurrent form" section).
"""
import json
import math
import os

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GOLDEN_RATIO = (1.0 + math.sqrt(5.0)) / 2.0


def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _rand(T, d, seed, unit_u=False):
    rng = np.random.default_rng(seed)
    q, k, v, u = (rng.standard_normal((T, d)) for _ in range(4))
    if unit_u:
        u = _unit(u)
    return q, k, v, u


# ------------------------------------------------------------ hand-worked example
def test_hand_worked_two_tokens():
    """Two tokens at d = 2 worked by hand from Eqs. (9)-(11)
    (tests/golden/hand_two_tokens_d2.json holds the derivation)."""
    with open(os.path.join(GOLDEN, "hand_two_tokens_d2.json")) as f:
        fx = json.load(f)
    inp = {n: np.array(fx["inputs"][n]) for n in "qkvu"}
    r = oracle.forward_head(inp["q"], inp["k"], inp["v"], inp["u"],
                            fx["lambda0"], fx["eps"], trace=True)
    exp = {n: np.array(x) for n, x in fx["expected"].items()}
    # The closed forms again, evaluated here, guard the stored numbers.
    rr, e1 = math.sqrt(7780.0), math.exp(-1.0)
    assert np.allclose(exp["o"][1], [(6 * e1 / rr - 2) / (5 + 6 * e1), (-6 * e1 / rr) / (5 + 6 * e1)],
                       rtol=0, atol=1e-15)
    assert np.allclose(exp["o"][0], [13 / rr, -13 / rr], rtol=0, atol=1e-15)
    for name in ("delta", "alpha", "e", "den", "o"):
        np.testing.assert_allclose(r[name], exp[name], rtol=1e-14, atol=1e-15, err_msg=name)
    np.testing.assert_allclose(r["A_t"][0], exp["A_1"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["S_t"][0], exp["S_1"], rtol=1e-14, atol=1e-15)
    for name in ("A", "S", "zkey"):
        np.testing.assert_allclose(r[name], exp[name], rtol=1e-14, atol=1e-15, err_msg=name)


# --------------------------------------------------------- penalty recurrence (Eq. 9)
@pytest.mark.parametrize("T,d,seed,unit_u", [(32, 4, 11, False), (256, 16, None, True)])
def test_A_equals_bruteforce_inverse(T, d, seed, unit_u):
    """A_t = (lambda0 I + sum_{s<=t} u^_s u^_s')^-1 at every t (section 3.2/3.3:
    A_t = M_t^-1 maintained by Sherman-Morrison)."""
    lam = 0.1
    if seed is None:  # the single-head workload's own inputs
        hi = gen.head_inputs(gen.config(1), 0, 0)
        q, k, v, u = (hi[n].astype(np.float64) for n in "qkvu")
    else:
        q, k, v, u = _rand(T, d, seed, unit_u)
    r = oracle.forward_head(q, k, v, u, lam, 1e-4, trace=True)
    uh = _unit(u)
    M = lam * np.eye(d)
    worst = 0.0
    for t in range(T):
        M = M + np.outer(uh[t], uh[t])
        Ainv = np.linalg.inv(M)
        worst = max(worst, np.abs(r["A_t"][t] - Ainv).max() / np.abs(Ainv).max())
    assert worst < 1e-10


def test_A_with_initial_state_bruteforce():
    """From a given SPD A_0: A_t = (A_0^-1 + sum u^ u^')^-1."""
    d, T = 6, 40
    rng = np.random.default_rng(5)
    G = rng.standard_normal((d, d))
    A0 = np.linalg.inv(G @ G.T + 0.5 * np.eye(d))
    q, k, v, u = _rand(T, d, 6)
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, A0=A0, trace=True)
    M = np.linalg.inv(A0)
    uh = _unit(u)
    for t in range(T):
        M = M + np.outer(uh[t], uh[t])
        np.testing.assert_allclose(r["A_t"][t], np.linalg.inv(M), rtol=1e-9, atol=1e-12)


def test_delta_at_least_one_and_A_spd():
    """delta_t >= 1 because A_{t-1} is positive definite (section 3.3); A_t stays
    symmetric (bit-exact) and positive definite."""
    q, k, v, u = _rand(300, 12, 21)
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, trace=True)
    assert np.all(r["delta"] >= 1.0)
    for t in range(0, 300, 7):
        At = r["A_t"][t]
        assert np.array_equal(At, At.T)
        np.linalg.cholesky(At)


# ----------------------------------------------------------------- gate (Eq. 10)
def test_alpha_is_normalised_updated_A_times_khat():
    """alpha^_t = A_t k^_t / |A_t k^_t| with the *updated* A_t, computed here from
    the brute-force inverse; |alpha^| = 1 and c_t = alpha^'k^ lies in (0, 1]."""
    d, T, lam = 8, 120, 0.1
    q, k, v, u = _rand(T, d, 31)
    r = oracle.forward_head(q, k, v, u, lam, 1e-4, trace=True)
    kh, uh = _unit(k), _unit(u)
    M = lam * np.eye(d)
    for t in range(T):
        M = M + np.outer(uh[t], uh[t])
        y = np.linalg.solve(M, kh[t])
        np.testing.assert_allclose(r["alpha"][t], y / np.linalg.norm(y), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(r["alpha"], axis=1), 1.0, atol=1e-12)
    c = np.sum(r["alpha"] * kh, axis=1)
    assert np.all(c > 0) and np.all(c <= 1 + 1e-12)


def test_jacobian_norm_closed_form():
    """J_t = I - alpha^ k^' (Eq. 14).  Its spectral norm is
    sqrt((3 - 2c + sqrt(5 - 4c)) / 2) with c = alpha^'k^ (derived from the 2x2
    action on span{alpha^, k^}); it lies in [1, golden ratio) and equals 1 only
    when alpha^ = k^ (Proposition 2's value 1 holds in that case, e.g. u = 0)."""
    d, T = 10, 60
    q, k, v, u = _rand(T, d, 41)
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, trace=True)
    kh = _unit(k)
    for t in range(T):
        J = np.eye(d) - np.outer(r["alpha"][t], kh[t])
        s = np.linalg.svd(J, compute_uv=False)[0]
        c = float(r["alpha"][t] @ kh[t])
        assert abs(s - math.sqrt((3 - 2 * c + math.sqrt(5 - 4 * c)) / 2)) < 1e-12
        assert 1 - 1e-12 <= s < GOLDEN_RATIO
    r0 = oracle.forward_head(q, k, v, np.zeros_like(u), 0.1, 1e-4, trace=True)
    for t in range(T):
        J = np.eye(d) - np.outer(r0["alpha"][t], kh[t])
        assert abs(np.linalg.svd(J, compute_uv=False)[0] - 1.0) < 1e-12


# --------------------------------------------------------- state write (Eq. 10)
def test_state_update_invariants():
    """Two properties that together fix S_t given S_{t-1} (for c_t != 0):
    (i) S_t x = S_{t-1} x for every x orthogonal to alpha^_t (rank-1 write along
    alpha^_t); (ii) S_t k^_t - v_t = (1 - c_t)(S_{t-1} k^_t - v_t), c_t = alpha^'k^."""
    d, T = 9, 80
    q, k, v, u = _rand(T, d, 51)
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, trace=True)
    kh = _unit(k)
    Sprev = np.zeros((d, d))
    for t in range(T):
        St, a = r["S_t"][t], r["alpha"][t]
        P = np.eye(d) - np.outer(a, a)
        np.testing.assert_allclose(St @ P, Sprev @ P, rtol=0, atol=1e-11)
        c = a @ kh[t]
        np.testing.assert_allclose(St @ kh[t] - v[t], (1 - c) * (Sprev @ kh[t] - v[t]),
                                   rtol=0, atol=1e-11)
        Sprev = St


def test_frobenius_bound_prop1():
    """|S_t|_F <= |S_0|_F + sum_{s<=t} |e_s| (Proposition 1, Eq. 13)."""
    d, T = 16, 400
    q, k, v, u = _rand(T, d, 61)
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, trace=True)
    bound = np.cumsum(np.linalg.norm(r["e"], axis=1))
    normS = np.linalg.norm(r["S_t"].reshape(T, -1), axis=1)
    assert np.all(normS <= bound * (1 + 1e-9))


# ------------------------------------------------- special cases (section 3.5)
def test_u_zero_reduces_to_delta_rule():
    """u = 0: no penalty update, A stays I/lambda0 exactly, alpha^ = k^, and S
    follows the delta rule W_t = W_{t-1} - (W_{t-1} k^ - v) k^' (step size 1) of
    the kexue.fm 'linear version' section, with normalised keys."""
    d, T, lam = 12, 150, 0.1
    q, k, v, u = _rand(T, d, 71)
    r = oracle.forward_head(q, k, v, np.zeros_like(u), lam, 1e-4, trace=True)
    assert np.array_equal(r["A"], np.eye(d) / lam)
    kh = _unit(k)
    W = np.zeros((d, d))
    for t in range(T):
        W = W - np.outer(W @ kh[t] - v[t], kh[t])
        np.testing.assert_allclose(r["S_t"][t], W, rtol=0, atol=1e-11)


def test_orthonormal_keys_cumulative_linear_attention():
    """u = 0 with mutually orthogonal keys (T <= d): the state is the cumulative
    sum sum_s v_s k^_s' of linear attention, every stored value is recovered
    exactly (Proposition 3's exact recovery in this case), and the readout equals
    the causal quadratic (attention-matrix) form of linear attention with k^ in
    the numerator and phi(k) in the denominator."""
    d, T = 16, 12
    rng = np.random.default_rng(81)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    scales = rng.uniform(0.5, 3.0, size=(T, 1))
    k = Qm[:T] * scales           # orthogonal, not unit length
    q = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    r = oracle.forward_head(q, k, v, np.zeros((T, d)), 0.1, 1e-4, trace=True)
    kh = _unit(k)
    np.testing.assert_allclose(r["S"], v.T @ kh, rtol=0, atol=1e-12)
    for i in range(T):
        np.testing.assert_allclose(r["S"] @ kh[i], v[i], rtol=0, atol=1e-12)
    pq, pk = _phi(q), _phi(k)
    mask = np.tril(np.ones((T, T)))
    num = (mask * (pq @ kh.T)) @ v
    den = np.maximum((mask * (pq @ pk.T)).sum(axis=1), 1e-4)
    np.testing.assert_allclose(r["o"], num / den[:, None], rtol=1e-12, atol=1e-13)


def test_d1_closed_form():
    """d = 1: u^ = sign(u) so A_t = 1/(lambda0 + t); alpha^ = k^ = sign(k) so
    S_t = v_t k^_t; o_t = v_t k^_t phi(q_t) / max(phi(q_t) sum_{s<=t} phi(k_s), eps).
    Very negative q puts some tokens in the eps branch of the denominator."""
    T, lam, eps = 64, 0.1, 1e-4
    rng = np.random.default_rng(91)
    q = rng.standard_normal((T, 1)) * 3
    q[::5] = -40.0                      # phi(q) = e^-40: denominator clamps to eps
    k = rng.standard_normal((T, 1)) * 2
    v = rng.standard_normal((T, 1))
    u = rng.standard_normal((T, 1))
    r = oracle.forward_head(q, k, v, u, lam, eps, trace=True)
    t1 = np.arange(1, T + 1)
    np.testing.assert_allclose(r["A_t"][:, 0, 0], 1.0 / (lam + t1), rtol=1e-13)
    sk = np.sign(k[:, 0])
    np.testing.assert_allclose(r["S_t"][:, 0, 0], v[:, 0] * sk, rtol=1e-13, atol=1e-15)
    pq = np.where(q[:, 0] > 0, q[:, 0] + 1, np.exp(np.minimum(q[:, 0], 0)))
    pk = np.where(k[:, 0] > 0, k[:, 0] + 1, np.exp(np.minimum(k[:, 0], 0)))
    den = np.maximum(pq * np.cumsum(pk), eps)
    assert np.sum(den == eps) >= T // 5
    np.testing.assert_allclose(r["o"][:, 0], v[:, 0] * sk * pq / den, rtol=1e-13, atol=1e-300)


def test_zero_vectors_leave_state_unchanged():
    """Reading for zero vectors: u = 0 leaves A unchanged, k = 0 leaves S
    unchanged (alpha^ = 0), and the key sum still gains phi(0) = 1 per entry."""
    d, T = 5, 30
    q, k, v, u = _rand(T, d, 101)
    u[7] = 0.0
    k[11] = 0.0
    r = oracle.forward_head(q, k, v, u, 0.1, 1e-4, trace=True)
    np.testing.assert_array_equal(r["A_t"][7], r["A_t"][6])
    assert r["delta"][7] == 1.0
    np.testing.assert_array_equal(r["S_t"][11], r["S_t"][10])
    np.testing.assert_array_equal(r["alpha"][11], 0.0)


# ------------------------------------------------------- state continuation
def test_continuation_and_empty_sequence():
    """forward(T1 + T2) == forward(T1) then forward(T2 | final state); T = 0
    returns the initial state unchanged."""
    d, T1, T2 = 8, 37, 29
    q, k, v, u = _rand(T1 + T2, d, 111)
    full = oracle.forward_head(q, k, v, u)
    a = oracle.forward_head(q[:T1], k[:T1], v[:T1], u[:T1])
    b = oracle.forward_head(q[T1:], k[T1:], v[T1:], u[T1:], S0=a["S"], A0=a["A"], zkey0=a["zkey"])
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]]), full["o"], rtol=1e-13, atol=1e-15)
    for n in ("S", "A", "zkey"):
        np.testing.assert_allclose(b[n], full[n], rtol=1e-13, atol=1e-15)
    e = oracle.forward_head(np.zeros((0, d)), np.zeros((0, d)), np.zeros((0, d)),
                            np.zeros((0, d)), S0=a["S"], A0=a["A"], zkey0=a["zkey"])
    for n in ("S", "A", "zkey"):
        np.testing.assert_array_equal(e[n], a[n])
    e0 = oracle.forward_head(np.zeros((0, d)), np.zeros((0, d)), np.zeros((0, d)), np.zeros((0, d)))
    np.testing.assert_array_equal(e0["A"], np.eye(d) * 10.0)
    np.testing.assert_array_equal(e0["S"], 0.0)


def test_head_independence():
    """Every quantity is per head (section 3.5, Table 1): permuting heads
    permutes outputs, and changing one head leaves the others bit-identical."""
    cfg = gen.config(2).with_sizes(B=2, H=3, T=40)
    x = gen.make_inputs(cfg)
    base = oracle.forward(x["q"], x["k"], x["v"], x["u"])
    perm = [2, 0, 1]
    p = oracle.forward(*(x[n][:, perm] for n in "qkvu"))
    for n in ("o", "S", "A", "zkey"):
        np.testing.assert_array_equal(p[n], base[n][:, perm])
    x2 = {n: x[n].copy() for n in "qkvu"}
    x2["v"][1, 2] += 1.0
    c = oracle.forward(*(x2[n] for n in "qkvu"))
    for n in ("o", "S", "A", "zkey"):
        np.testing.assert_array_equal(c[n][0], base[n][0])
        np.testing.assert_array_equal(c[n][1, :2], base[n][1, :2])
    assert not np.array_equal(c["o"][1, 2], base["o"][1, 2])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((3, 4))
    with pytest.raises(ValueError):
        oracle.forward_head(q, q, q, q, lambda0=0.0)
    with pytest.raises(ValueError):
        oracle.forward_head(q, q, q, q, eps=-1.0)
