"""Pins of the baseline oracles (the cumulative-sum linear attention of the
"Linear Attention" wiki article, "recurrent form" section, and DeltaNet as the
scalar-gate special case of the VLA layer, "Variational Linear Attention"
section 3.5, whose write is the delta rule of the kexue.fm article's "linear
version" section).

Each test ties a baseline to something other than its own recurrence: the
closed-form sum of the state, the article's causal quadratic (attention-like)
readout, the VLA oracle with u = 0, exact recovery with orthonormal keys, and
the delta rule's residual invariant.
"""
import numpy as np
import pytest

import oracle


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def _draw(T, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, d)) for _ in range(3)]


@pytest.mark.parametrize("given", [False, True])
def test_linear_attention_closed_form_state(given):
    """S_T = S_0 + V' Phi(K) (the sum of the rank-1 writes as one product) and
    zkey_T = zkey_0 + sum_t phi(k_t)."""
    T, d = 40, 6
    q, k, v = _draw(T, d, 1)
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((d, d)) if given else None
    z0 = rng.uniform(0.5, 2.0, d) if given else None
    r = oracle.linear_attention_head(q, k, v, S0, z0)
    S_want = v.T @ _phi(k) + (S0 if given else 0.0)
    z_want = _phi(k).sum(axis=0) + (z0 if given else 0.0)
    np.testing.assert_allclose(r["S"], S_want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["zkey"], z_want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("given", [False, True])
def test_linear_attention_causal_quadratic_readout(given):
    """The article's non-recurrent form: with causal weights
    w_ts = phi(k_s)'phi(q_t) for s <= t, o_t = sum_s w_ts v_s / sum_s w_ts
    (plus the initial state's share S_0 phi(q_t) and phi(q_t)'zkey_0)."""
    T, d = 33, 5
    q, k, v = _draw(T, d, 3)
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((d, d)) if given else None
    z0 = rng.uniform(0.5, 2.0, d) if given else None
    r = oracle.linear_attention_head(q, k, v, S0, z0)
    W = np.tril(_phi(q) @ _phi(k).T)            # [t][s], s <= t
    num = W @ v
    den = W.sum(axis=1)
    if given:
        num = num + _phi(q) @ S0.T
        den = den + _phi(q) @ z0
    np.testing.assert_allclose(r["o"], num / den[:, None], rtol=1e-12, atol=1e-13)


def test_deltanet_gate_one_is_vla_with_u_zero():
    """With beta = 1, DeltaNet is the VLA layer with u = 0: A stays I / lambda0, so
    alpha^ = k^ and the writes coincide (section 3.5's special cases)."""
    T, d = 60, 8
    q, k, v = _draw(T, d, 5)
    u = np.zeros((T, d))
    r_vla = oracle.forward_head(q, k, v, u, 0.25, 1e-4)
    r_dn = oracle.deltanet_head(q, k, v, 1.0, 1e-4)
    for key in ("o", "S", "zkey"):
        np.testing.assert_allclose(r_dn[key], r_vla[key], rtol=1e-12, atol=1e-13, err_msg=key)


def test_deltanet_exact_recovery_orthonormal_keys():
    """beta = 1 and orthonormal keys (T <= d): every stored pair is recalled
    exactly, S_T k^_i = v_i, and S_T = sum_i v_i k^_i'."""
    d, T = 8, 6
    rng = np.random.default_rng(6)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm[:T] * rng.uniform(0.5, 3.0, (T, 1))      # orthogonal, any lengths
    v = rng.standard_normal((T, d))
    q = rng.standard_normal((T, d))
    r = oracle.deltanet_head(q, k, v, 1.0, 1e-4)
    kh = _unit(k)
    np.testing.assert_allclose(r["S"] @ kh.T, v.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["S"], v.T @ kh, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("beta", [0.3, 0.75, 1.0])
def test_deltanet_residual_invariant(beta):
    """The delta rule shrinks the current token's residual by 1 - beta on the
    unit key: S_t k^_t - v_t = (1 - beta)(S_{t-1} k^_t - v_t), and leaves S
    unchanged on the complement of k^_t."""
    T, d = 25, 7
    q, k, v = _draw(T, d, 7)
    for t in (1, 9, 24):
        prev = oracle.deltanet_head(q[:t], k[:t], v[:t], beta, 1e-4)["S"]
        cur = oracle.deltanet_head(q[:t + 1], k[:t + 1], v[:t + 1], beta, 1e-4)["S"]
        kh = _unit(k[t])
        np.testing.assert_allclose(cur @ kh - v[t], (1.0 - beta) * (prev @ kh - v[t]),
                                   rtol=1e-11, atol=1e-12)
        P = np.eye(d) - np.outer(kh, kh)
        np.testing.assert_allclose(cur @ P, prev @ P, rtol=1e-11, atol=1e-12)


def test_deltanet_eps_floor_and_zero_key():
    """The Eq. (11) readout floor (queries far below zero) and a zero key (its
    unit key is 0: S unchanged) carry over to the baseline."""
    T, d = 12, 4
    q, k, v = _draw(T, d, 8)
    q[5] = -60.0
    k[7] = 0.0
    r = oracle.deltanet_head(q, k, v, 1.0, 1e-4)
    s6 = oracle.deltanet_head(q[:7], k[:7], v[:7], 1.0, 1e-4)["S"]
    s7 = oracle.deltanet_head(q[:8], k[:8], v[:8], 1.0, 1e-4)["S"]
    np.testing.assert_array_equal(s6, s7)
    s5 = oracle.deltanet_head(q[:6], k[:6], v[:6], 1.0, 1e-4)["S"]
    np.testing.assert_allclose(r["o"][5], s5 @ _phi(q[5]) / 1e-4, rtol=1e-13)


def test_linear_attention_norm_grows_delta_rule_norm_bounded():
    """The contrast of section 4.1 (Prop. 1 and the paragraph after it) on
    associative-recall-shaped inputs (a few keys written again and again): the
    cumulative state's |S|_F grows like T, the delta rule's stays near the norm
    of the stored pairs."""
    d, T, P = 16, 2000, 8
    rng = np.random.default_rng(9)
    keys = _unit(rng.standard_normal((P, d)))
    vals = rng.standard_normal((P, d))
    idx = rng.integers(0, P, T)
    k, v = keys[idx], vals[idx]
    q = rng.standard_normal((T, d))
    la = oracle.linear_attention_head(q, k, v)["S"]
    dn = oracle.deltanet_head(q, k, v, 1.0, 1e-4)["S"]
    la_half = oracle.linear_attention_head(q[:T // 2], k[:T // 2], v[:T // 2])["S"]
    assert np.linalg.norm(la) > 1.8 * np.linalg.norm(la_half)        # ~ linear growth
    assert np.linalg.norm(dn) < 2.0 * np.linalg.norm(vals)             # bounded
    assert np.linalg.norm(la) > 50 * np.linalg.norm(dn)


def test_baseline_all_heads_wrapper():
    rng = np.random.default_rng(10)
    B, H, T, d = 1, 3, 9, 4
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    for kind in ("linear", "delta"):
        res = oracle.baseline(kind, q, k, v, 0.6, 1e-4, workers=2)
        for h in range(H):
            one = (oracle.linear_attention_head(q[0, h], k[0, h], v[0, h]) if kind == "linear"
                   else oracle.deltanet_head(q[0, h], k[0, h], v[0, h], 0.6, 1e-4))
            for key in one:
                np.testing.assert_array_equal(res[key][0, h], one[key])


def test_baseline_scale_trace():
    """The per-token scale is |S_t|_F |phi(q_t)| / den_t with S_t the state after
    token t (checked against runs over each prefix)."""
    T, d = 7, 5
    q, k, v = _draw(T, d, 11)
    for fn, args in ((oracle.linear_attention_head, ()), (oracle.deltanet_head, (0.8, 1e-4))):
        r = fn(q, k, v, *args)
        for t in range(T):
            p = fn(q[:t + 1], k[:t + 1], v[:t + 1], *args)
            den = _phi(q[t]) @ p["zkey"]
            if fn is oracle.deltanet_head:
                den = max(den, 1e-4)
            want = np.linalg.norm(p["S"]) * np.linalg.norm(_phi(q[t])) / den
            assert abs(r["scale"][t] - want) <= 1e-12 * want
