"""Pins of the oracle's gradients (``oracle.backward_head``).

The pages give the forward recurrence ("Variational Linear Attention",
arXiv 2605.11196, section 3.3, Eqs. (9)-(11)) and say it is trained end to end;
its reverse mode is the chain rule through those equations.  Each test ties the
oracle's gradients to something other than their own formulas: central finite
differences of the oracle forward (itself pinned in test_oracle_pins.py), entry
by entry on tiny heads and along random directions on larger ones, and the
first token's gradient worked by hand.
"""
import numpy as np
import pytest

import oracle

LAMBDA0, EPS = 0.1, 1e-4


def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _spd(d, rng):
    m = rng.standard_normal((d, d))
    return m @ m.T / d + 0.5 * np.eye(d)


def _case(T, d, seed):
    rng = np.random.default_rng(seed)
    x = {n: rng.standard_normal((T, d)) for n in ("q", "k", "v", "u")}
    x["S0"] = 0.5 * rng.standard_normal((d, d))
    x["A0"] = _spd(d, rng)
    x["zkey0"] = rng.uniform(0.5, 2.0, d)
    adj = dict(dO=rng.standard_normal((T, d)), dS_T=rng.standard_normal((d, d)),
               dA_T=rng.standard_normal((d, d)), dzkey_T=rng.standard_normal(d))
    return x, adj


def _loss(x, adj):
    """sum dO.o + <dS_T, S_T> + <dA_T, A_T> + dzkey_T.zkey_T from the oracle forward."""
    r = oracle.forward_head(x["q"], x["k"], x["v"], x["u"], LAMBDA0, EPS,
                            x["S0"], x["A0"], x["zkey0"])
    return (np.sum(adj["dO"] * r["o"]) + np.sum(adj["dS_T"] * r["S"])
            + np.sum(adj["dA_T"] * r["A"]) + np.dot(adj["dzkey_T"], r["zkey"]))


def _grads(x, adj):
    return oracle.backward_head(x["q"], x["k"], x["v"], x["u"], adj["dO"], LAMBDA0, EPS,
                                x["S0"], x["A0"], x["zkey0"], adj["dS_T"], adj["dA_T"],
                                adj["dzkey_T"])


def _fd_entry(x, adj, name, idx, h, sym=False):
    """Central difference of the loss in one entry (A0: the symmetric pair)."""
    def shifted(s):
        y = {n: a.copy() for n, a in x.items()}
        y[name][idx] += s
        if sym and idx[0] != idx[1]:
            y[name][idx[::-1]] += s
        return y
    return (_loss(shifted(h), adj) - _loss(shifted(-h), adj)) / (2 * h)


GRAD_OF = dict(q="dq", k="dk", v="dv", u="du", S0="dS0", A0="dA0", zkey0="dzkey0")


def _check_entrywise(x, adj, skip=(), h=1e-6, rtol=2e-6):
    g = _grads(x, adj)
    for name, gname in GRAD_OF.items():
        scale = max(1.0, np.abs(g[gname]).max())
        for idx in np.ndindex(*x[name].shape):
            if (name, idx[0]) in skip:
                continue
            if name == "A0":
                if idx[0] > idx[1]:
                    continue
                fd = _fd_entry(x, adj, name, idx, h, sym=True)
                # a symmetric perturbation of an off-diagonal pair moves both entries
                want = g[gname][idx] * (2.0 if idx[0] != idx[1] else 1.0)
            else:
                fd = _fd_entry(x, adj, name, idx, h)
                want = g[gname][idx]
            assert abs(fd - want) <= rtol * scale, (name, idx, fd, want)
    return g


def test_grad_entrywise_finite_differences():
    """Every gradient entry of a d = 3, T = 7 head with a general initial state
    and adjoints on every output, against central differences of the forward."""
    x, adj = _case(7, 3, seed=11)
    _check_entrywise(x, adj)


def test_grad_entrywise_floor_and_zero_vectors():
    """The same with the denominator floor active (phi(q)'zkey far below eps),
    a zero key and a zero penalty vector.  At the zero vectors the
    normalisation has no derivative: those entries are left out of the
    comparison, and the zero u gets no gradient (the stated convention)."""
    x, adj = _case(9, 3, seed=12)
    # tokens 0, 1: keys far below zero and zkey_0 = 0 keep phi(q)'zkey ~ 1e-8
    # with phi(q) of order one, so the floor decides den where the gradient
    # through the key sum would be large
    x["zkey0"][:] = 0.0
    x["k"][0] = [-20.0, -21.0, -19.5]
    x["k"][1] = [-19.0, -20.5, -20.0]
    adj["dO"][:2] *= 1e-4   # o there is S phi(q) / eps ~ 1e4: keep the loss's rounding small
    x["q"][5] = [-40.0, -41.0, -39.0]   # phi(q) ~ 4e-18
    x["k"][3] = 0.0
    x["u"][6] = 0.0
    r = oracle.forward_head(x["q"], x["k"], x["v"], x["u"], LAMBDA0, EPS, x["S0"], x["A0"],
                            x["zkey0"], trace=True)
    assert r["den"][0] == EPS and r["den"][1] == EPS and r["den"][5] == EPS
    assert r["den"][2] > 10 * EPS
    g = _check_entrywise(x, adj, skip={("k", 3), ("u", 6)})
    assert np.all(g["du"][6] == 0.0)


@pytest.mark.parametrize("T,d,seed", [(48, 16, 21), (24, 32, 22)])
def test_grad_directional_finite_differences(T, d, seed):
    """Directional derivative along a random direction in every input and the
    initial state at once, against the gradients' inner product with it."""
    x, adj = _case(T, d, seed)
    g = _grads(x, adj)
    rng = np.random.default_rng(seed + 100)
    r = {n: rng.standard_normal(a.shape) for n, a in x.items()}
    r["A0"] = r["A0"] + r["A0"].T
    h = 1e-6

    def at(s):
        return _loss({n: x[n] + s * r[n] for n in x}, adj)
    fd = (at(h) - at(-h)) / (2 * h)
    want = sum(np.sum(g[GRAD_OF[n]] * r[n]) for n in x)
    assert abs(fd - want) <= 1e-6 * max(1.0, abs(want)), (fd, want)


def test_grad_first_token_by_hand():
    """One token from the default state (S_0 = 0, A_0 = I / lambda0, zkey_0 = 0):
    S_1 = v alpha^', o = v (alpha^'phi(q)) / den with den = phi(q)'phi(k), and
    A_1 k^ = k^/lambda0 - u^ (u^'k^) / (lambda0^2 (1 + 1/lambda0)).  With
    L = dO.o + <dS_T, S_1>:  dv = dO s / den + dS_T alpha^ (s = alpha^'phi(q)),
    and dq = phi'(q) (dO.v) (alpha^ / den - s phi(k) / den^2)."""
    rng = np.random.default_rng(31)
    d = 5
    q, k, v, u = (rng.standard_normal((1, d)) for _ in range(4))
    dO, dS_T = rng.standard_normal((1, d)), rng.standard_normal((d, d))
    g = oracle.backward_head(q, k, v, u, dO, LAMBDA0, EPS, dS_T=dS_T)
    kh, uh = _unit(k[0]), _unit(u[0])
    y = kh / LAMBDA0 - uh * (uh @ kh) / (LAMBDA0 ** 2 * (1.0 + 1.0 / LAMBDA0))
    al = y / np.linalg.norm(y)
    pq, pk = _phi(q[0]), _phi(k[0])
    den = pq @ pk
    assert den > EPS
    s = al @ pq
    np.testing.assert_allclose(g["dv"][0], dO[0] * s / den + dS_T @ al, rtol=1e-12, atol=1e-13)
    dphi_q = np.where(q[0] > 0, 1.0, np.exp(np.minimum(q[0], 0.0)))
    want_dq = dphi_q * (dO[0] @ v[0]) * (al / den - s * pk / den ** 2)
    np.testing.assert_allclose(g["dq"][0], want_dq, rtol=1e-12, atol=1e-13)


def test_grad_heads_independent():
    """The all-heads wrapper gives each head's own gradients."""
    rng = np.random.default_rng(41)
    B, H, T, d = 1, 2, 6, 4
    q, k, v, u, dO = (rng.standard_normal((B, H, T, d)) for _ in range(5))
    res = oracle.backward(q, k, v, u, dO, LAMBDA0, EPS, workers=2)
    for h in range(H):
        one = oracle.backward_head(q[0, h], k[0, h], v[0, h], u[0, h], dO[0, h], LAMBDA0, EPS)
        for key in one:
            np.testing.assert_array_equal(res[key][0, h], one[key])


@pytest.mark.parametrize("seg", [1, 7, 16, 60])
def test_grad_checkpointed_equals_whole(seg):
    """backward_head_checkpointed (segments of seg tokens, ragged last one)
    gives backward_head's gradients, with a general initial state and adjoints
    on every output; and along a random direction it matches central
    differences of the forward by itself."""
    x, adj = _case(50, 6, seed=51)
    whole = _grads(x, adj)
    ck = oracle.backward_head_checkpointed(x["q"], x["k"], x["v"], x["u"], adj["dO"], LAMBDA0,
                                           EPS, x["S0"], x["A0"], x["zkey0"], adj["dS_T"],
                                           adj["dA_T"], adj["dzkey_T"], seg=seg)
    for n, g in whole.items():
        np.testing.assert_allclose(ck[n], g, rtol=1e-11, atol=1e-12 * np.abs(g).max())
    rng = np.random.default_rng(52)
    r = {n: rng.standard_normal(a.shape) for n, a in x.items()}
    r["A0"] = r["A0"] + r["A0"].T
    h = 1e-6
    fd = (_loss({n: x[n] + h * r[n] for n in x}, adj)
          - _loss({n: x[n] - h * r[n] for n in x}, adj)) / (2 * h)
    want = sum(np.sum(ck[GRAD_OF[n]] * r[n]) for n in x)
    assert abs(fd - want) <= 1e-6 * max(1.0, abs(want)), (fd, want)
