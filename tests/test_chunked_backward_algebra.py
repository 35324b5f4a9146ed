"""The chunked form of the reverse sweep, in fp64, against the oracle's reverse mode.

The pages give the forward recurrence ("Variational Linear Attention", arXiv
2605.11196, section 3.3, Eqs. (9)-(11)) and no backward; the oracle's
``backward_head`` is its chain rule token by token (pinned in
test_oracle_grad_pins.py).  At d = 64 the sweep kernels (bwd_mc and bwd_pc in
vla_bwd_split.hip) advance sixteen tokens per step: each chain's per-token
recurrence unrolled over a chunk, products of the d x d states with 16-column
blocks plus 16 x 16 triangular couplings.  This test writes those chunk
formulas out in fp64 (columns = tokens of the chunk, states at the chunk's
end) and checks that they reproduce the oracle's gradients to rounding, at a
ragged length; a plausible slip in any coupling (a mask's diagonal, a dropped
term) must break the agreement.
"""
import numpy as np
import pytest

import oracle

LAMBDA0, EPS, C = 0.1, 1e-4, 16


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _dphi(x):
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def _head(T, d, seed):
    rng = np.random.default_rng(seed)
    q, k, v, u = (rng.standard_normal((T, d)) for _ in range(4))
    dO = rng.standard_normal((T, d))
    return q, k, v, u, dO


def chunked_backward(q, k, v, u, dO, slip=None):
    """Gradients of one head (default initial state, dL/do only) by the chunk
    formulas; ``slip`` plants one mistake for the sensitivity test."""
    T, d = q.shape
    fw = oracle.forward_head(q, k, v, u, LAMBDA0, EPS, trace=True)
    kn, un = np.linalg.norm(k, axis=1), np.linalg.norm(u, axis=1)
    kh, uh = k / kn[:, None], u / un[:, None]
    al, z, dl, e, den = fw["alpha"], fw["z"], fw["delta"], fw["e"], fw["den"]
    # |y_t| with y_t = A_t k^_t = alpha^_t |y_t|
    yn = np.linalg.norm(np.einsum("tij,tj->ti", fw["A_t"], kh), axis=1)
    zk = np.cumsum(_phi(k), axis=0)
    pq = _phi(q)
    iden = 1.0 / np.maximum(den, EPS)
    gm = dO * iden[:, None]

    G = np.zeros((d, d))                 # dL/dS
    Q = np.zeros((d, d))                 # A Sigma A
    A, S = fw["A"].copy(), fw["S"].copy()
    out = {n: np.zeros((T, d)) for n in ("ge", "p", "w", "c1", "c2")}
    for c0 in range((T - 1) // C * C, -1, -C):
        sl = slice(c0, min(T, c0 + C))
        n = sl.stop - sl.start
        Al, Kh, Ph, GM, E, Z, U, Go = (x[sl].T for x in (al, kh, pq, gm, e, z, uh, dO))
        ge_ = np.triu(np.ones((n, n)))       # [s, t] = 1 for s <= t
        le_ = ge_.T                          # s >= t
        gt_ = np.tril(np.ones((n, n)), -1)   # s > t
        # memory chain: GE (I + L) = G Al + GM (mask_{s>=t} Ph'Al), L[s, t] = k^_s'alpha^_t (s > t)
        L = (Kh.T @ Al) * gt_
        GE = (G @ Al + GM @ ((Ph.T @ Al) * le_)) @ np.linalg.inv(np.eye(n) + L)
        GA = G.T @ E + Ph @ ((GM.T @ E) * (gt_ if slip == "ga_diag" else le_)) \
            - Kh @ ((GE.T @ E) * gt_)
        G = G + GM @ Ph.T - GE @ Kh.T
        # penalty chain in the conjugated frame
        GY = (GA - Al * np.sum(Al * GA, axis=0)) / yn[sl]
        Y = Al * yn[sl]
        P = A @ GY + Z @ ((Z.T @ GY) / dl[sl][:, None] * (le_ if slip == "p_diag" else gt_))
        V3 = (P.T @ U) * le_
        W = Q @ U + P @ ((Y.T @ U) * le_) + (0.0 if slip == "w_term" else Y @ V3)
        Q = Q + P @ Y.T + Y @ P.T
        A = A + Z @ np.diag(1.0 / dl[sl]) @ Z.T
        C1 = S.T @ Go - Al @ ((E.T @ Go) * gt_)
        C2 = S.T @ GE - Al @ ((E.T @ GE) * (le_ if slip == "c2_diag" else gt_))
        S = S - E @ Al.T
        for nme, x in (("ge", GE), ("p", P), ("w", W), ("c1", C1), ("c2", C2)):
            out[nme][sl] = x.T
    # per-token gradients from the chunk results
    dq, dk, du = np.zeros((T, d)), np.zeros((T, d)), np.zeros((T, d))
    gzk = np.zeros(d)
    for t in range(T - 1, -1, -1):
        c1 = out["c1"][t]
        gden = -(c1 @ pq[t]) * iden[t] ** 2 if den[t] >= EPS else 0.0
        dq[t] = (c1 * iden[t] + gden * zk[t]) * _dphi(q[t])
        gzk = gzk + gden * pq[t]
        gkh = al[t] * (e[t] @ out["ge"][t]) - out["c2"][t] + out["p"][t]
        dk[t] = (gkh - kh[t] * (kh[t] @ gkh)) / kn[t] + gzk * _dphi(k[t])
        w = out["w"][t]
        du[t] = -(w - uh[t] * (uh[t] @ w)) / un[t]
    return dict(dq=dq, dk=dk, dv=out["ge"], du=du, dS0=G,
                dA0=0.5 * LAMBDA0 * LAMBDA0 * Q, dzkey0=gzk)


def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


@pytest.mark.parametrize("T,d", [(100, 12), (48, 8), (7, 5)])
def test_chunk_formulas_match_the_token_chain_rule(T, d):
    q, k, v, u, dO = _head(T, d, seed=T + d)
    ref = oracle.backward_head(q, k, v, u, dO, LAMBDA0, EPS)
    got = chunked_backward(q, k, v, u, dO)
    for name in ("dq", "dk", "dv", "du", "dS0", "dA0", "dzkey0"):
        assert _rel(got[name], ref[name]) < 1e-10, name


@pytest.mark.parametrize("slip", ["ga_diag", "p_diag", "w_term", "c2_diag"])
def test_a_slip_in_the_chunk_couplings_is_seen(slip):
    q, k, v, u, dO = _head(100, 12, seed=1)
    ref = oracle.backward_head(q, k, v, u, dO, LAMBDA0, EPS)
    got = chunked_backward(q, k, v, u, dO, slip=slip)
    worst = max(_rel(got[n], ref[n]) for n in ("dq", "dk", "dv", "du", "dS0", "dA0", "dzkey0"))
    assert worst > 1e-4
