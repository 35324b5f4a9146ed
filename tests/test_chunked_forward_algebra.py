"""The chunked form of the forward, in fp64, against the oracle's token chain.

The oracle runs the recurrence of "Variational Linear Attention" (arXiv
2605.11196, section 3.3, Eqs. (9)-(11)) one token at a time.  The two-pass
forward (vla_twopass.hip) advances sixteen tokens per step instead:

* penalty chain, per chunk with A at its start and U^, K^ the chunk's unit
  vectors as columns: Z0 = A U^, Y0 = A K^, I + G = I + U^'Z0 = L D L'; the
  downdate A <- A - Z0 (I + G)^-1 Z0' (the chunk's sixteen Sherman-Morrison
  steps of Eq. (9) as one Woodbury step, with -(I + G)^-1 formed explicitly);
  the gate inputs W = Y0 - Z0 L^-T ((D^-1 L^-1 Z0'K^) o Up) (column t is
  A_t k^_t, A after token t's own downdate; U^'A K^ = Z0'K^ as A is
  symmetric); alpha^_t = w_t / |w_t| (Eq. (10));
* segments: a chunk chain may start mid-sequence from
  A = (A_0^-1 + sum of the earlier u^ u^')^-1 (Eq. (9) summed);
* memory chain, per pair of chunks (a, b) with S at the pair's start:
  N = (Alpha^'K^) o strict-Up, T = (I + N)^-1; E_a = (V_a - S K^_a) T_a;
  E_b = (V_b - S K^_b) T_b + E_a X_ab with the stored cross factor
  X_ab = -(Alpha^_a'K^_b) T_b; S <- S + E_a Alpha^_a' + E_b Alpha^_b' (Eq. (10));
  readout o = (S Phi + E P) / den with P = (Alpha^'Phi) o Up, plus
  E_a Alpha^_a'Phi_b for chunk b (Eq. (11)).

Written out here with plain matrices, the chunk formulas must reproduce the
oracle to rounding at ragged lengths, from the default and from a given
initial state; a plausible slip in any of them must break the agreement.
"""
import numpy as np
import pytest

import oracle

LAMBDA0, EPS, C = 0.1, 1e-4, 16


def _phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _head(T, d, seed):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((T, d)) for _ in range(4))


def _ldl(M):
    """M = L D L' (L unit lower triangular), by columns."""
    n = M.shape[0]
    L, dg = np.eye(n), np.zeros(n)
    for j in range(n):
        dg[j] = M[j, j] - np.sum(L[j, :j] ** 2 * dg[:j])
        for i in range(j + 1, n):
            L[i, j] = (M[i, j] - np.sum(L[i, :j] * L[j, :j] * dg[:j])) / dg[j]
    return L, dg


def penalty_chain(kh, uh, A, slip=None):
    """alpha^ [T, d] and the final A by the chunk formulas, from A."""
    T, d = kh.shape
    al = np.zeros((T, d))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        n = sl.stop - sl.start
        U, K = uh[sl].T, kh[sl].T
        Z0, Y0 = A @ U, A @ K
        L, dg = _ldl(np.eye(n) + U.T @ Z0)
        Li = np.linalg.inv(L)
        up = np.triu(np.ones((n, n)), 1 if slip == "w_mask" else 0)   # [c, t] = 1 for c <= t
        W = Y0 - Z0 @ Li.T @ ((np.diag(1.0 / dg) @ Li @ (Z0.T @ K)) * up)
        M = -Li.T @ np.diag(1.0 / dg) @ Li                           # -(I + G)^-1
        A = A + (Z0 @ M @ Z0.T if slip != "down_sign" else -Z0 @ M @ Z0.T)
        al[sl] = (W / np.linalg.norm(W, axis=0)).T
    return al, A


def memory_chain(al, kh, v, pq, iden, S, slip=None):
    """o [T, d] and the final S by the pair steps, from S."""
    T, d = kh.shape
    o = np.zeros((T, d))
    chunks = [slice(c0, min(T, c0 + C)) for c0 in range(0, T, C)]
    for i in range(0, len(chunks), 2):
        a = chunks[i]
        b = chunks[i + 1] if i + 1 < len(chunks) else None
        Aa, Ka, Va, Pa = al[a].T, kh[a].T, v[a].T, pq[a].T
        na = a.stop - a.start
        sup_a, up_a = np.triu(np.ones((na, na)), 1), np.triu(np.ones((na, na)))
        Ta = np.linalg.inv(np.eye(na) + (Aa.T @ Ka) * sup_a)
        Ea = (Va - S @ Ka) @ Ta
        o[a] = ((S @ Pa + Ea @ ((Aa.T @ Pa) * up_a)) * iden[a]).T
        Sn = S + Ea @ Aa.T
        if b is not None:
            Ab, Kb, Vb, Pb = al[b].T, kh[b].T, v[b].T, pq[b].T
            nb = b.stop - b.start
            sup_b, up_b = np.triu(np.ones((nb, nb)), 1), np.triu(np.ones((nb, nb)))
            Tb = np.linalg.inv(np.eye(nb) + (Ab.T @ Kb) * sup_b)
            Xab = -(Aa.T @ Kb) @ (Tb if slip != "cross_unsolved" else np.eye(nb))
            Eb = (Vb - S @ Kb) @ Tb + Ea @ Xab
            cross = 0.0 if slip == "no_readout_cross" else Ea @ (Aa.T @ Pb)
            o[b] = ((S @ Pb + cross + Eb @ ((Ab.T @ Pb) * up_b)) * iden[b]).T
            Sn = Sn + Eb @ Ab.T
        S = Sn
    return o, S


def chunked_forward(q, k, v, u, S0=None, A0=None, zkey0=None, seg=None, slip=None):
    """One head by the chunk formulas; ``seg`` (a multiple of 2 C) starts a
    second penalty chain there from the summed Grams, as a later segment does."""
    T, d = q.shape
    kh = k / np.linalg.norm(k, axis=1)[:, None]
    uh = u / np.linalg.norm(u, axis=1)[:, None]
    A0 = np.eye(d) / LAMBDA0 if A0 is None else A0
    S0 = np.zeros((d, d)) if S0 is None else S0
    zk = np.cumsum(_phi(k), axis=0) + (0.0 if zkey0 is None else zkey0)
    pq = _phi(q)
    iden = 1.0 / np.maximum(np.sum(pq * zk, axis=1), EPS)
    if seg is None:
        al, A = penalty_chain(kh, uh, A0, slip)
    else:
        al0, _ = penalty_chain(kh[:seg], uh[:seg], A0, slip)
        Aseg = np.linalg.inv(np.linalg.inv(A0) + uh[:seg].T @ uh[:seg])
        al1, A = penalty_chain(kh[seg:], uh[seg:], Aseg, slip)
        al = np.concatenate([al0, al1])
    o, S = memory_chain(al, kh, v, pq, iden, S0, slip)
    return dict(o=o, S=S, A=A, zkey=zk[-1])


def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


@pytest.mark.parametrize("T,d,seg", [(100, 12, None), (100, 12, 64), (48, 8, None), (7, 5, None)])
def test_chunk_formulas_match_the_token_chain(T, d, seg):
    q, k, v, u = _head(T, d, seed=T + d)
    ref = oracle.forward_head(q, k, v, u, LAMBDA0, EPS)
    got = chunked_forward(q, k, v, u, seg=seg)
    for name in ("o", "S", "A", "zkey"):
        assert _rel(got[name], ref[name]) < 1e-10, name
    # and token by token for the readout, whose scale falls with t (Eq. (11))
    tok = np.linalg.norm(got["o"] - ref["o"], axis=1) / np.linalg.norm(ref["o"], axis=1)
    assert tok.max() < 1e-10


def test_chunk_formulas_from_a_given_state():
    T, d = 75, 10
    q, k, v, u = _head(T, d, seed=5)
    rng = np.random.default_rng(6)
    S0 = rng.standard_normal((d, d))
    B = rng.standard_normal((d, d))
    A0 = np.linalg.inv(np.eye(d) * 0.5 + B @ B.T / d)   # symmetric positive definite
    zkey0 = np.abs(rng.standard_normal(d)) * 3.0
    ref = oracle.forward_head(q, k, v, u, LAMBDA0, EPS, S0=S0, A0=A0, zkey0=zkey0)
    got = chunked_forward(q, k, v, u, S0=S0, A0=A0, zkey0=zkey0, seg=32)
    for name in ("o", "S", "A", "zkey"):
        assert _rel(got[name], ref[name]) < 1e-9, name


@pytest.mark.parametrize("slip", ["w_mask", "down_sign", "cross_unsolved", "no_readout_cross"])
def test_a_slip_in_the_chunk_formulas_is_seen(slip):
    q, k, v, u = _head(100, 12, seed=1)
    ref = oracle.forward_head(q, k, v, u, LAMBDA0, EPS)
    got = chunked_forward(q, k, v, u, slip=slip)
    worst = max(_rel(got[n], ref[n]) for n in ("o", "S", "A"))
    assert worst > 1e-4
