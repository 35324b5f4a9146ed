"""fp64 CPU oracle of the VLA per-head recurrence (forward and its gradients) -- TEST
INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and the
two share no code; the only common module is ``gen`` (seeded input draws).

The arithmetic lives in ``vla_oracle.c`` (plain C, fp64, one token at a time,
following "Variational Linear Attention" (arXiv 2605.11196) section 3.3,
Eqs. (9)-(11)).  This wrapper only marshals arrays and runs independent heads
on a thread pool (the C call releases the GIL).

Pins (tests/test_oracle_pins.py) tie each part to something other than the
oracle itself: brute-force inverses of the penalty matrix, the first token
worked by hand, the d = 1 closed form, the epsilon branch, the delta-rule and
cumulative-sum special cases, the state-update invariants, continuation and
head independence.  The gradients (``backward_head``) are pinned to central
finite differences of the forward, entry by entry on tiny heads (with the
denominator floor active and with zero keys and penalty vectors) and along
random directions on larger ones, and to the first token's gradient worked by
hand; ``backward_head_checkpointed`` (the same reverse mode split into
segments) to ``backward_head``.  The baselines: ``linear_attention_head`` to
the closed-form sum and the causal quadratic readout of the same article;
``deltanet_head`` to the VLA oracle with u = 0 (beta = 1), to exact recovery
with orthonormal keys and to the delta-rule residual invariant.  No function
here is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vla_oracle.c")
# VLA_ORACLE_LIB names another build of vla_oracle.c (the sanitizer test's)
_LIB = os.environ.get("VLA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile vla_oracle.c with the host C compiler (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if "VLA_ORACLE_LIB" not in os.environ and (
                not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.vla_oracle_forward
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double] + [_dp] * 18
        f = lib.vla_oracle_backward
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double] + [_dp] * 18
        f = lib.vla_oracle_linear_attention
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int] + [_dp] * 9
        f = lib.vla_oracle_deltanet
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double] + [_dp] * 9
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != shape:
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a


def forward_head(q, k, v, u, lambda0=0.1, eps=1e-4, S0=None, A0=None, zkey0=None,
                 trace=False):
    """Run one head: q, k, v, u are [T, d].  Returns a dict with ``o`` [T, d],
    final ``S``, ``A`` [d, d] and ``zkey`` [d]; with ``trace`` also per-token
    ``delta`` [T], ``alpha``, ``e``, ``z`` [T, d], ``den`` [T], ``A_t``, ``S_t``
    [T, d, d]."""
    q = _f64(q)
    T, d = q.shape
    k, v, u = _f64(k, (T, d)), _f64(v, (T, d)), _f64(u, (T, d))
    S0, A0, zkey0 = _f64(S0, (d, d)), _f64(A0, (d, d)), _f64(zkey0, (d,))
    o = np.zeros((T, d))
    S = np.zeros((d, d))
    A = np.zeros((d, d))
    zk = np.zeros(d)
    tr = {}
    if trace:
        tr = dict(delta=np.zeros(T), alpha=np.zeros((T, d)), e=np.zeros((T, d)),
                  z=np.zeros((T, d)), den=np.zeros(T), A_t=np.zeros((T, d, d)),
                  S_t=np.zeros((T, d, d)))
    rc = _load().vla_oracle_forward(
        T, d, float(lambda0), float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(u),
        _ptr(S0), _ptr(A0), _ptr(zkey0), _ptr(o), _ptr(S), _ptr(A), _ptr(zk),
        _ptr(tr.get("delta")), _ptr(tr.get("alpha")), _ptr(tr.get("e")), _ptr(tr.get("z")),
        _ptr(tr.get("den")), _ptr(tr.get("A_t")), _ptr(tr.get("S_t")))
    if rc != 0:
        raise ValueError(f"vla_oracle_forward failed with code {rc}")
    out = dict(o=o, S=S, A=A, zkey=zk)
    out.update(tr)
    return out


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, n)


def forward(q, k, v, u, lambda0=0.1, eps=1e-4, S0=None, A0=None, zkey0=None,
            workers=None):
    """All heads of [B, H, T, d] inputs (independent heads on a thread pool).

    S0, A0 ([B, H, d, d]) and zkey0 ([B, H, d]) are optional initial states.
    Returns ``o`` [B, H, T, d] and final ``S``, ``A``, ``zkey``.
    """
    q = np.asarray(q)
    B, H, T, d = q.shape
    o = np.zeros((B, H, T, d))
    S = np.zeros((B, H, d, d))
    A = np.zeros((B, H, d, d))
    zk = np.zeros((B, H, d))

    def one(bh):
        b, h = divmod(bh, H)
        r = forward_head(q[b, h], k[b, h], v[b, h], u[b, h], lambda0, eps,
                         None if S0 is None else S0[b, h],
                         None if A0 is None else A0[b, h],
                         None if zkey0 is None else zkey0[b, h])
        o[b, h], S[b, h], A[b, h], zk[b, h] = r["o"], r["S"], r["A"], r["zkey"]

    n = min(workers or default_workers(), B * H)
    if n <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, range(B * H)))
    return dict(o=o, S=S, A=A, zkey=zk)


def backward_head(q, k, v, u, dO, lambda0=0.1, eps=1e-4, S0=None, A0=None, zkey0=None,
                  dS_T=None, dA_T=None, dzkey_T=None):
    """Gradients of one head (q, k, v, u, dO are [T, d]; dS_T, dA_T [d, d] and
    dzkey_T [d] are the adjoints of the final state, None for 0).  Returns a
    dict with ``dq, dk, dv, du`` [T, d], ``dS0`` [d, d], ``dA0`` [d, d] (the
    gradient with respect to A_0 as a symmetric matrix) and ``dzkey0`` [d].
    Memory: 2 T d^2 doubles of per-token states."""
    q = _f64(q)
    T, d = q.shape
    k, v, u, dO = _f64(k, (T, d)), _f64(v, (T, d)), _f64(u, (T, d)), _f64(dO, (T, d))
    S0, A0, zkey0 = _f64(S0, (d, d)), _f64(A0, (d, d)), _f64(zkey0, (d,))
    dS_T, dA_T, dzkey_T = _f64(dS_T, (d, d)), _f64(dA_T, (d, d)), _f64(dzkey_T, (d,))
    out = dict(dq=np.zeros((T, d)), dk=np.zeros((T, d)), dv=np.zeros((T, d)),
               du=np.zeros((T, d)), dS0=np.zeros((d, d)), dA0=np.zeros((d, d)),
               dzkey0=np.zeros(d))
    rc = _load().vla_oracle_backward(
        T, d, float(lambda0), float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(u),
        _ptr(S0), _ptr(A0), _ptr(zkey0), _ptr(dO), _ptr(dS_T), _ptr(dA_T), _ptr(dzkey_T),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["du"]),
        _ptr(out["dS0"]), _ptr(out["dA0"]), _ptr(out["dzkey0"]))
    if rc != 0:
        raise ValueError(f"vla_oracle_backward failed with code {rc}")
    return out


def backward_head_checkpointed(q, k, v, u, dO, lambda0=0.1, eps=1e-4, S0=None, A0=None,
                               zkey0=None, dS_T=None, dA_T=None, dzkey_T=None, seg=512):
    """``backward_head`` for long sequences: the same gradients with memory of
    order (T / seg + seg) d^2 doubles instead of 2 T d^2.

    The forward runs once segment by segment (``seg`` tokens each), keeping only
    the state (S, A, zkey) at each segment start; then the segments are taken in
    reverse order, each by ``backward_head`` from its start state, with the
    adjoints of its final state set to the initial-state gradients of the
    segment after it.  The recurrence is the same token by token, so this is
    the chain rule split at the segment boundaries.  (The gradient with respect
    to A enters every step only through its symmetric part, so handing on the
    symmetrised dA0 of a segment changes nothing.)"""
    q = _f64(q)
    T, d = q.shape
    if T <= seg:
        return backward_head(q, k, v, u, dO, lambda0, eps, S0, A0, zkey0, dS_T, dA_T, dzkey_T)
    k, v, u, dO = _f64(k, (T, d)), _f64(v, (T, d)), _f64(u, (T, d)), _f64(dO, (T, d))
    bounds = list(range(0, T, seg)) + [T]
    starts = []
    st = (S0, A0, zkey0)
    for a, b in zip(bounds[:-1], bounds[1:]):
        starts.append(st)
        r = forward_head(q[a:b], k[a:b], v[a:b], u[a:b], lambda0, eps, *st)
        st = (r["S"], r["A"], r["zkey"])
    out = dict(dq=np.zeros((T, d)), dk=np.zeros((T, d)), dv=np.zeros((T, d)),
               du=np.zeros((T, d)))
    adj = (dS_T, dA_T, dzkey_T)
    for i in reversed(range(len(starts))):
        a, b = bounds[i], bounds[i + 1]
        r = backward_head(q[a:b], k[a:b], v[a:b], u[a:b], dO[a:b], lambda0, eps, *starts[i], *adj)
        for n in ("dq", "dk", "dv", "du"):
            out[n][a:b] = r[n]
        adj = (r["dS0"], r["dA0"], r["dzkey0"])
    out["dS0"], out["dA0"], out["dzkey0"] = adj
    return out


def linear_attention_head(q, k, v, S0=None, zkey0=None):
    """Cumulative-sum linear attention ("Linear Attention" wiki article,
    recurrent form) on one head: q, k, v are [T, d].  Returns ``o`` [T, d], the
    final ``S`` [d, d] (value-major, S += v phi(k)') and ``zkey`` [d], and
    ``scale`` [T] = |S_t|_F |phi(q_t)| / den_t (the size of o_t without
    cancellation)."""
    q = _f64(q)
    T, d = q.shape
    k, v = _f64(k, (T, d)), _f64(v, (T, d))
    S0, zkey0 = _f64(S0, (d, d)), _f64(zkey0, (d,))
    o, S, zk, sc = np.zeros((T, d)), np.zeros((d, d)), np.zeros(d), np.zeros(T)
    rc = _load().vla_oracle_linear_attention(T, d, _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                                             _ptr(zkey0), _ptr(o), _ptr(S), _ptr(zk), _ptr(sc))
    if rc != 0:
        raise ValueError(f"vla_oracle_linear_attention failed with code {rc}")
    return dict(o=o, S=S, zkey=zk, scale=sc)


def deltanet_head(q, k, v, beta=1.0, eps=1e-4, S0=None, zkey0=None):
    """DeltaNet as the VLA layer with the scalar gate beta in place of alpha^ and
    no A (delta rule on the unit key; Eq. (11) readout), one head.  Returns ``o``
    [T, d], the final ``S`` [d, d] and ``zkey`` [d], and ``scale`` [T] as for
    ``linear_attention_head``."""
    q = _f64(q)
    T, d = q.shape
    k, v = _f64(k, (T, d)), _f64(v, (T, d))
    S0, zkey0 = _f64(S0, (d, d)), _f64(zkey0, (d,))
    o, S, zk, sc = np.zeros((T, d)), np.zeros((d, d)), np.zeros(d), np.zeros(T)
    rc = _load().vla_oracle_deltanet(T, d, float(beta), float(eps), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(S0), _ptr(zkey0), _ptr(o), _ptr(S), _ptr(zk), _ptr(sc))
    if rc != 0:
        raise ValueError(f"vla_oracle_deltanet failed with code {rc}")
    return dict(o=o, S=S, zkey=zk, scale=sc)


def baseline(kind, q, k, v, beta=1.0, eps=1e-4, S0=None, zkey0=None, workers=None):
    """All heads of [B, H, T, d] inputs for kind "linear" or "delta" (thread
    pool over heads).  Returns ``o``, ``S``, ``zkey``."""
    q = np.asarray(q)
    B, H, T, d = q.shape
    res = dict(o=np.zeros((B, H, T, d)), S=np.zeros((B, H, d, d)), zkey=np.zeros((B, H, d)),
               scale=np.zeros((B, H, T)))

    def one(bh):
        b, h = divmod(bh, H)
        s0 = None if S0 is None else S0[b, h]
        z0 = None if zkey0 is None else zkey0[b, h]
        if kind == "linear":
            r = linear_attention_head(q[b, h], k[b, h], v[b, h], s0, z0)
        else:
            r = deltanet_head(q[b, h], k[b, h], v[b, h], beta, eps, s0, z0)
        for key in res:
            res[key][b, h] = r[key]

    n = min(workers or default_workers(), B * H)
    with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        list(ex.map(one, range(B * H)))
    return res


def backward(q, k, v, u, dO, lambda0=0.1, eps=1e-4, S0=None, A0=None, zkey0=None,
             dS_T=None, dA_T=None, dzkey_T=None, workers=None):
    """All heads of [B, H, T, d] inputs and output adjoints (independent heads on
    a thread pool).  Returns ``dq, dk, dv, du`` [B, H, T, d], ``dS0``, ``dA0``
    [B, H, d, d] and ``dzkey0`` [B, H, d]."""
    q = np.asarray(q)
    B, H, T, d = q.shape
    res = dict(dq=np.zeros((B, H, T, d)), dk=np.zeros((B, H, T, d)),
               dv=np.zeros((B, H, T, d)), du=np.zeros((B, H, T, d)),
               dS0=np.zeros((B, H, d, d)), dA0=np.zeros((B, H, d, d)),
               dzkey0=np.zeros((B, H, d)))

    def pick(x, b, h):
        return None if x is None else x[b, h]

    def one(bh):
        b, h = divmod(bh, H)
        r = backward_head(q[b, h], k[b, h], v[b, h], u[b, h], dO[b, h], lambda0, eps,
                          pick(S0, b, h), pick(A0, b, h), pick(zkey0, b, h),
                          pick(dS_T, b, h), pick(dA_T, b, h), pick(dzkey_T, b, h))
        for key, val in r.items():
            res[key][b, h] = val

    n = min(workers or default_workers(), B * H)
    if n <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, range(B * H)))
    return res
