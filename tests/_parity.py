"""Error metrics of the GPU parity tests.

Two gates, both at 2e-3, for every output compared with the oracle:

- global: max|x_gpu - x_ref| / max|x_ref| over the whole array;
- per token, for arrays with one row per token (o and the gradients dq, dk,
  dv, du): max over rows t of |x_gpu,t - x_ref,t| / |x_ref,t| (Euclidean norms
  over the row), skipping rows whose reference norm is exactly 0.

The per-token gate exists because the readout denominator of Eq. (11) of
"Variational Linear Attention" (section 3.3) grows with t: late outputs are
small next to the largest one, and the global gate alone would pass large
errors on them.  Where the oracle gives a per-token conditioning scale (the
baselines: |S_t|_F |phi(q_t)| / den_t, the size o_t has when nothing cancels),
a row whose reference norm is below 1% of that scale (a near-cancelling dot
product, where an fp32 result has no meaningful relative accuracy) is measured
against 1% of the scale instead.
"""
import numpy as np

GATE = 2e-3


def rel(g, r):
    """max|g - r| / max|r| over the whole array."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)) if r.size else 0.0


def rel_rows(g, r, scale=None):
    """Worst row-wise relative error |g_t - r_t| / |r_t| over the rows (last axis)
    whose reference norm is not 0, and the row's index (None if no such row).
    With ``scale`` (one value per row), |r_t| is floored at 1% of it."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0, None
    nr = np.sqrt((r * r).sum(axis=-1))
    if scale is not None:
        nr = np.maximum(nr, 1e-2 * np.asarray(scale, dtype=np.float64).reshape(nr.shape))
    nd = np.sqrt(((g - r) ** 2).sum(axis=-1))
    live = nr > 0.0
    if not live.any():
        return 0.0, None
    e = np.where(live, nd / np.where(live, nr, 1.0), 0.0)
    i = int(np.argmax(e))
    return float(e.flat[i]), np.unravel_index(i, e.shape)


# outputs with one row per token
TOKEN_ROWS = ("o", "dq", "dk", "dv", "du")


def is_token_rows(name):
    base = name.split("[")[0].split("_")[0]
    return base in TOKEN_ROWS


def check(name, got, ref, gate=GATE, scale=None):
    """Assert both gates (the per-token one for token-row outputs) and print
    the errors."""
    e = rel(got, ref)
    msg = f"  {name}: rel err {e:.3e}"
    et = 0.0
    if is_token_rows(name):
        et, at = rel_rows(got, ref, scale)
        msg += f", worst token {et:.3e} at {tuple(int(i) for i in at) if at is not None else '-'}"
    print(msg, flush=True)
    assert e <= gate, f"{name}: {e:.3e} > {gate}"
    assert et <= gate, f"{name}: per-token {et:.3e} > {gate}"
    return max(e, et)
