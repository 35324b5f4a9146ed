"""Seeded synthetic inputs for the VLA forward recurrence (input construction only).

This module is shared by the fp64 oracle side and the HIP side so that both read
bit-identical input values.  It holds no step of the method itself: it draws
q, k, v, u the way each workload describes them and rounds them to the storage
type the device reads (fp32, or bf16 with round-to-nearest-even).

Every (batch, head) slice has its own generator,
``PCG64(SeedSequence([seed, b, h]))``, so any single head can be regenerated
on its own (the oracle samples heads of the large workloads that way) and the
full tensors are assembled head by head.

Workloads (shapes and distributions from the method's evaluation setting; the
multi-query associative-recall (MQAR) shaped one stands in for the paper's MQAR
task, whose data and trained models are not available):

=====  ===========================  =====  ================================
id     B, H, d_h, T                 input  values
=====  ===========================  =====  ================================
1      1, 1, 16, 256                f32    q,k,v,u ~ N(0,1); k, u unit rows
2      4, 8, 64, 1024               f32    q,k,v ~ N(0,1); u unit rows
3      8, 16, 64, 4096              bf16   q,k,v,u ~ N(0,1), raw
4      4, 32, 96, 16384             f32    MQAR-shaped key/value pairs, then
                                           re-queries with noise tokens
5      2, 32, 128, 65536 (+4096)    bf16   q,k,v ~ N(0,1) * log-uniform
                                           per-token scale in [0.1, 10];
                                           u unit rows; plus a 4096-token
                                           decode continuation
=====  ===========================  =====  ================================
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Config", "CONFIGS", "config", "head_inputs", "make_inputs",
    "bf16_bits", "bf16_round", "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.  ``kind`` selects the value recipe."""
    cid: int
    name: str
    B: int
    H: int
    d: int
    T: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v, u
    kind: str             # "unit_ku" | "unit_u" | "raw" | "mqar" | "scaled"
    decode: int = 0       # decode-continuation tokens drawn after the T tokens
    lambda0: float = 0.1
    eps: float = 1e-4

    @property
    def seed(self) -> int:
        return self.cid

    def with_sizes(self, B=None, H=None, T=None, decode=None) -> "Config":
        """Same recipe and seed at other sizes (reduced-size test cases)."""
        return dataclasses.replace(
            self,
            B=self.B if B is None else B,
            H=self.H if H is None else H,
            T=self.T if T is None else T,
            decode=self.decode if decode is None else decode,
        )


CONFIGS = {
    1: Config(1, "single_head_d16_t256_f32", 1, 1, 16, 256, "f32", "unit_ku"),
    2: Config(2, "b4h8_d64_t1024_f32", 4, 8, 64, 1024, "f32", "unit_u"),
    3: Config(3, "b8h16_d64_t4096_bf16", 8, 16, 64, 4096, "bf16", "raw"),
    4: Config(4, "mqar_b4h32_d96_t16384_f32", 4, 32, 96, 16384, "f32", "mqar"),
    5: Config(5, "b2h32_d128_t65536_bf16_decode4096", 2, 32, 128, 65536, "bf16",
              "scaled", decode=4096),
}


def config(cid: int) -> Config:
    return CONFIGS[cid]


# ----------------------------------------------------------------- bf16 storage
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite; no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ------------------------------------------------------------ per-head recipes
def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.where(n > 0, n, 1.0)


def _draw_plain(rng, T, d, kind):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    u = rng.standard_normal((T, d))
    if kind == "unit_ku":
        k = _unit_rows(k)
        u = _unit_rows(u)
    elif kind == "unit_u":
        u = _unit_rows(u)
    return q, k, v, u


def _draw_scaled(rng, T, d):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    u = _unit_rows(rng.standard_normal((T, d)))
    lo, hi = math.log(0.1), math.log(10.0)
    sq = np.exp(rng.uniform(lo, hi, size=(T, 1)))
    sk = np.exp(rng.uniform(lo, hi, size=(T, 1)))
    sv = np.exp(rng.uniform(lo, hi, size=(T, 1)))
    return q * sq, k * sk, v * sv, u


def _draw_mqar(rng, T, d, pool=512):
    """Key/value pairs from a per-head pool in the first half; the second half
    alternates query tokens (q equals a key written earlier, k and v small
    noise) and noise tokens (q, k, v all small noise, std 0.1)."""
    P = _unit_rows(rng.standard_normal((pool, d)))
    Vp = rng.standard_normal((pool, d))
    half = T // 2
    n2 = T - half
    idx = rng.integers(0, pool, size=half)
    q1 = rng.standard_normal((half, d))
    nq = (n2 + 1) // 2
    written = np.unique(idx) if half > 0 else np.arange(pool)
    j = rng.choice(written, size=nq)
    qn = 0.1 * rng.standard_normal((n2, d))
    kn = 0.1 * rng.standard_normal((n2, d))
    vn = 0.1 * rng.standard_normal((n2, d))
    q2 = qn.copy()
    q2[0::2] = P[j]
    q = np.concatenate([q1, q2], axis=0)
    k = np.concatenate([P[idx], kn], axis=0)
    v = np.concatenate([Vp[idx], vn], axis=0)
    u = _unit_rows(rng.standard_normal((T, d)))
    return q, k, v, u


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast a float64 draw to the exact values the device reads (as float32)."""
    x32 = x.astype(np.float32)
    return bf16_round(x32) if dtype == "bf16" else x32


def head_inputs(cfg: Config, b: int, h: int) -> dict:
    """Inputs of one (b, h) head as float32 arrays of shape [T, d] holding the
    exact stored values.  With ``cfg.decode`` > 0 the dict also holds
    ``q_dec, k_dec, v_dec, u_dec`` ([decode, d]) drawn after the T tokens from
    the same generator."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, b, h])))
    if cfg.kind in ("unit_ku", "unit_u", "raw"):
        arrs = _draw_plain(rng, cfg.T, cfg.d, cfg.kind)
    elif cfg.kind == "scaled":
        arrs = _draw_scaled(rng, cfg.T, cfg.d)
    elif cfg.kind == "mqar":
        arrs = _draw_mqar(rng, cfg.T, cfg.d)
    else:
        raise ValueError(f"unknown input recipe {cfg.kind!r}")
    out = {n: _store(a, cfg.dtype) for n, a in zip("qkvu", arrs)}
    if cfg.decode:
        if cfg.kind == "scaled":
            dec = _draw_scaled(rng, cfg.decode, cfg.d)
        else:
            dec = _draw_plain(rng, cfg.decode, cfg.d, cfg.kind)
        for n, a in zip("qkvu", dec):
            out[n + "_dec"] = _store(a, cfg.dtype)
    return out


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(cfg: Config, workers: int | None = None) -> dict:
    """Full [B, H, T, d] tensors in device storage format.

    Returns a dict with ``q, k, v, u`` as float32 arrays (f32 workloads) or
    uint16 bf16 bit patterns (bf16 workloads), and the ``*_dec`` decode
    tensors ([B, H, decode, d]) when the workload has them.
    """
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    names = ["q", "k", "v", "u"] + (["q_dec", "k_dec", "v_dec", "u_dec"] if cfg.decode else [])
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = {}
    for n in names:
        tt = cfg.decode if n.endswith("_dec") else T
        out[n] = np.empty((B, H, tt, d), dtype=st)

    def fill(bh):
        b, h = divmod(bh, H)
        hi = head_inputs(cfg, b, h)
        for n in names:
            a = hi[n]
            out[n][b, h] = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16) \
                if cfg.dtype == "bf16" else a

    with ThreadPoolExecutor(max_workers=workers or _workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return out
