"""GPU parity of the baselines (vla_baseline_forward through the C ABI): the
cumulative-sum linear attention of the "Linear Attention" wiki article and
DeltaNet as the scalar-gate special case of the VLA layer, against their fp64
oracles on the same seeded inputs.  Gates as for the forward (tests/_parity.py):
global and per-token for o (floored at 1% of the oracle's per-token scale
|S_t|_F |phi(q_t)| / den_t), global for the final S and zkey."""
import dataclasses

import numpy as np
import pytest

import gen
import oracle
from _parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _vla():
    import long_context_sequence_amd as vla
    return vla


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _to_dev(x, cfg, dev):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t.view(torch.bfloat16) if cfg.dtype == "bf16" else t


def _f64(x, cfg):
    return (gen.bf16_bits_to_f32(x) if cfg.dtype == "bf16" else x).astype(np.float64)


def _run(kind, cfg, x, dev, beta=1.0, **kw):
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkv"}
    out = _vla().vla_baseline(kind, t["q"], t["k"], t["v"], beta, cfg.eps, return_state=True, **kw)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in out]


@pytest.mark.parametrize("kind", ["linear", "delta"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_baseline_sweep_every_head(kind, d, dtype, T):
    dev = _dev()
    base = gen.config(3 if dtype == "bf16" else 2)
    cfg = dataclasses.replace(base, d=d).with_sizes(B=2, H=3, T=T)
    print(f"{kind} d={d} {dtype} T={T}", flush=True)
    x = gen.make_inputs(cfg)
    o, S, zk = _run(kind, cfg, x, dev)
    ref = oracle.baseline(kind, *(_f64(x[n], cfg) for n in "qkv"), 1.0, cfg.eps)
    check("o", o, ref["o"], scale=ref["scale"])
    check("S", S, ref["S"])
    check("zkey", zk, ref["zkey"])


@pytest.mark.parametrize("beta", [0.5, 0.9])
def test_deltanet_gate_and_ragged_groups(beta):
    """A gate below 1, and lengths that end inside a chunk pair and inside a
    group of chunks (so a group's last chunk stands alone)."""
    dev = _dev()
    for T in (16 * 16 + 5, 16 * 33 + 9):
        cfg = gen.config(3).with_sizes(B=1, H=2, T=T)
        x = gen.make_inputs(cfg)
        o, S, zk = _run("delta", cfg, x, dev, beta)
        ref = oracle.baseline("delta", *(_f64(x[n], cfg) for n in "qkv"), beta, cfg.eps)
        check("o", o, ref["o"], scale=ref["scale"])
        check("S", S, ref["S"])
        check("zkey", zk, ref["zkey"])


@pytest.mark.parametrize("kind", ["linear", "delta"])
def test_baseline_given_state_and_continuation(kind):
    """A given initial state, and a sequence run in two calls from the first
    call's final state equals one call."""
    dev = _dev()
    vla = _vla()
    cfg = gen.config(2).with_sizes(B=1, H=2, T=700)
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    o1, S1, z1 = vla.vla_baseline(kind, *(t[n][:, :, :300].contiguous() for n in "qkv"),
                                  return_state=True)
    o2, S2, z2 = vla.vla_baseline(kind, *(t[n][:, :, 300:].contiguous() for n in "qkv"),
                                  S0=S1, zkey0=z1, return_state=True)
    torch.cuda.synchronize()
    ref = oracle.baseline(kind, *(x[n].astype(np.float64) for n in "qkv"))
    check("o", np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], axis=2), ref["o"],
          scale=ref["scale"])
    check("S", S2.cpu().numpy(), ref["S"])
    check("zkey", z2.cpu().numpy(), ref["zkey"])


def test_deltanet_equals_vla_forward_with_u_zero():
    """beta = 1 DeltaNet is the VLA layer with u = 0 (A stays I / lambda0, alpha^ =
    k^): the two GPU paths agree to fp32 rounding."""
    dev = _dev()
    vla = _vla()
    cfg = gen.config(3).with_sizes(B=2, H=4, T=1000)
    x = gen.make_inputs(cfg)
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkv"}
    u = torch.zeros_like(t["q"])
    o_v, S_v, _, z_v = vla.vla_forward(t["q"], t["k"], t["v"], u, 0.1, cfg.eps, return_state=True)
    o_d, S_d, z_d = vla.vla_baseline("delta", t["q"], t["k"], t["v"], 1.0, cfg.eps,
                                     return_state=True)
    torch.cuda.synchronize()
    check("o", o_d.cpu().numpy(), o_v.cpu().numpy().astype(np.float64))
    check("S", S_d.cpu().numpy(), S_v.cpu().numpy().astype(np.float64))
    check("zkey", z_d.cpu().numpy(), z_v.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("kind", ["linear", "delta"])
def test_baseline_bench_workload_sampled_heads(kind):
    """B=8, H=16, d=64, T=4096 bf16: every head on the GPU, sampled heads against
    the oracle."""
    dev = _dev()
    cfg = gen.config(3)
    x = gen.make_inputs(cfg)
    o, S, zk = _run(kind, cfg, x, dev)
    assert np.isfinite(o).all()
    for (b, h) in [(0, 0), (5, 9)]:
        fn = oracle.linear_attention_head if kind == "linear" else oracle.deltanet_head
        args = [_f64(x[n][b, h], cfg) for n in "qkv"]
        r = fn(*args) if kind == "linear" else fn(*args, 1.0, cfg.eps)
        print(f" {kind} head ({b},{h})", flush=True)
        check("o", o[b, h], r["o"], scale=r["scale"])
        check("S", S[b, h], r["S"])
        check("zkey", zk[b, h], r["zkey"])


def test_state_norm_growth_contrast():
    """Section 4.1's contrast on the GPU paths: over the recall-shaped inputs
    (pairs drawn from a pool and written again and again), the cumulative
    state's |S|_F grows about linearly with T, while the VLA state stays near
    the size of the stored pairs."""
    dev = _dev()
    vla = _vla()
    cfg = gen.config(4).with_sizes(B=1, H=2, T=4096)
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev) for n in "qkvu"}
    norms = {}
    for T in (1024, 2048):
        sl = {n: t[n][:, :, :T].contiguous() for n in "qkvu"}
        _, S_la, _ = vla.vla_baseline("linear", sl["q"], sl["k"], sl["v"], return_state=True)
        _, S_v, _, _ = vla.vla_forward(sl["q"], sl["k"], sl["v"], sl["u"], return_state=True)
        torch.cuda.synchronize()
        norms[T] = (float(S_la.norm(dim=(-2, -1)).max()), float(S_v.norm(dim=(-2, -1)).max()))
    print(" |S|_F linear / vla:", norms, flush=True)
    assert norms[2048][0] > 1.8 * norms[1024][0]
    assert norms[2048][0] > 20 * norms[2048][1]
