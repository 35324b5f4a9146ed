"""GPU parity of the gradients: vla_backward (through the C ABI) against the
fp64 reverse-mode oracle (itself pinned to finite differences of the forward)
on the same seeded inputs and output adjoints.

Gate, as for the forward: max|g_gpu - g_ref| / max|g_ref| <= 2e-3 for every
gradient (dq, dk, dv, du and those of the initial state), and for the per-token
gradients dq, dk, dv, du also max_t |g_gpu,t - g_ref,t| / |g_ref,t| <= 2e-3
(tests/_parity.py).
"""
import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import gen
import oracle
from _parity import GATE, is_token_rows, rel, rel_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "du", "dS0", "dA0", "dzkey0")


def _vla():
    import long_context_sequence_amd as vla
    return vla


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _to_dev(x, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t.view(torch.bfloat16) if dtype == "bf16" else t


def _f64(x, dtype):
    return (gen.bf16_bits_to_f32(x) if dtype == "bf16" else x).astype(np.float64)


def _adjoints(B, H, T, d, seed, state=True):
    rng = np.random.default_rng(seed)
    adj = dict(dO=rng.standard_normal((B, H, T, d)).astype(np.float32))
    if state:
        adj["dS_T"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        adj["dA_T"] = rng.standard_normal((B, H, d, d)).astype(np.float32)
        adj["dzkey_T"] = rng.standard_normal((B, H, d)).astype(np.float32)
    return adj


def _gpu_backward(cfg, x, adj, dev, init=None):
    t = {n: _to_dev(x[n], cfg.dtype, dev) for n in "qkvu"}
    a = {n: torch.from_numpy(v).to(dev) for n, v in adj.items()}
    st = {} if init is None else {n: torch.from_numpy(v).to(dev) for n, v in init.items()}
    out = _vla().vla_backward(t["q"], t["k"], t["v"], t["u"], a["dO"], cfg.lambda0, cfg.eps,
                              dS_T=a.get("dS_T"), dA_T=a.get("dA_T"), dzkey_T=a.get("dzkey_T"),
                              **st)
    torch.cuda.synchronize()
    return dict(zip(NAMES, (o.cpu().numpy() for o in out)))


def _oracle_head(cfg, x, adj, b, h, init=None):
    def pick(dct, n):
        return None if dct is None or n not in dct else dct[n][b, h].astype(np.float64)
    return oracle.backward_head(*(_f64(x[n][b, h], cfg.dtype) for n in "qkvu"),
                                adj["dO"][b, h].astype(np.float64), cfg.lambda0, cfg.eps,
                                pick(init, "S0"), pick(init, "A0"), pick(init, "zkey0"),
                                pick(adj, "dS_T"), pick(adj, "dA_T"), pick(adj, "dzkey_T"))


def _compare(cfg, x, adj, got, heads, init=None, gate=GATE):
    def one(bh):
        return bh, _oracle_head(cfg, x, adj, *bh, init=init)
    with ThreadPoolExecutor(max_workers=min(8, len(heads))) as ex:
        refs = dict(ex.map(one, heads))
    worst, worst_tok = {}, {}
    for (b, h), r in refs.items():
        for n in NAMES:
            worst[n] = max(worst.get(n, 0.0), rel(got[n][b, h], r[n]))
            if is_token_rows(n):
                worst_tok[n] = max(worst_tok.get(n, 0.0), rel_rows(got[n][b, h], r[n])[0])
    _say("  " + "  ".join(f"{n} {e:.2e}" for n, e in worst.items()))
    _say("  per token: " + "  ".join(f"{n} {e:.2e}" for n, e in worst_tok.items()))
    for n, e in worst.items():
        assert e <= gate, f"{n}: {e:.3e} > {gate}"
    for n, e in worst_tok.items():
        assert e <= gate, f"{n}: per-token {e:.3e} > {gate}"


def _cfg(d, dtype, B, H, T):
    base = gen.config(3 if dtype == "bf16" else 2)
    return dataclasses.replace(base, d=d).with_sizes(B=B, H=H, T=T)


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_backward_sweep_every_head(d, dtype, T):
    dev = _dev()
    cfg = _cfg(d, dtype, 1, 2, T)
    _say(f"backward d={d} {dtype} T={T}")
    x = gen.make_inputs(cfg)
    adj = _adjoints(1, 2, T, d, seed=1000 + d + T)
    got = _gpu_backward(cfg, x, adj, dev)
    _compare(cfg, x, adj, got, [(0, 0), (0, 1)])


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("T", [16, 250])
def test_backward_whole_and_ragged_chunks(d, T):
    """One whole 16-token chunk, and an even chunk count with a ragged last
    chunk (the forward that keeps the per-token records steps over chunk pairs)."""
    dev = _dev()
    cfg = _cfg(d, "bf16", 1, 3, T)
    _say(f"backward chunks d={d} T={T}")
    x = gen.make_inputs(cfg)
    adj = _adjoints(1, 3, T, d, seed=2000 + d + T)
    got = _gpu_backward(cfg, x, adj, dev)
    _compare(cfg, x, adj, got, [(0, 0), (0, 1), (0, 2)])


@pytest.mark.parametrize("d,T", [(64, 4096), (128, 1024)])
def test_backward_single_head_many_segments(d, T):
    """One head over a long sequence: the forward that keeps the records splits
    the penalty chain into many short segments (two chunks each)."""
    dev = _dev()
    cfg = _cfg(d, "bf16", 1, 1, T)
    _say(f"backward single head d={d} T={T}")
    x = gen.make_inputs(cfg)
    adj = _adjoints(1, 1, T, d, seed=3000 + d)
    got = _gpu_backward(cfg, x, adj, dev)
    _compare(cfg, x, adj, got, [(0, 0)])


@pytest.mark.parametrize("d", [64, 128])
def test_backward_given_initial_state(d):
    """A general initial state (S0, an SPD A0, zkey0) and only dL/do."""
    dev = _dev()
    cfg = _cfg(d, "f32", 1, 2, 70)
    _say(f"backward from a given state d={d}")
    x = gen.make_inputs(cfg)
    rng = np.random.default_rng(77 + d)
    m = rng.standard_normal((1, 2, d, d))
    init = dict(S0=(0.3 * rng.standard_normal((1, 2, d, d))).astype(np.float32),
                A0=(m @ m.transpose(0, 1, 3, 2) / d + 0.5 * np.eye(d)).astype(np.float32),
                zkey0=rng.uniform(0.5, 2.0, (1, 2, d)).astype(np.float32))
    adj = _adjoints(1, 2, 70, d, seed=78 + d, state=False)
    got = _gpu_backward(cfg, x, adj, dev, init=init)
    _compare(cfg, x, adj, got, [(0, 0), (0, 1)], init=init)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_backward_degenerate_tokens(d):
    """Zero keys and penalty vectors, and tokens where the denominator floor
    decides (keys far below zero at the start, queries far below zero later)."""
    dev = _dev()
    cfg = _cfg(d, "f32", 1, 2, 40)
    _say(f"backward degenerate tokens d={d}")
    x = gen.make_inputs(cfg)
    x["k"][:, :, 0:2] = -20.0
    x["q"][:, :, 9] = -40.0
    x["k"][:, :, 5] = 0.0
    x["u"][:, :, 7] = 0.0
    x["u"][:, 1, 20:23] = 0.0
    adj = _adjoints(1, 2, 40, d, seed=90 + d)
    adj["dO"][:, :, 0:2] *= 1e-4
    got = _gpu_backward(cfg, x, adj, dev)
    _compare(cfg, x, adj, got, [(0, 0), (0, 1)])
    assert np.all(got["du"][:, :, 7] == 0.0)


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
def test_backward_empty_sequence(d):
    """T = 0: the initial state's gradients are the final state's adjoints
    (dA0 symmetrised), at every head size; a missing adjoint gives zeros."""
    dev = _dev()
    vla = _vla()
    B, H = 1, 3
    e = torch.empty((B, H, 0, d), device=dev)
    dS = torch.randn(B, H, d, d, device=dev)
    dA = torch.randn(B, H, d, d, device=dev)
    dz = torch.randn(B, H, d, device=dev)
    out = vla.vla_backward(e, e, e, e, e, 0.1, 1e-4, dS_T=dS, dA_T=dA, dzkey_T=dz)
    torch.cuda.synchronize()
    assert torch.equal(out[4], dS)
    ref = (0.5 * (dA.double() + dA.double().transpose(-1, -2))).float()
    assert torch.equal(out[5], ref)
    assert torch.equal(out[6], dz)
    out = vla.vla_backward(e, e, e, e, e, 0.1, 1e-4, dA_T=dA)
    torch.cuda.synchronize()
    assert torch.equal(out[4], torch.zeros_like(dS))
    assert torch.equal(out[5], ref)
    assert torch.equal(out[6], torch.zeros_like(dz))


def test_backward_deterministic():
    dev = _dev()
    cfg = _cfg(64, "bf16", 2, 2, 50)
    x = gen.make_inputs(cfg)
    adj = _adjoints(2, 2, 50, 64, seed=5)
    a = _gpu_backward(cfg, x, adj, dev)
    b = _gpu_backward(cfg, x, adj, dev)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("d", [64, 128])
def test_backward_more_workgroups_than_fit(d):
    """Far more heads than the device holds workgroups at once (2 per head in the
    reverse sweep): the penalty-chain workgroups that start early wait only on
    memory-chain workgroups already running, so every head completes; sampled
    heads, the first and last included, against the oracle."""
    dev = _dev()
    B, H, T = 4, 160 if d == 64 else 96, 40
    cfg = _cfg(d, "bf16", B, H, T)
    _say(f"backward d={d} B={B} H={H} T={T} ({2 * B * H} sweep workgroups)")
    x = gen.make_inputs(cfg)
    adj = _adjoints(B, H, T, d, seed=11)
    got = _gpu_backward(cfg, x, adj, dev)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare(cfg, x, adj, got, [(0, 0), (1, H // 2), (2, 7), (B - 1, H - 1)])


@pytest.mark.parametrize("d,dtype", [(96, "f32"), (96, "bf16"), (128, "f32"), (128, "bf16")])
def test_backward_repeat_bitwise(d, dtype):
    """Repeated calls give the same bits at the head sizes whose token streams
    take several copies per token (every copy of a token must have landed
    before the token is used); 128 heads, so both chains of every head run side
    by side."""
    dev = _dev()
    cfg = _cfg(d, dtype, 4, 32, 160)
    x = gen.make_inputs(cfg)
    adj = _adjoints(4, 32, 160, d, seed=17)
    first = _gpu_backward(cfg, x, adj, dev)
    for rep in range(3):
        again = _gpu_backward(cfg, x, adj, dev)
        for n in NAMES:
            assert np.array_equal(again[n], first[n]), f"call {rep + 1}: {n}"


def test_backward_workload_every_head():
    """B=4, H=8, d=64, T=1024 fp32 (the forward parity workload), every head."""
    dev = _dev()
    cfg = gen.config(2)
    _say(f"backward workload {cfg.name}")
    x = gen.make_inputs(cfg)
    adj = _adjoints(cfg.B, cfg.H, cfg.T, cfg.d, seed=2)
    got = _gpu_backward(cfg, x, adj, dev)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    _compare(cfg, x, adj, got, heads)


def test_backward_bench_workload_sampled_heads():
    """B=8, H=16, d=64, T=4096 bf16 (the benchmark's forward workload): every head
    on the GPU, sampled heads against the oracle."""
    dev = _dev()
    cfg = gen.config(3)
    _say(f"backward workload {cfg.name} (full size)")
    x = gen.make_inputs(cfg)
    adj = _adjoints(cfg.B, cfg.H, cfg.T, cfg.d, seed=3)
    got = _gpu_backward(cfg, x, adj, dev)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare(cfg, x, adj, got, [(0, 0), (7, 15)])


def test_autograd_wrapper_matches_backward():
    """vla_attention's autograd gradients are vla_backward's (a loss o . w)."""
    dev = _dev()
    vla = _vla()
    cfg = _cfg(64, "f32", 1, 2, 40)
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(x[n]).to(dev).requires_grad_(True) for n in "qkvu"}
    w = torch.from_numpy(np.random.default_rng(9).standard_normal((1, 2, 40, 64))
                         .astype(np.float32)).to(dev)
    o = vla.vla_attention(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps)
    (o * w).sum().backward()
    torch.cuda.synchronize()
    ref = vla.vla_backward(*(t[n].detach() for n in "qkvu"), w, cfg.lambda0, cfg.eps)
    torch.cuda.synchronize()
    for n, r in zip("qkvu", ref[:4]):
        assert torch.equal(t[n].grad, r), n


@pytest.mark.parametrize("cid,T,heads", [
    (4, 2048, [(0, 0), (3, 31)]),     # MQAR-shaped recall workload, d = 96, fp32
    (5, 2048, [(0, 0), (1, 31)]),     # long-context recipe, d = 128, bf16, scaled inputs
])
def test_backward_other_workloads_sampled_heads(cid, T, heads):
    """The recall and long-context workloads' input recipes and head counts at
    T = 2048 (the oracle keeps 2 T d^2 doubles per head): every head on the
    GPU, sampled heads against the oracle."""
    dev = _dev()
    cfg = gen.config(cid).with_sizes(T=T, decode=0)
    _say(f"backward workload {cfg.name} at T={T}")
    x = gen.make_inputs(cfg)
    adj = _adjoints(cfg.B, cfg.H, cfg.T, cfg.d, seed=10 + cid)
    got = _gpu_backward(cfg, x, adj, dev)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare(cfg, x, adj, got, heads)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid,heads", [
    (4, [(0, 0), (3, 31)]),     # MQAR-shaped recall workload: B=4, H=32, d=96, T=16384, fp32
    (5, [(0, 5), (1, 30)]),     # long-context workload: B=2, H=32, d=128, T=65536, bf16
])
def test_backward_full_size(cid, heads):
    """The recall and long-context workloads at full size: gradients of every
    head on the GPU, all finite.  The first sampled head is checked everywhere:
    dq, dk, dv, du of every token and the initial state's gradients, against the
    oracle's reverse mode over the whole sequence (checkpointed, so that it keeps
    a few segments of per-token states instead of 2 T d^2 doubles).  For the
    other heads the last 64 tokens' dq, dk, dv, du against the oracle's reverse
    mode over those tokens, started from its forward state after the first
    T - 64 tokens (with no adjoint on the final state, the last tokens'
    gradients depend on the earlier ones only through that state)."""
    from concurrent.futures import ThreadPoolExecutor
    dev = _dev()
    vla = _vla()
    cfg = gen.config(cid).with_sizes(decode=0)
    _say(f"backward workload {cfg.name} (full size)")
    x = gen.make_inputs(cfg)
    B, H, T, d, m = cfg.B, cfg.H, cfg.T, cfg.d, 64
    g = torch.Generator(device=dev).manual_seed(50 + cid)
    dO = torch.randn((B, H, T, d), generator=g, device=dev)
    dO_h = {bh: dO[bh[0], bh[1]].cpu().numpy().astype(np.float64) for bh in heads}

    def ref_whole(bh):
        b, h = bh
        qkvu = [_f64(x[n][b, h], cfg.dtype) for n in "qkvu"]
        return oracle.backward_head_checkpointed(*qkvu, dO_h[bh], cfg.lambda0, cfg.eps, seg=512)

    def ref_tail(bh):
        b, h = bh
        qkvu = [_f64(x[n][b, h], cfg.dtype) for n in "qkvu"]
        st = oracle.forward_head(*(a[:T - m] for a in qkvu), cfg.lambda0, cfg.eps)
        return oracle.backward_head(*(a[T - m:] for a in qkvu), dO_h[bh][T - m:], cfg.lambda0,
                                    cfg.eps, st["S"], st["A"], st["zkey"])

    with ThreadPoolExecutor(max_workers=len(heads)) as ex:
        futs = [ex.submit(ref_whole if i == 0 else ref_tail, bh) for i, bh in enumerate(heads)]
        t = {n: _to_dev(x[n], cfg.dtype, dev) for n in "qkvu"}
        out = vla.vla_backward(t["q"], t["k"], t["v"], t["u"], dO, cfg.lambda0, cfg.eps)
        torch.cuda.synchronize()
        for n, o in zip(NAMES, out):
            assert bool(torch.isfinite(o).all()), n
        got = {bh: [o[bh[0], bh[1]].cpu().numpy() for o in out] for bh in heads}
        refs = [f.result() for f in futs]
    for i, (bh, r) in enumerate(zip(heads, refs)):
        if i == 0:
            names, gv = NAMES, got[bh]
            _say(f"  head {bh}, every token and the initial state:")
        else:
            names, gv = NAMES[:4], [a[T - m:] for a in got[bh][:4]]
            _say(f"  head {bh}, last {m} tokens:")
        errs = {n: rel(a, r[n]) for n, a in zip(names, gv)}
        tok = {n: rel_rows(a, r[n]) for n, a in zip(names, gv) if is_token_rows(n)}
        _say("   " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
        _say("   per token: " + "  ".join(f"{n} {e:.2e} at {at}" for n, (e, at) in tok.items()))
        for n in errs:
            assert errs[n] <= GATE, f"{bh} {n}: {errs[n]:.3e} > {GATE}"
        for n, (e, _) in tok.items():
            assert e <= GATE, f"{bh} {n}: per-token {e:.3e} > {GATE}"
