"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Gate (fp32 state): max|x_gpu - x_ref| / max|x_ref| <= 2e-3 for o and for the
final S, A and zkey, and for o also the per-token error
max_t |o_gpu,t - o_ref,t| / |o_ref,t| <= 2e-3 (tests/_parity.py).  Small cases
compare every head; the full-size workloads run every head on the GPU in the
benchmark's launch configuration and compare sampled heads (the oracle computes
heads independently).
"""
import numpy as np
import pytest

import gen
import oracle
from _parity import GATE, check

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


def _say(*a):
    print(*a, flush=True)


def _gpu_forward(cfg, x, dev, **kw):
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    out = _vla().vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps,
                             return_state=True, **kw)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in out]


def _check(name, got, ref, gate=GATE):
    check(name, got, ref, gate)


def _compare_heads(cfg, x, out, heads):
    o, S, A, zk = out
    for (b, h) in heads:
        r = oracle.forward_head(*(_f64(x[n][b, h], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
        _say(f" head ({b},{h})")
        _check("o", o[b, h], r["o"])
        _check("S", S[b, h], r["S"])
        _check("A", A[b, h], r["A"])
        _check("zkey", zk[b, h], r["zkey"])


@pytest.mark.parametrize("cid", [1, 2])
def test_small_workloads_every_head(cid):
    dev = _dev()
    cfg = gen.config(cid)
    _say(f"workload {cfg.name}")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), out):
        _check(name, g, ref[name])


@pytest.mark.parametrize("cid,heads", [
    (3, [(0, 0), (3, 7), (5, 11), (7, 15)]),
    (4, [(0, 0), (1, 17), (3, 31)]),
])
def test_full_size_sampled_heads(cid, heads):
    dev = _dev()
    cfg = gen.config(cid)
    _say(f"workload {cfg.name} (full size)")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    assert np.isfinite(out[0]).all()
    _compare_heads(cfg, x, out, heads)


@pytest.mark.slow
def test_long_context_full_size_with_decode():
    """B=2, H=32, d=128, T=65536 bf16, then 4096 single-token decode steps
    continuing from the final state; sampled heads checked over both parts."""
    from concurrent.futures import ThreadPoolExecutor
    dev = _dev()
    vla = _vla()
    cfg = gen.config(5)
    _say(f"workload {cfg.name} (full size)")
    x = gen.make_inputs(cfg)
    heads = [(0, 5), (1, 30)]

    def ref_head(bh):
        b, h = bh
        r1 = oracle.forward_head(*(_f64(x[n][b, h], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
        r2 = oracle.forward_head(*(_f64(x[n + "_dec"][b, h], cfg) for n in "qkvu"),
                                 cfg.lambda0, cfg.eps, S0=r1["S"], A0=r1["A"], zkey0=r1["zkey"])
        return r1, r2

    with ThreadPoolExecutor(max_workers=len(heads)) as ex:
        refs = ex.submit(lambda: list(map(ref_head, heads)))
        o, S, A, zk = _gpu_forward(cfg, x, dev)
        assert np.isfinite(o).all()
        _say(" decode 4096 steps")
        St, At, zt = (torch.from_numpy(a).to(dev) for a in (S, A, zk))
        dec = {n: _to_dev(x[n + "_dec"], cfg, dev) for n in "qkvu"}
        od = torch.empty((cfg.B, cfg.H, cfg.decode, cfg.d), dtype=torch.float32, device=dev)
        for t in range(cfg.decode):
            od[:, :, t] = vla.vla_step(*(dec[n][:, :, t].contiguous() for n in "qkvu"),
                                       St, At, zt, cfg.eps)
        torch.cuda.synchronize()
        od = od.cpu().numpy()
        refs = refs.result()
    for (b, h), (r1, r2) in zip(heads, refs):
        _say(f" head ({b},{h})")
        _check("o", o[b, h], r1["o"])
        _check("S", S[b, h], r1["S"])
        _check("A", A[b, h], r1["A"])
        _check("zkey", zk[b, h], r1["zkey"])
        _check("o_decode", od[b, h], r2["o"])
        _check("S_after_decode", St[b, h].cpu().numpy(), r2["S"])
        _check("A_after_decode", At[b, h].cpu().numpy(), r2["A"])
        _check("zkey_after_decode", zt[b, h].cpu().numpy(), r2["zkey"])


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_shape_sweep_every_head(d, dtype, T):
    dev = _dev()
    base = gen.config(3 if dtype == "bf16" else 2)
    import dataclasses
    cfg = dataclasses.replace(base, d=d).with_sizes(B=2, H=3, T=T)
    _say(f"sweep d={d} {dtype} T={T}")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), out):
        _check(name, g, ref[name])


@pytest.mark.parametrize("T", [2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 64, 65])
def test_tile_boundaries(T):
    """Sequence lengths around the 16-token chunks (a ragged last chunk, the
    memory chain one chunk behind the penalty chain, two-slot staging)."""
    dev = _dev()
    cfg = gen.config(3).with_sizes(B=1, H=2, T=T)
    _say(f"tile boundary T={T}")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), out):
        _check(name, g, ref[name])


def test_many_heads_grid():
    """More (b, h) heads than compute units: 512 workgroups."""
    dev = _dev()
    cfg = gen.config(2).with_sizes(B=4, H=128, T=40)
    _say("grid of 512 heads")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    heads = [(0, 0), (1, 77), (3, 127), (2, 5)]
    for (b, h) in heads:
        r = oracle.forward_head(*(x[n][b, h].astype(np.float64) for n in "qkvu"))
        _check(f"o[{b},{h}]", out[0][b, h], r["o"])
        _check(f"S[{b},{h}]", out[1][b, h], r["S"])


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
def test_empty_sequence_copies_state(d):
    """T = 0 writes the initial state to the outputs: the defaults of section 3.2
    (S0 = 0, A0 = I / lambda0, zkey0 = 0), a given state copied exactly, and a
    given state updated in place (outputs aliasing it) left as it is."""
    dev = _dev()
    vla = _vla()
    B, H = 2, 3
    _say(f"empty sequence d={d}")
    e = torch.empty((B, H, 0, d), device=dev)
    o, S, A, zk = vla.vla_forward(e, e, e, e, 0.25, 1e-4, return_state=True)
    torch.cuda.synchronize()
    assert o.shape == (B, H, 0, d)
    assert torch.equal(S.cpu(), torch.zeros(B, H, d, d))
    assert torch.equal(A.cpu(), (torch.eye(d) * 4.0).expand(B, H, d, d))
    assert torch.equal(zk.cpu(), torch.zeros(B, H, d))
    S0 = torch.randn(B, H, d, d, device=dev)
    A0 = torch.randn(B, H, d, d, device=dev)
    z0 = torch.rand(B, H, d, device=dev)
    o, S, A, zk = vla.vla_forward(e, e, e, e, 0.1, 1e-4, S0=S0, A0=A0, zkey0=z0, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(A, A0) and torch.equal(zk, z0)
    # only some outputs requested, one of them in place
    keepS = S0.clone()
    A2 = torch.full((B, H, d, d), float("nan"), device=dev)
    vla.vla_forward(e, e, e, e, 0.5, 1e-4, S0=S0, A0=None, zkey0=None, S_out=S0, A_out=A2)
    torch.cuda.synchronize()
    assert torch.equal(S0, keepS)
    assert torch.equal(A2.cpu(), (torch.eye(d) * 2.0).expand(B, H, d, d))


def test_continuation_from_state_and_in_place():
    dev = _dev()
    vla = _vla()
    cfg = gen.config(2).with_sizes(B=2, H=2, T=200)
    x = gen.make_inputs(cfg)
    T1 = 83
    t = {n: torch.from_numpy(x[n]).to(dev) for n in "qkvu"}
    first = {n: t[n][:, :, :T1].contiguous() for n in "qkvu"}
    second = {n: t[n][:, :, T1:].contiguous() for n in "qkvu"}
    o1, S, A, zk = vla.vla_forward(*(first[n] for n in "qkvu"), return_state=True)
    # second part updates the state in place (outputs alias the initial state)
    o2 = vla.vla_forward(*(second[n] for n in "qkvu"), S0=S, A0=A, zkey0=zk,
                         S_out=S, A_out=A, zkey_out=zk)[0]
    torch.cuda.synchronize()
    ref = oracle.forward(*(x[n].astype(np.float64) for n in "qkvu"))
    _check("o", np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], axis=2), ref["o"])
    _check("S", S.cpu().numpy(), ref["S"])
    _check("A", A.cpu().numpy(), ref["A"])
    _check("zkey", zk.cpu().numpy(), ref["zkey"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_matches_oracle(dtype):
    dev = _dev()
    vla = _vla()
    cfg = gen.config(5 if dtype == "bf16" else 2).with_sizes(B=2, H=2, T=64, decode=0)
    x = gen.make_inputs(cfg)
    B, H, d = cfg.B, cfg.H, cfg.d
    S = torch.zeros(B, H, d, d, device=dev)
    A = (torch.eye(d, device=dev) / cfg.lambda0).expand(B, H, d, d).contiguous()
    zk = torch.zeros(B, H, d, device=dev)
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    outs = []
    for i in range(cfg.T):
        outs.append(vla.vla_step(*(t[n][:, :, i].contiguous() for n in "qkvu"), S, A, zk, cfg.eps))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).cpu().numpy()
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    _check("o", o, ref["o"])
    _check("S", S.cpu().numpy(), ref["S"])
    _check("A", A.cpu().numpy(), ref["A"])
    _check("zkey", zk.cpu().numpy(), ref["zkey"])


@pytest.mark.parametrize("d", [64, 128])
def test_step_graph_replay(d):
    """Decode steps captured in a HIP graph (one node per token, the way a serving
    loop launches them) give, on every replay, exactly the eager steps' outputs
    and state; the state is reset by eager copies between the replays."""
    dev = _dev()
    vla = _vla()
    import dataclasses
    cfg = dataclasses.replace(gen.config(5), d=d).with_sizes(B=2, H=3, T=24, decode=0)
    x = gen.make_inputs(cfg)
    B, H, n = cfg.B, cfg.H, cfg.T
    t = {m: _to_dev(x[m], cfg, dev).permute(2, 0, 1, 3).contiguous() for m in "qkvu"}
    S0 = 0.1 * torch.randn(B, H, d, d, device=dev)
    A0 = (torch.eye(d, device=dev) / cfg.lambda0).expand(B, H, d, d).contiguous()
    z0 = torch.rand(B, H, d, device=dev) + 0.5
    S, A, zk = S0.clone(), A0.clone(), z0.clone()
    o_eager = torch.empty(n, B, H, d, device=dev)
    for i in range(n):
        vla.vla_step(*(t[m][i] for m in "qkvu"), S, A, zk, cfg.eps, o=o_eager[i])
    torch.cuda.synchronize()
    want = [a.clone() for a in (o_eager, S, A, zk)]
    S.copy_(S0), A.copy_(A0), zk.copy_(z0)
    o = torch.empty_like(o_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(n):
                vla.vla_step(*(t[m][i] for m in "qkvu"), S, A, zk, cfg.eps, o=o[i])
    torch.cuda.synchronize()
    for rep in range(3):
        S.copy_(S0), A.copy_(A0), zk.copy_(z0), o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "S", "A", "zkey"), (o, S, A, zk), want):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager steps"
    ref = oracle.forward(*(_f64(x[m], cfg) for m in "qkvu"), cfg.lambda0, cfg.eps,
                         S0=S0.double().cpu().numpy(), A0=A0.double().cpu().numpy(),
                         zkey0=z0.double().cpu().numpy())
    check("o", o.permute(1, 2, 0, 3).cpu().numpy(), ref["o"])
    check("S", S.cpu().numpy(), ref["S"])


@pytest.mark.parametrize("d", [16, 32, 64, 96, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_degenerate_tokens_every_d(d, dtype):
    """Decode steps for every head dimension (the decode kernel for d >= 64, the
    LDS kernel with T = 1 in place for d = 16, 32), after a forward, with zero
    keys, zero penalty directions and very negative queries among the steps."""
    dev = _dev()
    vla = _vla()
    import dataclasses
    base = gen.config(3 if dtype == "bf16" else 2)
    cfg = dataclasses.replace(base, d=d).with_sizes(B=1, H=3, T=70)
    _say(f"steps d={d} {dtype}")
    x = gen.make_inputs(cfg)
    neg = gen.bf16_bits(np.float32([-60.0]))[0] if dtype == "bf16" else np.float32(-60.0)
    x["k"][:, :, 40] = 0     # +0.0 in both storage types
    x["u"][:, :, 45] = 0
    x["u"][:, 1, 50:60] = 0
    x["q"][:, :, 47] = neg
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    T1 = 37
    _, S, A, zk = vla.vla_forward(*(t[n][:, :, :T1].contiguous() for n in "qkvu"), cfg.lambda0,
                                  cfg.eps, return_state=True)
    outs = [vla.vla_step(*(t[n][:, :, i].contiguous() for n in "qkvu"), S, A, zk, cfg.eps)
            for i in range(T1, cfg.T)]
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2).cpu().numpy()
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    _check("o", o, ref["o"][:, :, T1:])
    _check("S", S.cpu().numpy(), ref["S"])
    _check("A", A.cpu().numpy(), ref["A"])
    _check("zkey", zk.cpu().numpy(), ref["zkey"])


def test_degenerate_tokens():
    """Zero keys, zero penalty directions and very negative queries (the eps
    branch of the readout denominator)."""
    dev = _dev()
    cfg = gen.config(2).with_sizes(B=1, H=2, T=96)
    x = gen.make_inputs(cfg)
    x["k"][:, :, 5] = 0.0
    x["u"][:, :, 9] = 0.0
    x["u"][:, 1, 20:40] = 0.0
    x["q"][:, :, 0:3] = -60.0
    x["q"][:, :, 50] = -60.0
    out = _gpu_forward(cfg, x, dev)
    ref = oracle.forward(*(x[n].astype(np.float64) for n in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), out):
        _check(name, g, ref[name])


def test_run_to_run_bitwise_deterministic():
    dev = _dev()
    cfg = gen.config(3).with_sizes(B=2, H=4, T=512)
    x = gen.make_inputs(cfg)
    a = _gpu_forward(cfg, x, dev)
    b = _gpu_forward(cfg, x, dev)
    for ga, gb in zip(a, b):
        assert np.array_equal(ga, gb)


# ---------------------------------------------------------------------------
# The two-pass forward (d_h in {64, 96, 128}): the penalty chain restarts at
# segment boundaries from a directly formed inverse, so these cases vary the
# number and length of segments (set by B*H and T) and the initial state.


@pytest.mark.parametrize("d,dtype,B,H,T", [
    (64, "bf16", 1, 1, 2000),     # one head: many short segments
    (96, "f32", 1, 3, 1111),      # ragged last segment and chunk
    (128, "bf16", 1, 2, 1500),
    (128, "f32", 3, 1, 33),       # three chunks, one segment
    (64, "f32", 4, 128, 160),     # 512 heads: a single segment each
    (96, "bf16", 2, 2, 8192),     # 64 segments of two Gram parts, summed by the prefix pass
])
def test_segments_every_head(d, dtype, B, H, T):
    dev = _dev()
    import dataclasses
    base = gen.config(3 if dtype == "bf16" else 2)
    cfg = dataclasses.replace(base, d=d).with_sizes(B=B, H=H, T=T)
    _say(f"segments d={d} {dtype} B={B} H={H} T={T}")
    x = gen.make_inputs(cfg)
    out = _gpu_forward(cfg, x, dev)
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), out):
        _check(name, g, ref[name])


def test_continuation_given_state_many_segments():
    """A caller-given initial state with many segments (the inverse of A0 is
    formed too), written to separate outputs and then in place."""
    dev = _dev()
    vla = _vla()
    cfg = gen.config(3).with_sizes(B=1, H=2, T=1200)
    x = gen.make_inputs(cfg)
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    T1 = 700
    o1, S1, A1, z1 = vla.vla_forward(*(t[n][:, :, :T1].contiguous() for n in "qkvu"),
                                     return_state=True)
    rest = [t[n][:, :, T1:].contiguous() for n in "qkvu"]
    o2, S2, A2, z2 = vla.vla_forward(*rest, S0=S1, A0=A1, zkey0=z1, return_state=True)
    o3 = vla.vla_forward(*rest, S0=S1, A0=A1, zkey0=z1, S_out=S1, A_out=A1, zkey_out=z1)[0]
    torch.cuda.synchronize()
    ref = oracle.forward(*(_f64(x[n], cfg) for n in "qkvu"), cfg.lambda0, cfg.eps)
    _check("o", np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], axis=2), ref["o"])
    for name, g in (("S", S2), ("A", A2), ("zkey", z2)):
        _check(name, g.cpu().numpy(), ref[name])
    assert torch.equal(o2, o3)
    assert torch.equal(S1, S2) and torch.equal(A1, A2) and torch.equal(z1, z2)


def test_workspace_reuse_and_stream():
    """An explicit workspace (dirty from an earlier call of another shape) and a
    side stream give the same bits as a fresh allocation."""
    dev = _dev()
    vla = _vla()
    cfg = gen.config(3).with_sizes(B=2, H=3, T=777)
    x = gen.make_inputs(cfg)
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    ref = vla.vla_forward(*(t[n] for n in "qkvu"), return_state=True)
    ws = torch.full((vla.workspace_size(2, 3, 2000, 64),), 0xAB, dtype=torch.uint8, device=dev)
    other = gen.config(3).with_sizes(B=2, H=3, T=2000)
    xo = gen.make_inputs(other)
    vla.vla_forward(*(_to_dev(xo[n], other, dev) for n in "qkvu"), workspace=ws)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = vla.vla_forward(*(t[n] for n in "qkvu"), return_state=True, workspace=ws,
                              stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,dtype,B,H,T", [
    (64, "bf16", 2, 3, 777),      # odd chunk count: a lone last chunk
    (96, "f32", 1, 2, 500),
    (128, "bf16", 1, 1, 48),      # three chunks
    (64, "f32", 1, 1, 3000),      # one head: many segments
])
def test_workspace_of_nans(d, dtype, B, H, T):
    """A workspace whose every float is NaN gives the bits of a zeroed one: no
    field the forward leaves unwritten (the cross factors of odd chunks, a
    record's padding) is ever used."""
    dev = _dev()
    vla = _vla()
    import dataclasses
    base = gen.config(3 if dtype == "bf16" else 2)
    cfg = dataclasses.replace(base, d=d).with_sizes(B=B, H=H, T=T)
    _say(f"NaN workspace d={d} {dtype} B={B} H={H} T={T}")
    x = gen.make_inputs(cfg)
    t = {n: _to_dev(x[n], cfg, dev) for n in "qkvu"}
    n = vla.workspace_size(B, H, T, d)
    outs = []
    for fill in (0xFF, 0x00):
        ws = torch.full((n,), fill, dtype=torch.uint8, device=dev)
        outs.append(vla.vla_forward(*(t[k] for k in "qkvu"), cfg.lambda0, cfg.eps,
                                    return_state=True, workspace=ws))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    ref = oracle.forward(*(_f64(x[k], cfg) for k in "qkvu"), cfg.lambda0, cfg.eps)
    for name, g in zip(("o", "S", "A", "zkey"), outs[0]):
        _check(name, g.cpu().numpy(), ref[name])


def test_phases_equal_forward_and_pipeline_on_two_streams():
    """vla_forward_penalty then vla_forward_memory give vla_forward's bits; two
    batches pipelined over two streams (penalty pass of batch 2 while the memory
    pass of batch 1 runs) give the same bits as well."""
    dev = _dev()
    vla = _vla()
    cfgs = [gen.config(3).with_sizes(B=2, H=2, T=500), gen.config(2).with_sizes(B=1, H=3, T=333)]
    xs = [gen.make_inputs(c) for c in cfgs]
    ts = [{n: _to_dev(x[n], c, dev) for n in "qkvu"} for x, c in zip(xs, cfgs)]
    refs = [vla.vla_forward(*(t[n] for n in "qkvu"), return_state=True) for t in ts]
    torch.cuda.synchronize()
    ws = [torch.empty(vla.workspace_size(c.B, c.H, c.T, c.d), dtype=torch.uint8, device=dev)
          for c in cfgs]
    outs = []
    for t, c, w in zip(ts, cfgs, ws):
        A = torch.empty((c.B, c.H, c.d, c.d), device=dev)
        z = torch.empty((c.B, c.H, c.d), device=dev)
        S = torch.empty((c.B, c.H, c.d, c.d), device=dev)
        outs.append((A, z, S))
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    done_pen = []
    for i, (t, w, (A, z, S)) in enumerate(zip(ts, ws, outs)):
        with torch.cuda.stream(s1):
            vla.vla_forward_penalty(t["q"], t["k"], t["u"], workspace=w, A_out=A, zkey_out=z,
                                    stream=s1)
            ev = torch.cuda.Event()
            ev.record(s1)
            done_pen.append(ev)
    os_ = []
    for i, (t, w, (A, z, S)) in enumerate(zip(ts, ws, outs)):
        with torch.cuda.stream(s2):
            s2.wait_event(done_pen[i])
            os_.append(vla.vla_forward_memory(t["v"], workspace=w, S_out=S,
                                              stream=s2))
    s1.synchronize()
    s2.synchronize()
    torch.cuda.synchronize()
    for (o_ref, S_ref, A_ref, z_ref), o, (A, z, S) in zip(refs, os_, outs):
        assert torch.equal(o, o_ref)
        assert torch.equal(S, S_ref) and torch.equal(A, A_ref) and torch.equal(z, z_ref)
