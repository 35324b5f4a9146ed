"""The library's launches captured in a HIP graph (the way a serving or
training loop replays them): vla_forward with a caller workspace and
vla_backward (whose sweep resets its own synchronisation words with a kernel,
not a memset).  Each graph is replayed several times, with eager work and
synchronisations between the replays, and every replay must give the eager
call's bits."""
import dataclasses

import numpy as np
import pytest

import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _vla():
    import long_context_sequence_amd as vla
    return vla


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _inputs(cfg, dev):
    x = gen.make_inputs(cfg)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev) for n in "qkvu"}
    if cfg.dtype == "bf16":
        t = {n: a.view(torch.bfloat16) for n, a in t.items()}
    return t


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fn()
    torch.cuda.synchronize()
    return graph


def _replays(graph, outs, want, reps=3):
    for rep in range(reps):
        for a in outs:
            a.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=outs[0].device).sum()   # eager work between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (a, b) in enumerate(zip(outs, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (96, "f32"), (128, "bf16")])
def test_forward_graph_replay(d, dtype):
    dev = _dev()
    vla = _vla()
    cfg = dataclasses.replace(gen.config(3 if dtype == "bf16" else 2), d=d).with_sizes(B=2, H=4, T=333)
    B, H, T = cfg.B, cfg.H, cfg.T
    t = _inputs(cfg, dev)
    ws = torch.empty(vla.workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, H, T, d), device=dev), torch.empty((B, H, d, d), device=dev),
            torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d), device=dev)]

    def run():
        vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=outs[0],
                        S_out=outs[1], A_out=outs[2], zkey_out=outs[3], workspace=ws)

    run()
    torch.cuda.synchronize()
    want = [a.clone() for a in outs]
    _replays(_capture(run), outs, want)


@pytest.mark.parametrize("d", [64, 96])
def test_backward_graph_replay(d):
    dev = _dev()
    vla = _vla()
    cfg = dataclasses.replace(gen.config(3), d=d).with_sizes(B=2, H=4, T=200)
    B, H, T = cfg.B, cfg.H, cfg.T
    t = _inputs(cfg, dev)
    dO = torch.randn((B, H, T, d), generator=torch.Generator(device=dev).manual_seed(7), device=dev)
    ws = torch.empty(vla.backward_workspace_size(B, H, T, d), dtype=torch.uint8, device=dev)
    res = {}

    def run():
        res["g"] = vla.vla_backward(t["q"], t["k"], t["v"], t["u"], dO, cfg.lambda0, cfg.eps,
                                    workspace=ws)

    run()
    torch.cuda.synchronize()
    want = [a.clone() for a in res["g"]]
    graph = _capture(run)
    outs = list(res["g"])   # the captured call's outputs (allocated from the graph's pool)
    _replays(graph, outs, want)
