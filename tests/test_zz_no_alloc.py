"""vla_forward_noalloc (the forward with the library's own fixed workspace, for
callers that cannot allocate) against vla_forward with a caller workspace:
bit-identical results on two calls in a row, the second with a smaller input,
through the C ABI."""
import numpy as np
import pytest

import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def test_noalloc_matches_forward_twice():
    import long_context_sequence_amd as vla
    dev = _dev()
    import dataclasses
    cases = [gen.config(2),                                                  # 32 heads, T = 1024, fp32
             dataclasses.replace(gen.config(3), d=96).with_sizes(B=2, H=3, T=300)]   # smaller, bf16
    for cfg in cases:
        B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
        print(f"noalloc B={B} H={H} T={T} d={d} {cfg.dtype}", flush=True)
        assert vla.workspace_size(B, H, T, d) <= vla.NOALLOC_SCRATCH_BYTES
        t = _inputs(cfg, dev)
        ref = vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps,
                              return_state=True)
        o = torch.full((B, H, T, d), float("nan"), device=dev)
        S = torch.full((B, H, d, d), float("nan"), device=dev)
        A = torch.full((B, H, d, d), float("nan"), device=dev)
        z = torch.full((B, H, d), float("nan"), device=dev)
        vla.vla_forward_noalloc(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, o=o,
                                S_out=S, A_out=A, zkey_out=z)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "S", "A", "zkey"), (o, S, A, z), ref):
            assert torch.equal(a, b), name


def test_noalloc_rejects_oversized():
    import long_context_sequence_amd as vla
    dev = _dev()
    cfg = gen.config(3)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    e = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    o = torch.empty((B, H, T, d), device=dev)
    with pytest.raises(vla.VLAError):
        vla.vla_forward_noalloc(e, e, e, e, o=o)


def test_noalloc_graph_replay():
    """The use it exists for: captured in a HIP graph (nothing allocated inside
    the capture), replayed three times with eager work between, every replay
    equal to vla_forward's result."""
    import dataclasses
    import long_context_sequence_amd as vla
    dev = _dev()
    cfg = dataclasses.replace(gen.config(3), d=64).with_sizes(B=2, H=4, T=500)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    t = _inputs(cfg, dev)
    ref = vla.vla_forward(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps, return_state=True)
    outs = [torch.empty((B, H, T, d), device=dev), torch.empty((B, H, d, d), device=dev),
            torch.empty((B, H, d, d), device=dev), torch.empty((B, H, d), device=dev)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            vla.vla_forward_noalloc(t["q"], t["k"], t["v"], t["u"], cfg.lambda0, cfg.eps,
                                    o=outs[0], S_out=outs[1], A_out=outs[2], zkey_out=outs[3])
    torch.cuda.synchronize()
    for rep in range(3):
        for a in outs:
            a.fill_(float("nan"))
        torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "S", "A", "zkey"), outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"
