"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented codes before
launching anything (these calls return before any HIP runtime call)."""
import ctypes
import os
import re

import pytest

import long_context_sequence_amd as vla
from long_context_sequence_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "vla.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vla_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _declared_functions()
    assert {"vla_forward", "vla_forward_penalty", "vla_forward_memory", "vla_forward_noalloc",
            "vla_forward_workspace_size", "vla_step", "vla_backward",
            "vla_backward_workspace_size", "vla_status_string"} <= set(names)
    lib = ctypes.CDLL(vla.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in vla.h but not exported"


def test_status_strings():
    for code in range(4):
        s = vla.vla_status_string(code)
        assert s.startswith("VLA_")
    assert "unknown" in vla.vla_status_string(99)


FAKE = 0x10000           # 256-byte aligned, never dereferenced: checks fail first
MIS = 0x10004            # misaligned


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, dt=0, B=1, H=1, T=4, d=64, lam=0.1, eps=1e-4,
             o=FAKE, S=None, A=None, z=None, S0=None, A0=None, z0=None, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.load().vla_forward(a["q"], a["k"], a["v"], a["u"], a["dt"], a["B"], a["H"], a["T"],
                                a["d"], a["lam"], a["eps"], a["o"], a["S"], a["A"], a["z"],
                                a["S0"], a["A0"], a["z0"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), B.VLA_ERR_INVALID_ARG),
    (dict(o=None), B.VLA_ERR_INVALID_ARG),
    (dict(k=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(S=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(B=0), B.VLA_ERR_INVALID_ARG),
    (dict(H=-1), B.VLA_ERR_INVALID_ARG),
    (dict(T=-1), B.VLA_ERR_INVALID_ARG),
    (dict(lam=0.0), B.VLA_ERR_INVALID_ARG),
    (dict(lam=float("nan")), B.VLA_ERR_INVALID_ARG),
    (dict(eps=0.0), B.VLA_ERR_INVALID_ARG),
    (dict(eps=float("inf")), B.VLA_ERR_INVALID_ARG),
    (dict(d=48), B.VLA_ERR_UNSUPPORTED),
    (dict(d=256), B.VLA_ERR_UNSUPPORTED),
    (dict(dt=2), B.VLA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 16), B.VLA_ERR_INVALID_ARG),
    (dict(ws=None), B.VLA_ERR_INVALID_ARG),
    (dict(ws=FAKE + 16), B.VLA_ERR_INVALID_ARG),
    (dict(ws_bytes=1024), B.VLA_ERR_INVALID_ARG),
])
def test_forward_argument_errors(kw, code):
    assert _fwd(**kw) == code


def test_workspace_size():
    # the per-chunk records dominate: (48 d + 1040) floats per 16 tokens of a head
    for d in (64, 96, 128):
        n1 = vla.workspace_size(1, 1, 4096, d)
        assert n1 >= 256 * (48 * d + 1040) * 4
        assert n1 % 256 == 0
        assert vla.workspace_size(8, 16, 4096, d) >= 128 * 256 * (48 * d + 1040) * 4
        assert vla.workspace_size(2, 3, 0, d) == 0
    assert vla.workspace_size(4, 4, 1000, 16) == 0
    assert vla.workspace_size(4, 4, 1000, 32) == 0
    n = ctypes.c_size_t(0)
    lib = B.load()
    assert lib.vla_forward_workspace_size(1, 1, 8, 48, ctypes.byref(n)) == B.VLA_ERR_UNSUPPORTED
    assert lib.vla_forward_workspace_size(0, 1, 8, 64, ctypes.byref(n)) == B.VLA_ERR_INVALID_ARG
    assert lib.vla_forward_workspace_size(1, 1, -1, 64, ctypes.byref(n)) == B.VLA_ERR_INVALID_ARG
    assert lib.vla_forward_workspace_size(1, 1, 8, 64, None) == B.VLA_ERR_INVALID_ARG


def _pen(**kw):
    a = dict(q=FAKE, k=FAKE, u=FAKE, dt=1, B=2, H=2, T=64, d=64, lam=0.1, eps=1e-4, A=None, z=None,
             A0=None, z0=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.load().vla_forward_penalty(a["q"], a["k"], a["u"], a["dt"], a["B"], a["H"], a["T"],
                                        a["d"], a["lam"], a["eps"], a["A"], a["z"], a["A0"],
                                        a["z0"], a["ws"], a["ws_bytes"], a["stream"])


def _mem(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, B=2, H=2, T=64, d=64, o=FAKE, S=None, S0=None,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.load().vla_forward_memory(a["v"], a["dt"], a["B"], a["H"], a["T"], a["d"], a["o"],
                                       a["S"], a["S0"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=16), B.VLA_ERR_UNSUPPORTED),
    (dict(d=32), B.VLA_ERR_UNSUPPORTED),
    (dict(d=80), B.VLA_ERR_UNSUPPORTED),
    (dict(T=0), B.VLA_ERR_INVALID_ARG),
    (dict(ws=None), B.VLA_ERR_INVALID_ARG),
    (dict(ws=FAKE + 64), B.VLA_ERR_INVALID_ARG),
    (dict(ws_bytes=4096), B.VLA_ERR_INVALID_ARG),
    (dict(dt=5), B.VLA_ERR_UNSUPPORTED),
    (dict(B=0), B.VLA_ERR_INVALID_ARG),
])
def test_phase_argument_errors(kw, code):
    assert _pen(**kw) == code
    assert _mem(**kw) == code


def test_phase_specific_argument_errors():
    assert _pen(q=None) == B.VLA_ERR_INVALID_ARG
    assert _pen(k=MIS) == B.VLA_ERR_INVALID_ARG
    assert _mem(v=MIS) == B.VLA_ERR_INVALID_ARG
    assert _pen(lam=-1.0) == B.VLA_ERR_INVALID_ARG
    assert _pen(u=None) == B.VLA_ERR_INVALID_ARG
    assert _pen(A=MIS) == B.VLA_ERR_INVALID_ARG
    assert _mem(v=None) == B.VLA_ERR_INVALID_ARG
    assert _mem(o=None) == B.VLA_ERR_INVALID_ARG
    assert _mem(S0=MIS) == B.VLA_ERR_INVALID_ARG


def test_forward_empty_no_outputs_is_ok():
    # T = 0 with no state outputs requested: nothing to do, nothing launched.
    assert _fwd(T=0, q=None, k=None, v=None, u=None, o=None) == B.VLA_OK


def _step(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, dt=1, B=2, H=2, d=128, eps=1e-4,
             S=FAKE, A=FAKE, z=FAKE, o=FAKE, stream=None)
    a.update(kw)
    return B.load().vla_step(a["q"], a["k"], a["v"], a["u"], a["dt"], a["B"], a["H"], a["d"],
                             a["eps"], a["S"], a["A"], a["z"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(S=None), B.VLA_ERR_INVALID_ARG),
    (dict(A=None), B.VLA_ERR_INVALID_ARG),
    (dict(z=None), B.VLA_ERR_INVALID_ARG),
    (dict(o=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(eps=-1.0), B.VLA_ERR_INVALID_ARG),
    (dict(d=100), B.VLA_ERR_UNSUPPORTED),
    (dict(B=0), B.VLA_ERR_INVALID_ARG),
])
def test_step_argument_errors(kw, code):
    assert _step(**kw) == code


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        vla.vla_forward(x, x, x, x)


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, dt=0, B=1, H=2, T=8, d=64, lam=0.1, eps=1e-4,
             S0=None, A0=None, z0=None, dO=FAKE, dS=None, dA=None, dz=None, dq=FAKE, dk=FAKE,
             dv=FAKE, du=FAKE, gS0=None, gA0=None, gz0=None, ws=FAKE, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return B.load().vla_backward(a["q"], a["k"], a["v"], a["u"], a["dt"], a["B"], a["H"],
                                 a["T"], a["d"], a["lam"], a["eps"], a["S0"], a["A0"], a["z0"],
                                 a["dO"], a["dS"], a["dA"], a["dz"], a["dq"], a["dk"], a["dv"],
                                 a["du"], a["gS0"], a["gA0"], a["gz0"], a["ws"], a["ws_bytes"],
                                 a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), B.VLA_ERR_INVALID_ARG),
    (dict(dq=None), B.VLA_ERR_INVALID_ARG),
    (dict(du=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(dS=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(gA0=MIS), B.VLA_ERR_INVALID_ARG),
    (dict(T=-1), B.VLA_ERR_INVALID_ARG),
    (dict(lam=0.0), B.VLA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), B.VLA_ERR_INVALID_ARG),
    (dict(d=80), B.VLA_ERR_UNSUPPORTED),
    (dict(dt=3), B.VLA_ERR_UNSUPPORTED),
    (dict(ws=None), B.VLA_ERR_INVALID_ARG),
    (dict(ws=FAKE + 64), B.VLA_ERR_INVALID_ARG),
    (dict(ws_bytes=4096), B.VLA_ERR_INVALID_ARG),
])
def test_backward_argument_errors(kw, code):
    assert _bwd(**kw) == code


def test_backward_empty_no_outputs_is_ok():
    # T = 0 and no initial-state gradients requested: nothing launched.
    assert _bwd(T=0, q=None, k=None, v=None, u=None, dO=None, dq=None, dk=None, dv=None,
                du=None, ws=None) == B.VLA_OK


def test_backward_workspace_size():
    # (4 d + 8) floats per token of each head, rounded up to 256 bytes; for the
    # head sizes of the two-pass forward also its workspace, the final state,
    # d floats per token of each head (the gate adjoints), B H + 1 ints and a
    # d x d matrix per head
    def up(x):
        return (x + 255) // 256 * 256
    for d in (16, 32, 64, 96, 128):
        n = vla.backward_workspace_size(2, 3, 100, d)
        want = up(2 * 3 * 100 * (4 * d + 8) * 4)
        if d >= 64:
            want += (up(vla.workspace_size(2, 3, 100, d)) + up(2 * 3 * (2 * d * d + d) * 4)
                     + up(2 * 3 * 100 * d * 4) + up((2 * 3 + 1) * 4) + up(2 * 3 * d * d * 4))
        assert n == want, d
    assert vla.backward_workspace_size(1, 1, 0, 64) == 0
    with pytest.raises(vla.VLAError):
        vla.backward_workspace_size(1, 1, 4, 48)


def test_scan_argument_errors():
    lib = B.load()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, dt=0, B=1, H=1, T=32, d=64, lam=0.1, eps=1e-4,
                 o=FAKE, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.vla_forward_scan(a["q"], a["k"], a["v"], a["u"], a["dt"], a["B"], a["H"],
                                    a["T"], a["d"], a["lam"], a["eps"], a["o"], None, None, None,
                                    None, None, None, a["ws"], a["ws_bytes"], None)
    assert call(d=32) == B.VLA_ERR_UNSUPPORTED
    assert call(d=48) == B.VLA_ERR_UNSUPPORTED
    assert call(T=0) == B.VLA_ERR_INVALID_ARG
    assert call(o=None) == B.VLA_ERR_INVALID_ARG
    assert call(ws=None) == B.VLA_ERR_INVALID_ARG
    assert call(ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert call(eps=0.0) == B.VLA_ERR_INVALID_ARG
    # workspace: the forward's plus (n + 1) maps of 2 d^2 floats per head, n a
    # power of two >= the chunk count (>= 2)
    for d in (64, 96, 128):
        for T in (1, 16, 17, 4096):
            nc = (T + 15) // 16
            n = 2
            while n < nc:
                n *= 2
            maps = 2 * 3 * (n + 1) * 2 * d * d * 4
            got = vla.scan_workspace_size(2, 3, T, d)
            assert vla.workspace_size(2, 3, T, d) + maps <= got < vla.workspace_size(2, 3, T, d) + maps + 512
    with pytest.raises(vla.VLAError):
        vla.scan_workspace_size(1, 1, 64, 32)


def test_sequence_length_limit():
    """The passes address a head's buffers (per-chunk records, per-token
    records, inputs, o) with 32-bit byte offsets, so a sequence whose per-head
    buffers would reach 2^31 bytes is VLA_ERR_UNSUPPORTED, before anything is
    launched (a too small workspace shows that a length passed that check)."""
    lib = B.load()
    n = ctypes.c_size_t(0)
    for d in (16, 32, 64, 96, 128):
        over = (1 << 31) // (4 * d) + 1           # o alone reaches 2^31 bytes
        assert _fwd(d=d, T=over) == B.VLA_ERR_UNSUPPORTED
        assert _bwd(d=d, T=over) == B.VLA_ERR_UNSUPPORTED
        assert lib.vla_forward_workspace_size(1, 1, over, d, ctypes.byref(n)) == \
            B.VLA_ERR_UNSUPPORTED
        # the gradients' per-token records: (4 d + 8) floats per token
        over_keep = (1 << 31) // (4 * (4 * d + 8)) + 1
        assert _bwd(d=d, T=over_keep) == B.VLA_ERR_UNSUPPORTED
        assert lib.vla_backward_workspace_size(1, 1, over_keep, d, ctypes.byref(n)) == \
            B.VLA_ERR_UNSUPPORTED
    # long sequences well inside the limits pass the check
    assert _fwd(d=128, T=1_000_000, ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert _fwd(d=64, T=2_000_000, ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert _bwd(d=128, T=1_000_000, ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert _pen(d=128, T=1_000_000, ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert _pen(d=128, T=5_000_000) == B.VLA_ERR_UNSUPPORTED
    assert _mem(d=128, T=5_000_000) == B.VLA_ERR_UNSUPPORTED


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, dt=0, B=1, H=1, T=4, d=64, lam=0.1, eps=1e-4,
             o=FAKE, S=None, A=None, z=None, S0=None, A0=None, z0=None, stream=None)
    a.update(kw)
    return B.load().vla_forward_noalloc(a["q"], a["k"], a["v"], a["u"], a["dt"], a["B"], a["H"],
                                        a["T"], a["d"], a["lam"], a["eps"], a["o"], a["S"],
                                        a["A"], a["z"], a["S0"], a["A0"], a["z0"], a["stream"])


def test_noalloc_argument_errors_and_size_limit():
    """vla_forward_noalloc checks the arguments as vla_forward does, before any
    runtime call, and refuses sizes whose workspace exceeds its fixed array."""
    assert vla.NOALLOC_SCRATCH_BYTES == 64 << 20
    with open(os.path.join(ROOT, "include", "vla.h")) as f:
        assert re.search(r"#define VLA_NOALLOC_SCRATCH_BYTES \(64u << 20\)", f.read())
    assert _noalloc(q=None) == B.VLA_ERR_INVALID_ARG
    assert _noalloc(o=MIS) == B.VLA_ERR_INVALID_ARG
    assert _noalloc(d=48) == B.VLA_ERR_UNSUPPORTED
    assert _noalloc(eps=0.0) == B.VLA_ERR_INVALID_ARG
    # the bench workload needs 546.5 MiB of workspace: more than the array
    assert vla.workspace_size(8, 16, 4096, 64) > vla.NOALLOC_SCRATCH_BYTES
    assert _noalloc(B=8, H=16, T=4096, d=64, dt=1) == B.VLA_ERR_UNSUPPORTED
    assert vla.workspace_size(4, 8, 1024, 64) <= vla.NOALLOC_SCRATCH_BYTES
    # T = 0 with no outputs: nothing to do, nothing touched
    assert _noalloc(T=0, q=None, k=None, v=None, u=None, o=None) == B.VLA_OK


def test_baseline_argument_errors():
    lib = B.load()

    def call(**kw):
        a = dict(kind=0, q=FAKE, k=FAKE, v=FAKE, dt=1, B=1, H=2, T=32, d=64, beta=1.0,
                 eps=1e-4, o=FAKE, S=None, z=None, S0=None, z0=None, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.vla_baseline_forward(a["kind"], a["q"], a["k"], a["v"], a["dt"], a["B"],
                                        a["H"], a["T"], a["d"], a["beta"], a["eps"], a["o"],
                                        a["S"], a["z"], a["S0"], a["z0"], a["ws"], a["ws_bytes"],
                                        None)
    assert call(kind=2) == B.VLA_ERR_UNSUPPORTED
    assert call(d=32) == B.VLA_ERR_UNSUPPORTED
    assert call(d=48) == B.VLA_ERR_UNSUPPORTED
    assert call(dt=7) == B.VLA_ERR_UNSUPPORTED
    assert call(q=None) == B.VLA_ERR_INVALID_ARG
    assert call(v=MIS) == B.VLA_ERR_INVALID_ARG
    assert call(o=None) == B.VLA_ERR_INVALID_ARG
    assert call(beta=float("nan")) == B.VLA_ERR_INVALID_ARG
    assert call(eps=0.0) == B.VLA_ERR_INVALID_ARG
    assert call(T=-1) == B.VLA_ERR_INVALID_ARG
    assert call(ws=None) == B.VLA_ERR_INVALID_ARG
    assert call(ws_bytes=1024) == B.VLA_ERR_INVALID_ARG
    assert call(T=0, q=None, k=None, v=None, o=None, ws=None) == B.VLA_OK
    # records as the forward's (48 d + 1040 floats per chunk) plus fp64 group sums
    n = vla.baseline_workspace_size(2, 3, 1000, 64)
    assert n >= 2 * 3 * 63 * (48 * 64 + 1040) * 4 and n % 256 == 0
    assert vla.baseline_workspace_size(1, 1, 0, 96) == 0
    with pytest.raises(vla.VLAError):
        vla.baseline_workspace_size(1, 1, 16, 32)
