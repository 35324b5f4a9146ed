"""Seeded input generators: determinism, bf16 rounding, per-head assembly and
the structure each workload recipe promises."""
import numpy as np

import gen


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)          # bf16 spacing at 1.0
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                  -2.5, 3.0e-39, 65504.0], dtype=np.float32)
    r = gen.bf16_round(x)
    assert r[0] == one
    assert r[1] == one                    # tie -> even (1.0)
    assert r[2] == one + 2 * ulp          # tie -> even (1 + 2^-6)
    assert r[3] == one + ulp              # above the tie -> up
    assert r[4] == np.float32(-2.5)       # exactly representable
    assert np.all(gen.bf16_round(r) == r)  # idempotent
    bits = gen.bf16_bits(x)
    assert bits.dtype == np.uint16
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(bits), r)


def test_head_inputs_deterministic_and_independent():
    cfg = gen.config(2).with_sizes(B=2, H=2, T=64)
    a = gen.head_inputs(cfg, 1, 0)
    b = gen.head_inputs(cfg, 1, 0)
    c = gen.head_inputs(cfg, 0, 1)
    for n in "qkvu":
        np.testing.assert_array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_make_inputs_matches_per_head():
    for cid in (2, 3):
        cfg = gen.config(cid).with_sizes(B=2, H=3, T=48)
        x = gen.make_inputs(cfg)
        for b in range(2):
            for h in range(3):
                hi = gen.head_inputs(cfg, b, h)
                for n in "qkvu":
                    got = x[n][b, h]
                    if cfg.dtype == "bf16":
                        assert got.dtype == np.uint16
                        got = gen.bf16_bits_to_f32(got)
                    np.testing.assert_array_equal(got, hi[n])


def test_recipe_structure():
    h1 = gen.head_inputs(gen.config(1), 0, 0)
    np.testing.assert_allclose(np.linalg.norm(h1["k"], axis=1), 1.0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(h1["u"], axis=1), 1.0, atol=1e-6)
    h3 = gen.head_inputs(gen.config(3).with_sizes(T=32), 0, 0)
    for n in "qkvu":
        np.testing.assert_array_equal(gen.bf16_round(h3[n]), h3[n])
    cfg4 = gen.config(4).with_sizes(T=256)
    h4 = gen.head_inputs(cfg4, 0, 0)
    half = 128
    firstkeys = {tuple(r) for r in h4["k"][:half]}
    for t in range(half, 256, 2):         # query tokens re-ask a written key
        assert tuple(h4["q"][t]) in firstkeys
    assert np.abs(h4["k"][half:]).max() < 1.0   # small noise keys in the second half
    np.testing.assert_allclose(np.linalg.norm(h4["u"], axis=1), 1.0, atol=1e-6)
    cfg5 = gen.config(5).with_sizes(T=512, decode=64)
    h5 = gen.head_inputs(cfg5, 1, 3)
    assert h5["q_dec"].shape == (64, 128)
    n = np.linalg.norm(h5["q"], axis=1) / np.sqrt(128)
    assert n.min() < 0.2 and n.max() > 5.0      # per-token scales span ~[0.1, 10]
    np.testing.assert_allclose(np.linalg.norm(h5["u"], axis=1), 1.0, atol=1e-2)
