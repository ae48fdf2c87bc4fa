"""The seeded input generator: determinism, bf16 rounding, the margin filter."""
import numpy as np

from moe_synth import (MARGIN, WORKLOADS, LayerShape, bf16_bits_to_f32, f32_to_bf16_bits,
                       make_inputs, workload)


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                   # bf16 spacing just above 1.0
    vals = np.array([1.0, 1.0 + 2.0 ** -8,        # exact tie -> even (1.0)
                     1.0 + 3 * 2.0 ** -8,         # tie -> even (1 + 2 ulp)
                     1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above the tie -> up
                     -2.5, 0.0], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    assert got.tolist() == [1.0, 1.0, float(one + 2 * ulp), float(one + ulp), -2.5, 0.0]


def test_bf16_is_exact_on_representable_values():
    rng = np.random.default_rng(0)
    b = rng.integers(0, 0x7F80, size=1000, dtype=np.uint16)  # finite positive patterns
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(b)), b)


def test_deterministic_and_seed_sensitive():
    s = LayerShape("g", T=50, d=32, F=48, E=6, k=2)
    a, b, c = make_inputs(s, 1), make_inputs(s, 1), make_inputs(s, 2)
    for key in ("x", "Wg", "W1", "b1", "W2", "b2"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_margin_filter_holds():
    for name in ("tiny_f32", "page1_b4s512"):
        s = WORKLOADS[name]
        inp = make_inputs(s, 0)
        x = bf16_bits_to_f32(inp["x"]) if s.dtype == "bf16" else inp["x"]
        sc = x.astype(np.float64) @ inp["Wg"].astype(np.float64).T
        if inp["bg"] is not None:
            sc += inp["bg"]
        top = -np.sort(-sc, axis=1)[:, :s.k + 1]
        assert np.all(top[:, :-1] - top[:, 1:] >= MARGIN)


def test_workload_shapes():
    assert workload(0).name == "tiny_f32" and workload(1).T == 2048
    sw = workload(3)
    assert sw.capacity == int(1.25 * sw.T / sw.E) == 160 and sw.k == 1 and sw.act == "relu"
    ds = workload(4)
    assert (ds.E, ds.k, ds.Fs, ds.d) == (256, 8, 2048, 7168)


def test_zipf_router_bias():
    s = LayerShape("z", T=4, d=8, F=8, E=64, k=1, router_bias="zipf1.1")
    bg = make_inputs(s, 0)["bg"]
    p = np.exp(bg.astype(np.float64))
    assert abs(p.sum() - 1.0) < 1e-6
    assert np.all(np.diff(bg) < 0)
    assert np.allclose(p[0] / p[1], 2.0 ** 1.1, rtol=1e-5)
