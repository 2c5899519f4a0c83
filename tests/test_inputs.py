"""The seeded input generator: determinism, shapes and bf16 rounding. CPU only."""
import numpy as np

from mixture_experts_layer_37_amd import configs as C
from mixture_experts_layer_37_amd.inputs import (as_float, bf16_bits_to_f32, f32_to_bf16_bits,
                                                 make_inputs)


def test_bf16_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 1.5 * ulp, one + ulp / 2 + 2 ** -20,
                     -2.5, np.inf, -np.inf, np.finfo(np.float32).max, 0.0, -0.0],
                    dtype=np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    want = np.array([one, one, one + 2 * ulp, one + ulp, -2.5, np.inf, -np.inf,
                     np.inf, 0.0, -0.0], dtype=np.float32)   # float32 max overflows bf16
    np.testing.assert_array_equal(back, want)
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
    assert np.signbit(back[-1])


def test_generator_is_deterministic_and_shaped():
    cfg = C.SMALL.with_(tokens=300, hidden=64, inter=128)
    a = make_inputs(cfg, seed=0)
    b = make_inputs(cfg, seed=0)
    c = make_inputs(cfg, seed=1)
    for k in ("x", "w_router", "w_gate", "w_up", "w_down", "bias"):
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])
    assert a["x"].shape == (300, 64) and a["x"].dtype == np.uint16
    assert a["w_gate"].shape == (8, 64, 128) and a["w_down"].shape == (8, 128, 64)
    x = as_float(cfg, a["x"])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    wd = as_float(cfg, a["w_down"])
    assert abs(wd.std() * np.sqrt(128) - 1) < 0.05
    assert abs(a["bias"].std() - np.sqrt(0.5)) < 0.6     # 8 draws only


def test_tiny_is_fp32_and_gelu_has_no_gate():
    a = make_inputs(C.TINY, seed=0)
    assert a["x"].dtype == np.float32 and a["w_gate"] is None and a["bias"] is None


def test_zipf_bias_is_log_popularity():
    cfg = C.CAP32
    b = make_inputs(cfg.with_(tokens=4, hidden=8, inter=8), weights=False)["bias"]
    p = np.exp(b.astype(np.float64))
    p /= p.sum()
    ratio = p[0] / p[1:]
    np.testing.assert_allclose(ratio, np.arange(2, 33) ** 1.1, rtol=1e-5)
