"""The seeded input generator: determinism, distributions and bf16 rounding."""
import numpy as np
import torch

import lrgen


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]   # ties to even
    mine = lrgen.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(lrgen.bits_to_f32(mine),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    a = lrgen.make(3, L=70, B=2, H=3)
    b = lrgen.make(3, L=70, B=2, H=3)
    for k in a.tensors:
        np.testing.assert_array_equal(a[k], b[k])
    assert a["x"].shape == (2, 70, 3, 64)
    assert a["B"].shape == (2, 70, 1, 128)
    # bf16 tensors hold bf16-representable values
    np.testing.assert_array_equal(lrgen.bits_to_f32(a.t("x").bits()), a["x"])
    assert (a["dt"] > 0).all() and (a["A"] < 0).all() and (a["A"] >= -16).all()


def test_distributions():
    g = lrgen.make(4, B=1, L=512, H=2)
    assert 0.8 < g["g"].mean() < 0.97 and (g["g"] <= 1).all() and (g["g"] > 0).all()
    assert abs(g["q"].std() * np.sqrt(128) - 1) < 0.05
    d = lrgen.make(1)
    assert d["a"].min() >= 0.90 and d["a"].max() <= 0.999
    s = lrgen.make(2, B=1, L=64, D=32)
    np.testing.assert_array_equal(s["A"][5], -np.arange(1, 17))
