"""Hand-derived fixtures under tests/golden/ (the pages print no worked
example; each fixture states its derivation)."""
import json
import os

import numpy as np

from oracle import diag_scan, discretize, gla_scan, selective_scan

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_diag_halving():
    g = _load("diag_halving.json")
    a = np.array(g["a"])[None, :, None]
    b = np.array(g["b"])[None, :, None]
    h, _ = diag_scan(a, b)
    np.testing.assert_array_equal(h[0, :, 0], g["h"])


def test_zoh_ln2():
    g = _load("zoh_ln2.json")
    e, phi = discretize(np.array(g["dt"]), np.array(g["A"]), "zoh")
    assert abs(e - g["e"]) < 1e-15
    assert abs(phi - g["phi"]) < 1e-15
    L = len(g["y"])
    y, _ = selective_scan(np.ones((1, L, 1)), np.full((1, L, 1), g["dt"]),
                          np.full((1, 1), g["A"]), np.ones((1, L, 1)), np.ones((1, L, 1)))
    np.testing.assert_allclose(y[0, :, 0], g["y"], rtol=1e-15)


def test_gla_two_step():
    g = _load("gla_two_step.json")
    q = np.array(g["q"])[None, :, None, :]
    k = np.array(g["k"])[None, :, None, :]
    v = np.array(g["v"])[None, :, None, :]
    gg = np.array(g["g"])[None, :, None]
    o, S = gla_scan(q, k, v, gg)
    np.testing.assert_array_equal(o[0, :, 0], g["o"])
    np.testing.assert_array_equal(S[0, 0], g["S_last"])
