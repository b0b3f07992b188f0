"""The oracle checked against what the pages and the mathematics fix (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from pins import ALL_PINS, rand_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.forward)


def test_cumsum_matches_product_of_decays():
    """2^{G_t} is the product of the per-token decays e^{A dt_k} from the chunk start to t
    (the base-2 rescaling of the page's log-space cumulative sum, restarted every chunk)."""
    p = rand_problem(21, 2, 70, 3, 2, 2, 1)
    T = 16
    G = oracle.chunk_cumsum_log2(p["dt"], p["A"], T)
    dt = p["dt"].astype(np.float64)
    A = p["A"].astype(np.float64)
    for b in range(2):
        for h in range(3):
            for t in range(70):
                c0 = (t // T) * T
                prod = 1.0
                for k in range(c0, t + 1):
                    prod *= math.exp(A[h] * dt[b, k, h])
                assert abs(2.0 ** G[b, h, t] - prod) <= 1e-13 * prod


def test_cumsum_monotone_and_kept_exponents_nonpositive():
    """With A < 0 and dt > 0 every exponent the output keeps is <= 0 (g_i - g_j for i >= j,
    g_last - g_j, and g_i itself), so no kept decay can overflow."""
    p = rand_problem(22, 1, 512, 4, 2, 2, 1)
    T = 256
    G = oracle.chunk_cumsum_log2(p["dt"], p["A"], T)
    for c0 in range(0, 512, T):
        g = G[:, :, c0:c0 + T]
        assert np.all(g <= 0)
        assert np.all(np.diff(g, axis=-1) <= 0)
        diff = g[..., :, None] - g[..., None, :]
        i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
        assert np.all(diff[..., i >= j] <= 0)
        assert np.all(g[..., -1:] - g <= 0)


def test_cumsum_restarts_each_chunk():
    p = rand_problem(23, 1, 64, 2, 2, 2, 1)
    G = oracle.chunk_cumsum_log2(p["dt"], p["A"], 16)
    for c0 in range(0, 64, 16):
        first = p["A"].astype(np.float64) * p["dt"][0, c0].astype(np.float64) / math.log(2.0)
        assert np.allclose(G[0, :, c0], first, rtol=1e-15, atol=0)


def test_golden_regression():
    """Guards the oracle against accidental change: values written by
    tests/golden/make_golden.py, which calls only the oracle."""
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        gold = json.load(f)
    p = rand_problem(gold["seed"], *gold["shape"])
    out = oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"])
    assert np.allclose(out["y"].ravel()[: len(gold["y_head"])], gold["y_head"], rtol=1e-12, atol=1e-14)
    assert np.allclose(out["final"].ravel()[: len(gold["final_head"])], gold["final_head"], rtol=1e-12,
                       atol=1e-14)
    assert abs(float(np.sum(out["y"])) - gold["y_sum"]) < 1e-9 * max(1.0, abs(gold["y_sum"]))


def test_oracle_rejects_bad_arguments():
    p = rand_problem(24, 1, 4, 3, 2, 2, 1)
    with pytest.raises(ValueError):
        oracle.forward(p["x"], p["dt"][:, :2], p["A"], p["B"], p["C"])
    B3 = np.zeros((1, 4, 2, 2), np.float32)   # 3 heads cannot share 2 groups
    with pytest.raises(ValueError):
        oracle.forward(p["x"], p["dt"], p["A"], B3, B3)


def test_forward_pairs_matches_full():
    p = rand_problem(25, 2, 33, 4, 3, 5, 2)
    full = oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"])
    pairs = [(1, 3), (0, 0), (1, 1)]
    sub = oracle.forward_pairs(pairs, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"])
    for k, (b, h) in enumerate(pairs):
        assert np.array_equal(sub["y"][k], full["y"][b, :, h, :])
        assert np.array_equal(sub["final"][k], full["final"][b, h])
