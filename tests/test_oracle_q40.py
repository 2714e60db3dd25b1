"""Pins of the oracle's 4-bit group quantisation and Q4_0 matvec (the
Q4_0 variant named in the ainews article's technical deep dive and tables,
and as a next step in the gitcode guide; reading stated in
golden/q40_handworked.json).

- hand-worked groups: scales, clamped codes, tie rules and the nibble order;
- invariants on random data: codes in [-8, 7], the largest-magnitude value
  maps to -8, dequantisation error within half a step except for clamped
  values;
- the matvec against a closed form: weights and inputs whose quantisation
  is exact (power-of-two scales), so W x is known exactly and fits fp64.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q40_handworked.json")


def _codes(q: np.ndarray) -> np.ndarray:
    q = q.reshape(-1, 16).astype(np.int64)
    return np.concatenate([(q & 15) - 8, (q >> 4) - 8], axis=1).reshape(-1)


def test_q40_handworked_golden():
    g = json.load(open(GOLDEN))
    x = np.concatenate([np.array(gr["x"], np.float32) for gr in g["groups"]])
    q, s = oracle.quantize_q40(x)
    codes = _codes(q)
    for i, gr in enumerate(g["groups"]):
        assert s[i] == np.float32(gr["scale"]), (i, s[i])
        np.testing.assert_array_equal(codes[32 * i:32 * (i + 1)], gr["codes"])
        if "bytes" in gr:
            np.testing.assert_array_equal(q[16 * i:16 * (i + 1)], gr["bytes"])


def test_q40_invariants():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(32 * 400) * rng.uniform(1e-3, 10, 32 * 400)).astype(np.float32)
    q, s = oracle.quantize_q40(x)
    c = _codes(q).reshape(-1, 32)
    xg = x.reshape(-1, 32)
    assert c.min() >= -8 and c.max() <= 7
    arg = np.abs(xg).argmax(axis=1)
    np.testing.assert_array_equal(c[np.arange(len(arg)), arg], -8)
    np.testing.assert_array_equal(s, (xg[np.arange(len(arg)), arg] / np.float32(-8)).astype(np.float32))
    err = np.abs(xg.astype(np.float64) - c * s[:, None].astype(np.float64))
    step = np.abs(s[:, None].astype(np.float64))
    clamped = np.abs(xg / s[:, None]) > 7.5
    assert (err[~clamped] <= step.repeat(32, 1)[~clamped] * (0.5 + 1e-6) + 1e-30).all()
    assert (err[clamped] <= step.repeat(32, 1)[clamped] * (1 + 1e-6)).all()


def test_q40_bad_sizes():
    with pytest.raises(ValueError):
        oracle.quantize_q40(np.zeros(48, np.float32))


def test_q40_matvec_closed_form():
    rng = np.random.default_rng(21)
    rows, cols = 37, 256
    ng = cols // 32
    # weights: codes in [-8, 7] with a -8 at a random place of every group
    # (the unique largest magnitude), power-of-two scales
    wc = rng.integers(-7, 8, (rows, cols))
    for r in range(rows):
        for g in range(ng):
            wc[r, 32 * g + rng.integers(0, 32)] = -8
    ws = 2.0 ** rng.integers(-6, 3, (rows, ng))
    W = (wc * np.repeat(ws, 32, axis=1)).astype(np.float32)
    # inputs: Q8_0 codes with a +-127 in every group, power-of-two scales
    xc = rng.integers(-126, 127, cols)
    for g in range(ng):
        xc[32 * g + rng.integers(0, 32)] = 127 * rng.choice([-1, 1])
    xs = 2.0 ** rng.integers(-5, 2, ng)
    x = (xc * np.repeat(xs, 32)).astype(np.float32)
    q = np.concatenate([oracle.quantize_q40(W[r])[0] for r in range(rows)]).reshape(rows, cols // 2)
    S = np.stack([oracle.quantize_q40(W[r])[1] for r in range(rows)])
    np.testing.assert_array_equal(S, ws.astype(np.float32))
    exact = (W.astype(np.float64) * x.astype(np.float64)).sum(axis=1)  # exact: small integers times powers of two
    out = oracle.matvec_q40(q, S, x)
    np.testing.assert_array_equal(out, exact.astype(np.float32))
    # group dots: the exact integer sums
    aq, _ = oracle.quantize(x, 32)
    np.testing.assert_array_equal(aq.astype(np.int64), xc)
    gd = oracle.group_dots_q40(q[5], aq)
    np.testing.assert_array_equal(gd, (wc[5] * xc).reshape(ng, 32).sum(axis=1))
