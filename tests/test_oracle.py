"""The fp64 oracle against its pins (closed forms, library routines, invariants)."""
import numpy as np
import pytest

import oracle
import oracle_pins
import workloads


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _np_twin(inp):
    """Per-timestep recurrence vectorised over channels in numpy (a second,
    independently typed implementation; catches indexing slips in the C loop)."""
    x, delta, z = (inp[k].astype(np.float64) for k in ("x", "delta", "z"))
    Bm, Cm, A = (inp[k].astype(np.float64) for k in ("Bm", "Cm", "A"))
    v = delta + inp["delta_bias"].astype(np.float64)
    dt = np.logaddexp(0.0, v)
    batch, L, D = x.shape
    h = np.zeros((batch, D, A.shape[1]))
    ys = np.empty_like(x)
    for t in range(L):
        h = np.exp(dt[:, t, :, None] * A[None]) * h + dt[:, t, :, None] * Bm[:, t, None, :] * x[:, t, :, None]
        y = np.einsum("bdn,bn->bd", h, Cm[:, t]) + inp["Dskip"] * x[:, t]
        ys[:, t] = y * z[:, t] / (1.0 + np.exp(-z[:, t]))
    return ys, h


def test_numpy_twin_tiny_config():
    inp = workloads.make_inputs("S1")
    y, hf = oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                  inp["Dskip"], inp["z"], inp["delta_bias"])
    yt, ht = _np_twin(inp)
    assert oracle.rel_l2(y, yt) < 1e-13 and oracle.rel_l2(hf, ht) < 1e-13


def test_oracle_rejects_bad_channel():
    inp = workloads.scan_inputs(1, 4, 3, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                              channels=[5])


def test_oracle_empty_sequence():
    inp = workloads.scan_inputs(2, 0, 3, 4, seed=1, with_h0=True)
    y, hf = oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                  inp["Dskip"], inp["z"], inp["delta_bias"], inp["h0"])
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(hf, inp["h0"].astype(np.float64))
