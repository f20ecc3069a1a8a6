"""The seeded input generator (CPU): bf16 rounding agrees with torch's
round-to-nearest-even conversion, and the recipe is reproducible."""
import numpy as np
import torch

import workloads


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=1 << 18, dtype=np.uint32)
    a = bits.view(np.float32)
    edge = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45,
                     1.00390625, 1.01171875, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0],
                    dtype=np.float32)
    a = np.concatenate([a, edge, rng.standard_normal(1 << 16).astype(np.float32)])
    ours = workloads.round_bf16(a)
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).float().numpy()
    finite = ~np.isnan(a)
    assert np.array_equal(ours[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.isnan(ours[~finite]).all()
    assert np.array_equal(workloads.bf16_bits(a[finite]),
                          (ref[finite].view(np.uint32) >> 16).astype(np.uint16))


def test_inputs_are_reproducible_and_bf16_exact():
    a = workloads.scan_inputs(2, 33, 70, 16, "bf16", seed=5, with_h0=True)
    b = workloads.scan_inputs(2, 33, 70, 16, "bf16", seed=5, with_h0=True)
    for k in ("x", "delta", "z", "Bm", "Cm", "Dskip", "delta_bias", "A", "h0"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("x", "delta", "z", "Bm", "Cm"):
        assert np.array_equal(workloads.round_bf16(a[k]), a[k]), k
