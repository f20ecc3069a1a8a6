"""Scalar-A (SSD) chunked form on the GPU matrix cores vs the fp64 oracle
(plain per-step recurrence). bf16 inputs, fp32 state: relative L2 <= 3e-3 on y
and on the final state."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL, oracle_ssd, rel_l2_blocked, report, run_ssd

pytestmark = pytest.mark.gpu


def _check(name, inp, chunk, softplus=True):
    y, hf = run_ssd(inp, chunk, softplus)
    yo, ho = oracle_ssd(inp, softplus)
    ey, eh = oracle.rel_l2(y, yo), oracle.rel_l2(hf, ho)
    report(name, ey, eh)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"], (name, ey, eh)
    assert np.isfinite(y).all()
    return y, hf


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("L", [1, 64, 150, 600])
def test_lengths_and_chunks(L, chunk):
    inp = workloads.ssd_inputs(1, L, 3, 64, 128, "bf16", seed=L + chunk, with_h0=True)
    _check("L=%d Q=%d" % (L, chunk), inp, chunk)


@pytest.mark.parametrize("N", [64, 128, 256])
def test_state_sizes(N):
    inp = workloads.ssd_inputs(2, 300, 4, 64, N, "bf16", seed=N, with_h0=True)
    _check("N=%d" % N, inp, 128)


@pytest.mark.parametrize("batch,L,H,N,chunk", [(2, 700, 9, 128, 256), (2, 513, 5, 256, 128),
                                                 (3, 200, 6, 64, 64), (1, 1000, 13, 128, 128)])
def test_head_groups(batch, L, H, N, chunk):
    """Head counts that leave the last group of heads partly empty, several batch
    rows and chunks, every time block of a chunk."""
    inp = workloads.ssd_inputs(batch, L, H, 64, N, "bf16", seed=H * 31 + N, with_h0=True, with_z=True)
    _check("heads B%d L%d H%d N%d Q%d" % (batch, L, H, N, chunk), inp, chunk)


@pytest.mark.parametrize("H,N,G,chunk,L", [(8, 128, 2, 256, 600), (6, 64, 3, 64, 300),
                                           (10, 128, 2, 128, 500), (8, 256, 8, 256, 300)])
def test_groups(H, N, G, chunk, L):
    """G groups of B, C shared by H / G heads each (odd heads per group leave
    partly empty workgroups)."""
    inp = workloads.ssd_inputs(2, L, H, 64, N, "bf16", seed=H + G * 7, with_h0=True, with_z=True, ngroups=G)
    _check("groups H%d N%d G%d Q%d" % (H, N, G, chunk), inp, chunk)


@pytest.mark.parametrize("N", [64, 128])
def test_chunk256_two_workgroups(N):
    """Chunk 256, where the output kernel splits each chunk's time blocks over two
    workgroups (0 and 3, 1 and 2): a ragged last chunk of 88 steps (blocks 2 and 3
    empty), an odd head count (a half-empty head pair), the gate and an initial
    state."""
    inp = workloads.ssd_inputs(2, 600, 3, 64, N, "bf16", seed=40 + N, with_h0=True, with_z=True)
    _check("chunk 256 N=%d" % N, inp, 256)


def test_gate_and_no_skip():
    inp = workloads.ssd_inputs(2, 333, 3, 64, 64, "bf16", seed=21, with_z=True, with_D=False)
    _check("z, no D", inp, 64)


def test_no_bias_softplus_off():
    inp = workloads.ssd_inputs(1, 260, 2, 64, 64, "bf16", seed=22, with_bias=False)
    inp["dt"] = workloads.round_bf16(np.abs(inp["dt"]) * np.float32(0.1))
    _check("softplus off", inp, 128, softplus=False)


def test_chunk_invariance():
    inp = workloads.ssd_inputs(1, 1024, 2, 64, 128, "bf16", seed=23, with_h0=True)
    ya, ha = run_ssd(inp, 64)
    yb, hb = run_ssd(inp, 256)
    # both are within tolerance of the oracle; they also agree with each other
    assert oracle.rel_l2(ya, yb) <= 3e-3 and oracle.rel_l2(ha, hb) <= 3e-3


def test_empty_sequence_copies_state():
    inp = workloads.ssd_inputs(1, 0, 2, 64, 64, "bf16", seed=1, with_h0=True)
    y, hf = run_ssd(inp, 64)
    assert y.shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(hf, inp["h0"])


def test_deterministic():
    inp = workloads.ssd_inputs(1, 700, 4, 64, 128, "bf16", seed=24)
    y1, h1 = run_ssd(inp, 256)
    y2, h2 = run_ssd(inp, 256)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_full_size_whole_tensor():
    """The Mamba-2 SSD workload (batch 2, L 8192, 64 heads x 64, N 128, chunk 256):
    every element of y and of the final state against the oracle run over all
    (b, h, p) channels and the whole sequence."""
    cfg = workloads.CONFIGS["S5"]
    print("generating S5", flush=True)
    inp = workloads.make_inputs("S5")
    y, hf = run_ssd(inp, cfg.chunk)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    print("oracle S5", flush=True)
    yo, ho = oracle_ssd(inp)
    ey, eh = rel_l2_blocked(y, yo), rel_l2_blocked(hf, ho)
    report("S5 whole tensor", ey, eh)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_long_memory_large_state():
    """Long-memory steps (dt in [1e-4, 1e-2]: little decay per chunk, so every
    chunk's state reaches far ahead) with the largest state (N 256), chunk 256,
    16 chunks, the gate and an initial state: the case where bf16 rounding of
    carried states would accumulate."""
    inp = workloads.ssd_inputs(1, 4096, 8, 64, 256, "bf16", seed=77, dt_range=(1e-4, 1e-2),
                               with_h0=True, with_z=True)
    _check("long memory N=256 Q=256 L=4096", inp, 256)
