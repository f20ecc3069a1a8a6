"""Gradients of the scalar-A (SSD) form on the GPU vs the fp64 oracle (the scan
gradients of the broadcast problem), element by element, for the loss
sum(dy*y) + sum(dh_final*h_final).

Tolerance: relative L2 <= 3e-3 per gradient tensor (bf16 storage, as for the
forward). The GPU rounds the matrix-core operands of dx, dB, dC to bf16 (one
rounding of a product of exact inputs: ~1e-3) and splits into bf16 hi + lo every
operand of the sums the decay gradients come from; dDskip is an fp32 sum of
exact products (1e-5)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_70_amd as ssm
import workloads
from gpu_util import DEV

pytestmark = pytest.mark.gpu
TOL = 3e-3


def _dev(a, dt=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)


def _case(batch, L, H, N, seed, G=1, z=False, h0=True, dh=True, **kw):
    inp = workloads.ssd_inputs(batch, L, H, 64, N, "bf16", seed=seed, with_h0=h0, with_z=z, ngroups=G, **kw)
    rng = np.random.default_rng(seed + 100)
    inp["dy"] = workloads.round_bf16(rng.standard_normal((batch, L, H, 64)).astype(np.float32))
    inp["dh_final"] = rng.standard_normal((batch, H, 64, N)).astype(np.float32) if dh else None
    return inp


def _gpu(inp, chunk, softplus=True):
    bf = torch.bfloat16
    g = ssm.ssd_chunked_bwd(_dev(inp["x"], bf), _dev(inp["dt"], bf), _dev(inp["A"]), _dev(inp["Bm"], bf),
                            _dev(inp["Cm"], bf), _dev(inp["dy"], bf), _dev(inp.get("Dskip")),
                            _dev(inp.get("z"), bf), _dev(inp.get("dt_bias")), _dev(inp.get("h0")),
                            _dev(inp.get("dh_final")), chunk=chunk, dt_softplus=softplus)
    torch.cuda.synchronize()
    return g


def _check(name, inp, chunk, softplus=True, heads=None):
    print("case %s" % name, flush=True)
    g = _gpu(inp, chunk, softplus)
    o = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"], inp.get("Dskip"),
                       inp.get("z"), inp.get("dt_bias"), inp.get("h0"), inp.get("dh_final"), softplus,
                       heads=heads)
    errs = {}
    for k, want in o.items():
        got = g.get(k)
        if want is None or got is None:
            assert (want is None) == (got is None) or k == "dh0", k
            continue
        got = got.float().cpu().numpy()
        if heads is not None:
            if k in ("dB", "dC"):
                continue                     # a subset of heads has only part of the sum
            ax = {"dx": 2, "ddt": 2, "dz": 2, "dh0": 1, "dA": 0, "dDskip": 0, "ddt_bias": 0}[k]
            got = np.take(got, heads, axis=ax)
        e = oracle.rel_l2(got.reshape(want.shape), want)
        errs[k] = e
    print("%s: %s" % (name, "  ".join("%s %.2e" % kv for kv in errs.items())), flush=True)
    for k, e in errs.items():
        assert e <= TOL, (name, k, e)


@pytest.mark.parametrize("L,chunk", [(1, 64), (64, 64), (150, 64), (150, 128), (300, 256), (600, 256)])
def test_lengths_and_chunks(L, chunk):
    """Shorter than one 64-row block, exactly one chunk, ragged last chunks, and
    several chunks of each size."""
    _check("L=%d Q=%d" % (L, chunk), _case(2, L, 4, 128, seed=L + chunk), chunk)


@pytest.mark.parametrize("N", [64, 128, 256])
def test_state_sizes(N):
    _check("N=%d" % N, _case(2, 200, 4, N, seed=N), 128)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_large_state_gate_h0(chunk):
    """N = 256 (the largest state the pages name for Mamba-2) at every chunk
    length, with the gate, an initial state and a final-state gradient, an odd
    head count and a ragged last chunk."""
    _check("N=256 z h0 Q=%d" % chunk, _case(2, 333, 5, 256, seed=256 + chunk, z=True), chunk)


@pytest.mark.parametrize("N,H", [(128, 4), (64, 5)])
def test_gate(N, H):
    """With the gate the pass recomputes the pre-gate output (the forward's output
    kernel, at chunk 256 split over two workgroups per chunk and head pair)."""
    _check("z N=%d H=%d" % (N, H), _case(2, 300, H, N, seed=3 + N + H, z=True), 256)


@pytest.mark.parametrize("H,G", [(6, 1), (5, 1), (8, 2), (9, 3)])
def test_heads_and_groups(H, G):
    """Head counts that leave a slice of heads partly empty, and groups of B, C."""
    _check("H=%d G=%d" % (H, G), _case(1, 260, H, 64, seed=H + G, G=G, z=(H == 9)), 128)


def test_optional_inputs_absent():
    inp = _case(2, 200, 4, 64, seed=7, h0=False, dh=False, with_D=False, with_bias=False)
    _check("no options", inp, 64)


def test_softplus_off():
    inp = _case(2, 200, 4, 64, seed=8, with_bias=False)
    inp["dt"] = workloads.round_bf16(np.abs(inp["dt"]) * np.float32(0.1) + np.float32(0.01))
    _check("softplus off", inp, 128, softplus=False)


def test_chunk_invariance():
    """Results do not depend on the chunk length beyond rounding."""
    inp = _case(1, 512, 4, 128, seed=9, z=True)
    a = _gpu(inp, 64)
    b = _gpu(inp, 256)
    for k in ("dx", "ddt", "dz", "dB", "dC", "dA", "dh0"):
        e = oracle.rel_l2(a[k].float().cpu().numpy(), b[k].float().cpu().numpy().astype(np.float64))
        assert e <= TOL, (k, e)


def test_deterministic_outputs():
    """dx, ddt, dz, dB, dC and dh0 have no atomics: two runs agree bit for bit."""
    inp = _case(1, 300, 6, 128, seed=10, z=True)
    a, b = _gpu(inp, 256), _gpu(inp, 256)
    for k in ("dx", "ddt", "dz", "dB", "dC", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_mamba2_layer_shape_sampled_heads():
    """Batch 2, L 8192, 64 heads x P 64, N 128, chunk 256 (the SSD workload): every
    per-head gradient of 4 sampled heads against the oracle over the whole
    sequence (dB, dC sum over all 64 heads and are checked at a smaller size)."""
    inp = workloads.make_inputs("S5")
    rng = np.random.default_rng(78)
    inp["dy"] = workloads.round_bf16(rng.standard_normal(inp["x"].shape).astype(np.float32))
    inp["dh_final"] = None
    _check("S5 bwd", inp, 256, heads=[0, 21, 42, 63])


def test_all_heads_medium():
    """64 heads over 1024 steps: dB and dC (sums over all heads) element by element."""
    _check("H=64 L=1024", _case(1, 1024, 64, 128, seed=11), 256)


def test_empty_sequence():
    """L = 0: every gradient is zero except dh0, which is dh_final."""
    inp = _case(2, 0, 4, 64, seed=12)
    g = _gpu(inp, 64)
    assert g["dx"].numel() == 0 and g["ddt"].numel() == 0
    for k in ("dA", "dDskip", "ddt_bias"):
        assert torch.count_nonzero(g[k]) == 0, k
    assert torch.equal(g["dh0"].cpu(), torch.from_numpy(inp["dh_final"])), "dh0"


def test_empty_batch():
    inp = _case(0, 100, 4, 64, seed=13)
    g = _gpu(inp, 64)
    assert g["dx"].numel() == 0 and g["dh0"].numel() == 0
