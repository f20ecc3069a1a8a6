"""Decode steps (state updated in place) on the GPU vs the fp64 oracle, element
by element: y and the new state. Tolerances as for the scan: relative L2 <= 1e-5
(fp32 storage), <= 3e-3 (bf16 storage, fp32 state)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_70_amd as ssm
import workloads
from gpu_util import DEV, TOL

pytestmark = pytest.mark.gpu
_TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def _scan_step_case(batch, D, N, dtype, seed, general_A=False):
    inp = workloads.scan_inputs(batch, 1, D, N, dtype, seed=seed, with_h0=True)
    if general_A:
        rng = np.random.default_rng(seed)
        inp["A"] = -rng.uniform(0.05, 4.0, size=(D, N)).astype(np.float32)
    return inp


def _gpu_scan_step(inp, t=0, state=None, softplus=True):
    td = _TD[inp["dtype"]]
    st = state if state is not None else _dev(inp["h0"])
    col = lambda k: None if inp.get(k) is None else _dev(inp[k][:, t], td)
    y = ssm.selective_state_update(st, col("x"), col("delta"), _dev(inp["A"]), col("Bm"), col("Cm"),
                                   _dev(inp.get("Dskip")), col("z"), _dev(inp.get("delta_bias")),
                                   delta_softplus=softplus)
    return y, st


def _oracle_scan_step(inp, state, t=0, softplus=True):
    col = lambda k: None if inp.get(k) is None else inp[k][:, t]
    return oracle.selective_state_update(state, col("x"), col("delta"), inp["A"], col("Bm"), col("Cm"),
                                         inp.get("Dskip"), col("z"), inp.get("delta_bias"),
                                         delta_softplus=softplus)


def _cmp(name, dtype, y, st, yo, so):
    ey = oracle.rel_l2(y.float().cpu().numpy(), yo)
    es = oracle.rel_l2(st.cpu().numpy(), so)
    print("%s: rel_l2 y %.3e  state %.3e" % (name, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= TOL[dtype], (name, ey, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_scan_step(dtype, N):
    inp = _scan_step_case(5, 100, N, dtype, seed=N)
    y, st = _gpu_scan_step(inp)
    torch.cuda.synchronize()
    yo, so = _oracle_scan_step(inp, inp["h0"])
    _cmp("step N=%d %s" % (N, dtype), dtype, y, st, yo, so)


def test_scan_step_general_A_and_no_options():
    inp = _scan_step_case(3, 70, 16, "f32", seed=2, general_A=True)
    for k in ("z", "Dskip", "delta_bias"):
        inp[k] = None
    inp["delta"] = np.abs(inp["delta"]) * np.float32(0.3)
    y, st = _gpu_scan_step(inp, softplus=False)
    torch.cuda.synchronize()
    yo, so = _oracle_scan_step(inp, inp["h0"], softplus=False)
    _cmp("step general A", "f32", y, st, yo, so)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_steps_reproduce_the_scan(dtype):
    """30 decode steps from h0 against the oracle's scan over the same 30 tokens."""
    T = 30
    inp = workloads.scan_inputs(2, T, 96, 16, dtype, seed=7, with_h0=True)
    yo, ho = oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                   inp["Dskip"], inp["z"], inp["delta_bias"], inp["h0"])
    st = _dev(inp["h0"])
    ys = []
    for t in range(T):
        y, _ = _gpu_scan_step(inp, t, st)
        ys.append(y.float())
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    _cmp("30 steps %s" % dtype, dtype, y, st, yo, ho)


def test_scan_step_serving_batch():
    """Batch 256 at the 2.8B layer width (D 5120, N 16), bf16: every output."""
    inp = _scan_step_case(256, 5120, 16, "bf16", seed=11)
    y, st = _gpu_scan_step(inp)
    torch.cuda.synchronize()
    yo, so = _oracle_scan_step(inp, inp["h0"])
    _cmp("step B256 D5120", "bf16", y, st, yo, so)


def _gpu_ssd_step(inp, t, st, softplus=True):
    td = _TD[inp["dtype"]]
    col = lambda k: None if inp.get(k) is None else _dev(inp[k][:, t], td)
    return ssm.ssd_state_update(st, col("x"), col("dt"), _dev(inp["A"]), col("Bm"), col("Cm"),
                                _dev(inp.get("Dskip")), col("z"), _dev(inp.get("dt_bias")),
                                dt_softplus=softplus)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,P,N", [(4, 64, 64), (3, 64, 128), (2, 64, 256), (5, 3, 16), (2, 7, 32)])
def test_ssd_steps(dtype, H, P, N):
    """Decode steps of the scalar-A form chained over 5 tokens, vs the oracle's
    recurrence over the same tokens (each step's y and the final state)."""
    T = 5
    inp = workloads.ssd_inputs(3, T, H, P, N, dtype, seed=H * P + N, with_h0=True, with_z=True)
    yo, ho = oracle.ssd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["z"],
                        inp["dt_bias"], inp["h0"])
    st = _dev(inp["h0"])
    ys = [_gpu_ssd_step(inp, t, st).float() for t in range(T)]
    torch.cuda.synchronize()
    _cmp("ssd steps H%d P%d N%d %s" % (H, P, N, dtype), dtype, torch.stack(ys, dim=1), st, yo, ho)


def test_ssd_step_serving_batch():
    """Batch 32 of the 64-head, P 64, N 128 layer (state 2 MiB per sequence), bf16."""
    inp = workloads.ssd_inputs(32, 1, 64, 64, 128, "bf16", seed=12, with_h0=True, with_z=True)
    st = _dev(inp["h0"])
    y = _gpu_ssd_step(inp, 0, st)
    torch.cuda.synchronize()
    yo, so = oracle.ssd_state_update(inp["h0"], inp["x"][:, 0], inp["dt"][:, 0], inp["A"],
                                     inp["Bm"][:, 0], inp["Cm"][:, 0], inp["Dskip"], inp["z"][:, 0],
                                     inp["dt_bias"])
    _cmp("ssd step B32", "bf16", y, st, yo, so)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_step_groups(dtype):
    """B, C with 4 groups (25 channels each)."""
    inp = workloads.scan_inputs(3, 1, 100, 16, dtype, seed=41, with_h0=True, ngroups=4)
    y, st = _gpu_scan_step(inp)
    torch.cuda.synchronize()
    yo, so = _oracle_scan_step(inp, inp["h0"])
    _cmp("step groups %s" % dtype, dtype, y, st, yo, so)


def test_ssd_step_groups():
    T = 3
    inp = workloads.ssd_inputs(2, T, 6, 64, 128, "bf16", seed=42, with_h0=True, with_z=True, ngroups=3)
    yo, ho = oracle.ssd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["z"],
                        inp["dt_bias"], inp["h0"])
    st = _dev(inp["h0"])
    ys = [_gpu_ssd_step(inp, t, st).float() for t in range(T)]
    torch.cuda.synchronize()
    _cmp("ssd steps groups", "bf16", torch.stack(ys, dim=1), st, yo, ho)
