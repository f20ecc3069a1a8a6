"""Helpers for the GPU parity tests: seeded inputs to device tensors, a call
through the C ABI (via the binding), and the fp64 oracle on the same inputs."""
import numpy as np
import torch

import oracle
import selective_state_space_70_amd as ssm

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-5, "bf16": 3e-3}
_TD = {"f32": torch.float32, "bf16": torch.bfloat16}
STORAGE = ("x", "delta", "dt", "z", "Bm", "Cm")


def to_dev(inp):
    dt = _TD[inp["dtype"]]
    out = {}
    for k, v in inp.items():
        if isinstance(v, np.ndarray):
            t = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
            out[k] = t.to(dt) if k in STORAGE else t
        else:
            out[k] = v
    return out


def run_scan(inp, softplus=True, **kw):
    t = to_dev(inp)
    y, hf = ssm.selective_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], t.get("Dskip"),
                                   t.get("z"), t.get("delta_bias"), t.get("h0"),
                                   delta_softplus=softplus, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), (hf.cpu().numpy() if hf is not None else None)


def oracle_scan(inp, softplus=True, channels=None):
    return oracle.selective_scan(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                 inp.get("Dskip"), inp.get("z"), inp.get("delta_bias"),
                                 inp.get("h0"), delta_softplus=softplus, channels=channels)


def run_ssd(inp, chunk, softplus=True, **kw):
    t = to_dev(inp)
    y, hf = ssm.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t.get("Dskip"),
                                t.get("z"), t.get("dt_bias"), t.get("h0"), chunk=chunk,
                                dt_softplus=softplus, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), (hf.cpu().numpy() if hf is not None else None)


def oracle_ssd(inp, softplus=True, channels=None):
    return oracle.ssd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp.get("Dskip"),
                      inp.get("z"), inp.get("dt_bias"), inp.get("h0"), dt_softplus=softplus,
                      channels=channels)


def sample_channels(total, count, seed):
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(total, size=min(count, total), replace=False).tolist())
    picks.update({0, total - 1})
    return np.array(sorted(picks), dtype=np.int64)


def rel_l2_blocked(u, v, rows=1 << 22):
    """||u - v||_2 / ||v||_2 over the whole tensor in fp64, accumulated over
    blocks of the flattened arrays (full-size outputs do not need fp64 copies
    of the whole tensor)."""
    u = np.asarray(u).reshape(-1)
    v = np.asarray(v).reshape(-1)
    assert u.shape == v.shape, (u.shape, v.shape)
    num = den = 0.0
    for i in range(0, u.size, rows):
        a = u[i:i + rows].astype(np.float64)
        b = v[i:i + rows].astype(np.float64)
        num += float(np.dot(a - b, a - b))
        den += float(np.dot(b, b))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(np.sqrt(num / den))


def report(name, ey, eh):
    print("%s: rel_l2 y %.3e  state %.3e" % (name, ey, eh), flush=True)
