"""Benchmark of the selective-scan hot path on one MI355X.

Default workload: the long-context scan (batch 1, L 131072, D 2048, N 16,
bf16 storage, fp32 state, dt in [1e-4, 1e-2]), the largest of the scan
workloads. One step = one selective_scan_fwd call over one batch of synthetic
inputs already resident in HBM (every row of the path: stream in, softplus,
discretise, recurrence, readout, gate, store, final state). Several
input/output sets are rotated so that repeated steps cannot be served from the
256 MB Infinity Cache.

Prints ONE JSON line on stdout (progress goes to stderr). `value` is the
effective HBM bandwidth over the algorithmic bytes (x, delta, z, y once per
(b,t,d), B and C once per (b,t), parameters and the final state once), from the
mean time per call; `ms_median` and `ms_min` are over the same timed calls.
`copy_GBps` is a 512 MiB device-to-device copy timed in the same run (bytes read
+ written per second), the practical HBM rate.

`roofline` is that of the dominant kernel, the apply pass (readout over every
element): the call's algorithmic bytes divided by the kernel's mean duration,
timed live with HIP events around selective_scan_apply calls on the stream the
kernels run on, against the 8 TB/s HBM peak. `alu` relates the same duration to
the fp32 vector issue rate (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane
slots/s, no packed fp32), with the lane slots per element counted by rocprofv3
(SQ_INSTS_VALU of the kernel at this workload, 64 lanes each). `S2`, `S3` and
`S5` time the other bf16 workloads in the same run (S5: the chunked SSD form,
with its matrix-core rate over the useful causal flop count). `parity` is the
relative L2 error of the whole y and final-state tensors against the fp64
oracle, which `cpu_baseline` also times on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak, TFLOP/s
ALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12   # non-packed fp32 VALU issue slots, T/s

# Per-launch counter figures of the apply kernel, keyed by (workload, hash of the
# scan kernel sources): any change to the sources turns them into null until they
# are measured again. "traffic": HBM bytes from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs (KiB per dispatch) scaled by what the same counters read for a
# plain 256 MiB device copy (FETCH x2.0, WRITE x1.0). "valu": SQ_INSTS_VALU per
# dispatch (wave instructions; 64 lane slots each).
COUNTERS = {
    # long-context scan, apply kernel: FETCH_SIZE 864175 KiB, WRITE_SIZE 524416 KiB
    # per dispatch (12 dispatches), copy calibration FETCH x2.0 (131085 KiB read for
    # a 256 MiB copy), WRITE x1.0; SQ_INSTS_VALU 3.688e8 per dispatch
    ("S4", "dae4e3f7dfb79270"): {"traffic": 864175 * 1024 * 2 + 524416 * 1024, "valu": 368799488},
}
METRIC = "scan effective HBM GB/s (% of peak) + Gelem/s over B·L·D·N"


def scan_alg_bytes(cfg) -> int:
    """x, delta, z read and y written once per (b,t,d); B, C once per (b,t,n);
    A, bias, D once; the fp32 final state written once."""
    e = 2 if cfg.dtype == "bf16" else 4
    bld = cfg.batch * cfg.seqlen * cfg.dim
    bln = cfg.batch * cfg.seqlen * cfg.dstate
    params = 4 * (cfg.dim * cfg.dstate + 2 * cfg.dim)
    state = 4 * cfg.batch * cfg.dim * cfg.dstate
    return 4 * e * bld + 2 * e * bln + params + state


def ssd_alg_bytes(cfg) -> int:
    e = 2
    blhp = cfg.batch * cfg.seqlen * cfg.nheads * cfg.headdim
    return (2 * e * blhp + e * cfg.batch * cfg.seqlen * cfg.nheads
            + 2 * e * cfg.batch * cfg.seqlen * cfg.dstate + 3 * 4 * cfg.nheads
            + 4 * cfg.batch * cfg.nheads * cfg.headdim * cfg.dstate)


def ssd_alg_flops(cfg) -> float:
    """Useful matrix flops of the chunked form, counting the causal half of the
    two Q x Q products: C B^T, the masked product with x, the chunk states and
    the carried-state readout."""
    Q = cfg.chunk
    nch = math.ceil(cfg.seqlen / Q)
    b, H, P, N = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate
    cb = 2.0 * b * nch * Q * Q * N / 2
    diag = 2.0 * b * H * nch * Q * Q * P / 2
    states = 2.0 * b * H * nch * Q * N * P
    off = 2.0 * b * H * nch * Q * N * P
    return cb + diag + states + off


def ssd_bwd_alg_flops(cfg) -> float:
    """Useful matrix flops of the chunked SSD gradients (single-precision count,
    causal halves of the Q x Q products): per (batch, chunk, head) the tiles
    (dyc_t.x_s), dx += M1 dyc, dB += M2 C, dC += M3 B (Q^2 P, Q^2 P, Q^2 N, Q^2 N)
    and the chunk-state products (recomputed chunk states, adjoint aggregates, the
    dx, dB, dC chunk-end terms: 5 x 2 Q N P); (C_t.B_s) once per group."""
    Q = cfg.chunk
    nch = math.ceil(cfg.seqlen / Q)
    b, H, P, N = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate
    per_head = Q * Q * (2 * P + 2 * N) + 5 * 2.0 * Q * N * P
    return b * nch * (H * per_head + Q * Q * N)


def _device_inputs(inp, torch, dev):
    td = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if isinstance(v, np.ndarray):
            t = torch.from_numpy(v).to(dev)
            out[k] = t.to(td) if k in ("x", "delta", "dt", "z", "Bm", "Cm") else t
    return out


def scan_source_hash() -> str:
    """Hash of what decides the scan kernels' work: their sources and the host
    function that splits a call along time."""
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "selective_state_space_70_amd", "csrc")
    for name in ("scan_kernels.h", "scan_fwd.hip", "scan_fwd_n16.hip", "device_common.h", "chain.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "plan.cpp")) as f:
        text = f.read()
    a = text.index("ScanPlan scan_plan(")
    h.update(text[a:text.index("\n}\n", a)].encode())
    return h.hexdigest()[:16]


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def time_scan(key, steps, warmup, torch, ssm, split=False, keep=False):
    """Mean / median / min HIP-event time per selective_scan_fwd call on one scan
    workload, rotating input/output sets. With `split` the chunk-state and apply
    passes are also timed separately (same calls, one pass at a time); with
    `keep` the outputs of the unrotated set come back to the host for parity."""
    cfg = workloads.CONFIGS[key]
    dev = torch.device("cuda:0")
    log("%s: generating inputs" % key)
    base = workloads.make_inputs(key)
    nsets = max(2, math.ceil(768e6 / scan_alg_bytes(cfg)))
    sets = []
    for i in range(nsets):
        t = _device_inputs(base, torch, dev)
        if i:  # distinct buffers with the same statistics: roll along time
            for k in ("x", "delta", "z"):
                t[k] = torch.roll(t[k], shifts=97 * i, dims=1).contiguous()
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device=dev)
        sets.append(t)
    ws = [torch.empty(max(1, ssm.scan_workspace_bytes(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate,
                                                      sets[0]["x"].dtype)),
                      dtype=torch.uint8, device=dev) for _ in range(nsets)]

    def call(i, which):
        t = sets[i % nsets]
        ssm.selective_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                               t["delta_bias"], None, out=t["y"], final_state_out=t["hf"],
                               workspace=ws[i % nsets], passes=which)

    log("%s: timing %d calls" % (key, steps))
    for i in range(warmup):
        call(i, "all")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = _events(torch, steps)
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        call(i, "all")
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    out = {"cfg": cfg, "wall": time.perf_counter() - t0,
           "per_call": [a.elapsed_time(b) for a, b in ev]}
    if split:
        ev1, ev2 = _events(torch, steps), _events(torch, steps)
        for i in range(steps):
            ev1[i][0].record(stream)
            call(i, "chunk_states")
            ev1[i][1].record(stream)
            ev2[i][0].record(stream)
            call(i, "apply")
            ev2[i][1].record(stream)
        torch.cuda.synchronize()
        out["states"] = [a.elapsed_time(b) for a, b in ev1]
        out["apply"] = [a.elapsed_time(b) for a, b in ev2]
    if keep:
        out["inputs"] = base
        out["y"] = sets[0]["y"].float().cpu().numpy()
        out["hf"] = sets[0]["hf"].cpu().numpy()
    del sets, ws
    torch.cuda.empty_cache()
    return out


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def summary(per_call):
    srt = sorted(per_call)
    return sum(per_call) / len(per_call), srt[len(srt) // 2], srt[0]


def time_ssd(steps, warmup, torch, ssm, keep=False):
    """HIP-event time per ssd_chunked_fwd call on the SSD workload, rotating
    input/output sets; with `keep` the unrotated set's outputs come back."""
    cfg = workloads.CONFIGS["S5"]
    dev = torch.device("cuda:0")
    log("S5: generating inputs")
    base = workloads.make_inputs("S5")
    nsets = max(2, math.ceil(768e6 / ssd_alg_bytes(cfg)))
    sets = []
    for i in range(nsets):
        t = _device_inputs(base, torch, dev)
        if i:
            t["x"] = torch.roll(t["x"], shifts=97 * i, dims=1).contiguous()
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32,
                              device=dev)
        sets.append(t)
    ws = torch.empty(ssm.ssd_workspace_bytes(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim,
                                             cfg.dstate, cfg.chunk), dtype=torch.uint8, device=dev)

    def step(i):
        t = sets[i % nsets]
        ssm.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], None,
                            t["dt_bias"], None, chunk=cfg.chunk, out=t["y"],
                            final_state_out=t["hf"], workspace=ws)

    log("S5: timing %d calls" % steps)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = _events(torch, steps)
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    out = {"cfg": cfg, "per_call": [a.elapsed_time(b) for a, b in ev]}
    if keep:
        out["inputs"] = base
        out["y"] = sets[0]["y"].float().cpu().numpy()
        out["hf"] = sets[0]["hf"].cpu().numpy()
    del sets, ws
    torch.cuda.empty_cache()
    return out


def measure_copy_rate(torch):
    """Device-to-device copy of 512 MiB, timed with HIP events: the practical HBM rate
    (bytes read + written per second) to quote next to the 8 TB/s spec."""
    n = 512 * 1024 * 1024
    a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in ev:
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[len(ev) // 2]
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def _time_rotating(call, nsets, steps, warmup, torch):
    """Mean HIP-event time (ms) of call(i) over `steps` calls, rotating i over the sets."""
    for i in range(warmup):
        call(i % nsets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        call(i % nsets)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def time_next_rows(steps, warmup, torch, ssm):
    """Decode steps and the short convolution at serving / layer shapes: effective
    GB/s over their algorithmic bytes (each input and output once; the state read
    and written once)."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    rn = lambda *s, dt=bf: torch.randn(*s, generator=g, device=dev, dtype=torch.float32).to(dt)
    out = {}
    # per-channel decode step: batch 256, D 5120, N 16 (state 84 MB)
    Bt, D, N = 256, 5120, 16
    A = -torch.arange(1, N + 1, device=dev, dtype=torch.float32).repeat(D, 1).contiguous()
    par = [rn(D, dt=torch.float32) for _ in range(2)]
    sets = []
    for _ in range(4):
        sets.append(dict(st=rn(Bt, D, N, dt=torch.float32), x=rn(Bt, D), dl=rn(Bt, D) * 0.5, z=rn(Bt, D),
                         B=rn(Bt, N), C=rn(Bt, N), y=torch.empty(Bt, D, dtype=bf, device=dev)))
    dbias = par[1] - 3.0          # formed once, outside the timed calls
    ms = _time_rotating(lambda i: ssm.selective_state_update(
        sets[i]["st"], sets[i]["x"], sets[i]["dl"], A, sets[i]["B"], sets[i]["C"], par[0], sets[i]["z"],
        dbias, out=sets[i]["y"]), 4, steps, warmup, torch)
    alg = 8 * Bt * D * N + 2 * 4 * Bt * D + 2 * 2 * Bt * N + 4 * D * N + 8 * D
    out["decode_B256_D5120_N16"] = {"ms": round(ms, 5), "GB/s": round(alg / ms / 1e6, 1),
                                    "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del sets
    # scalar-A decode step: batch 32, 64 heads x P 64, N 128 (state 134 MB)
    Bt, H, P, N = 32, 64, 64, 128
    Ah = -torch.rand(H, generator=g, device=dev) * 15.0 - 1.0
    hp = [rn(H, dt=torch.float32) for _ in range(2)]
    sets = []
    for _ in range(3):
        sets.append(dict(st=rn(Bt, H, P, N, dt=torch.float32), x=rn(Bt, H, P), dt=rn(Bt, H) * 0.5,
                         B=rn(Bt, N), C=rn(Bt, N), y=torch.empty(Bt, H, P, dtype=bf, device=dev)))
    hbias = hp[1] - 3.0
    ms = _time_rotating(lambda i: ssm.ssd_state_update(
        sets[i]["st"], sets[i]["x"], sets[i]["dt"], Ah, sets[i]["B"], sets[i]["C"], hp[0], None,
        hbias, out=sets[i]["y"]), 3, steps, warmup, torch)
    alg = 8 * Bt * H * P * N + 2 * 2 * Bt * H * P + 2 * Bt * H + 2 * 2 * Bt * N + 12 * H
    out["ssd_decode_B32_H64_P64_N128"] = {"ms": round(ms, 5), "GB/s": round(alg / ms / 1e6, 1),
                                          "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del sets
    # conv1d (width 4) + SiLU at the scan workload shapes
    for key in ("S2", "S3"):
        c = workloads.CONFIGS[key]
        w = rn(c.dim, 4, dt=torch.float32)
        bias = rn(c.dim, dt=torch.float32)
        nsets = max(2, math.ceil(768e6 / (4 * c.batch * c.seqlen * c.dim)))
        xs = [rn(c.batch, c.seqlen, c.dim) for _ in range(nsets)]
        ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
        ms = _time_rotating(lambda i: ssm.causal_conv1d_fwd(xs[i], w, bias, out=ys[i]), nsets, steps,
                            warmup, torch)
        alg = 2 * 2 * c.batch * c.seqlen * c.dim + 5 * 4 * c.dim
        out["conv1d_%s_B%d_L%d_D%d" % (key, c.batch, c.seqlen, c.dim)] = {
            "ms": round(ms, 5), "GB/s": round(alg / ms / 1e6, 1),
            "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
        del xs, ys
    return out


def time_bwd(key, steps, warmup, torch, ssm):
    """Gradients of the scan workload (selective_scan_bwd) with rotated inputs.
    Algorithmic bytes: x, delta, z, dy read and dx, ddelta, dz written once per
    (b,t,d); B, C read and dB, dC (fp32) written once per (b,t,n); parameters."""
    cfg = workloads.CONFIGS[key]
    dev = torch.device("cuda:0")
    base = workloads.make_inputs(key)
    es = 2 if cfg.dtype == "bf16" else 4
    bld = cfg.batch * cfg.seqlen * cfg.dim
    bln = cfg.batch * cfg.seqlen * cfg.dstate
    alg = 7 * bld * es + 2 * bln * es + 2 * bln * 4 + 3 * cfg.dim * cfg.dstate * 4
    nsets = max(2, math.ceil(768e6 / alg))
    sets = []
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for i in range(nsets):
        t = _device_inputs(base, torch, dev)
        if i:
            t["x"] = torch.roll(t["x"], shifts=131 * i, dims=1).contiguous()
        t["dy"] = torch.randn(t["x"].shape, generator=g, device=dev).to(t["x"].dtype)
        sets.append(t)
    ws = torch.empty(1, dtype=torch.uint8, device=dev)

    def call(i):
        t = sets[i]
        ssm.selective_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"],
                               t["delta_bias"], None, None)

    ms = _time_rotating(call, nsets, steps, warmup, torch)
    return {"ms": round(ms, 4), "GB/s": round(alg / ms / 1e6, 1), "Gelem/s": round(cfg.elements / ms / 1e6, 1)}


def cpu_baseline(key, inp, budget_s=10.0):
    """The fp64 oracle on the host cores over the same workload (all channels,
    whole sequence), repeated until ~budget_s of wall time; effective GB/s on the
    same algorithmic-bytes count as the GPU figure. Also one run on a single
    thread over a sample of 64 channels (scaled to the whole workload). Returns
    the baseline record and the oracle's (y, h_final) of the first run."""
    import oracle
    cfg = workloads.CONFIGS[key]
    threads = oracle.num_threads()
    args = (inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["z"],
            inp["delta_bias"])
    log("%s: oracle on %d threads" % (key, threads))
    runs, t0 = 0, time.perf_counter()
    ref = None
    while True:
        res = oracle.selective_scan(*args)
        if ref is None:
            ref = res
        del res
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 200:
            break
    per = el / runs
    oracle.set_num_threads(1)
    chans = np.arange(0, cfg.batch * cfg.dim, max(1, cfg.batch * cfg.dim // 64))[:64]
    t1 = time.perf_counter()
    oracle.selective_scan(*args, channels=chans)
    single = (time.perf_counter() - t1) * (cfg.batch * cfg.dim) / len(chans)
    oracle.set_num_threads(threads)
    rec = {"value": round(scan_alg_bytes(cfg) / per / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "single_thread_GBps": round(scan_alg_bytes(cfg) / single / 1e9, 4),
           "sample": "full %s workload (all %d channels x L %d), fp64 C recurrence, %d run(s), "
                     "%.2f s per run; single thread timed on 64 channels and scaled"
                     % (key, cfg.batch * cfg.dim, cfg.seqlen, runs, per)}
    return rec, ref


def parity(key, got, inputs):
    """Relative L2 error of the whole y and final-state tensors against the fp64
    oracle on the same inputs."""
    import oracle
    if key == "S5":
        yo, ho = oracle.ssd(inputs["x"], inputs["dt"], inputs["A"], inputs["Bm"], inputs["Cm"],
                            inputs["Dskip"], None, inputs["dt_bias"], None)
    else:
        yo, ho = oracle.selective_scan(inputs["x"], inputs["delta"], inputs["A"], inputs["Bm"],
                                       inputs["Cm"], inputs["Dskip"], inputs["z"],
                                       inputs["delta_bias"])
    return parity_of(got, (yo, ho))


def parity_of(got, ref):
    def rel(u, v):
        u = u.reshape(-1)
        v = v.reshape(-1)
        num = den = 0.0
        for i in range(0, u.size, 1 << 22):
            a = u[i:i + (1 << 22)].astype(np.float64)
            b = v[i:i + (1 << 22)]
            num += float(np.dot(a - b, a - b))
            den += float(np.dot(b, b))
        return math.sqrt(num / den) if den else 0.0
    return {"y_rel_l2": float("%.4g" % rel(got[0], ref[0])),
            "state_rel_l2": float("%.4g" % rel(got[1], ref[1]))}


def gpu_name(torch):
    p = torch.cuda.get_device_properties(0)
    return "%s (%s, %d CUs)" % (p.name, getattr(p, "gcnArchName", "?"), p.multi_processor_count)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_ssd_bwd(steps, warmup, torch, ssm):
    """Gradients of the SSD workload (ssd_chunked_bwd) with rotated inputs."""
    cfg = workloads.CONFIGS["S5"]
    dev = torch.device("cuda:0")
    base = workloads.make_inputs("S5")
    nsets = 2
    sets = []
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    for i in range(nsets):
        t = _device_inputs(base, torch, dev)
        if i:
            t["x"] = torch.roll(t["x"], shifts=97 * i, dims=1).contiguous()
        t["dy"] = torch.randn(t["x"].shape, generator=g, device=dev).to(t["x"].dtype)
        sets.append(t)

    def call(i):
        t = sets[i]
        ssm.ssd_chunked_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], None,
                            t["dt_bias"], None, None, chunk=cfg.chunk)

    ms = _time_rotating(call, nsets, steps, warmup, torch)
    tf = ssd_bwd_alg_flops(cfg) / ms / 1e9
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="S4", choices=["S1", "S2", "S3", "S4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle runs that give the rel-L2 fields")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline workload (no other workloads, oracle or copy probe)")
    ap.add_argument("--extra", action="store_true",
                    help="(the default) also time the decode steps, the short convolution and the "
                         "gradients, as the line's \"extra\" object")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the decode, convolution and gradient timings")
    ap.add_argument("--ssd-only", action="store_true",
                    help="time only the Mamba-2 SSD workload and print its own JSON line "
                         "(for profiling the SSD kernels; not the headline line)")
    ap.add_argument("--next-only", action="store_true",
                    help="time only the decode steps, the short convolution and the gradients "
                         "(own JSON line)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run three plain 256 MiB device-to-device copies (the reference "
                         "kernel of known size that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        import torch
        n = 256 * 1024 * 1024
        a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda")
        a.fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
        return

    import torch
    import selective_state_space_70_amd as ssm

    if args.next_only:
        out = time_next_rows(args.steps, args.warmup, torch, ssm)
        out["bwd_S2"] = time_bwd("S2", args.steps, args.warmup, torch, ssm)
        out["bwd_S5"] = time_ssd_bwd(args.steps, args.warmup, torch, ssm)
        print(json.dumps(out), flush=True)
        return

    if args.ssd_only:
        r5 = time_ssd(args.steps, args.warmup, torch, ssm)
        print(json.dumps(dict({"workload": "S5 " + r5["cfg"].name}, **ssd_fields(r5))), flush=True)
        return

    key = args.config
    want_parity = not (args.no_parity or args.headline_only)
    want_cpu = not (args.no_cpu_baseline or args.headline_only)
    r = time_scan(key, args.steps, args.warmup, torch, ssm, split=True,
                  keep=want_parity or want_cpu)
    cfg = r["cfg"]
    ms, ms_median, ms_min = summary(r["per_call"])
    ms_states = sum(r["states"]) / len(r["states"])
    ms_apply = sum(r["apply"]) / len(r["apply"])
    alg = scan_alg_bytes(cfg)
    gbs = alg / (ms * 1e-3) / 1e9
    kern_gbs = alg / (ms_apply * 1e-3) / 1e9
    src_hash = scan_source_hash()
    cnt = COUNTERS.get((key, src_hash), {})
    valu = cnt.get("valu")
    slots = valu * 64 / cfg.elements if valu else None
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": "%s %s" % (key, cfg.name), "batch": cfg.batch,
                   "seq_len": cfg.seqlen, "dim": cfg.dim, "dstate": cfg.dstate,
                   "storage": cfg.dtype, "compute": "f32", "state": "f32"},
        "gpu": gpu_name(torch),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "ms_median": round(ms_median, 5), "ms_min": round(ms_min, 5),
        "gelem_per_s": round(cfg.elements / (ms * 1e-3) / 1e9, 2),
        "wall_s_timed": round(r["wall"], 4),
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": cnt.get("traffic"),
                     "kernel": "scan_main_kernel (selective_scan_apply)",
                     "kernel_ms": round(ms_apply, 5),
                     "alg_per_unit": "%d algorithmic bytes per call (x, delta, z, y per (b,t,d); "
                                     "B, C per (b,t); parameters; final state), one launch per call"
                                     % alg,
                     "source_hash": src_hash},
        "alu": {"bound": "fp32 VALU issue", "peak": round(ALU_PEAK_TSLOTS, 2),
                "unit": "T lane slots/s",
                "slots_per_elem": round(slots, 3) if slots else None,
                "achieved": round(slots * cfg.elements / (ms_apply * 1e-3) / 1e12, 2) if slots else None,
                "frac": round(slots * cfg.elements / (ms_apply * 1e-3) / 1e12 / ALU_PEAK_TSLOTS, 4)
                if slots else None,
                "kernel": "scan_main_kernel"},
        "passes_ms": {"chunk_states": round(ms_states, 5), "apply": round(ms_apply, 5)},
    }
    head_out = (r.get("y"), r.get("hf"))
    head_in = r.get("inputs")
    del r
    if not args.headline_only:
        line["copy_GBps"] = round(measure_copy_rate(torch), 1)
        line["copy_frac"] = round(gbs / line["copy_GBps"], 4)
        for k2 in ("S2", "S3"):
            if k2 == key:
                continue
            r2 = time_scan(k2, max(10, args.steps // 2), 3, torch, ssm, keep=want_parity)
            m2, _, mn2 = summary(r2["per_call"])
            c2 = r2["cfg"]
            line[k2] = {"ms": round(m2, 5), "ms_min": round(mn2, 5),
                        "GB/s": round(scan_alg_bytes(c2) / m2 / 1e6, 1),
                        "hbm_frac": round(scan_alg_bytes(c2) / m2 / 1e6 / HBM_PEAK_GBS, 4),
                        "Gelem/s": round(c2.elements / m2 / 1e6, 1)}
            if want_parity:
                log("%s: oracle for parity" % k2)
                line[k2]["parity"] = parity(k2, (r2["y"], r2["hf"]), r2["inputs"])
            del r2
        r5 = time_ssd(max(10, args.steps // 2), 3, torch, ssm, keep=want_parity)
        line["S5"] = ssd_fields(r5)
        if want_parity:
            log("S5: oracle for parity")
            line["S5"]["parity"] = parity("S5", (r5["y"], r5["hf"]), r5["inputs"])
        del r5
    if not (args.no_extra or args.headline_only):
        extra = time_next_rows(max(10, args.steps), 3, torch, ssm)
        extra["bwd_S2"] = time_bwd("S2", max(10, args.steps // 2), 2, torch, ssm)
        extra["bwd_S5"] = time_ssd_bwd(max(10, args.steps // 2), 2, torch, ssm)
        line["extra"] = extra
    if want_cpu:
        rec, ref = cpu_baseline(key, head_in)
        line["cpu_baseline"] = rec
        if want_parity:
            line["parity"] = parity_of(head_out, ref)
        del ref
    elif want_parity:
        log("%s: oracle for parity" % key)
        line["parity"] = parity(key, head_out, head_in)
    print(json.dumps(line), flush=True)


def ssd_fields(r5):
    c5 = r5["cfg"]
    m5, _, mn5 = summary(r5["per_call"])
    tf = ssd_alg_flops(c5) / m5 / 1e9
    return {"ms": round(m5, 5), "ms_min": round(mn5, 5),
            "GB/s": round(ssd_alg_bytes(c5) / m5 / 1e6, 1),
            "hbm_frac": round(ssd_alg_bytes(c5) / m5 / 1e6 / HBM_PEAK_GBS, 4),
            "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


if __name__ == "__main__":
    main()
