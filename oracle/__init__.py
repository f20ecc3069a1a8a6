"""fp64 CPU oracle (ctypes front-end of ``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``. The HIP product package never
imports it, and it imports nothing from the product package.

Every function evaluates the plain per-timestep recurrence in double precision
(see the header of ``oracle.c`` for the definition and the page citations).
Inputs are the float32 storage values both sides read (bf16 inputs arrive as
their exact float32 upcast).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)
            L = ctypes.CDLL(_LIB)
        L.oracle_selective_scan_f64.restype = ctypes.c_int
        L.oracle_selective_scan_f64.argtypes = [
            _i64, _i64, _i64, _i64, _i64, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
            _f64p, ctypes.c_int, _i64p, _i64, _f64p, _f64p]
        L.oracle_ssd_f64.restype = ctypes.c_int
        L.oracle_ssd_f64.argtypes = [
            _i64, _i64, _i64, _i64, _i64, _i64, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
            _f32p, _f64p, ctypes.c_int, _i64p, _i64, _f64p, _f64p]
        L.oracle_selective_scan_bwd_f64.restype = ctypes.c_int
        L.oracle_selective_scan_bwd_f64.argtypes = [
            _i64, _i64, _i64, _i64, _i64, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
            _f64p, ctypes.c_int, _f32p, _f64p] + [_f64p] * 9
        L.oracle_causal_conv1d_f64.restype = ctypes.c_int
        L.oracle_causal_conv1d_f64.argtypes = [_i64, _i64, _i64, _i64, _f32p, _f32p, _f32p,
                                               _f32p, ctypes.c_int, _f64p, _f64p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


class using_library:
    """Context manager that points this module at another build of the oracle
    (the mutation tests load deliberately broken copies through it)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = None
        globals()["_LIB_OVERRIDE"] = self.path
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        globals()["_LIB_OVERRIDE"] = None
        return False


_LIB_OVERRIDE = None


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def _f64(a, shape=None):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("oracle input has shape %s, expected %s" % (arr.shape, tuple(shape)))
    return arr, arr.ctypes.data_as(_f64p)


def _f32(a, shape=None):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("oracle input has shape %s, expected %s" % (arr.shape, tuple(shape)))
    return arr, arr.ctypes.data_as(_f32p)


def selective_scan(x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None, h0=None,
                   delta_softplus: bool = True, channels: Optional[Sequence[int]] = None):
    """Reference selective scan in fp64.

    Shapes: x, delta, z (batch, L, D); Bm, Cm (batch, L, N), or (batch, L, G, N)
    for G groups (channel d reads group d // (D // G)); A (D, N);
    Dskip, delta_bias (D,); h0 (batch, D, N).
    Returns ``(y, h_final)``. With ``channels`` (ids ``b*D + d``) the outputs are
    ``y (len(channels), L)`` and ``h_final (len(channels), N)``; otherwise
    ``y (batch, L, D)`` and ``h_final (batch, D, N)``.
    """
    batch, L, D = np.shape(x)
    N = np.shape(A)[1]
    G = np.shape(Bm)[2] if np.ndim(Bm) == 4 else 1
    keep = []
    xs, xp = _f32(x, (batch, L, D)); keep.append(xs)
    ds, dp = _f32(delta, (batch, L, D)); keep.append(ds)
    zs, zp = _f32(z, (batch, L, D)); keep.append(zs)
    bs, bp = _f32(np.reshape(Bm, (batch, L, G, N)), (batch, L, G, N)); keep.append(bs)
    cs, cp = _f32(np.reshape(Cm, (batch, L, G, N)), (batch, L, G, N)); keep.append(cs)
    as_, ap = _f32(A, (D, N)); keep.append(as_)
    bis, bip = _f32(delta_bias, (D,)); keep.append(bis)
    dks, dkp = _f32(Dskip, (D,)); keep.append(dks)
    hs, hp = _f64(h0, (batch, D, N)); keep.append(hs)
    if channels is None:
        chp, nch = None, 0
        y = np.empty((batch, L, D), dtype=np.float64)
        hf = np.empty((batch, D, N), dtype=np.float64)
    else:
        ch = np.ascontiguousarray(channels, dtype=np.int64)
        keep.append(ch)
        chp, nch = ch.ctypes.data_as(_i64p), len(ch)
        y = np.empty((nch, L), dtype=np.float64)
        hf = np.empty((nch, N), dtype=np.float64)
    rc = lib().oracle_selective_scan_f64(batch, L, D, N, G, xp, dp, zp, bp, cp, ap, bip, dkp, hp,
                                         int(bool(delta_softplus)), chp, nch,
                                         y.ctypes.data_as(_f64p), hf.ctypes.data_as(_f64p))
    if rc != 0:
        raise ValueError("oracle_selective_scan_f64 rejected its arguments")
    return y, hf


def selective_scan_bwd(x, delta, A, Bm, Cm, dy, Dskip=None, z=None, delta_bias=None, h0=None,
                       dh_final=None, delta_softplus: bool = True) -> dict:
    """Gradients of the selective scan in fp64 (reverse-mode through the
    recurrence, see ``oracle_selective_scan_bwd_f64``) for the loss
    sum(dy * y) + sum(dh_final * h_final). Shapes as :func:`selective_scan`;
    dy (batch, L, D); dh_final (batch, D, N). Returns a dict with dx, ddelta, dz
    (None without z), dB, dC (the shape of Bm), dA, dDskip, ddelta_bias, dh0."""
    batch, L, D = np.shape(x)
    N = np.shape(A)[1]
    G = np.shape(Bm)[2] if np.ndim(Bm) == 4 else 1
    keep = []
    xs, xp = _f32(x, (batch, L, D)); keep.append(xs)
    ds, dp = _f32(delta, (batch, L, D)); keep.append(ds)
    zs, zp = _f32(z, (batch, L, D)); keep.append(zs)
    bs, bp = _f32(np.reshape(Bm, (batch, L, G, N)), (batch, L, G, N)); keep.append(bs)
    cs, cp = _f32(np.reshape(Cm, (batch, L, G, N)), (batch, L, G, N)); keep.append(cs)
    as_, ap = _f32(A, (D, N)); keep.append(as_)
    bis, bip = _f32(delta_bias, (D,)); keep.append(bis)
    dks, dkp = _f32(Dskip, (D,)); keep.append(dks)
    hs, hp = _f64(h0, (batch, D, N)); keep.append(hs)
    dys, dyp = _f32(dy, (batch, L, D)); keep.append(dys)
    dhs, dhp = _f64(dh_final, (batch, D, N)); keep.append(dhs)
    out = {"dx": np.empty((batch, L, D)), "ddelta": np.empty((batch, L, D)),
           "dz": np.empty((batch, L, D)) if z is not None else None,
           "dB": np.empty((batch, L, G, N)), "dC": np.empty((batch, L, G, N)),
           "dA": np.empty((D, N)), "dDskip": np.empty(D), "ddelta_bias": np.empty(D),
           "dh0": np.empty((batch, D, N))}
    ptr = lambda a: None if a is None else a.ctypes.data_as(_f64p)
    rc = lib().oracle_selective_scan_bwd_f64(
        batch, L, D, N, G, xp, dp, zp, bp, cp, ap, bip, dkp, hp, int(bool(delta_softplus)), dyp, dhp,
        ptr(out["dx"]), ptr(out["ddelta"]), ptr(out["dz"]), ptr(out["dB"]), ptr(out["dC"]),
        ptr(out["dA"]), ptr(out["dDskip"]), ptr(out["ddelta_bias"]), ptr(out["dh0"]))
    if rc != 0:
        raise ValueError("oracle_selective_scan_bwd_f64 rejected its arguments")
    if np.ndim(Bm) == 3:
        out["dB"] = out["dB"].reshape(batch, L, N)
        out["dC"] = out["dC"].reshape(batch, L, N)
    return out


def ssd(x, dt, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
        dt_softplus: bool = True, channels: Optional[Sequence[int]] = None):
    """Reference scalar-A (SSD) form in fp64, evaluated as the plain recurrence.

    Shapes: x, z (batch, L, H, P); dt (batch, L, H); A, Dskip, dt_bias (H,);
    Bm, Cm (batch, L, N), or (batch, L, G, N) for G groups (head h reads group
    h // (H // G)); h0 (batch, H, P, N). ``channels`` are ids
    ``(b*H + h)*P + p``; outputs as for :func:`selective_scan`.
    """
    batch, L, H, P = np.shape(x)
    G = np.shape(Bm)[2] if np.ndim(Bm) == 4 else 1
    N = np.shape(Bm)[-1]
    keep = []
    xs, xp = _f32(x, (batch, L, H, P)); keep.append(xs)
    ds, dp = _f32(dt, (batch, L, H)); keep.append(ds)
    bis, bip = _f32(dt_bias, (H,)); keep.append(bis)
    as_, ap = _f32(A, (H,)); keep.append(as_)
    bs, bp = _f32(np.reshape(Bm, (batch, L, G, N)), (batch, L, G, N)); keep.append(bs)
    cs, cp = _f32(np.reshape(Cm, (batch, L, G, N)), (batch, L, G, N)); keep.append(cs)
    dks, dkp = _f32(Dskip, (H,)); keep.append(dks)
    zs, zp = _f32(z, (batch, L, H, P)); keep.append(zs)
    hs, hp = _f64(h0, (batch, H, P, N)); keep.append(hs)
    if channels is None:
        chp, nch = None, 0
        y = np.empty((batch, L, H, P), dtype=np.float64)
        hf = np.empty((batch, H, P, N), dtype=np.float64)
    else:
        ch = np.ascontiguousarray(channels, dtype=np.int64)
        keep.append(ch)
        chp, nch = ch.ctypes.data_as(_i64p), len(ch)
        y = np.empty((nch, L), dtype=np.float64)
        hf = np.empty((nch, N), dtype=np.float64)
    rc = lib().oracle_ssd_f64(batch, L, H, P, N, G, xp, dp, bip, ap, bp, cp, dkp, zp, hp,
                              int(bool(dt_softplus)), chp, nch,
                              y.ctypes.data_as(_f64p), hf.ctypes.data_as(_f64p))
    if rc != 0:
        raise ValueError("oracle_ssd_f64 rejected its arguments")
    return y, hf


def ssd_bwd(x, dt, A, Bm, Cm, dy, Dskip=None, z=None, dt_bias=None, h0=None, dh_final=None,
            dt_softplus: bool = True, heads: Optional[Sequence[int]] = None) -> dict:
    """Gradients of the scalar-A (SSD) form in fp64 for the loss
    sum(dy * y) + sum(dh_final * h_final).

    The SSD form is the selective scan in which every channel p of head h shares
    the head's raw step dt[:, :, h], decay A[h] (the same for every state n), skip
    D[h] and bias [Mamba-2 page, key point 3: the decay becomes a scalar times the
    identity]. By the chain rule the gradient of a shared parameter is the sum of
    the gradients of its copies, so this runs :func:`selective_scan_bwd` on the
    broadcast inputs (channel d = h*P + p, the layout of x) and sums the copies:
    ddt over p, dA over (p, n), dDskip and ddt_bias over p.

    Shapes as :func:`ssd`; dy (batch, L, H, P); dh_final (batch, H, P, N).
    ``heads`` restricts the computation to a subset of heads: then dx, ddt, dz,
    dh0 and the per-head gradients are those of the listed heads (in that order)
    and dB, dC hold only the listed heads' share of the sum over heads.
    Returns dx, ddt (batch, L, H'), dA, dDskip, ddt_bias (H',), dB, dC (the shape
    of Bm), dz (None without z), dh0 (batch, H', P, N).
    """
    batch, L, H, P = np.shape(x)
    G = np.shape(Bm)[2] if np.ndim(Bm) == 4 else 1
    N = np.shape(Bm)[-1]
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    Hs = len(hs)
    take = lambda a, ax: None if a is None else np.take(np.asarray(a), hs, axis=ax)
    xs = take(x, 2).reshape(batch, L, Hs * P)
    ds = np.repeat(take(dt, 2), P, axis=2)
    As = np.repeat(take(A, 0), P)[:, None] * np.ones((1, N))
    bias = None if dt_bias is None else np.repeat(take(dt_bias, 0), P)
    Dk = None if Dskip is None else np.repeat(take(Dskip, 0), P)
    zs = None if z is None else take(z, 2).reshape(batch, L, Hs * P)
    h0s = None if h0 is None else take(h0, 1).reshape(batch, Hs * P, N)
    dhs = None if dh_final is None else take(dh_final, 1).reshape(batch, Hs * P, N)
    dys = take(dy, 2).reshape(batch, L, Hs * P)
    # channel d = i*P + p of the subset reads group hs[i] // (H/G): expand B, C so
    # that every selected head sees its own group (one group per head)
    Bg = np.reshape(Bm, (batch, L, G, N))[:, :, hs // (H // G)]
    Cg = np.reshape(Cm, (batch, L, G, N))[:, :, hs // (H // G)]
    o = selective_scan_bwd(xs, ds, As.astype(np.float32), Bg, Cg, dys, Dk, zs, bias, h0s, dhs, dt_softplus)
    # dB, dC per selected head, summed back onto their groups
    dB = np.zeros((batch, L, G, N))
    dC = np.zeros((batch, L, G, N))
    for i, h in enumerate(hs):
        dB[:, :, h // (H // G)] += o["dB"][:, :, i]
        dC[:, :, h // (H // G)] += o["dC"][:, :, i]
    shape_bc = np.shape(Bm)
    return {"dx": o["dx"].reshape(batch, L, Hs, P),
            "ddt": o["ddelta"].reshape(batch, L, Hs, P).sum(-1),
            "dA": o["dA"].reshape(Hs, P, N).sum((1, 2)),
            "dDskip": None if Dskip is None else o["dDskip"].reshape(Hs, P).sum(1),
            "ddt_bias": None if dt_bias is None else o["ddelta_bias"].reshape(Hs, P).sum(1),
            "dB": dB.reshape(shape_bc), "dC": dC.reshape(shape_bc),
            "dz": None if z is None else o["dz"].reshape(batch, L, Hs, P),
            "dh0": o["dh0"].reshape(batch, Hs, P, N)}


def causal_conv1d(x, w, bias=None, apply_silu: bool = True, x0=None, return_state: bool = False):
    """Reference causal depthwise conv1d (+ SiLU) in fp64. x (batch, L, D), w (D, K),
    bias (D,), x0 (batch, K-1, D) the inputs before t = 0 (zeros when None).
    Returns out (batch, L, D), and with ``return_state`` also the last K-1 inputs
    of [x0; x] as (batch, K-1, D)."""
    batch, L, D = np.shape(x)
    K = np.shape(w)[1]
    xs, xp = _f32(x, (batch, L, D))
    ws, wp = _f32(w, (D, K))
    bs, bp = _f32(bias, (D,))
    x0s, x0p = _f32(x0, (batch, K - 1, D))
    out = np.empty((batch, L, D), dtype=np.float64)
    fs = np.empty((batch, K - 1, D), dtype=np.float64)
    rc = lib().oracle_causal_conv1d_f64(batch, L, D, K, xp, wp, bp, x0p, int(bool(apply_silu)),
                                        out.ctypes.data_as(_f64p), fs.ctypes.data_as(_f64p))
    if rc != 0:
        raise ValueError("oracle_causal_conv1d_f64 rejected its arguments")
    del xs, ws, bs, x0s
    return (out, fs) if return_state else out


def selective_state_update(state, x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                           delta_softplus: bool = True):
    """One decode step of the selective scan: by definition the scan over a
    sequence of length 1 that starts from ``state`` [Juejin page, streaming
    step(x, state) -> (y, state)]. Shapes: state (batch, D, N); x, delta, z
    (batch, D); Bm, Cm (batch, N). Returns (y (batch, D), new_state (batch, D, N))."""
    col = lambda a: None if a is None else np.asarray(a)[:, None]
    y, hf = selective_scan(col(x), col(delta), A, col(Bm), col(Cm), Dskip, col(z), delta_bias,
                           state, delta_softplus)
    return y[:, 0], hf


def ssd_state_update(state, x, dt, A, Bm, Cm, Dskip=None, z=None, dt_bias=None,
                     dt_softplus: bool = True):
    """One decode step of the scalar-A (SSD) form: the recurrence over one step
    from ``state``. Shapes: state (batch, H, P, N); x, z (batch, H, P); dt (batch, H);
    Bm, Cm (batch, N). Returns (y (batch, H, P), new_state (batch, H, P, N))."""
    col = lambda a: None if a is None else np.asarray(a)[:, None]
    y, hf = ssd(col(x), col(dt), A, col(Bm), col(Cm), Dskip, col(z), dt_bias, state, dt_softplus)
    return y[:, 0], hf


def rel_l2(u, v) -> float:
    """||u - v||_2 / ||v||_2 over the whole tensor, in fp64 (v is the reference)."""
    u = np.asarray(u, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    den = np.linalg.norm(v.ravel())
    num = np.linalg.norm((u - v).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
