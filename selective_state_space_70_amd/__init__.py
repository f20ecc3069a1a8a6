"""MI355X (gfx950) selective state-space scan and scalar-A SSD form.

Thin binding over the C ABI of ``libssm.so`` (see ``include/ssm.h``): it checks
torch tensors, allocates outputs and workspace with torch, and passes raw
device pointers and torch's current HIP stream. Every arithmetic step runs in
the HIP kernels; there is no CPU or PyTorch fallback, and a missing library
raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _capi
from ._capi import SSMError

__all__ = ["selective_scan_fwd", "selective_scan_bwd", "ssd_chunked_fwd", "ssd_chunked_bwd", "selective_state_update", "ssd_state_update",
           "causal_conv1d_fwd", "scan_workspace_bytes", "ssd_workspace_bytes", "abi_version",
           "SSMError"]

_DT = {torch.float32: _capi.SSM_F32, torch.bfloat16: _capi.SSM_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _span(t: Optional[torch.Tensor]):
    if t is None or t.numel() == 0:
        return None
    start = t.data_ptr()
    return start, start + t.numel() * t.element_size()


def _no_overlap(outs, ins):
    """Raise if a written buffer shares memory with another written buffer or with an
    input. The kernels read their inputs while the outputs are being written, so
    aliasing gives wrong results, not an in-place update. ``outs`` and ``ins`` are
    (name, tensor or None) pairs; tensors are contiguous, so byte ranges are exact."""
    spans = [(n, _span(t)) for n, t in outs]
    others = [(n, _span(t)) for n, t in ins]
    for i, (n, s) in enumerate(spans):
        if s is None:
            continue
        for m, r in spans[i + 1:] + others:
            if r is not None and s[0] < r[1] and r[0] < s[1]:
                raise ValueError("%s shares memory with %s: outputs must not alias inputs or "
                                 "each other" % (n, m))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def abi_version() -> int:
    return _capi.lib().ssm_abi_version()


def _groups(Bm: torch.Tensor, plain_dims: int) -> int:
    """Number of B/C groups: Bm carries a group axis just before N when it has
    one more dimension than the single-group layout."""
    return Bm.shape[-2] if Bm.dim() == plain_dims + 1 else 1


def _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, delta_softplus, y, h_final):
    batch, L, D = x.shape
    N = A.shape[1]
    a = _capi.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, D, N
    a.ngroups = _groups(Bm, 3)
    a.dtype = _DT[x.dtype]
    a.delta_softplus = 1 if delta_softplus else 0
    a.x, a.delta, a.z = _ptr(x), _ptr(delta), _ptr(z)
    a.Bm, a.Cm, a.A = _ptr(Bm), _ptr(Cm), _ptr(A)
    a.delta_bias, a.Dskip, a.h0 = _ptr(delta_bias), _ptr(Dskip), _ptr(h0)
    a.y, a.h_final = _ptr(y), _ptr(h_final)
    return a


def scan_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int,
                         dtype=torch.bfloat16) -> int:
    a = _capi.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate, a.dtype = batch, seqlen, dim, dstate, _DT[dtype]
    return _capi.lib().selective_scan_workspace_bytes(ctypes.byref(a))


def selective_scan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                       h0: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                       return_final_state: bool = True, out: Optional[torch.Tensor] = None,
                       final_state_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, passes: str = "all"
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective scan. x, delta, z: (batch, L, D); Bm, Cm: (batch, L, N), or
    (batch, L, G, N) for G groups (channel d reads group d // (D // G)); all
    fp32 or all bf16; A: (D, N) fp32; Dskip, delta_bias: (D,) fp32;
    h0: (batch, D, N) fp32. Returns (y (batch, L, D) in x's dtype,
    h_final (batch, D, N) fp32 or None).

    ``passes`` selects the C entry point: "all" (selective_scan_fwd),
    "chunk_states" (selective_scan_chunk_states: fills ``workspace`` only),
    "apply" (selective_scan_apply: needs the ``workspace`` a "chunk_states" call
    with the same arguments filled) or "noalloc" (selective_scan_fwd_noalloc:
    the library's fixed scratch array instead of a workspace; ``out`` and, with
    ``return_final_state``, ``final_state_out`` must be given, so that nothing
    is allocated, here or in the library)."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    if x.dtype not in _DT:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device (got %s)" % dev)
    batch, L, D = x.shape
    N = A.shape[1]
    bc = (batch, L, N) if Bm.dim() == 3 else (batch, L, Bm.shape[2], N)
    _need(x, "x", (batch, L, D), x.dtype, dev)
    _need(delta, "delta", (batch, L, D), x.dtype, dev)
    _need(z, "z", (batch, L, D), x.dtype, dev)
    _need(Bm, "Bm", bc, x.dtype, dev)
    _need(Cm, "Cm", bc, x.dtype, dev)
    _need(A, "A", (D, N), torch.float32, dev)
    _need(Dskip, "Dskip", (D,), torch.float32, dev)
    _need(delta_bias, "delta_bias", (D,), torch.float32, dev)
    _need(h0, "h0", (batch, D, N), torch.float32, dev)
    if passes == "noalloc" and (out is None or (return_final_state and final_state_out is None)):
        raise ValueError("passes='noalloc' allocates nothing: pass out (and final_state_out)")
    y = out if out is not None else torch.empty((batch, L, D), dtype=x.dtype, device=dev)
    _need(y, "out", (batch, L, D), x.dtype, dev)
    hf = None
    if return_final_state:
        hf = (final_state_out if final_state_out is not None
              else torch.empty((batch, D, N), dtype=torch.float32, device=dev))
        _need(hf, "final_state_out", (batch, D, N), torch.float32, dev)
    a = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, delta_softplus, y, hf)
    L_ = _capi.lib()
    _capi.check(L_.selective_scan_validate(ctypes.byref(a)))
    need = L_.selective_scan_workspace_bytes(ctypes.byref(a))
    entry = {"all": L_.selective_scan_fwd, "chunk_states": L_.selective_scan_chunk_states,
             "apply": L_.selective_scan_apply, "noalloc": L_.selective_scan_fwd_noalloc}[passes]
    if passes == "noalloc":
        need = 0                      # the library's own scratch array
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            if passes == "apply":
                raise ValueError("passes='apply' needs the workspace filled by 'chunk_states'")
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    _no_overlap([("out", y), ("final_state_out", hf), ("workspace", workspace if need else None)],
                [("x", x), ("delta", delta), ("z", z), ("Bm", Bm), ("Cm", Cm), ("A", A),
                 ("Dskip", Dskip), ("delta_bias", delta_bias), ("h0", h0)])
    _capi.check(entry(ctypes.byref(a), _stream(dev)))
    return y, hf


def _ssd_args(x, dt, A, Bm, Cm, Dskip, z, dt_bias, h0, chunk, dt_softplus, y, h_final):
    batch, L, H, P = x.shape
    a = _capi.SSDArgs()
    a.batch, a.seqlen, a.nheads, a.headdim = batch, L, H, P
    a.dstate, a.chunk = Bm.shape[-1], chunk
    a.ngroups = _groups(Bm, 3)
    a.dtype = _DT[x.dtype]
    a.dt_softplus = 1 if dt_softplus else 0
    a.x, a.dt, a.dt_bias, a.A = _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A)
    a.Bm, a.Cm, a.Dskip, a.z, a.h0 = _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0)
    a.y, a.h_final = _ptr(y), _ptr(h_final)
    return a


def ssd_workspace_bytes(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                        chunk: int = 256) -> int:
    a = _capi.SSDArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.chunk = (batch, seqlen, nheads, headdim,
                                                                  dstate, chunk)
    a.dtype = _capi.SSM_BF16
    return _capi.lib().ssd_chunked_workspace_bytes(ctypes.byref(a))


def ssd_chunked_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                    Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                    z: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                    h0: Optional[torch.Tensor] = None, chunk: int = 256, dt_softplus: bool = True,
                    return_final_state: bool = True, out: Optional[torch.Tensor] = None,
                    final_state_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Scalar-A (SSD) form. x, z: (batch, L, H, P) bf16; dt: (batch, L, H) bf16;
    Bm, Cm: (batch, L, N) bf16, or (batch, L, G, N) for G groups (head h reads
    group h // (H // G)); A, Dskip, dt_bias: (H,) fp32; h0: (batch, H, P, N)
    fp32. Returns (y (batch, L, H, P) bf16, h_final (batch, H, P, N) fp32 or None)."""
    if x.dim() != 4 or Bm.dim() not in (3, 4):
        raise ValueError("x must be (batch, L, H, P) and Bm (batch, L, [G,] N)")
    if x.dtype not in _DT:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device (got %s)" % dev)
    batch, L, H, P = x.shape
    N = Bm.shape[-1]
    bc = (batch, L, N) if Bm.dim() == 3 else (batch, L, Bm.shape[2], N)
    _need(dt, "dt", (batch, L, H), x.dtype, dev)
    _need(z, "z", (batch, L, H, P), x.dtype, dev)
    _need(Bm, "Bm", bc, x.dtype, dev)
    _need(Cm, "Cm", bc, x.dtype, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(Dskip, "Dskip", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _need(h0, "h0", (batch, H, P, N), torch.float32, dev)
    _need(x, "x", (batch, L, H, P), x.dtype, dev)
    y = out if out is not None else torch.empty((batch, L, H, P), dtype=x.dtype, device=dev)
    _need(y, "out", (batch, L, H, P), x.dtype, dev)
    hf = None
    if return_final_state:
        hf = (final_state_out if final_state_out is not None
              else torch.empty((batch, H, P, N), dtype=torch.float32, device=dev))
        _need(hf, "final_state_out", (batch, H, P, N), torch.float32, dev)
    a = _ssd_args(x, dt, A, Bm, Cm, Dskip, z, dt_bias, h0, chunk, dt_softplus, y, hf)
    L_ = _capi.lib()
    _capi.check(L_.ssd_chunked_validate(ctypes.byref(a)))
    need = L_.ssd_chunked_workspace_bytes(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    _no_overlap([("out", y), ("final_state_out", hf), ("workspace", workspace if need else None)],
                [("x", x), ("dt", dt), ("z", z), ("Bm", Bm), ("Cm", Cm), ("A", A),
                 ("Dskip", Dskip), ("dt_bias", dt_bias), ("h0", h0)])
    _capi.check(L_.ssd_chunked_fwd(ctypes.byref(a), _stream(dev)))
    return y, hf


def _device_of(x: torch.Tensor):
    if x.dtype not in _DT:
        raise TypeError("inputs must be float32 or bfloat16")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device (got %s)" % x.device)
    return x.device


def selective_state_update(state: torch.Tensor, x: torch.Tensor, delta: torch.Tensor,
                           A: torch.Tensor, Bm: torch.Tensor, Cm: torch.Tensor,
                           Dskip: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                           delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step; ``state`` (batch, D, N) fp32 is updated in place.
    x, delta, z: (batch, D); Bm, Cm: (batch, N) or (batch, G, N), all in one dtype; A (D, N),
    Dskip, delta_bias (D,) fp32. Returns y (batch, D) in x's dtype."""
    dev = _device_of(x)
    if x.dim() != 2 or A.dim() != 2:
        raise ValueError("x must be (batch, D) and A (D, N)")
    batch, D = x.shape
    N = A.shape[1]
    bc = (batch, N) if Bm.dim() == 2 else (batch, Bm.shape[1], N)
    _need(x, "x", (batch, D), x.dtype, dev)
    _need(delta, "delta", (batch, D), x.dtype, dev)
    _need(z, "z", (batch, D), x.dtype, dev)
    _need(Bm, "Bm", bc, x.dtype, dev)
    _need(Cm, "Cm", bc, x.dtype, dev)
    _need(A, "A", (D, N), torch.float32, dev)
    _need(Dskip, "Dskip", (D,), torch.float32, dev)
    _need(delta_bias, "delta_bias", (D,), torch.float32, dev)
    _need(state, "state", (batch, D, N), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, D), dtype=x.dtype, device=dev)
    _need(y, "out", (batch, D), x.dtype, dev)
    a = _capi.ScanStepArgs()
    a.batch, a.dim, a.dstate, a.dtype = batch, D, N, _DT[x.dtype]
    a.ngroups = _groups(Bm, 2)
    a.delta_softplus = 1 if delta_softplus else 0
    a.x, a.delta, a.z, a.Bm, a.Cm = _ptr(x), _ptr(delta), _ptr(z), _ptr(Bm), _ptr(Cm)
    a.A, a.delta_bias, a.Dskip = _ptr(A), _ptr(delta_bias), _ptr(Dskip)
    a.state, a.y = _ptr(state), _ptr(y)
    _no_overlap([("out", y), ("state", state)],
                [("x", x), ("delta", delta), ("z", z), ("Bm", Bm), ("Cm", Cm), ("A", A),
                 ("Dskip", Dskip), ("delta_bias", delta_bias)])
    _capi.check(_capi.lib().selective_state_update(ctypes.byref(a), _stream(dev)))
    return y


def ssd_state_update(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                     Bm: torch.Tensor, Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                     z: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                     dt_softplus: bool = True, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step of the scalar-A form; ``state`` (batch, H, P, N) fp32 is
    updated in place. x, z: (batch, H, P); dt: (batch, H); Bm, Cm: (batch, N) or
    (batch, G, N);
    A, Dskip, dt_bias: (H,) fp32. Returns y (batch, H, P) in x's dtype."""
    dev = _device_of(x)
    if x.dim() != 3 or Bm.dim() not in (2, 3):
        raise ValueError("x must be (batch, H, P) and Bm (batch, [G,] N)")
    batch, H, P = x.shape
    N = Bm.shape[-1]
    bc = (batch, N) if Bm.dim() == 2 else (batch, Bm.shape[1], N)
    _need(x, "x", (batch, H, P), x.dtype, dev)
    _need(dt, "dt", (batch, H), x.dtype, dev)
    _need(z, "z", (batch, H, P), x.dtype, dev)
    _need(Bm, "Bm", bc, x.dtype, dev)
    _need(Cm, "Cm", bc, x.dtype, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(Dskip, "Dskip", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _need(state, "state", (batch, H, P, N), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, H, P), dtype=x.dtype, device=dev)
    _need(y, "out", (batch, H, P), x.dtype, dev)
    a = _capi.SSDStepArgs()
    a.batch, a.nheads, a.headdim, a.dstate, a.dtype = batch, H, P, N, _DT[x.dtype]
    a.ngroups = _groups(Bm, 2)
    a.dt_softplus = 1 if dt_softplus else 0
    a.x, a.dt, a.dt_bias, a.A = _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A)
    a.Bm, a.Cm, a.Dskip, a.z = _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z)
    a.state, a.y = _ptr(state), _ptr(y)
    _no_overlap([("out", y), ("state", state)],
                [("x", x), ("dt", dt), ("z", z), ("Bm", Bm), ("Cm", Cm), ("A", A),
                 ("Dskip", Dskip), ("dt_bias", dt_bias)])
    _capi.check(_capi.lib().ssd_state_update(ctypes.byref(a), _stream(dev)))
    return y


def causal_conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      init_state: Optional[torch.Tensor] = None, apply_silu: bool = True,
                      return_final_state: bool = False, out: Optional[torch.Tensor] = None,
                      final_state_out: Optional[torch.Tensor] = None):
    """Causal depthwise conv1d + bias (+ SiLU). x: (batch, L, D) fp32 or bf16;
    weight: (D, K) fp32; bias: (D,) fp32; init_state: (batch, K-1, D) in x's dtype.
    Returns y (batch, L, D), and with ``return_final_state`` also the
    (batch, K-1, D) state that continues the sequence."""
    dev = _device_of(x)
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be (batch, L, D) and weight (D, K)")
    batch, L, D = x.shape
    K = weight.shape[1]
    _need(x, "x", (batch, L, D), x.dtype, dev)
    _need(weight, "weight", (D, K), torch.float32, dev)
    _need(bias, "bias", (D,), torch.float32, dev)
    _need(init_state, "init_state", (batch, K - 1, D), x.dtype, dev)
    y = out if out is not None else torch.empty((batch, L, D), dtype=x.dtype, device=dev)
    _need(y, "out", (batch, L, D), x.dtype, dev)
    fs = None
    if return_final_state:
        fs = (final_state_out if final_state_out is not None
              else torch.empty((batch, K - 1, D), dtype=x.dtype, device=dev))
        _need(fs, "final_state_out", (batch, K - 1, D), x.dtype, dev)
    a = _capi.ConvArgs()
    a.batch, a.seqlen, a.dim, a.width, a.dtype = batch, L, D, K, _DT[x.dtype]
    a.apply_silu = 1 if apply_silu else 0
    a.x, a.weight, a.bias, a.init_state = _ptr(x), _ptr(weight), _ptr(bias), _ptr(init_state)
    a.y, a.final_state = _ptr(y), _ptr(fs)
    _no_overlap([("out", y), ("final_state_out", fs)],
                [("x", x), ("weight", weight), ("bias", bias), ("init_state", init_state)])
    _capi.check(_capi.lib().causal_conv1d_fwd(ctypes.byref(a), _stream(dev)))
    return (y, fs) if return_final_state else y


def selective_scan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, dy: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                       h0: Optional[torch.Tensor] = None, dh_final: Optional[torch.Tensor] = None,
                       delta_softplus: bool = True, workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of :func:`selective_scan_fwd` for the loss sum(dy * y) +
    sum(dh_final * h_final). Inputs as for the forward; dy (batch, L, D) in x's
    dtype; dh_final (batch, D, N) fp32 or None. Returns a dict: dx, ddelta, dz
    (x's dtype; dz None without z), dB, dC (fp32, Bm's shape), dA (fp32),
    dDskip / ddelta_bias (fp32, None when that input is None), dh0 (fp32, None
    without h0)."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, D) and A (D, N)")
    dev = _device_of(x)
    batch, L, D = x.shape
    N = A.shape[1]
    bc = (batch, L, N) if Bm.dim() == 3 else (batch, L, Bm.shape[2], N)
    for t, name, shape, dt in ((x, "x", (batch, L, D), x.dtype), (delta, "delta", (batch, L, D), x.dtype),
                               (z, "z", (batch, L, D), x.dtype), (Bm, "Bm", bc, x.dtype),
                               (Cm, "Cm", bc, x.dtype), (A, "A", (D, N), torch.float32),
                               (Dskip, "Dskip", (D,), torch.float32),
                               (delta_bias, "delta_bias", (D,), torch.float32),
                               (h0, "h0", (batch, D, N), torch.float32), (dy, "dy", (batch, L, D), x.dtype),
                               (dh_final, "dh_final", (batch, D, N), torch.float32)):
        _need(t, name, shape, dt, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
           "dz": torch.empty_like(x) if z is not None else None,
           "dB": torch.empty(bc, **f32), "dC": torch.empty(bc, **f32), "dA": torch.empty((D, N), **f32),
           "dDskip": torch.empty((D,), **f32) if Dskip is not None else None,
           "ddelta_bias": torch.empty((D,), **f32) if delta_bias is not None else None,
           "dh0": torch.empty((batch, D, N), **f32) if h0 is not None else None}
    a = _capi.ScanBwdArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, D, N
    a.ngroups = _groups(Bm, 3)
    a.dtype = _DT[x.dtype]
    a.delta_softplus = 1 if delta_softplus else 0
    a.x, a.delta, a.z, a.Bm, a.Cm = _ptr(x), _ptr(delta), _ptr(z), _ptr(Bm), _ptr(Cm)
    a.A, a.delta_bias, a.Dskip, a.h0 = _ptr(A), _ptr(delta_bias), _ptr(Dskip), _ptr(h0)
    a.dy, a.dh_final = _ptr(dy), _ptr(dh_final)
    for k in ("dx", "ddelta", "dz", "dB", "dC", "dA", "dDskip", "ddelta_bias", "dh0"):
        setattr(a, k, _ptr(out[k]))
    L_ = _capi.lib()
    need = L_.selective_scan_bwd_workspace_bytes(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    _capi.check(L_.selective_scan_bwd(ctypes.byref(a), _stream(dev)))
    return out


def ssd_chunked_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                    Cm: torch.Tensor, dy: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                    z: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                    h0: Optional[torch.Tensor] = None, dh_final: Optional[torch.Tensor] = None,
                    chunk: int = 256, dt_softplus: bool = True,
                    workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of :func:`ssd_chunked_fwd` for the loss sum(dy * y) +
    sum(dh_final * h_final). Inputs as for the forward; dy (batch, L, H, P) bf16;
    dh_final (batch, H, P, N) fp32 or None. Returns a dict: dx, ddt, dz (bf16; dz
    None without z), dB, dC (fp32, Bm's shape), dA (fp32, (H,)), dDskip / ddt_bias
    (fp32, None when that input is None), dh0 (fp32, None without h0)."""
    if x.dim() != 4 or Bm.dim() not in (3, 4):
        raise ValueError("x must be (batch, L, H, P) and Bm (batch, L, [G,] N)")
    dev = _device_of(x)
    batch, L, H, P = x.shape
    N = Bm.shape[-1]
    bc = (batch, L, N) if Bm.dim() == 3 else (batch, L, Bm.shape[2], N)
    for t, name, shape, dty in ((x, "x", (batch, L, H, P), x.dtype), (dt, "dt", (batch, L, H), x.dtype),
                                (z, "z", (batch, L, H, P), x.dtype), (Bm, "Bm", bc, x.dtype),
                                (Cm, "Cm", bc, x.dtype), (A, "A", (H,), torch.float32),
                                (Dskip, "Dskip", (H,), torch.float32), (dt_bias, "dt_bias", (H,), torch.float32),
                                (h0, "h0", (batch, H, P, N), torch.float32),
                                (dy, "dy", (batch, L, H, P), x.dtype),
                                (dh_final, "dh_final", (batch, H, P, N), torch.float32)):
        _need(t, name, shape, dty, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
           "dz": torch.empty_like(x) if z is not None else None,
           "dB": torch.empty(bc, **f32), "dC": torch.empty(bc, **f32), "dA": torch.empty((H,), **f32),
           "dDskip": torch.empty((H,), **f32) if Dskip is not None else None,
           "ddt_bias": torch.empty((H,), **f32) if dt_bias is not None else None,
           "dh0": torch.empty((batch, H, P, N), **f32) if h0 is not None else None}
    a = _capi.SSDBwdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.chunk = batch, L, H, P, N, chunk
    a.ngroups = _groups(Bm, 3)
    a.dtype = _DT[x.dtype]
    a.dt_softplus = 1 if dt_softplus else 0
    a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm = _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm)
    a.Dskip, a.z, a.h0, a.dy, a.dh_final = _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_final)
    for k in ("dx", "ddt", "dz", "dB", "dC", "dA", "dDskip", "ddt_bias", "dh0"):
        setattr(a, k, _ptr(out[k]))
    L_ = _capi.lib()
    need = L_.ssd_chunked_bwd_workspace_bytes(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    _capi.check(L_.ssd_chunked_bwd(ctypes.byref(a), _stream(dev)))
    return out
