"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function builds a small input, evaluates the oracle, and checks
the result against something fixed independently of the recurrence code:
a closed form, a library routine that uses a different algorithm, an
invariant of the mathematics, or a special case. They raise AssertionError on
failure. ``tests/test_oracle.py`` runs them against the oracle; the mutation
test runs them against copies of the oracle with planted mistakes and
requires every mutant to fail at least one of them.

Sources of the facts (page titles as published):
  * LTI convolution view: with time-invariant parameters the recurrence is a
    convolution with kernel K_k = C Abar^k Bbar ["Mamba-2：把状态空间模型和
    Attention 统一到一个数学框架里", Background; juejin SSM article, "基本原理"].
  * Semiseparable / matrix view: y = (L o M) x with M[t,s] = C_t Abar_t ...
    Abar_{s+1} Bbar_s for t >= s [same Mamba-2 page, Core idea step 2].
  * Small step keeps the state, large step overwrites it [same page, step 1].
  * The state is the only carrier between calls (streaming step(x, state))
    [juejin SSM article, long-document encoder].
"""
from __future__ import annotations

import math

import numpy as np
import scipy.signal

import oracle

TOL = 1e-12


def _rel(u, v):
    return oracle.rel_l2(u, v)


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _silu_tanh(z):
    # sigma(z) = (1 + tanh(z/2)) / 2: a different route to the logistic function
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def _softplus_np(v):
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


def _rand_case(rng, batch, L, D, N, time_varying=True):
    x = _f32(rng.standard_normal((batch, L, D)))
    z = _f32(rng.standard_normal((batch, L, D)))
    Dsk = _f32(rng.standard_normal(D))
    A = _f32(-rng.uniform(0.3, 3.0, size=(D, N)))
    if time_varying:
        dt = _f32(rng.uniform(0.02, 0.4, size=(batch, L, D)))
        Bm = _f32(rng.standard_normal((batch, L, N)))
        Cm = _f32(rng.standard_normal((batch, L, N)))
    else:
        dt = _f32(np.broadcast_to(rng.uniform(0.02, 0.4, size=D), (batch, L, D)))
        Bm = _f32(np.broadcast_to(rng.standard_normal(N), (batch, L, N)))
        Cm = _f32(np.broadcast_to(rng.standard_normal(N), (batch, L, N)))
    return x, z, Dsk, A, dt, Bm, Cm


def pin_lti_convolution(seed=1):
    """Time-invariant dt, B, C and h0 = 0: y = K * x + D x, K_k = sum_n C_n e^{k dt A_n} dt B_n."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 48, 3, 5
    x, z, Dsk, A, dt, Bm, Cm = _rand_case(rng, batch, L, D, N, time_varying=False)
    y, _ = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, delta_softplus=False)
    k = np.arange(L, dtype=np.float64)
    B64, C64 = Bm[0, 0].astype(np.float64), Cm[0, 0].astype(np.float64)
    want = np.empty_like(y)
    for d in range(D):
        dtd = float(dt[0, 0, d])
        K = (C64[None, :] * np.exp(k[:, None] * dtd * A[d].astype(np.float64)[None, :])
             * dtd * B64[None, :]).sum(axis=1)
        for b in range(batch):
            xs = x[b, :, d].astype(np.float64)
            conv = np.convolve(xs, K)[:L]
            want[b, :, d] = (conv + float(Dsk[d]) * xs) * _silu_tanh(z[b, :, d])
    err = _rel(y, want)
    assert err < TOL, "LTI convolution form differs: rel %.3g" % err


def pin_lti_lfilter(seed=2):
    """Same LTI case via scipy.signal.lfilter per state (first-order IIR), softplus on."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 40, 2, 4
    x, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N, time_varying=False)
    v = _f32(rng.uniform(-4.0, 1.0, size=D))
    bias = _f32(rng.uniform(-1.0, 1.0, size=D))
    delta = _f32(np.broadcast_to(v, (batch, L, D)))
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, Dskip=Dsk, z=z, delta_bias=bias)
    dtv = _softplus_np(v.astype(np.float64) + bias.astype(np.float64))
    want = np.zeros_like(y)
    want_h = np.zeros_like(hf)
    for b in range(batch):
        for d in range(D):
            xs = x[b, :, d].astype(np.float64)
            acc = np.zeros(L)
            for n in range(N):
                a = math.exp(dtv[d] * float(A[d, n]))
                hs = scipy.signal.lfilter([dtv[d] * float(Bm[0, 0, n])], [1.0, -a], xs)
                acc += float(Cm[0, 0, n]) * hs
                want_h[b, d, n] = hs[-1]
            want[b, :, d] = (acc + float(Dsk[d]) * xs) * _silu_tanh(z[b, :, d])
    err = max(_rel(y, want), _rel(hf, want_h))
    assert err < 1e-11, "lfilter form differs: rel %.3g" % err


def pin_semiseparable(seed=3):
    """Time-varying case, L small: y = (M + diag D) x with the materialised
    semiseparable matrix M[t,s] = sum_n C_t[n] exp(A_n (cs_t - cs_s)) dt_s B_s[n],
    plus the initial-state term C_t . (exp(A cs_t) o h0)."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 24, 3, 6
    x, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    bias = _f32(rng.uniform(-3.0, -1.0, size=D))
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, Dskip=Dsk, z=z, delta_bias=bias, h0=h0)
    want = np.empty_like(y)
    want_h = np.empty_like(hf)
    for b in range(batch):
        for d in range(D):
            dt = _softplus_np(delta[b, :, d].astype(np.float64) + float(bias[d]))
            cs = np.cumsum(dt)
            An = A[d].astype(np.float64)
            Bb, Cb = Bm[b].astype(np.float64), Cm[b].astype(np.float64)
            seg = cs[:, None] - cs[None, :]                              # (t, s)
            decay = np.exp(seg[:, :, None] * An[None, None, :])          # (t, s, n)
            M = np.einsum("tn,tsn,s,sn->ts", Cb, decay, dt, Bb)
            M = np.tril(M)
            xs = x[b, :, d].astype(np.float64)
            init = (Cb * np.exp(cs[:, None] * An[None, :]) * h0[b, d][None, :]).sum(axis=1)
            want[b, :, d] = (M @ xs + init + float(Dsk[d]) * xs) * _silu_tanh(z[b, :, d])
            dec_end = np.exp((cs[-1] - cs)[:, None] * An[None, :])       # (s, n)
            want_h[b, d] = (dec_end * (dt * xs)[:, None] * Bb).sum(axis=0) \
                + np.exp(cs[-1] * An) * h0[b, d]
    err = max(_rel(y, want), _rel(hf, want_h))
    assert err < TOL, "semiseparable form differs: rel %.3g" % err


def pin_small_step_keeps_state(seed=4):
    """delta + bias = -60 gives dt ~ 8.8e-27: the state is held and the output
    reads it: h_final = h0, y_t = (C_t . h0 + D x_t) silu(z_t)."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 16, 3, 4
    x, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    delta = _f32(np.full((batch, L, D), -60.0))
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, Dskip=Dsk, z=z, h0=h0)
    want = (np.einsum("btn,bdn->btd", Cm.astype(np.float64), h0)
            + Dsk[None, None, :].astype(np.float64) * x) * _silu_tanh(z)
    err = max(_rel(hf, h0), _rel(y, want))
    assert err < TOL, "small-step limit differs: rel %.3g" % err


def pin_large_step_forgets(seed=5):
    """A large step overwrites the state: with dt = 40 and A <= -1 the old
    state is scaled by <= e^{-40}, so h_L = dt_L B_L x_L to fp64 precision."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 1, 6, 2, 3
    x, z, Dsk, _, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    A = _f32(-rng.uniform(1.0, 2.0, size=(D, N)))
    delta = _f32(np.full((batch, L, D), 40.0))
    h0 = rng.standard_normal((batch, D, N)) * 1e3
    _, hf = oracle.selective_scan(x, delta, A, Bm, Cm, h0=h0, delta_softplus=False)
    want = 40.0 * Bm[:, -1, None, :].astype(np.float64) * x[:, -1, :, None].astype(np.float64)
    err = _rel(hf, want)
    assert err < 1e-12, "large-step limit differs: rel %.3g" % err


def pin_zero_input_pure_decay(seed=6):
    """x = 0: h_final = exp(A * sum_t dt_t) o h0 and y_t = C_t . (exp(A cs_t) o h0) silu(z_t):
    the product of per-step decays equals the exponential of the summed steps."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 30, 3, 5
    _, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    x = np.zeros((batch, L, D), dtype=np.float32)
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    bias = _f32(rng.uniform(-3.0, 0.0, size=D))
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, Dskip=Dsk, z=z, delta_bias=bias, h0=h0)
    dt = _softplus_np(delta.astype(np.float64) + bias.astype(np.float64)[None, None, :])
    cs = np.cumsum(dt, axis=1)                                           # (b, t, d)
    hs = np.exp(cs[..., None] * A.astype(np.float64)[None, None]) * h0[:, None]  # (b,t,d,n)
    want_y = np.einsum("btn,btdn->btd", Cm.astype(np.float64), hs) * _silu_tanh(z)
    err = max(_rel(hf, hs[:, -1]), _rel(y, want_y))
    assert err < TOL, "pure-decay closed form differs: rel %.3g" % err


def pin_split_invariance(seed=7):
    """Handing the final state of x[0:L1] to a second call on x[L1:L] gives the
    same output and state as one call on x[0:L]; so do L calls of length 1."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 33, 3, 4
    x, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    bias = _f32(rng.uniform(-3.0, 0.0, size=D))
    h0 = rng.standard_normal((batch, D, N))
    args = dict(Dskip=Dsk, delta_bias=bias)
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, z=z, h0=h0, **args)
    worst = 0.0
    for L1 in (1, 7, 16, 32):
        y1, h1 = oracle.selective_scan(x[:, :L1], delta[:, :L1], A, Bm[:, :L1], Cm[:, :L1],
                                       z=z[:, :L1], h0=h0, **args)
        y2, h2 = oracle.selective_scan(x[:, L1:], delta[:, L1:], A, Bm[:, L1:], Cm[:, L1:],
                                       z=z[:, L1:], h0=h1, **args)
        worst = max(worst, _rel(np.concatenate([y1, y2], axis=1), y), _rel(h2, hf))
    h = h0
    ys = []
    for t in range(L):
        yt, h = oracle.selective_scan(x[:, t:t + 1], delta[:, t:t + 1], A, Bm[:, t:t + 1],
                                      Cm[:, t:t + 1], z=z[:, t:t + 1], h0=h, **args)
        ys.append(yt)
    worst = max(worst, _rel(np.concatenate(ys, axis=1), y), _rel(h, hf))
    assert worst < TOL, "split invariance broken: rel %.3g" % worst


def pin_linearity(seed=8):
    """dt, B, C, z fixed: the map (x, h0) -> (y, h_final) is linear.
    Inputs are small dyadic numbers so that 2 x1 + x2 is exact in float32."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 20, 3, 4
    _, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    x1 = _f32(rng.integers(-16, 17, size=(batch, L, D)) / 8.0)
    x2 = _f32(rng.integers(-16, 17, size=(batch, L, D)) / 8.0)
    g1 = rng.standard_normal((batch, D, N))
    g2 = rng.standard_normal((batch, D, N))
    common = dict(Dskip=Dsk, z=z)
    ya, ha = oracle.selective_scan(x1, delta, A, Bm, Cm, h0=g1, **common)
    yb, hb = oracle.selective_scan(x2, delta, A, Bm, Cm, h0=g2, **common)
    yc, hc = oracle.selective_scan(_f32(2.0 * x1 + x2), delta, A, Bm, Cm, h0=2.0 * g1 + g2,
                                   **common)
    err = max(_rel(yc, 2.0 * ya + yb), _rel(hc, 2.0 * ha + hb))
    assert err < TOL, "linearity broken: rel %.3g" % err


def pin_geometric_series():
    """N = D = 1, constant a = e^{dt A}, b = dt B x with x = 1:
    h_t = b (1 - a^{t+1}) / (1 - a)  (finite geometric series)."""
    L = 50
    dt, Av, Bv, Cv = 0.25, -2.0, 1.5, 0.75
    x = np.ones((1, L, 1), dtype=np.float32)
    delta = np.full((1, L, 1), dt, dtype=np.float32)
    y, hf = oracle.selective_scan(x, delta, np.array([[Av]], np.float32),
                                  np.full((1, L, 1), Bv, np.float32),
                                  np.full((1, L, 1), Cv, np.float32), delta_softplus=False)
    a = math.exp(dt * Av)
    b = dt * Bv
    t = np.arange(L)
    h = b * (1.0 - a ** (t + 1)) / (1.0 - a)
    err = max(_rel(y[0, :, 0], Cv * h), _rel(hf[0, 0], h[-1:]))
    assert err < TOL, "geometric series differs: rel %.3g" % err


def pin_softplus_identities():
    """dt read out through a one-step scan (N=1, A=0, B=C=x=1, h0=0: y = dt):
    softplus(v) - softplus(-v) = v, softplus(0) = ln 2, softplus(ln(e^k - 1)) = k,
    and softplus(v) = e^v (1 - e^v/2 + ...) for very negative v."""
    v = np.array([-30.0, -12.0, -5.5, -1.0, -0.25, 0.0, 0.25, 1.0, 5.5, 12.0, 30.0])
    vals = np.concatenate([v, -v, [math.log(math.expm1(0.5)), math.log(math.expm1(3.0))]])
    n = len(vals)
    delta = vals.astype(np.float32).reshape(1, 1, n)
    vals32 = delta.reshape(-1).astype(np.float64)
    one = np.ones((1, 1, 1), np.float32)
    y, _ = oracle.selective_scan(np.ones((1, 1, n), np.float32), delta,
                                 np.zeros((n, 1), np.float32), one, one)
    sp = y.reshape(-1)
    m = len(v)
    diff = sp[:m] - sp[m:2 * m]
    assert np.allclose(diff, vals32[:m], rtol=1e-14, atol=1e-300), "softplus odd-part identity"
    assert abs(sp[list(v).index(0.0)] - math.log(2.0)) < 1e-15, "softplus(0) != ln 2"
    # the float32 rounding of ln(e^k - 1) moves k by ~1e-8 relative
    assert abs(sp[2 * m] - 0.5) < 1e-7 and abs(sp[2 * m + 1] - 3.0) < 1e-6
    e = math.exp(vals32[0])
    assert abs(sp[0] - (e - e * e / 2.0)) <= 1e-15 * e, "softplus small-v asymptote"


def pin_gate_identity(seed=9):
    """silu(z) - silu(-z) = z: out(z) - out(-z) = (C.h + D x) z, and silu(0) = 0."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 1, 12, 3, 4
    x, z, Dsk, A, dt, Bm, Cm = _rand_case(rng, batch, L, D, N)
    z[0, 0, 0] = 0.0
    yp, _ = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, delta_softplus=False)
    ym, _ = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=-z, delta_softplus=False)
    yu, _ = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, delta_softplus=False)
    err = _rel(yp - ym, yu * z)
    assert err < TOL, "gate identity broken: rel %.3g" % err
    assert yp[0, 0, 0] == 0.0


def pin_skip_only(seed=10):
    """B = 0 removes the state path: y = D x silu(z), h_final = decayed h0 = 0."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 9, 3, 4
    x, z, Dsk, A, dt, _, Cm = _rand_case(rng, batch, L, D, N)
    Bm = np.zeros((batch, L, N), np.float32)
    y, hf = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, delta_softplus=False)
    want = Dsk[None, None, :].astype(np.float64) * x * _silu_tanh(z)
    assert _rel(y, want) < TOL and np.all(hf == 0.0), "skip path differs"


def pin_channel_subset(seed=11):
    """Evaluating a subset of channels gives those channels of the full result."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 3, 17, 5, 4
    x, z, Dsk, A, dt, Bm, Cm = _rand_case(rng, batch, L, D, N)
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, h0=h0)
    ch = [0, 7, 14, 3, 11]
    ys, hs = oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, h0=h0, channels=ch)
    yfull = y.transpose(0, 2, 1).reshape(batch * D, L)[ch]
    hfull = hf.reshape(batch * D, N)[ch]
    assert np.array_equal(ys, yfull) and np.array_equal(hs, hfull), "channel subset differs"


# ----------------------------------------------------------------------------- SSD form

def _ssd_case(rng, batch, L, H, P, N):
    x = _f32(rng.standard_normal((batch, L, H, P)))
    dt = _f32(rng.normal(0.0, 0.5, size=(batch, L, H)))
    bias = _f32(rng.uniform(-3.0, -1.0, size=H))
    A = _f32(-rng.uniform(1.0, 16.0, size=H))
    Bm = _f32(rng.standard_normal((batch, L, N)))
    Cm = _f32(rng.standard_normal((batch, L, N)))
    Dsk = _f32(rng.standard_normal(H))
    z = _f32(rng.standard_normal((batch, L, H, P)))
    h0 = rng.standard_normal((batch, H, P, N))
    return x, dt, bias, A, Bm, Cm, Dsk, z, h0


def pin_ssd_semiseparable(seed=12):
    """Scalar A per head: M_h = (C B^T) o exp(A_h (cs_t - cs_s)) o dt_s (t >= s);
    y = M_h x_{h,p} + exp(A_h cs_t) C_t . h0 + D_h x, then the gate."""
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 20, 3, 4, 5
    x, dt, bias, A, Bm, Cm, Dsk, z, h0 = _ssd_case(rng, batch, L, H, P, N)
    y, hf = oracle.ssd(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, dt_bias=bias, h0=h0)
    want = np.empty_like(y)
    want_h = np.empty_like(hf)
    for b in range(batch):
        G = Cm[b].astype(np.float64) @ Bm[b].astype(np.float64).T          # (t, s)
        for h in range(H):
            d = _softplus_np(dt[b, :, h].astype(np.float64) + float(bias[h]))
            cs = np.cumsum(d) * float(A[h])
            M = np.tril(G * np.exp(cs[:, None] - np.where(
                np.tri(L, dtype=bool), cs[None, :], cs[:, None])) * d[None, :])
            xs = x[b, :, h, :].astype(np.float64)                           # (t, p)
            init = np.exp(cs)[:, None] * (Cm[b].astype(np.float64) @ h0[b, h].T)
            want[b, :, h, :] = (M @ xs + init + float(Dsk[h]) * xs) * _silu_tanh(z[b, :, h, :])
            wend = np.exp(cs[-1] - cs) * d                                  # (s,)
            want_h[b, h] = (xs * wend[:, None]).T @ Bm[b].astype(np.float64) \
                + math.exp(cs[-1]) * h0[b, h]
    err = max(_rel(y, want), _rel(hf, want_h))
    assert err < TOL, "SSD semiseparable form differs: rel %.3g" % err


def pin_ssd_is_broadcast_scan(seed=13):
    """The scalar-A form is the Mamba-1 scan with dt, bias, A, D broadcast over
    the P channels of a head and A constant over n."""
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 15, 3, 2, 4
    x, dt, bias, A, Bm, Cm, Dsk, z, h0 = _ssd_case(rng, batch, L, H, P, N)
    y, hf = oracle.ssd(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, dt_bias=bias, h0=h0)
    D = H * P
    ys, hs = oracle.selective_scan(
        x.reshape(batch, L, D), np.repeat(dt, P, axis=2), np.repeat(A, P)[:, None].repeat(N, 1),
        Bm, Cm, Dskip=np.repeat(Dsk, P), z=z.reshape(batch, L, D),
        delta_bias=np.repeat(bias, P), h0=h0.reshape(batch, D, N))
    err = max(_rel(y.reshape(batch, L, D), ys), _rel(hf.reshape(batch, D, N), hs))
    assert err < 1e-14, "SSD differs from the broadcast scan: rel %.3g" % err


def pin_ssd_channel_subset(seed=14):
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 11, 3, 4, 5
    x, dt, bias, A, Bm, Cm, Dsk, z, h0 = _ssd_case(rng, batch, L, H, P, N)
    y, hf = oracle.ssd(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, dt_bias=bias, h0=h0)
    ch = [0, 5, 23, 17, 9]
    ys, hs = oracle.ssd(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, dt_bias=bias, h0=h0, channels=ch)
    assert np.array_equal(ys, y.transpose(0, 2, 3, 1).reshape(-1, L)[ch])
    assert np.array_equal(hs, hf.reshape(-1, N)[ch])


# ----------------------------------------------------------------------------- conv1d

def pin_conv1d_numpy(seed=15):
    """Causal depthwise conv1d: equals numpy's full convolution truncated to the
    first L outputs (zero history), then SiLU."""
    rng = np.random.default_rng(seed)
    batch, L, D, K = 2, 19, 3, 4
    x = _f32(rng.standard_normal((batch, L, D)))
    w = _f32(rng.standard_normal((D, K)))
    bias = _f32(rng.standard_normal(D))
    out = oracle.causal_conv1d(x, w, bias)
    raw = oracle.causal_conv1d(x, w, bias, apply_silu=False)
    want = np.empty_like(out)
    for b in range(batch):
        for d in range(D):
            # weight index k multiplies x[t - (K-1) + k]: reverse it for np.convolve
            c = np.convolve(x[b, :, d].astype(np.float64), w[d, ::-1].astype(np.float64))[:L]
            want[b, :, d] = c + float(bias[d])
    assert _rel(raw, want) < TOL and _rel(out, _silu_tanh(want)) < TOL, "conv1d differs"


def pin_conv1d_history(seed=16):
    """With a history x0 the output is numpy's convolution of [x0; x] with the
    first K-1 outputs dropped; the returned state is the last K-1 inputs."""
    rng = np.random.default_rng(seed)
    for batch, L, D, K in ((2, 9, 3, 4), (1, 2, 2, 4), (2, 5, 2, 3)):
        x = _f32(rng.standard_normal((batch, L, D)))
        x0 = _f32(rng.standard_normal((batch, K - 1, D)))
        w = _f32(rng.standard_normal((D, K)))
        bias = _f32(rng.standard_normal(D))
        out, fs = oracle.causal_conv1d(x, w, bias, x0=x0, return_state=True)
        want = np.empty_like(out)
        for b in range(batch):
            for d in range(D):
                xx = np.concatenate([x0[b, :, d], x[b, :, d]]).astype(np.float64)
                c = np.convolve(xx, w[d, ::-1].astype(np.float64))[K - 1:K - 1 + L]
                want[b, :, d] = _silu_tanh(c + float(bias[d]))
        xx_all = np.concatenate([x0, x], axis=1).astype(np.float64)
        assert _rel(out, want) < TOL, "conv1d with history differs"
        assert np.array_equal(fs, xx_all[:, -(K - 1):]), "conv1d final state is not the last inputs"


def pin_conv1d_streaming(seed=17):
    """Two calls chained through the state equal one call over the whole sequence."""
    rng = np.random.default_rng(seed)
    batch, L, D, K = 2, 23, 3, 4
    x = _f32(rng.standard_normal((batch, L, D)))
    w = _f32(rng.standard_normal((D, K)))
    bias = _f32(rng.standard_normal(D))
    full, fs_full = oracle.causal_conv1d(x, w, bias, return_state=True)
    for cut in (1, 2, 11):
        a, st = oracle.causal_conv1d(x[:, :cut], w, bias, return_state=True)
        b, st2 = oracle.causal_conv1d(x[:, cut:], w, bias, x0=_f32(st), return_state=True)
        assert _rel(np.concatenate([a, b], axis=1), full) < 1e-15, "conv1d streaming differs"
        assert np.array_equal(st2, fs_full)


def pin_decode_steps_equal_scan(seed=18):
    """Decode steps chained through the state reproduce the scan over the same
    tokens: outputs per step and the final state (the recurrence is a semigroup)."""
    rng = np.random.default_rng(seed)
    batch, L, D, N = 2, 6, 3, 4
    x, z, Dsk, A, _, Bm, Cm = _rand_case(rng, batch, L, D, N)
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    bias = _f32(rng.uniform(-3.0, -1.0, size=D))
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, delta, A, Bm, Cm, Dsk, z, bias, h0)
    st = h0
    for t in range(L):
        yt, st = oracle.selective_state_update(st, x[:, t], delta[:, t], A, Bm[:, t], Cm[:, t],
                                               Dsk, z[:, t], bias)
        assert _rel(yt, y[:, t]) < TOL, "decode step %d differs from the scan" % t
    assert _rel(st, hf) < TOL, "decode state differs from the scan's final state"


def pin_ssd_decode_steps_equal_ssd(seed=19):
    rng = np.random.default_rng(seed)
    batch, L, H, P, N = 2, 5, 3, 2, 4
    x, dt, bias, A, Bm, Cm, Dsk, z, h0 = _ssd_case(rng, batch, L, H, P, N)
    y, hf = oracle.ssd(x, dt, A, Bm, Cm, Dskip=Dsk, z=z, dt_bias=bias, h0=h0)
    st = h0
    for t in range(L):
        yt, st = oracle.ssd_state_update(st, x[:, t], dt[:, t], A, Bm[:, t], Cm[:, t], Dskip=Dsk,
                                         z=z[:, t], dt_bias=bias)
        assert _rel(yt, y[:, t]) < TOL, "SSD decode step %d differs" % t
    assert _rel(st, hf) < TOL


def pin_groups_split(seed=20):
    """With G groups of B, C, the scan equals G separate single-group scans, one
    per contiguous block of D / G channels with that group's B and C."""
    rng = np.random.default_rng(seed)
    batch, L, D, N, G = 2, 7, 6, 3, 3
    x, z, Dsk, A, dt, _, _ = _rand_case(rng, batch, L, D, N)
    Bg = _f32(rng.standard_normal((batch, L, G, N)))
    Cg = _f32(rng.standard_normal((batch, L, G, N)))
    h0 = rng.standard_normal((batch, D, N))
    y, hf = oracle.selective_scan(x, dt, A, Bg, Cg, Dsk, z, None, h0, delta_softplus=False)
    k = D // G
    for g in range(G):
        sl = slice(g * k, (g + 1) * k)
        yg, hg = oracle.selective_scan(x[:, :, sl], dt[:, :, sl], A[sl], Bg[:, :, g], Cg[:, :, g],
                                       Dsk[sl], z[:, :, sl], None, h0[:, sl], delta_softplus=False)
        assert np.array_equal(y[:, :, sl], yg) and np.array_equal(hf[:, sl], hg), "group %d" % g


def pin_ssd_groups_split(seed=21):
    rng = np.random.default_rng(seed)
    batch, L, H, P, N, G = 2, 6, 4, 2, 3, 2
    x, dt, bias, A, _, _, Dsk, z, h0 = _ssd_case(rng, batch, L, H, P, N)
    Bg = _f32(rng.standard_normal((batch, L, G, N)))
    Cg = _f32(rng.standard_normal((batch, L, G, N)))
    y, hf = oracle.ssd(x, dt, A, Bg, Cg, Dskip=Dsk, z=z, dt_bias=bias, h0=h0)
    k = H // G
    for g in range(G):
        sl = slice(g * k, (g + 1) * k)
        yg, hg = oracle.ssd(x[:, :, sl], dt[:, :, sl], A[sl], Bg[:, :, g], Cg[:, :, g], Dskip=Dsk[sl],
                            z=z[:, :, sl], dt_bias=bias[sl], h0=h0[:, sl])
        assert np.array_equal(y[:, :, sl], yg) and np.array_equal(hf[:, sl], hg), "SSD group %d" % g


# ----------------------------------------------------------------------------- gradients

def _bwd_case(rng, batch, L, D, N, G):
    x = _f32(rng.standard_normal((batch, L, D)))
    z = _f32(rng.standard_normal((batch, L, D)))
    delta = _f32(rng.normal(0.0, 0.5, size=(batch, L, D)))
    bias = _f32(rng.uniform(-3.0, -1.0, size=D))
    A = _f32(-rng.uniform(0.3, 3.0, size=(D, N)))
    Bm = _f32(rng.standard_normal((batch, L, G, N)))
    Cm = _f32(rng.standard_normal((batch, L, G, N)))
    Dsk = _f32(rng.standard_normal(D))
    h0 = rng.standard_normal((batch, D, N))
    dy = _f32(rng.standard_normal((batch, L, D)))
    dhf = rng.standard_normal((batch, D, N))
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dsk, z=z, delta_bias=bias, h0=h0,
                dy=dy, dh_final=dhf)


def _loss(c, softplus=True):
    y, hf = oracle.selective_scan(c["x"], c["delta"], c["A"], c["Bm"], c["Cm"], c["Dskip"], c["z"],
                                  c["delta_bias"], c["h0"], delta_softplus=softplus)
    return float(np.sum(y * c["dy"].astype(np.float64)) + np.sum(hf * c["dh_final"]))


def pin_bwd_finite_differences(seed=22):
    """Every gradient of the backward oracle equals the central difference of the
    forward oracle's loss sum(dy*y) + sum(dh_final*h_final). Steps of 2^-10 are
    exact in the fp32 inputs; the truncation error is O(h^2)."""
    rng = np.random.default_rng(seed)
    for softplus, G in ((True, 2), (False, 1)):
        c = _bwd_case(rng, 2, 5, 4, 3, G)
        if not softplus:
            c["delta"] = np.abs(c["delta"]) + _f32(0.05)
            c["delta_bias"] = _f32(np.zeros(4))
        gr = oracle.selective_scan_bwd(c["x"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], c["Dskip"],
                                       c["z"], c["delta_bias"], c["h0"], c["dh_final"], softplus)
        names = {"x": "dx", "delta": "ddelta", "z": "dz", "Bm": "dB", "Cm": "dC", "A": "dA",
                 "Dskip": "dDskip", "delta_bias": "ddelta_bias", "h0": "dh0"}
        for key, gname in names.items():
            base = c[key]
            step = 2.0 ** -10 if base.dtype == np.float32 else 1e-6
            fd = np.empty(base.shape)
            for idx in np.ndindex(base.shape):
                orig = base[idx]
                base[idx] = orig + step
                lp = _loss(c, softplus)
                base[idx] = orig - step
                lm = _loss(c, softplus)
                base[idx] = orig
                fd[idx] = (lp - lm) / (2.0 * step)
            got = np.reshape(gr[gname], fd.shape)
            err = np.max(np.abs(got - fd)) / max(1e-12, np.max(np.abs(fd)))
            assert err < 1e-4, "gradient %s differs from finite differences: %.3g" % (gname, err)


def pin_bwd_autograd(seed=23):
    """The backward oracle equals fp64 reverse-mode autodiff (torch, CPU) of a
    separately written, vectorised forward recurrence."""
    import torch
    rng = np.random.default_rng(seed)
    batch, L, D, N, G = 2, 9, 6, 4, 3
    c = _bwd_case(rng, batch, L, D, N, G)
    T = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
         for k, v in c.items() if k not in ("dy", "dh_final")}
    grp = torch.arange(D) // (D // G)
    v = T["delta"] + T["delta_bias"]
    dt = torch.nn.functional.softplus(v)
    h = T["h0"]
    ys = []
    for t in range(L):
        Bt = T["Bm"][:, t][:, grp]                     # (batch, D, N)
        Ct = T["Cm"][:, t][:, grp]
        h = torch.exp(dt[:, t, :, None] * T["A"]) * h + dt[:, t, :, None] * Bt * T["x"][:, t, :, None]
        yc = (Ct * h).sum(-1) + T["Dskip"] * T["x"][:, t]
        ys.append(yc * torch.sigmoid(T["z"][:, t]) * T["z"][:, t])
    y = torch.stack(ys, dim=1)
    loss = (y * torch.tensor(c["dy"], dtype=torch.float64)).sum() + (h * torch.tensor(c["dh_final"])).sum()
    loss.backward()
    gr = oracle.selective_scan_bwd(c["x"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], c["Dskip"],
                                   c["z"], c["delta_bias"], c["h0"], c["dh_final"])
    pairs = {"dx": "x", "ddelta": "delta", "dz": "z", "dB": "Bm", "dC": "Cm", "dA": "A",
             "dDskip": "Dskip", "ddelta_bias": "delta_bias", "dh0": "h0"}
    for gname, key in pairs.items():
        want = T[key].grad.numpy()
        assert _rel(np.reshape(gr[gname], want.shape), want) < 1e-11, "autograd differs on %s" % gname


SCAN_PINS = [pin_lti_convolution, pin_lti_lfilter, pin_semiseparable, pin_small_step_keeps_state,
             pin_large_step_forgets, pin_zero_input_pure_decay, pin_split_invariance,
             pin_linearity, pin_geometric_series, pin_softplus_identities, pin_gate_identity,
             pin_skip_only, pin_channel_subset, pin_decode_steps_equal_scan, pin_groups_split]
SSD_PINS = [pin_ssd_semiseparable, pin_ssd_is_broadcast_scan, pin_ssd_channel_subset,
            pin_ssd_decode_steps_equal_ssd, pin_ssd_groups_split]
CONV_PINS = [pin_conv1d_numpy, pin_conv1d_history, pin_conv1d_streaming]
BWD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd]
def _ssd_bwd_case(rng, batch, L, H, P, N, G):
    return dict(x=_f32(rng.standard_normal((batch, L, H, P))),
                dt=_f32(rng.normal(0.0, 0.5, size=(batch, L, H))),
                A=_f32(-rng.uniform(0.5, 4.0, size=H)),
                Bm=_f32(rng.standard_normal((batch, L, G, N))),
                Cm=_f32(rng.standard_normal((batch, L, G, N))),
                Dskip=_f32(rng.standard_normal(H)),
                z=_f32(rng.standard_normal((batch, L, H, P))),
                dt_bias=_f32(rng.uniform(-3.0, -1.0, size=H)),
                h0=rng.standard_normal((batch, H, P, N)),
                dy=_f32(rng.standard_normal((batch, L, H, P))),
                dh_final=rng.standard_normal((batch, H, P, N)))


def _ssd_loss(c, softplus=True):
    y, hf = oracle.ssd(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], c["Dskip"], c["z"], c["dt_bias"],
                       c["h0"], dt_softplus=softplus)
    return float(np.sum(y * c["dy"].astype(np.float64)) + np.sum(hf * c["dh_final"]))


def pin_ssd_bwd_finite_differences(seed=24):
    """The SSD-form gradients (the scan gradients of the broadcast problem, summed
    over each shared parameter's copies) equal central differences of the
    separately written SSD forward oracle, for every input, with B/C groups."""
    rng = np.random.default_rng(seed)
    for softplus, H, G in ((True, 6, 3), (False, 4, 1)):
        c = _ssd_bwd_case(rng, 2, 5, H, 2, 3, G)
        if not softplus:
            c["dt"] = np.abs(c["dt"]) + _f32(0.05)
            c["dt_bias"] = _f32(np.zeros(H))
        gr = oracle.ssd_bwd(c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], c["dy"], c["Dskip"], c["z"],
                            c["dt_bias"], c["h0"], c["dh_final"], softplus)
        names = {"x": "dx", "dt": "ddt", "z": "dz", "Bm": "dB", "Cm": "dC", "A": "dA",
                 "Dskip": "dDskip", "dt_bias": "ddt_bias", "h0": "dh0"}
        for key, gname in names.items():
            base = c[key]
            step = 2.0 ** -10 if base.dtype == np.float32 else 1e-6
            fd = np.empty(base.shape)
            for idx in np.ndindex(base.shape):
                orig = base[idx]
                base[idx] = orig + step
                lp = _ssd_loss(c, softplus)
                base[idx] = orig - step
                lm = _ssd_loss(c, softplus)
                base[idx] = orig
                fd[idx] = (lp - lm) / (2.0 * step)
            got = np.reshape(gr[gname], fd.shape)
            err = np.max(np.abs(got - fd)) / max(1e-12, np.max(np.abs(fd)))
            assert err < 1e-4, "SSD gradient %s differs from finite differences: %.3g" % (gname, err)


def pin_ssd_bwd_head_subset(seed=25):
    """Restricting the SSD gradients to a subset of heads returns exactly those
    heads' rows of the full result, and the shares of dB, dC over a partition of
    the heads add up to the full dB, dC."""
    rng = np.random.default_rng(seed)
    c = _ssd_bwd_case(rng, 1, 7, 6, 2, 4, 3)
    args = (c["x"], c["dt"], c["A"], c["Bm"], c["Cm"], c["dy"], c["Dskip"], c["z"], c["dt_bias"], c["h0"],
            c["dh_final"])
    full = oracle.ssd_bwd(*args)
    parts = [oracle.ssd_bwd(*args, heads=hs) for hs in ([4, 0, 5], [1, 3, 2])]
    for k, ax in (("dx", 2), ("ddt", 2), ("dz", 2), ("dh0", 1), ("dA", 0), ("dDskip", 0), ("ddt_bias", 0)):
        assert np.array_equal(np.take(full[k], [4, 0, 5], axis=ax), parts[0][k]), k
    for k in ("dB", "dC"):
        assert _rel(parts[0][k] + parts[1][k], full[k]) < 1e-14, k


SSD_BWD_PINS = [pin_ssd_bwd_finite_differences, pin_ssd_bwd_head_subset]

ALL_PINS = SCAN_PINS + SSD_PINS + CONV_PINS + BWD_PINS + SSD_BWD_PINS
