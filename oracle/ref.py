"""Plain fp64 CPU oracle for the linear-recurrence scans.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports it and shares no code
with it; both sides only consume the same seeded inputs from ``lrgen``.

Every function is sequential in time and vectorised only across independent
channels (batch, channel, head, state index).  Nothing is blocked, chunked,
fused or reordered.  Inputs are taken as given (bf16 values arrive as exact
float32 values) and promoted to float64.

Sources (cited by page title and section):
  [KS]  IBM Research blog "K-Search for MLX" (repost), section
        "A 20x faster prefill: the Mamba SSM kernel": the recurrence
        h_t = a_t h_{t-1} + b_t and the associative combine of (a, b) pairs.
  [MR]  "mlx-recurrence" post, Apple Developer Forums thread 840535: the
        kernel list (ssd_scan, gla_scan, rglru_scan) with state shapes, and
        the segment checkpoint-and-recompute training path.
  [LX]  "lrnnx: A library for Linear RNNs" (paper summary), Key Contributions
        2-3: ZOH as a discretisation of the time-varying selective scan, and
        the fused scan + output projection.

Readings where the pages are silent (each is listed in the design doc):
  * ZOH: e = exp(dt*A), phi = expm1(dt*A)/A (phi = dt when A == 0), i.e. the
    textbook exact zero-order hold for a diagonal A.  "euler" gives phi = dt.
  * The readout is inclusive: y_t reads h_t after token t has been written.
  * h_{-1} = h0 (zero when not given).
  * SSD: A and Dskip are per head; B, C are shared by the H/G heads of a group.
  * GLA: S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, no extra scaling.
  * The backward differentiates loss = sum(dy * y) + <dh_last, h_last>.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, brute-force unrolls, library routines (numpy matmul,
torch.autograd) or finite differences.  No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f(x):
    return None if x is None else np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------
# The associative combine  [KS, combine equation]
# ---------------------------------------------------------------------------
def combine(later, earlier):
    """(a2, b2) o (a1, b1) = (a2*a1, a2*b1 + b2): apply ``earlier`` first,
    then ``later``.  The operator is associative but not commutative."""
    a2, b2 = later
    a1, b1 = earlier
    return (a2 * a1, a2 * b1 + b2)


# ---------------------------------------------------------------------------
# Diagonal recurrence  [KS, recurrence equation; MR, rglru_scan state [B, D]]
# ---------------------------------------------------------------------------
def diag_scan(a, b, h0=None):
    """h[:, t] = a[:, t] * h[:, t-1] + b[:, t]; a, b: [B, L, D].

    Returns (h [B, L, D], h_last [B, D]) in float64."""
    a, b = _f(a), _f(b)
    Bn, L, D = a.shape
    h = np.zeros((Bn, D), F64) if h0 is None else _f(h0).copy()
    out = np.empty((Bn, L, D), F64)
    for t in range(L):
        h = a[:, t] * h + b[:, t]
        out[:, t] = h
    return out, h


def diag_scan_bwd(a, h, dh, h0=None, dh_last=None):
    """Reverse-time adjoint of ``diag_scan`` for the loss
    sum_t <dh[:, t], h[:, t]> + <dh_last, h[:, L-1]>  (h = forward outputs).

    g_t = dl/dh_t (through every later step):
        g_{L-1} = dh_{L-1} + dh_last,   g_t = dh_t + a_{t+1} g_{t+1}
    then db_t = g_t, da_t = g_t h_{t-1} (h_{-1} = h0 or 0), dh0 = a_0 g_0.
    Returns (da, db, dh0) in float64 (dh0 = dh_last when L = 0)."""
    a, h, dh = _f(a), _f(h), _f(dh)
    Bn, L, D = a.shape
    g = np.zeros((Bn, D), F64) if dh_last is None else _f(dh_last).copy()
    hm1 = np.zeros((Bn, D), F64) if h0 is None else _f(h0)
    da = np.empty((Bn, L, D), F64)
    db = np.empty((Bn, L, D), F64)
    for t in range(L - 1, -1, -1):
        if t < L - 1:
            g = a[:, t + 1] * g
        g = g + dh[:, t]
        db[:, t] = g
        da[:, t] = g * (h[:, t - 1] if t > 0 else hm1)
    dh0 = a[:, 0] * g if L > 0 else g
    return da, db, dh0


# ---------------------------------------------------------------------------
# Discretisation  [LX, Key Contributions 2-3: ZOH]
# ---------------------------------------------------------------------------
def discretize(dt, A, disc="zoh"):
    """Return (e, phi): the decay e and the input factor phi of one step, so
    that h <- e h + phi B x.  With l = dt*A:
    zoh:      e = exp(l),                phi = expm1(l) / A  (phi = dt at A = 0)
    euler:    e = exp(l),                phi = dt
    bilinear: e = (1 + l/2) / (1 - l/2), phi = dt / (1 - l/2)   (Tustin)
    dirac:    e = exp(l),                phi = 1   (the input is an impulse of
              area x at the sample: the state jumps by B x, no dt factor)
    ``dt`` and ``A`` broadcast against each other."""
    dt, A = np.broadcast_arrays(_f(dt), _f(A))
    lam = dt * A
    if disc == "bilinear":
        den = 1.0 - 0.5 * lam
        return (1.0 + 0.5 * lam) / den, dt / den
    e = np.exp(lam)
    if disc == "zoh":
        safe = np.where(A == 0.0, 1.0, A)
        phi = np.where(A == 0.0, dt, np.expm1(lam) / safe)
    elif disc == "euler":
        phi = dt.copy()
    elif disc == "dirac":
        phi = np.ones_like(dt)
    else:
        raise ValueError(disc)
    return e, phi


def discretize_grads(dt, A, e, phi, disc="zoh"):
    """Partial derivatives (de/ddt, de/dA, dphi/ddt, dphi/dA).

    zoh: dphi/dA = (dt*e - phi)/A, evaluated as dt^2 (1/2 + l/3 + l^2/8 +
    l^3/30) for |l| = |dt*A| < 1e-3 to avoid cancellation.
    bilinear: with den = 1 - l/2, de/dl = 1/den^2, dphi/ddt = 1/den^2 and
    dphi/dA = dt^2 / (2 den^2)."""
    dt, A = np.broadcast_arrays(_f(dt), _f(A))
    if disc == "bilinear":
        den2 = (1.0 - 0.5 * dt * A) ** 2
        return A / den2, dt / den2, 1.0 / den2, dt * dt / (2.0 * den2)
    de_ddt = A * e
    de_dA = dt * e
    if disc == "zoh":
        lam = dt * A
        small = np.abs(lam) < 1e-3
        safe = np.where(A == 0.0, 1.0, A)
        direct = (dt * e - phi) / safe
        series = dt * dt * (0.5 + lam / 3.0 + lam * lam / 8.0 + lam ** 3 / 30.0)
        dphi_ddt = e
        dphi_dA = np.where(small, series, direct)
    elif disc == "euler":
        dphi_ddt = np.ones_like(dt)
        dphi_dA = np.zeros_like(dt)
    else:  # dirac
        dphi_ddt = np.zeros_like(dt)
        dphi_dA = np.zeros_like(dt)
    return de_ddt, de_dA, dphi_ddt, dphi_dA


# ---------------------------------------------------------------------------
def selective_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh"):
    """x, dt: [B, L, D]; A: [D, N]; Bm, Cm: [B, L, N]; Dskip: [D]; h0: [B, D, N].

    h[b, d, n] <- e*h + phi*Bm[b, t, n]*x[b, t, d],  e, phi from dt[b,t,d]*A[d,n]
    y[b, t, d]  = sum_n Cm[b, t, n]*h[b, d, n] + Dskip[d]*x[b, t, d]
    Returns (y [B, L, D], h_last [B, D, N])."""
    x, dt, A, Bm, Cm = map(_f, (x, dt, A, Bm, Cm))
    Bn, L, D = x.shape
    N = A.shape[1]
    h = np.zeros((Bn, D, N), F64) if h0 is None else _f(h0).copy()
    Dv = np.zeros(D, F64) if Dskip is None else _f(Dskip)
    y = np.empty((Bn, L, D), F64)
    for t in range(L):
        e, phi = discretize(dt[:, t, :, None], A[None], disc)
        h = e * h + phi * Bm[:, t, None, :] * x[:, t, :, None]
        y[:, t] = np.einsum("bdn,bn->bd", h, Cm[:, t]) + Dv * x[:, t]
    return y, h


def selective_scan_bwd(x, dt, A, Bm, Cm, Dskip, h0, dy, dh_last=None, disc="zoh"):
    """Gradients of loss = sum(dy*y) + <dh_last, h_last> for ``selective_scan``.

    Reverse-time adjoint written out directly: with G_t = dloss/dh_t
    ([B, D, N]),
        G_{L-1} = dh_last + dy_{L-1} C_{L-1},   G_t = e_{t+1} G_{t+1} + dy_t C_t,
    the input gradients are
        dx_t[d] = sum_n G phi B_t[n] + Dskip[d] dy_t[d],
        dB_t[n] = sum_d G phi x_t[d],     dC_t[n] = sum_d h_t dy_t[d],
        dphi = G B_t[n] x_t[d],           de = G h_{t-1},
        dD[d]  = sum_{b,t} dy x,          dh0 = e_0 G_0,
    and dt, A follow by the chain rule through (e, phi).  The full forward
    state history is kept.  Returns a dict of float64 arrays."""
    x, dt, A, Bm, Cm, dy = map(_f, (x, dt, A, Bm, Cm, dy))
    Bn, L, D = x.shape
    N = A.shape[1]
    Dv = np.zeros(D, F64) if Dskip is None else _f(Dskip)
    hist = np.empty((L + 1, Bn, D, N), F64)
    hist[0] = np.zeros((Bn, D, N), F64) if h0 is None else _f(h0)
    for t in range(L):
        e, phi = discretize(dt[:, t, :, None], A[None], disc)
        hist[t + 1] = e * hist[t] + phi * Bm[:, t, None, :] * x[:, t, :, None]
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dB = np.empty_like(Bm)
    dC = np.empty_like(Cm)
    dA = np.zeros((D, N), F64)
    Gt = np.zeros((Bn, D, N), F64) if dh_last is None else _f(dh_last).copy()
    for t in range(L - 1, -1, -1):
        e, phi = discretize(dt[:, t, :, None], A[None], disc)
        Gt = Gt + dy[:, t, :, None] * Cm[:, t, None, :]
        gphi = Gt * phi
        dx[:, t] = np.einsum("bdn,bn->bd", gphi, Bm[:, t]) + Dv * dy[:, t]
        dB[:, t] = np.einsum("bdn,bd->bn", gphi, x[:, t])
        dC[:, t] = np.einsum("bdn,bd->bn", hist[t + 1], dy[:, t])
        dphi = Gt * Bm[:, t, None, :] * x[:, t, :, None]
        de = Gt * hist[t]
        de_ddt, de_dA, dphi_ddt, dphi_dA = discretize_grads(dt[:, t, :, None], A[None], e, phi, disc)
        ddt[:, t] = (de * de_ddt + dphi * dphi_ddt).sum(axis=2)
        dA += (de * de_dA + dphi * dphi_dA).sum(axis=0)
        Gt = e * Gt
    dD = np.einsum("bld,bld->d", dy, x)
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=Gt)


# ---------------------------------------------------------------------------
# Mamba-2 head-wise SSD scan  [MR, ssd_scan: state [B, H, Dh, N]]
# ---------------------------------------------------------------------------
def _expand_groups(M, H):
    """[B, L, G, N] -> [B, L, H, N]: head h reads group h // (H // G)."""
    G = M.shape[2]
    return np.repeat(M, H // G, axis=2)


def ssd_scan(x, dt, A, Bm, Cm, Dskip=None, h0=None, disc="zoh", seg=0):
    """x: [B, L, H, P]; dt: [B, L, H]; A, Dskip: [H]; Bm, Cm: [B, L, G, N];
    h0: [B, H, P, N].

    h[b,h,p,n] <- e*h + phi*x[b,t,h,p]*Bm[b,t,g,n],  e, phi from dt[b,t,h]*A[h]
    y[b,t,h,p]  = sum_n Cm[b,t,g,n]*h[b,h,p,n] + Dskip[h]*x[b,t,h,p]
    With seg > 0 also returns ckpt[s] = the state entering token s*seg
    ([ceil(L/seg), B, H, P, N]); ckpt[0] = h0 (or 0).
    Returns (y, h_last, ckpt or None)."""
    x, dt, A, Bm, Cm = map(_f, (x, dt, A, Bm, Cm))
    Bn, L, H, P = x.shape
    N = Bm.shape[3]
    Bh, Ch = _expand_groups(Bm, H), _expand_groups(Cm, H)
    h = np.zeros((Bn, H, P, N), F64) if h0 is None else _f(h0).copy()
    Dv = np.zeros(H, F64) if Dskip is None else _f(Dskip)
    y = np.empty((Bn, L, H, P), F64)
    ckpt = None
    if seg:
        ckpt = np.empty(((L + seg - 1) // seg, Bn, H, P, N), F64)
    for t in range(L):
        if seg and t % seg == 0:
            ckpt[t // seg] = h
        e, phi = discretize(dt[:, t], A[None], disc)          # [B, H]
        h = (e[:, :, None, None] * h
             + phi[:, :, None, None] * x[:, t, :, :, None] * Bh[:, t, :, None, :])
        y[:, t] = np.einsum("bhpn,bhn->bhp", h, Ch[:, t]) + Dv[None, :, None] * x[:, t]
    return y, h, ckpt


def ssd_scan_bwd(x, dt, A, Bm, Cm, Dskip, h0, dy, dh_last=None, disc="zoh"):
    """Gradients of loss = sum(dy*y) + <dh_last, h_last> for ``ssd_scan``.

    Reverse-time adjoint of the recurrence, written out directly: with
    G_t = dloss/dh_t (P x N per head),
        G_{L-1} = dh_last + dy_{L-1} (x) C_{L-1},
        G_t     = e_{t+1} G_{t+1} + dy_t (x) C_t,
    the input gradients are
        dx_t  = phi_t G_t B_t + Dskip dy_t,        dB_t += phi_t G_t^T x_t,
        dC_t += h_t^T dy_t,                        dphi_t = x_t^T G_t B_t,
        de_t  = <G_t, h_{t-1}>_F,                  dh0 = e_0 G_0,
        dD   += <dy_t, x_t>,
    and dt, A follow by the chain rule through (e, phi).  dB and dC sum over
    the heads of a group.  The full forward state history is kept (no
    checkpointing).  Returns a dict of float64 arrays."""
    x, dt, A, Bm, Cm, dy = map(_f, (x, dt, A, Bm, Cm, dy))
    Bn, L, H, P = x.shape
    G = Bm.shape[2]
    N = Bm.shape[3]
    hpg = H // G
    Bh, Ch = _expand_groups(Bm, H), _expand_groups(Cm, H)
    Dv = np.zeros(H, F64) if Dskip is None else _f(Dskip)
    h_init = np.zeros((Bn, H, P, N), F64) if h0 is None else _f(h0)

    # forward, keeping h_{t} for t = -1 .. L-1
    hist = np.empty((L + 1, Bn, H, P, N), F64)
    hist[0] = h_init
    E = np.empty((Bn, L, H), F64)
    PHI = np.empty((Bn, L, H), F64)
    for t in range(L):
        e, phi = discretize(dt[:, t], A[None], disc)
        E[:, t], PHI[:, t] = e, phi
        hist[t + 1] = (e[:, :, None, None] * hist[t]
                       + phi[:, :, None, None] * x[:, t, :, :, None] * Bh[:, t, :, None, :])

    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dBh = np.empty((Bn, L, H, N), F64)
    dCh = np.empty((Bn, L, H, N), F64)
    dA = np.zeros(H, F64)
    Gt = np.zeros((Bn, H, P, N), F64) if dh_last is None else _f(dh_last).copy()
    for t in range(L - 1, -1, -1):
        Gt = Gt + dy[:, t, :, :, None] * Ch[:, t, :, None, :]
        h_t, h_prev = hist[t + 1], hist[t]
        e, phi = E[:, t], PHI[:, t]
        dCh[:, t] = np.einsum("bhpn,bhp->bhn", h_t, dy[:, t])
        gB = np.einsum("bhpn,bhn->bhp", Gt, Bh[:, t])
        dx[:, t] = phi[:, :, None] * gB + Dv[None, :, None] * dy[:, t]
        dBh[:, t] = phi[:, :, None] * np.einsum("bhpn,bhp->bhn", Gt, x[:, t])
        dphi = np.einsum("bhp,bhp->bh", x[:, t], gB)
        de = np.einsum("bhpn,bhpn->bh", Gt, h_prev)
        de_ddt, de_dA, dphi_ddt, dphi_dA = discretize_grads(dt[:, t], A[None], e, phi, disc)
        ddt[:, t] = de * de_ddt + dphi * dphi_ddt
        dA += (de * de_dA + dphi * dphi_dA).sum(axis=0)
        Gt = e[:, :, None, None] * Gt
    dh0 = Gt
    dD = np.einsum("blhp,blhp->h", dy, x)
    dB = dBh.reshape(Bn, L, G, hpg, N).sum(axis=3)
    dC = dCh.reshape(Bn, L, G, hpg, N).sum(axis=3)
    return dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


# ---------------------------------------------------------------------------
# Gated linear attention  [MR, gla_scan: scalar forget gate, outer-product
# write, state [B, H, Dh, Dh]]
# ---------------------------------------------------------------------------
def gla_scan(q, k, v, g, S0=None):
    """q, k: [B, L, H, K]; v: [B, L, H, V]; g: [B, L, H]; S0: [B, H, K, V].

    S[b,h] <- g[b,t,h]*S[b,h] + k[b,t,h] v[b,t,h]^T
    o[b,t,h] = S[b,h]^T q[b,t,h]
    Returns (o [B, L, H, V], S_last [B, H, K, V])."""
    q, k, v, g = map(_f, (q, k, v, g))
    Bn, L, H, K = q.shape
    V = v.shape[3]
    S = np.zeros((Bn, H, K, V), F64) if S0 is None else _f(S0).copy()
    o = np.empty((Bn, L, H, V), F64)
    for t in range(L):
        S = g[:, t, :, None, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


def gla_scan_bwd(q, k, v, g, S0, do, dS_last=None):
    """Gradients of loss = sum(do*o) + <dS_last, S_last> for ``gla_scan``.

    Reverse-time adjoint written out directly: with G_t = dloss/dS_t (K x V),
        G_{L-1} = dS_last + q_{L-1} do_{L-1}^T,   G_t = g_{t+1} G_{t+1} + q_t do_t^T,
    the input gradients are
        dq_t = S_t do_t,   dk_t = G_t v_t,   dv_t = G_t^T k_t,
        dg_t = <G_t, S_{t-1}>_F,   dS0 = g_0 G_0.
    The forward state history is kept for every (b, h) (no checkpointing).
    Returns a dict of float64 arrays dq, dk, dv, dg, dS0."""
    q, k, v, g, do = map(_f, (q, k, v, g, do))
    Bn, L, H, K = q.shape
    V = v.shape[3]
    S_init = np.zeros((Bn, H, K, V), F64) if S0 is None else _f(S0)
    hist = np.empty((L + 1, Bn, H, K, V), F64)
    hist[0] = S_init
    for t in range(L):
        hist[t + 1] = (g[:, t, :, None, None] * hist[t]
                       + k[:, t, :, :, None] * v[:, t, :, None, :])
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dg = np.empty_like(g)
    Gt = np.zeros((Bn, H, K, V), F64) if dS_last is None else _f(dS_last).copy()
    for t in range(L - 1, -1, -1):
        Gt = Gt + q[:, t, :, :, None] * do[:, t, :, None, :]
        dq[:, t] = np.einsum("bhkv,bhv->bhk", hist[t + 1], do[:, t])
        dk[:, t] = np.einsum("bhkv,bhv->bhk", Gt, v[:, t])
        dv[:, t] = np.einsum("bhkv,bhk->bhv", Gt, k[:, t])
        dg[:, t] = np.einsum("bhkv,bhkv->bh", Gt, hist[t])
        Gt = g[:, t, :, None, None] * Gt
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dS0=Gt)


# ---------------------------------------------------------------------------
# Rotational LRU  ["mlx-recurrence" post, rotlru_scan: complex-diagonal
# recurrence, magnitude gate, per-step rotation of two-dimensional channel
# pairs, state [B, D] as interleaved pairs]
# ---------------------------------------------------------------------------
def rotlru_scan(r, theta, u, h0=None):
    """r, theta: [B, L, D/2]; u: [B, L, D] (pairs (2i, 2i+1) = (re, im)).

    Per pair, with z = h[2i] + 1j h[2i+1]:
        z_t = r_t exp(1j theta_t) z_{t-1} + (u_t[2i] + 1j u_t[2i+1])
    i.e. each pair is rotated by theta_t, scaled by the gate r_t, then the
    input pair is added.  Returns (h [B, L, D], h_last [B, D]) in float64."""
    r, theta, u = map(_f, (r, theta, u))
    Bn, L, D = u.shape
    z = np.zeros((Bn, D // 2), np.complex128) if h0 is None else _f(h0)[:, 0::2] + 1j * _f(h0)[:, 1::2]
    out = np.empty((Bn, L, D), F64)
    for t in range(L):
        a = r[:, t] * np.exp(1j * theta[:, t])
        z = a * z + (u[:, t, 0::2] + 1j * u[:, t, 1::2])
        out[:, t, 0::2] = z.real
        out[:, t, 1::2] = z.imag
    last = np.empty((Bn, D), F64)
    last[:, 0::2] = z.real
    last[:, 1::2] = z.imag
    return out, last


def rotlru_scan_bwd(r, theta, h, dh, h0=None, dh_last=None):
    """Reverse-time adjoint of ``rotlru_scan`` for the loss
    sum_t <dh[:, t], h[:, t]> + <dh_last, h_last>  (h = forward outputs,
    real inner products over the interleaved pairs).

    With z, g complex per pair (g = dl/dre + 1j dl/dim), a_t = r_t e^{1j theta_t}:
        g_{L-1} = dh_{L-1} + dh_last,   g_t = dh_t + conj(a_{t+1}) g_{t+1}
    then du_t = g_t (split back into (re, im)), and with q = g_t conj(e^{1j theta_t} z_{t-1})
    (z_{-1} = h0 or 0):  dr_t = Re q,  dtheta_t = r_t Im q;  dh0 = conj(a_0) g_0.
    Returns (dr, dtheta, du, dh0) in float64 (dh0 = dh_last when L = 0)."""
    r, theta, h, dh = map(_f, (r, theta, h, dh))
    Bn, L, D = h.shape
    c = lambda v: v[..., 0::2] + 1j * v[..., 1::2]   # noqa: E731
    g = np.zeros((Bn, D // 2), np.complex128) if dh_last is None else c(_f(dh_last))
    zm1 = np.zeros((Bn, D // 2), np.complex128) if h0 is None else c(_f(h0))
    dr = np.empty((Bn, L, D // 2), F64)
    dth = np.empty((Bn, L, D // 2), F64)
    du = np.empty((Bn, L, D), F64)
    for t in range(L - 1, -1, -1):
        if t < L - 1:
            g = np.conj(r[:, t + 1] * np.exp(1j * theta[:, t + 1])) * g
        g = g + c(dh[:, t])
        du[:, t, 0::2], du[:, t, 1::2] = g.real, g.imag
        zp = c(h[:, t - 1]) if t > 0 else zm1
        q = g * np.conj(np.exp(1j * theta[:, t]) * zp)
        dr[:, t] = q.real
        dth[:, t] = r[:, t] * q.imag
    if L > 0:
        g = np.conj(r[:, 0] * np.exp(1j * theta[:, 0])) * g
    dh0 = np.empty((Bn, D), F64)
    dh0[:, 0::2], dh0[:, 1::2] = g.real, g.imag
    return dr, dth, du, dh0
