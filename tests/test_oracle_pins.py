"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's loop: each compares it with a
different formulation of the same result (a convolution, a closed-form
double sum, an associative scan, a limit, a library routine) or with an
identity that any correct scan must satisfy.  Softplus and SiLU on the test
side come from library routines (numpy.logaddexp, scipy.special.expit).

Sources (page, section):
  * LTI convolution kernel K = (C B_bar, C A_bar B_bar, C A_bar^2 B_bar, ...):
    Mamba tutorial (pwwt.cn) §2.3; Gu & Dao deep-reading report §2.2 (Eq. 3).
  * closed form h_t = sum_{s<=t} (prod_{s<k<=t} a_k) b_s: tutorial §4.3.
  * associative operator (a,b)o(c,d) = (ac, ad+b): selection-mechanism article
    (discosf.com) §3.1; paper walkthrough (m.lqnn.cn) §3.1.
  * Delta -> 0 keeps the state, large Delta resets it toward the input:
    tutorial §3.1; selection-mechanism article §2.1.
  * decode = one step of the recurrence: tutorial §5.1 and §6.3.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def softplus_lib(x):
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def silu_lib(z):
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def rng_inputs(seed, batch, L, dim, N, A=None):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    u = f(batch, L, dim)
    delta = (0.5 * f(batch, L, dim)).astype(np.float32)
    Bm = f(batch, L, N)
    Cm = f(batch, L, N)
    z = f(batch, L, dim)
    if A is None:
        A = (-rng.uniform(0.05, 2.0, size=(dim, N))).astype(np.float32)
    D = f(dim)
    bias = rng.uniform(-4.0, -1.0, size=dim).astype(np.float32)
    h0 = f(batch, dim, N)
    return u, delta, A, Bm, Cm, D, z, bias, h0


# ----------------------------------------------------------------------------
# LTI special case == convolution with K_k = C A_bar^k B_bar (brute force)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("with_h0", [False, True])
def test_lti_equals_convolution(with_h0):
    batch, L, dim, N = 2, 48, 3, 4
    u, _, A, _, _, D, _, bias, h0 = rng_inputs(1, batch, L, dim, N)
    rng = np.random.default_rng(2)
    # Delta constant in time per (b, d), B and C constant in time per b.
    c = rng.uniform(-1.0, 1.0, size=(batch, 1, dim)).astype(np.float32)
    delta = np.broadcast_to(c, (batch, L, dim)).copy()
    Bv = rng.standard_normal((batch, 1, N)).astype(np.float32)
    Cv = rng.standard_normal((batch, 1, N)).astype(np.float32)
    Bm = np.broadcast_to(Bv, (batch, L, N)).copy()
    Cm = np.broadcast_to(Cv, (batch, L, N)).copy()
    y, h_last = oracle.fwd(u, delta, A, Bm, Cm, D, None, bias, True,
                           h0=h0 if with_h0 else None)

    dt = softplus_lib(c[:, 0, :].astype(np.float64) + bias)          # (batch, dim)
    expect = np.zeros((batch, L, dim))
    for b in range(batch):
        for d in range(dim):
            Abar = np.exp(dt[b, d] * A[d].astype(np.float64))         # (N,)
            Bbar = dt[b, d] * Bv[b, 0].astype(np.float64)             # (N,)
            Cb = Cv[b, 0].astype(np.float64)
            K = np.array([np.sum(Cb * Abar ** k * Bbar) for k in range(L)])
            for t in range(L):
                acc = sum(K[k] * float(u[b, t - k, d]) for k in range(t + 1))
                if with_h0:
                    acc += np.sum(Cb * Abar ** (t + 1) * h0[b, d].astype(np.float64))
                expect[b, t, d] = acc + float(D[d]) * float(u[b, t, d])
    assert rel(y, expect) < 1e-12


# ----------------------------------------------------------------------------
# Time-varying case == closed-form double sum over s <= t
# ----------------------------------------------------------------------------
def closed_form(u, delta, A, Bm, Cm, D, z, bias, h0):
    batch, L, dim = u.shape
    N = A.shape[1]
    dt = softplus_lib(delta.astype(np.float64) + bias)                  # (b, L, d)
    S = np.cumsum(dt, axis=1)
    y = np.zeros((batch, L, dim))
    hL = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            An = A[d].astype(np.float64)
            for t in range(L):
                h = np.exp(An * S[b, t, d]) * (h0[b, d].astype(np.float64) if h0 is not None
                                               else 0.0)
                for s in range(t + 1):
                    h = h + np.exp(An * (S[b, t, d] - S[b, s, d])) * dt[b, s, d] \
                        * Bm[b, s].astype(np.float64) * float(u[b, s, d])
                yv = np.dot(Cm[b, t].astype(np.float64), h) + float(D[d]) * float(u[b, t, d])
                if z is not None:
                    yv *= silu_lib(float(z[b, t, d]))
                y[b, t, d] = yv
                if t == L - 1:
                    hL[b, d] = h
    return y, hL


@pytest.mark.parametrize("gate", [False, True])
def test_time_varying_equals_closed_form(gate):
    batch, L, dim, N = 2, 40, 3, 5
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(3, batch, L, dim, N)
    zz = z if gate else None
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, zz, bias, True, h0=h0)
    ey, ehL = closed_form(u, delta, A, Bm, Cm, D, zz, bias, h0)
    assert rel(y, ey) < 1e-11
    assert rel(hL, ehL) < 1e-11


def test_closed_form_catches_swapped_B_C():
    """Meta-check: with B and C swapped the closed form disagrees, so the pin
    above distinguishes the two roles (they commute only in the LTI case)."""
    batch, L, dim, N = 1, 24, 2, 4
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(4, batch, L, dim, N)
    y, _ = oracle.fwd(u, delta, A, Cm, Bm, D, None, bias, True)
    ey, _ = closed_form(u, delta, A, Bm, Cm, D, None, bias, None)
    assert rel(y, ey) > 1e-3


# ----------------------------------------------------------------------------
# Associative-operator scan == sequential loop
# ----------------------------------------------------------------------------
def combine(earlier, later):
    """(a1,b1) then (a2,b2): the later element acts on the left, so the
    composite maps h -> a2 (a1 h + b1) + b2 = (a2 a1) h + (a2 b1 + b2)."""
    a1, b1 = earlier
    a2, b2 = later
    return a2 * a1, a2 * b1 + b2


def hillis_steele(a, b):
    """Inclusive scan along axis 0 with ``combine`` (log-depth, fp64)."""
    a = a.copy()
    b = b.copy()
    L = a.shape[0]
    off = 1
    while off < L:
        na, nb = a.copy(), b.copy()
        na[off:], nb[off:] = combine((a[:-off], b[:-off]), (a[off:], b[off:]))
        a, b = na, nb
        off *= 2
    return a, b


def blelloch_exclusive(a, b):
    """Work-efficient (up-sweep / down-sweep) exclusive scan, L a power of 2."""
    L = a.shape[0]
    a = a.copy()
    b = b.copy()
    d = 1
    while d < L:
        idx = np.arange(2 * d - 1, L, 2 * d)
        a[idx], b[idx] = combine((a[idx - d], b[idx - d]), (a[idx], b[idx]))
        d *= 2
    a[L - 1], b[L - 1] = 1.0, 0.0
    d = L // 2
    while d >= 1:
        idx = np.arange(2 * d - 1, L, 2 * d)
        la, lb = a[idx - d].copy(), b[idx - d].copy()
        a[idx - d], b[idx - d] = a[idx], b[idx]
        a[idx], b[idx] = combine((a[idx], b[idx]), (la, lb))
        d //= 2
    return a, b


@pytest.mark.parametrize("scan", ["hillis_steele", "blelloch"])
def test_associative_scan_equals_loop(scan):
    batch, L, dim, N = 1, 64, 3, 6
    u, delta, A, Bm, Cm, D, _, bias, h0 = rng_inputs(5, batch, L, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, None, bias, True, h0=h0)
    dt = softplus_lib(delta.astype(np.float64) + bias)[0]               # (L, dim)
    for d in range(dim):
        a = np.exp(dt[:, d:d + 1] * A[d].astype(np.float64))            # (L, N)
        bb = dt[:, d:d + 1] * Bm[0].astype(np.float64) * u[0, :, d:d + 1]
        # fold h0 into the first element: h_0 = a_0 h0 + b_0
        bb[0] += a[0] * h0[0, d]
        if scan == "hillis_steele":
            _, h = hillis_steele(a, bb)
        else:
            ea, eb = blelloch_exclusive(a, bb)
            _, h = combine((ea, eb), (a, bb))   # inclusive = exclusive then own
        ey = np.sum(Cm[0].astype(np.float64) * h, axis=1) + float(D[d]) * u[0, :, d].astype(
            np.float64)
        assert rel(y[0, :, d], ey) < 1e-12
        assert rel(hL[0, d], h[-1]) < 1e-12


def test_operator_associative_with_identity():
    rng = np.random.default_rng(6)
    for _ in range(100):
        x, y, w = [(rng.uniform(0, 1), rng.standard_normal()) for _ in range(3)]
        l1 = combine(combine(x, y), w)
        l2 = combine(x, combine(y, w))
        assert np.allclose(l1, l2, rtol=1e-13, atol=1e-13)
        assert np.allclose(combine((1.0, 0.0), x), x) and np.allclose(combine(x, (1.0, 0.0)), x)


# ----------------------------------------------------------------------------
# Delta limits
# ----------------------------------------------------------------------------
def test_delta_to_zero_keeps_state():
    batch, L, dim, N = 2, 16, 4, 8
    u, _, A, Bm, Cm, D, z, _, h0 = rng_inputs(7, batch, L, dim, N)
    delta = np.full((batch, L, dim), -40.0, np.float32)       # softplus(-40) ~ 4e-18
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, None, True, h0=h0)
    assert rel(hL, h0) < 1e-15
    ey = (np.einsum("bln,bdn->bld", Cm.astype(np.float64), h0.astype(np.float64))
          + D.astype(np.float64) * u.astype(np.float64)) * silu_lib(z)
    assert rel(y, ey) < 1e-14


def test_large_delta_resets_state():
    batch, L, dim, N = 1, 12, 3, 4
    u, delta, A, Bm, Cm, D, _, _, h0 = rng_inputs(8, batch, L, dim, N)
    A = -np.ones((dim, N), np.float32) * np.arange(1, N + 1, dtype=np.float32)
    k = 5
    delta[:, k, :] = 60.0                                      # Delta_t = 60 at step k
    h0 = 1e3 * h0
    y1, h1 = oracle.fwd(u, delta, A, Bm, Cm, D, None, None, True, h0=h0)
    # state right after step k is Delta_k B_k u_k, whatever came before
    yk, hk = oracle.fwd(u[:, :k + 1], delta[:, :k + 1], A, Bm[:, :k + 1], Cm[:, :k + 1], D,
                        None, None, True, h0=h0)
    expect = softplus_lib(60.0) * Bm[0, k][None, :].astype(np.float64) \
        * u[0, k][:, None].astype(np.float64)
    assert rel(hk[0], expect) < 1e-14
    # and nothing before step k reaches any later output
    u2 = u.copy()
    u2[:, :k] = 7.0
    y2, h2 = oracle.fwd(u2, delta, A, Bm, Cm, D, None, None, True, h0=-h0)
    assert rel(y2[:, k:], y1[:, k:]) < 1e-14
    assert rel(h2, h1) < 1e-14


# ----------------------------------------------------------------------------
# softplus, SiLU, skip path
# ----------------------------------------------------------------------------
def test_softplus_round_trip_and_values():
    # one channel per test value; L = 1, N = 1, u = B = 1, no initial state,
    # so h_last = Delta_0 = softplus(0 + bias)
    dt = np.array([1e-3, 3.1e-3, 0.05, 0.1, 2.0, 30.0])
    xs = np.concatenate([np.log(np.expm1(dt)), [-30.0, -9.0, -0.5, 0.0, 0.7, 25.0]])
    dim = xs.size
    bias = xs.astype(np.float32)
    ones = np.ones((1, 1, dim), np.float32)
    zeros = np.zeros((1, 1, dim), np.float32)
    A = -np.ones((dim, 1), np.float32)
    B1 = np.ones((1, 1, 1), np.float32)
    _, hL = oracle.fwd(ones, zeros, A, B1, B1, None, None, bias, True)
    assert rel(hL[0, :, 0], softplus_lib(bias.astype(np.float64))) < 1e-15
    # elementwise relative too (the small values matter for the fp32 path)
    got = hL[0, :, 0]
    want = softplus_lib(bias.astype(np.float64))
    assert np.max(np.abs(got - want) / want) < 1e-14
    # the round trip softplus(log(expm1(dt))) = dt up to the fp32 rounding of bias
    assert np.max(np.abs(got[:6] - dt) / dt) < 1e-6
    # without softplus, Delta is the raw sum
    _, hL2 = oracle.fwd(ones, zeros, A, B1, B1, None, None, bias, False)
    assert np.array_equal(hL2[0, :, 0], bias.astype(np.float64))


@pytest.mark.parametrize("zero", ["B", "C"])
def test_skip_path_is_D_u_silu_z(zero):
    batch, L, dim, N = 2, 10, 5, 4
    u, delta, A, Bm, Cm, D, z, bias, _ = rng_inputs(9, batch, L, dim, N)
    z = np.concatenate([z[..., :3], np.array([-30.0, 25.0], np.float32)[None, None, :]
                        .repeat(L, 1).repeat(batch, 0)], axis=-1)
    if zero == "B":
        Bm = np.zeros_like(Bm)
    else:
        Cm = np.zeros_like(Cm)
    y, _ = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True)
    ey = D.astype(np.float64) * u.astype(np.float64) * silu_lib(z)
    assert np.max(np.abs(y - ey)) <= 1e-15 * np.max(np.abs(ey))


# ----------------------------------------------------------------------------
# structural identities
# ----------------------------------------------------------------------------
def test_split_invariance():
    batch, L, dim, N = 2, 64, 3, 7
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(10, batch, L, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    for L1 in (1, 27, 63):
        ya, ha = oracle.fwd(u[:, :L1], delta[:, :L1], A, Bm[:, :L1], Cm[:, :L1], D, z[:, :L1],
                            bias, True, h0=h0)
        yb, hb = oracle.fwd(u[:, L1:], delta[:, L1:], A, Bm[:, L1:], Cm[:, L1:], D, z[:, L1:],
                            bias, True, h0=ha)
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y)
        assert np.array_equal(hb, hL)


def test_zero_length_returns_h0():
    batch, dim, N = 1, 3, 4
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(11, batch, 0, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    assert y.shape == (batch, 0, dim)
    assert np.array_equal(hL, h0.astype(np.float64))


def test_decode_steps_equal_forward():
    batch, L, dim, N = 3, 20, 4, 8
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(12, batch, L, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    state = h0.astype(np.float64).copy()
    for t in range(L):
        yt = oracle.state_update(state, u[:, t], delta[:, t], A, Bm[:, t], Cm[:, t], D, z[:, t],
                                 bias, True)
        assert rel(yt, y[:, t]) < 1e-15
    assert rel(state, hL) < 1e-15


def test_causality():
    batch, L, dim, N = 1, 30, 3, 4
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(13, batch, L, dim, N)
    y, _ = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    s = 17
    for name in ("u", "delta", "B", "C", "z"):
        u2, d2, B2, C2, z2 = u.copy(), delta.copy(), Bm.copy(), Cm.copy(), z.copy()
        {"u": u2, "delta": d2, "B": B2, "C": C2, "z": z2}[name][:, s] += 1.0
        y2, _ = oracle.fwd(u2, d2, A, B2, C2, D, z2, bias, True, h0=h0)
        assert np.array_equal(y2[:, :s], y[:, :s])
        assert not np.array_equal(y2[:, s], y[:, s])


def test_channel_permutation_and_batch_independence():
    batch, L, dim, N = 3, 25, 6, 4
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(14, batch, L, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    p = np.random.default_rng(0).permutation(dim)
    yp, hp = oracle.fwd(u[..., p], delta[..., p], A[p], Bm, Cm, D[p], z[..., p], bias[p], True,
                        h0=h0[:, p])
    assert np.array_equal(yp, y[..., p]) and np.array_equal(hp, hL[:, p])
    for b in range(batch):
        sl = slice(b, b + 1)
        yb, hb = oracle.fwd(u[sl], delta[sl], A, Bm[sl], Cm[sl], D, z[sl], bias, True, h0=h0[sl])
        assert np.array_equal(yb, y[sl]) and np.array_equal(hb, hL[sl])


def test_linearity_in_u():
    batch, L, dim, N = 1, 32, 3, 5
    _, delta, A, Bm, Cm, D, _, bias, _ = rng_inputs(15, batch, L, dim, N)
    rng = np.random.default_rng(16)
    # multiples of 1/8 in a small range: sums and doublings are exact in fp32
    u1 = (rng.integers(-16, 16, size=(batch, L, dim)) / 8.0).astype(np.float32)
    u2 = (rng.integers(-16, 16, size=(batch, L, dim)) / 8.0).astype(np.float32)
    y1, h1 = oracle.fwd(u1, delta, A, Bm, Cm, D, None, bias, True)
    y2, h2 = oracle.fwd(u2, delta, A, Bm, Cm, D, None, bias, True)
    y3, h3 = oracle.fwd(2 * u1 + u2, delta, A, Bm, Cm, D, None, bias, True)
    assert rel(y3, 2 * y1 + y2) < 1e-13
    assert rel(h3, 2 * h1 + h2) < 1e-13


def test_oracle_regression_fixture():
    """Frozen oracle output on one tiny seeded case (tests/golden/oracle_tiny.json,
    written by tests/golden/make_golden.py from the oracle alone)."""
    import json
    import os

    import selscan_inputs as si
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    with open(path) as f:
        g = json.load(f)
    inp = si.make_fwd_inputs(**g["case"])
    y, h = oracle.fwd_inputs(inp, threads=1)
    assert np.max(np.abs(y.ravel() - np.array(g["y"]))) <= 1e-15 * np.max(np.abs(g["y"]))
    assert np.max(np.abs(h.ravel() - np.array(g["h_last"]))) <= 1e-15 * np.max(np.abs(g["h_last"]))


# ----------------------------------------------------------------------------
# Variants: exact zero-order hold, reverse direction, conv1d + SiLU prologue
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("with_h0", [False, True])
def test_zoh_exact_lti_equals_convolution(with_h0):
    """Exact ZOH (tutorial §2.2): B_bar = (exp(Delta A) - 1) / A * B.  In the
    LTI case y is the convolution with K_k = C A_bar^k B_bar (tutorial §2.3)."""
    batch, L, dim, N = 1, 40, 3, 4
    u, _, A, _, _, D, _, bias, h0 = rng_inputs(31, batch, L, dim, N)
    rng = np.random.default_rng(32)
    c = rng.uniform(-1.0, 2.0, size=(batch, 1, dim)).astype(np.float32)
    delta = np.broadcast_to(c, (batch, L, dim)).copy()
    Bv = rng.standard_normal((batch, 1, N)).astype(np.float32)
    Cv = rng.standard_normal((batch, 1, N)).astype(np.float32)
    Bm = np.broadcast_to(Bv, (batch, L, N)).copy()
    Cm = np.broadcast_to(Cv, (batch, L, N)).copy()
    y, _ = oracle.fwd(u, delta, A, Bm, Cm, D, None, bias, True, h0=h0 if with_h0 else None,
                      flags=oracle.ZOH_EXACT)
    dt = softplus_lib(c[0, 0].astype(np.float64) + bias)
    expect = np.zeros((batch, L, dim))
    for d in range(dim):
        An = A[d].astype(np.float64)
        Abar = np.exp(dt[d] * An)
        Bbar = (Abar - 1.0) / An * Bv[0, 0].astype(np.float64)       # textbook ZOH
        Cb = Cv[0, 0].astype(np.float64)
        K = np.array([np.sum(Cb * Abar ** k * Bbar) for k in range(L)])
        for t in range(L):
            acc = sum(K[k] * float(u[0, t - k, d]) for k in range(t + 1))
            if with_h0:
                acc += np.sum(Cb * Abar ** (t + 1) * h0[0, d].astype(np.float64))
            expect[0, t, d] = acc + float(D[d]) * float(u[0, t, d])
    assert rel(y, expect) < 1e-11


def test_zoh_exact_small_A_tends_to_euler():
    batch, L, dim, N = 2, 30, 3, 4
    u, delta, _, Bm, Cm, D, z, bias, h0 = rng_inputs(33, batch, L, dim, N)
    A = np.full((dim, N), -1e-9, np.float32)
    y1, h1 = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0, flags=oracle.ZOH_EXACT)
    y2, h2 = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    assert rel(y1, y2) < 1e-7 and rel(h1, h2) < 1e-7
    # and for larger |Delta A| the two discretisations differ
    A2 = np.full((dim, N), -2.0, np.float32)
    y3, _ = oracle.fwd(u, delta, A2, Bm, Cm, D, z, bias, True, flags=oracle.ZOH_EXACT)
    y4, _ = oracle.fwd(u, delta, A2, Bm, Cm, D, z, bias, True)
    assert rel(y3, y4) > 1e-3


def test_reverse_equals_suffix_closed_form():
    """Reverse direction: h_t = A_bar_t h_{t+1} + Delta_t B_t u_t, whose closed
    form is h_t = sum_{s>=t} exp(A sum_{k=t}^{s-1} Delta_k) Delta_s B_s u_s
    + exp(A sum_{k>=t} Delta_k) h0."""
    batch, L, dim, N = 1, 30, 3, 5
    u, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(34, batch, L, dim, N)
    y, hL = oracle.fwd(u, delta, A, Bm, Cm, D, z, bias, True, h0=h0, flags=oracle.REVERSE)
    dt = softplus_lib(delta.astype(np.float64) + bias)[0]          # (L, dim)
    ey = np.zeros((L, dim))
    eh = np.zeros((dim, N))
    for d in range(dim):
        An = A[d].astype(np.float64)
        for t in range(L):
            h = np.exp(An * dt[t:, d].sum()) * h0[0, d].astype(np.float64)
            for s_ in range(t, L):
                h = h + np.exp(An * dt[t:s_, d].sum()) * dt[s_, d] \
                    * Bm[0, s_].astype(np.float64) * float(u[0, s_, d])
            ey[t, d] = (np.dot(Cm[0, t].astype(np.float64), h) + float(D[d]) * float(u[0, t, d])) \
                * silu_lib(float(z[0, t, d]))
            if t == 0:
                eh[d] = h
    assert rel(y[0], ey) < 1e-11
    assert rel(hL[0], eh) < 1e-11


def conv_lib(x, w, b):
    """Causal depthwise conv1d + SiLU with torch (fp64, CPU): Conv1d with
    groups = channels and padding k-1, first L outputs (tutorial §4.2)."""
    import torch
    L = x.shape[1]
    xt = torch.from_numpy(x.astype(np.float64)).transpose(1, 2)            # (b, d, L)
    wt = torch.from_numpy(w.astype(np.float64))[:, None, :]                 # (d, 1, k)
    bt = None if b is None else torch.from_numpy(b.astype(np.float64))
    out = torch.nn.functional.conv1d(xt, wt, bt, padding=w.shape[1] - 1, groups=w.shape[0])
    out = out[..., :L].transpose(1, 2).numpy()
    return out * expit(out)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_conv_prologue_matches_torch_conv1d(k):
    """With B = 0 only the skip path remains: y = D * u_conv * SiLU(z), where
    u_conv is torch's causal depthwise conv1d followed by SiLU."""
    batch, L, dim, N = 2, 17, 5, 4
    x, delta, A, Bm, Cm, D, z, bias, _ = rng_inputs(40 + k, batch, L, dim, N)
    rng = np.random.default_rng(50 + k)
    w = rng.standard_normal((dim, k)).astype(np.float32)
    cb = rng.standard_normal(dim).astype(np.float32)
    y, _ = oracle.fwd(x, delta, A, np.zeros_like(Bm), Cm, D, z, bias, True, conv_w=w, conv_b=cb)
    uc = conv_lib(x, w, cb)
    ey = D.astype(np.float64) * uc * silu_lib(z)
    assert rel(y, ey) < 1e-13


def test_conv_prologue_then_scan():
    """The conv output feeds the scan exactly like a precomputed u."""
    batch, L, dim, N = 2, 25, 4, 6
    x, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(60, batch, L, dim, N)
    rng = np.random.default_rng(61)
    w = rng.standard_normal((dim, 4)).astype(np.float32)
    y, hL = oracle.fwd(x, delta, A, Bm, Cm, D, z, bias, True, h0=h0, conv_w=w)
    uc = conv_lib(x, w, None).astype(np.float32)                            # rounded to fp32
    y2, h2 = oracle.fwd(uc, delta, A, Bm, Cm, D, z, bias, True, h0=h0)
    assert rel(y, y2) < 1e-6 and rel(hL, h2) < 1e-6


@pytest.mark.parametrize("flags", [0, 1])
def test_reverse_is_forward_on_flipped_sequence(flags):
    """REVERSE computes the forward (conv prologue included) on the
    time-reversed sequence and returns it in the original order."""
    batch, L, dim, N = 2, 23, 4, 5
    x, delta, A, Bm, Cm, D, z, bias, h0 = rng_inputs(62, batch, L, dim, N)
    w = np.random.default_rng(63).standard_normal((dim, 3)).astype(np.float32)
    f = lambda a: np.ascontiguousarray(a[:, ::-1])
    y, hL = oracle.fwd(x, delta, A, Bm, Cm, D, z, bias, True, h0=h0, conv_w=w,
                       flags=flags | oracle.REVERSE)
    yf, hf = oracle.fwd(f(x), f(delta), A, f(Bm), f(Cm), D, f(z), bias, True, h0=h0, conv_w=w,
                        flags=flags)
    assert np.array_equal(y, f(yf)) and np.array_equal(hL, hf)
