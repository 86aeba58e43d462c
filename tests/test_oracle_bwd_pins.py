"""Pins of the oracle's backward (``oracle.bwd``) against two independent
routes to the same derivatives:

* torch autograd (fp64, CPU) through a plain loop of the recurrence built
  from torch's own softplus and SiLU: reverse-mode differentiation by the
  library, not by the oracle's hand-written adjoint recurrence;
* central finite differences of the (separately pinned) oracle forward on
  dyadic inputs, whose perturbed values are exact in fp32, so that the only
  error is the O(eps^2) truncation of the difference quotient.

Both use the loss  sum(dy * y) + sum(dh_last * h_last), whose gradient is
what the backward returns for upstream gradients dy and dh_last.
"""
import numpy as np
import pytest
import torch

import oracle


def rng_case(seed, batch, L, dim, N, dyadic=False):
    rng = np.random.default_rng(seed)
    if dyadic:
        # multiples of 1/64 in a small range: exact in fp32, and x +- 2^-12 too
        g = lambda *s, lo=-64, hi=64: (rng.integers(lo, hi, size=s) / 64.0).astype(np.float32)
        u, delta, Bm, Cm, z = g(batch, L, dim), g(batch, L, dim, lo=-32, hi=32), \
            g(batch, L, N), g(batch, L, N), g(batch, L, dim)
        A = (-(rng.integers(4, 128, size=(dim, N)) / 64.0)).astype(np.float32)
        D = g(dim)
        bias = (-(rng.integers(64, 256, size=dim) / 64.0)).astype(np.float32)
    else:
        f = lambda *s: rng.standard_normal(s).astype(np.float32)
        u, delta, Bm, Cm, z = f(batch, L, dim), (0.5 * f(batch, L, dim)).astype(np.float32), \
            f(batch, L, N), f(batch, L, N), f(batch, L, dim)
        A = (-rng.uniform(0.05, 2.0, size=(dim, N))).astype(np.float32)
        D = f(dim)
        bias = rng.uniform(-4.0, -1.0, size=dim).astype(np.float32)
    h0 = rng.standard_normal((batch, dim, N))
    dy = rng.standard_normal((batch, L, dim)).astype(np.float32)
    dh_last = rng.standard_normal((batch, dim, N))
    return dict(u=u, delta=delta, A=A, Bm=Bm, Cm=Cm, D_skip=D, z=z, delta_bias=bias, h0=h0,
                dy=dy, dh_last=dh_last)


def torch_loop_grads(c, softplus, use):
    """fp64 autograd through a plain loop over t (all channels and states at
    once): h = exp(Delta A) h + Delta B u, y = (C.h + D u) * SiLU(z)."""
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    u, delta, A, Bm, Cm = (T(c[k]) for k in ("u", "delta", "A", "Bm", "Cm"))
    D = T(c["D_skip"]) if use["D"] else None
    z = T(c["z"]) if use["z"] else None
    bias = T(c["delta_bias"]) if use["bias"] else None
    h0 = T(c["h0"]) if use["h0"] else None
    batch, L, dim = u.shape
    N = A.shape[1]
    x = delta + (bias if bias is not None else 0.0)
    dt = torch.nn.functional.softplus(x) if softplus else x
    h = h0 if h0 is not None else torch.zeros((batch, dim, N), dtype=torch.float64)
    ys = []
    for t in range(L):
        abar = torch.exp(dt[:, t, :, None] * A[None])
        h = abar * h + dt[:, t, :, None] * Bm[:, t, None, :] * u[:, t, :, None]
        y = (h * Cm[:, t, None, :]).sum(-1)
        if D is not None:
            y = y + D * u[:, t]
        if z is not None:
            y = y * torch.nn.functional.silu(z[:, t])
        ys.append(y)
    y = torch.stack(ys, 1)
    loss = (y * torch.from_numpy(c["dy"].astype(np.float64))).sum()
    if use["dh_last"]:
        loss = loss + (h * torch.from_numpy(c["dh_last"])).sum()
    loss.backward()
    g = dict(du=u.grad, ddelta=delta.grad, dA=A.grad, dB=Bm.grad, dC=Cm.grad,
             dD=None if D is None else D.grad, dz=None if z is None else z.grad,
             dbias=None if bias is None else bias.grad, dh0=None if h0 is None else h0.grad)
    return {k: (None if v is None else v.numpy()) for k, v in g.items()}


def oracle_grads(c, softplus, use):
    return oracle.bwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"],
                      c["D_skip"] if use["D"] else None, c["z"] if use["z"] else None,
                      c["delta_bias"] if use["bias"] else None, softplus,
                      c["h0"] if use["h0"] else None, c["dh_last"] if use["dh_last"] else None)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


USES = [
    dict(D=True, z=True, bias=True, h0=True, dh_last=True),
    dict(D=False, z=False, bias=False, h0=False, dh_last=False),
    dict(D=True, z=False, bias=True, h0=False, dh_last=True),
    dict(D=False, z=True, bias=False, h0=True, dh_last=False),
]


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("ui", range(len(USES)))
def test_bwd_matches_torch_autograd(softplus, ui):
    use = USES[ui]
    c = rng_case(10 + ui, 2, 9, 5, 4)
    if not softplus:
        # keep Delta = Delta_raw + bias positive without softplus
        c["delta"] = (np.abs(c["delta"]) * 0.2).astype(np.float32)
        c["delta_bias"] = np.full_like(c["delta_bias"], 0.05)
    ref = torch_loop_grads(c, softplus, use)
    got = oracle_grads(c, softplus, use)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0"):
        if ref[k] is None:
            continue
        assert rel(got[k], ref[k]) < 1e-11, k


def test_bwd_gradient_of_absent_inputs():
    """With no h0 the gradient dh0 still exists (the state entering t = 0),
    and dD, dbias are defined even when D, bias are absent (taken as 0)."""
    use = dict(D=True, z=True, bias=True, h0=True, dh_last=True)
    c = rng_case(20, 1, 6, 3, 4)
    c["D_skip"] = np.zeros_like(c["D_skip"])
    c["delta_bias"] = np.zeros_like(c["delta_bias"])
    c["h0"] = np.zeros_like(c["h0"])
    ref = torch_loop_grads(c, True, use)
    got = oracle.bwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], None, c["z"], None,
                     True, None, c["dh_last"])
    for k in ("dD", "dbias", "dh0", "du", "dA"):
        assert rel(got[k], ref[k]) < 1e-11, k


def fd_loss(c, softplus):
    y, hL = oracle.fwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["D_skip"], c["z"],
                       c["delta_bias"], softplus, c["h0"])
    return float(np.sum(y * c["dy"].astype(np.float64)) + np.sum(hL * c["dh_last"]))


@pytest.mark.parametrize("softplus", [True, False])
def test_bwd_central_differences(softplus):
    c = rng_case(30, 2, 6, 3, 4, dyadic=True)
    if not softplus:
        c["delta"] = (np.abs(c["delta"]) / 8.0).astype(np.float32)
        c["delta_bias"] = np.full_like(c["delta_bias"], 1.0 / 16.0)
    use = dict(D=True, z=True, bias=True, h0=True, dh_last=True)
    g = oracle_grads(c, softplus, use)
    eps = 2.0 ** -12
    rng = np.random.default_rng(31)
    names = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "D_skip": "dD",
             "z": "dz", "delta_bias": "dbias", "h0": "dh0"}
    for key, gk in names.items():
        arr = c[key]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            base = arr[idx]
            arr[idx] = base + eps
            lp = fd_loss(c, softplus)
            arr[idx] = base - eps
            lm = fd_loss(c, softplus)
            arr[idx] = base
            assert arr[idx] == base
            fd = (lp - lm) / (2 * eps)
            scale = max(1.0, float(np.max(np.abs(g[gk]))))
            assert abs(fd - g[gk][idx]) < 2e-6 * scale, (key, idx, fd, g[gk][idx])


# ----------------------------------------------------------------------------
# Backward of the variants: exact ZOH, reverse direction, conv1d + SiLU prologue
# ----------------------------------------------------------------------------
def torch_loop_variant_grads(c, softplus, zoh, rev, conv):
    """fp64 autograd through a plain loop of the variant forward: the conv
    prologue by torch's grouped conv1d (padding k-1, first L outputs) then
    SiLU, the reverse direction by flipping the time axis of every per-step
    input and of y, exact ZOH by expm1(Delta A) / A."""
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, delta, A, Bm, Cm, D, z, bias, h0 = (T(c[k]) for k in ("u", "delta", "A", "Bm", "Cm",
                                                             "D_skip", "z", "delta_bias", "h0"))
    cw = T(c["conv_w"]) if conv else None
    cb = T(c["conv_b"]) if conv else None
    batch, L, dim = x.shape
    N = A.shape[1]
    f = (lambda a: a.flip(1)) if rev else (lambda a: a)
    xs, ds, Bs, Cs, zs = f(x), f(delta), f(Bm), f(Cm), f(z)
    if conv:
        k = cw.shape[1]
        acc = torch.nn.functional.conv1d(xs.transpose(1, 2), cw[:, None, :], cb,
                                         padding=k - 1, groups=dim)[..., :L].transpose(1, 2)
        us = torch.nn.functional.silu(acc)
    else:
        us = xs
    xx = ds + bias
    dt = torch.nn.functional.softplus(xx) if softplus else xx
    h = h0
    ys = []
    for t in range(L):
        dA_ = dt[:, t, :, None] * A[None]
        abar = torch.exp(dA_)
        coef = torch.expm1(dA_) / A[None] if zoh else dt[:, t, :, None]
        h = abar * h + coef * Bs[:, t, None, :] * us[:, t, :, None]
        y = ((h * Cs[:, t, None, :]).sum(-1) + D * us[:, t]) * torch.nn.functional.silu(zs[:, t])
        ys.append(y)
    y = f(torch.stack(ys, 1))
    loss = (y * torch.from_numpy(c["dy"].astype(np.float64))).sum() + \
        (h * torch.from_numpy(c["dh_last"])).sum()
    loss.backward()
    g = dict(du=x.grad, ddelta=delta.grad, dA=A.grad, dB=Bm.grad, dC=Cm.grad, dD=D.grad,
             dz=z.grad, dbias=bias.grad, dh0=h0.grad,
             dconv_w=None if cw is None else cw.grad, dconv_b=None if cb is None else cb.grad)
    return {k: (None if v is None else v.numpy()) for k, v in g.items()}


def variant_case(seed, batch, L, dim, N, k):
    c = rng_case(seed, batch, L, dim, N)
    rng = np.random.default_rng(seed + 1)
    c["conv_w"] = rng.uniform(-0.5, 0.5, size=(dim, k)).astype(np.float32)
    c["conv_b"] = rng.uniform(-0.5, 0.5, size=dim).astype(np.float32)
    return c


VARIANTS = [(False, True, False), (True, False, False), (False, False, True),
            (True, True, True), (True, True, False)]


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("zoh,rev,conv", VARIANTS)
def test_bwd_variants_match_torch_autograd(zoh, rev, conv, softplus):
    c = variant_case(70, 2, 9, 4, 4, 3)
    if not softplus:
        c["delta"] = (np.abs(c["delta"]) * 0.2).astype(np.float32)
        c["delta_bias"] = np.full_like(c["delta_bias"], 0.05)
    ref = torch_loop_variant_grads(c, softplus, zoh, rev, conv)
    flags = (oracle.ZOH_EXACT if zoh else 0) | (oracle.REVERSE if rev else 0)
    got = oracle.bwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], c["D_skip"], c["z"],
                     c["delta_bias"], softplus, c["h0"], c["dh_last"], flags=flags,
                     conv_w=c["conv_w"] if conv else None, conv_b=c["conv_b"] if conv else None)
    for key in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0", "dconv_w",
                "dconv_b"):
        if ref[key] is None:
            assert got[key] is None
            continue
        assert rel(got[key], ref[key]) < 1e-10, key


def test_bwd_zoh_small_A_limit():
    """For |Delta A| -> 0 the exact-ZOH gradients tend to the Euler ones, and
    the dA of the coefficient (a series there) stays finite."""
    c = rng_case(80, 1, 7, 3, 4)
    c["A"] = np.full_like(c["A"], -1e-7)
    args = (c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], c["D_skip"], c["z"],
            c["delta_bias"], True, c["h0"], c["dh_last"])
    gz = oracle.bwd(*args, flags=oracle.ZOH_EXACT)
    ge = oracle.bwd(*args)
    for key in ("du", "ddelta", "dB", "dC", "dz", "dh0"):
        assert rel(gz[key], ge[key]) < 1e-5, key
    # dA differs by sum lambda B u d(coef)/dA = Delta^2/2 * ... : finite and small
    assert np.all(np.isfinite(gz["dA"]))


@pytest.mark.parametrize("zoh,rev,conv", [(True, True, True), (False, True, True)])
def test_bwd_variants_central_differences(zoh, rev, conv):
    c = rng_case(90, 2, 6, 3, 4, dyadic=True)
    rng = np.random.default_rng(91)
    c["conv_w"] = (rng.integers(-32, 32, size=(3, 4)) / 64.0).astype(np.float32)
    c["conv_b"] = (rng.integers(-32, 32, size=3) / 64.0).astype(np.float32)
    flags = (oracle.ZOH_EXACT if zoh else 0) | (oracle.REVERSE if rev else 0)
    g = oracle.bwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["dy"], c["D_skip"], c["z"],
                   c["delta_bias"], True, c["h0"], c["dh_last"], flags=flags,
                   conv_w=c["conv_w"], conv_b=c["conv_b"])

    def loss():
        y, hL = oracle.fwd(c["u"], c["delta"], c["A"], c["Bm"], c["Cm"], c["D_skip"], c["z"],
                           c["delta_bias"], True, c["h0"], flags=flags, conv_w=c["conv_w"],
                           conv_b=c["conv_b"])
        return float(np.sum(y * c["dy"].astype(np.float64)) + np.sum(hL * c["dh_last"]))

    eps = 2.0 ** -12
    names = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "conv_w": "dconv_w",
             "conv_b": "dconv_b", "h0": "dh0"}
    for key, gk in names.items():
        arr = c[key]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            base = arr[idx]
            arr[idx] = base + eps
            lp = loss()
            arr[idx] = base - eps
            lm = loss()
            arr[idx] = base
            fd = (lp - lm) / (2 * eps)
            scale = max(1.0, float(np.max(np.abs(g[gk]))))
            assert abs(fd - g[gk][idx]) < 2e-6 * scale, (key, idx, fd, g[gk][idx])
