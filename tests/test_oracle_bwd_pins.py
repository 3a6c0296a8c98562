"""Pins of the backward oracle (oracle.ssd_bwd), on the CPU.

The oracle differentiates the per-token recurrence by hand (reverse sweep).
It is checked here against things it shares no code with:

* torch autograd of the forward written in its quadratic (semiseparable)
  form, y = M x with M_ij = (C_i . B_j) exp(sum_{k=j+1..i} dt_k A) dt_j plus
  the decayed initial state (youngju.dev "Mamba / selective SSM" page,
  section "State Space Dualityの発見"), a different algorithm from the
  recurrence and differentiated by the library;
* central finite differences (Richardson-extrapolated) of the forward oracle
  itself, along random directions, for every input;
* closed forms: dD is a plain sum of dy x; with dy = 0 the gradients follow
  from the decayed dfinal alone; a single token; linearity in (dy, dfinal).

A dropped term, a wrong sign, a missing decay factor or a transposed operand
anywhere in the reverse sweep changes at least one gradient by far more than
these tolerances.
"""
import numpy as np
import pytest

import oracle

NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def _problem(rng, b, T, H, P, N, G, coarse=False):
    """Random inputs; coarse=True rounds them to multiples of 2^-8 so that a
    finite-difference step of 2^-12 or 2^-13 stays exact in float32."""
    def q(a):
        a = np.asarray(a, dtype=np.float64)
        if coarse:
            a = np.round(a * 256.0) / 256.0
        return a.astype(np.float32)
    x = q(rng.standard_normal((b, T, H, P)))
    dt = q(rng.uniform(0.05, 0.6, (b, T, H)))
    A = q(-rng.uniform(0.3, 2.0, H))
    B = q(rng.standard_normal((b, T, G, N)) * 0.5)
    C = q(rng.standard_normal((b, T, G, N)) * 0.5)
    D = q(rng.standard_normal(H))
    init = rng.standard_normal((b, H, N, P))
    dy = q(rng.standard_normal((b, T, H, P)))
    dfinal = rng.standard_normal((b, H, N, P))
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init=init, dy=dy, dfinal=dfinal)


def _close(got, ref, tol=1e-10):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = max(float(np.max(np.abs(ref))), 1e-300)
    err = float(np.max(np.abs(got - ref))) / den
    assert err <= tol, err


def _torch_quadratic_grads(pr, G):
    """Autograd of the quadratic form, fp64."""
    import torch
    t = {k: torch.tensor(np.asarray(pr[k], np.float64), requires_grad=True)
         for k in ("x", "dt", "A", "B", "C", "D", "init")}
    x, dt, A, B, C, D, init = (t[k] for k in ("x", "dt", "A", "B", "C", "D", "init"))
    b, T, H, P = x.shape
    hg = torch.arange(H) // (H // G)                     # group of each head
    Bh, Ch = B[:, :, hg, :], C[:, :, hg, :]              # [b,T,H,N]
    cs = torch.cumsum(dt * A, dim=1)                     # [b,T,H]
    seg = cs[:, :, None, :] - cs[:, None, :, :]          # [b,i,j,H] = cs_i - cs_j
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))[None, :, :, None]
    L = torch.exp(torch.where(causal, seg, torch.full_like(seg, -torch.inf)))
    CB = torch.einsum("bihn,bjhn->bijh", Ch, Bh)
    M = CB * L * dt[:, None, :, :]                       # [b,i,j,H]
    y = torch.einsum("bijh,bjhp->bihp", M, x)
    y = y + torch.exp(cs)[..., None] * torch.einsum("bihn,bhnp->bihp", Ch, init)
    y = y + D[None, None, :, None] * x
    wlast = torch.exp(cs[:, -1:, :] - cs) * dt           # [b,T,H]
    fin = torch.einsum("bjh,bjhn,bjhp->bhnp", wlast, Bh, x)
    fin = fin + torch.exp(cs[:, -1, :])[:, :, None, None] * init
    loss = (y * torch.tensor(np.asarray(pr["dy"], np.float64))).sum() + \
           (fin * torch.tensor(pr["dfinal"])).sum()
    loss.backward()
    g = {("d" + k if k != "init" else "dinit"): t[k].grad.numpy() for k in t}
    return g


@pytest.mark.parametrize("b,T,H,P,N,G", [(1, 1, 1, 1, 1, 1), (2, 9, 4, 3, 5, 2), (1, 17, 2, 4, 3, 1),
                                         (2, 6, 6, 2, 4, 3)])
def test_bwd_matches_autograd_of_quadratic_form(b, T, H, P, N, G):
    rng = np.random.default_rng(900 + T + H)
    pr = _problem(rng, b, T, H, P, N, G)
    got = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["D"], pr["init"], pr["dy"],
                         pr["dfinal"])
    ref = _torch_quadratic_grads(pr, G)
    for k in NAMES:
        _close(got[k], ref[k])


def _loss(pr, over=None):
    q = dict(pr)
    if over:
        q.update(over)
    y, fin = oracle.ssd_fwd(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["init"])
    return float(np.sum(y * np.asarray(q["dy"], np.float64)) + np.sum(fin * q["dfinal"]))


def test_bwd_matches_finite_differences_of_forward_oracle():
    rng = np.random.default_rng(950)
    b, T, H, P, N, G = 2, 11, 4, 3, 4, 2
    pr = _problem(rng, b, T, H, P, N, G, coarse=True)
    got = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["D"], pr["init"], pr["dy"],
                         pr["dfinal"])
    for k in ("x", "dt", "A", "B", "C", "D", "init"):
        for trial in range(2):
            v = np.asarray(pr[k])
            d = rng.integers(-1, 2, size=v.shape).astype(np.float64)
            if not np.any(d):
                d.flat[0] = 1.0

            def fd(eps):
                dd = (d * eps).astype(v.dtype)
                assert np.array_equal((v + dd).astype(np.float64) - v.astype(np.float64), d * eps)
                return (_loss(pr, {k: v + dd}) - _loss(pr, {k: v - dd})) / (2 * eps)

            e = 2.0 ** -12
            est = (4 * fd(e / 2) - fd(e)) / 3            # Richardson: error O(eps^4)
            name = "dinit" if k == "init" else "d" + k
            ana = float(np.sum(got[name] * d))
            scale = float(np.sum(np.abs(got[name] * d))) + 1e-30
            assert abs(est - ana) <= 1e-8 * scale, (k, trial, est, ana)


def test_bwd_dD_is_sum_of_dy_times_x_and_D_only_enters_there():
    rng = np.random.default_rng(960)
    pr = _problem(rng, 2, 13, 4, 3, 4, 2)
    g1 = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["D"], pr["init"], pr["dy"],
                        pr["dfinal"])
    ref = np.einsum("bthp,bthp->h", pr["x"].astype(np.float64), pr["dy"].astype(np.float64))
    _close(g1["dD"], ref, 1e-13)
    # D adds D dy to dx and nothing anywhere else
    g0 = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], None, pr["init"], pr["dy"],
                        pr["dfinal"])
    _close(g1["dx"] - g0["dx"], pr["D"][None, None, :, None].astype(np.float64) * pr["dy"], 1e-12)
    for k in ("ddt", "dA", "dB", "dC", "dinit"):
        np.testing.assert_array_equal(g1[k], g0[k])


def test_bwd_from_dfinal_only_closed_form():
    """dy = 0: g_t = exp(A sum_{k>t} dt_k) dfinal, so dinit = exp(A sum dt)
    dfinal and dx_t[p] = dt_t B_t . g_t[:, p]; dC = 0."""
    rng = np.random.default_rng(970)
    b, T, H, P, N, G = 1, 7, 2, 3, 4, 1
    pr = _problem(rng, b, T, H, P, N, G)
    dy = np.zeros_like(pr["dy"])
    g = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["D"], pr["init"], dy, pr["dfinal"])
    dt = pr["dt"].astype(np.float64)
    A = pr["A"].astype(np.float64)
    for h in range(H):
        tot = np.exp(A[h] * dt[0, :, h].sum())
        _close(g["dinit"][0, h], tot * pr["dfinal"][0, h], 1e-13)
        for t in range(T):
            gt = np.exp(A[h] * dt[0, t + 1:, h].sum()) * pr["dfinal"][0, h]        # [N, P]
            _close(g["dx"][0, t, h], dt[0, t, h] * (pr["B"][0, t, 0].astype(np.float64) @ gt), 1e-12)
    np.testing.assert_array_equal(g["dC"], 0.0)
    np.testing.assert_array_equal(g["dD"], 0.0)


def test_bwd_single_token_closed_form():
    """T = 1: y = C.(a init + dt B x) + D x with a = exp(dt A)."""
    rng = np.random.default_rng(980)
    H, P, N = 2, 3, 4
    pr = _problem(rng, 1, 1, H, P, N, 1)
    g = oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["D"], pr["init"], pr["dy"],
                       pr["dfinal"])
    f64 = lambda a: np.asarray(a, np.float64)
    x, dt, A, B, C, D, init, dy, df = (f64(pr[k]) for k in ("x", "dt", "A", "B", "C", "D", "init", "dy",
                                                             "dfinal"))
    for h in range(H):
        a = np.exp(dt[0, 0, h] * A[h])
        s = a * init[0, h] + dt[0, 0, h] * np.outer(B[0, 0, 0], x[0, 0, h])        # [N, P]
        gs = np.outer(C[0, 0, 0], dy[0, 0, h]) + df[0, h]                           # dL/ds
        _close(g["dx"][0, 0, h], dt[0, 0, h] * (B[0, 0, 0] @ gs) + D[h] * dy[0, 0, h], 1e-13)
        _close(g["dinit"][0, h], a * gs, 1e-13)
        dsd = A[h] * a * init[0, h] + np.outer(B[0, 0, 0], x[0, 0, h])              # ds/d dt
        _close(g["ddt"][0, 0, h], np.sum(gs * dsd), 1e-13)
        _close(g["dA"][h], np.sum(gs * dt[0, 0, h] * a * init[0, h]), 1e-13)
    gs_all = [np.outer(C[0, 0, 0], dy[0, 0, h]) + df[0, h] for h in range(H)]
    sv = [np.exp(dt[0, 0, h] * A[h]) * init[0, h] + dt[0, 0, h] * np.outer(B[0, 0, 0], x[0, 0, h])
          for h in range(H)]
    _close(g["dB"][0, 0, 0], sum(dt[0, 0, h] * gs_all[h] @ x[0, 0, h] for h in range(H)), 1e-13)
    _close(g["dC"][0, 0, 0], sum(sv[h] @ dy[0, 0, h] for h in range(H)), 1e-13)


def test_bwd_linear_in_upstream_gradients():
    rng = np.random.default_rng(990)
    pr = _problem(rng, 1, 10, 2, 3, 4, 1, coarse=True)     # dy + 2 dy2 exact in float32
    args = [pr[k] for k in ("x", "dt", "A", "B", "C", "D", "init")]
    dy2 = (np.round(rng.standard_normal(pr["dy"].shape) * 256) / 256).astype(np.float32)
    df2 = rng.standard_normal(pr["dfinal"].shape)
    g1 = oracle.ssd_bwd(*args, pr["dy"], pr["dfinal"])
    g2 = oracle.ssd_bwd(*args, dy2, df2)
    g3 = oracle.ssd_bwd(*args, (pr["dy"].astype(np.float64) + 2 * dy2).astype(np.float32), pr["dfinal"] + 2 * df2)
    for k in NAMES:
        _close(g3[k], g1[k] + 2 * g2[k], 1e-12)


def test_bwd_no_dfinal_equals_zero_dfinal_and_rejects_bad_dims():
    rng = np.random.default_rng(995)
    pr = _problem(rng, 1, 5, 2, 2, 3, 1)
    args = [pr[k] for k in ("x", "dt", "A", "B", "C", "D", "init")]
    a = oracle.ssd_bwd(*args, pr["dy"], None)
    b = oracle.ssd_bwd(*args, pr["dy"], np.zeros_like(pr["dfinal"]))
    for k in NAMES:
        np.testing.assert_array_equal(a[k], b[k])
    with pytest.raises((RuntimeError, AssertionError)):
        oracle.ssd_bwd(pr["x"], pr["dt"], pr["A"][:1], pr["B"], pr["C"], pr["D"], None, pr["dy"])
