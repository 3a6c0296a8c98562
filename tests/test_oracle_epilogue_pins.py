"""Pins of oracle.epilogue (gated RMS normalisation, depthwise causal conv1d)
against things other than itself: closed forms, invariances, and library
routines that implement the same operation independently (numpy.convolve,
scipy.special.expit). CPU only.

Mistakes each group of pins is there to catch: a flipped convolution kernel
(impulse response, numpy.convolve), a missing or doubled bias, padding on the
wrong side (causality), a state that is not the last K-1 tokens (split /
resume, decode chain), gating before normalising, normalising over the wrong
axis or group (constant-per-group inputs, per-head vs whole-vector), a wrong
SiLU (expit form, zero gate)."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import epilogue as ep


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ gated RMSNorm

def test_silu_against_expit():
    z = np.linspace(-60.0, 60.0, 2001)
    np.testing.assert_allclose(ep.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert ep.silu(np.array([0.0]))[0] == 0.0


def test_gated_norm_constant_rows_closed_form():
    # y constant c inside each group: rmsnorm(y) = c / sqrt(c^2 + eps) exactly
    r = rng(1)
    T, H, P, eps = 5, 3, 8, 1e-3
    c = r.normal(size=(T, H, 1))
    y = np.broadcast_to(c, (T, H, P)).reshape(T, H * P)
    z = r.normal(size=(T, H * P)) * 3
    w = r.normal(size=H * P)
    got = ep.gated_rmsnorm(y, z, w, group=P, eps=eps)
    want = (np.broadcast_to(c / np.sqrt(c * c + eps), (T, H, P)).reshape(T, H * P)
            * w * z * expit(z))
    np.testing.assert_allclose(got, want, rtol=1e-13)


def test_gated_norm_unit_rms_and_scale_invariance():
    r = rng(2)
    T, D, eps = 7, 48, 1e-5
    y = r.normal(size=(T, D)) * 0.7
    w = np.ones(D)
    z = np.full((T, D), 40.0)            # silu(40) = 40 (1 - ~4e-18): the gate is a constant 40
    out = ep.gated_rmsnorm(y, z, w, group=D, eps=eps) / 40.0
    ms = np.mean(y * y, axis=1)
    np.testing.assert_allclose(np.mean(out * out, axis=1), ms / (ms + eps), rtol=1e-13)
    # eps = 0: the normalisation does not see a positive rescaling of y
    z2 = r.normal(size=(T, D))
    a = ep.gated_rmsnorm(y, z2, w, group=D, eps=0.0)
    b = ep.gated_rmsnorm(3.75 * y, z2, w, group=D, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_gated_norm_groups():
    r = rng(3)
    T, H, P, eps = 4, 4, 16, 1e-4
    y = r.normal(size=(T, H * P))
    z, w = r.normal(size=(T, H * P)), r.normal(size=H * P)
    # each head normalised alone equals the per-head grouping
    per_head = ep.gated_rmsnorm(y, z, w, group=P, eps=eps)
    for h in range(H):
        sl = slice(h * P, (h + 1) * P)
        np.testing.assert_allclose(per_head[:, sl], ep.gated_rmsnorm(y[:, sl], z[:, sl], w[sl], P, eps),
                                   rtol=1e-14)
    # with every head holding the same values, whole-vector and per-head agree
    y_rep = np.tile(y[:, :P], (1, H))
    np.testing.assert_allclose(ep.gated_rmsnorm(y_rep, z, w, H * P, eps),
                               ep.gated_rmsnorm(y_rep, z, w, P, eps), rtol=1e-13)
    # ... and differ otherwise (the group axis matters)
    assert not np.allclose(ep.gated_rmsnorm(y, z, w, H * P, eps), per_head, rtol=1e-3)


def test_gated_norm_gate_after_norm():
    # gating before normalising would make the output independent of the
    # gate's scale; here doubling z's magnitude region changes it as silu does
    r = rng(4)
    T, D = 3, 32
    y = r.normal(size=(T, D))
    w = r.normal(size=D)
    z = np.zeros((T, D))
    assert np.all(ep.gated_rmsnorm(y, z, w, D, 1e-5) == 0.0)
    z1 = np.full((T, D), 1.5)
    z2 = np.full((T, D), 3.0)
    ratio = ep.gated_rmsnorm(y, z2, w, D, 1e-5) / ep.gated_rmsnorm(y, z1, w, D, 1e-5)
    np.testing.assert_allclose(ratio, (3.0 * expit(3.0)) / (1.5 * expit(1.5)), rtol=1e-13)


def test_gated_norm_bad_shapes():
    with pytest.raises(ValueError):
        ep.gated_rmsnorm(np.zeros((2, 10)), np.zeros((2, 10)), np.zeros(10), group=4, eps=1e-5)


# ------------------------------------------------------------ causal conv1d

def test_conv_impulse_response():
    # bias 0, no activation: a unit impulse at token t0 in channel c comes out
    # as w[c, K-1], w[c, K-2], ..., w[c, 0] at tokens t0, t0+1, ..., t0+K-1
    r = rng(10)
    b, T, C, K = 1, 12, 3, 4
    w = r.normal(size=(C, K))
    for c in range(C):
        x = np.zeros((b, T, C))
        x[0, 5, c] = 1.0
        out, _ = ep.causal_conv1d(x, w, None, None, "none")
        want = np.zeros(T)
        want[5:5 + K] = w[c, ::-1]
        assert np.array_equal(out[0, :, c], want)
        others = [cc for cc in range(C) if cc != c]
        assert np.all(out[0, :, others] == 0.0)


def test_conv_against_numpy_convolve():
    r = rng(11)
    b, T, C, K = 2, 37, 5, 4
    x = r.normal(size=(b, T, C))
    w = r.normal(size=(C, K))
    bias = r.normal(size=C)
    out, final = ep.causal_conv1d(x, w, bias, None, "silu")
    for bb in range(b):
        for c in range(C):
            pre = np.convolve(x[bb, :, c], w[c, ::-1])[:T] + bias[c]
            np.testing.assert_allclose(out[bb, :, c], pre * expit(pre), rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(final, x[:, T - (K - 1):, :])


def test_conv_linearity_and_causality():
    r = rng(12)
    b, T, C, K = 1, 20, 4, 3
    x1, x2 = r.normal(size=(b, T, C)), r.normal(size=(b, T, C))
    w = r.normal(size=(C, K))
    o1, _ = ep.causal_conv1d(x1, w, None, None, "none")
    o2, _ = ep.causal_conv1d(x2, w, None, None, "none")
    o12, _ = ep.causal_conv1d(2.0 * x1 - 0.5 * x2, w, None, None, "none")
    np.testing.assert_allclose(o12, 2.0 * o1 - 0.5 * o2, rtol=1e-12, atol=1e-13)
    # changing tokens from t onward leaves outputs before t untouched
    x3 = x1.copy()
    x3[:, 9:, :] += 1.0
    o3, _ = ep.causal_conv1d(x3, w, None, None, "none")
    assert np.array_equal(o3[:, :9], o1[:, :9])
    assert not np.allclose(o3[:, 9], o1[:, 9])


def test_conv_k1_is_elementwise():
    r = rng(13)
    x = r.normal(size=(2, 9, 6))
    w = r.normal(size=(6, 1))
    bias = r.normal(size=6)
    out, final = ep.causal_conv1d(x, w, bias, None, "silu")
    pre = x * w[:, 0] + bias
    np.testing.assert_allclose(out, pre * expit(pre), rtol=1e-13)
    assert final.shape == (2, 0, 6)


def test_conv_split_resume_and_decode_chain():
    r = rng(14)
    b, T, C, K = 2, 23, 7, 4
    x = r.normal(size=(b, T, C))
    w, bias = r.normal(size=(C, K)), r.normal(size=C)
    init = r.normal(size=(b, K - 1, C))
    full, fin = ep.causal_conv1d(x, w, bias, init)
    # two pieces, the first piece's final state carried into the second
    a, fa = ep.causal_conv1d(x[:, :10], w, bias, init)
    bpart, fb = ep.causal_conv1d(x[:, 10:], w, bias, fa)
    assert np.array_equal(np.concatenate([a, bpart], axis=1), full)
    assert np.array_equal(fb, fin)
    # token by token
    st = init.copy()
    outs = []
    for t in range(T):
        o, st = ep.causal_conv1d_update(st, x[:, t], w, bias)
        outs.append(o)
    assert np.array_equal(np.stack(outs, axis=1), full)
    assert np.array_equal(st, fin)


def test_conv_short_sequence_state():
    # T < K - 1: the final state still ends with the T new tokens
    r = rng(15)
    b, C, K = 1, 3, 4
    init = r.normal(size=(b, K - 1, C))
    x = r.normal(size=(b, 2, C))
    _, fin = ep.causal_conv1d(x, r.normal(size=(C, K)), None, init)
    np.testing.assert_array_equal(fin, np.concatenate([init[:, 2:], x], axis=1))
