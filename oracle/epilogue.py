"""fp64 CPU oracle of the two element-wise stages around the SSD layer core.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it; the GPU
library never calls it and it imports nothing from the GPU package.

Both are written out as their definitions, in double precision, with numpy
arrays as the only machinery.

Gated RMS normalisation (Qiita "Mamba-2" article, section 4.2, SSD block step
4: the SSD output y is RMS-normalised and multiplied by SiLU of the gate
branch z, ``rmsnorm(y) * silu(z)``). Readings taken where the page is silent:
the normalisation runs over groups of ``group`` consecutive channels of the
feature vector (``group = H*P``, the whole vector, is the page's plain
reading; ``group = P`` normalises each head), with a learnable per-channel
weight and no bias (the RMSNorm modules in the pages' code are
``nn.RMSNorm(d)``), ``eps`` given by the caller, normalisation first and the
gate after it (the page's order), ``silu(z) = z / (1 + exp(-z))``.

    out[t, c] = y[t, c] / sqrt(mean_{c' in group(c)} y[t, c']^2 + eps)
                * w[c] * silu(z[t, c])

Depthwise causal convolution (youngju.dev "Mamba / selective SSM" page, the
Mamba block code: ``nn.Conv1d(d, d, kernel_size=d_conv, padding=d_conv - 1,
groups=d, bias=True)`` followed by a trim to the first L outputs and SiLU;
the same block in the waylandz LLM book, chapter 32). A PyTorch Conv1d is a
cross-correlation, so with the K - 1 zeros of left padding the trimmed output
at token t is

    out[t, c] = act(bias[c] + sum_{k=0..K-1} w[c, k] * x[t - (K-1) + k, c])

with x = 0 before token 0. Readings: channels-last layout ``[b, T, C]`` (the
layer's activations are token-major); ``act`` is SiLU or the identity; the
K - 1 tokens before token 0 may be given as a state ``[b, K-1, C]`` (zeros
otherwise) and the last K - 1 tokens of the padded sequence are returned as the
final state, so that a sequence processed in pieces, or token by token (the
recurrent decode form), gives the same outputs as one call.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(z) -> np.ndarray:
    """z / (1 + exp(-z)) in double precision."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gated_rmsnorm(y, z, w, group: int, eps: float) -> np.ndarray:
    """out = y / sqrt(mean over the channel group of y^2 + eps) * w * silu(z).

    y, z: [..., D] (any leading shape), w: [D]; D % group == 0.
    Returns float64 of y's shape.
    """
    y, z, w = _f64(y), _f64(z), _f64(w)
    D = y.shape[-1]
    if group <= 0 or D % group or z.shape != y.shape or w.shape != (D,):
        raise ValueError("bad shapes for gated_rmsnorm")
    yg = y.reshape(y.shape[:-1] + (D // group, group))
    ms = np.mean(yg * yg, axis=-1, keepdims=True)            # mean square per group
    normed = (yg / np.sqrt(ms + float(eps))).reshape(y.shape)
    return normed * w * silu(z)


def causal_conv1d(x, w, bias=None, init=None, activation: str = "silu"):
    """Depthwise causal convolution over tokens, channels last.

    x: [b, T, C]; w: [C, K]; bias: [C] or None; init: [b, K-1, C] or None (the
    K-1 tokens before token 0; zeros when None). Returns (out [b, T, C],
    final [b, K-1, C]) in float64: out as defined in the module docstring,
    final = the last K-1 tokens of (init, x).
    """
    x, w = _f64(x), _f64(w)
    b, T, C = x.shape
    K = w.shape[1]
    if w.shape != (C, K) or K < 1:
        raise ValueError("bad weight shape")
    prev = np.zeros((b, K - 1, C)) if init is None else _f64(init)
    if prev.shape != (b, K - 1, C):
        raise ValueError("bad init shape")
    xp = np.concatenate([prev, x], axis=1)                   # token t of x at xp[:, t + K - 1]
    acc = np.zeros((b, T, C)) if bias is None else np.broadcast_to(_f64(bias), (b, T, C)).copy()
    for k in range(K):                                       # k = 0 .. K-1, in order
        acc = acc + w[:, k] * xp[:, k:k + T, :]              # x[t - (K-1) + k] = xp[t + k]
    if activation == "silu":
        out = silu(acc)
    elif activation == "none":
        out = acc
    else:
        raise ValueError(activation)
    final = xp[:, T:, :].copy()                               # the last K-1 tokens
    return out, final


def causal_conv1d_update(state, x, w, bias=None, activation: str = "silu"):
    """One token of the same convolution in recurrent form.

    state: [b, K-1, C] (the K-1 previous tokens, oldest first); x: [b, C].
    Returns (out [b, C], new_state [b, K-1, C]) in float64.
    """
    state, x = _f64(state), _f64(x)
    out, new_state = causal_conv1d(x[:, None, :], w, bias, state, activation)
    return out[:, 0, :], new_state
