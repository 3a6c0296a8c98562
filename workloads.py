"""Seeded synthetic workloads for the SSD layer core.

This module only draws inputs. It holds none of the SSD arithmetic and is the
one piece of code that both the GPU path's tests/bench and the CPU oracle
consume. Every array it returns is float32 holding the *exact* value the
device receives: on bf16 workloads each value has already been rounded to
bf16 (round-to-nearest-even), so widening it to fp64 on the host loses
nothing.

Distributions (the selective-SSM parametrisation on the youngju.dev
"Mamba / selective SSM" page, section on switching from LTI to selection:
dt comes out of a softplus; Qiita "Mamba-2" article, section 4.2: A is a
negative scalar per head, A = -exp(A_log)):

    x      ~ N(0, 1)
    dt     = clamp(softplus(N(0,1) - 4), 1e-3, 0.1)   (long-context workload:
             dt = exp(U(ln 1e-4, ln 1e-1)), no clamp; fast-decay test cases:
             dt = exp(U(ln 1e-2, ln 2)), so dt |A| reaches 32 per token)
    A_h    = -exp(U(0, ln 16))                       in [-16, -1]
    B, C   ~ N(0, 1) / sqrt(N)
    D_h    ~ N(0, 1)
    init   = 0, or N(0, 0.1) (std 0.1) fp32 where the workload asks for it

Draw order for a forward workload is x, dt, A, B, C, D, init; the generator is
numpy's PCG64 ``default_rng(seed)``. Normal draws use numpy's float32
ziggurat (``standard_normal(dtype=float32)``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# bf16 carriers
# --------------------------------------------------------------------------

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as
    float32 carriers. NaN/Inf never occur in these workloads."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The 16-bit patterns of float32 carriers that already hold bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class FwdWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    dtype: str                 # "f32" or "bf16": dtype of x, dt, B, C, y
    dt_mode: str = "softplus"  # "softplus" (clamped), "loguniform" or "fast"
    init: str = "zero"         # "zero" or "normal0.1"
    seed: int = 0
    tag: str = ""              # short name (profile summaries are named by it)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    steps: int
    dtype: str = "bf16"
    seed: int = 0


# The five named workloads (shapes and distributions of the method's layer
# sizes: a tiny fp32 case, a 130M-shaped layer, a 2.7B-shaped layer with a
# nonzero initial state, a 128K-token long-context case, and a decode batch).
TINY_F32 = FwdWorkload("tiny_f32_b1_T256_H2_P16_N16_Q64", 1, 256, 2, 16, 16, 1, 64,
                       "f32", seed=4600, tag="tiny_f32")
MAMBA2_130M = FwdWorkload("mamba2_130m_b8_T2048_H24_P64_N128_Q256", 8, 2048, 24, 64, 128, 1, 256,
                          "bf16", seed=4601, tag="mamba2_130m")
MAMBA2_2P7B = FwdWorkload("mamba2_2p7b_b4_T4096_H80_P64_N128_Q256_init", 4, 4096, 80, 64, 128, 1, 256,
                          "bf16", init="normal0.1", seed=4602, tag="mamba2_2p7b")
LONG_128K = FwdWorkload("long_b1_T131072_H24_P64_N256_Q256", 1, 131072, 24, 64, 256, 1, 256,
                        "bf16", dt_mode="loguniform", seed=4603, tag="long_128k")
DECODE_B256 = DecodeWorkload("decode_b256_H128_P64_N128_G8_64steps", 256, 128, 64, 128, 8, 64,
                             "bf16", seed=4604)

FWD_WORKLOADS = {w.name: w for w in (TINY_F32, MAMBA2_130M, MAMBA2_2P7B, LONG_128K)}


def with_shape(w: FwdWorkload, **kw) -> FwdWorkload:
    """A variant of w (a different shape is no longer the named workload, so
    its tag is dropped unless given)."""
    kw.setdefault("tag", "")
    return dataclasses.replace(w, **kw)


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def _softplus(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float64)
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_to_bf16(a) if dtype == "bf16" else a


def draw_dt(rng: np.random.Generator, shape, mode: str) -> np.ndarray:
    if mode == "softplus":
        v = rng.standard_normal(shape, dtype=np.float32).astype(np.float64) - 4.0
        return np.clip(_softplus(v), 1e-3, 0.1).astype(np.float32)
    if mode == "loguniform":
        u = rng.uniform(math.log(1e-4), math.log(1e-1), size=shape)
        return np.exp(u).astype(np.float32)
    if mode == "fast":
        u = rng.uniform(math.log(1e-2), math.log(2.0), size=shape)
        return np.exp(u).astype(np.float32)
    raise ValueError(mode)


def draw_A(rng: np.random.Generator, nheads: int) -> np.ndarray:
    return (-np.exp(rng.uniform(0.0, math.log(16.0), size=nheads))).astype(np.float32)


def make_fwd_inputs(w: FwdWorkload, seed: Optional[int] = None) -> dict:
    """Inputs of one forward call, all float32 carriers of the stored values.

    x [b,T,H,P], dt [b,T,H], A [H], B/C [b,T,G,N], D [H], init [b,H,N,P] or None.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = _store(rng.standard_normal((b, T, H, P), dtype=np.float32), w.dtype)
    dt = _store(draw_dt(rng, (b, T, H), w.dt_mode), w.dtype)
    A = draw_A(rng, H)
    s = np.float32(1.0 / math.sqrt(N))
    B = _store(rng.standard_normal((b, T, G, N), dtype=np.float32) * s, w.dtype)
    C = _store(rng.standard_normal((b, T, G, N), dtype=np.float32) * s, w.dtype)
    D = rng.standard_normal(H, dtype=np.float32)
    init = None
    if w.init == "normal0.1":
        init = (rng.standard_normal((b, H, N, P), dtype=np.float32) * np.float32(0.1))
    elif w.init != "zero":
        raise ValueError(w.init)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init=init)


def make_decode_inputs(w: DecodeWorkload, seed: Optional[int] = None) -> dict:
    """Inputs of ``w.steps`` chained decode steps.

    state [b,H,N,P] f32 ~ N(0,1); per step: x [b,H,P], dt [b,H], B/C [b,G,N]
    (stacked along a leading steps axis); A [H], D [H] fixed.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, H, P, N, G, S = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.steps
    A = draw_A(rng, H)
    D = rng.standard_normal(H, dtype=np.float32)
    state = rng.standard_normal((b, H, N, P), dtype=np.float32)
    s = np.float32(1.0 / math.sqrt(N))
    xs = _store(rng.standard_normal((S, b, H, P), dtype=np.float32), w.dtype)
    dts = _store(draw_dt(rng, (S, b, H), "softplus"), w.dtype)
    Bs = _store(rng.standard_normal((S, b, G, N), dtype=np.float32) * s, w.dtype)
    Cs = _store(rng.standard_normal((S, b, G, N), dtype=np.float32) * s, w.dtype)
    return dict(state=state, xs=xs, dts=dts, A=A, Bs=Bs, Cs=Cs, D=D)


# --------------------------------------------------------------------------
# The element-wise stages next to the core (gated RMS normalisation after it,
# depthwise causal convolution before it). Distributions: activations N(0,1);
# normalisation weights 1 + N(0, 0.1); convolution weights and bias
# U(-1/sqrt(K), 1/sqrt(K)) (the default initialisation of a Conv1d with
# fan-in K); carried convolution state N(0, 1).
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class NormWorkload:
    name: str
    ntokens: int
    dim: int
    group: int
    dtype: str = "bf16"
    eps: float = 1e-5
    seed: int = 0


@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    name: str
    batch: int
    seqlen: int
    channels: int
    width: int = 4
    dtype: str = "bf16"
    with_init: bool = False
    seed: int = 0


# the 130M-shaped layer: y and z are [b*T, H*P] = [16384, 1536], normalised
# over the whole feature vector; the convolution runs over x, B and C
# together, H*P + 2*G*N = 1792 channels, kernel width 4
NORM_130M = NormWorkload("gated_norm_130m_16384x1536_bf16", 8 * 2048, 24 * 64, 24 * 64, seed=4610)
CONV_130M = ConvWorkload("conv_xbc_130m_b8_T2048_C1792_K4_bf16", 8, 2048, 24 * 64 + 2 * 128, seed=4611)


def make_norm_inputs(w: NormWorkload, seed: Optional[int] = None) -> dict:
    """y, z [ntokens, dim] (dtype carriers), weight [dim] fp32."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    y = _store(rng.standard_normal((w.ntokens, w.dim), dtype=np.float32), w.dtype)
    z = _store(rng.standard_normal((w.ntokens, w.dim), dtype=np.float32), w.dtype)
    weight = (1.0 + 0.1 * rng.standard_normal(w.dim)).astype(np.float32)
    return dict(y=y, z=z, weight=weight)


def make_conv_inputs(w: ConvWorkload, seed: Optional[int] = None) -> dict:
    """x [b, T, C] (dtype carrier), weight [C, K] and bias [C] fp32, init
    [b, K-1, C] (dtype carrier) or None."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = _store(rng.standard_normal((w.batch, w.seqlen, w.channels), dtype=np.float32), w.dtype)
    bound = 1.0 / math.sqrt(w.width)
    weight = rng.uniform(-bound, bound, size=(w.channels, w.width)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=w.channels).astype(np.float32)
    init = None
    if w.with_init:
        init = _store(rng.standard_normal((w.batch, w.width - 1, w.channels), dtype=np.float32), w.dtype)
    return dict(x=x, weight=weight, bias=bias, init=init)


# --------------------------------------------------------------------------
# Packed variable-length sequences: one token axis holding sequences of mixed
# length, each with its own initial state.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    name: str
    total: int                 # packed tokens
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    min_len: int = 64          # sequence lengths: log-uniform in [min_len, max_len],
    max_len: int = 4096        # the last one cut so that they sum to `total`
    dtype: str = "bf16"
    init: str = "normal0.1"    # "zero" or "normal0.1"
    seed: int = 0


# the 130M-shaped layer over 16384 packed tokens (the token count of the
# batched 8 x 2048 layer), sequences of 64 .. 4096 tokens
VARLEN_130M = VarlenWorkload("varlen_130m_T16384_H24_P64_N128_Q256_len64-4096", 16384, 24, 64, 128, 1, 256,
                             seed=4620)
# long packed sequences on the 131072-token layer's heads: a few sequences of
# 8K .. 64K tokens
VARLEN_LONG = VarlenWorkload("varlen_long_T131072_H24_P64_N256_Q256_len8192-65536", 131072, 24, 64, 256, 1, 256,
                             min_len=8192, max_len=65536, seed=4621)


def draw_seqlens(rng: np.random.Generator, total: int, lo: int, hi: int) -> np.ndarray:
    lens = []
    left = total
    while left > 0:
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        n = max(1, min(n, left))
        lens.append(n)
        left -= n
    return np.asarray(lens, dtype=np.int64)


def make_varlen_inputs(w: VarlenWorkload, seed: Optional[int] = None) -> dict:
    """x [T,H,P], dt [T,H], B/C [T,G,N] (dtype carriers), A, D [H] fp32,
    cu_seqlens [nseq+1] int32, init [nseq,H,N,P] fp32 or None."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lens = draw_seqlens(rng, w.total, w.min_len, w.max_len)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, P, N, G = w.total, w.nheads, w.headdim, w.dstate, w.ngroups
    x = _store(rng.standard_normal((T, H, P), dtype=np.float32), w.dtype)
    dt = _store(draw_dt(rng, (T, H), "softplus"), w.dtype)
    A = draw_A(rng, H)
    s = np.float32(1.0 / math.sqrt(N))
    B = _store(rng.standard_normal((T, G, N), dtype=np.float32) * s, w.dtype)
    C = _store(rng.standard_normal((T, G, N), dtype=np.float32) * s, w.dtype)
    D = rng.standard_normal(H, dtype=np.float32)
    init = None
    if w.init == "normal0.1":
        init = rng.standard_normal((len(lens), H, N, P), dtype=np.float32) * np.float32(0.1)
    elif w.init != "zero":
        raise ValueError(w.init)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, cu_seqlens=cu, init=init)
