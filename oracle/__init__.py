"""fp64 CPU oracle of the selective state space layer core.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package. The GPU library never
links, loads or calls it, and it imports nothing from the GPU package.

The arithmetic lives in ``ssd_oracle.c`` (plain C, double precision, one
sequential recurrence per column, threads over independent columns); this
module only builds that file with gcc and marshals numpy arrays to it.

Definition followed (youngju.dev "Mamba / selective SSM" page, section
"LTIからSelectionへの切り替え", the selective SSM equations; scalar A per head
and B/C groups from the Qiita "Mamba-2" article, sections 4.1-4.2):

    abar_t = exp(dt_t A_h);  S_t = abar_t S_{t-1} + (dt_t B_t) x_t^T;
    y_t = C_t^T S_t + D_h x_t

Every function here is pinned by the closed forms and invariants in
``tests/test_oracle_pins.py`` (quadratic semiseparable form, A=0 linear
attention, T=1, constant dt, dt=0 identity, large-decay reset, split/resume,
decode chain == forward).

``ssd_bwd`` (``ssd_oracle_bwd.c``) gives the gradients of the forward by
reverse-mode differentiation of the same per-token recurrence, pinned in
``tests/test_oracle_bwd_pins.py`` against torch autograd of an independent
fp64 forward, central finite differences of ``ssd_fwd`` and closed forms.

``oracle.epilogue`` holds the two element-wise stages next to the core (the
gated RMS normalisation after it, the depthwise causal convolution before
it), pinned in ``tests/test_oracle_epilogue_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_SRC_BWD = os.path.join(_HERE, "ssd_oracle_bwd.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_ssd.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c and ssd_oracle_bwd.c into liboracle_ssd.so next
    to them (gcc, -O3)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_BWD, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_ssd_fwd.argtypes = [P] * 9 + [I, L, I, I, I, I, I]
    lib.oracle_ssd_fwd.restype = I
    lib.oracle_ssd_fwd_columns.argtypes = [P] * 7 + [I, P, P, P, P, P] + [I, L, I, I, I, I, I]
    lib.oracle_ssd_fwd_columns.restype = I
    lib.oracle_ssd_decode.argtypes = [P] * 9 + [I, I, I, I, I, I, I, P, P, I]
    lib.oracle_ssd_decode.restype = I
    lib.oracle_ssd_fwd_varlen.argtypes = [P] * 7 + [I, P, P, P, L, I, I, I, I, I]
    lib.oracle_ssd_fwd_varlen.restype = I
    lib.oracle_ssd_bwd.argtypes = [P] * 16 + [L, L, I, I, I, I, I]
    lib.oracle_ssd_bwd.restype = I
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses: the cores this process may run on, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        b = a.astype(np.float32)
        if not np.array_equal(b.astype(a.dtype), a):
            raise ValueError("oracle inputs must be exactly representable in float32")
        a = b
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def ssd_fwd(x, dt, A, B, C, D=None, init=None, nthreads: Optional[int] = None,
            want_y: bool = True, want_final: bool = True):
    """Full forward. x [b,T,H,P], dt [b,T,H], A [H], B/C [b,T,G,N], D [H] or
    None, init [b,H,N,P] or None. Returns (y [b,T,H,P], final [b,H,N,P]) in
    float64 (None for an output not asked for)."""
    x, dt, A, B, C = (_f32(v) for v in (x, dt, A, B, C))
    D = None if D is None else _f32(D)
    init = None if init is None else _f64(init)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, T, H) and A.shape == (H,) and B.shape == (b, T, G, N) == C.shape
    y = np.empty((b, T, H, P), np.float64) if want_y else None
    fin = np.empty((b, H, N, P), np.float64) if want_final else None
    r = _load().oracle_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
                               _ptr(y), _ptr(fin), b, T, H, P, N, G,
                               nthreads or default_threads())
    if r != 0:
        raise RuntimeError(f"oracle_ssd_fwd failed ({r})")
    return y, fin


def ssd_fwd_columns(x, dt, A, B, C, D, init, cols: Sequence[Sequence[int]],
                    nthreads: Optional[int] = None):
    """Forward on selected columns cols = [(b, h, p), ...]. Returns
    (y_cols [ncols, T], final_cols [ncols, N]) in float64."""
    x, dt, A, B, C = (_f32(v) for v in (x, dt, A, B, C))
    D = None if D is None else _f32(D)
    init = None if init is None else _f64(init)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    cols = np.asarray(cols, dtype=np.int32).reshape(-1, 3)
    cb, ch, cp = (np.ascontiguousarray(cols[:, i]) for i in range(3))
    y = np.empty((len(cols), T), np.float64)
    fin = np.empty((len(cols), N), np.float64)
    r = _load().oracle_ssd_fwd_columns(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(init), len(cols), _ptr(cb), _ptr(ch), _ptr(cp),
                                       _ptr(y), _ptr(fin), b, T, H, P, N, G,
                                       nthreads or default_threads())
    if r != 0:
        raise RuntimeError(f"oracle_ssd_fwd_columns failed ({r})")
    return y, fin


def ssd_decode(state0, xs, dts, A, Bs, Cs, D=None, heads: Optional[Sequence[Sequence[int]]] = None,
               nthreads: Optional[int] = None):
    """Chained recurrent steps. state0 [b,H,N,P]; xs [S,b,H,P]; dts [S,b,H];
    Bs/Cs [S,b,G,N]. Returns (ys [S,b,H,P], state [b,H,N,P]) in float64, or,
    with heads = [(b, h), ...], (ys [nsel,S,P], states [nsel,N,P])."""
    xs, dts, A, Bs, Cs = (_f32(v) for v in (xs, dts, A, Bs, Cs))
    D = None if D is None else _f32(D)
    state0 = _f64(state0)
    S, b, H, P = xs.shape
    G, N = Bs.shape[2], Bs.shape[3]
    assert state0.shape == (b, H, N, P) and dts.shape == (S, b, H) and Bs.shape == Cs.shape
    if heads is None:
        nsel, sb, sh = 0, None, None
        ys = np.empty((S, b, H, P), np.float64)
        st = np.empty((b, H, N, P), np.float64)
    else:
        hs = np.asarray(heads, dtype=np.int32).reshape(-1, 2)
        nsel = len(hs)
        sb, sh = np.ascontiguousarray(hs[:, 0]), np.ascontiguousarray(hs[:, 1])
        ys = np.empty((nsel, S, P), np.float64)
        st = np.empty((nsel, N, P), np.float64)
    r = _load().oracle_ssd_decode(_ptr(state0), _ptr(xs), _ptr(dts), _ptr(A), _ptr(Bs), _ptr(Cs),
                                  _ptr(D), _ptr(ys), _ptr(st), b, S, H, P, N, G,
                                  nsel, _ptr(sb), _ptr(sh), nthreads or default_threads())
    if r != 0:
        raise RuntimeError(f"oracle_ssd_decode failed ({r})")
    return ys, st


def ssd_state_update(state, x, dt, A, B, C, D=None, nthreads: Optional[int] = None):
    """One recurrent step: state [b,H,N,P], x [b,H,P], dt [b,H], B/C [b,G,N].
    Returns (y [b,H,P], new_state [b,H,N,P]) in float64."""
    ys, st = ssd_decode(state, np.asarray(x)[None], np.asarray(dt)[None], A,
                        np.asarray(B)[None], np.asarray(C)[None], D, nthreads=nthreads)
    return ys[0], st


def ssd_fwd_varlen(x, dt, A, B, C, D, cu_seqlens, init=None, nthreads: Optional[int] = None,
                   want_y: bool = True, want_final: bool = True):
    """Packed variable-length sequences (one token axis): x [T,H,P], dt [T,H],
    B/C [T,G,N], cu_seqlens [nseq+1] (0 = cu[0] <= ... <= cu[nseq] = T),
    init [nseq,H,N,P] or None. The state restarts from init[i] (or zeros) at
    the first token of sequence i. Returns (y [T,H,P], final [nseq,H,N,P])
    float64 (None where not wanted)."""
    x, dt, A, B, C = (_f32(v) for v in (x, dt, A, B, C))
    D = _f32(D) if D is not None else None
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = cu.shape[0] - 1
    init = _f64(init) if init is not None else None
    y = np.empty((T, H, P)) if want_y else None
    fin = np.empty((nseq, H, N, P)) if want_final else None
    r = _load().oracle_ssd_fwd_varlen(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(cu),
                                      nseq, _ptr(init), _ptr(y), _ptr(fin), T, H, P, N, G,
                                      nthreads or default_threads())
    if r != 0:
        raise ValueError(f"oracle_ssd_fwd_varlen failed ({r})")
    return y, fin


def ssd_bwd(x, dt, A, B, C, D, init, dy, dfinal=None, nthreads: Optional[int] = None,
            want_dinit: bool = True) -> dict:
    """Gradients of ssd_fwd (ssd_oracle_bwd.c): for upstream dy [b,T,H,P] and
    dfinal [b,H,N,P] (None = 0), returns float64 dx [b,T,H,P], ddt [b,T,H],
    dA [H], dB [b,T,G,N], dC [b,T,G,N], dD [H] and dinit [b,H,N,P] (None
    unless wanted). Inputs as for ssd_fwd."""
    x, dt, A, B, C, dy = (_f32(v) for v in (x, dt, A, B, C, dy))
    D = None if D is None else _f32(D)
    init = None if init is None else _f64(init)
    dfinal = None if dfinal is None else _f64(dfinal)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, T, H) and A.shape == (H,) and B.shape == (b, T, G, N) == C.shape
    assert dy.shape == x.shape
    out = dict(dx=np.empty((b, T, H, P)), ddt=np.empty((b, T, H)), dA=np.empty(H),
               dB=np.empty((b, T, G, N)), dC=np.empty((b, T, G, N)), dD=np.empty(H),
               dinit=np.empty((b, H, N, P)) if want_dinit else None)
    r = _load().oracle_ssd_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
                               _ptr(dy), _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
                               _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]),
                               b, T, H, P, N, G, nthreads or default_threads())
    if r != 0:
        raise RuntimeError(f"oracle_ssd_bwd failed ({r})")
    return out


def rel_l2(got, ref) -> float:
    """||got - ref||_2 / ||ref||_2 over the whole array, in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    return num / den if den > 0 else num
