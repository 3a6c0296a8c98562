"""MI355X (gfx950) selective-state-space layer core: Python binding of libssd.so.

This module only marshals arguments: it checks dtypes/devices, allocates
outputs and the workspace with torch when the caller does not pass them, and
calls the C ABI declared in ``include/ssd_api.h`` on torch's current stream.
Every step of the computation runs in the HIP kernels of ``libssd.so``; there
is no CPU or PyTorch fallback. If the library has not been built, importing
the entry points raises.

Entry points (same names as the C ABI):
    ssd_chunk_scan_fwd_workspace(...) -> bytes
    ssd_chunk_scan_fwd_fused_states(...) -> int (0: two launches for chunk states + passing;
                                                 k: one fused launch, k segments per row)
    ssd_chunk_scan_fwd(x, dt, A, B, C, D, init_state, chunk_len) -> (y, final_state)
    ssd_state_update(state, x, dt, A, B, C, D) -> y     (state updated in place)
    ssd_status_string(code) -> str
    ssd_chunk_scan_fwd_varlen(x, dt, A, B, C, D, cu_seqlens, init_states, chunk_len)
        -> (y, final_states)                          (packed variable-length sequences)
    ssd_chunk_scan_fwd_varlen_plan(...) -> (segments, chunk slots per segment) ((0, 0): per chunk)
and, from ``include/ssd_backward.h``, the backward pass:
    ssd_chunk_scan_bwd(x, dt, A, B, C, D, init_state, dy, dfinal)
        -> dict(dx, ddt, dA, dB, dC, dD, dinit)
and, from ``include/ssd_epilogue.h``, the element-wise stages next to the core:
    ssd_gated_rmsnorm(y, z, weight, group, eps) -> out
    ssd_causal_conv1d_fwd(x, weight, bias, init_state, activation) -> (out, final_state)
    ssd_causal_conv1d_update(state, x, weight, bias, activation) -> out   (state in place)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "SSD_F32", "SSD_BF16", "SSDError", "lib", "lib_path",
    "ssd_chunk_scan_fwd_workspace", "ssd_chunk_scan_fwd", "ssd_chunk_scan_fwd_timed",
    "ssd_chunk_scan_fwd_fused_states", "ssd_chunk_scan_fwd_plan", "ssd_chunk_scan_fwd_noalloc",
    "SSD_NOALLOC_SCRATCH_BYTES",
    "ssd_state_update", "ssd_status_string", "ssd_chunk_scan_fwd_varlen",
    "ssd_chunk_scan_fwd_varlen_workspace", "ssd_chunk_scan_fwd_varlen_plan", "ssd_gated_rmsnorm", "ssd_causal_conv1d_fwd",
    "ssd_causal_conv1d_update", "ssd_chunk_scan_bwd_workspace", "ssd_chunk_scan_bwd",
    "ssd_chunk_scan_bwd_fused_walks",
]

SSD_F32 = 0
SSD_BF16 = 1
SSD_NOALLOC_SCRATCH_BYTES = 64 << 20   # the scratch array of ssd_chunk_scan_fwd_noalloc, per GPU

STATUS_NAMES = {
    0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE", 4: "SSD_ERR_CHUNK",
    5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_HIP", 7: "SSD_ERR_ALIAS", 8: "SSD_ERR_ALIGN",
    9: "SSD_ERR_VALUE",
}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssd.so")
_lib = None


class SSDError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({ssd_status_string(code)})")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libssd.so with argument types set. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m selective_state_space_46_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.ssd_chunk_scan_fwd_workspace.argtypes = [i32] * 7 + [i32]
    L.ssd_chunk_scan_fwd_workspace.restype = sz
    L.ssd_chunk_scan_fwd_fused_states.argtypes = [i32] * 7 + [i32]
    L.ssd_chunk_scan_fwd_fused_states.restype = i32
    L.ssd_chunk_scan_fwd_plan.argtypes = [i32] * 7 + [i32, i32, ctypes.POINTER(i32)]
    L.ssd_chunk_scan_fwd_plan.restype = i32
    L.ssd_chunk_scan_fwd.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp, sz, vp]
    L.ssd_chunk_scan_fwd.restype = i32
    L.ssd_chunk_scan_fwd_timed.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp, sz, vp, vp]
    L.ssd_chunk_scan_fwd_timed.restype = i32
    L.ssd_chunk_scan_fwd_noalloc.argtypes = [vp] * 9 + [i32] * 7 + [i32, vp]
    L.ssd_chunk_scan_fwd_noalloc.restype = i32
    L.ssd_state_update.argtypes = [vp] * 8 + [i32] * 5 + [i32, vp]
    L.ssd_state_update.restype = i32
    L.ssd_status_string.argtypes = [i32]
    L.ssd_status_string.restype = ctypes.c_char_p
    i64, f32 = ctypes.c_long, ctypes.c_float
    L.ssd_chunk_scan_fwd_varlen_workspace.argtypes = [i32] * 8
    L.ssd_chunk_scan_fwd_varlen_workspace.restype = sz
    L.ssd_chunk_scan_fwd_varlen.argtypes = [vp] * 10 + [i32] * 8 + [vp, sz, vp]
    L.ssd_chunk_scan_fwd_varlen.restype = i32
    L.ssd_chunk_scan_fwd_varlen_plan.argtypes = [i32] * 8 + [i32, ctypes.POINTER(i32)]
    L.ssd_chunk_scan_fwd_varlen_plan.restype = i32
    L.ssd_gated_rmsnorm.argtypes = [vp] * 4 + [i64, i32, i32, f32, i32, vp]
    L.ssd_gated_rmsnorm.restype = i32
    L.ssd_causal_conv1d_fwd.argtypes = [vp] * 6 + [i32] * 5 + [i32, vp]
    L.ssd_causal_conv1d_fwd.restype = i32
    L.ssd_causal_conv1d_update.argtypes = [vp] * 5 + [i32] * 4 + [i32, vp]
    L.ssd_causal_conv1d_update.restype = i32
    L.ssd_chunk_scan_bwd_workspace.argtypes = [i32] * 7
    L.ssd_chunk_scan_bwd_workspace.restype = sz
    L.ssd_mfma_bf16_probe.argtypes = [i32, i32, vp, vp]
    L.ssd_mfma_bf16_probe.restype = i32
    L.ssd_chunk_scan_bwd_fused_walks.argtypes = [i32] * 7
    L.ssd_chunk_scan_bwd_fused_walks.restype = i32
    L.ssd_chunk_scan_bwd.argtypes = [vp] * 16 + [i32] * 7 + [vp, sz, vp]
    L.ssd_chunk_scan_bwd.restype = i32
    _lib = L
    return L


def ssd_status_string(code: int) -> str:
    return lib().ssd_status_string(int(code)).decode()


def ssd_chunk_scan_fwd_workspace(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                 ngroups: int, chunk_len: int, dtype: int) -> int:
    _bring_up_device()
    return int(lib().ssd_chunk_scan_fwd_workspace(batch, seqlen, nheads, headdim, dstate, ngroups,
                                                  chunk_len, dtype))


def _bring_up_device():
    """The library asks the HIP runtime for the device's compute units; torch's
    runtime is brought up first (as every tensor-taking call here does
    implicitly), since a process whose first HIP call comes from the library
    leaves torch without a device."""
    import torch
    if torch.cuda.is_available():
        torch.cuda.current_device()


def ssd_chunk_scan_fwd_fused_states(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                    ngroups: int, chunk_len: int, dtype: int) -> int:
    """How the forward forms the states entering each chunk on the current
    device (see ssd_api.h): 0 = chunk-state and state-passing launches,
    k >= 1 = one fused launch of walks over k segments per batch row."""
    _bring_up_device()
    return int(lib().ssd_chunk_scan_fwd_fused_states(batch, seqlen, nheads, headdim, dstate, ngroups,
                                                     chunk_len, dtype))


def ssd_chunk_scan_fwd_plan(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int,
                            chunk_len: int, dtype: int, compute_units: int) -> Tuple[int, int]:
    """(segments per row, chunks per segment) the forward chooses on a device
    with `compute_units` compute units; (0, 0) = chunk-state and
    state-passing launches. Needs no device."""
    sl = ctypes.c_int(0)
    n = int(lib().ssd_chunk_scan_fwd_plan(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, dtype,
                                          compute_units, ctypes.byref(sl)))
    return n, int(sl.value)


def ssd_chunk_scan_fwd_varlen_plan(total_tokens: int, nseq: int, nheads: int, headdim: int, dstate: int,
                                   ngroups: int, chunk_len: int, dtype: int, compute_units: int) -> Tuple[int, int]:
    """(segments, chunk slots per segment) of the packed row that the packed
    forward's walks take on a device with `compute_units` compute units;
    (0, 0) = chunk-state launch and a recurrence per sequence over its
    chunks. Needs no device."""
    sl = ctypes.c_int(0)
    n = int(lib().ssd_chunk_scan_fwd_varlen_plan(total_tokens, nseq, nheads, headdim, dstate, ngroups, chunk_len,
                                                 dtype, compute_units, ctypes.byref(sl)))
    return n, int(sl.value)


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, dev, name):
    if t is None:
        return None
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    return t.contiguous()


def _same(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev, stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ssd_chunk_scan_fwd(x, dt, A, B, C, D=None, init_state=None, chunk_len: int = 256, *,
                       y=None, final_state=None, return_final_state: bool = True,
                       workspace=None, stream=None) -> Tuple[object, object]:
    """Chunked forward. x [b,T,H,P], dt [b,T,H], B/C [b,T,G,N] (fp32 or bf16,
    all the same dtype), A/D [H] fp32, init_state [b,H,N,P] fp32 or None.
    Returns (y [b,T,H,P] in x's dtype, final_state [b,H,N,P] fp32 or None)."""
    return ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init_state, chunk_len, y=y,
                                    final_state=final_state, return_final_state=return_final_state,
                                    workspace=workspace, stream=stream, stage_events=None)


def ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D=None, init_state=None, chunk_len: int = 256, *,
                             y=None, final_state=None, return_final_state: bool = True,
                             workspace=None, stream=None, stage_events=None):
    """ssd_chunk_scan_fwd that also records 8 caller-created hipEvent_t handles
    (ints), a start / end pair per stage (cumulative sums, chunk states, state
    passing, chunk outputs), recorded by each kernel's own dispatch; on the
    bf16 matrix-core path the first pair is recorded back to back (the
    chunk-state launch does that work). stage_events=None skips them."""
    import torch
    dev = x.device
    x = _dev(x, dev, "x")
    dt, A, B, C = (_dev(v, dev, n) for v, n in ((dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D = _dev(D, dev, "D")
    init_state = _dev(init_state, dev, "init_state")
    code = _dtype_code(x)
    for v, n in ((dt, "dt"), (B, "B"), (C, "C")):
        _same(v, x.dtype, n)
    for v, n in ((A, "A"), (D, "D"), (init_state, "init_state")):
        _same(v, torch.float32, n)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, T, H) or tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N):
        raise ValueError("shape mismatch among x, dt, B, C")
    if tuple(A.shape) != (H,) or (D is not None and tuple(D.shape) != (H,)):
        raise ValueError("A and D must be [nheads]")
    if init_state is not None and tuple(init_state.shape) != (b, H, N, P):
        raise ValueError("init_state must be [b,H,N,P]")
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    need = ssd_chunk_scan_fwd_workspace(b, T, H, P, N, G, chunk_len, code)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(y),
            _ptr(final_state), b, T, H, P, N, G, chunk_len, code, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev, stream))
    if stage_events is None:
        r = lib().ssd_chunk_scan_fwd(*args)
    else:
        if len(stage_events) != 8:
            raise ValueError("stage_events needs 8 hipEvent_t handles")
        ev = (ctypes.c_void_p * 8)(*[int(e) if e else None for e in stage_events])
        r = lib().ssd_chunk_scan_fwd_timed(*args, ev)
    if r != 0:
        raise SSDError(r, "ssd_chunk_scan_fwd")
    return y, final_state


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D=None, init_state=None, chunk_len: int = 256, *,
                               y, final_state=None, stream=None) -> Tuple[object, object]:
    """ssd_chunk_scan_fwd through the allocation-free entry point: the caller
    passes y (and final_state, or None) preallocated; the library runs on its
    per-GPU scratch array (SSD_NOALLOC_SCRATCH_BYTES) and this wrapper
    allocates nothing either. Raises SSDError (SSD_ERR_WORKSPACE) for sizes
    whose workspace exceeds the scratch array."""
    import torch
    dev = x.device
    for v, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C"), (D, "D"), (init_state, "init_state")):
        if v is not None and not v.is_contiguous():
            raise ValueError(f"{n} must be contiguous (this entry point makes no copies)")
    x = _dev(x, dev, "x")
    dt, A, B, C = (_dev(v, dev, n) for v, n in ((dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D = _dev(D, dev, "D")
    init_state = _dev(init_state, dev, "init_state")
    code = _dtype_code(x)
    for v, n in ((dt, "dt"), (B, "B"), (C, "C"), (y, "y")):
        _same(v, x.dtype, n)
    for v, n in ((A, "A"), (D, "D"), (init_state, "init_state"), (final_state, "final_state")):
        _same(v, torch.float32, n)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, T, H) or tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N):
        raise ValueError("shape mismatch among x, dt, B, C")
    if tuple(A.shape) != (H,) or (D is not None and tuple(D.shape) != (H,)):
        raise ValueError("A and D must be [nheads]")
    for v, n, shp in ((init_state, "init_state", (b, H, N, P)), (final_state, "final_state", (b, H, N, P)),
                      (y, "y", (b, T, H, P))):
        if v is not None and (tuple(v.shape) != shp or not v.is_contiguous() or v.device != dev):
            raise ValueError(f"{n} must be a contiguous {list(shp)} tensor on {dev}")
    r = lib().ssd_chunk_scan_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
                                         _ptr(y), _ptr(final_state), b, T, H, P, N, G, chunk_len, code,
                                         _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_chunk_scan_fwd_noalloc")
    return y, final_state


def ssd_state_update(state, x, dt, A, B, C, D=None, *, y=None, stream=None):
    """One recurrent step, in place on state [b,H,N,P] fp32. x [b,H,P],
    dt [b,H], B/C [b,G,N] (fp32 or bf16), A/D [H] fp32. Returns y [b,H,P]."""
    import torch
    dev = state.device
    if not state.is_contiguous():
        raise ValueError("state must be contiguous (it is updated in place)")
    _same(state, torch.float32, "state")
    x = _dev(x, dev, "x")
    dt, A, B, C = (_dev(v, dev, n) for v, n in ((dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D = _dev(D, dev, "D")
    code = _dtype_code(x)
    for v, n in ((dt, "dt"), (B, "B"), (C, "C")):
        _same(v, x.dtype, n)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if tuple(state.shape) != (b, H, N, P) or tuple(dt.shape) != (b, H) or tuple(C.shape) != (b, G, N):
        raise ValueError("shape mismatch among state, x, dt, B, C")
    if y is None:
        y = torch.empty_like(x)
    r = lib().ssd_state_update(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(y), b, H, P, N, G, code, _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_state_update")
    return y


# --------------------------------------------------------------------------
# element-wise stages next to the core (include/ssd_epilogue.h)
# --------------------------------------------------------------------------

def _inout(t, dev, name):
    """A buffer the call writes: it must already be dense on the device."""
    if t is None:
        return None
    if not t.is_cuda or t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    return t


def ssd_gated_rmsnorm(y, z, weight, group: Optional[int] = None, eps: float = 1e-5, *, out=None,
                      stream=None):
    """rmsnorm(y) * silu(z) over groups of `group` channels of the last axis
    (default: the whole last axis). y, z [..., dim] fp32 or bf16, weight [dim]
    fp32. Returns out (y's shape and dtype); out may be y itself."""
    import torch
    dev = y.device
    y = _dev(y, dev, "y")
    z = _dev(z, dev, "z")
    weight = _dev(weight, dev, "weight")
    code = _dtype_code(y)
    _same(z, y.dtype, "z")
    _same(weight, torch.float32, "weight")
    if z.shape != y.shape or weight.dim() != 1 or weight.shape[0] != y.shape[-1]:
        raise ValueError("z must match y and weight must be [dim]")
    dim = int(y.shape[-1])
    ntok = y.numel() // max(dim, 1)
    group = dim if group is None else int(group)
    out = torch.empty_like(y) if out is None else _inout(out, dev, "out")
    _same(out, y.dtype, "out")
    r = lib().ssd_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(weight), _ptr(out), ntok, dim, group, float(eps),
                                code, _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_gated_rmsnorm")
    return out


def _act_code(activation) -> int:
    if activation in ("silu", 1, True):
        return 1
    if activation in (None, "none", 0, False):
        return 0
    raise ValueError(f"activation must be 'silu' or None, got {activation!r}")


def ssd_causal_conv1d_fwd(x, weight, bias=None, init_state=None, activation="silu", *, out=None,
                          final_state=None, return_final_state: bool = False, stream=None):
    """Depthwise causal convolution over tokens. x [b, T, C] fp32 or bf16,
    weight [C, K] fp32, bias [C] fp32 or None, init_state [b, K-1, C] (x's
    dtype) or None. Returns (out [b, T, C], final_state [b, K-1, C] or None);
    final_state may be passed as init_state itself to carry it in place."""
    import torch
    dev = x.device
    x = _dev(x, dev, "x")
    weight, bias = _dev(weight, dev, "weight"), _dev(bias, dev, "bias")
    code = _dtype_code(x)
    _same(weight, torch.float32, "weight")
    _same(bias, torch.float32, "bias")
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[2]:
        raise ValueError("x must be [b, T, C] and weight [C, K]")
    b, T, C = (int(v) for v in x.shape)
    K = int(weight.shape[1])
    if init_state is not None:
        init_state = _inout(init_state, dev, "init_state")
        _same(init_state, x.dtype, "init_state")
        if tuple(init_state.shape) != (b, K - 1, C):
            raise ValueError("init_state must be [b, K-1, C]")
    out = torch.empty_like(x) if out is None else _inout(out, dev, "out")
    _same(out, x.dtype, "out")
    if final_state is None and return_final_state:
        final_state = torch.empty((b, K - 1, C), dtype=x.dtype, device=dev)
    elif final_state is not None:
        final_state = _inout(final_state, dev, "final_state")
        _same(final_state, x.dtype, "final_state")
    r = lib().ssd_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(init_state), _ptr(out),
                                    _ptr(final_state), b, T, C, K, _act_code(activation), code,
                                    _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_causal_conv1d_fwd")
    return out, final_state


def ssd_causal_conv1d_update(state, x, weight, bias=None, activation="silu", *, out=None, stream=None):
    """One token of the convolution: state [b, K-1, C] (x's dtype) updated in
    place, x [b, C]. Returns out [b, C]."""
    import torch
    dev = x.device
    x = _dev(x, dev, "x")
    weight, bias = _dev(weight, dev, "weight"), _dev(bias, dev, "bias")
    code = _dtype_code(x)
    _same(weight, torch.float32, "weight")
    _same(bias, torch.float32, "bias")
    if x.dim() != 2 or weight.dim() != 2 or weight.shape[0] != x.shape[1]:
        raise ValueError("x must be [b, C] and weight [C, K]")
    b, C = (int(v) for v in x.shape)
    K = int(weight.shape[1])
    if state is not None:
        state = _inout(state, dev, "state")
        _same(state, x.dtype, "state")
        if tuple(state.shape) != (b, K - 1, C):
            raise ValueError("state must be [b, K-1, C]")
    out = torch.empty_like(x) if out is None else _inout(out, dev, "out")
    r = lib().ssd_causal_conv1d_update(_ptr(state), _ptr(x), _ptr(weight), _ptr(bias), _ptr(out), b, C, K,
                                       _act_code(activation), code, _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_causal_conv1d_update")
    return out


# --------------------------------------------------------------------------
# packed variable-length sequences
# --------------------------------------------------------------------------

def ssd_chunk_scan_fwd_varlen_workspace(total_tokens: int, nseq: int, nheads: int, headdim: int, dstate: int,
                                        ngroups: int, chunk_len: int, dtype: int) -> int:
    return int(lib().ssd_chunk_scan_fwd_varlen_workspace(total_tokens, nseq, nheads, headdim, dstate, ngroups,
                                                         chunk_len, dtype))


def ssd_chunk_scan_fwd_varlen(x, dt, A, B, C, D, cu_seqlens, init_states=None, chunk_len: int = 256, *,
                              y=None, final_states=None, return_final_states: bool = True, workspace=None,
                              stream=None):
    """Packed sequences: x [T,H,P], dt [T,H], B/C [T,G,N] (bf16), A/D [H] fp32,
    cu_seqlens [nseq+1] int32 on the device, init_states [nseq,H,N,P] fp32 or
    None. Returns (y [T,H,P], final_states [nseq,H,N,P] or None)."""
    import torch
    dev = x.device
    x = _dev(x, dev, "x")
    dt, A, B, C = (_dev(v, dev, n) for v, n in ((dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D = _dev(D, dev, "D")
    cu = _dev(cu_seqlens, dev, "cu_seqlens")
    if cu.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    init_states = _dev(init_states, dev, "init_states")
    code = _dtype_code(x)
    for v, n in ((dt, "dt"), (B, "B"), (C, "C")):
        _same(v, x.dtype, n)
    for v, n in ((A, "A"), (D, "D"), (init_states, "init_states")):
        _same(v, torch.float32, n)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nseq = cu.numel() - 1
    if tuple(dt.shape) != (T, H) or tuple(B.shape) != (T, G, N) or tuple(C.shape) != (T, G, N):
        raise ValueError("shape mismatch among x, dt, B, C")
    if init_states is not None and tuple(init_states.shape) != (nseq, H, N, P):
        raise ValueError("init_states must be [nseq,H,N,P]")
    y = torch.empty_like(x) if y is None else _inout(y, dev, "y")
    if final_states is None and return_final_states:
        final_states = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev)
    elif final_states is not None:
        final_states = _inout(final_states, dev, "final_states")
    need = ssd_chunk_scan_fwd_varlen_workspace(T, nseq, H, P, N, G, chunk_len, code)
    if need == 0:
        raise SSDError(2, "ssd_chunk_scan_fwd_varlen_workspace")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    r = lib().ssd_chunk_scan_fwd_varlen(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(cu),
                                        _ptr(init_states), _ptr(y), _ptr(final_states), T, nseq, H, P, N, G,
                                        chunk_len, code, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_chunk_scan_fwd_varlen")
    return y, final_states


def ssd_chunk_scan_bwd_workspace(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                 ngroups: int, dtype: int) -> int:
    _bring_up_device()
    return int(lib().ssd_chunk_scan_bwd_workspace(batch, seqlen, nheads, headdim, dstate, ngroups, dtype))


def ssd_chunk_scan_bwd_fused_walks(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                                   ngroups: int, dtype: int) -> int:
    """Bit 0: the backward's recomputation runs as one walk launch; bit 1: its
    state gradients come from the reverse walk (see ssd_backward.h)."""
    _bring_up_device()
    return int(lib().ssd_chunk_scan_bwd_fused_walks(batch, seqlen, nheads, headdim, dstate, ngroups, dtype))


def ssd_chunk_scan_bwd(x, dt, A, B, C, D=None, init_state=None, dy=None, dfinal=None, *, out=None,
                       want_dD: bool = True, want_dinit: bool = True, workspace=None, stream=None) -> dict:
    """Gradients of ssd_chunk_scan_fwd for upstream dy [b,T,H,P] (x's dtype)
    and dfinal [b,H,N,P] fp32 or None. Returns dict(dx, ddt, dB, dC in x's
    dtype, dA [H] fp32, dD [H] fp32 or None, dinit [b,H,N,P] fp32 or None).
    `out` may hold preallocated outputs under the same names."""
    import torch
    if dy is None:
        raise ValueError("dy is required")
    dev = x.device
    x = _dev(x, dev, "x")
    dt, A, B, C, dy = (_dev(v, dev, n) for v, n in ((dt, "dt"), (A, "A"), (B, "B"), (C, "C"), (dy, "dy")))
    D, init_state, dfinal = (_dev(v, dev, n) for v, n in ((D, "D"), (init_state, "init_state"),
                                                          (dfinal, "dfinal")))
    code = _dtype_code(x)
    for v, n in ((dt, "dt"), (B, "B"), (C, "C"), (dy, "dy")):
        _same(v, x.dtype, n)
    for v, n in ((A, "A"), (D, "D"), (init_state, "init_state"), (dfinal, "dfinal")):
        _same(v, torch.float32, n)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, T, H) or tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N) \
            or tuple(dy.shape) != (b, T, H, P):
        raise ValueError("shape mismatch among x, dt, B, C, dy")
    o = dict(out or {})
    f32 = torch.float32
    shapes = dict(dx=((b, T, H, P), x.dtype), ddt=((b, T, H), x.dtype), dA=((H,), f32),
                  dB=((b, T, G, N), x.dtype), dC=((b, T, G, N), x.dtype), dD=((H,), f32),
                  dinit=((b, H, N, P), f32))
    for k, (shp, dty) in shapes.items():
        if k == "dD" and not want_dD or k == "dinit" and not want_dinit:
            o[k] = None
        elif o.get(k) is None:
            o[k] = torch.empty(shp, dtype=dty, device=dev)
        else:
            o[k] = _inout(o[k], dev, k)
    need = ssd_chunk_scan_bwd_workspace(b, T, H, P, N, G, code)
    if need == 0:
        raise SSDError(2, "ssd_chunk_scan_bwd_workspace")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    r = lib().ssd_chunk_scan_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
                                 _ptr(dy), _ptr(dfinal), _ptr(o["dx"]), _ptr(o["ddt"]), _ptr(o["dA"]),
                                 _ptr(o["dB"]), _ptr(o["dC"]), _ptr(o["dD"]), _ptr(o["dinit"]), b, T, H, P, N,
                                 G, code, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(dev, stream))
    if r != 0:
        raise SSDError(r, "ssd_chunk_scan_bwd")
    return o
