#!/usr/bin/env python3
"""Benchmark of the SSD layer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-extra]

One step = one ssd_chunk_scan_fwd call over one batch of the workload, inputs
resident in HBM: on the bf16 matrix-core path one launch computes the
in-chunk cumulative sums, the C B^T tiles and the states entering each chunk
(whole rows, or segments of rows followed by a short recurrence over the
segments, see ssd_chunk_scan_fwd_fused_states), then chunk_scan. The
headline workload is the largest single-GPU configuration: one 131072-token
row, H 24, P 64, N 256, 1 group, chunk 256, bf16 inputs with fp32
accumulation and state. Prints ONE JSON line on stdout; progress goes to
stderr.

Kernel durations are measured live with hipEvents that each kernel's own
dispatch records at its start and end (ssd_chunk_scan_fwd_timed, through
hipExtLaunchKernel). Algorithmic bytes and flops per kernel follow the
minimal I/O of the four-step chunked algorithm (in-chunk sums, chunk states,
state passing, chunk outputs, with the chunk states in fp32 between them);
each launch's own minimal I/O in this implementation is reported beside it.
The other workloads (the 130M-shaped layer warm and cold, the 2.7B-shaped
layer, the decode update, the backward pass, packed sequences, and the
stages next to the core) are measured in the same run, and the fp64 CPU
oracle is timed on the host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "SSD fwd tokens/s per layer + % of bf16 MFMA / HBM roofline on 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
# Before a forward workload's warm-up steps the step runs untimed for this
# long: under a sudden sustained load the GPU's clocks dip and recover over
# the first ~20 ms (measured on the 128K-token layer: per-call times rise
# from 0.63 to 0.83 ms within 5 calls and settle back over ~20 more), so 5
# warm-up steps alone leave the timed window in that transient (0.706 ms per
# step against 0.630 with 50 or 200 warm-up steps).
SETTLE_S = 0.15
KERNEL_SOURCES = {
    "chunk_cumsum": ["chunk_cumsum.hip"],
    "chunk_state": ["chunk_state.hip", "chunk_state_mfma.hip", "mfma_util.h"],
    "state_passing": ["state_passing.hip"],
    "chunk_scan": ["chunk_scan.hip", "chunk_scan_mfma.hip", "mfma_util.h"],
    "state_update": ["state_update.hip"],
}
# the library's event windows, in launch order (chunk_cumsum is empty on the
# matrix-core path, where chunk_state does its work)
STAGES = ["chunk_cumsum", "chunk_state", "state_passing", "chunk_scan"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# HIP events through the runtime's C API (the library records them itself)
# --------------------------------------------------------------------------

class Hip:
    def __init__(self):
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.rt = ctypes.CDLL(name)
                break
            except OSError:
                continue
        else:
            raise RuntimeError("libamdhip64.so not found")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, e, stream):
        if self.rt.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


# --------------------------------------------------------------------------
# Algorithmic work per kernel
# --------------------------------------------------------------------------

def alg_work(w: workloads.FwdWorkload) -> dict:
    """Minimal I/O (bytes) and useful flops of the four steps of the chunked
    algorithm, each step a kernel of its own, the chunk states in fp32
    between them (the per-token figures below times the b T tokens of one
    call; e = element size of x, dt, B, C, y):
      cumsum        dt read, Acs written                                   (H e + 4 H per token)
      chunk_state   x, B, dt, Acs read, fp32 chunk states written
      state_passing chunk states read and written, final (and init) state
      chunk_scan    x read, y written, B and C read, chunk states and Acs, dt read
    flops: chunk_state 2 N P per token and head; state_passing 2 N P per
    chunk and head; chunk_scan (Q + 1) N / (H / G) (C B^T, lower triangle,
    once per group) + (Q + 1) P (masked product) + 2 N P (C H_c) per token
    and head."""
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    nc = -(-T // Q)
    e = 2 if w.dtype == "bf16" else 4
    tok = b * T
    x, dtb, bc = tok * H * P * e, tok * H * e, tok * G * N * e
    acs = 4 * b * H * nc * Q
    st = 4 * b * nc * H * N * P
    fst = 4 * b * H * N * P * (2 if w.init != "zero" else 1)
    return {
        "chunk_cumsum": {"bytes": dtb + acs, "flops": 2 * tok * H},
        "chunk_state": {"bytes": x + bc + dtb + acs + st, "flops": 2 * tok * H * N * P},
        "state_passing": {"bytes": 2 * st + fst, "flops": 2 * b * nc * H * N * P},
        "chunk_scan": {"bytes": 2 * x + 2 * bc + st + acs + dtb,
                       "flops": tok * H * ((Q + 1) * N * G // H + (Q + 1) * P + 2 * N * P)},
    }


def impl_work(w: workloads.FwdWorkload, nseg: int) -> dict:
    """Each launch's own minimal I/O in this implementation (nseg: the
    forward's segments per row, 0 = separate chunk-state and state-passing
    launches). The bf16 matrix-core path computes the cumulative sums and C B^T
    per chunk and group (bf16 32x32 tiles) in its chunk-state launch and hands
    the passed states to chunk_scan as bf16; the fused launch keeps the fp32
    chunk states on chip (with segments it writes each segment's last local
    state, and chunk_scan reads the state entering each segment once per
    segment and head)."""
    b, T, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    nc = -(-T // Q)
    e = 2 if w.dtype == "bf16" else 4
    x, dtb, bc = b * T * H * P * e, b * T * H * e, b * T * G * N * e
    acs = 4 * b * H * nc * Q
    st = 4 * b * nc * H * N * P
    fst = 4 * b * H * N * P
    ini = fst if w.init != "zero" else 0
    mfma = w.dtype == "bf16" and N in (32, 64, 128, 256) and P in (32, 64, 128) and Q >= 32
    lpc = Q // 32
    cbt = b * nc * G * (lpc * (lpc + 1) // 2) * 1024 * 2 if mfma else 0
    hst = st // 2 if mfma else st
    out = {"chunk_cumsum": {"bytes": dtb + 2 * acs}, "chunk_state": {"bytes": x + bc + 2 * acs + st},
           "state_passing": {"bytes": st + hst + 4 * b * H * nc + fst + ini},
           "chunk_scan": {"bytes": 2 * x + (bc + cbt if mfma else 2 * bc) + 2 * acs + hst}}
    if mfma:
        out["chunk_cumsum"] = {"bytes": 0}
        out["chunk_state"] = {"bytes": x + 2 * bc + dtb + 2 * acs + st + cbt}
    if nseg >= 1:
        sst = 4 * b * nseg * H * N * P
        # with segments the tiles launch also writes C in operand order (bc
        # bytes), which chunk_scan reads in place of C
        out["chunk_state"] = {"bytes": x + 2 * bc + dtb + 2 * acs + cbt + hst + ini
                              + (fst if nseg == 1 else sst + 4 * b * H * (nc + nseg) + bc)}
        out["state_passing"] = {"bytes": 0 if nseg == 1 else 2 * sst + fst + 4 * b * H * nseg}
        if nseg > 1:
            out["chunk_scan"] = {"bytes": out["chunk_scan"]["bytes"] + sst + 4 * b * H * nc}
    return out


def decode_work(w: workloads.DecodeWorkload) -> dict:
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    e = 2 if w.dtype == "bf16" else 4
    return {"bytes": 8 * b * H * N * P + 2 * b * H * P * e + b * H * e + 2 * b * G * N * e + 8 * H,
            "flops": b * H * N * P * 5}


# --------------------------------------------------------------------------
# HBM traffic from committed rocprofv3 counter summaries
# --------------------------------------------------------------------------

def _code_only(text: str) -> str:
    """C++ source without its comments and whitespace: edits to comments
    leave a kernel's digest (and its counted traffic) as it was."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


def sources_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["ssd_internal.h"]:
        p = os.path.join(ROOT, "selective_state_space_46_amd", "csrc", f)
        if os.path.exists(p):
            h.update(_code_only(open(p).read()).encode())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str, tag: str):
    """HBM bytes per dispatch from profiles/traffic_<kernel>_<tag>.txt (tag: the
    workload's short name), or None when there is no such summary, the
    workload has no tag, or the kernel's sources changed since it was taken."""
    if not tag:
        return None
    p = os.path.join(PROFILES, f"traffic_{kernel}_{tag}.txt")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m_src = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_dispatch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != sources_digest(kernel):
        return None
    return float(m_b.group(1))


# --------------------------------------------------------------------------
# GPU measurements
# --------------------------------------------------------------------------

def to_dev(a, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def bench_fwd(hip, w, steps, warmup, cold=False, settle=True):
    import torch
    import selective_state_space_46_amd as ssd

    inp = workloads.make_fwd_inputs(w)
    x, dt, B, C = (to_dev(inp[k], w.dtype) for k in ("x", "dt", "B", "C"))
    A, D = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32")
    init = to_dev(inp["init"], "f32") if inp["init"] is not None else None
    y = torch.empty_like(x)
    fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
    code = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    nbytes = ssd.ssd_chunk_scan_fwd_workspace(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                              w.ngroups, w.chunk_len, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    del inp

    def call(ev=None):
        ssd.ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init, w.chunk_len, y=y, final_state=fin,
                                     workspace=ws, stream=stream, stage_events=ev)

    # untimed: clocks settled (SETTLE_S of back-to-back steps), then the
    # warm-up steps
    t_settle = time.perf_counter()
    while settle and time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if cold else None

    # pass 1: the step as callers run it (plain entry point), events around all K steps
    t_start, t_end = hip.event(), hip.event()
    if cold:
        call_ms = []
        for k in range(steps):
            flush.fill_(k & 0xFF)     # evict the inputs from L2 / Infinity Cache
            hip.record(t_start, stream)
            call()
            hip.record(t_end, stream)
            torch.cuda.synchronize()
            call_ms.append(hip.ms(t_start, t_end))
        ms_per_step = float(np.mean(call_ms))
        wall = 0.0
    else:
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        hip.record(t_start, stream)
        for _ in range(steps):
            call()
        hip.record(t_end, stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_per_step = hip.ms(t_start, t_end) / steps

    # pass 2: per-kernel durations from start / end events recorded by each kernel's dispatch
    evs = [[hip.event() for _ in range(2 * len(STAGES))] for _ in range(steps)]
    for k in range(steps):
        call(evs[k])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([hip.ms(ev[2 * i], ev[2 * i + 1]) for ev in evs]))
                for i, s in enumerate(STAGES)}
    call_ms = float(np.mean([hip.ms(ev[0], ev[-1]) for ev in evs]))
    for e in [t_start, t_end] + [e for ev in evs for e in ev]:
        hip.destroy(e)
    return dict(ms_per_step=ms_per_step, call_ms=call_ms, stage_ms=stage_ms, wall_s=wall,
                tokens_per_s=w.tokens / (ms_per_step * 1e-3))


def bench_decode(hip, w, warmup=4):
    import torch
    import selective_state_space_46_amd as ssd
    inp = workloads.make_decode_inputs(w)
    state = to_dev(inp["state"], "f32")
    A, D = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32")
    xs, dts, Bs, Cs = (to_dev(inp[k], w.dtype) for k in ("xs", "dts", "Bs", "Cs"))
    ys = torch.empty_like(xs)
    del inp
    stream = torch.cuda.current_stream().cuda_stream
    for s in range(warmup):
        ssd.ssd_state_update(state, xs[s], dts[s], A, Bs[s], Cs[s], D, y=ys[s], stream=stream)
    torch.cuda.synchronize()
    evs = [hip.event() for _ in range(w.steps + 1)]
    hip.record(evs[0], stream)
    for s in range(w.steps):
        ssd.ssd_state_update(state, xs[s], dts[s], A, Bs[s], Cs[s], D, y=ys[s], stream=stream)
        hip.record(evs[s + 1], stream)
    torch.cuda.synchronize()
    per = [hip.ms(evs[i], evs[i + 1]) for i in range(w.steps)]
    total = hip.ms(evs[0], evs[-1])
    for e in evs:
        hip.destroy(e)
    work = decode_work(w)
    avg = float(np.mean(per))
    gbs = work["bytes"] / (avg * 1e-3) / 1e9
    return {
        "workload": w.name, "steps_chained": w.steps, "ms_per_update": avg,
        "tokens_per_s": w.batch * w.steps / (total * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("state_update", "decode_b256")},
        "alg_bytes_per_update": work["bytes"],
    }


_HEAD_START = []


def gpu_head_start():
    """Device copies (about 1.5 ms of work) enqueued on torch's current stream
    ahead of a timed region: while they run, the host enqueues the timed
    calls, so calls whose kernels take less time than the binding spends per
    call still run back to back and the events time the device, not the
    host."""
    import torch
    if not _HEAD_START:
        n = 1 << 28                    # 1 GiB of fp32 each
        _HEAD_START.extend([torch.empty(n, dtype=torch.float32, device="cuda"),
                            torch.empty(n, dtype=torch.float32, device="cuda")])
    src, dst = _HEAD_START
    for _ in range(4):
        dst.copy_(src)


def bench_next_to_core(hip, steps=20, warmup=3):
    """The element-wise stages next to the core on the 130M-shaped layer: the
    depthwise causal conv1d over x, B, C (1792 channels, width 4) before it,
    the gated RMS normalisation of y (16384 x 1536, whole-vector groups)
    after it, and the conv's decode update on the batch-256 decode layer
    (128 x 64 + 2 x 8 x 128 = 10240 channels). Algorithmic bytes: every
    tensor element read or written once (weights included). The timed calls
    run back to back on the device (gpu_head_start)."""
    import torch
    import selective_state_space_46_amd as ssd
    stream = torch.cuda.current_stream().cuda_stream
    out = {}

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        gpu_head_start()
        hip.record(a, stream)
        for _ in range(steps):
            fn()
        hip.record(b, stream)
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / steps
        hip.destroy(a)
        hip.destroy(b)
        return ms

    def entry(ms, nbytes, extra):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return dict(extra, ms=round(ms, 5), alg_bytes=nbytes, GB_per_s=round(gbs, 1),
                    hbm_frac=round(gbs / HBM_PEAK_GBS, 4))

    cw = workloads.CONV_130M
    ci = workloads.make_conv_inputs(cw)
    x = to_dev(ci["x"], cw.dtype)
    wt, bias = to_dev(ci["weight"], "f32"), to_dev(ci["bias"], "f32")
    y = torch.empty_like(x)
    state = torch.zeros((cw.batch, cw.width - 1, cw.channels), dtype=x.dtype, device="cuda")
    ms = timed(lambda: ssd.ssd_causal_conv1d_fwd(x, wt, bias, None, out=y, final_state=state, stream=stream))
    e = x.element_size()
    out["causal_conv1d"] = entry(ms, 2 * x.numel() * e + state.numel() * e + 4 * (wt.numel() + bias.numel()),
                                 {"workload": cw.name})
    del x, y

    nw = workloads.NORM_130M
    ni = workloads.make_norm_inputs(nw)
    yv, zv, nwt = to_dev(ni["y"], nw.dtype), to_dev(ni["z"], nw.dtype), to_dev(ni["weight"], "f32")
    o = torch.empty_like(yv)
    ms = timed(lambda: ssd.ssd_gated_rmsnorm(yv, zv, nwt, nw.group, nw.eps, out=o, stream=stream))
    out["gated_rmsnorm"] = entry(ms, 3 * yv.numel() * yv.element_size() + 4 * nwt.numel(),
                                 {"workload": nw.name, "group": nw.group})
    del yv, zv, o

    dw = workloads.DECODE_B256
    C = dw.nheads * dw.headdim + 2 * dw.ngroups * dw.dstate
    uw = workloads.ConvWorkload("conv_decode_b256_C10240_K4_bf16", dw.batch, 1, C, 4, "bf16", True, seed=4612)
    ui = workloads.make_conv_inputs(uw)
    st = to_dev(ui["init"], "bf16")
    xt = to_dev(ui["x"][:, 0], "bf16")
    uwt, ub = to_dev(ui["weight"], "f32"), to_dev(ui["bias"], "f32")
    ot = torch.empty_like(xt)
    ms = timed(lambda: ssd.ssd_causal_conv1d_update(st, xt, uwt, ub, out=ot, stream=stream))
    out["causal_conv1d_update"] = entry(ms, 2 * st.numel() * 2 + 2 * xt.numel() * 2 + 4 * (uwt.numel() + ub.numel()),
                                        {"workload": uw.name})
    return out


def bench_varlen(hip, vw, steps=20, warmup=3):
    """The forward over packed variable-length sequences (one token axis, a
    per-sequence initial and final state): the whole call, chunk table build
    included, timed with HIP events around `steps` calls on one stream, back
    to back on the device (gpu_head_start)."""
    import torch
    import selective_state_space_46_amd as ssd
    stream = torch.cuda.current_stream().cuda_stream
    vi = workloads.make_varlen_inputs(vw)
    x, dt, B, C = (to_dev(vi[k], vw.dtype) for k in ("x", "dt", "B", "C"))
    A, D = to_dev(vi["A"], "f32"), to_dev(vi["D"], "f32")
    init = to_dev(vi["init"], "f32") if vi["init"] is not None else None
    cu = torch.from_numpy(vi["cu_seqlens"]).cuda()
    nseq = cu.numel() - 1
    y = torch.empty_like(x)
    fin = torch.empty((nseq, vw.nheads, vw.dstate, vw.headdim), dtype=torch.float32, device="cuda")
    need = ssd.ssd_chunk_scan_fwd_varlen_workspace(vw.total, nseq, vw.nheads, vw.headdim, vw.dstate,
                                                   vw.ngroups, vw.chunk_len, 1 if vw.dtype == "bf16" else 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        ssd.ssd_chunk_scan_fwd_varlen(x, dt, A, B, C, D, cu, init, vw.chunk_len, y=y, final_states=fin,
                                      workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = hip.event(), hip.event()
    gpu_head_start()
    hip.record(a, stream)
    for _ in range(steps):
        call()
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    lens = np.diff(vi["cu_seqlens"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nseg, seglen = ssd.ssd_chunk_scan_fwd_varlen_plan(vw.total, nseq, vw.nheads, vw.headdim, vw.dstate, vw.ngroups,
                                                      vw.chunk_len, 1 if vw.dtype == "bf16" else 0, cus)
    return {"workload": vw.name, "nseq": nseq, "min_len": int(lens.min()), "max_len": int(lens.max()),
            "segments": nseg, "slots_per_segment": seglen,
            "ms_per_call": round(ms, 5), "tokens_per_s": round(vw.total / (ms * 1e-3), 1)}


def bench_backward(hip, w, steps=10, warmup=3):
    """The backward pass on a forward workload: one ssd_chunk_scan_bwd call
    (recomputation included) per step, upstream dy ~ N(0, 1) in bf16, timed
    with HIP events around `steps` calls on one stream. Algorithmic bytes: its
    minimal I/O, every input and output element once (x, dy, B, C, dt, A, D
    and init read; dx, ddt, dB, dC, dA, dD and dinit written)."""
    import torch
    import selective_state_space_46_amd as ssd
    stream = torch.cuda.current_stream().cuda_stream
    inp = workloads.make_fwd_inputs(w)
    x, dt, B, C = (to_dev(inp[k], w.dtype) for k in ("x", "dt", "B", "C"))
    A, D = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32")
    init = to_dev(inp["init"], "f32") if inp["init"] is not None else None
    rng = np.random.default_rng(w.seed + 100)
    dy = to_dev(workloads.round_to_bf16(rng.standard_normal(inp["x"].shape, dtype=np.float32)), w.dtype)
    code = 1 if w.dtype == "bf16" else 0
    need = ssd.ssd_chunk_scan_bwd_workspace(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, code)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = ssd.ssd_chunk_scan_bwd(x, dt, A, B, C, D, init, dy, None, workspace=ws, stream=stream)

    def call():
        ssd.ssd_chunk_scan_bwd(x, dt, A, B, C, D, init, dy, None, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = hip.event(), hip.event()
    hip.record(a, stream)
    for _ in range(steps):
        call()
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    e = 2 if w.dtype == "bf16" else 4
    tok = w.batch * w.seqlen
    st = w.batch * w.nheads * w.dstate * w.headdim * 4
    nbytes = (3 * tok * w.nheads * w.headdim * e + 4 * tok * w.ngroups * w.dstate * e + 2 * tok * w.nheads * e
              + 4 * w.nheads * 4 + (2 * st if init is not None else st))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "ms_per_call": round(ms, 5), "tokens_per_s": round(tok / (ms * 1e-3), 1),
            "alg_bytes": nbytes, "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "workspace_bytes": need}


def measured_peaks(hip, iters=2000):
    """Achievable rates on this device, beside the published ones: the bf16
    matrix-core probe of the library (ssd_mfma_bf16_probe: 8 independent
    32x32x16 MFMA chains per wave, 4 work-groups of 4 waves per compute unit)
    and a 1 GiB device-to-device copy (read + write)."""
    import torch
    import selective_state_space_46_amd as ssd
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg = 4 * cus
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    L = ssd.lib()
    for _ in range(2):
        assert L.ssd_mfma_bf16_probe(wg, iters, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    a, b = hip.event(), hip.event()
    hip.record(a, stream)
    assert L.ssd_mfma_bf16_probe(wg, iters, out.data_ptr(), stream) == 0
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.ms(a, b)
    tflops = wg * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    hip.record(a, stream)
    for _ in range(5):
        dst.copy_(src)
    hip.record(b, stream)
    torch.cuda.synchronize()
    gbs = 5 * 2 * (1 << 30) / (hip.ms(a, b) * 1e-3) / 1e9
    hip.destroy(a)
    hip.destroy(b)
    del src, dst
    return {"mfma_bf16_TFLOP_per_s": round(tflops, 1), "mfma_bf16_frac_of_published": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "copy_GB_per_s": round(gbs, 1), "copy_frac_of_published": round(gbs / HBM_PEAK_GBS, 4),
            "copy_bytes": 1 << 30, "mfma_probe": f"{wg} work-groups x 4 waves x {iters} x 8 MFMA 32x32x16 bf16"}


def decode_probe():
    """Eight chained decode updates, then three copies of a 256 MiB buffer (the
    counter calibration of --traffic-probe)."""
    import torch
    import selective_state_space_46_amd as ssd
    dw = workloads.DECODE_B256
    inp = workloads.make_decode_inputs(workloads.DecodeWorkload(dw.name, dw.batch, dw.nheads, dw.headdim, dw.dstate,
                                                                dw.ngroups, 8, dw.dtype, seed=dw.seed))
    state = to_dev(inp["state"], "f32")
    A, D = to_dev(inp["A"], "f32"), to_dev(inp["D"], "f32")
    for s in range(8):
        ssd.ssd_state_update(state, to_dev(inp["xs"][s], "bf16"), to_dev(inp["dts"][s], "bf16"), A,
                             to_dev(inp["Bs"][s], "bf16"), to_dev(inp["Cs"][s], "bf16"), D)
    torch.cuda.synchronize()
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] decode probe done (8 updates, copy of 268435456 bytes x3)")


def traffic_probe(w):
    """Three forward calls, then three copies of a 256 MiB buffer: a plain
    copy kernel that reads and writes exactly 256 MiB, against which the
    FETCH_SIZE / WRITE_SIZE counters are calibrated."""
    import torch
    bench_fwd(Hip(), w, 3, 0, settle=False)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] traffic probe done (copy of 268435456 bytes x3)")


def backward_probe():
    """Four backward calls on the 130M-shaped layer (one warm-up and three
    timed by bench_backward's loop; for rocprofv3 --pmc runs on the backward
    kernels)."""
    r = bench_backward(Hip(), workloads.MAMBA2_130M, steps=3, warmup=1)
    log(f"[bench] backward probe done ({r['ms_per_call']} ms per call)")


def cpu_baseline(w, min_seconds=10.0):
    import oracle
    inp = workloads.make_fwd_inputs(w)
    n = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init"],
                       nthreads=n)
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    cpu = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(w.tokens * runs / el, 1), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"the whole {w.name} forward, {runs} run(s) in {el:.1f} s, fp64, {cpu}"}


def extras(hip) -> dict:
    """The sections beside the headline forward."""
    out = {}
    dw = workloads.DECODE_B256
    log(f"[bench] decode {dw.name}")
    out["decode"] = bench_decode(hip, dw)
    log(f"[bench] decode {out['decode']['ms_per_update']:.4f} ms/update")
    bw = workloads.MAMBA2_130M
    log(f"[bench] backward {bw.name}")
    out["backward"] = bench_backward(hip, bw)
    log(f"[bench]   {out['backward']}")
    log(f"[bench] packed sequences {workloads.VARLEN_130M.name}")
    out["varlen"] = bench_varlen(hip, workloads.VARLEN_130M)
    log(f"[bench]   {out['varlen']}")
    log(f"[bench] packed sequences {workloads.VARLEN_LONG.name}")
    out["varlen_long"] = bench_varlen(hip, workloads.VARLEN_LONG, steps=10)
    log(f"[bench]   {out['varlen_long']}")
    log("[bench] stages next to the core (conv1d, gated RMSNorm, conv decode update)")
    out["next_to_core"] = bench_next_to_core(hip)
    log(f"[bench]   {out['next_to_core']}")
    return out


# which steps of the chunked algorithm each of the library's stage windows
# covers, by path (see ssd_chunk_scan_fwd_fused_states)
def stage_steps(w: workloads.FwdWorkload, nseg: int) -> dict:
    mfma = w.dtype == "bf16" and w.dstate in (32, 64, 128, 256) and w.headdim in (32, 64, 128) and w.chunk_len >= 32
    if not mfma:
        return {s: [s] for s in STAGES}
    if nseg == 0:
        return {"chunk_cumsum": [], "chunk_state": ["chunk_cumsum", "chunk_state"],
                "state_passing": ["state_passing"], "chunk_scan": ["chunk_scan"]}
    # fused walk: sums, chunk states and the passing inside each segment;
    # with segments, stage 2 is the short recurrence over the segments
    return {"chunk_cumsum": [], "chunk_state": ["chunk_cumsum", "chunk_state", "state_passing"],
            "state_passing": [], "chunk_scan": ["chunk_scan"]}


def fwd_report(w: workloads.FwdWorkload, r: dict, nseg: int) -> tuple:
    """Per-launch entries and the roofline of the dominant launch."""
    alg, impl, cov = alg_work(w), impl_work(w, nseg), stage_steps(w, nseg)
    kernels = {}
    for s in STAGES:
        if impl[s]["bytes"] == 0 and not cov[s]:
            continue                      # empty window on this path
        ms = max(r["stage_ms"][s], 1e-6)
        ab = sum(alg[k]["bytes"] for k in cov[s]) or impl[s]["bytes"]
        af = sum(alg[k]["flops"] for k in cov[s])
        kernels[s] = {"ms": round(ms, 5), "covers": cov[s] or ["recurrence over segments"],
                      "alg_bytes": ab, "alg_GB_per_s": round(ab / (ms * 1e-3) / 1e9, 1),
                      "alg_TFLOP_per_s": round(af / (ms * 1e-3) / 1e12, 2), "alg_flops": af,
                      "impl_bytes": impl[s]["bytes"],
                      "impl_GB_per_s": round(impl[s]["bytes"] / (ms * 1e-3) / 1e9, 1)}
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    k = kernels[dom]
    achieved = k["alg_GB_per_s"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counted_traffic(dom, w.tag),
                "kernel": dom, "alg_bytes_per_launch": k["alg_bytes"],
                "alg_bytes_basis": "minimal I/O of the covered steps of the four-step chunked algorithm "
                                   "(fp32 chunk states between the steps), per launch",
                "impl_bytes_per_launch": k["impl_bytes"],
                "impl_frac": round(k["impl_GB_per_s"] / HBM_PEAK_GBS, 4),
                "mfma_frac_alg": round(k["alg_TFLOP_per_s"] / MFMA_BF16_PEAK_TFLOPS, 4)}
    return kernels, roofline


def plan_of(w: workloads.FwdWorkload) -> int:
    import selective_state_space_46_amd as ssd
    return ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                               w.chunk_len, ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=workloads.LONG_128K.name,
                    choices=sorted(workloads.FWD_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip decode / other workloads")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run a few forward calls and three copies of a 256 MiB buffer (for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs and their calibration)")
    ap.add_argument("--decode-probe", action="store_true",
                    help="only run eight decode updates and the calibration copies (for rocprofv3 --pmc)")
    ap.add_argument("--backward-probe", action="store_true",
                    help="only run a few backward calls on the 130M-shaped layer (for rocprofv3 --pmc)")
    ap.add_argument("--extras-only", action="store_true",
                    help="only the sections beside the headline (decode, backward, packed sequences, "
                         "stages next to the core), one JSON line (for kernel traces of them)")
    ap.add_argument("--peaks", action="store_true", help="only the measured MFMA and copy rates, one JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip = Hip()
    w = workloads.FWD_WORKLOADS[args.workload]
    if args.traffic_probe:
        traffic_probe(w)
        return
    if args.decode_probe:
        decode_probe()
        return
    if args.backward_probe:
        backward_probe()
        return
    if args.peaks:
        print(json.dumps(measured_peaks(hip)), flush=True)
        return
    if args.extras_only:
        print(json.dumps(extras(hip)), flush=True)
        return
    log(f"[bench] {w.name}: warmup {args.warmup}, steps {args.steps}")
    r = bench_fwd(hip, w, args.steps, args.warmup)
    log(f"[bench] {r['ms_per_step']:.4f} ms/step, {r['tokens_per_s']:.4g} tok/s, stages {r['stage_ms']}")
    cold = bench_fwd(hip, w, max(3, args.steps // 4), 1, cold=True, settle=False)
    log(f"[bench] cold (Infinity Cache flushed): {cold['ms_per_step']:.4f} ms/step")
    nseg = plan_of(w)
    kernels, roofline = fwd_report(w, r, nseg)

    out = {
        "metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_len": w.chunk_len, "io_dtype": w.dtype, "state_dtype": "f32",
                   "segments_per_row": nseg},
        "roofline": roofline,
        "kernels": kernels,
        "cold_cache_ms_per_step": round(cold["ms_per_step"], 5),
    }
    if not args.no_extra:
        others = {}
        for ow in (workloads.MAMBA2_130M, workloads.MAMBA2_2P7B):
            if ow.name == w.name:
                continue
            log(f"[bench] {ow.name}")
            rr = bench_fwd(hip, ow, 20, 5)
            rc = bench_fwd(hip, ow, 5, 1, cold=True, settle=False)
            ok, oroof = fwd_report(ow, rr, plan_of(ow))
            others[ow.name] = {"tokens_per_s": round(rr["tokens_per_s"], 1),
                               "ms_per_step": round(rr["ms_per_step"], 5),
                               "cold_cache_ms_per_step": round(rc["ms_per_step"], 5),
                               "segments_per_row": plan_of(ow), "kernels": ok, "roofline": oroof}
            log(f"[bench]   {rr['ms_per_step']:.4f} ms/step (cold {rc['ms_per_step']:.4f})")
        out["other_workloads"] = others
        out.update(extras(hip))
        log("[bench] measured peaks")
        out["measured_peaks"] = measured_peaks(hip)
        log(f"[bench]   {out['measured_peaks']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on host cores")
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
