"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: relative L2 error (||gpu - oracle||_2 / ||oracle||_2) <= 1e-5 on the
fp32 path and <= 1e-2 on y and final_state on the bf16 path, over the whole
tensor of every workload, full sizes included -- and the same bar for every
(batch row, head, chunk) block of y and every token row of y, so that an
error confined to one chunk, ragged tail or token is not diluted by the rest.
"""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import assert_fwd_close, dev, fwd_dev, fwd_errors, gpu_fwd, host, rel_l2

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _check_full(w, inp, chunk_len=None, init_in_place=False):
    q = chunk_len or w.chunk_len
    y, fin = gpu_fwd(inp, w.dtype, q, init_in_place=init_in_place)
    assert np.all(np.isfinite(y))
    assert_fwd_close(fwd_errors(inp, y, fin, q), TOL[w.dtype], f"{w.name} Q={q}")
    return y, fin


# ---------------------------------------------------------------- small cases

def test_tiny_f32_workload():
    w = workloads.TINY_F32
    _check_full(w, workloads.make_fwd_inputs(w))


@pytest.mark.parametrize("q", [16, 32, 64, 128, 256])
def test_tiny_f32_chunk_len_invariance(q):
    w = workloads.TINY_F32
    _check_full(w, workloads.make_fwd_inputs(w), chunk_len=q)


@pytest.mark.parametrize("T", [1, 15, 63, 64, 65, 200, 257])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_lengths(T, dtype):
    w = workloads.with_shape(workloads.TINY_F32, batch=2, seqlen=T, nheads=4, ngroups=2,
                             dtype=dtype, init="normal0.1", seed=900 + T)
    _check_full(w, workloads.make_fwd_inputs(w))


@pytest.mark.parametrize("P,N,G,H", [(16, 16, 1, 2), (8, 24, 2, 4), (64, 128, 1, 3), (32, 64, 4, 8),
                                     (3, 5, 1, 2), (128, 32, 1, 2), (64, 256, 1, 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shapes(P, N, G, H, dtype):
    w = workloads.with_shape(workloads.TINY_F32, batch=2, seqlen=300, nheads=H, headdim=P,
                             dstate=N, ngroups=G, chunk_len=64, dtype=dtype, init="normal0.1",
                             seed=1000 + P + N)
    _check_full(w, workloads.make_fwd_inputs(w))


@pytest.mark.parametrize("q", [32, 64, 128, 256])
def test_bf16_large_shape_small_batch(q):
    """The 130M-layer shapes (H, P, N) on a short sequence that several chunks and
    a ragged tail span, checked on every element."""
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=2, seqlen=3 * 256 + 77, init="normal0.1",
                             chunk_len=q, seed=1200 + q)
    _check_full(w, workloads.make_fwd_inputs(w))


@pytest.mark.parametrize("dtype,q", [("f32", 64), ("bf16", 64), ("bf16", 256)])
def test_fast_decay(dtype, q):
    """dt |A| up to 32 per token: the summed exponent over 31 tokens reaches
    about 280 here, far outside the fp32 range (about 88), so any product of decay
    factors in which one factor has a positive exponent overflows. Every
    output must stay finite and within the bar."""
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=2, seqlen=2 * 256 + 77, dt_mode="fast",
                             init="normal0.1", chunk_len=q, dtype=dtype, seed=1400 + q)
    inp = workloads.make_fwd_inputs(w)
    assert float(np.max(inp["dt"][..., None] * -inp["A"])) > 20.0
    _check_full(w, inp)


def test_long_context_shape_short_sequence():
    w = workloads.with_shape(workloads.LONG_128K, seqlen=4 * 256 + 3, seed=1300)
    _check_full(w, workloads.make_fwd_inputs(w))


def test_init_state_in_place():
    w = workloads.with_shape(workloads.TINY_F32, batch=2, seqlen=129, init="normal0.1", seed=1400)
    _check_full(w, workloads.make_fwd_inputs(w), init_in_place=True)


def test_no_D_no_final():
    import selective_state_space_46_amd as ssd
    import torch
    w = workloads.with_shape(workloads.TINY_F32, seqlen=100, seed=1500)
    inp = workloads.make_fwd_inputs(w)
    y, fin = ssd.ssd_chunk_scan_fwd(dev(inp["x"]), dev(inp["dt"]), dev(inp["A"]), dev(inp["B"]),
                                    dev(inp["C"]), None, None, 64, return_final_state=False)
    torch.cuda.synchronize()
    assert fin is None
    y_ref, _ = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, None)
    assert rel_l2(host(y), y_ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_and_resume(dtype):
    """fwd(T1) then fwd(T2, init = final of the first) equals fwd(T1 + T2)."""
    w = workloads.with_shape(workloads.MAMBA2_130M if dtype == "bf16" else workloads.TINY_F32,
                             batch=2, seqlen=700, init="normal0.1", chunk_len=64, seed=1600)
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, dtype, 64)
    T1 = 300
    a = {k: (v[:, :T1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    ya, fa = gpu_fwd(a, dtype, 64)
    bb = {k: (v[:, T1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    bb["init"] = fa.astype(np.float32)
    yb, fb = gpu_fwd(bb, dtype, 64)
    assert rel_l2(np.concatenate([ya, yb], axis=1), y) <= TOL[dtype]
    assert rel_l2(fb, fin) <= TOL[dtype]


def test_deterministic():
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=2, seqlen=1000, seed=1700)
    inp = workloads.make_fwd_inputs(w)
    y1, f1 = gpu_fwd(inp, "bf16", 256)
    y2, f2 = gpu_fwd(inp, "bf16", 256)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(f1, f2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_timed_entry_point(dtype):
    """The timed entry point computes bit-for-bit what the plain one does, and
    its per-stage event pairs give ordered, non-negative kernel times."""
    import torch
    import selective_state_space_46_amd as ssd
    from ssd_testlib import HipEvents
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=2, seqlen=700, dtype=dtype,
                             init="normal0.1", seed=1750)
    inp = workloads.make_fwd_inputs(w)
    x, dt, B, C = (dev(inp[k], dtype) for k in ("x", "dt", "B", "C"))
    A, D, init = dev(inp["A"]), dev(inp["D"]), dev(inp["init"])
    y1, f1 = ssd.ssd_chunk_scan_fwd(x, dt, A, B, C, D, init, 256)
    hip = HipEvents()
    ev = hip.create(8)
    y2, f2 = ssd.ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init, 256, stage_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    stage = [hip.ms(ev[2 * i], ev[2 * i + 1]) for i in range(4)]
    gaps = [hip.ms(ev[2 * i + 1], ev[2 * i + 2]) for i in range(3)]
    hip.destroy(ev)
    print(f"[timed {dtype}] stage ms {stage} gaps {gaps}", flush=True)
    assert all(t >= 0.0 for t in stage) and all(g >= 0.0 for g in gaps)
    assert all(t > 0.0 for t in stage[1:])          # stages 1..3 always launch a kernel
    with pytest.raises(ValueError):
        ssd.ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init, 256, stage_events=ev[:5])


# ---------------------------------------------------------------- decode

def _gpu_decode(inp, dtype, steps=None):
    import torch
    import selective_state_space_46_amd as ssd
    state = dev(inp["state"])
    A, D = dev(inp["A"]), dev(inp["D"])
    S = inp["xs"].shape[0] if steps is None else steps
    ys = []
    for s in range(S):
        y = ssd.ssd_state_update(state, dev(inp["xs"][s], dtype), dev(inp["dts"][s], dtype), A,
                                 dev(inp["Bs"][s], dtype), dev(inp["Cs"][s], dtype), D)
        ys.append(y)
    torch.cuda.synchronize()
    return np.stack([host(y) for y in ys]), host(state)


@pytest.mark.parametrize("dtype,P,N,G,H", [("f32", 64, 128, 2, 4), ("bf16", 64, 128, 8, 16),
                                           ("f32", 6, 10, 1, 3), ("bf16", 16, 16, 1, 2)])
def test_decode_small(dtype, P, N, G, H):
    w = workloads.DecodeWorkload("dec", 3, H, P, N, G, 5, dtype, seed=1800 + P)
    inp = workloads.make_decode_inputs(w)
    ys, st = _gpu_decode(inp, dtype)
    ys_ref, st_ref = oracle.ssd_decode(inp["state"], inp["xs"], inp["dts"], inp["A"], inp["Bs"],
                                       inp["Cs"], inp["D"])
    ey, es = rel_l2(ys, ys_ref), rel_l2(st, st_ref)
    print(f"[decode {dtype} P{P} N{N}] y={ey:.3e} state={es:.3e}", flush=True)
    assert ey <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_equals_chained_decode(dtype):
    """Parallel (chunked) form and recurrent form give the same result."""
    w = workloads.with_shape(workloads.TINY_F32, batch=2, seqlen=70, nheads=4, headdim=16,
                             dstate=32, ngroups=2, init="normal0.1", dtype=dtype, chunk_len=32,
                             seed=1900)
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, dtype, 32)
    dinp = dict(state=inp["init"], xs=inp["x"].transpose(1, 0, 2, 3), dts=inp["dt"].transpose(1, 0, 2),
                A=inp["A"], Bs=inp["B"].transpose(1, 0, 2, 3), Cs=inp["C"].transpose(1, 0, 2, 3),
                D=inp["D"])
    ys, st = _gpu_decode(dinp, dtype)
    assert rel_l2(ys.transpose(1, 0, 2, 3), y) <= TOL[dtype]
    assert rel_l2(st, fin) <= TOL[dtype]


# ---------------------------------------------------------------- full sizes

def _check_workload_whole(w):
    """A named workload at its full size, in the launch configuration bench.py
    times, every element of y and of the final state against the oracle."""
    import selective_state_space_46_amd as ssd
    inp = workloads.make_fwd_inputs(w)
    plan = ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                               w.chunk_len, ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32)
    print(f"[{w.name}] states entering each chunk: {'fused walk, %d segment(s) per row' % plan if plan else 'two launches'}",
          flush=True)
    y, fin = fwd_dev(inp, w.dtype, w.chunk_len)
    assert_fwd_close(fwd_errors(inp, y, fin, w.chunk_len), TOL[w.dtype], w.name)


@pytest.mark.slow
def test_mamba2_130m_full():
    _check_workload_whole(workloads.MAMBA2_130M)


@pytest.mark.slow
def test_mamba2_2p7b_full():
    _check_workload_whole(workloads.MAMBA2_2P7B)


@pytest.mark.slow
def test_long_context_full():
    _check_workload_whole(workloads.LONG_128K)


@pytest.mark.slow
def test_decode_full_size_every_head():
    """The batch-256 decode workload, 64 chained steps on fresh inputs: every y
    of every step and the whole state after the last step against the oracle
    (streamed over blocks of batch rows), plus the worst relative L2 of any
    single (batch row, head) over the 64 steps."""
    w = workloads.DECODE_B256
    inp = workloads.make_decode_inputs(w)
    ys, st = _gpu_decode(inp, w.dtype)
    sd = sr = fd = fr = 0.0
    worst = 0.0
    rows = 32
    for b0 in range(0, w.batch, rows):
        heads = [(b, h) for b in range(b0, min(w.batch, b0 + rows)) for h in range(w.nheads)]
        ys_ref, st_ref = oracle.ssd_decode(inp["state"], inp["xs"], inp["dts"], inp["A"], inp["Bs"],
                                           inp["Cs"], inp["D"], heads=heads)
        nb = len(heads) // w.nheads
        yg = ys[:, b0:b0 + nb].transpose(1, 2, 0, 3).reshape(len(heads), w.steps, w.headdim)
        sg = st[b0:b0 + nb].reshape(len(heads), w.dstate, w.headdim)
        d2 = ((yg - ys_ref) ** 2).sum(axis=(1, 2))
        r2 = (ys_ref ** 2).sum(axis=(1, 2))
        sd += float(d2.sum()); sr += float(r2.sum())
        worst = max(worst, float(np.max(np.sqrt(d2 / r2))))
        fd += float(((sg - st_ref) ** 2).sum()); fr += float((st_ref ** 2).sum())
    ey, es = np.sqrt(sd / sr), np.sqrt(fd / fr)
    print(f"[{w.name}] every head: y={ey:.3e} state={es:.3e} worst head y={worst:.3e}", flush=True)
    assert ey <= 1e-2 and es <= 1e-2 and worst <= 1e-2


# ---------------------------------------------------------------- errors on device tensors

def test_errors_leave_outputs_untouched():
    import torch
    import selective_state_space_46_amd as ssd
    L = ssd.lib()
    x = torch.zeros(1, 64, 2, 16, device="cuda")
    y = torch.full_like(x, 7.0)
    dt = torch.zeros(1, 64, 2, device="cuda")
    A = torch.zeros(2, device="cuda")
    B = torch.zeros(1, 64, 1, 16, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = lambda **k: dict(dict(x=x.data_ptr(), y=y.data_ptr(), q=64, ws=ws.data_ptr(), nbytes=ws.numel()), **k)

    def call(a):
        return L.ssd_chunk_scan_fwd(a["x"], dt.data_ptr(), A.data_ptr(), B.data_ptr(), B.data_ptr(),
                                    None, None, a["y"], None, 1, 64, 2, 16, 16, 1, a["q"], 0,
                                    a["ws"], a["nbytes"], s)

    assert call(args(q=48)) == 4
    assert call(args(nbytes=16)) == 5
    assert call(args(y=x.data_ptr())) == 7             # y aliases x
    assert call(args(x=x.data_ptr() + 4)) == 8         # misaligned
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)                        # failed calls wrote nothing
    assert call(args()) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 0)                          # the good call wrote y (x = 0, so y = 0)
