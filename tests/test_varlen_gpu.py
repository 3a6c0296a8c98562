"""GPU parity of packed variable-length sequences (ssd_chunk_scan_fwd_varlen)
against the fp64 oracle (oracle.ssd_fwd_varlen), through the C ABI, and
against the equal-length forward run on the same sequences.

Bar: relative L2 <= 1e-2 on y and on the final states (bf16 tensors, fp32
states). Sequence layouts cover empty sequences, sequences shorter than a
chunk, exact multiples of the chunk and long ones, several chunk lengths
(one and several chunks per 256-token work-group in chunk_scan). At dstate
128 and 256 the call takes the fused walk over equal segments of the packed
row of chunks (ssd_chunk_scan_fwd_varlen_plan): sequences that begin and end
inside one segment, several per segment, and sequences across one or more
segment boundaries; at dstate 32 and 64 the per-chunk launches."""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import dev, host, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _inputs(total, H, P, N, G, nseq, seed, with_init=True):
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=1, seqlen=total, nheads=H, headdim=P, dstate=N,
                             ngroups=G, init="zero", seed=seed)
    inp = workloads.make_fwd_inputs(w)
    rng = np.random.default_rng(seed + 1)
    init = (rng.standard_normal((nseq, H, N, P), dtype=np.float32) * np.float32(0.1)) if with_init else None
    return {k: (v[0] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()} | {"init": init}


def _plan(inp, cu, Q):
    """(segments, chunk slots per segment) the call takes on this device"""
    import torch
    import selective_state_space_46_amd as ssd
    T, H, P = inp["x"].shape
    N, G = inp["B"].shape[2], inp["B"].shape[1]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return ssd.ssd_chunk_scan_fwd_varlen_plan(T, len(cu) - 1, H, P, N, G, Q, ssd.SSD_BF16, cus)


def _gpu(inp, cu, Q, final_in_place=False):
    import torch
    import selective_state_space_46_amd as ssd
    x, dt, B, C = (dev(inp[k], "bf16") for k in ("x", "dt", "B", "C"))
    A, D = dev(inp["A"]), dev(inp["D"])
    init = dev(inp["init"]) if inp["init"] is not None else None
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    fin = init if (final_in_place and init is not None) else None
    y, f = ssd.ssd_chunk_scan_fwd_varlen(x, dt, A, B, C, D, cu_d, init, Q, final_states=fin)
    torch.cuda.synchronize()
    return host(y), host(f)


def _check(inp, cu, Q, final_in_place=False):
    y, f = _gpu(inp, cu, Q, final_in_place)
    y_ref, f_ref = oracle.ssd_fwd_varlen(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], cu,
                                         inp["init"])
    ey, ef = rel_l2(y, y_ref), rel_l2(f, f_ref)
    nseg, L = _plan(inp, cu, Q)
    print(f"[varlen Q={Q} nseq={len(cu) - 1} segments={nseg} of {L} slots] rel_l2 y={ey:.3e} final={ef:.3e}",
          flush=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(f))
    assert ey <= TOL and ef <= TOL, (ey, ef)
    return y, f, y_ref


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_varlen_mixed_lengths(Q):
    lens = [300, 0, 17, 256, 1, 129, 64, 511, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 4, 64, 128, 2, len(lens), seed=6000 + Q)
    _check(inp, cu, Q)


def test_varlen_no_init_and_in_place_final():
    lens = [100, 200, 0, 57]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 3, 64, 64, 1, len(lens), seed=6100, with_init=False)
    _check(inp, cu, 64)
    inp = _inputs(cu[-1], 3, 64, 64, 1, len(lens), seed=6101)
    _check(inp, cu, 64, final_in_place=True)


@pytest.mark.parametrize("P,N", [(32, 32), (128, 256), (64, 256)])
def test_varlen_shapes(P, N):
    lens = [70, 300, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 2, P, N, 1, len(lens), seed=6200 + P + N)
    _check(inp, cu, 128)


@pytest.mark.parametrize("N", [64, 128])
def test_varlen_equals_equal_length_batch(N):
    """Sequences of one length packed against the batched forward on the same
    rows: bit for bit where both take the per-chunk launches (dstate 64);
    where the packed call walks segments (dstate 128) the two round
    differently, and agree within the bf16 bar, each with the oracle too."""
    import torch
    import selective_state_space_46_amd as ssd
    nseq, L, H, P = 3, 600, 4, 64
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=nseq, seqlen=L, nheads=H, headdim=P, dstate=N,
                             init="normal0.1", seed=6300)
    inp = workloads.make_fwd_inputs(w)
    xb, dtb, Bb, Cb = (dev(inp[k], "bf16") for k in ("x", "dt", "B", "C"))
    A, D, init = dev(inp["A"]), dev(inp["D"]), dev(inp["init"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for Q in (128, 256):
        yb, fb = ssd.ssd_chunk_scan_fwd(xb, dtb, A, Bb, Cb, D, init, Q)
        cu = torch.arange(0, (nseq + 1) * L, L, dtype=torch.int32, device="cuda")
        yv, fv = ssd.ssd_chunk_scan_fwd_varlen(xb.reshape(nseq * L, H, P), dtb.reshape(nseq * L, H),
                                               A, Bb.reshape(nseq * L, 1, N), Cb.reshape(nseq * L, 1, N), D, cu,
                                               init, Q)
        torch.cuda.synchronize()
        walked = ssd.ssd_chunk_scan_fwd_varlen_plan(nseq * L, nseq, H, P, N, 1, Q, ssd.SSD_BF16, cus)[0] > 0
        batched_walk = ssd.ssd_chunk_scan_fwd_plan(nseq, L, H, P, N, 1, Q, ssd.SSD_BF16, cus)[0] > 0
        assert walked == (N == 128), (N, Q)
        if not walked and not batched_walk:
            assert torch.equal(yv.reshape(nseq, L, H, P), yb), Q
            assert torch.equal(fv, fb), Q
            continue
        y_ref, f_ref = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init"])
        ev, efv = rel_l2(host(yv).reshape(nseq, L, H, P), y_ref), rel_l2(host(fv), f_ref)
        eb, efb = rel_l2(host(yb), y_ref), rel_l2(host(fb), f_ref)
        ex, efx = rel_l2(host(yv).reshape(nseq, L, H, P), host(yb)), rel_l2(host(fv), host(fb))
        print(f"[varlen vs batch N={N} Q={Q}] packed {ev:.3e}/{efv:.3e} batched {eb:.3e}/{efb:.3e} "
              f"between {ex:.3e}/{efx:.3e}", flush=True)
        assert max(ev, efv, eb, efb, ex, efx) <= TOL


def test_varlen_long_packed_workload():
    """The long packed workload that bench.py times (131072 tokens in 8
    sequences of 4.9K .. 28.9K tokens, dstate 256, per-sequence initial
    states: several segments per sequence), whole output against the oracle,
    and per sequence."""
    vw = workloads.VARLEN_LONG
    vi = workloads.make_varlen_inputs(vw)
    cu = vi["cu_seqlens"].tolist()
    inp = {k: vi[k] for k in ("x", "dt", "A", "B", "C", "D", "init")}
    nseg, L = _plan(inp, cu, vw.chunk_len)
    assert nseg > 1 and L * vw.chunk_len < max(np.diff(cu)), (nseg, L)   # a sequence crosses segments
    y, _, y_ref = _check(inp, cu, vw.chunk_len)
    worst = max(rel_l2(y[a:b], y_ref[a:b]) for a, b in zip(cu[:-1], cu[1:]))
    print(f"[varlen long] worst sequence rel_l2 y={worst:.3e}", flush=True)
    assert worst <= TOL


def test_varlen_130m_packed_workload():
    """The packed 130M-shaped workload that bench.py times (16384 tokens,
    sequences of 64 .. 4096 tokens, per-sequence initial states), whole
    output against the oracle."""
    vw = workloads.VARLEN_130M
    vi = workloads.make_varlen_inputs(vw)
    cu = vi["cu_seqlens"].tolist()
    inp = {k: vi[k] for k in ("x", "dt", "A", "B", "C", "D", "init")}
    _check(inp, cu, vw.chunk_len)


@pytest.mark.parametrize("N", [64, 128])
def test_varlen_malformed_offsets_stay_in_bounds(N):
    """Offsets that decrease or leave [0, T] are clamped on the device: the
    call completes and writes finite values (results unspecified). dstate 64:
    the per-chunk launches; 128: the walks over segments, whose tables the
    clamped spans fill (two sequences may then share a chunk slot)."""
    import torch
    import selective_state_space_46_amd as ssd
    inp = _inputs(200, 2, 64, N, 1, 5, seed=6500)
    x, dt, B, C = (dev(inp[k], "bf16") for k in ("x", "dt", "B", "C"))
    A, D = dev(inp["A"]), dev(inp["D"])
    cu = torch.tensor([0, 150, 90, 400, -5, 10**6], dtype=torch.int32, device="cuda")
    print(f"[varlen malformed N={N}] plan {_plan(inp, cu.tolist(), 64)}", flush=True)
    y, f = ssd.ssd_chunk_scan_fwd_varlen(x, dt, A, B, C, D, cu, None, 64)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(f)))


@pytest.mark.parametrize("Q,N,with_init", [(256, 128, True), (128, 128, False), (64, 128, True), (256, 256, True)])
def test_varlen_long_sequences_span_segments(Q, N, with_init):
    """Sequences longer than several segments (their chunks past the first
    segment take the state entering theirs through the recurrence over
    segments, their final state completed there) next to short and empty
    ones, several in a segment, with and without initial states, final
    states in place; 24 heads so that segments stay short."""
    lens = [4000, 0, 90, 2500, 256, 1, 3100]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 24, 64, N, 1, len(lens), seed=6600 + Q + N, with_init=with_init)
    nseg, L = _plan(inp, cu, Q)
    assert nseg > 1 and 2 * L * Q < max(lens), (nseg, L)
    _check(inp, cu, Q, final_in_place=with_init)


def test_varlen_many_short_sequences():
    """150 sequences of 0 .. 300 tokens (several restarts inside each walk,
    sequences of one chunk and less, empty ones) with initial states,
    dstate 128, chunk_len 128, 24 heads (about 21 segments): the fused walk
    over segments"""
    rng = np.random.default_rng(6700)
    lens = rng.integers(0, 301, size=150)
    lens[::17] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 24, 64, 128, 1, len(lens), seed=6701)
    nseg, L = _plan(inp, cu, 128)
    assert nseg > 1 and len(lens) >= 4 * nseg, (nseg, L)
    _check(inp, cu, 128, final_in_place=True)


def test_varlen_more_sequences_than_the_table_stages():
    """4500 sequences of 0 .. 6 tokens (more than the 4096 whose first slots
    the chunk-table kernel stages in LDS, so every slot bisects over the
    offsets in memory), no initial states, headdim 32, chunk_len 64: most
    chunk slots are a whole sequence, many sequences are empty"""
    rng = np.random.default_rng(7300)
    lens = rng.integers(0, 7, size=4500)
    lens[::13] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = _inputs(cu[-1], 2, 32, 128, 1, len(lens), seed=7301, with_init=False)
    assert len(lens) > 4096
    nseg, L = _plan(inp, cu, 64)
    assert nseg > 1, (nseg, L)
    _check(inp, cu, 64)
