"""GPU parity of the backward pass (ssd_chunk_scan_bwd) against the fp64
backward oracle (oracle.ssd_bwd), through the C ABI.

Bar: relative L2 <= 1e-2 for every gradient (bf16 inputs and outputs; dA,
dD, dinit fp32). Cases span several backward chunks with a ragged tail,
every chunk length the backward picks (128 for dstate 128 / headdim 64, 64
for the larger tiles, ...), groups, absent D / init / dfinal, a single
token, sequences shorter than one chunk, fast decays and the full 130M-shaped
layer."""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import dev, host, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-2
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def _inputs(b, T, H, P, N, G, seed, init=True, dfinal=True, D=True, dt_mode="softplus"):
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=b, seqlen=T, nheads=H, headdim=P, dstate=N,
                             ngroups=G, init="normal0.1" if init else "zero", dt_mode=dt_mode, seed=seed)
    inp = workloads.make_fwd_inputs(w)
    rng = np.random.default_rng(seed + 7)
    inp["dy"] = workloads.round_to_bf16(rng.standard_normal((b, T, H, P), dtype=np.float32))
    inp["dfinal"] = rng.standard_normal((b, H, N, P), dtype=np.float32) * np.float32(0.1) if dfinal else None
    if not D:
        inp["D"] = None
    return inp


def _check(inp, tol=TOL):
    import torch
    import selective_state_space_46_amd as ssd
    g = ssd.ssd_chunk_scan_bwd(dev(inp["x"], "bf16"), dev(inp["dt"], "bf16"), dev(inp["A"]),
                               dev(inp["B"], "bf16"), dev(inp["C"], "bf16"),
                               dev(inp["D"]) if inp["D"] is not None else None,
                               dev(inp["init"]) if inp["init"] is not None else None,
                               dev(inp["dy"], "bf16"),
                               dev(inp["dfinal"]) if inp["dfinal"] is not None else None)
    torch.cuda.synchronize()
    ref = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init"], inp["dy"],
                         inp["dfinal"])
    errs = {}
    for k in NAMES:
        got = host(g[k])
        assert np.all(np.isfinite(got)), k
        errs[k] = rel_l2(got, ref[k])
    b, T, H, P = inp["x"].shape
    print(f"[bwd b={b} T={T} H={H} P={P} N={inp['B'].shape[3]} G={inp['B'].shape[2]}] " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol, (k, v)
    return g, ref


def test_bwd_several_chunks_ragged():
    _check(_inputs(2, 300, 4, 64, 128, 2, seed=7000))


@pytest.mark.parametrize("P,N", [(32, 32), (64, 64), (32, 128), (128, 64), (128, 128), (64, 256), (32, 256)])
def test_bwd_shapes(P, N):
    """backward chunk lengths 128 (small tiles) and 64 (headdim 128 with dstate
    128, dstate 256)"""
    _check(_inputs(1, 200, 2, P, N, 1, seed=7100 + P + N))


def test_bwd_without_optional_inputs():
    _check(_inputs(1, 257, 3, 64, 128, 1, seed=7200, init=False, dfinal=False, D=False))


@pytest.mark.parametrize("T", [1, 5, 127, 128, 129])
def test_bwd_short_sequences(T):
    _check(_inputs(2, T, 2, 64, 128, 1, seed=7300 + T))


def test_bwd_fast_decay():
    """dt |A| up to 32 per token: every decay factor must stay finite"""
    _check(_inputs(1, 300, 4, 64, 128, 1, seed=7400, dt_mode="fast"))


def test_bwd_deterministic_and_repeated_calls():
    import torch
    import selective_state_space_46_amd as ssd
    inp = _inputs(1, 260, 4, 64, 128, 2, seed=7500)
    args = [dev(inp["x"], "bf16"), dev(inp["dt"], "bf16"), dev(inp["A"]), dev(inp["B"], "bf16"),
            dev(inp["C"], "bf16"), dev(inp["D"]), dev(inp["init"]), dev(inp["dy"], "bf16"), dev(inp["dfinal"])]
    g1 = ssd.ssd_chunk_scan_bwd(*args)
    g2 = ssd.ssd_chunk_scan_bwd(*args)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_full_130m_layer():
    w = workloads.MAMBA2_130M
    inp = _inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, seed=7600)
    _check(inp)


@pytest.mark.parametrize("b,T,H,G", [(2, 300, 4, 4), (8, 4096, 2, 1)])
def test_bwd_whole_group_per_work_group(b, T, H, G):
    """one work-group holds every head of its group (one head per group, or
    256 (batch, chunk, group) items, a work-group per compute unit already):
    dB and dC are written as bf16 by the per-chunk kernel itself, with no fp32
    partials and no reduction after it"""
    _check(_inputs(b, T, H, 64, 128, G, seed=7650 + H + G))


def _walks(b, T, H, P, N, G):
    import selective_state_space_46_amd as ssd
    return ssd.ssd_chunk_scan_bwd_fused_walks(b, T, H, P, N, G, ssd.SSD_BF16)


@pytest.mark.parametrize("b,T,H,P,N,G", [(4, 300, 32, 64, 128, 2), (4, 330, 64, 32, 128, 4),
                                         (2, 200, 64, 128, 128, 2), (2, 260, 64, 64, 256, 4)])
def test_bwd_reverse_walk_shapes(b, T, H, P, N, G):
    """128..256 work-groups of 64 (head, p) columns: the recomputation is one
    walk and the gradients of the chunk states come from the one reverse
    walk (several chunks, ragged tail, head pairs at headdim 32, dstate 256)"""
    assert _walks(b, T, H, P, N, G) == 3
    _check(_inputs(b, T, H, P, N, G, seed=7700 + P + N + H))


def test_bwd_reverse_walk_without_optional_inputs():
    assert _walks(4, 300, 32, 64, 128, 2) == 3
    _check(_inputs(4, 300, 32, 64, 128, 2, seed=7800, init=False, dfinal=False, D=False))


def test_bwd_reverse_walk_odd_batch_tokens_heads():
    """b, T, H all odd (135 walks): the dt tensor's last element at an even
    index, read alone by both walks that reach it"""
    assert _walks(3, 301, 45, 64, 128, 1) == 3
    _check(_inputs(3, 301, 45, 64, 128, 1, seed=7850))


def test_bwd_two_walks_per_unit():
    """320 walks (the 2.7B layer's heads, batch 4): the recomputation runs two
    walks per unit (three slices resident, fp32 states and tiles); the state
    gradients take the per-chunk launch and the reverse state passing"""
    assert _walks(4, 300, 80, 64, 128, 1) == 1
    _check(_inputs(4, 300, 80, 64, 128, 1, seed=7900))


def test_bwd_path_choice():
    """the 130M layer's backward (chunk 128: 192 walks) takes both walks; a
    small problem (8 walks) neither"""
    assert _walks(8, 2048, 24, 64, 128, 1) == 3
    assert _walks(1, 300, 8, 64, 128, 1) == 0
