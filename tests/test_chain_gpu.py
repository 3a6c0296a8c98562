"""GPU parity of the fused chunk-state + state-passing launch (the forward
path for equal-length rows with dstate 128 or 256 and chunk_len a multiple
of 64 whose work-groups -- one per batch row and 64 columns of the flattened
(head, headdim) axis -- fill a 256-unit MI355X in one round: 128 .. 256 of
them, one per unit, or at dstate 128 with chunk_len >= 128 up to 512, two per
unit) against the fp64 oracle, through the C ABI.

Every shape here takes that path. Bar as for the other
bf16 forward cases: relative L2 <= 1e-2 on y and on the final state. Cases
span several chunks with a ragged tail, every chunk length the path takes,
both dstate values, every headdim (two heads per work-group at headdim 32,
one to two work-groups per head above), groups, no initial state, the
shortest rows, fast decays, long rows, the 130M and 2.7B layers' head
layouts, and the two-per-unit regime."""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import columns_of, gpu_fwd, rel_l2, sample_columns

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _w(b, T, H, P, N, G, q, seed, init=True, dt_mode="softplus"):
    wgs = b * H * P // 64
    top = 512 if (N == 128 and q >= 128) else 256
    assert 128 <= wgs <= top and (P != 32 or (H // G) % 2 == 0), "shape must take the fused path"
    return workloads.with_shape(workloads.MAMBA2_130M, batch=b, seqlen=T, nheads=H, headdim=P, dstate=N,
                                ngroups=G, chunk_len=q, init="normal0.1" if init else "zero",
                                dt_mode=dt_mode, seed=seed)


def _check(w):
    import selective_state_space_46_amd as ssd
    assert ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                               w.chunk_len, ssd.SSD_BF16)
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, "bf16", w.chunk_len)
    y_ref, fin_ref = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["init"])
    ey, ef = rel_l2(y, y_ref), rel_l2(fin, fin_ref)
    print(f"[chain b={w.batch} T={w.seqlen} H={w.nheads} P={w.headdim} N={w.dstate} G={w.ngroups} "
          f"Q={w.chunk_len}] y={ey:.3e} final={ef:.3e}", flush=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    assert ey <= TOL and ef <= TOL, (ey, ef)


@pytest.mark.parametrize("q", [64, 128, 256])
def test_chain_chunk_lengths_ragged(q):
    _check(_w(2, 3 * 256 + 77, 64, 64, 128, 1, q, seed=8000 + q))


@pytest.mark.parametrize("P,N,H", [(32, 128, 128), (128, 128, 32), (32, 256, 128), (64, 256, 64), (128, 256, 32)])
def test_chain_shapes(P, N, H):
    _check(_w(2, 300, H, P, N, 1, 256, seed=8100 + P + N))


def test_chain_groups_no_init():
    _check(_w(2, 520, 64, 64, 128, 4, 128, seed=8200, init=False))


def test_chain_head_pairs_in_groups():
    """headdim 32: each work-group takes two heads, which share their B/C group"""
    _check(_w(2, 410, 128, 32, 128, 4, 128, seed=8250))


def test_chain_130m_head_layout():
    """the 130M layer's batch and heads (192 work-groups) on a shorter row"""
    _check(_w(8, 700, 24, 64, 128, 1, 256, seed=8260))


def test_chain_2p7b_head_layout_two_per_unit():
    """the 2.7B layer's batch and heads (320 work-groups: two per unit, three
    slices resident) with an initial state, on a shorter ragged row"""
    _check(_w(4, 777, 80, 64, 128, 1, 256, seed=8270))


@pytest.mark.parametrize("P,H,G", [(32, 192, 2), (64, 96, 1), (128, 48, 4)])
def test_chain_two_per_unit_shapes(P, H, G):
    """384 work-groups at chunk length 128, every headdim"""
    _check(_w(4, 500, H, P, 128, G, 128, seed=8280 + P))


@pytest.mark.parametrize("T", [1, 63, 64, 65])
def test_chain_short_rows(T):
    _check(_w(4, T, 64, 64, 128, 2, 64, seed=8300 + T))


def test_chain_fast_decay():
    """dt |A| up to 32 per token: the chunk decays underflow toward zero"""
    _check(_w(2, 600, 64, 64, 128, 1, 256, seed=8400, dt_mode="fast"))


def test_chain_long_row():
    """8192-token rows: 128 slices walked in order by every chain (checked on
    sampled (b, h, p) columns, which the oracle computes one by one)"""
    import selective_state_space_46_amd as ssd
    w = _w(2, 8192, 64, 64, 128, 1, 256, seed=8500)
    assert ssd.ssd_chunk_scan_fwd_fused_states(2, 8192, 64, 64, 128, 1, 256, ssd.SSD_BF16)
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, "bf16", w.chunk_len)
    cols = sample_columns(w.batch, w.nheads, w.headdim, 32, seed=w.seed)
    yc_ref, fc_ref = oracle.ssd_fwd_columns(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                            inp["init"], cols)
    yc, fc = columns_of(y, fin, cols)
    ey, ef = rel_l2(yc, yc_ref), rel_l2(fc, fc_ref)
    print(f"[chain long row] sampled {len(cols)} columns: y={ey:.3e} final={ef:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert ey <= TOL and ef <= TOL, (ey, ef)


def test_fused_path_choice_on_the_workloads():
    """The 130M-shaped layer (192 work-groups, one per unit) and the 2.7B-shaped
    one (320, two per unit) take the fused launch; the 128K-token row (24
    work-groups) does not."""
    import selective_state_space_46_amd as ssd
    for w, want in ((workloads.MAMBA2_130M, True), (workloads.MAMBA2_2P7B, True), (workloads.LONG_128K, False)):
        got = ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                                  w.chunk_len, ssd.SSD_BF16)
        assert got == want, w.name
