"""GPU parity of the fused chunk-state + state-passing launch (the forward
path for equal-length rows with dstate 128 or 256 and chunk_len a multiple
of 64 whose work-groups -- one per batch row and 64 columns of the flattened
(head, headdim) axis, 128 at dstate 256 with headdim 64 and chunk_len 256 --
fill a 256-unit MI355X in one round: 128 .. 256 of them, one per unit, or at
dstate 128 with chunk_len >= 128 up to 512, two per unit) against the fp64
oracle, through the C ABI.

Where whole rows give fewer walks than half the units, each row is cut into
segments walked from zero, a recurrence over the segments gives the state
entering each one, and chunk_scan adds its decayed contribution; the second
half of this file covers that form.

Every shape here takes the fused path (each test asserts the library's
choice). Bar as for the other bf16 forward cases: relative L2 <= 1e-2 on y
and on the final state, whole tensors, and per (batch row, head, chunk)
block and token row of y. Cases span several chunks with a ragged tail,
every chunk length the path takes, both dstate values, every headdim (two
heads per work-group at headdim 32, one to two work-groups per head above),
groups, no initial state, the shortest rows, fast decays, long rows, odd
batch / token / head counts, the 130M and 2.7B layers' head layouts, the
two-per-unit regime, and segments of unequal length."""
import numpy as np
import pytest

import workloads
from ssd_testlib import assert_fwd_close, fwd_errors, gpu_fwd

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _units():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _cols(N, P, q):
    """columns per walk work-group (the library's rule)"""
    return 128 if N == 256 and P == 64 and q == 256 else 64


def _w(b, T, H, P, N, G, q, seed, init=True, dt_mode="softplus"):
    wgs = b * H * P // _cols(N, P, q)
    top = 512 if (N == 128 and q >= 128) else 256
    assert 128 <= wgs <= top and (P != 32 or (H // G) % 2 == 0), "shape must take the fused path"
    return workloads.with_shape(workloads.MAMBA2_130M, batch=b, seqlen=T, nheads=H, headdim=P, dstate=N,
                                ngroups=G, chunk_len=q, init="normal0.1" if init else "zero",
                                dt_mode=dt_mode, seed=seed)


def _check(w, segments=1, init_in_place=False):
    """segments: the number of segments per row the library must choose (1 =
    whole rows; 0 = any number above 1)"""
    import selective_state_space_46_amd as ssd
    got = ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                              w.chunk_len, ssd.SSD_BF16)
    assert (got > 1) if segments == 0 else (got == segments), (got, segments)
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, "bf16", w.chunk_len, init_in_place=init_in_place)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    assert_fwd_close(fwd_errors(inp, y, fin, w.chunk_len), TOL,
                     f"chain b={w.batch} T={w.seqlen} H={w.nheads} P={w.headdim} N={w.dstate} G={w.ngroups} "
                     f"Q={w.chunk_len} segments={got}")


@pytest.mark.parametrize("q", [64, 128, 256])
def test_chain_chunk_lengths_ragged(q):
    _check(_w(2, 3 * 256 + 77, 64, 64, 128, 1, q, seed=8000 + q))


@pytest.mark.parametrize("P,N,H", [(32, 128, 128), (128, 128, 32), (32, 256, 128), (64, 256, 128), (128, 256, 32)])
def test_chain_shapes(P, N, H):
    """(64, 256): 128-column work-groups (two heads each), the C B^T tiles
    in the same launch behind the walks"""
    _check(_w(2, 300, H, P, N, 1, 256, seed=8100 + P + N))


def test_chain_128_columns_groups_and_odd_heads():
    """128-column walks whose two heads share a B/C group (4 groups of 32
    heads); an odd number of heads per group at the same shape cannot pair
    its heads and takes the two-kernel path, with the same results"""
    import selective_state_space_46_amd as ssd
    _check(_w(2, 555, 128, 64, 256, 4, 256, seed=8150))
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=2, seqlen=555, nheads=129, headdim=64, dstate=256,
                             ngroups=3, chunk_len=256, init="normal0.1", seed=8151)
    assert ssd.ssd_chunk_scan_fwd_fused_states(2, 555, 129, 64, 256, 3, 256, ssd.SSD_BF16) == 0
    inp = workloads.make_fwd_inputs(w)
    y, fin = gpu_fwd(inp, "bf16", 256)
    assert_fwd_close(fwd_errors(inp, y, fin, 256), TOL, "two-kernel path, 43 heads per group")


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
    """8192-token rows: 128 slices walked in order by every chain"""
    _check(_w(2, 8192, 64, 64, 128, 1, 256, seed=8500))


@pytest.mark.parametrize("b,T,H", [(5, 301, 27), (3, 301, 45)])
def test_chain_odd_batch_tokens_heads(b, T, H):
    """batch, tokens and heads all odd (135 walks): the dt tensor's last
    element sits at an even index, the one element whose 32-bit word would
    end past the tensor -- read alone by the walk that holds it"""
    assert (b * T * H - 1) % 2 == 0
    _check(_w(b, T, H, 64, 128, 1, 256, seed=8600 + H))


# ---------------------------------------------------------------- segmented rows

def _seg_plan(b, T, H, P, N, q):
    """the segment count the library documents: whole rows give b H P / cols
    walks; below half the units each row is cut into ceil(nc / seglen)
    segments of seglen = ceil(nc / min(nc, units // walks)) chunks"""
    cus, wgs, nc = _units(), b * H * P // _cols(N, P, q), -(-T // q)
    want = min(nc, cus // wgs)
    seglen = -(-nc // want)
    nseg = -(-nc // seglen)
    return nseg if 2 * wgs * nseg >= cus else 0


def _ws(b, T, H, P, N, G, q, seed, init=True, dt_mode="softplus"):
    assert 2 * (b * H * P // _cols(N, P, q)) < _units() and _seg_plan(b, T, H, P, N, q) > 1, \
        "shape must take segments"
    return workloads.with_shape(workloads.MAMBA2_130M, batch=b, seqlen=T, nheads=H, headdim=P, dstate=N,
                                ngroups=G, chunk_len=q, init="normal0.1" if init else "zero",
                                dt_mode=dt_mode, seed=seed)


@pytest.mark.parametrize("q", [64, 128, 256])
def test_segments_long_context_shape(q):
    """the 128K-token layer's heads (24 walks of whole rows) on a 40-chunk
    row with a ragged tail, an initial state, every chunk length the fused
    walk takes (256: the state correction where H_c is staged; 64, 128:
    per fragment)"""
    w = _ws(1, 40 * 256 + 77, 24, 64, 256, 1, q, seed=8700 + q)
    _check(w, segments=_seg_plan(1, w.seqlen, 24, 64, 256, q))


@pytest.mark.parametrize("P,N,H,G", [(32, 128, 48, 2), (128, 128, 8, 1), (64, 128, 24, 4), (128, 256, 12, 3)])
def test_segments_shapes(P, N, H, G):
    _check(_ws(1, 7000, H, P, N, G, 256, seed=8800 + P + N + H), segments=0)


def test_segments_odd_batch_tokens_heads_short_last_segment():
    """b, T, H odd (the dt tail element in the last segment's last chunk); 11
    chunks in segments of 2, the last one a single chunk"""
    w = _ws(3, 2801, 9, 64, 128, 1, 256, seed=8900)
    assert (3 * 2801 * 9 - 1) % 2 == 0
    _check(w, segments=_seg_plan(3, 2801, 9, 64, 128, 256))


def test_segments_no_init_fast_decay():
    _check(_ws(2, 5000, 8, 64, 256, 1, 128, seed=8950, init=False, dt_mode="fast"), segments=0)


def test_segments_init_in_place():
    _check(_ws(1, 6000, 16, 64, 128, 2, 256, seed=8960), segments=0, init_in_place=True)


def test_fused_path_choice_on_the_workloads():
    """The 130M-shaped layer (192 work-groups, one per unit) and the 2.7B-shaped
    one (320, two per unit) take the fused launch over whole rows; the
    128K-token row (12 walks of whole rows, 128 columns each) is cut into
    segments, 21 on a 256-unit MI355X."""
    import selective_state_space_46_amd as ssd
    for w in (workloads.MAMBA2_130M, workloads.MAMBA2_2P7B, workloads.LONG_128K):
        want = 1 if w is not workloads.LONG_128K else _seg_plan(w.batch, w.seqlen, w.nheads, w.headdim,
                                                                 w.dstate, w.chunk_len)
        got = ssd.ssd_chunk_scan_fwd_fused_states(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                                  w.chunk_len, ssd.SSD_BF16)
        assert got == want, (w.name, got, want)
    if _units() == 256:
        assert _seg_plan(1, 131072, 24, 64, 256, 256) == 21
