"""CPU checks of host-side index arithmetic that the GPU kernels rely on.

The fused chunk-state walk reads dt (bf16, [b, T, H]) as aligned 32-bit words:
element e lives in the word that starts at element e & ~1, and the tensor's
last element, when its index is even, is read alone with a 16-bit load (its
word would end past the tensor). These tests restate that addressing in
numpy and check, over many shapes (odd and even b, T, H; one or two heads
per walk; every chunk length the walk takes), that every 32-bit load is
4-byte aligned and inside the tensor, that the one 16-bit load happens only
on the uniform tail branch the kernel takes for it, and that the half picked
out of each word is element e itself. A second group checks the cut of a
row into segments (every chunk in exactly one segment, segments in order)."""
import itertools
import os

import numpy as np
import pytest


def _dt_word_loads(nb, T, H, nhw, Q):
    """Per (walk, chunk, head of the walk, lane, i): (byte address of the load,
    its width in bytes, which half holds e, e), as the table wave forms them."""
    last_e = nb * T * H - 1
    nc = -(-T // Q)
    out = []
    for b, h0 in itertools.product(range(nb), range(0, H, nhw)):
        for c in range(nc):
            r0, n = b * T + c * Q, min(Q, T - c * Q)
            tail = (last_e & 1) == 0 and r0 + n == nb * T and h0 + nhw == H
            lanes = np.arange(64)[:, None] * 4 + np.arange(4)[None, :]        # tokens 4 lane + i
            rows = r0 + np.minimum(lanes, n - 1)
            for q in range(nhw):
                e = rows * H + h0 + q
                up = e & 1
                alone = tail & (e == last_e)
                addr = np.where(alone, 2 * e, 2 * (e - up))
                width = np.where(alone, 2, 4)
                out.append((addr.ravel(), width.ravel(), np.where(alone, 0, up).ravel(), e.ravel(), tail))
    return out, last_e


@pytest.mark.parametrize("nb,T,H,nhw,Q", [(5, 301, 27, 1, 256), (3, 301, 45, 1, 64), (2, 300, 24, 1, 128),
                                          (3, 2801, 9, 1, 256), (1, 257, 3, 1, 64), (4, 63, 2, 2, 64),
                                          (1, 1, 1, 1, 64), (3, 65, 6, 2, 128), (1, 131, 5, 1, 64)])
def test_dt_word_loads_aligned_and_in_bounds(nb, T, H, nhw, Q):
    loads, last_e = _dt_word_loads(nb, T, H, nhw, Q)
    nbytes = 2 * (last_e + 1)
    saw_alone = False
    for addr, width, half, e, tail in loads:
        assert np.all(addr >= 0) and np.all(addr + width <= nbytes), "load past the tensor"
        four = width == 4
        assert np.all(addr[four] % 4 == 0), "misaligned 32-bit load"
        assert np.all(addr[~four] % 2 == 0)
        # the half the kernel keeps is element e: byte offset 2 e
        assert np.all(addr + 2 * half == 2 * e)
        if np.any(~four):
            assert tail, "a 16-bit load outside the tail branch"
            assert np.all(e[~four] == last_e) and last_e % 2 == 0
            saw_alone = True
    assert saw_alone == (last_e % 2 == 0)


def _segments(nc, want):
    seglen = -(-nc // want)
    nseg = -(-nc // seglen)
    return [(k * seglen, min(nc, (k + 1) * seglen)) for k in range(nseg)], seglen


@pytest.mark.parametrize("nc,want", [(512, 10), (41, 10), (11, 9), (5, 5), (1, 7), (28, 16), (7, 3)])
def test_segments_cover_each_chunk_once(nc, want):
    segs, seglen = _segments(nc, want)
    covered = [c for a, b in segs for c in range(a, b)]
    assert covered == list(range(nc))
    assert all(b > a for a, b in segs)
    assert len(segs) <= want
    # chunk c's segment, as chunk_scan finds it
    for c in range(nc):
        k = c // seglen
        assert segs[k][0] <= c < segs[k][1]


# ---------------------------------------------------------------- fused walk plans

PLAN_SHAPES = [
    # b, T, H, P, N, G, Q: the named layers, odd shapes, segmented rows, short rows
    (8, 2048, 24, 64, 128, 1, 256), (4, 4096, 80, 64, 128, 1, 256), (1, 131072, 24, 64, 256, 1, 256),
    (8, 2048, 24, 64, 128, 1, 128), (5, 301, 27, 64, 128, 1, 256), (3, 301, 45, 64, 128, 1, 64),
    (3, 2801, 9, 64, 128, 1, 256), (1, 10317, 24, 64, 256, 1, 64), (1, 10317, 24, 64, 256, 1, 128),
    (2, 845, 24, 64, 128, 1, 256), (2, 845, 24, 64, 128, 1, 64), (1, 7000, 48, 32, 128, 2, 256),
    (1, 7000, 8, 128, 128, 1, 256), (2, 5000, 8, 64, 256, 1, 128), (4, 1, 64, 64, 128, 2, 64),
    (4, 63, 64, 64, 128, 2, 64), (4, 500, 96, 64, 128, 1, 128), (2, 300, 64, 128, 256, 1, 256),
]


def _cols(N, P, Q):
    """columns per walk work-group: 128 for the forward at dstate 256,
    headdim 64, chunk_len 256, else 64 (restated from the library)"""
    return 128 if N == 256 and P == 64 and Q == 256 else 64


def _plan(b, T, H, P, N, G, Q, cus=256):
    import selective_state_space_46_amd as ssd
    return ssd.ssd_chunk_scan_fwd_plan(b, T, H, P, N, G, Q, ssd.SSD_BF16, cus)


@pytest.mark.parametrize("shape", PLAN_SHAPES)
def test_walk_plan_covers_every_chunk(shape):
    """The library's plan: segments of at least one chunk that cover the row
    exactly, and walks that fill at least half of a 256-unit device and at
    most what fits there in one round."""
    b, T, H, P, N, G, Q = shape
    nseg, seglen = _plan(*shape)
    nc = -(-T // Q)
    if nseg == 0:
        assert seglen == 0
        return
    assert seglen >= 1 and (nseg - 1) * seglen < nc <= nseg * seglen
    walks = b * H * P // _cols(N, P, Q) * nseg
    assert 128 <= walks <= (512 if N == 128 and Q >= 128 else 256)
    if nseg > 1:
        assert walks <= 256


@pytest.mark.parametrize("shape", PLAN_SHAPES)
def test_walk_copies_stay_inside_the_tensors(shape):
    """Every slice copy of every walk of the library's plan, restated from the
    kernel: its token rows lie in the tensor (a partial slice repeats its
    chunk's last token), its B and x element offsets lie inside B and x, and
    the states it writes lie inside the state buffers."""
    b, T, H, P, N, G, Q = shape
    nseg, seglen = _plan(*shape)
    if nseg == 0:
        return
    cw = _cols(N, P, Q)
    nc, SPC, cpr = -(-T // Q), Q // 64, H * P // cw
    rows = np.arange(64)
    for wid in range(b * cpr * nseg):
        c0 = (wid % cpr) * cw
        seg, bb = (wid // cpr) % nseg, wid // cpr // nseg
        h0 = c0 // P
        g = h0 // (H // G)
        cbeg = seg * seglen
        ncw = min(nc, cbeg + seglen) - cbeg
        assert ncw >= 1
        for k in range(ncw * SPC):                    # the clamped copies repeat these
            ksl = cbeg * SPC + k
            c, s0 = ksl // SPC, (ksl % SPC) * 64
            r0, n = bb * T + c * Q, min(Q, T - c * Q)
            assert 0 <= c < nc and n >= 1
            tok = r0 + s0 + (rows if s0 + 64 <= n else np.minimum(rows, n - 1 - s0))
            assert tok.min() >= bb * T and tok.max() < (bb + 1) * T
            assert ((tok.max() * G + g) * N + N - 1) < b * T * G * N
            assert tok.max() * H * P + c0 + cw - 1 < b * T * H * P
        # states entering each chunk, and a segment's last local state
        hlast = (c0 + cw - 1) // P                    # the work-group's last head
        assert hlast < H and hlast // (H // G) == g   # its heads share the B group
        hmax = ((bb * nc + cbeg + ncw - 1) * H + hlast) * P * N + P * N - 1
        assert hmax < b * nc * H * P * N
        if nseg > 1:
            assert ((bb * nseg + seg) * H + hlast) * P * N + P * N - 1 < b * nseg * H * P * N
    # chunk_scan: chunk c's segment and the state entering it
    if nseg > 1:
        assert all(c // seglen < nseg for c in range(nc))


def test_walk_plan_on_other_unit_counts():
    """the plan follows the unit count it is given (no device involved)"""
    assert _plan(8, 2048, 24, 64, 128, 1, 256, cus=256) == (1, 8)
    assert _plan(8, 2048, 24, 64, 128, 1, 256, cus=128) == (1, 8)      # 192 walks, two per unit
    assert _plan(8, 2048, 24, 64, 128, 1, 256, cus=512) == (2, 4)      # under half the units: two segments
    assert _plan(1, 300, 8, 64, 128, 1, 256, cus=256) == (0, 0)        # too little work even in segments
    assert _plan(1, 131072, 24, 64, 256, 1, 256, cus=256) == (21, 25)  # 128-column walks: 12 per row
    assert _plan(1, 131072, 24, 64, 256, 1, 256, cus=0) == (0, 0)


# ---------------------------------------------------------------- bf16 chunk-entry states in fragment order

def _hb_off(p, n, N):
    """the fragment-order offset of element (p, n) of a P x N state (restated
    from the library's layout description)"""
    return ((((p >> 5) * (N >> 5) + (n >> 5)) * 4 + ((n & 31) >> 3)) * 64 + (p & 31) + 32 * ((n & 7) >> 2)) * 4 + (n & 3)


@pytest.mark.parametrize("P,N", [(32, 32), (32, 64), (64, 128), (64, 256), (128, 128), (128, 256)])
def test_fragment_order_is_a_bijection_with_runs_of_four(P, N):
    p, n = np.meshgrid(np.arange(P), np.arange(N), indexing="ij")
    off = _hb_off(p, n, N)
    assert sorted(off.ravel().tolist()) == list(range(P * N))
    assert np.all(off[:, 1:][:, (n[0, 1:] % 4) != 0] == off[:, :-1][:, (n[0, 1:] % 4) != 0] + 1)


@pytest.mark.parametrize("P,N", [(32, 32), (64, 128), (64, 256), (128, 256)])
def test_fragment_order_writers_and_readers_agree(P, N):
    """the walk's stores (accumulator u of column block pj, register run jj,
    lane), the staging in chunk_scan (16-byte piece e -> rows p, p + 1 at n)
    and the per-fragment reads (two runs of four) all address hb_off."""
    # walk: lane L holds p = pj + L % 32, n = 32 nt + 8 jj + 4 (L // 32) + 0..3
    for pj in range(0, P, 32):
        for nt in range(N // 32):
            for jj in range(4):
                for lane in range(64):
                    at = (((pj // 32) * (N // 32) + nt) * 4 + jj) * 256 + lane * 4
                    assert at == _hb_off(pj + lane % 32, 32 * nt + 8 * jj + 4 * (lane // 32), N)
    # chunk_scan staging: piece e holds runs 2e, 2e + 1
    for e in range(P * N // 8):
        r = 2 * e
        q, blk = r >> 6, (r >> 6) >> 2
        p = 32 * (blk // (N // 32)) + (r & 31)
        n = 32 * (blk % (N // 32)) + 8 * (q & 3) + 4 * ((r & 63) >> 5)
        assert _hb_off(p, n, N) == 8 * e and _hb_off(p + 1, n, N) == 8 * e + 4


@pytest.mark.parametrize("P,N", [(32, 32), (64, 128), (64, 256), (128, 256)])
def test_fragment_order_operand_reads(P, N):
    """chunk_scan's H^T operand: for lane (l32, g2), column block pb and k step
    ks it reads n = 16 ks + 8 g2 .. + 7 of row 32 pb + l32 as two runs, at
    256 g2 + 4 l32 + 256 ((pb N / 32 + ks / 2) 4 + 2 (ks % 2)) and 128 after"""
    for pb in range(P // 32):
        for ks in range(N // 16):
            for lane in range(64):
                l32, g2 = lane % 32, lane // 32
                o = 256 * g2 + 4 * l32 + 256 * ((pb * (N // 32) + ks // 2) * 4 + 2 * (ks % 2))
                p, n = 32 * pb + l32, 16 * ks + 8 * g2
                assert o == _hb_off(p, n, N) and o + 128 == _hb_off(p, n + 4, N)


def test_traffic_digest_ignores_comments_only():
    """bench.py keeps a committed traffic summary while the kernel's code is
    unchanged: comments and whitespace do not enter the digest, code does"""
    import bench
    a = "int f(int x) {  // first\n  return x + 1; /* note */ }\n"
    b = "int f(int x) {\n  // reworded comment\n  return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


# ---------------------------------------------------------------- packed sequences through the walk

VARLEN_PLAN_SHAPES = [
    # T, nseq, H, P, N, G, Q: the packed 130M workload, few and many sequences, both dstates, headdim 32/128
    (16384, 13, 24, 64, 128, 1, 256), (16384, 13, 24, 64, 128, 1, 128), (16384, 13, 24, 64, 128, 1, 64),
    (1800, 3, 4, 64, 128, 1, 128), (131072, 4, 24, 64, 256, 1, 256), (5000, 40, 24, 64, 128, 1, 256),
    (4000, 9, 8, 32, 128, 2, 128), (3000, 5, 2, 128, 256, 1, 128), (700, 300, 24, 64, 128, 1, 256),
    (1, 1, 2, 64, 128, 1, 64), (375, 3, 2, 64, 256, 1, 128),
]


def _varlen_plan(T, nseq, H, P, N, G, Q, cus=256):
    import selective_state_space_46_amd as ssd
    return ssd.ssd_chunk_scan_fwd_varlen_plan(T, nseq, H, P, N, G, Q, ssd.SSD_BF16, cus)


@pytest.mark.parametrize("shape", VARLEN_PLAN_SHAPES)
def test_varlen_walk_plan(shape):
    """The packed plan: the row of ceil(T / Q) + nseq chunk slots cut into
    equal segments of at least one slot that cover it exactly, as many walks
    (segments x 64-column blocks) as fit a 256-unit device at once (two per
    unit at dstate 128 with chunk_len >= 128), no more segments than slots
    and at most 128 slots each; none for shapes the walk does not serve."""
    T, nseq, H, P, N, G, Q = shape
    nseg, L = _varlen_plan(*shape)
    cpr = H * P // _cols(N, P, Q)
    cap = (512 if N == 128 and Q >= 128 else 256)
    nslots = -(-T // Q) + nseq
    if nseg == 0:
        assert L == 0 and cpr > cap
        return
    assert L >= 1 and (nseg - 1) * L < nslots <= nseg * L
    want = min(nslots, cap // cpr)
    assert L == min(-(-nslots // want), 128)           # at most 128 slots per walk
    assert nseg * cpr <= cap or L == 128
    assert _varlen_plan(*shape, cus=0) == (0, 0)
    import selective_state_space_46_amd as ssd
    assert ssd.ssd_chunk_scan_fwd_varlen_plan(T, nseq, H, P, 64, G, Q, ssd.SSD_BF16, 256) == (0, 0)
    assert ssd.ssd_chunk_scan_fwd_varlen_plan(T, nseq, H, P, N, G, Q, ssd.SSD_F32, 256) == (0, 0)
    assert ssd.ssd_chunk_scan_fwd_varlen_plan(T, 0, H, P, N, G, Q, ssd.SSD_BF16, 256) == (0, 0)


run_xcd = [None]   # set by the varlen_tables fixture: the library's xcd_swizzle on the host


@pytest.fixture(scope="module")
def varlen_tables(tmp_path_factory):
    """builds the packed-sequence chunk table on the host with the library's
    own varlen_slot_entry, slot by slot (tests/varlen_tables_driver.hip)"""
    import subprocess
    from selective_state_space_46_amd import build
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    exe = str(tmp_path_factory.mktemp("vt") / "varlen_tables")
    r = subprocess.run([hipcc, f"--offload-arch={build.ARCH}", "-O1",
                        "-I", os.path.join(root, "selective_state_space_46_amd", "csrc"),
                        "-I", os.path.join(root, "include"), "-o", exe,
                        os.path.join(here, "varlen_tables_driver.hip")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    def xcd(n):
        out = subprocess.run([exe], input=f"xcd {n}\n", capture_output=True, text=True, check=True).stdout.split()
        return np.array(out, dtype=np.int64)
    run_xcd[0] = xcd

    def run(T, Q, cu):
        inp = f"{T} {len(cu) - 1} {Q}\n" + " ".join(str(int(v)) for v in cu) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split()
        v = np.array(out, dtype=np.int64)
        nslots = int(v[0])
        return v[1:1 + 4 * nslots].reshape(nslots, 4)
    return run


def _varlen_cases():
    rng = np.random.default_rng(7100)
    cases = []
    for Q in (64, 128, 256):
        lens = [300, 0, 17, 256, 1, 129, 64, 511, 33, 3515, 2048, 0]
        cases.append((Q, np.concatenate([[0], np.cumsum(lens)]).tolist(), int(sum(lens))))
        for _ in range(6):
            n = int(rng.integers(1, 20))
            lens = rng.integers(0, 5 * Q, size=n)
            cases.append((Q, np.concatenate([[0], np.cumsum(lens)]).tolist(), max(1, int(lens.sum()))))
        # malformed: decreasing, negative, past the end
        cases.append((Q, [0, 150, 90, 400, -5, 10**6], 200))
        cases.append((Q, [-40, 7000, 3, 3, 2999], 3000))
        for _ in range(2):
            cases.append((Q, rng.integers(-Q, 6 * Q, size=int(rng.integers(2, 16))).tolist(), 4 * Q))
    return cases


@pytest.mark.parametrize("case", _varlen_cases())
def test_varlen_tables(varlen_tables, case):
    """With well-formed offsets every sequence's chunks fill consecutive
    slots from slot floor(cu[i] / Q) + i with their rows, valid tokens,
    sequence and first / last flags, no entry is dropped by the table bound
    (the slot count holds every span) and everything else stays empty; every
    used slot's sequence begins at a slot flagged first and ends at one
    flagged last, in slot order, which is what the packed walks restart and
    finish on. With any offsets (clamped as the device clamps them) a used
    slot holds the chunk of its own sequence that belongs at that slot, so
    its rows stay inside that sequence's clamped span and the tokens."""
    Q, cu, T = case
    tab = varlen_tables(T, Q, cu)
    nseq = len(cu) - 1
    assert len(tab) == -(-T // Q) + nseq
    want = np.zeros_like(tab)
    spans = []
    for i in range(nseq):
        s0 = min(max(cu[i], 0), T)
        s1 = min(max(cu[i + 1], s0), T)
        ln = s1 - s0
        nch = -(-ln // Q)
        first = s0 // Q + i
        spans.append((s0, ln, nch, first))
        for k in range(nch):
            want[first + k] = (s0 + k * Q, min(Q, ln - k * Q), i, (k == 0) | ((k == nch - 1) << 1))
    used = tab[:, 1] > 0
    assert np.all((tab[used, 0] >= 0) & (tab[used, 0] + tab[used, 1] <= T) & (tab[used, 1] <= Q))
    for c in np.flatnonzero(used):
        r0, n, seq, flags = (int(v) for v in tab[c])
        assert 0 <= seq < nseq
        s0, ln, nch, first = spans[seq]
        k = c - first
        assert 0 <= k < nch
        assert (r0, n, flags) == (s0 + k * Q, min(Q, ln - k * Q), (k == 0) | ((k == nch - 1) << 1))
    assert np.all(tab[~used] == 0)
    well_formed = cu[0] == 0 and cu[-1] == T and all(a <= b for a, b in zip(cu, cu[1:]))
    if well_formed:
        assert np.array_equal(tab, want)
        cur = -1                               # the sequence running, slot by slot
        for r0, n, seq, flags in tab:
            if n == 0:
                assert cur == -1               # unused slots only between sequences
                continue
            assert bool(flags & 1) == (cur == -1) and (cur == -1 or seq == cur)
            cur = -1 if flags & 2 else seq
        assert cur == -1


@pytest.mark.parametrize("n", [1, 7, 8, 9, 240, 252, 255, 256, 257, 12288, 12291])
def test_xcd_swizzle_is_a_bijection_with_contiguous_ranges(varlen_tables, n):
    """the library's XCD renumbering (ssd_internal.h, run on the host): a
    bijection of [0, n) for any n, under which the work-groups the hardware
    gives XCD x (ids x, x + 8, ...) take one contiguous range of logical ids,
    in order; multiples of 8 keep the former mapping x (n / 8) + id / 8"""
    ids = run_xcd[0](n)
    assert sorted(ids.tolist()) == list(range(n))
    for x in range(min(n, 8)):
        mine = ids[x::8]
        assert np.array_equal(mine, np.arange(mine[0], mine[0] + len(mine)))
    if n % 8 == 0:
        b = np.arange(n)
        assert np.array_equal(ids, (b % 8) * (n // 8) + b // 8)
