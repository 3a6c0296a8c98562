"""The allocation-free forward (ssd_chunk_scan_fwd_noalloc), through the C ABI,
against the forward that takes a caller-owned workspace (ssd_chunk_scan_fwd):
two calls in a row -- the 130M-shaped layer at full size, then a smaller
input on the same scratch array -- must each give bit-for-bit the same y and
final state (so also within the bf16 bar of relative L2 <= 1e-2), and a size
whose workspace exceeds the scratch array is refused before any launch."""
import numpy as np
import pytest

import workloads
from ssd_testlib import dev, rel_l2

pytestmark = pytest.mark.gpu


def _inputs(w):
    inp = workloads.make_fwd_inputs(w)
    t = {k: dev(inp[k], w.dtype) for k in ("x", "dt", "B", "C")}
    t.update(A=dev(inp["A"]), D=dev(inp["D"]), init=dev(inp["init"]) if inp["init"] is not None else None)
    return t


def _both(w):
    import torch
    import selective_state_space_46_amd as ssd
    t = _inputs(w)
    y_ref, f_ref = ssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["init"], w.chunk_len)
    y = torch.full_like(t["x"], 3.0)
    fin = torch.full((w.batch, w.nheads, w.dstate, w.headdim), 3.0, dtype=torch.float32, device="cuda")
    ssd.ssd_chunk_scan_fwd_noalloc(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["init"], w.chunk_len,
                                   y=y, final_state=fin)
    torch.cuda.synchronize()
    ey = rel_l2(y.double().cpu().numpy(), y_ref.double().cpu().numpy())
    ef = rel_l2(fin.double().cpu().numpy(), f_ref.double().cpu().numpy())
    print(f"[noalloc {w.name} b={w.batch} T={w.seqlen}] rel_l2 vs workspace entry y={ey:.1e} final={ef:.1e}",
          flush=True)
    assert ey <= 1e-2 and ef <= 1e-2
    assert torch.equal(y, y_ref) and torch.equal(fin, f_ref)


def test_noalloc_two_calls_equal_workspace_entry_point():
    import selective_state_space_46_amd as ssd
    w = workloads.MAMBA2_130M
    need = ssd.ssd_chunk_scan_fwd_workspace(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                            w.chunk_len, ssd.SSD_BF16)
    assert 0 < need <= ssd.SSD_NOALLOC_SCRATCH_BYTES
    _both(w)                                                   # full size first
    _both(workloads.with_shape(w, batch=2, seqlen=700, init="normal0.1", seed=4700))   # then smaller, with init


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import torch
    import selective_state_space_46_amd as ssd
    w = workloads.with_shape(workloads.MAMBA2_130M, batch=32)  # about 4x the 130M layer's workspace
    need = ssd.ssd_chunk_scan_fwd_workspace(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                            w.chunk_len, ssd.SSD_BF16)
    assert need > ssd.SSD_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((w.batch, w.seqlen, w.nheads, w.headdim), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((w.batch, w.seqlen, w.nheads), dtype=torch.bfloat16, device="cuda")
    Bm = torch.zeros((w.batch, w.seqlen, w.ngroups, w.dstate), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(w.nheads, device="cuda")
    y = torch.full_like(x, 5.0)
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_chunk_scan_fwd_noalloc(x, dt, A, Bm, Bm, None, None, w.chunk_len, y=y)
    assert e.value.code == 5                                   # SSD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)                                 # nothing launched, nothing written
