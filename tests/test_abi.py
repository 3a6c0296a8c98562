"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/ssd_api.h declares, and rejects bad arguments with
the documented status codes before launching anything."""
import ctypes
import os
import re

import pytest

import selective_state_space_46_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a non-NULL, 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ssd.lib_path()):
        from selective_state_space_46_amd import build
        build.build()
    return ssd.lib()


def declared_symbols():
    out = []
    for h in ("ssd_api.h", "ssd_epilogue.h", "ssd_backward.h", "ssd_measure.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        out += re.findall(r"SSD_API\s+[\w\s\*]*?\b(ssd_\w+)\s*\(", text)
    return out


def test_header_declares_the_entry_points():
    assert set(declared_symbols()) == {"ssd_chunk_scan_fwd_workspace", "ssd_chunk_scan_fwd",
                                       "ssd_chunk_scan_fwd_timed", "ssd_state_update",
                                       "ssd_status_string", "ssd_gated_rmsnorm",
                                       "ssd_causal_conv1d_fwd", "ssd_causal_conv1d_update",
                                       "ssd_chunk_scan_fwd_varlen", "ssd_chunk_scan_fwd_varlen_workspace",
                                       "ssd_chunk_scan_bwd", "ssd_chunk_scan_bwd_workspace",
                                       "ssd_chunk_scan_fwd_fused_states", "ssd_chunk_scan_bwd_fused_walks",
                                       "ssd_chunk_scan_fwd_plan", "ssd_chunk_scan_fwd_noalloc",
                                       "ssd_chunk_scan_fwd_varlen_plan", "ssd_mfma_bf16_probe"}


def test_fused_states_query_rejects_what_the_forward_rejects():
    """0 for sizes the forward would reject (answered before any device query)
    and for the generic fp32 path, which never fuses."""
    q = ssd.ssd_chunk_scan_fwd_fused_states
    assert not q(8, 2048, 24, 64, 128, 1, 256, 7)            # bad dtype
    assert not q(8, 2048, 24, 64, 128, 1, 48, ssd.SSD_BF16)  # bad chunk length
    assert not q(0, 2048, 24, 64, 128, 1, 256, ssd.SSD_BF16)
    assert not q(8, 2048, 24, 64, 128, 5, 256, ssd.SSD_BF16)  # groups must divide heads
    assert not q(8, 2048, 24, 64, 128, 1, 256, ssd.SSD_F32)


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_headers_compile_as_c_and_cpp(tmp_path, lang):
    """the public headers are plain C (C11) and also valid C++17, pedantic,
    with no warning"""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip(f"no {lang} compiler")
    src = tmp_path / "h.c"
    src.write_text("".join(f'#include "{h}"\n' for h in ("ssd_api.h", "ssd_epilogue.h", "ssd_backward.h",
                                                          "ssd_measure.h")) +
                   "int main(void) { ssd_dtype d = SSD_BF16; ssd_status s = SSD_OK; return (int)d + (int)s; }\n")
    std = ["-std=c11"] if lang == "c" else ["-std=c++17", "-x", "c++"]
    r = subprocess.run([cc] + std + ["-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                                      "-c", str(src), "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(10):
        s = ssd.ssd_status_string(code)
        assert s and s != "unknown status"
    assert ssd.ssd_status_string(99) == "unknown status"


def ws(b, T, H, P, N, G, Q, dt=ssd.SSD_BF16):
    return ssd.ssd_chunk_scan_fwd_workspace(b, T, H, P, N, G, Q, dt)


def test_workspace_query():
    """Acs and dt rows (fp32), chunk states (fp32) and, on the bf16 matrix-core
    path (dstate in {32,64,128,256}, headdim in {32,64,128}, chunk >= 32), a bf16
    copy of the passed states, the bf16 C B^T tiles (2 KB per lower-triangle
    32x32 tile per chunk and group) and a bf16 copy of C (one chunk's rows per
    chunk and group, in the matrix cores' operand order); each region 256-byte
    aligned. Without a
    GPU the library cannot choose the fused walk (it needs the device's
    compute-unit count), so this is the two-launch layout."""
    def expect(b, T, H, P, N, Q, dtype):
        nc = -(-T // Q)
        up = lambda v: -(-v // 256) * 256
        row = up(b * H * nc * Q * 4)
        nst = b * nc * H * N * P
        mfma = dtype == ssd.SSD_BF16 and N in (32, 64, 128, 256) and P in (32, 64, 128) and Q >= 32
        lpc = Q // 32
        cbt = b * nc * G * (lpc * (lpc + 1) // 2) * 1024 * 2
        cf = b * nc * G * Q * N * 2               # C in the matrix cores' operand order
        return up(2 * row + up(nst * 4) + (up(nst * 2) + up(cbt) + cf if mfma else 0))
    for args in [(8, 2048, 24, 64, 128, 1, 256), (1, 131072, 24, 64, 256, 1, 256), (1, 1, 1, 1, 1, 1, 16),
                 (2, 100, 4, 3, 5, 2, 32), (2, 100, 4, 64, 128, 2, 16), (2, 100, 4, 32, 64, 2, 32)]:
        b, T, H, P, N, G, Q = args
        for dt in (ssd.SSD_F32, ssd.SSD_BF16):
            assert ws(*args, dt=dt) == expect(b, T, H, P, N, Q, dt), (args, dt)
    assert ws(1, 256, 3, 16, 16, 2, 64) == 0          # H % G != 0
    assert ws(1, 256, 2, 16, 16, 1, 48) == 0          # chunk
    assert ws(1, 0, 2, 16, 16, 1, 64) == 0            # T = 0
    assert ws(1, 256, 2, 257, 16, 1, 64) == 0         # headdim too large
    assert ws(1, 256, 2, 16, 16, 1, 64, dt=5) == 0    # dtype
    # 2^23 chunk-heads: the bf16 matrix-core chunk_state launch (512 work-items
    # per chunk-head plus 64 per C B^T tile) would reach 2^32 work-items; the
    # fp32 path's grids stay below it. 61 chunks instead of 64 fit.
    big = (1024, 16384, 128, 64, 128, 1, 256)
    assert ws(*big, dt=ssd.SSD_BF16) == 0
    assert ws(*big, dt=ssd.SSD_F32) == expect(1024, 16384, 128, 64, 128, 256, ssd.SSD_F32)
    assert ws(1024, 61 * 256, 128, 64, 128, 1, 256, dt=ssd.SSD_BF16) > 0


def fwd(L, **kw):
    a = dict(x=FAKE, dt=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000, C=FAKE + 0x400000,
             D=None, init=None, y=FAKE + 0x500000, fin=None, b=1, T=64, H=2, P=16, N=16, G=1, Q=64,
             dtype=0, ws=FAKE + 0x600000, nbytes=1 << 30, stream=None)
    a.update(kw)
    return L.ssd_chunk_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"], a["y"],
                                a["fin"], a["b"], a["T"], a["H"], a["P"], a["N"], a["G"], a["Q"],
                                a["dtype"], a["ws"], a["nbytes"], a["stream"])


def test_forward_argument_errors(L):
    assert fwd(L, dtype=2) == 3
    assert fwd(L, T=0) == 2
    assert fwd(L, b=0) == 2
    assert fwd(L, H=3, G=2) == 2
    assert fwd(L, P=300) == 2
    assert fwd(L, N=300) == 2
    assert fwd(L, Q=100) == 4
    assert fwd(L, Q=512) == 4
    assert fwd(L, T=16 * 65536, Q=16) == 2          # more chunks than the grid allows
    assert fwd(L, b=1024, T=16384, H=128, P=64, N=128, Q=256, dtype=1) == 2   # 2^32 work-items
    for k in ("x", "dt", "A", "B", "C", "y"):
        assert fwd(L, **{k: None}) == 1, k
    assert fwd(L, ws=None) == 5
    assert fwd(L, nbytes=100) == 5
    assert fwd(L, x=FAKE + 8) == 8
    assert fwd(L, init=FAKE + 0x700004) == 8
    assert fwd(L, y=FAKE) == 7                        # y over x
    assert fwd(L, y=FAKE + 0x600000) == 7             # y over the workspace
    assert fwd(L, fin=FAKE + 0x300000) == 7           # final over B
    assert fwd(L, init=FAKE + 0x700000, fin=FAKE + 0x700010) == 7   # partial overlap
    assert fwd(L, ws=FAKE + 0x100000) == 7            # workspace over dt


def upd(L, **kw):
    a = dict(state=FAKE, x=FAKE + 0x100000, dt=FAKE + 0x200000, A=FAKE + 0x300000, B=FAKE + 0x400000,
             C=FAKE + 0x500000, D=None, y=FAKE + 0x600000, b=2, H=4, P=16, N=16, G=2, dtype=1,
             stream=None)
    a.update(kw)
    return L.ssd_state_update(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["y"],
                              a["b"], a["H"], a["P"], a["N"], a["G"], a["dtype"], a["stream"])


def test_decode_argument_errors(L):
    assert upd(L, dtype=7) == 3
    assert upd(L, H=3) == 2
    assert upd(L, N=0) == 2
    for k in ("state", "x", "dt", "A", "B", "C", "y"):
        assert upd(L, **{k: None}) == 1, k
    assert upd(L, y=FAKE + 0x100000) == 7             # y over x
    assert upd(L, state=FAKE + 0x600000) == 7         # state over y
    assert upd(L, x=FAKE + 0x100002) == 8


def norm(L, **kw):
    a = dict(y=FAKE, z=FAKE + 0x100000, w=FAKE + 0x200000, out=FAKE + 0x300000, n=16, dim=64, group=64,
             eps=1e-5, dtype=1, stream=None)
    a.update(kw)
    return L.ssd_gated_rmsnorm(a["y"], a["z"], a["w"], a["out"], a["n"], a["dim"], a["group"], a["eps"],
                               a["dtype"], a["stream"])


def test_gated_rmsnorm_argument_errors(L):
    assert norm(L, dtype=4) == 3
    assert norm(L, n=0) == 2
    assert norm(L, dim=0) == 2
    assert norm(L, group=0) == 2
    assert norm(L, dim=64, group=48) == 2             # dim % group
    assert norm(L, n=1 << 27, dim=64, group=1) == 2   # more rows than the grid allows
    assert norm(L, eps=-1.0) == 9
    assert norm(L, eps=float("inf")) == 9
    assert norm(L, eps=float("nan")) == 9
    for k in ("y", "z", "w", "out"):
        assert norm(L, **{k: None}) == 1, k
    assert norm(L, z=FAKE + 0x100008) == 8
    assert norm(L, out=FAKE + 0x40) == 7              # out partly over y
    assert norm(L, out=FAKE + 0x100000) == 7          # out over z
    assert norm(L, out=FAKE + 0x200000) == 7          # out over the weight


def conv(L, **kw):
    a = dict(x=FAKE, w=FAKE + 0x100000, bias=None, init=None, out=FAKE + 0x300000, fin=None, b=2, T=64,
             C=32, K=4, act=1, dtype=1, stream=None)
    a.update(kw)
    return L.ssd_causal_conv1d_fwd(a["x"], a["w"], a["bias"], a["init"], a["out"], a["fin"], a["b"], a["T"],
                                   a["C"], a["K"], a["act"], a["dtype"], a["stream"])


def test_conv1d_argument_errors(L):
    assert conv(L, dtype=2) == 3
    assert conv(L, T=0) == 2
    assert conv(L, C=0) == 2
    assert conv(L, K=0) == 2
    assert conv(L, K=9) == 2
    assert conv(L, b=65536, T=65536 * 16, C=16) == 2  # more threads than allowed
    assert conv(L, act=2) == 9
    for k in ("x", "w", "out"):
        assert conv(L, **{k: None}) == 1, k
    assert conv(L, init=FAKE + 0x400004) == 8
    assert conv(L, out=FAKE + 0x100) == 7             # out over x
    assert conv(L, fin=FAKE + 0x10) == 7              # final state over x
    assert conv(L, init=FAKE + 0x400000, fin=FAKE + 0x400010) == 7   # partial overlap
    assert conv(L, bias=FAKE + 0x300000) == 7         # out over the bias


def upd1(L, **kw):
    a = dict(state=FAKE, x=FAKE + 0x100000, w=FAKE + 0x200000, bias=None, out=FAKE + 0x300000, b=2, C=32,
             K=4, act=1, dtype=1, stream=None)
    a.update(kw)
    return L.ssd_causal_conv1d_update(a["state"], a["x"], a["w"], a["bias"], a["out"], a["b"], a["C"],
                                      a["K"], a["act"], a["dtype"], a["stream"])


def test_conv1d_update_argument_errors(L):
    assert upd1(L, dtype=5) == 3
    assert upd1(L, C=0) == 2
    assert upd1(L, K=9) == 2
    assert upd1(L, act=-1) == 9
    for k in ("state", "x", "w", "out"):
        assert upd1(L, **{k: None}) == 1, k
    assert upd1(L, out=FAKE + 0x100000) == 7          # out over x
    assert upd1(L, state=FAKE + 0x300000) == 7        # state over out
    assert upd1(L, x=FAKE + 0x100002) == 8


def vl(L, **kw):
    a = dict(x=FAKE, dt=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000, C=FAKE + 0x400000, D=None,
             cu=FAKE + 0x500000, init=None, y=FAKE + 0x600000, fin=None, T=300, nseq=3, H=2, P=64, N=128,
             G=1, Q=64, dtype=1, ws=FAKE + 0x800000, nbytes=1 << 30, stream=None)
    a.update(kw)
    return L.ssd_chunk_scan_fwd_varlen(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["cu"], a["init"],
                                       a["y"], a["fin"], a["T"], a["nseq"], a["H"], a["P"], a["N"], a["G"],
                                       a["Q"], a["dtype"], a["ws"], a["nbytes"], a["stream"])


def test_varlen_workspace_and_errors(L):
    wsq = ssd.ssd_chunk_scan_fwd_varlen_workspace
    assert wsq(300, 3, 2, 64, 128, 1, 64, ssd.SSD_BF16) > 0
    assert wsq(300, 3, 2, 64, 128, 1, 64, ssd.SSD_F32) == 0      # matrix-core configuration only
    assert wsq(300, 3, 2, 16, 16, 1, 64, ssd.SSD_BF16) == 0      # headdim 16: no matrix-core path
    assert wsq(300, 0, 2, 64, 128, 1, 64, ssd.SSD_BF16) == 0
    assert wsq(300, 70000, 2, 64, 128, 1, 64, ssd.SSD_BF16) == 0
    # more sequences need more chunk slots (one partial chunk each at most)
    assert wsq(300, 9, 2, 64, 128, 1, 64, ssd.SSD_BF16) > wsq(300, 3, 2, 64, 128, 1, 64, ssd.SSD_BF16)
    assert vl(L, dtype=3) == 3
    assert vl(L, dtype=0) == 2          # fp32: not the matrix-core configuration
    assert vl(L, nseq=0) == 2
    assert vl(L, T=0) == 2
    assert vl(L, Q=48) == 4
    for k in ("x", "dt", "A", "B", "C", "y", "cu"):
        assert vl(L, **{k: None}) == 1, k
    assert vl(L, ws=None) == 5
    assert vl(L, nbytes=1000) == 5
    assert vl(L, cu=FAKE + 0x500002) == 8
    assert vl(L, x=FAKE + 0x8) == 8
    assert vl(L, y=FAKE) == 7                                    # y over x
    assert vl(L, fin=FAKE + 0x500000) == 7                       # final states over cu_seqlens
    assert vl(L, ws=FAKE + 0x300000) == 7                        # workspace over B


def bw(L, **kw):
    a = dict(x=FAKE, dt=FAKE + 0x100000, A=FAKE + 0x200000, B=FAKE + 0x300000, C=FAKE + 0x400000, D=None,
             init=None, dy=FAKE + 0x500000, dfinal=None, dx=FAKE + 0x600000, ddt=FAKE + 0x700000,
             dA=FAKE + 0x800000, dB=FAKE + 0x900000, dC=FAKE + 0xa00000, dD=None, dinit=None, b=1, T=300, H=2,
             P=64, N=128, G=1, dtype=1, ws=FAKE + 0x1000000, nbytes=1 << 30, stream=None)
    a.update(kw)
    return L.ssd_chunk_scan_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"], a["dy"], a["dfinal"],
                                a["dx"], a["ddt"], a["dA"], a["dB"], a["dC"], a["dD"], a["dinit"], a["b"], a["T"],
                                a["H"], a["P"], a["N"], a["G"], a["dtype"], a["ws"], a["nbytes"], a["stream"])


def test_bwd_workspace_and_errors(L):
    wsq = ssd.ssd_chunk_scan_bwd_workspace
    assert wsq(1, 300, 2, 64, 128, 1, ssd.SSD_BF16) > 0
    assert wsq(1, 300, 2, 64, 128, 1, ssd.SSD_F32) == 0       # bf16 matrix-core configuration only
    assert wsq(1, 300, 2, 128, 256, 1, ssd.SSD_BF16) == 0     # tiles too large for one CU's LDS
    assert wsq(1, 300, 2, 16, 16, 1, ssd.SSD_BF16) == 0
    assert wsq(1, 300, 3, 64, 128, 2, ssd.SSD_BF16) == 0      # H % G
    # per-head dB / dC partials grow with the heads
    assert wsq(1, 300, 8, 64, 128, 1, ssd.SSD_BF16) > wsq(1, 300, 2, 64, 128, 1, ssd.SSD_BF16)
    walks = ssd.ssd_chunk_scan_bwd_fused_walks
    assert walks(1, 300, 2, 64, 128, 1, ssd.SSD_F32) == 0
    assert walks(1, 300, 3, 64, 128, 2, ssd.SSD_BF16) == 0
    assert walks(1, 300, 2, 128, 256, 1, ssd.SSD_BF16) == 0
    assert bw(L, dtype=3) == 3
    assert bw(L, dtype=0) == 2
    assert bw(L, P=128, N=256) == 2
    assert bw(L, T=0) == 2
    for k in ("x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC"):
        assert bw(L, **{k: None}) == 1, k
    assert bw(L, ws=None) == 5
    assert bw(L, nbytes=1000) == 5
    assert bw(L, dy=FAKE + 0x500008) == 8
    assert bw(L, dx=FAKE) == 7                                    # dx over x
    assert bw(L, dB=FAKE + 0x600000) == 7                         # dB over dx
    assert bw(L, dD=FAKE + 0x200000) == 7                         # dD over A
    assert bw(L, dinit=FAKE + 0x1000000) == 7                     # dinit over the workspace
    assert bw(L, ws=FAKE + 0x500000) == 7                         # workspace over dy

