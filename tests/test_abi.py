"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tw.h")


@pytest.fixture(scope="module")
def tw():
    from activation_sparse_feed_gate_amd import build as b

    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES] + [HEADER]
    lib = b.LIBRARY
    if not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib) for s in srcs):
        b.build()
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tw_[a-z_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared()
    for n in ("tw_pack_gate", "tw_sparse_ffn_fwd", "tw_ffn_fwd", "tw_workspace_bytes"):
        assert n in names


def test_exports_every_declared_symbol(tw):
    out = subprocess.run(["nm", "-D", "--defined-only", tw.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared():
        assert n in exported, n
        assert hasattr(tw._lib, n)


def test_status_strings(tw):
    assert tw._lib.tw_status_str(0) == b"TW_OK"
    assert tw._lib.tw_status_str(1) == b"TW_EINVAL"
    assert tw._lib.tw_status_str(2) == b"TW_EUNSUPPORTED"
    assert tw._lib.tw_status_str(3) == b"TW_EHIP"


def test_workspace_bytes(tw):
    assert tw.tw_workspace_bytes(4096, 1024, 4096, 128, 8, 512) > 512 * 4096 * 2
    assert tw.tw_workspace_bytes(4096, 1024, 4096, 64, 8, 512) == 0
    assert tw.tw_workspace_bytes(4096, 1000, 4096, 128, 8, 512) == 0
    assert tw.tw_workspace_bytes(4096, 1024, 4096, 128, 0, 512) == 0
    assert tw.tw_workspace_bytes(4096, 1024, 4096, 128, 8, 5000) == 0
    assert tw.tw_ffn_workspace_bytes(64, 256, 1024) >= 64 * 1024 * 2


def test_workspace_covers_small_batch_buffers(tw):
    """The workspace also holds the small-batch gate's partial gates (a few
    rows: 8 K-slices of M x N fp32), the sparse kernel's partial rows (32 to
    128 rows: 256 / M per row, M x K fp32 each) and the backup's split
    partial tiles (16 MB)."""
    # 16 rows of the 2B block: the gate's reduction in 8 slices
    assert tw.tw_workspace_bytes(16, 2048, 8192, 256, 16, 2) >= 8 * 16 * 8192 * 4
    # 64 rows of the 0.5B block: 4 partial rows per row, after the backup's
    # h rows and split partials
    need = 8 * 4096 * 2 + (16 << 20) + 4 * 64 * 1024 * 4
    assert tw.tw_workspace_bytes(64, 1024, 4096, 128, 8, 8) >= need
    # no backup room: the partial rows alone still fit
    assert tw.tw_workspace_bytes(64, 1024, 4096, 128, 8, 0) >= 4 * 64 * 1024 * 4


# Fake, 16-byte-aligned device addresses: every case below must be rejected
# on the host before any of them is dereferenced or any HIP call is made.
P = 0x100000


def _pack(tw, M=64, K=256, N=1024, T=128, C=16, R=64, ws=1 << 20, **ptrs):
    a = dict(x=P, wg=P, val=P, idx=P, cnt=P, ovf=P, n=P, z=None, w=P)
    a.update(ptrs)
    return tw._lib.tw_pack_gate(a["x"], a["wg"], M, K, N, T, C, a["val"], a["idx"], a["cnt"],
                                a["ovf"], a["n"], R, a["z"], a["w"], ws, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=64), 2), (dict(T=512, N=1024), 2), (dict(N=1000), 1), (dict(C=0), 1),
    (dict(C=129), 1), (dict(K=192), 2), (dict(K=8192), 2), (dict(R=65), 1), (dict(R=-1), 1),
    (dict(M=-1), 1), (dict(K=0), 1), (dict(x=None), 1), (dict(wg=None), 1), (dict(val=None), 1),
    (dict(n=None), 1), (dict(w=None), 1), (dict(x=P + 8), 1), (dict(z=P + 4), 1), (dict(ws=16), 1),
    (dict(N=128 * 300), 2), (dict(M=1 << 20, K=4096, R=0), 2), (dict(M=1 << 19, K=4096, R=0), 2),
    # the overflow list: both pointers or neither, and with neither the other
    # checks still apply
    (dict(ovf=None), 1), (dict(ovf=P + 4), 1), (dict(ovf=None, n=None, C=0), 1),
    (dict(ovf=None, n=None, x=None), 1),
])
def test_pack_rejects(tw, kw, code):
    assert _pack(tw, **kw) == code
    assert tw._lib.tw_last_error()


def test_sparse_and_dense_reject(tw):
    L = tw._lib
    assert L.tw_sparse_ffn_fwd(P, P, P, P, 64, 256, 1024, 128, 16, P, P, P, P, P, 64, None, P,
                               1 << 20, None, None) == 1
    assert L.tw_sparse_ffn_fwd(P, P, P, P, 64, 256, 1024, 100, 16, P, P, P, P, P, 64, P, P,
                               1 << 20, None, None) == 2
    assert L.tw_sparse_ffn_fwd(P, P, P, P, 64, 256, 1024, 128, 16, P, P, P, P, P, 64, P, P,
                               8, None, None) == 1
    assert L.tw_ffn_fwd(P, P, P, P, 64, 256, 1000, P, P, 1 << 24, None, None) == 2
    assert L.tw_ffn_fwd(P, P, P, None, 64, 256, 1024, P, P, 1 << 24, None, None) == 1
    assert L.tw_ffn_fwd(P, P, P, P, 64, 256, 1024, P, P, 16, None, None) == 1
    # weights of 4 GiB or more are outside the 32-bit buffer offsets
    assert L.tw_ffn_fwd(P, P, P, P, 64, 4096, 1 << 19, P, P, 1 << 40, None, None) == 2


def test_unfused_entry_points_reject(tw):
    L = tw._lib
    assert L.tw_gate_dense(P, P, 64, 100, 1024, P, None, None) == 2   # K not a multiple of 128
    assert L.tw_gate_dense(P, P, 64, 256, 1000, P, None, None) == 2   # N not a multiple of 128
    assert L.tw_gate_dense(None, P, 64, 256, 1024, P, None, None) == 1
    assert L.tw_gate_dense(P, P, 64, 256, 1024, P + 4, None, None) == 1
    assert L.tw_gate_dense(P, P, 64, 8192, 1024, P, None, None) == 2      # K above 4096
    assert L.tw_gate_dense(P, P, 1 << 20, 4096, 1024, P, None, None) == 2  # x of 4 GiB or more
    assert L.tw_pack_dense_workspace_bytes(64, 1024) >= 4 * 4
    ws = L.tw_pack_dense_workspace_bytes(64, 1024)
    # z, M, N, T, C, val, idx, cnt, ovf_rows, ovf_count, R_max, ws, ws_bytes, stream, events
    assert L.tw_pack_dense(P, 64, 1024, 64, 8, P, P, P, P, P, 64, P, ws, None, None) == 2
    assert L.tw_pack_dense(P, 64, 1024, 128, 0, P, P, P, P, P, 64, P, ws, None, None) == 1
    assert L.tw_pack_dense(P, 64, 1000, 128, 8, P, P, P, P, P, 64, P, ws, None, None) == 1
    assert L.tw_pack_dense(P, 64, 1024, 128, 8, P, P, P, P, P, 65, P, ws, None, None) == 1
    assert L.tw_pack_dense(P, 64, 1024, 128, 8, P, P, P, P, P, 64, P, 8, None, None) == 1
    assert L.tw_pack_dense(None, 64, 1024, 128, 8, P, P, P, P, P, 64, P, ws, None, None) == 1
    assert tw._lib.tw_last_error()


def test_hybrid_entry_points_reject(tw):
    L = tw._lib
    def H(M=64, N=1024, T=128, C=16, cap=128, R=8, route=P, bk=P, hv=P):
        return L.tw_hybrid_pack(M, N, T, C, P, P, P, cap, hv, P, P, route, bk, P, R, None, None)
    assert H(cap=0) == 1 and H(cap=1025) == 1      # sparse capacity outside [1, N]
    assert H(T=64) == 2 and H(C=0) == 1 and H(N=1000) == 1
    assert H(R=65) == 1 and H(R=-1) == 1
    assert H(route=None) == 1 and H(route=P + 1) == 1 and H(bk=None) == 1 and H(hv=None) == 1
    # backup rows of 4 GiB or more are outside the 32-bit buffer offsets
    assert H(M=1 << 17, N=1 << 15, R=1 << 17) == 2
    # more stored slots than the kernels' 32-bit slot ids m * P + s can name
    assert H(M=1 << 20, N=4096, cap=4096, R=0) == 2

    def U(K=256, cap=128, R=8, hy_h=P, bk_h=P, hy_u=None):
        return L.tw_hybrid_up(P, P, P, 64, K, 1024, cap, P, P, P, P, P, P, R, hy_u, hy_h, None,
                              None, bk_h, None, None)
    assert U(K=100) == 2 and U(cap=0) == 1 and U(hy_h=None) == 1
    assert L.tw_hybrid_up(P, P, P, 1 << 20, 256, 4096, 4096, P, P, P, P, P, P, 0, None, P, None,
                          None, P, None, None) == 2  # M * P >= 2^31 slot ids
    assert U(bk_h=None) == 1 and U(hy_u=P + 4) == 1

    nws = L.tw_hybrid_down_workspace_bytes(8)
    assert nws > 0 and L.tw_hybrid_down_workspace_bytes(0) == 0

    def D(y=P, ws=P, nb=nws, R=8, cap=128):
        return L.tw_hybrid_down(P, 64, 256, 1024, cap, P, P, P, P, P, P, R, P, y, ws, nb, None,
                                None)
    assert D(y=None) == 1 and D(nb=nws - 1) == 1 and D(ws=None) == 1 and D(cap=2048) == 1
    assert tw._lib.tw_last_error()


def test_hybrid_backward_entry_points_reject(tw):
    L = tw._lib

    def DH(K=256, cap=128, R=8, bk_g=P, du=P):
        return L.tw_hybrid_bwd_dh(P, P, 64, K, 1024, cap, 0.01, P, P, P, P, P, P, P, R, bk_g, P,
                                  du, P, P, P, None, None)
    assert DH(K=100) == 2 and DH(cap=0) == 1 and DH(R=65) == 1
    assert DH(bk_g=None) == 1 and DH(du=None) == 1 and DH(du=P + 4) == 1

    nx = L.tw_hybrid_bwd_dx_workspace_bytes(8)
    assert nx > 0 and L.tw_hybrid_bwd_dx_workspace_bytes(0) == 0

    def DX(dx=P, nb=nx, ws=P, bk=P):
        return L.tw_hybrid_bwd_dx(P, P, 64, 256, 1024, 128, P, P, P, P, P, P, P, 8, bk, P, dx, ws,
                                  nb, None, None)
    assert DX(dx=None) == 1 and DX(nb=nx - 1) == 1 and DX(ws=None) == 1 and DX(bk=None) == 1

    nw = L.tw_hybrid_bwd_dw_workspace_bytes(64, 256, 1024, 128, 8)
    assert nw >= 16 * 64 * 128 + 4 * 32 * 256

    def DW(M=64, N=1024, cap=128, R=8, nb=nw, dwd=P):
        return L.tw_hybrid_bwd_dw(P, P, M, 256, N, cap, P, P, P, P, P, P, P, P, R, P, P, P, P, P,
                                  dwd, P, nb, None, None)
    assert DW(nb=nw - 1) == 1 and DW(dwd=None) == 1 and DW(cap=2048) == 1
    # more stored entries than 32-bit entry ids can name
    assert DW(M=1 << 20, N=1 << 15, cap=1 << 12, R=0, nb=1 << 62) == 2
    assert tw._lib.tw_last_error()


def test_pack_gate_noalloc_rejects(tw):
    """The entry point without a workspace: the shape checks of tw_pack_gate,
    and shapes whose workspace would not fit its 16 MiB static scratch
    (here 32 MiB of row-overflow bits) rejected before anything runs."""
    L = tw._lib

    def NA(M=64, K=256, N=1024, T=128, C=16, R=64, x=P):
        return L.tw_pack_gate_noalloc(x, P, M, K, N, T, C, P, P, P, P, P, R, None, None, None)
    assert NA(T=64) == 2 and NA(C=0) == 1 and NA(R=65) == 1 and NA(x=None) == 1
    assert NA(x=P + 8) == 1 and NA(K=192) == 2
    assert NA(M=524287, K=4096, N=65536, T=256, R=0) == 2
    assert b"static scratch" in L.tw_last_error()


def test_binding_fails_loudly_without_the_library():
    """With libtw.so absent the binding raises ImportError naming the build
    step: there is no fallback path (checked in a child process that hides
    the built library from the loader's existence check)."""
    code = ("import os, sys\n"
            "real = os.path.exists\n"
            "os.path.exists = lambda p: False if str(p).endswith('libtw.so') else real(p)\n"
            "try:\n"
            "    import activation_sparse_feed_gate_amd.tw\n"
            "except ImportError as e:\n"
            "    print('IMPORT-ERROR', e)\n"
            "    sys.exit(0)\n"
            "sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "IMPORT-ERROR" in r.stdout and "libtw.so is missing" in r.stdout
