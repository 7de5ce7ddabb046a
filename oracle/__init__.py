"""CPU oracle of the ReLU-gated sparse FFN forward (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: this package may be imported only by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.
The product path (the HIP library and its binding) never imports, links or
runs it, and it imports nothing from the product path.

The arithmetic lives in ``tw_oracle.c`` (plain sequential double loops, each
function citing the passage of "Sparser, Faster, Lighter Transformer Language
Models Review" it follows).  This wrapper only widens bfloat16 bit patterns
to double (exact) and marshals numpy arrays.

Pinned by the ``-m "not gpu"`` tests: a hand-worked example
(``tests/golden/handworked_4x4x8.txt``), exact brute force with Python
integers on small integer matrices, one-hot token rows, the row-wide ELL and
lossless special cases, exact density 0 and 1, the invariants (each active
entry appears exactly once, counts sum to the number of non-zeros, the
sparse evaluation equals the dense one bit for bit), and planted mistakes
that each of these must catch.  The hybrid storage of the training forward
(``hybrid_pack``, ``hybrid_up``, ``hybrid_down``) is pinned the same way: a
hand-worked fixture (``tests/golden/handworked_hybrid_4x4x8.txt``), integer
brute force, scipy's CSR rows and numpy products in the lossless case,
density 0 and 1, and the composed hybrid forward equalling the dense block
output bit for bit.  The backward over hybrid storage (``hybrid_bwd``) is
pinned to torch autograd in float64 on the CPU: exactly on small integer
problems (including rows past the backup room), within rounding on generator
inputs, for the input and weight gradients and the gradients of u and z at
the stored entries.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tw_oracle.c")
LIBRARY = os.path.join(_HERE, "libtw_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc (no HIP involved)."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype == np.float64:
        return np.ascontiguousarray(b)
    if b.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bits or float64, got {b.dtype}")
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(f32, dtype=np.float64)


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_int = ctypes.c_int


def _p(a, t):
    return a.ctypes.data_as(t)


class Oracle:
    """Handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and not os.path.exists(path):
            build()
        self.path = path
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.tw_oracle_threads.restype = _int
        L.tw_oracle_gate.argtypes = [_D, _D, _int, _int, _int, _D]
        L.tw_oracle_pack.argtypes = [_D, _int, _int, _int, _int, _int, _I, _I, _D, _U8, _I, _I]
        L.tw_oracle_dense_ffn.argtypes = [_D, _D, _D, _D, _int, _int, _int, _D]
        L.tw_oracle_sparse_ffn.argtypes = [_D, _D, _D, _D, _int, _int, _int, _int, _int,
                                           _I, _I, _D, _D]
        L.tw_oracle_hybrid_pack.argtypes = [_int, _int, _int, _I, _I, _D, _int, _int,
                                            _I, _I, _D, _U8, _I, _I]
        L.tw_oracle_hybrid_up.argtypes = [_D, _D, _D, _int, _int, _int, _int, _I, _I, _D,
                                          _U8, _I, _int, _D, _D, _D, _D, _D]
        L.tw_oracle_hybrid_down.argtypes = [_D, _int, _int, _int, _int, _I, _I, _D, _U8, _I,
                                            _int, _D, _D]
        L.tw_oracle_hybrid_bwd.argtypes = [_D, _D, _D, _D, _D, _int, _int, _int, _int,
                                           ctypes.c_double, _I, _I, _D, _D, _D, _U8, _I, _int,
                                           _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D]
        for f in ("tw_oracle_gate", "tw_oracle_pack", "tw_oracle_dense_ffn",
                  "tw_oracle_sparse_ffn", "tw_oracle_hybrid_pack", "tw_oracle_hybrid_up",
                  "tw_oracle_hybrid_down", "tw_oracle_hybrid_bwd"):
            getattr(L, f).restype = None

    def threads(self) -> int:
        return int(self.lib.tw_oracle_threads())

    def gate(self, x, wg_t) -> np.ndarray:
        """z = x W_g as float64 [M, N]."""
        x, wg = widen_bf16(x), widen_bf16(wg_t)
        M, K = x.shape
        N = wg.shape[0]
        assert wg.shape == (N, K)
        z = np.empty((M, N), dtype=np.float64)
        self.lib.tw_oracle_gate(_p(x, _D), _p(wg, _D), M, K, N, _p(z, _D))
        return z

    def pack(self, z, T: int, C: int, R_max: int) -> dict:
        """TwELL packing + overflow routing of any gate matrix z [M, N].

        ``z`` may be the oracle's own float64 gate or a float32 gate produced
        elsewhere; float32 is widened exactly, so packed values keep its bits.
        """
        z = np.ascontiguousarray(np.asarray(z), dtype=np.float64)
        M, N = z.shape
        if T <= 0 or N % T or not (1 <= C <= T) or R_max < 0:
            raise ValueError("bad T / C / R_max")
        NT = N // T
        cnt = np.empty((M, NT), dtype=np.int32)
        idx = np.empty((M, NT, C), dtype=np.int32)
        val = np.empty((M, NT, C), dtype=np.float64)
        flag = np.empty(M, dtype=np.uint8)
        ovf = np.full(max(R_max, 1), -1, dtype=np.int32)
        count = np.zeros(1, dtype=np.int32)
        self.lib.tw_oracle_pack(_p(z, _D), M, N, T, C, R_max, _p(cnt, _I), _p(idx, _I),
                                _p(val, _D), _p(flag, _U8), _p(ovf, _I), _p(count, _I))
        c = int(count[0])
        return {"cnt": cnt, "idx": idx, "val": val, "flag": flag,
                "ovf_rows": ovf[: min(c, R_max)].copy(), "ovf_count": c}

    def dense_ffn(self, x, wg_t, wu_t, wd) -> np.ndarray:
        """y = (ReLU(x W_g) * (x W_u)) W_d as float64 [M, K]."""
        x, wg, wu, w_d = (widen_bf16(a) for a in (x, wg_t, wu_t, wd))
        M, K = x.shape
        N = wg.shape[0]
        assert wg.shape == wu.shape == w_d.shape == (N, K)
        y = np.empty((M, K), dtype=np.float64)
        self.lib.tw_oracle_dense_ffn(_p(x, _D), _p(wg, _D), _p(wu, _D), _p(w_d, _D),
                                     M, K, N, _p(y, _D))
        return y

    def sparse_ffn(self, x, wg_t, wu_t, wd, T: int, C: int, packed: dict) -> np.ndarray:
        """y from a TwELL packing (dense recompute for overflow rows)."""
        x, wg, wu, w_d = (widen_bf16(a) for a in (x, wg_t, wu_t, wd))
        M, K = x.shape
        N = wg.shape[0]
        cnt = np.ascontiguousarray(packed["cnt"], dtype=np.int32)
        idx = np.ascontiguousarray(packed["idx"], dtype=np.int32)
        val = np.ascontiguousarray(packed["val"], dtype=np.float64)
        assert cnt.shape == (M, N // T) and idx.shape == val.shape == (M, N // T, C)
        y = np.empty((M, K), dtype=np.float64)
        self.lib.tw_oracle_sparse_ffn(_p(x, _D), _p(wg, _D), _p(wu, _D), _p(w_d, _D),
                                      M, K, N, T, C, _p(cnt, _I), _p(idx, _I), _p(val, _D),
                                      _p(y, _D))
        return y

    # ---------------- hybrid storage of the training forward ----------------
    def hybrid_pack(self, packed: dict, C: int, P: int, R_max: int) -> dict:
        """Hybrid storage (sparse rows of capacity P, dense backup) from a
        TwELL packing ``packed`` (``pack``'s output, or the GPU's arrays with
        ``cnt``, ``idx`` and ``val``) of capacity C."""
        cnt = np.ascontiguousarray(packed["cnt"], dtype=np.int32)
        M, NT = cnt.shape
        idx = np.ascontiguousarray(packed["idx"], dtype=np.int32)
        val = np.ascontiguousarray(packed["val"], dtype=np.float64)
        assert idx.shape == val.shape == (M, NT, C)
        if P < 1 or R_max < 0:
            raise ValueError("bad P / R_max")
        hy_cnt = np.empty(M, dtype=np.int32)
        hy_idx = np.empty((M, P), dtype=np.int32)
        hy_val = np.empty((M, P), dtype=np.float64)
        route = np.empty(M, dtype=np.uint8)
        bk = np.full(max(R_max, 1), -1, dtype=np.int32)
        count = np.zeros(1, dtype=np.int32)
        self.lib.tw_oracle_hybrid_pack(M, NT, C, _p(cnt, _I), _p(idx, _I), _p(val, _D), P, R_max,
                                       _p(hy_cnt, _I), _p(hy_idx, _I), _p(hy_val, _D),
                                       _p(route, _U8), _p(bk, _I), _p(count, _I))
        c = int(count[0])
        return {"hy_cnt": hy_cnt, "hy_idx": hy_idx, "hy_val": hy_val, "route": route,
                "bk_rows": bk[: min(c, R_max)].copy(), "bk_count": c, "P": P}

    @staticmethod
    def _hy_arrays(hy: dict):
        hy_cnt = np.ascontiguousarray(hy["hy_cnt"], dtype=np.int32)
        hy_idx = np.ascontiguousarray(hy["hy_idx"], dtype=np.int32)
        route = np.ascontiguousarray(hy["route"], dtype=np.uint8)
        bk = np.ascontiguousarray(hy["bk_rows"], dtype=np.int32)
        if bk.size == 0:
            bk = np.zeros(1, dtype=np.int32)
        nbk = min(int(hy["bk_count"]), len(hy["bk_rows"]))
        return hy_cnt, hy_idx, route, bk, nbk

    def hybrid_up(self, x, wg_t, wu_t, hy: dict) -> dict:
        """Up projection at the hybrid pattern and the product with the gate:
        hy_u, hy_h [M][P] for sparse rows (NaN elsewhere); bk_g, bk_u, bk_h
        [nbk][N] for the backup rows."""
        x, wg, wu = (widen_bf16(a) for a in (x, wg_t, wu_t))
        M, K = x.shape
        N = wg.shape[0]
        P = hy["hy_idx"].shape[1]
        hy_cnt, hy_idx, route, bk, nbk = self._hy_arrays(hy)
        hy_g = np.ascontiguousarray(hy["hy_val"], dtype=np.float64)
        hy_u = np.full((M, P), np.nan)
        hy_h = np.full((M, P), np.nan)
        shp = (max(nbk, 1), N)
        bk_g, bk_u, bk_h = (np.full(shp, np.nan) for _ in range(3))
        self.lib.tw_oracle_hybrid_up(_p(x, _D), _p(wg, _D), _p(wu, _D), M, K, N, P,
                                     _p(hy_cnt, _I), _p(hy_idx, _I), _p(hy_g, _D), _p(route, _U8),
                                     _p(bk, _I), nbk, _p(hy_u, _D), _p(hy_h, _D), _p(bk_g, _D),
                                     _p(bk_u, _D), _p(bk_h, _D))
        return {"hy_u": hy_u, "hy_h": hy_h, "bk_g": bk_g[:nbk], "bk_u": bk_u[:nbk],
                "bk_h": bk_h[:nbk]}

    def hybrid_down(self, wd, hy: dict, hy_h, bk_h) -> np.ndarray:
        """y = h W_d from hybrid h: stored entries ``hy_h`` [M][P] of sparse
        rows, dense rows ``bk_h`` [nbk][N] of the backup.  Rows that are
        routed to the backup but not on its list stay NaN."""
        w_d = widen_bf16(wd)
        N, K = w_d.shape
        hy_cnt, hy_idx, route, bk, nbk = self._hy_arrays(hy)
        M, P = hy_idx.shape
        h = np.ascontiguousarray(hy_h, dtype=np.float64)
        b = np.ascontiguousarray(bk_h, dtype=np.float64).reshape(-1, N)
        assert h.shape == (M, P) and b.shape[0] >= nbk
        if b.shape[0] == 0:
            b = np.zeros((1, N))
        y = np.full((M, K), np.nan)
        self.lib.tw_oracle_hybrid_down(_p(w_d, _D), M, K, N, P, _p(hy_cnt, _I), _p(hy_idx, _I),
                                       _p(h, _D), _p(route, _U8), _p(bk, _I), nbk, _p(b, _D),
                                       _p(y, _D))
        return y

    def hybrid_bwd(self, x, wg_t, wu_t, wd, dy, hy: dict, acts: dict, l1: float) -> dict:
        """Backward over hybrid storage: ``hy`` the storage (``hybrid_pack``'s
        output, or the GPU's arrays), ``acts`` its stored activations (hy_g in
        ``hy['hy_val']``; ``acts`` holds hy_u, hy_h [M][P] and bk_g, bk_u,
        bk_h [nbk][N]), ``dy`` [M][K] (bf16 bits or float64), ``l1`` the L1
        penalty's gradient on a positive gate activation.  Returns hy_du,
        hy_dz, bk_du, bk_dz, dx (NaN on rows with no stored activation),
        dwg_t, dwu_t, dwd."""
        x, wg, wu, w_d, g_y = (widen_bf16(a) for a in (x, wg_t, wu_t, wd, dy))
        M, K = x.shape
        N = wg.shape[0]
        hy_cnt, hy_idx, route, bk, nbk = self._hy_arrays(hy)
        P = hy_idx.shape[1]
        f = lambda a, shp: np.ascontiguousarray(np.asarray(a, dtype=np.float64).reshape(shp))
        hy_g = f(hy["hy_val"], (M, P))
        hy_u, hy_h = f(acts["hy_u"], (M, P)), f(acts["hy_h"], (M, P))
        nb1 = max(nbk, 1)
        pad = lambda a: np.concatenate([f(a, (-1, N))[:nbk], np.zeros((nb1 - nbk, N))])
        bk_g, bk_u, bk_h = pad(acts["bk_g"]), pad(acts["bk_u"]), pad(acts["bk_h"])
        hy_du, hy_dz = np.full((M, P), np.nan), np.full((M, P), np.nan)
        bk_du, bk_dz = np.full((nb1, N), np.nan), np.full((nb1, N), np.nan)
        dx = np.full((M, K), np.nan)
        dwg, dwu, dwd = (np.empty((N, K)) for _ in range(3))
        self.lib.tw_oracle_hybrid_bwd(
            _p(x, _D), _p(wg, _D), _p(wu, _D), _p(w_d, _D), _p(g_y, _D), M, K, N, P, float(l1),
            _p(hy_cnt, _I), _p(hy_idx, _I), _p(hy_g, _D), _p(hy_u, _D), _p(hy_h, _D),
            _p(route, _U8), _p(bk, _I), nbk, _p(bk_g, _D), _p(bk_u, _D), _p(bk_h, _D),
            _p(hy_du, _D), _p(hy_dz, _D), _p(bk_du, _D), _p(bk_dz, _D), _p(dx, _D),
            _p(dwg, _D), _p(dwu, _D), _p(dwd, _D))
        return {"hy_du": hy_du, "hy_dz": hy_dz, "bk_du": bk_du[:nbk], "bk_dz": bk_dz[:nbk],
                "dx": dx, "dwg_t": dwg, "dwu_t": dwu, "dwd": dwd}


_default = None


def default() -> Oracle:
    """The oracle built from ``tw_oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default
