"""Pins of the CPU oracle to facts outside the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` when the oracle disagrees with what the method's
definition, a library routine or exact arithmetic fixes.  They are run on the
real oracle (``test_oracle_pins.py``) and on builds of the oracle with a
planted mistake (``test_oracle_mutants.py``), where at least one of them must
fail.

Definitions ("Sparser, Faster, Lighter Transformer Language Models Review"):
section 1-1 (the gated FFN equation and exact ReLU zeros), section 3-3 (the
row-wide ELL component table), section 3-4 (TwELL tiles, local packing with
the original hidden index and a per-(row, tile) count), section 3-5 (the
per-token sparse equation), section 3-6 / 4-3 (whole-row dense backup with a
routing vector and retry on overflow).
"""
from __future__ import annotations

import os
import random

import numpy as np

from activation_sparse_feed_gate_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "handworked_4x4x8.txt")


# --------------------------------------------------------------------------
# golden fixture
# --------------------------------------------------------------------------
def load_golden(path: str = GOLDEN) -> dict:
    """Parse the hand-worked fixture: scalars, integer matrices, slot tables."""
    lines = []
    with open(path) as f:
        for raw in f:
            s = raw.split("#", 1)[0].strip()
            if s:
                lines.append(s)
    out, i = {}, 0
    while i < len(lines):
        head = lines[i].split()
        if len(head) >= 2 and head[0] in ("M", "K", "N", "T", "C", "ovf_count"):
            out[head[0]] = int(head[1])
            i += 1
        elif head[0] == "ovf_rows":
            out["ovf_rows"] = [int(v) for v in head[1:]]
            i += 1
        else:
            name = head[0]
            i += 1
            rows = []
            while i < len(lines) and (lines[i][0].isdigit() or lines[i][0] in "-.|"):
                rows.append(lines[i])
                i += 1
            out[name] = rows
    M, K, N, T, C = (out[k] for k in "MKNTC")
    NT = N // T
    for name in ("x", "wg_t", "wu_t", "wd", "z", "cnt", "y"):
        out[name] = np.array([[int(v) for v in r.split()] for r in out[name]], dtype=np.int64)
    for name in ("idx", "val"):
        tab = np.full((M, NT, C), -1, dtype=np.int64)
        used = np.zeros((M, NT, C), dtype=bool)
        for m, r in enumerate(out[name]):
            for t, part in enumerate(r.split("|")):
                for s, v in enumerate(part.split()):
                    if v != ".":
                        tab[m, t, s] = int(v)
                        used[m, t, s] = True
        out[name] = tab
        out[name + "_used"] = used
    return out


def _bits(a) -> np.ndarray:
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _check_packing(p: dict, cnt, idx, val, used, ovf_rows, ovf_count):
    assert np.array_equal(p["cnt"], cnt), "cnt"
    assert np.array_equal(np.where(used, p["idx"], -1), np.where(used, idx, -1)), "idx"
    assert np.array_equal(np.where(used, p["val"], 0.0), np.where(used, val, 0.0)), "val"
    assert list(p["ovf_rows"]) == list(ovf_rows), "ovf_rows"
    assert p["ovf_count"] == ovf_count, "ovf_count"


def pin_golden(orc) -> None:
    """Hand-worked 4x4x8 example: every intermediate and output exact."""
    g = load_golden()
    T, C = g["T"], g["C"]
    x, wg, wu, wd = (_bits(g[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    z = orc.gate(x, wg)
    assert np.array_equal(z, g["z"].astype(np.float64)), "z"
    p = orc.pack(z, T, C, R_max=g["M"])
    _check_packing(p, g["cnt"], g["idx"], g["val"].astype(np.float64), g["idx_used"],
                   g["ovf_rows"], g["ovf_count"])
    assert np.array_equal(p["flag"].astype(bool), np.isin(np.arange(g["M"]), g["ovf_rows"]))
    y_dense = orc.dense_ffn(x, wg, wu, wd)
    assert np.array_equal(y_dense, g["y"].astype(np.float64)), "dense y"
    y_sparse = orc.sparse_ffn(x, wg, wu, wd, T, C, p)
    assert np.array_equal(y_sparse, g["y"].astype(np.float64)), "sparse y"
    # no room in the dense backup: the list stays empty, the true count remains
    p0 = orc.pack(z, T, C, R_max=0)
    assert list(p0["ovf_rows"]) == [] and p0["ovf_count"] == g["ovf_count"], "R_max=0"


# --------------------------------------------------------------------------
# exact brute force with Python integers
# --------------------------------------------------------------------------
def _brute(x, wg, wu, wd, T, C, R_max):
    M, K = len(x), len(x[0])
    N = len(wg)
    z = [[sum(x[m][k] * wg[j][k] for k in range(K)) for j in range(N)] for m in range(M)]
    g = [[v if v > 0 else 0 for v in row] for row in z]
    u = [[sum(x[m][k] * wu[j][k] for k in range(K)) for j in range(N)] for m in range(M)]
    y = [[sum(g[m][j] * u[m][j] * wd[j][k] for j in range(N)) for k in range(K)]
         for m in range(M)]
    NT = N // T
    cnt = [[0] * NT for _ in range(M)]
    slots = [[[] for _ in range(NT)] for _ in range(M)]
    over = []
    for m in range(M):
        for t in range(NT):
            act = [j for j in range(t * T, (t + 1) * T) if g[m][j] != 0]
            cnt[m][t] = len(act)
            slots[m][t] = [(j, g[m][j]) for j in act[:C]]
        if any(c > C for c in cnt[m]):
            over.append(m)
    return z, cnt, slots, over[:R_max], len(over), y


def pin_bruteforce(orc, cases: int = 40, seed: int = 1234) -> None:
    """Random small integer problems, exact in bfloat16 and double."""
    rnd = random.Random(seed)
    for _ in range(cases):
        T = rnd.choice([1, 2, 3, 4])
        NT = rnd.randint(1, 3)
        N = T * NT
        K = rnd.randint(1, max(1, N))
        M = rnd.randint(1, 6)
        C = rnd.randint(1, T)
        R_max = rnd.randint(0, M)
        draw = lambda r, c: [[rnd.randint(-3, 3) for _ in range(c)] for _ in range(r)]
        x, wg, wu, wd = draw(M, K), draw(N, K), draw(N, K), draw(N, K)
        z, cnt, slots, ovf, n_ovf, y = _brute(x, wg, wu, wd, T, C, R_max)
        bx, bg, bu, bd = (_bits(a) for a in (x, wg, wu, wd))
        zo = orc.gate(bx, bg)
        assert np.array_equal(zo, np.array(z, dtype=np.float64)), "z"
        p = orc.pack(zo, T, C, R_max)
        assert np.array_equal(p["cnt"], np.array(cnt)), "cnt"
        for m in range(M):
            for t in range(NT):
                for s, (j, v) in enumerate(slots[m][t]):
                    assert p["idx"][m, t, s] == j, "idx"
                    assert p["val"][m, t, s] == v, "val"
        assert list(p["ovf_rows"]) == ovf and p["ovf_count"] == n_ovf, "ovf"
        yd = orc.dense_ffn(bx, bg, bu, bd)
        assert np.array_equal(yd, np.array(y, dtype=np.float64)), "dense y"
        ys = orc.sparse_ffn(bx, bg, bu, bd, T, C, p)
        assert np.array_equal(ys, np.array(y, dtype=np.float64)), "sparse y"


# --------------------------------------------------------------------------
# special cases reducing to a library routine or a closed form
# --------------------------------------------------------------------------
def _tiny(**kw):
    w = synth.WORKLOADS["tiny"].with_(**kw)
    return w, synth.make_inputs(w)


def pin_csr_library(orc) -> None:
    """Per-tile packing equals scipy's CSR of each column tile of ReLU(z).

    With T = N the tile is the whole row and TwELL is the row-wide ELL of
    section 3-3 (value matrix, index matrix, count vector); CSR holds the same
    per-row counts, ascending column indices and values.
    """
    import scipy.sparse as sp

    w, d = _tiny(M=24)
    z = orc.gate(d["x"], d["wg_t"])
    g = np.where(z > 0.0, z, 0.0)
    for T, C in ((w.N, w.N), (w.N, 20), (128, 16), (128, 3), (256, 256)):
        p = orc.pack(z, T, C, R_max=w.M)
        for t in range(w.N // T):
            csr = sp.csr_matrix(g[:, t * T:(t + 1) * T])
            csr.sort_indices()
            counts = np.diff(csr.indptr)
            assert np.array_equal(p["cnt"][:, t], counts), "cnt vs CSR"
            for m in range(w.M):
                a, b = csr.indptr[m], csr.indptr[m + 1]
                n = min(b - a, C)
                assert np.array_equal(p["idx"][m, t, :n], csr.indices[a:a + n] + t * T), "idx"
                assert np.array_equal(p["val"][m, t, :n], csr.data[a:a + n]), "val"
        rows = np.nonzero((p["cnt"] > C).any(axis=1))[0]
        assert np.array_equal(p["ovf_rows"], rows) and p["ovf_count"] == len(rows), "routing"
        if C == T:
            assert p["ovf_count"] == 0, "lossless capacity never overflows"


def pin_numpy_dense(orc) -> None:
    """Gate and output agree with numpy's float64 matrix products to rounding."""
    w, d = _tiny(M=32)
    x, wg, wu, wd = (orc_widen(a) for a in (d["x"], d["wg_t"], d["wu_t"], d["wd"]))
    z = orc.gate(d["x"], d["wg_t"])
    z_np = x @ wg.T
    bound_z = 4 * w.K * 2.0 ** -53 * (np.abs(x) @ np.abs(wg).T) + 1e-300
    assert np.all(np.abs(z - z_np) <= bound_z), "gate vs numpy"
    y = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    h = np.where(z_np > 0, z_np, 0.0) * (x @ wu.T)
    y_np = h @ wd
    scale = np.abs(h) @ np.abs(wd) + 1e-300
    assert np.all(np.abs(y - y_np) <= 1e-9 * scale + 1e-12 * np.abs(y_np).max()), "y vs numpy"


def orc_widen(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def pin_onehot(orc) -> None:
    """One-hot token rows select one input coordinate, so z is a column of W_g
    exactly, and y is the closed-form sum over that coordinate's actives."""
    w, d = _tiny(M=1)
    K, N, T, C = w.K, w.N, 128, 128
    ks = np.arange(0, K, 17)
    x = np.zeros((len(ks), K), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    xb = _bits(x)
    z = orc.gate(xb, d["wg_t"])
    wg = orc_widen(d["wg_t"])
    wu = orc_widen(d["wu_t"])
    wd = orc_widen(d["wd"])
    assert np.array_equal(z, wg[:, ks].T), "one-hot gate"
    p = orc.pack(z, T, C, R_max=len(ks))
    for r, k in enumerate(ks):
        for t in range(N // T):
            act = np.nonzero(wg[t * T:(t + 1) * T, k] > 0)[0] + t * T
            assert p["cnt"][r, t] == len(act), "one-hot count"
            assert np.array_equal(p["idx"][r, t, :len(act)], act), "one-hot idx"
    y = orc.dense_ffn(xb, d["wg_t"], d["wu_t"], d["wd"])
    for r, k in enumerate(ks):
        act = np.nonzero(wg[:, k] > 0)[0]
        # each term is a product of three bf16 values: exact in double when
        # the summation is done in the same ascending order
        acc = np.zeros(K)
        for j in act:
            acc = acc + (wu[j, k] * wg[j, k]) * wd[j]
        assert np.array_equal(y[r], acc), "one-hot y"


def pin_invariants(orc) -> None:
    """Invariants on generator inputs, with and without overflow.

    Sum of tile counts equals the number of positive gate entries; every
    active (row, column) appears exactly once -- in the packed slots of a
    non-overflow row or through that row's place on the overflow list; the
    indices of a tile are strictly ascending and inside the tile; packed
    values equal the gate entries; the sparse evaluation is bit-for-bit the
    dense one (same dot products, same ascending order; an inactive term
    only ever adds a signed zero).
    """
    for C, R_max in ((16, 64), (12, 64), (4, 64), (4, 10)):
        w, d = _tiny(C=C)
        z = orc.gate(d["x"], d["wg_t"])
        p = orc.pack(z, w.T, C, R_max)
        NT = w.N // w.T
        act = z > 0.0
        assert int(p["cnt"].sum()) == int(act.sum()), "sum of counts"
        flagged = (p["cnt"] > C).any(axis=1)
        rows = np.nonzero(flagged)[0]
        assert p["ovf_count"] == len(rows) and np.array_equal(p["ovf_rows"], rows[:R_max])
        seen = np.zeros_like(act, dtype=np.int64)
        for m in range(w.M):
            if flagged[m]:
                seen[m] += act[m]
                continue
            for t in range(NT):
                n = p["cnt"][m, t]
                ids = p["idx"][m, t, :n]
                assert np.all(np.diff(ids) > 0), "ascending"
                assert np.all((ids >= t * w.T) & (ids < (t + 1) * w.T)), "inside tile"
                assert np.array_equal(p["val"][m, t, :n], z[m, ids]), "values"
                seen[m, ids] += 1
        assert np.array_equal(seen, act.astype(np.int64)), "each active exactly once"
        yd = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
        ys = orc.sparse_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"], w.T, C, p)
        assert np.array_equal(ys.view(np.uint64), yd.view(np.uint64)), "sparse == dense bitwise"


def pin_density_extremes(orc) -> None:
    """Exactly 0 and exactly 1 density."""
    w, d = _tiny(density=0.0)
    z = orc.gate(d["x"], d["wg_t"])
    p = orc.pack(z, w.T, w.C, w.M)
    assert not p["cnt"].any() and p["ovf_count"] == 0, "density 0 packing"
    yd = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    ys = orc.sparse_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"], w.T, w.C, p)
    assert not yd.any() and not ys.any(), "density 0 output"

    w, d = _tiny(density=1.0, C=128)
    z = orc.gate(d["x"], d["wg_t"])
    p = orc.pack(z, w.T, w.C, w.M)
    NT = w.N // w.T
    assert np.all(p["cnt"] == w.T) and p["ovf_count"] == 0, "density 1, C = T"
    full = np.arange(w.N).reshape(NT, w.T)
    assert np.all(p["idx"] == full[None]), "density 1 indices"
    yd = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    ys = orc.sparse_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"], w.T, w.C, p)
    assert np.array_equal(ys, yd), "density 1, C = T: sparse == dense"

    p = orc.pack(z, w.T, 16, w.M)
    assert p["ovf_count"] == w.M and np.array_equal(p["ovf_rows"], np.arange(w.M)), \
        "density 1, C < T: every row overflows"
    p = orc.pack(z, w.T, 16, 5)
    assert p["ovf_count"] == w.M and np.array_equal(p["ovf_rows"], np.arange(5)), \
        "overflow beyond R_max is reported for retry"


# --------------------------------------------------------------------------
# hybrid storage of the training forward (sections 3-6, 3-7, 4-3)
# --------------------------------------------------------------------------
HYBRID_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                             "handworked_hybrid_4x4x8.txt")


def load_hybrid_golden(path: str = HYBRID_GOLDEN) -> dict:
    """Parse the hand-worked hybrid fixture into its cases and value tables."""
    out = {"cases": [], "up": {}, "backup_g": {}, "backup_u": {}, "backup_h": {}}
    case = None
    with open(path) as f:
        for raw in f:
            s = raw.split("#", 1)[0].strip()
            if not s:
                continue
            head = s.split()
            key = head[0]
            if key == "hy_cnt":
                out["hy_cnt"] = [int(v) for v in head[1:]]
            elif key == "case":
                case = {"P": int(head[2]), "R_max": int(head[4]), "sparse": {}}
                out["cases"].append(case)
            elif key in ("route", "bk_rows"):
                case[key] = [int(v) for v in head[1:]]
            elif key == "bk_count":
                case[key] = int(head[1])
            else:
                row = int(head[1])
                body = s.split(":", 1)[1].strip()
                items = [[int(v) for v in e.split()] for e in body.split(",")] if body else []
                if key == "sparse":
                    case["sparse"][row] = items
                elif key == "up":
                    out["up"][row] = items
                else:
                    out[key][row] = items[0]
    return out


def pin_hybrid_golden(orc) -> None:
    """Hand-worked hybrid storage, up values and output of the 4x4x8 example."""
    g = load_golden()
    hg = load_hybrid_golden()
    T, C, M = g["T"], g["C"], g["M"]
    x, wg, wu, wd = (_bits(g[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    p = orc.pack(orc.gate(x, wg), T, C, R_max=M)
    for case in hg["cases"]:
        P, R_max = case["P"], case["R_max"]
        hy = orc.hybrid_pack(p, C, P, R_max)
        tag = f"P={P} R_max={R_max}"
        assert list(hy["hy_cnt"]) == hg["hy_cnt"], "hy_cnt " + tag
        assert list(hy["route"]) == case["route"], "route " + tag
        assert list(hy["bk_rows"]) == case["bk_rows"], "bk_rows " + tag
        assert hy["bk_count"] == case["bk_count"], "bk_count " + tag
        for m, items in case["sparse"].items():
            n = len(items)
            assert hy["hy_cnt"][m] == n, "sparse count " + tag
            assert [int(v) for v in hy["hy_idx"][m, :n]] == [e[0] for e in items], "idx " + tag
            assert [float(v) for v in hy["hy_val"][m, :n]] == [e[1] for e in items], "val " + tag
        if R_max < case["bk_count"]:
            continue
        up = orc.hybrid_up(x, wg, wu, hy)
        for m, items in hg["up"].items():
            if hy["route"][m]:
                continue
            n = len(items)
            assert [int(v) for v in hy["hy_idx"][m, :n]] == [e[0] for e in items], "up idx " + tag
            assert list(up["hy_u"][m, :n]) == [e[1] for e in items], "hy_u " + tag
            assert list(up["hy_h"][m, :n]) == [e[2] for e in items], "hy_h " + tag
        for r, m in enumerate(hy["bk_rows"]):
            for key in ("bk_g", "bk_u", "bk_h"):
                want = hg["backup_" + key[3:]][int(m)]
                assert list(up[key][r]) == want, f"{key} row {m} " + tag
        y = orc.hybrid_down(wd, hy, up["hy_h"], up["bk_h"])
        assert np.array_equal(y, g["y"].astype(np.float64)), "hybrid y " + tag


def _brute_hybrid(cnt, slots, C, P, R_max):
    """Hybrid storage from a TwELL packing given as Python lists."""
    M = len(cnt)
    hy_cnt, route, ell = [], [], []
    for m in range(M):
        n = sum(cnt[m])
        heavy = n > P or any(c > C for c in cnt[m])
        hy_cnt.append(n)
        route.append(1 if heavy else 0)
        ell.append([] if heavy else [e for t in range(len(cnt[m])) for e in slots[m][t]])
    bk = [m for m in range(M) if route[m]]
    return hy_cnt, route, ell, bk[:R_max], len(bk)


def pin_hybrid_bruteforce(orc, cases: int = 40, seed: int = 4321) -> None:
    """Random small integer problems: hybrid storage, up values at the stored
    entries, dense backup rows and y, exact against Python integers."""
    rnd = random.Random(seed)
    for _ in range(cases):
        T = rnd.choice([1, 2, 3, 4])
        NT = rnd.randint(1, 3)
        N = T * NT
        K = rnd.randint(1, max(1, N))
        M = rnd.randint(1, 6)
        C = rnd.randint(1, T)
        P = rnd.randint(1, N)
        draw = lambda r, c: [[rnd.randint(-3, 3) for _ in range(c)] for _ in range(r)]
        x, wg, wu, wd = draw(M, K), draw(N, K), draw(N, K), draw(N, K)
        z, cnt, slots, _, _, y = _brute(x, wg, wu, wd, T, C, M)
        hy_cnt, route, ell, _, n_bk = _brute_hybrid(cnt, slots, C, P, M)
        R_max = rnd.randint(n_bk, M) if rnd.random() < 0.7 else rnd.randint(0, M)
        bk = [m for m in range(M) if route[m]][:R_max]
        bx, bg, bu, bd = (_bits(a) for a in (x, wg, wu, wd))
        p = orc.pack(orc.gate(bx, bg), T, C, M)
        hy = orc.hybrid_pack(p, C, P, R_max)
        assert list(hy["hy_cnt"]) == hy_cnt and list(hy["route"]) == route, "routing"
        assert list(hy["bk_rows"]) == bk and hy["bk_count"] == n_bk, "backup list"
        for m in range(M):
            if route[m]:
                continue
            n = len(ell[m])
            assert [int(v) for v in hy["hy_idx"][m, :n]] == [j for j, _ in ell[m]], "idx"
            assert [float(v) for v in hy["hy_val"][m, :n]] == [v for _, v in ell[m]], "val"
        up = orc.hybrid_up(bx, bg, bu, hy)
        u = [[sum(x[m][k] * wu[j][k] for k in range(K)) for j in range(N)] for m in range(M)]
        for m in range(M):
            if route[m]:
                continue
            for s, (j, gv) in enumerate(ell[m]):
                assert up["hy_u"][m, s] == u[m][j] and up["hy_h"][m, s] == u[m][j] * gv, "up"
        for r, m in enumerate(bk):
            gr = [v if v > 0 else 0 for v in z[m]]
            assert list(up["bk_g"][r]) == gr and list(up["bk_u"][r]) == u[m], "backup g/u"
            assert list(up["bk_h"][r]) == [a * b for a, b in zip(gr, u[m])], "backup h"
        yh = orc.hybrid_down(bd, hy, up["hy_h"], up["bk_h"])
        for m in range(M):
            if route[m] and m not in bk:
                assert np.all(np.isnan(yh[m])), "rows past the backup room stay unwritten"
            else:
                assert list(yh[m]) == y[m], "hybrid y"


def pin_hybrid_library(orc) -> None:
    """With room for every entry (P = N, lossless TwELL C = T) no row is
    heavy and the sparse store is the row-wide ELL of section 3-3, which holds
    exactly scipy's CSR rows of ReLU(z); the up values at the stored entries
    and the output agree with numpy's float64 products to rounding."""
    import scipy.sparse as sp

    w, d = _tiny(M=24)
    x, wu, wd = (orc_widen(a) for a in (d["x"], d["wu_t"], d["wd"]))
    z = orc.gate(d["x"], d["wg_t"])
    g = np.where(z > 0.0, z, 0.0)
    p = orc.pack(z, w.T, w.T, w.M)
    hy = orc.hybrid_pack(p, w.T, w.N, w.M)
    assert not hy["route"].any() and hy["bk_count"] == 0, "nothing is heavy"
    csr = sp.csr_matrix(g)
    csr.sort_indices()
    assert np.array_equal(hy["hy_cnt"], np.diff(csr.indptr)), "counts vs CSR"
    up = orc.hybrid_up(d["x"], d["wg_t"], d["wu_t"], hy)
    u_np = x @ wu.T
    bound_u = 4 * w.K * 2.0 ** -53 * (np.abs(x) @ np.abs(wu).T) + 1e-300
    h_dense = np.zeros((w.M, w.N))
    for m in range(w.M):
        a, b = csr.indptr[m], csr.indptr[m + 1]
        ids = csr.indices[a:b]
        assert np.array_equal(hy["hy_idx"][m, :b - a], ids), "idx vs CSR"
        assert np.array_equal(hy["hy_val"][m, :b - a], csr.data[a:b]), "val vs CSR"
        assert np.all(np.abs(up["hy_u"][m, :b - a] - u_np[m, ids]) <= bound_u[m, ids]), "u"
        h_dense[m, ids] = up["hy_h"][m, :b - a]
    y = orc.hybrid_down(d["wd"], hy, up["hy_h"], up["bk_h"])
    y_np = h_dense @ wd
    scale = np.abs(h_dense) @ np.abs(wd) + 1e-300
    assert np.all(np.abs(y - y_np) <= 1e-12 * scale), "y vs numpy"


def pin_hybrid_invariants(orc) -> None:
    """Generator inputs at several capacities: each active entry is stored
    exactly once (a sparse slot, or its row in the backup); the routing is the
    stated rule; stored indices ascend; the composed hybrid forward equals the
    oracle's dense block output bit for bit (same dot products, same
    ascending order, inactive terms only add signed zeros)."""
    for C, P, R_max in ((16, 128, 64), (12, 64, 64), (4, 40, 64), (16, 48, 64), (16, 48, 3)):
        w, d = _tiny(C=C)
        z = orc.gate(d["x"], d["wg_t"])
        p = orc.pack(z, w.T, C, w.M)
        hy = orc.hybrid_pack(p, C, P, R_max)
        act = z > 0.0
        nnz = act.sum(axis=1)
        heavy = (nnz > P) | (p["cnt"] > C).any(axis=1)
        assert np.array_equal(hy["hy_cnt"], nnz), "true counts"
        assert np.array_equal(hy["route"].astype(bool), heavy), "routing rule"
        rows = np.nonzero(heavy)[0]
        assert hy["bk_count"] == len(rows) and np.array_equal(hy["bk_rows"], rows[:R_max])
        for m in np.nonzero(~heavy)[0]:
            n = nnz[m]
            ids = hy["hy_idx"][m, :n]
            assert np.array_equal(ids, np.nonzero(act[m])[0]), "stored entries"
            assert np.array_equal(hy["hy_val"][m, :n], z[m, ids]), "stored values"
            assert np.all(hy["hy_idx"][m, n:] == -1), "unused slots"
        up = orc.hybrid_up(d["x"], d["wg_t"], d["wu_t"], hy)
        y = orc.hybrid_down(d["wd"], hy, up["hy_h"], up["bk_h"])
        yd = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
        done = ~heavy
        done[hy["bk_rows"]] = True
        assert np.array_equal(y[done].view(np.uint64), yd[done].view(np.uint64)), \
            "hybrid forward == dense bitwise"
        assert np.all(np.isnan(y[~done])), "rows past the backup room are not written"


def pin_hybrid_extremes(orc) -> None:
    """Density 0: every row sparse and empty, y = 0.  Density 1 with P < N:
    every row heavy; with a small backup room the true count is reported."""
    w, d = _tiny(density=0.0)
    p = orc.pack(orc.gate(d["x"], d["wg_t"]), w.T, w.C, w.M)
    hy = orc.hybrid_pack(p, w.C, 128, w.M // 8)
    assert not hy["hy_cnt"].any() and not hy["route"].any() and hy["bk_count"] == 0
    up = orc.hybrid_up(d["x"], d["wg_t"], d["wu_t"], hy)
    y = orc.hybrid_down(d["wd"], hy, up["hy_h"], up["bk_h"])
    assert not y.any(), "density 0 output"

    w, d = _tiny(density=1.0, C=128)
    p = orc.pack(orc.gate(d["x"], d["wg_t"]), w.T, w.C, w.M)
    hy = orc.hybrid_pack(p, w.C, 128, w.M // 8)
    assert np.all(hy["hy_cnt"] == w.N) and hy["route"].all(), "density 1: every row heavy"
    assert hy["bk_count"] == w.M and np.array_equal(hy["bk_rows"], np.arange(w.M // 8)), \
        "backup room exceeded: retry signalled"
    hy = orc.hybrid_pack(p, w.C, w.N, w.M)
    assert not hy["route"].any() and np.all(hy["hy_idx"] == np.arange(w.N)[None]), \
        "density 1, P = N: every row sparse and full"


# --------------------------------------------------------------------------
# backward over hybrid storage (section 3-7, L1 of section 3-2)
# --------------------------------------------------------------------------
def _autograd(x, wg, wu, wd, dy, l1):
    """Gradients of sum(y * dy) + l1 * sum(ReLU(x W_g)) by torch autograd in
    float64 on the CPU (a library routine, independent of the oracle),
    with the gradients of u = x W_u and z = x W_g kept."""
    import torch

    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    X, Wg, Wu, Wd = t(x), t(wg), t(wu), t(wd)
    z = X @ Wg.T
    u = X @ Wu.T
    z.retain_grad()
    u.retain_grad()
    g = torch.relu(z)
    y = (g * u) @ Wd
    loss = (y * torch.tensor(np.asarray(dy, dtype=np.float64))).sum() + l1 * g.sum()
    loss.backward()
    return {"dx": X.grad.numpy(), "dwg_t": Wg.grad.numpy(), "dwu_t": Wu.grad.numpy(),
            "dwd": Wd.grad.numpy(), "du": u.grad.numpy(), "dz": z.grad.numpy()}


def _stored_rows(hy):
    listed = set(int(m) for m in hy["bk_rows"])
    return np.array([m for m in range(len(hy["route"])) if not hy["route"][m] or m in listed],
                    dtype=np.int64)


def _check_bwd(orc, bx, bg, bu, bd, bdy, T, C, P, R_max, l1, exact):
    """Hybrid forward then backward on the oracle against autograd over the
    rows whose activations are stored."""
    p = orc.pack(orc.gate(bx, bg), T, C, len(bx))
    hy = orc.hybrid_pack(p, C, P, R_max)
    up = orc.hybrid_up(bx, bg, bu, hy)
    b = orc.hybrid_bwd(bx, bg, bu, bd, bdy, hy, up, l1)
    rows = _stored_rows(hy)
    X, DY = orc_widen(bx), orc_widen(bdy)
    ref = _autograd(X[rows], orc_widen(bg), orc_widen(bu), orc_widen(bd), DY[rows], l1)
    if exact:
        close = lambda a, r: np.array_equal(a, r)
    else:
        close = lambda a, r: np.all(np.abs(a - r) <= 1e-12 * (np.abs(r).max(initial=0) + 1))
    assert close(b["dx"][rows], ref["dx"]), "dx"
    assert np.all(np.isnan(np.delete(b["dx"], rows, axis=0))), "rows with nothing stored"
    for k in ("dwg_t", "dwu_t", "dwd"):
        assert close(b[k], ref[k]), k
    pos = {int(m): i for i, m in enumerate(rows)}
    for m in range(len(hy["route"])):
        if hy["route"][m]:
            continue
        n = int(hy["hy_cnt"][m])
        ids = hy["hy_idx"][m, :n]
        i = pos[m]
        assert close(b["hy_du"][m, :n], ref["du"][i, ids]), "du at the stored entries"
        assert close(b["hy_dz"][m, :n], ref["dz"][i, ids]), "dz at the stored entries"
    for r, m in enumerate(hy["bk_rows"]):
        i = pos[int(m)]
        assert close(b["bk_du"][r], ref["du"][i]), "backup du"
        assert close(b["bk_dz"][r], ref["dz"][i]), "backup dz"
    return hy


def pin_hybrid_bwd_exact(orc, cases: int = 30, seed: int = 777) -> None:
    """Random small integer problems and integer L1 gradients: every gradient
    exactly torch autograd's (all values are small integers, exact in bf16
    and double), including a backup room too small for every heavy row."""
    rnd = random.Random(seed)
    for _ in range(cases):
        T = rnd.choice([1, 2, 4])
        N = T * rnd.randint(1, 3)
        K = rnd.randint(1, 5)
        M = rnd.randint(1, 6)
        C = rnd.randint(1, T)
        P = rnd.randint(1, N)
        R_max = rnd.randint(0, M)
        l1 = rnd.choice([0, 1, 2])
        draw = lambda r, c: [[rnd.randint(-3, 3) for _ in range(c)] for _ in range(r)]
        bx, bg, bu, bd, bdy = (_bits(a) for a in (draw(M, K), draw(N, K), draw(N, K),
                                                  draw(N, K), draw(M, K)))
        _check_bwd(orc, bx, bg, bu, bd, bdy, T, C, P, R_max, l1, exact=True)


def pin_hybrid_bwd_autograd(orc) -> None:
    """Generator inputs: sparse rows only, many backup rows, and the tile
    rule, against autograd within rounding."""
    for C, P, l1 in ((16, 128, 0.0), (12, 40, 0.01), (4, 128, 0.05)):
        w, d = _tiny(C=C)
        rng = np.random.default_rng(5)
        dy = synth.f32_to_bf16_bits(rng.standard_normal((w.M, w.K)).astype(np.float32))
        hy = _check_bwd(orc, d["x"], d["wg_t"], d["wu_t"], d["wd"], dy, w.T, C, P, w.M, l1,
                        exact=False)
        if P == 40:
            assert hy["bk_count"] > 10, "the backup path is exercised"


ALL_PINS = [pin_golden, pin_bruteforce, pin_csr_library, pin_numpy_dense, pin_onehot,
            pin_invariants, pin_density_extremes, pin_hybrid_golden, pin_hybrid_bruteforce,
            pin_hybrid_library, pin_hybrid_invariants, pin_hybrid_extremes,
            pin_hybrid_bwd_exact, pin_hybrid_bwd_autograd]
