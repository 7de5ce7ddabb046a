"""The hybrid training storage through the C ABI against the CPU oracle.

- TwELL -> hybrid is bit-exact: the oracle converts the GPU's own TwELL
  packing and must reproduce the GPU's counts, routing vector, backup list,
  backup count and the stored indices and values of every sparse row.
- Up values at the stored entries and the backup rows' dense g, u, h agree
  with the oracle's float64 values within the dot-product bound
  2 gamma_K sum_k |x_k w_k| (plus bf16 rounding, relative 2^-8, for the
  backup rows, which are stored in bf16).
- The down product agrees with the oracle's down product of the GPU's own
  stored h within 2 gamma_N sum |h w|, and the block output with the
  oracle's dense output within 1e-2 max|y_ref| + 1e-3.
- Rows routed to the backup beyond its room are left untouched.
"""
import numpy as np
import pytest

import oracle
import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
U24 = 2.0 ** -24
BF = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits)


@pytest.fixture(scope="module")
def tw():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def _bf16_to_f64(t):
    import torch

    return oracle.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _run(tw, dev, w, P, R_max):
    """Gate + TwELL, then the three hybrid calls; y prefilled with NaN."""
    import torch

    M, K = dev["x"].shape
    p = tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C, M)
    hy = tw.alloc_hybrid(M, w.N, P, R_max, keep=True)
    tw.tw_hybrid_pack(w.T, w.C, p["tw_val"], p["tw_idx"], p["tw_cnt"], P, hy["hy_g"],
                      hy["hy_idx"], hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"],
                      R_max)
    tw.tw_hybrid_up(dev["x"], dev["wg_t"], dev["wu_t"], P, hy["hy_g"], hy["hy_idx"],
                    hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"], R_max, hy["hy_u"],
                    hy["hy_h"], hy["bk_g"], hy["bk_u"], hy["bk_h"])
    y = torch.full((M, K), float("nan"), dtype=torch.float32, device=dev["x"].device)
    nws = tw.tw_hybrid_down_workspace_bytes(R_max)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev["x"].device)
    tw.tw_hybrid_down(dev["wd"], M, P, hy["hy_h"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                      hy["bk_rows"], hy["bk_count"], R_max, hy["bk_h"], y, ws)
    torch.cuda.synchronize()
    g = {k: p[k].cpu().numpy() for k in ("tw_val", "tw_idx", "tw_cnt")}
    for k in ("hy_cnt", "hy_idx", "hy_g", "hy_u", "hy_h", "route", "bk_rows"):
        g[k] = hy[k].cpu().numpy()
    g["bk_count"] = int(hy["bk_count"].cpu()[0])
    nbk = min(g["bk_count"], R_max)  # slots past it hold nothing
    for k in ("bk_g", "bk_u", "bk_h"):
        g[k] = _bf16_to_f64(hy[k][:nbk])
    g["y"] = y.cpu().numpy()
    return g


def _check_pack(g, C, P, R_max):
    ref = oracle.default().hybrid_pack({"cnt": g["tw_cnt"], "idx": g["tw_idx"],
                                        "val": g["tw_val"].astype(np.float64)}, C, P, R_max)
    assert np.array_equal(g["hy_cnt"], ref["hy_cnt"]), "counts differ"
    assert np.array_equal(g["route"], ref["route"]), "routing vector differs"
    assert g["bk_count"] == ref["bk_count"], (g["bk_count"], ref["bk_count"])
    nbk = min(ref["bk_count"], R_max)
    assert np.array_equal(g["bk_rows"][:nbk], ref["bk_rows"][:nbk]), "backup list differs"
    sparse = ref["route"] == 0
    used = (np.arange(P)[None, :] < ref["hy_cnt"][:, None]) & sparse[:, None]
    assert np.array_equal(np.where(used, g["hy_idx"], -1), np.where(used, ref["hy_idx"], -1)), \
        "stored indices differ"
    gv = g["hy_g"].astype(np.float64)
    assert np.array_equal(np.where(used, gv, 0.0).view(np.uint64),
                          np.where(used, ref["hy_val"], 0.0).view(np.uint64)), "stored values differ"
    return ref, used


def _sub_hybrid(g, rows):
    """The GPU's hybrid storage restricted to `rows` (ascending), with the
    backup slots renumbered within the subset, plus the GPU slot of each."""
    nbk = min(g["bk_count"], len(g["bk_rows"]))
    slot_of = {int(m): r for r, m in enumerate(g["bk_rows"][:nbk])}
    listed = [i for i, m in enumerate(rows) if g["route"][m] and int(m) in slot_of]
    hy = {"hy_cnt": g["hy_cnt"][rows], "hy_idx": g["hy_idx"][rows],
          "hy_val": g["hy_g"][rows].astype(np.float64), "route": g["route"][rows],
          "bk_rows": np.array(listed, dtype=np.int32), "bk_count": len(listed)}
    gslots = [slot_of[int(rows[i])] for i in listed]
    return hy, listed, gslots


def _check_values(g, d, rows, w, y_ref=None):
    """Up values, backup rows and y on `rows` against the oracle (y_ref: the
    oracle's dense output of those rows, if already computed)."""
    orc = oracle.default()
    x = d["x"][rows]
    hy, listed, gslots = _sub_hybrid(g, rows)
    up = orc.hybrid_up(x, d["wg_t"], d["wu_t"], hy)
    xa = np.abs(oracle.widen_bf16(x))
    K = xa.shape[1]
    gamma = K * U24 / (1 - K * U24)
    wua = np.abs(oracle.widen_bf16(d["wu_t"]))
    wga = np.abs(oracle.widen_bf16(d["wg_t"]))
    # sparse rows: hy_u and hy_h at the stored entries
    for i, m in enumerate(rows):
        if hy["route"][i]:
            continue
        n = int(hy["hy_cnt"][i])
        if n == 0:
            continue
        ids = hy["hy_idx"][i, :n]
        bu = 2 * gamma * (xa[i] @ wua[ids].T)
        u_ref = up["hy_u"][i, :n]
        gv = hy["hy_val"][i, :n]
        assert np.all(np.abs(g["hy_u"][m, :n] - u_ref) <= bu), f"hy_u row {m}"
        bh = gv * bu + 2 * U24 * np.abs(u_ref * gv) + 1e-30
        assert np.all(np.abs(g["hy_h"][m, :n] - u_ref * gv) <= bh), f"hy_h row {m}"
    # backup rows: dense bf16 g, u, h (the subset's backup slot k is listed[k])
    if listed:
        bz = 2 * gamma * (xa[listed] @ wga.T)
        bu = 2 * gamma * (xa[listed] @ wua.T)
        g_ref, u_ref, h_ref = up["bk_g"], up["bk_u"], up["bk_h"]
        gg, gu, gh = g["bk_g"][gslots], g["bk_u"][gslots], g["bk_h"][gslots]
        assert np.all(np.abs(gg - g_ref) <= bz + BF * (g_ref + bz)), "bk_g"
        assert np.all(np.abs(gu - u_ref) <= bu + BF * (np.abs(u_ref) + bu)), "bk_u"
        dh = g_ref * bu + np.abs(u_ref) * bz + bz * bu
        assert np.all(np.abs(gh - h_ref) <= dh + BF * (np.abs(h_ref) + dh) + 1e-30), "bk_h"
    # the down product of the GPU's own h, and the block output
    bk_h = g["bk_h"][gslots] if gslots else np.zeros((0, w.N))
    y_own = orc.hybrid_down(d["wd"], hy, g["hy_h"][rows].astype(np.float64), bk_h)
    done = ~np.isnan(y_own).any(axis=1)
    wda = np.abs(oracle.widen_bf16(d["wd"]))
    gamma_n = w.N * U24 / (1 - w.N * U24)
    h_abs = np.zeros((len(rows), w.N))
    for i in range(len(rows)):
        if not hy["route"][i]:
            n = int(hy["hy_cnt"][i])
            np.add.at(h_abs[i], hy["hy_idx"][i, :n], np.abs(g["hy_h"][rows[i], :n]))
    for k, i in enumerate(hy["bk_rows"]):
        h_abs[i] = np.abs(bk_h[k])
    bound = 2 * gamma_n * (h_abs @ wda) + 1e-30
    assert np.all(np.abs(g["y"][rows][done] - y_own[done]) <= bound[done]), "down product"
    if y_ref is None:
        y_ref = orc.dense_ffn(x, d["wg_t"], d["wu_t"], d["wd"])
    parity.check_y(g["y"][rows][done], y_ref[done], "hybrid y")
    # rows routed to the backup but past its room keep the NaN prefill
    assert np.all(np.isnan(g["y"][rows][~done])), "a row past the backup room was written"
    return int(done.sum()), int((~done).sum())


CASES = [
    ("tiny", dict(), 128, 8),
    ("tiny", dict(), 32, 8),                 # most rows heavy: backup room exceeded (retry)
    ("tiny", dict(), 32, 64),                # the same with room for every backup row
    ("tiny", dict(C=4), 128, 64),            # TwELL tiles overflow: routed by the tile rule
    ("tiny", dict(M=300, K=384, N=1152, C=6, density=0.03, sigma_s=0.5), 16, 300),
    ("tiny", dict(M=513, K=512, N=2048, T=256, C=12, density=0.01, sigma_s=0.7, seed=3), 24, 64),
    ("tiny", dict(M=1, K=128, N=128, C=3, density=0.1), 4, 1),
    ("tiny", dict(density=0.0), 128, 8),     # no active neuron: y = 0
    ("tiny", dict(density=1.0, C=128), 128, 64),  # every row heavy, all on the matrix cores
    ("tiny", dict(M=200, K=4096, N=256, C=64, density=0.1), 64, 200),  # the largest K
]


@pytest.mark.parametrize("name,kw,P,R_max", CASES)
def test_hybrid_parity(tw, name, kw, P, R_max):
    w = W[name].with_(**kw)
    print(f"case {w} P={P} R_max={R_max}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    g = _run(tw, dev, w, P, R_max)
    ref, _ = _check_pack(g, w.C, P, R_max)
    done, left = _check_values(g, d, np.arange(w.M), w)
    assert left == max(0, ref["bk_count"] - R_max)
    if kw.get("density") == 0.0:
        assert not g["y"].any() and g["bk_count"] == 0


@pytest.mark.parametrize("name", ["ffn-0.5b", "ffn-1b", "ffn-2b", "ffn-ovf", "ffn-paper"])
def test_hybrid_full_size(tw, name):
    """Full shapes at the static capacities (P = 128, backup room M / 8):
    the whole conversion bit-exact, and the up values, the backup rows and
    y of every row against the oracle (in blocks of rows)."""
    w = W[name]
    P, R_max = 128, w.M // 8
    print(f"case {w} P={P} R_max={R_max}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    g = _run(tw, dev, w, P, R_max)
    del dev
    ref, _ = _check_pack(g, w.C, P, R_max)
    assert ref["bk_count"] <= R_max, "the static backup room overflowed at this workload"
    y_ref = parity.dense_reference(w, d)
    done = left = 0
    for r0 in range(0, w.M, 2048):
        rows = np.arange(r0, min(r0 + 2048, w.M))
        a, b = _check_values(g, d, rows, w, y_ref[rows])
        done, left = done + a, left + b
    assert done == w.M and left == 0
    print(f"all {w.M} rows ({ref['bk_count']} backup rows)", flush=True)


def test_hybrid_forward_wrapper(tw):
    """hybrid_forward (the allocating wrapper) gives the same y as the three
    calls, and the same y twice in a row (no state between calls)."""
    import torch

    w = W["tiny"].with_(M=700, C=6, density=0.03, sigma_s=0.5)
    print(f"case {w}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    p = tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C)
    y1, hy1 = tw.hybrid_forward(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"], p, P=32, R_max=700)
    y2, _ = tw.hybrid_forward(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"], p, P=32, R_max=700,
                              keep=False)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert int(hy1["bk_count"].cpu()[0]) > 0


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(C=12)),
    ("ffn-2b", dict(M=16)),      # the small-batch gate's K-sliced route
    ("ffn-0.5b", dict()),
])
def test_pack_gate_without_overflow_list(tw, name, kw):
    """tw_pack_gate with no overflow list (both pointers NULL, as the
    training path calls it: tw_hybrid_pack routes from tw_cnt) writes the
    same TwELL packing, bit for bit, as with the list."""
    import torch

    w = W[name].with_(**kw)
    print(f"case {w}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    M, R_max = w.M, w.M
    a = tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C, R_max)
    b = tw.alloc_pack(M, w.N, w.T, w.C, R_max)
    for k in ("tw_val", "tw_idx"):
        b[k].fill_(-7)
    ws = tw.workspace(M, w.K, w.N, w.T, w.C, R_max)
    tw.tw_pack_gate(dev["x"], dev["wg_t"], w.T, w.C, b["tw_val"], b["tw_idx"], b["tw_cnt"],
                    None, None, R_max, ws)
    torch.cuda.synchronize()
    assert torch.equal(a["tw_cnt"], b["tw_cnt"])
    C = w.C
    used = (torch.arange(C, device="cuda")[None, None, :] <
            torch.clamp(a["tw_cnt"], max=C)[:, :, None])
    assert torch.equal(torch.where(used, a["tw_idx"], -1), torch.where(used, b["tw_idx"], -1))
    assert torch.equal(torch.where(used, a["tw_val"], 0).view(torch.int32),
                       torch.where(used, b["tw_val"], 0).view(torch.int32))
