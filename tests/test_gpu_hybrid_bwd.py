"""The backward over hybrid storage through the C ABI against the CPU oracle.

The GPU forward (tw_pack_gate, tw_hybrid_pack, tw_hybrid_up with g and u
kept) provides the stored activations; the oracle's backward runs on exactly
those values (fp32 sparse rows, bf16 backup rows widened), so every
difference is the backward's own arithmetic:
- du, dz at the stored entries: dh is an fp32 dot product, within
  2 gamma_K sum_k |dy_k w_k| of the oracle's, then one or two roundings (and
  bf16 rounding, relative 2^-8, for the backup rows);
- dx and the weight gradients: within the propagated du / dz differences
  plus 2 gamma_n of the sum of the absolute terms (fp32 accumulation), and
  within 1e-2 max|ref| + 1e-3 overall;
- rows past the backup room get no dx; the gradients are bit-identical run
  to run (fixed-order sums, the transpose sorted by row).
"""
import numpy as np
import pytest

import oracle
import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
U24 = 2.0 ** -24
BF = 2.0 ** -8


@pytest.fixture(scope="module")
def tw():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def _f64(t):
    import torch

    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def _gamma(n):
    return n * U24 / (1 - n * U24)


def _run(tw, dev, w, P, R_max, l1, dy_dev, twice=False):
    """GPU forward keeping g and u, then the three backward calls with dx
    prefilled with NaN."""
    import torch

    M, K = dev["x"].shape
    N = w.N
    p = tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C, M)
    y, hy = tw.hybrid_forward(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"], p, P=P, R_max=R_max,
                              keep=True)
    outs = []
    for _ in range(2 if twice else 1):
        R1 = max(R_max, 1)
        o = {"hy_du": torch.empty((M, P), dtype=torch.float32, device="cuda"),
             "hy_dz": torch.empty((M, P), dtype=torch.float32, device="cuda"),
             "bk_du": torch.empty((R1, N), dtype=torch.bfloat16, device="cuda"),
             "bk_dz": torch.empty((R1, N), dtype=torch.bfloat16, device="cuda"),
             "dx": torch.full((M, K), float("nan"), dtype=torch.float32, device="cuda"),
             "dwg_t": torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda"),
             "dwu_t": torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda"),
             "dwd": torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")}
        tw.tw_hybrid_bwd_dh(dy_dev, dev["wd"], P, l1, hy["hy_g"], hy["hy_u"], hy["hy_idx"],
                            hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"], R_max,
                            hy["bk_g"], hy["bk_u"], o["hy_du"], o["hy_dz"], o["bk_du"],
                            o["bk_dz"])
        nx = tw.tw_hybrid_bwd_dx_workspace_bytes(R_max)
        wsx = torch.empty((max(nx, 1),), dtype=torch.uint8, device="cuda")
        tw.tw_hybrid_bwd_dx(dev["wg_t"], dev["wu_t"], M, P, o["hy_du"], o["hy_dz"], hy["hy_idx"],
                            hy["hy_cnt"], hy["route"], hy["bk_rows"], hy["bk_count"], R_max,
                            o["bk_du"], o["bk_dz"], o["dx"], wsx)
        wsw = torch.empty((tw.tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, R_max),),
                          dtype=torch.uint8, device="cuda")
        tw.tw_hybrid_bwd_dw(dev["x"], dy_dev, P, hy["hy_h"], o["hy_du"], o["hy_dz"],
                            hy["hy_idx"], hy["hy_cnt"], hy["route"], hy["bk_rows"],
                            hy["bk_count"], R_max, hy["bk_h"], o["bk_du"], o["bk_dz"],
                            o["dwg_t"], o["dwu_t"], o["dwd"], wsw)
        outs.append(o)
    torch.cuda.synchronize()
    g = {"hy_cnt": hy["hy_cnt"].cpu().numpy(), "hy_idx": hy["hy_idx"].cpu().numpy(),
         "hy_val": _f64(hy["hy_g"]), "route": hy["route"].cpu().numpy(),
         "bk_count": int(hy["bk_count"].cpu()[0])}
    nbk = min(g["bk_count"], R_max)
    g["bk_rows"] = hy["bk_rows"].cpu().numpy()[:nbk]
    acts = {"hy_u": _f64(hy["hy_u"]), "hy_h": _f64(hy["hy_h"])}
    for k in ("bk_g", "bk_u", "bk_h"):
        acts[k] = _f64(hy[k][:nbk]) if nbk else np.zeros((0, N))
    res = []
    for o in outs:
        r = {k: _f64(o[k]) for k in ("hy_du", "hy_dz", "dx", "dwg_t", "dwu_t", "dwd")}
        r["bk_du"] = _f64(o["bk_du"][:nbk]) if nbk else np.zeros((0, N))
        r["bk_dz"] = _f64(o["bk_dz"][:nbk]) if nbk else np.zeros((0, N))
        res.append(r)
    return g, acts, res


def _dense(hy, vals_sp, vals_bk, N):
    """Scatter per-entry values of sparse rows and backup rows to [M][N]."""
    M, P = hy["hy_idx"].shape
    out = np.zeros((M, N))
    for m in range(M):
        if hy["route"][m]:
            continue
        n = int(hy["hy_cnt"][m])
        out[m, hy["hy_idx"][m, :n]] = vals_sp[m, :n]
    for r, m in enumerate(hy["bk_rows"]):
        out[m] = vals_bk[r]
    return out


def _check(g, acts, r, d, dy_bits, w, l1, weights=True):
    orc = oracle.default()
    ref = orc.hybrid_bwd(d["x"], d["wg_t"], d["wu_t"], d["wd"], dy_bits, g, acts, l1)
    N, K = w.N, w.K
    x, dy = oracle.widen_bf16(d["x"]), oracle.widen_bf16(dy_bits)
    wg, wu, wd = (oracle.widen_bf16(d[k]) for k in ("wg_t", "wu_t", "wd"))
    gk = _gamma(K)
    # du, dz at the stored entries of sparse rows
    for m in range(w.M):
        if g["route"][m]:
            continue
        n = int(g["hy_cnt"][m])
        if n == 0:
            continue
        ids = g["hy_idx"][m, :n]
        bdh = 2 * gk * (np.abs(dy[m]) @ np.abs(wd[ids]).T)
        gv, uv = g["hy_val"][m, :n], acts["hy_u"][m, :n]
        du_ref, dz_ref = ref["hy_du"][m, :n], ref["hy_dz"][m, :n]
        assert np.all(np.abs(r["hy_du"][m, :n] - du_ref)
                      <= gv * bdh + 2 * U24 * np.abs(du_ref) + 1e-30), f"du row {m}"
        # dz = (dh u) + l1: the product and the sum each round once
        assert np.all(np.abs(r["hy_dz"][m, :n] - dz_ref)
                      <= np.abs(uv) * bdh + 2 * U24 * (np.abs(dz_ref - l1) + np.abs(dz_ref))
                      + 1e-30), f"dz row {m}"
    # backup rows (bf16), all slots at once
    bk = np.asarray(g["bk_rows"], dtype=np.int64)
    if len(bk):
        bdh = 2 * gk * (np.abs(dy[bk]) @ np.abs(wd).T)
        gv, uv = acts["bk_g"], acts["bk_u"]
        du_ref, dz_ref = ref["bk_du"], ref["bk_dz"]
        e_du = gv * bdh
        assert np.all(np.abs(r["bk_du"] - du_ref) <= e_du + BF * (np.abs(du_ref) + e_du)
                      + 1e-30), "backup du"
        e_dz = np.abs(uv) * bdh + 2 * U24 * (np.abs(dz_ref - l1 * (gv > 0)) + np.abs(dz_ref))
        assert np.all(np.abs(r["bk_dz"] - dz_ref) <= e_dz + BF * (np.abs(dz_ref) + e_dz)
                      + 1e-30), "backup dz"
        assert np.all(r["bk_dz"][gv == 0] == 0), "dz outside the active entries"
    # dense views of the gradients of the activations, GPU and oracle
    du_g = _dense(g, r["hy_du"], r["bk_du"], N)
    dz_g = _dense(g, r["hy_dz"], r["bk_dz"], N)
    du_r = _dense(g, ref["hy_du"], ref["bk_du"], N)
    dz_r = _dense(g, ref["hy_dz"], ref["bk_dz"], N)
    h = _dense(g, acts["hy_h"], acts["bk_h"], N)
    stored = ~g["route"].astype(bool)
    stored[g["bk_rows"]] = True
    gn = _gamma(2 * N)
    # dx
    bdx = (np.abs(du_g - du_r) @ np.abs(wu) + np.abs(dz_g - dz_r) @ np.abs(wg)
           + 2 * gn * (np.abs(du_g) @ np.abs(wu) + np.abs(dz_g) @ np.abs(wg)) + 1e-30)
    assert np.all(np.abs(r["dx"][stored] - ref["dx"][stored]) <= bdx[stored]), "dx"
    parity.check_y(r["dx"][stored], ref["dx"][stored], "dx")
    assert np.all(np.isnan(r["dx"][~stored])), "a row with nothing stored got a dx"
    if not weights:
        return int(stored.sum())
    # weight gradients
    gm = _gamma(w.M)
    xs, dys = x * stored[:, None], dy * stored[:, None]
    b_wd = 2 * gm * (np.abs(h).T @ np.abs(dys)) + 1e-30
    assert np.all(np.abs(r["dwd"] - ref["dwd"]) <= b_wd), "dwd"
    b_wu = np.abs(du_g - du_r).T @ np.abs(xs) + 2 * gm * (np.abs(du_g).T @ np.abs(xs)) + 1e-30
    assert np.all(np.abs(r["dwu_t"] - ref["dwu_t"]) <= b_wu), "dwu_t"
    b_wg = np.abs(dz_g - dz_r).T @ np.abs(xs) + 2 * gm * (np.abs(dz_g).T @ np.abs(xs)) + 1e-30
    assert np.all(np.abs(r["dwg_t"] - ref["dwg_t"]) <= b_wg), "dwg_t"
    for k in ("dwd", "dwu_t", "dwg_t"):
        parity.check_y(r[k], ref[k], k)
    return int(stored.sum())


def _dy(w, seed=11):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(rng.standard_normal((w.M, w.K)).astype(np.float32))


CASES = [
    ("tiny", dict(), 128, 8, 0.0),
    ("tiny", dict(), 32, 64, 0.01),             # many backup rows on the matrix cores
    ("tiny", dict(), 32, 8, 0.01),              # backup room exceeded: those rows store nothing
    ("tiny", dict(C=4), 128, 64, 0.02),         # TwELL tile rule
    ("tiny", dict(M=300, K=384, N=1152, C=6, density=0.03, sigma_s=0.5), 16, 300, 0.01),
    ("tiny", dict(M=513, K=512, N=2048, T=256, C=12, density=0.01, sigma_s=0.7, seed=3), 24, 64,
     0.005),
    ("tiny", dict(M=1, K=128, N=128, C=3, density=0.1), 4, 1, 0.01),
    ("tiny", dict(density=0.0), 128, 8, 0.01),  # nothing active: every gradient 0
    ("tiny", dict(density=1.0, C=128), 128, 64, 0.01),  # every row in the backup
    ("tiny", dict(M=200, K=4096, N=256, C=64, density=0.1), 64, 200, 0.01),  # K-sliced gradients
]


@pytest.mark.parametrize("name,kw,P,R_max,l1", CASES)
def test_hybrid_bwd_parity(tw, name, kw, P, R_max, l1):
    w = W[name].with_(**kw)
    print(f"case {w} P={P} R_max={R_max} l1={l1}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    dy_bits = _dy(w)
    g, acts, (r,) = _run(tw, dev, w, P, R_max, l1, parity.to_dev(dy_bits))
    _check(g, acts, r, d, dy_bits, w, l1)
    if kw.get("density") == 0.0:
        for k in ("dx", "dwg_t", "dwu_t", "dwd"):
            assert not r[k].any(), k


def test_hybrid_bwd_full_size_and_determinism(tw):
    """The full 0.5B block at the static capacities (P = 128, backup room
    M / 8), and two backward runs bit for bit equal."""
    w = W["ffn-0.5b"]
    P, R_max, l1 = 128, w.M // 8, 2e-5 * 1000
    print(f"case {w} P={P} R_max={R_max} l1={l1}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    dy_bits = _dy(w)
    g, acts, (r1, r2) = _run(tw, dev, w, P, R_max, l1, parity.to_dev(dy_bits), twice=True)
    used = (np.arange(P)[None, :] < g["hy_cnt"][:, None]) & (g["route"] == 0)[:, None]
    for k in r1:
        a, b = r1[k], r2[k]
        if k in ("hy_du", "hy_dz"):  # slots past a row's count are not written
            a, b = np.where(used, a, 0.0), np.where(used, b, 0.0)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64)), f"{k} not repeatable"
    assert g["bk_count"] <= R_max
    _check(g, acts, r1, d, dy_bits, w, l1)


def test_hybrid_bwd_2b_full(tw):
    """The full 2B block at the static capacities: the whole backward on the
    GPU against the oracle's backward of the GPU's own stored activations,
    on every row and every hidden column: du and dz at every stored entry,
    dx of every row, and the three weight gradients (each a sum over all
    rows)."""
    w = W["ffn-2b"]
    P, R_max, l1 = 128, w.M // 8, 2e-5 * 1000
    print(f"case {w} P={P} R_max={R_max} l1={l1}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    dy_bits = _dy(w)
    g, acts, (r,) = _run(tw, dev, w, P, R_max, l1, parity.to_dev(dy_bits))
    del dev
    assert 0 < g["bk_count"] <= R_max
    n = _check(g, acts, r, d, dy_bits, w, l1)
    print(f"checked all {w.M} rows ({g['bk_count']} backup), {n} with stored activations, "
          f"and all {w.N} columns of the weight gradients", flush=True)
