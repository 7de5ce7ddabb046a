"""Comparison of the HIP path with the CPU oracle (test infrastructure).

Rules (the tolerances the hot path is held to):
- packing is bit-exact when the oracle packs the very gate values the GPU
  packed (the GPU's own fp32 z): counts, indices, values, overflow list and
  count;
- the GPU gate itself agrees with the oracle's float64 gate within the
  standard dot-product bound 2 * gamma_K * sum_k |x_k w_k| (bf16 products
  are exact in fp32; gamma_K = K u / (1 - K u), u = 2^-24);
- against the oracle's own gate, per tile the GPU count lies between the
  counts of z_ref > 1e-3 and z_ref > -1e-3, the index sets agree outside the
  band |z_ref| < 1e-3, and the overflow status agrees on every row whose
  status the band cannot change;
- the output satisfies max |y - y_ref| <= 1e-2 * max |y_ref| + 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BAND = 1e-3


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor (bit-preserving)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def upload(d: dict, device="cuda") -> dict:
    return {k: to_dev(d[k], device) for k in ("x", "wg_t", "wu_t", "wd")}


def run_path(tw, dev: dict, T: int, C: int, R_max: int, z_debug=True, dense=True) -> dict:
    """Run pack + sparse (+ dense) through the C ABI; results to host numpy."""
    p = tw.pack_gate(dev["x"], dev["wg_t"], T, C, R_max, z_debug=z_debug)
    y = tw.sparse_ffn(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"], p)
    yd = tw.ffn(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"]) if dense else None
    torch.cuda.synchronize()
    out = {k: p[k].cpu().numpy() for k in ("tw_val", "tw_idx", "tw_cnt", "ovf_rows")}
    out["ovf_count"] = int(p["ovf_count"].cpu()[0])
    if z_debug:
        out["z"] = p["z"].cpu().numpy()
    out["y"] = y.cpu().numpy()
    if dense:
        out["y_dense"] = yd.cpu().numpy()
    return out


def check_packing_bitexact(g: dict, T: int, C: int, R_max: int, rows=None) -> None:
    """The oracle packer applied to the GPU's own fp32 gate reproduces the
    GPU packing exactly (all rows, or the given rows for counts/slots)."""
    z = g["z"]
    M = z.shape[0]
    ref = oracle.default().pack(z.astype(np.float64), T, C, R_max)
    assert np.array_equal(g["tw_cnt"], ref["cnt"]), "counts differ"
    used = np.arange(C)[None, None, :] < np.minimum(ref["cnt"], C)[:, :, None]
    assert np.array_equal(np.where(used, g["tw_idx"], -1), np.where(used, ref["idx"], -1)), \
        "indices differ"
    gv = g["tw_val"].astype(np.float64)
    assert np.array_equal(np.where(used, gv, 0.0).view(np.uint64),
                          np.where(used, ref["val"], 0.0).view(np.uint64)), "values differ"
    assert g["ovf_count"] == ref["ovf_count"], (g["ovf_count"], ref["ovf_count"])
    n = min(ref["ovf_count"], R_max)
    assert np.array_equal(g["ovf_rows"][:n], ref["ovf_rows"][:n]), "overflow list differs"
    assert M == g["tw_cnt"].shape[0]


def check_gate_bound(z_gpu_rows: np.ndarray, z_ref_rows: np.ndarray, x_rows, wg_t) -> None:
    """|z_gpu - z_ref| <= 2 gamma_K sum_k |x_k w_k| on the given rows."""
    xa = np.abs(oracle.widen_bf16(x_rows))
    wa = np.abs(oracle.widen_bf16(wg_t))
    K = xa.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    bound = 2 * gamma * (xa @ wa.T)
    err = np.abs(z_gpu_rows.astype(np.float64) - z_ref_rows)
    assert np.all(err <= bound), f"gate error {err.max()} above bound"


def check_index_parity(g: dict, rows: np.ndarray, z_ref_rows: np.ndarray, T: int, C: int) -> None:
    """GPU packing vs the oracle's own gate on the given rows, outside the band."""
    M_s, N = z_ref_rows.shape
    NT = N // T
    zt = z_ref_rows.reshape(M_s, NT, T)
    lo = (zt > BAND).sum(axis=2)
    hi = (zt > -BAND).sum(axis=2)
    cnt = g["tw_cnt"][rows]
    assert np.all((cnt >= lo) & (cnt <= hi)), "count outside the band's range"
    ids = g["tw_idx"][rows]                                    # [M_s][NT][C]
    used = np.arange(C)[None, None, :] < np.minimum(cnt, C)[:, :, None]
    if C > 1:
        assert np.all(np.diff(ids, axis=2)[used[:, :, 1:]] > 0), "indices not ascending"
    t0 = (np.arange(NT) * T)[None, :, None]
    assert np.all(((ids >= t0) & (ids < t0 + T))[used]), "index outside its tile"
    # tiles whose whole active set was stored (at most C even at the band's
    # top): the stored set equals the firmly active columns, up to columns
    # inside the band
    stored = np.zeros((M_s, N), dtype=bool)
    r_i, t_i, s_i = np.nonzero(used)
    stored[r_i, ids[r_i, t_i, s_i]] = True
    whole = np.repeat(hi <= C, T, axis=1)                      # [M_s][N]
    firm = np.abs(z_ref_rows) >= BAND
    want = (z_ref_rows > 0) & firm
    assert not np.any(want & ~stored & whole), "a firmly active column is missing"
    assert not np.any(stored & ~want & firm & whole), "a firmly inactive column was packed"
    # overflow status on determined rows
    over_gpu = np.isin(rows, g["ovf_rows"][: min(g["ovf_count"], len(g["ovf_rows"]))]) | \
        (cnt > C).any(axis=1)
    surely_over = (lo > C).any(axis=1)
    surely_not = (hi <= C).all(axis=1)
    assert np.all(over_gpu[surely_over]), "row that must overflow did not"
    assert not np.any(over_gpu[surely_not]), "row that cannot overflow did"


def check_gate_rows(g: dict, d: dict, T: int, C: int, chunk: int = 2048) -> int:
    """The GPU gate of every row against the oracle's float64 gate (the
    2 gamma_K bound) and the GPU packing against it (index parity), in
    blocks of rows so that the float64 gate of a large batch is never held
    whole.  Returns the number of rows checked."""
    orc = oracle.default()
    M = g["z"].shape[0]
    for r0 in range(0, M, chunk):
        rows = np.arange(r0, min(r0 + chunk, M))
        z_ref = orc.gate(d["x"][rows], d["wg_t"])
        check_gate_bound(g["z"][rows], z_ref, d["x"][rows], d["wg_t"])
        check_index_parity(g, rows, z_ref, T, C)
    return M


_DENSE_REF = {}


def dense_reference(w, d: dict) -> np.ndarray:
    """The oracle's dense block output y_ref [M][K] (float64) for workload
    ``w`` (inputs ``d`` = synth.make_inputs(w)), computed once per test
    session: several full-size tests compare against the same block."""
    key = w.with_(T=0, C=0)  # the inputs do not depend on the tile shape
    if key not in _DENSE_REF:
        _DENSE_REF[key] = oracle.default().dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    return _DENSE_REF[key]


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what="y") -> float:
    err = float(np.abs(y_gpu.astype(np.float64) - y_ref).max(initial=0.0))
    tol = 1e-2 * float(np.abs(y_ref).max(initial=0.0)) + 1e-3
    assert err <= tol, f"{what}: max error {err} > tolerance {tol}"
    return err


def hybrid_row_subset(g: dict, acts: dict, r: dict, d: dict, dy_bits, rows):
    """The storage, activations, GPU gradients and inputs of a subset of
    token rows (ascending): every quantity but the weight gradients is per
    row, so the oracle's backward on the subset is the full one's rows."""
    pos = {int(m): i for i, m in enumerate(rows)}
    sel = [k for k, m in enumerate(g["bk_rows"]) if int(m) in pos]
    gs = {"hy_cnt": g["hy_cnt"][rows], "hy_idx": g["hy_idx"][rows], "hy_val": g["hy_val"][rows],
          "route": g["route"][rows], "bk_count": len(sel),
          "bk_rows": np.array([pos[int(g["bk_rows"][k])] for k in sel], dtype=g["bk_rows"].dtype)}
    acs = {"hy_u": acts["hy_u"][rows], "hy_h": acts["hy_h"][rows]}
    rs = {"hy_du": r["hy_du"][rows], "hy_dz": r["hy_dz"][rows], "dx": r["dx"][rows]}
    for k in ("bk_g", "bk_u", "bk_h"):
        acs[k] = acts[k][sel]
    for k in ("bk_du", "bk_dz"):
        rs[k] = r[k][sel]
    ds = dict(d, x=d["x"][rows])
    return gs, acs, rs, ds, dy_bits[rows]
