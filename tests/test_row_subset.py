"""The row-subset helper the full-size backward test samples with: the
oracle's backward over a subset of token rows (their storage, activations
and inputs) gives exactly the full backward's values on those rows, for
every per-row quantity (du, dz at the stored entries, the backup rows' du,
dz, and dx).  CPU only."""
import numpy as np

import oracle
import parity
from activation_sparse_feed_gate_amd import synth


def test_oracle_backward_on_a_row_subset_equals_its_rows():
    w = synth.WORKLOADS["tiny"].with_(M=300, K=384, N=1152, C=6, density=0.03, sigma_s=0.5)
    d = synth.make_inputs(w)
    orc = oracle.default()
    P, R_max, l1 = 16, 300, 0.01
    packed = orc.pack(orc.gate(d["x"], d["wg_t"]), w.T, w.C, w.M)
    hy = orc.hybrid_pack(packed, w.C, P, R_max)
    acts = orc.hybrid_up(d["x"], d["wg_t"], d["wu_t"], hy)
    rng = np.random.default_rng(2)
    dy = synth.f32_to_bf16_bits(rng.standard_normal((w.M, w.K)).astype(np.float32))
    full = orc.hybrid_bwd(d["x"], d["wg_t"], d["wu_t"], d["wd"], dy, hy, acts, l1)
    g = {k: np.asarray(hy[k]) for k in ("hy_cnt", "hy_idx", "hy_val", "route")}
    g["bk_count"] = int(hy["bk_count"])
    g["bk_rows"] = np.asarray(hy["bk_rows"])[:min(g["bk_count"], R_max)]
    assert g["bk_count"] > 10
    rows = np.array(sorted({0, 5, 17, w.M - 1} | set(g["bk_rows"][::3].tolist())), dtype=np.int64)
    gs, acs, rs, ds, dys = parity.hybrid_row_subset(g, acts, full, d, dy, rows)
    assert 0 < gs["bk_count"] < len(rows)
    sub = orc.hybrid_bwd(ds["x"], ds["wg_t"], ds["wu_t"], ds["wd"], dys, gs, acs, l1)
    for k in ("hy_du", "hy_dz", "dx", "bk_du", "bk_dz"):
        a, b = sub[k], rs[k]
        assert a.shape == b.shape, k
        assert np.array_equal(np.isnan(a), np.isnan(b)), k
        assert np.array_equal(np.nan_to_num(a), np.nan_to_num(b)), k
