"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case is compared on every row: the packing bit for bit (the oracle
re-packs the GPU's own gate), the gate within its dot-product rounding bound,
the index sets against the oracle's float64 gate, and the output within the
output tolerance, at small shapes and at every full-size workload.
"""
import numpy as np
import pytest

import oracle
import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module")
def tw():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def _full_check(tw, w, R_max=None, dense=True):
    """Every row against the oracle: packing, gate bound, index parity, y."""
    print(f"case {w} R_max={R_max}", flush=True)
    d = synth.make_inputs(w)
    R_max = w.M if R_max is None else R_max
    g = parity.run_path(tw, parity.upload(d), w.T, w.C, R_max, dense=dense)
    parity.check_packing_bitexact(g, w.T, w.C, R_max)
    orc = oracle.default()
    z_ref = orc.gate(d["x"], d["wg_t"])
    rows = np.arange(w.M)
    parity.check_gate_bound(g["z"], z_ref, d["x"], d["wg_t"])
    parity.check_index_parity(g, rows, z_ref, w.T, w.C)
    y_ref = orc.dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    covered = np.ones(w.M, dtype=bool)
    if g["ovf_count"] > R_max:  # rows past R_max are left for the retry
        flagged = (g["tw_cnt"] > w.C).any(axis=1)
        listed = np.zeros(w.M, dtype=bool)
        listed[g["ovf_rows"][:R_max]] = True
        covered = ~flagged | listed
    parity.check_y(g["y"][covered], y_ref[covered], "sparse y")
    if dense:
        parity.check_y(g["y_dense"], y_ref, "dense y")
    return g, d


@pytest.mark.parametrize("kw", [
    dict(),                                   # tiny: 64 x 256 x 1024, T=128, C=16
    dict(C=12), dict(C=4), dict(C=1),         # some / all rows overflow
    dict(T=256, C=16), dict(T=256, C=40),     # tile spanning two waves
    dict(M=300, K=384, N=1152, T=128, C=8, density=0.02, sigma_s=0.5),  # ragged M, half column block
    dict(M=513, K=512, N=2048, T=256, C=12, density=0.01, sigma_s=0.7, seed=3),
    dict(M=1, K=128, N=128, T=128, C=3, density=0.1),
    # batches large enough for the 256 x 256 gate kernel (the others take the
    # small-batch one): a half-empty last column block, and T = 256
    dict(M=4096, K=256, N=1152, T=128, C=8, density=0.02, sigma_s=0.5),
    dict(M=2048, K=256, N=2048, T=256, C=12, density=0.01, sigma_s=0.7, seed=5),
    # batches of 32 to 128 rows: each row over 256 / M workgroups whose
    # partial rows a second kernel sums (2B and 0.5B block shapes)
    dict(M=32, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5),
    # few rows at the 2B block: the gate's reduction split into 8 K-slices
    dict(M=16, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=6),
    dict(M=3, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=7),
    dict(M=100, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=2),
    dict(M=128, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=4),
])
def test_tiny_all_rows(tw, kw):
    _full_check(tw, W["tiny"].with_(**kw))


@pytest.mark.parametrize("kw", [
    # both sides of each batch-size route change, every row checked: at the
    # 0.5B block the 256 x 256 gate kernel takes over above 768 rows, at the
    # 2B block above 256; the sparse kernel drops from 16 to 4 waves per row
    # above 256 rows
    dict(M=256, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=31),
    dict(M=257, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=32),
    dict(M=768, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=33),
    dict(M=769, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=34),
    dict(M=256, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=35),
    dict(M=257, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=36),
    # inside the small-batch gate: its reduction split into K-slices up to 8
    # rows (0.5B block) or 16 (2B), two K halves per workgroup up to 448 rows
    # (0.5B) or 192 (2B), one beyond
    dict(M=8, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=37),
    dict(M=9, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=38),
    dict(M=448, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=39),
    dict(M=449, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=40),
    dict(M=17, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=41),
    dict(M=192, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=42),
    dict(M=193, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=43),
    # the sparse kernel spreads a row over 256 / M workgroups for 32 to 128 rows
    dict(M=31, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=44),
    dict(M=129, K=2048, N=8192, T=256, C=16, density=0.003, sigma_s=0.5, seed=45),
    # heaviest-first order of the sparse kernel from 257 rows (above, and
    # the 0.5B block sizes) up to 8192, in segments of 256 rows: its last
    # batch size and the first without it, with a heavy tail (rows of more
    # than 64 entries and none over capacity)
    dict(M=8192, K=256, N=4096, T=128, C=8, density=0.01, sigma_s=0.7, seed=46),
    dict(M=8193, K=256, N=4096, T=128, C=8, density=0.01, sigma_s=0.7, seed=47),
])
def test_route_boundaries(tw, kw):
    _full_check(tw, W["tiny"].with_(**kw))


@pytest.mark.parametrize("kw", [
    # the largest shapes the library accepts: K = 4096 and 256 tiles per row
    # (here with the 256 x 256 gate kernel and several workgroups per row) ...
    dict(M=40, K=4096, N=32768, T=128, C=8, density=0.003, sigma_s=0.5, seed=11),
    # ... and K = 4096 in the few-row gate whose reduction is split into K-slices
    dict(M=8, K=4096, N=1024, T=128, C=8, density=0.02, sigma_s=0.5, seed=12),
])
def test_maximum_sizes(tw, kw):
    _full_check(tw, W["tiny"].with_(**kw))


@pytest.mark.parametrize("kw", [
    dict(density=0.0), dict(density=1.0, C=128), dict(density=1.0, C=16),
    dict(density=1.0, T=256, C=256),
    # 1024 rows take the sparse kernel's heaviest-first order: no heavy row
    # at all, and every row heavy with none over capacity
    dict(M=1024, density=0.0), dict(M=1024, density=1.0, C=128),
])
def test_density_extremes(tw, kw):
    g, _ = _full_check(tw, W["tiny"].with_(**kw))
    M = kw.get("M", 64)
    if kw["density"] == 0.0:
        assert not g["tw_cnt"].any() and g["ovf_count"] == 0 and not g["y"].any()
    elif kw["C"] == kw.get("T", 128):
        assert (g["tw_cnt"] == kw.get("T", 128)).all() and g["ovf_count"] == 0
    else:
        assert g["ovf_count"] == M


@pytest.mark.parametrize("kw,R_max", [
    (dict(C=12), 8),                                     # ~7 listed rows of 8
    (dict(M=64, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5), 8),  # 0.5B block
    (dict(M=16, K=2048, N=8192, T=256, C=16, density=0.01, sigma_s=0.5, seed=9), 2),
    # a capacity of none (an eighth of a batch under 8 tokens, rounded down):
    # no backup kernel runs; without overflow every row is the sparse
    # kernel's, with overflow the listed rows are left for the retry
    (dict(M=4, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=52), 0),
    (dict(M=7, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=51), 0),
    (dict(M=7, C=4), 0),                                 # every row overflows
    # the heaviest-first order (1024 rows) with a room smaller than the
    # overflow list: the rows past it are left for the retry
    (dict(M=1024, K=1024, N=4096, T=128, C=8, density=0.01, sigma_s=0.5, seed=53), 16),
])
def test_few_overflow_rows(tw, kw, R_max):
    """A backup capacity of a handful of rows (decode-size batches): the
    backup's split partials for one row block, summed by the sparse kernel."""
    g, _ = _full_check(tw, W["tiny"].with_(**kw), R_max=R_max)
    print(f"overflow rows {g['ovf_count']} of capacity {R_max}", flush=True)


def test_capacity_retry(tw):
    """Too small a dense backup: the true count comes back, and a retry with
    enough room gives the full result (the retry of the static-capacity
    scheme)."""
    w = W["tiny"].with_(C=4)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    g = parity.run_path(tw, dev, w.T, w.C, 5, dense=False)
    assert g["ovf_count"] > 5
    need = g["ovf_count"]
    g2 = parity.run_path(tw, dev, w.T, w.C, need, dense=False)
    y_ref = oracle.default().dense_ffn(d["x"], d["wg_t"], d["wu_t"], d["wd"])
    parity.check_y(g2["y"], y_ref)


def test_empty_batch(tw):
    import torch

    w = W["tiny"].with_(M=0)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    p = tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C, 0)
    y = tw.sparse_ffn(dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"], p)
    torch.cuda.synchronize()
    assert int(p["ovf_count"].cpu()[0]) == 0 and y.numel() == 0


@pytest.mark.parametrize("M", [512, 48])  # one workgroup per row; several per row
def test_deterministic(tw, M):
    w = W["tiny"].with_(M=M, C=6, sigma_s=0.5, density=0.03)
    print(f"case {w}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    a = parity.run_path(tw, dev, w.T, w.C, w.M)
    b = parity.run_path(tw, dev, w.T, w.C, w.M)
    assert a["ovf_count"] == b["ovf_count"]
    n = a["ovf_count"]  # list entries past the count are unspecified
    assert np.array_equal(a["ovf_rows"][:n], b["ovf_rows"][:n])
    for k in ("tw_cnt", "y", "y_dense", "z"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    used = np.arange(w.C)[None, None, :] < np.minimum(a["tw_cnt"], w.C)[:, :, None]
    assert np.array_equal(np.where(used, a["tw_idx"], 0), np.where(used, b["tw_idx"], 0))


@pytest.mark.parametrize("name", ["ffn-0.5b", "ffn-2b"])
def test_deterministic_full_size(tw, name):
    """The benchmark's configuration (full block, backup room M / 8) gives
    the same bits run after run: counts, overflow list, y and the dense y."""
    w = W[name]
    R_max = w.M // 8
    print(f"case {w} R_max={R_max}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    a = parity.run_path(tw, dev, w.T, w.C, R_max, z_debug=False)
    b = parity.run_path(tw, dev, w.T, w.C, R_max, z_debug=False)
    assert 0 < a["ovf_count"] <= R_max and a["ovf_count"] == b["ovf_count"]
    n = a["ovf_count"]  # list entries past the count are unspecified
    assert np.array_equal(a["ovf_rows"][:n], b["ovf_rows"][:n])
    for k in ("tw_cnt", "y", "y_dense"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


@pytest.mark.parametrize("name,dens,cap", [
    ("ffn-0.5b", None, 8), ("ffn-1b", None, 8), ("ffn-2b", None, 8), ("ffn-ovf", None, 8),
    ("ffn-2b", 0.0, 8), ("ffn-2b", 0.05, 8), ("ffn-paper", None, 8),
    ("ffn-0.5b", None, 1),  # room for every row: the other overflow-row tiling
])
def test_full_size(tw, name, dens, cap):
    """Full sizes with the backup capacity the benchmark uses (an eighth of
    the batch, retried with the true count when the batch overflows it).
    Every row is compared with the oracle: packing bit-exact on the GPU's
    own gate, the gate within its rounding bound and the index sets against
    the oracle's float64 gate, and y (sparse and dense paths) within the
    output tolerance of the oracle's dense block."""
    w = W[name] if dens is None else W[name].with_(density=dens)
    R_max = w.M // cap
    print(f"case {w} R_max={R_max}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    g = parity.run_path(tw, dev, w.T, w.C, R_max)
    if g["ovf_count"] > R_max:
        R_max = g["ovf_count"]
        print(f"retry with R_max={R_max}", flush=True)
        g = parity.run_path(tw, dev, w.T, w.C, R_max)
    del dev
    parity.check_packing_bitexact(g, w.T, w.C, R_max)
    parity.check_gate_rows(g, d, w.T, w.C)
    y_ref = parity.dense_reference(w, d)
    e_sp = parity.check_y(g["y"], y_ref, "sparse y")
    e_dn = parity.check_y(g["y_dense"], y_ref, "dense y")
    print(f"all {w.M} rows: max|dy| sparse {e_sp:.3g} dense {e_dn:.3g}, "
          f"{g['ovf_count']} overflow rows", flush=True)
    # properties on every row: overflow rows are exactly the listed ones, and
    # rows without an active neuron produce exact zeros
    flagged = (g["tw_cnt"] > w.C).any(axis=1)
    assert np.array_equal(np.nonzero(flagged)[0], g["ovf_rows"][: g["ovf_count"]])
    empty = g["tw_cnt"].sum(axis=1) == 0
    assert not g["y"][empty].any()
